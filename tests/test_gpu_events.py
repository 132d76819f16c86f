"""The measurement hook mla_set_attention_events: the partial-attention kernel records the
caller's events around itself, the results do not change, and NULL, NULL turns it off."""
import ctypes

import numpy as np
import pytest

from mla_latent_kv_03_amd import workloads
from gpu_helpers import DeviceCase

pytestmark = pytest.mark.gpu


def _hip():
    import torch  # noqa: F401  (loads the HIP runtime)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def test_attention_events_time_the_kernel():
    print("[case] attention_events", flush=True)
    import torch
    x = workloads.make_decode([700, 64, 1500], n_h=128, page_size=64, seed=91)
    case = DeviceCase(x, num_splits=8)
    out_plain, lse_plain, _ = case.run()
    torch.cuda.synchronize()
    hip = _hip()
    start, stop = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(start)) == 0 and hip.hipEventCreate(ctypes.byref(stop)) == 0
    lib = case.binding.LIB
    try:
        assert lib.mla_set_attention_events(start, stop) == 0
        out_ev, lse_ev, _ = case.run()
        torch.cuda.synchronize()
    finally:
        assert lib.mla_set_attention_events(None, None) == 0
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), start, stop) == 0
    assert 0.0 < ms.value < 1000.0, ms.value
    hip.hipEventDestroy(start)
    hip.hipEventDestroy(stop)
    # Same kernel, same inputs: bit-identical results.
    assert np.array_equal(out_ev.cpu().float().numpy(), out_plain.cpu().float().numpy())
    assert np.array_equal(lse_ev.cpu().numpy(), lse_plain.cpu().numpy())
