"""GPU tests of the split partials, the standalone combine, paging and determinism."""
import numpy as np
import pytest
import torch

from mla_latent_kv_03_amd import workloads
from oracle import mla_ref as ref

from gpu_helpers import BF16_TOL, F32_TOL, DeviceCase, assert_close, record, to_np

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_partials_and_split_table(kv):
    _print_case("partials", kv=kv)
    lens = [300, 0, 1025, 64, 5]
    dims = dict(n_h=128, d_c=512, d_r=64, d_v=128) if kv != "f32" else dict(n_h=16, d_c=40, d_r=8, d_v=8)
    x = workloads.make_decode(lens, page_size=64, kv_dtype=kv, q_dtype="f32" if kv == "f32" else "bf16",
                              seed=101, **dims)
    G = 7
    case = DeviceCase(x, num_splits=G)
    _, _, ws = case.run(partials_only=True)
    table, plse, pu = case.binding.workspace_views(case.params, ws)
    want_table, pieces = ref.split_table(lens, G)
    assert np.array_equal(table.cpu().numpy(), want_table), "split table differs"
    qn, qp = x.q_nope.double().numpy(), x.q_pe.double().numpy()
    plse_h, pu_h = plse.cpu().numpy(), pu.float().cpu().numpy()
    tol = F32_TOL if kv == "f32" else BF16_TOL
    for (b, w, slot, t0, t1) in pieces:
        c, kp = case.rows_of(b)
        u_ref, lse_ref = ref.split_partial(qn[b, 0], qp[b, 0], c, kp, x.softmax_scale, t0, t1)
        assert_close(pu_h[slot, 0], u_ref, tol, f"partial u b={b} slot={slot}")
        assert np.max(np.abs(plse_h[slot, 0] - lse_ref)) <= (1e-5 if kv == "f32" else 5e-3)


@pytest.mark.parametrize("B,G,seed", [(64, 256, 11), (65, 7, 12), (130, 256, 13), (200, 64, 14), (130, 1, 15)])
def test_split_table_across_wave_steps(B, G, seed):
    """The device split walk takes 64 sequences per scan step: batches of one, two and four
    steps, zero lengths among them, and share counts below, at and above the batch."""
    _print_case("split walk", B=B, G=G, seed=seed)
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 260, size=B)
    lens[rng.random(B) < 0.15] = 0
    lens[rng.integers(0, B, size=3)] = [1500, 64, 65]
    lens = [int(v) for v in lens]
    x = workloads.make_decode(lens, page_size=64, kv_dtype="bf16", q_dtype="bf16", seed=seed + 100,
                              n_h=128, d_c=512, d_r=64, d_v=128)
    case = DeviceCase(x, num_splits=G)
    _, _, ws = case.run(partials_only=True)
    table, plse, pu = case.binding.workspace_views(case.params, ws)
    want_table, pieces = ref.split_table(lens, G)
    assert np.array_equal(table.cpu().numpy(), want_table), "split table differs"
    # A sample of pieces, most of them past the first 64 sequences, against the oracle.
    qn, qp = x.q_nope.double().numpy(), x.q_pe.double().numpy()
    plse_h, pu_h = plse.cpu().numpy(), pu.float().cpu().numpy()
    late = [pc for pc in pieces if pc[0] >= 64] or pieces
    sample = [pieces[0], pieces[-1]] + [late[i] for i in rng.choice(len(late), size=min(4, len(late)), replace=False)]
    for (b, w, slot, t0, t1) in sample:
        c, kp = case.rows_of(b)
        u_ref, lse_ref = ref.split_partial(qn[b, 0], qp[b, 0], c, kp, x.softmax_scale, t0, t1)
        assert_close(pu_h[slot, 0], u_ref, BF16_TOL, f"partial u b={b} slot={slot} tokens [{t0}, {t1})")
        assert np.max(np.abs(plse_h[slot, 0] - lse_ref)) <= 5e-3, f"partial lse b={b} slot={slot}"


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_standalone_combine_on_oracle_partials(kv):
    """Partials of an arbitrary partition (oracle-made) merged by mla_decode_splitkv_combine."""
    _print_case("combine", kv=kv)
    rng = np.random.default_rng(202)
    lens = [90, 400, 1, 0]
    dims = dict(n_h=128, d_c=512, d_r=64, d_v=128) if kv == "bf16" else dict(n_h=8, d_c=24, d_r=4, d_v=6)
    x = workloads.make_decode(lens, s_q=2, page_size=64, kv_dtype=kv, q_dtype=kv, seed=203, **dims)
    G = 20
    case = DeviceCase(x, num_splits=G)
    ws = case.binding.alloc_workspace(case.params)
    table, plse, pu = case.binding.workspace_views(case.params, ws)
    plse.fill_(float("nan"))
    pu.fill_(float("nan"))
    qn, qp = x.q_nope.double().numpy(), x.q_pe.double().numpy()
    w = x.w_uv.double().numpy()
    B, s_q = x.batch, x.s_q
    tab = np.zeros((B, 2), np.int32)
    next_slot = 1
    o_ref = np.zeros((B, s_q, x.n_h, x.d_v))
    lse_ref = np.full((B, s_q, x.n_h), -np.inf)
    for b in range(B):
        L = lens[b]
        c, kp = case.rows_of(b)
        n_parts = int(rng.integers(1, 5))
        cuts = sorted(rng.integers(0, L + 1, size=n_parts - 1)) if L else [0] * (n_parts - 1)
        edges = [0, *cuts, L]
        tab[b] = (next_slot, n_parts)
        for q in range(s_q):
            n_vis = ref.visible_len(L, s_q, q)
            us, ls = [], []
            for i in range(n_parts):
                t0, t1 = edges[i], min(edges[i + 1], n_vis)
                u_s, l_s = ref.split_partial(qn[b, q], qp[b, q], c, kp, x.softmax_scale, t0, max(t0, t1))
                plse[next_slot + i, q] = torch.from_numpy(l_s.astype(np.float32))
                pu[next_slot + i, q] = torch.from_numpy(u_s.astype(np.float32))
                us.append(u_s)
                ls.append(l_s)
            u, l = ref.combine(np.array(us), np.array(ls))
            o_ref[b, q] = ref.up_project(u, w)
            lse_ref[b, q] = l
        next_slot += n_parts
    assert next_slot <= G + B
    table.copy_(torch.from_numpy(tab))
    out = torch.empty(B, s_q, x.n_h, x.d_v, dtype=x.q_nope.dtype, device="cuda")
    lse = torch.empty(B, s_q, x.n_h, dtype=torch.float32, device="cuda")
    case.binding.mla_decode_splitkv_combine(case.params, ws, case.w_uv, out, lse)
    torch.cuda.synchronize()
    tol = BF16_TOL if kv == "bf16" else F32_TOL
    assert_close(to_np(out), o_ref, tol, "combine out")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    assert np.max(np.abs(to_np(lse)[fin] - lse_ref[fin])) <= 1e-5


def test_standalone_combine_slot_counts():
    """40 rows of 128 heads (two 32-row blocks, eight units per wave): slot counts that take every
    merge path of the combine, oracle-made partials.  Units of at most 8 slots are merged all at
    once per wave (at most 4 of them from the first loads, 5..8 with a second batch); a wave with a
    unit of 9..64 slots takes the per-unit merge, and one of more than 64 its second loop."""
    _print_case("combine slot counts")
    rng = np.random.default_rng(204)
    counts = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 33, 64, 65, 70]
    B = 40
    parts = [counts[b] if b < len(counts) else int(rng.integers(1, 9)) for b in range(B)]
    lens = [int(rng.integers(40, 300)) for _ in range(B)]
    x = workloads.make_decode(lens, s_q=1, page_size=64, seed=205, n_h=128, d_c=512, d_r=64, d_v=128)
    G = sum(parts)
    case = DeviceCase(x, num_splits=G)
    ws = case.binding.alloc_workspace(case.params)
    table, plse, pu = case.binding.workspace_views(case.params, ws)
    plse.fill_(float("nan"))
    pu.fill_(float("nan"))
    qn, qp = x.q_nope.double().numpy(), x.q_pe.double().numpy()
    w = x.w_uv.double().numpy()
    tab = np.zeros((B, 2), np.int32)
    next_slot = 0
    o_ref = np.zeros((B, 1, x.n_h, x.d_v))
    lse_ref = np.full((B, 1, x.n_h), -np.inf)
    for b in range(B):
        L, n_parts = lens[b], parts[b]
        c, kp = case.rows_of(b)
        edges = [0, *sorted(rng.integers(0, L + 1, size=n_parts - 1)), L]
        tab[b] = (next_slot, n_parts)
        us, ls = [], []
        for i in range(n_parts):
            u_s, l_s = ref.split_partial(qn[b, 0], qp[b, 0], c, kp, x.softmax_scale, edges[i], edges[i + 1])
            plse[next_slot + i, 0] = torch.from_numpy(l_s.astype(np.float32))
            pu[next_slot + i, 0] = torch.from_numpy(u_s.astype(np.float32))
            us.append(u_s)
            ls.append(l_s)
        u, l = ref.combine(np.array(us), np.array(ls))
        o_ref[b, 0] = ref.up_project(u, w)
        lse_ref[b, 0] = l
        next_slot += n_parts
    assert next_slot <= G + B
    table.copy_(torch.from_numpy(tab))
    out = torch.empty(B, 1, x.n_h, x.d_v, dtype=x.q_nope.dtype, device="cuda")
    lse = torch.empty(B, 1, x.n_h, dtype=torch.float32, device="cuda")
    case.binding.mla_decode_splitkv_combine(case.params, ws, case.w_uv, out, lse)
    torch.cuda.synchronize()
    record("standalone combine, 1..70 slots per row", *assert_close(to_np(out), o_ref, BF16_TOL, "combine out"),
           n=o_ref.size)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    assert np.max(np.abs(to_np(lse)[fin] - lse_ref[fin])) <= 1e-5


def _contiguous_copy(x):
    """Same logical rows as x, one page per sequence, identity block table."""
    L_max = int(x.seq_lens.max())
    P = max(64, -(-L_max // 64) * 64)
    pool = torch.zeros(x.batch * P, x.pool.shape[1], dtype=x.pool.dtype)
    tab = x.block_table.numpy()
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        j = np.arange(L)
        slots = tab[b, j // x.page_size].astype(np.int64) * x.page_size + j % x.page_size
        pool[b * P: b * P + L] = x.pool[torch.from_numpy(slots)]
    return workloads.DecodeInputs(q_nope=x.q_nope, q_pe=x.q_pe, pool=pool,
                                  block_table=torch.arange(x.batch, dtype=torch.int32)[:, None],
                                  seq_lens=x.seq_lens, w_uv=x.w_uv, page_size=P, softmax_scale=x.softmax_scale,
                                  kv_dtype=x.kv_dtype)


@pytest.mark.parametrize("kv,s_q", [("bf16", 1), ("bf16", 2), ("fp8", 1)])
def test_paged_equals_contiguous_bitwise(kv, s_q):
    _print_case("paged_vs_contiguous", kv=kv, s_q=s_q)
    x = workloads.make_decode([1500, 64, 3000, 200], s_q=s_q, page_size=64, kv_dtype=kv, seed=303)
    y = _contiguous_copy(x)
    a = DeviceCase(x, num_splits=11)
    c = DeviceCase(y, num_splits=11)
    if kv == "fp8":
        for b in range(x.batch):
            sa, sc = a.slots_of(b), c.slots_of(b)
            assert torch.equal(a.pool[torch.from_numpy(sa).cuda()], c.pool[torch.from_numpy(sc).cuda()])
    oa, la, _ = a.run()
    oc, lc, _ = c.run()
    assert torch.equal(oa.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lc.view(torch.int32))


def test_poisoned_unused_slots_are_never_read():
    _print_case("poison")
    x = workloads.make_decode([130, 1, 64, 65], page_size=64, seed=404, poison=True)
    assert torch.isnan(x.pool.float()).any()
    clean = workloads.DecodeInputs(**{**x.__dict__, "pool": torch.nan_to_num(x.pool, nan=0.0)})
    a = DeviceCase(x, num_splits=5)
    b = DeviceCase(clean, num_splits=5)
    oa, la, _ = a.run()
    ob, lb, _ = b.run()
    assert torch.isfinite(oa.float()).all() and torch.isfinite(la).all()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_deterministic_repeat():
    _print_case("determinism")
    x = workloads.make_decode([2048, 777, 5], s_q=2, page_size=64, seed=505)
    case = DeviceCase(x)
    o1, l1, ws = case.run()
    o2, l2, _ = case.run(workspace=ws)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_empty_and_invisible_rows():
    _print_case("empty_rows")
    x = workloads.make_decode([0, 1, 2, 0], s_q=2, page_size=64, seed=606)
    case = DeviceCase(x, num_splits=3)
    out, lse, _ = case.run()
    o, l = to_np(out), to_np(lse)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0])) and np.all(o[3] == 0)
    assert np.all(o[1, 0] == 0) and np.all(np.isneginf(l[1, 0]))            # L = 1: first query sees nothing
    o_ref, lse_ref = case.oracle([1, 2])
    assert_close(o[1:3], o_ref[1:3], BF16_TOL, "tiny lengths")


def test_invalid_page_ids_hide_tokens():
    _print_case("invalid_pages")
    x = workloads.make_decode([256, 256], page_size=64, seed=707)
    bad = x.block_table.clone()
    bad[1, 2] = 10 ** 6                                  # tokens 128..191 of sequence 1 become invisible
    y = workloads.DecodeInputs(**{**x.__dict__, "block_table": bad})
    case = DeviceCase(y, num_splits=4)
    out, lse, _ = case.run()
    qn, qp, w = x.q_nope.double().numpy(), x.q_pe.double().numpy(), x.w_uv.double().numpy()
    tab = x.block_table.numpy()
    rows = x.pool.double().numpy()
    keep = [j for j in range(256) if j // 64 != 2]
    slots = [tab[1, j // 64] * 64 + j % 64 for j in keep]
    o_ref, lse_ref, _ = ref.mla_absorbed(qn[1, 0], qp[1, 0], rows[slots, :512], rows[slots, 512:], w,
                                         x.softmax_scale, len(keep))
    assert_close(to_np(out)[1, 0], o_ref, BF16_TOL, "invalid page")
