"""OCP FP8 E4M3 ("fn" variant) reference and the per-token cache quantizer.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

The pages treat cache quantization only as the orthogonal bytes-per-element lever
([AA] "Attention-head anatomy", sections 4 and 7: the calculator's low-bit MLA rows,
KIVI/KVQuant-style 4- and 2-bit caches).  The deliverable's long-context layout
stores every value of the 576-wide row as OCP E4M3 with one float32 scale per token.
This module is written from the OCP 8-bit floating point format definition:
1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 encodes
subnormals m * 2^-9; exponent field 15 with mantissa 7 is NaN (no infinities);
the largest finite magnitude is 1.75 * 2^8 = 448.

Readings (numbered as in the design notes):
  R11 all 576 values (c and k^R) are E4M3 codes; one float32 scale per token;
      dequantized value = code value * scale; queries stay bf16.
  R12 quantizer: amax = max |x| in float32; amax == 0 -> scale = inv = 1; otherwise
      inv = fp32(448 / amax), scale = fp32(amax / 448); code = E4M3_RNE_sat(fp32(x * inv)).
      Round to nearest, ties to even, saturating to +-448; subnormals kept; the sign
      of zero is kept.

Pins (tests/test_fp8_ref.py): the decode table against the format's closed-form
values (max 448, min subnormal 2^-9, NaN codes); the encoder against torch's
float8_e4m3fn cast on a dense sweep of in-range float32 inputs (a library routine),
and against brute-force nearest-value search over the decode table.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table():
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_encode(x):
    """Round float32 values to E4M3 codes: nearest, ties to even, saturate at 448.

    Magnitudes >= 448 give 448 (code 0x7E); below the smallest normal 2^-6 the
    quantum is 2^-9 (subnormal codes 0..7, a carry to 8 is the smallest normal);
    in binade [2^E, 2^(E+1)) the quantum is 2^(E-3).  NaN gives 0x7F.  The sign bit
    is copied, also for zeros.
    """
    x = np.asarray(x, dtype=np.float32)
    v = x.astype(np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    with np.errstate(invalid="ignore"):
        k_sub = np.rint(a / 2.0 ** -9).astype(np.int64)          # subnormal branch
        _, e2 = np.frexp(np.where(a > 0, a, 1.0))                 # a = f * 2^e2, f in [0.5, 1)
        E = e2.astype(np.int64) - 1                               # a in [2^E, 2^(E+1))
        k = np.rint(a / np.ldexp(1.0, E - 3)).astype(np.int64)    # 8..16 in the normal branch
    carry = k == 16
    E = np.where(carry, E + 1, E)
    k = np.where(carry, 8, k)
    code_norm = np.minimum(((E + 7) << 3) | (k - 8), 0x7E)
    code = np.where(a < 2.0 ** -6, k_sub, code_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | sign
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows(rows):
    """Per-token quantization of cache rows (reading R12), one scale per row.

    rows: float32 [N, D] (D = 576 for the V3 shape).  Returns (codes uint8 [N, D],
    scales float32 [N]).  Each row: amax = max |x| in float32; amax == 0 gives
    scale = inv = 1; otherwise inv = fp32(448 / amax), scale = fp32(amax / 448);
    codes = E4M3_RNE_sat(fp32(x * inv)).
    """
    rows = np.asarray(rows, dtype=np.float32)
    amax = np.abs(rows).max(axis=1) if rows.shape[1] else np.zeros(rows.shape[0], np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    scaled = (rows * inv[:, None]).astype(np.float32)
    return e4m3_encode(scaled), scale


def quantize_row(row):
    """Per-token quantization of one cache row; see quantize_rows."""
    codes, scale = quantize_rows(np.asarray(row, dtype=np.float32)[None, :])
    return codes[0], scale[0]
