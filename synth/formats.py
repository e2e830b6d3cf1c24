"""Storage-format encoders used to build synthetic inputs.

* bf16: the upper 16 bits of an IEEE-754 binary32, rounded to nearest-even.
* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits, no infinities, S.1111.111 is NaN, largest finite magnitude 448.  The
  "推理优化" tag page's quantisation article lists E4M3 as 4 exponent / 3
  mantissa bits with range +-448 (its FP8 format table).
* Per-token KV quantisation: one fp32 scale per stored token row (the whole
  latent+rope row), scale = absmax / 448, code = RNE(x / scale) saturated to
  +-448; an all-zero row gets scale 1 and zero codes.

These run on the host only while inputs are drawn.  Decoding (code -> value)
is deliberately not here: the oracle and the kernels each decode on their own.
"""
import numpy as np

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F
E4M3_MAX = 448.0


def f32_to_bf16_bits(x):
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs never overflow uint32 here (largest is 0xFF7FFFFF + 0x8000)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(b):
    """uint16 bf16 bit patterns -> fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3_codes(v):
    """fp32 array -> uint8 OCP e4m3 codes, round-to-nearest-even, saturating at +-448.

    Works exponent by exponent: a normal value with binary exponent e (>= -6)
    has quantum 2**(e-3); below 2**-6 the quantum is the subnormal step 2**-9.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    _, ex = np.frexp(a)              # a = m * 2**ex, m in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1, -6, 8)
    quantum = np.ldexp(1.0, e - 3)
    n = np.rint(a / quantum)         # numpy rint: ties to even
    val = np.minimum(n * quantum, E4M3_MAX)
    # re-derive the fields from the rounded value (handles mantissa carry)
    _, ex2 = np.frexp(val)
    e2 = ex2.astype(np.int64) - 1
    sub = val < 2.0 ** -6
    mant_sub = np.rint(val / 2.0 ** -9).astype(np.int64)
    exp_field = np.where(sub, 0, e2 + 7)
    mant_norm = np.rint((val / np.ldexp(1.0, e2) - 1.0) * 8.0).astype(np.int64)
    mant = np.where(sub, mant_sub, mant_norm)
    code = (exp_field << 3 | mant).astype(np.uint8) | sign
    nan = np.isnan(v)
    if nan.any():
        code[nan] = E4M3_NAN_CODE
    return code


def quantize_rows_e4m3(x):
    """Per-row fp32 scale (absmax/448) and e4m3 codes for x[..., D] (fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1).astype(np.float32)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(absmax == 0, np.float32(1.0), scale).astype(np.float32)
    v = (x / scale[..., None]).astype(np.float32)
    return f32_to_e4m3_codes(v), scale
