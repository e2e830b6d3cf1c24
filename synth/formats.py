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
import os
from concurrent.futures import ThreadPoolExecutor

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

    Works on the binary32 bit patterns.  A magnitude of at least 2**-6 (E4M3's
    smallest normal) keeps 3 of its 23 fraction bits: the pattern is rounded
    to nearest-even at bit 20 (a carry into the exponent is the correct next
    binade), the exponent is rebiased from 127 to 7 and codes past 0x7E (448)
    saturate.  Below 2**-6 the values are the multiples of the subnormal step
    2**-9: code = rint(|v| * 512) (exact scaling; 8 is 2**-6 itself, which is
    also the code of the smallest normal).  NaN -> 0x7F.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32)
    sign = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    a = u & np.uint32(0x7FFFFFFF)
    r = a + np.uint32(0x7FFFF) + ((a >> np.uint32(20)) & np.uint32(1))
    exp = (r >> np.uint32(23)).astype(np.int32) - 127 + 7
    mant = ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    normal = np.minimum((exp << 3) | mant, 0x7E)
    mag = a.view(np.float32)
    small = a < np.uint32(0x3C800000)          # |v| < 2**-6
    sub = np.rint(np.where(small, mag, np.float32(0.0)) * np.float32(512.0)).astype(np.int32)
    code = np.where(small, sub, normal).astype(np.uint8) | sign
    nan = a > np.uint32(0x7F800000)
    if nan.any():
        code[nan] = E4M3_NAN_CODE
    return code


def _by_row_blocks(fn, rows, block_rows=8192):
    """Apply ``fn(r0, r1)`` to consecutive row blocks [r0, r1) on a few host
    threads (numpy releases the GIL inside its loops); every block writes its
    own slice of the result, so the outcome does not depend on the blocking."""
    blocks = [(r0, min(rows, r0 + block_rows)) for r0 in range(0, rows, block_rows)]
    if len(blocks) <= 1:
        for r0, r1 in blocks:
            fn(r0, r1)
        return
    workers = max(1, min(16, os.cpu_count() or 1, len(blocks)))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(lambda b: fn(*b), blocks))


def f32_to_bf16_bits_blocked(x):
    """f32_to_bf16_bits over the last axis of a large array, in row blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.reshape(-1, x.shape[-1]) if x.ndim > 1 else x.reshape(1, -1)
    out = np.empty(rows.shape, dtype=np.uint16)

    def enc(r0, r1):
        out[r0:r1] = f32_to_bf16_bits(rows[r0:r1])
    _by_row_blocks(enc, rows.shape[0])
    return out.reshape(x.shape)


def quantize_rows_e4m3(x):
    """Per-row fp32 scale (absmax/448) and e4m3 codes for x[..., D] (fp32).

    Rows are encoded in blocks on a few host threads, which keeps the
    temporaries small for multi-GB caches (the result does not depend on the
    blocking)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.reshape(-1, x.shape[-1])
    codes = np.empty(rows.shape, dtype=np.uint8)
    scale = np.empty(rows.shape[0], dtype=np.float32)

    def enc(r0, r1):
        absmax = np.max(np.abs(rows[r0:r1]), axis=-1).astype(np.float32)
        s = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
        s = np.where(absmax == 0, np.float32(1.0), s).astype(np.float32)
        scale[r0:r1] = s
        codes[r0:r1] = f32_to_e4m3_codes((rows[r0:r1] / s[:, None]).astype(np.float32))
    _by_row_blocks(enc, rows.shape[0])
    return codes.reshape(x.shape), scale.reshape(x.shape[:-1])
