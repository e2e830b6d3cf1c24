"""Workload table and seeded generator for MLA decode inputs.

Shapes follow the decode problem the pages describe: one stored row per token
of 512 latent + 64 rope values that serves as both key and value (TokenSpeed
code-audit article, technology list, MLA kernel entry), pages of fixed size
addressed through a per-request block table (the "推理优化" tag page,
PagedAttention article), and a prefix whose pages are shared by reference
between requests (TokenSpeed 580 tok/s zero-copy article, KV-cache prefix
sharing).

Draw order per workload (numpy PCG64, seed = 1000 + workload index unless a
seed is given): seq_lens -> physical page permutation -> KV values -> q_abs ->
q_rope.  Values are drawn in fp32, multiplied by sigma and rounded once to the
storage type (bf16 RNE, or e4m3 codes with a per-token fp32 scale).
Unused storage (decoy pages, slots past the end of a request's last page) is
filled with NaN when ``poison`` is set; page-table entries past a request's
last page are -1.
"""
from dataclasses import dataclass, replace
import math

import numpy as np

from .formats import (f32_to_bf16_bits, f32_to_bf16_bits_blocked, quantize_rows_e4m3, BF16_NAN_BITS,
                      E4M3_NAN_CODE)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    heads: int
    d_latent: int
    d_rope: int
    page_size: int
    seq_lens: tuple            # ("fixed", (L0, L1, ...)) or ("uniform", lo, hi) inclusive
    kv_dtype: str              # "f32" | "bf16" | "fp8"
    q_dtype: str               # "f32" | "bf16"
    out_dtype: str             # "f32" | "bf16"
    sigma: float
    scale: float               # softmax scale, passed as float32
    causal: bool = False
    shared_prefix: int = 0     # tokens whose pages every request aliases
    num_splits: int = 0        # 0 = library chooses
    decoys: int = 64           # extra NaN-filled physical pages
    index: int = -1            # position in WORKLOADS (seed base)

    @property
    def d(self):
        return self.d_latent + self.d_rope

    @property
    def max_seq_len(self):
        if self.seq_lens[0] == "fixed":
            return int(max(self.seq_lens[1]))
        return int(self.seq_lens[2])

    @property
    def max_pages(self):
        return -(-self.max_seq_len // self.page_size)

    @property
    def rows(self):
        return self.q_len * self.heads

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny_f32", batch=2, q_len=1, heads=16, d_latent=64, d_rope=16, page_size=16,
             seq_lens=("fixed", (37, 100)), kv_dtype="f32", q_dtype="f32", out_dtype="f32",
             sigma=1.0, scale=1.0 / math.sqrt(80.0), decoys=6, index=0),
    Workload("deepseek_v3_bf16", batch=64, q_len=1, heads=128, d_latent=512, d_rope=64,
             page_size=64, seq_lens=("uniform", 1024, 8192), kv_dtype="bf16", q_dtype="bf16",
             out_dtype="bf16", sigma=0.5, scale=1.0 / math.sqrt(192.0), index=1),
    Workload("agentic_long_bf16", batch=8, q_len=1, heads=128, d_latent=512, d_rope=64,
             page_size=64, seq_lens=("uniform", 32768, 131072), kv_dtype="bf16", q_dtype="bf16",
             out_dtype="bf16", sigma=0.5, scale=1.0 / math.sqrt(192.0), shared_prefix=16384,
             num_splits=16, index=2),
    Workload("spec_decode_bf16", batch=256, q_len=4, heads=64, d_latent=512, d_rope=64,
             page_size=64, seq_lens=("fixed", (4096,) * 256), kv_dtype="bf16", q_dtype="bf16",
             out_dtype="bf16", sigma=0.5, scale=1.0 / math.sqrt(192.0), causal=True, index=3),
    Workload("fp8_kv", batch=128, q_len=1, heads=128, d_latent=512, d_rope=64, page_size=64,
             seq_lens=("uniform", 8192, 16384), kv_dtype="fp8", q_dtype="bf16", out_dtype="bf16",
             sigma=0.5, scale=1.0 / math.sqrt(192.0), index=4),
]


def workload(i):
    return WORKLOADS[i]


def _draw_seq_lens(w, rng):
    kind = w.seq_lens[0]
    if kind == "fixed":
        vals = np.asarray(w.seq_lens[1], dtype=np.int64)
        if vals.size != w.batch:
            vals = np.resize(vals, w.batch)
        return vals.astype(np.int32)
    lo, hi = w.seq_lens[1], w.seq_lens[2]
    return rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def make_inputs(w, seed=None, poison=True, seq_lens=None):
    """Draw one batch of inputs for workload ``w``.

    Returns a dict of host numpy arrays:
      seq_lens int32 [B]; page_table int32 [B, MP];
      kv  [NP, P, D]  (float32, uint16 bf16 bits, or uint8 e4m3 codes);
      kv_scales float32 [NP, P] (fp8 only, else None);
      q_abs [B, T, H, Dc], q_rope [B, T, H, Dr] (float32 or uint16 bf16 bits);
      scale float32; plus the workload itself under "workload".
    ``seq_lens`` overrides the drawn lengths (the draw still happens so the
    rest of the stream is unchanged).
    """
    if seed is None:
        seed = 1000 + max(w.index, 0)
    rng = np.random.default_rng(seed)
    B, T, H, Dc, Dr, P = w.batch, w.q_len, w.heads, w.d_latent, w.d_rope, w.page_size
    D = Dc + Dr
    L = _draw_seq_lens(w, rng)
    if seq_lens is not None:
        L = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    MP = w.max_pages
    if int(L.max(initial=0)) > MP * P:
        raise ValueError("seq_len exceeds the page table")
    shared_pages = w.shared_prefix // P
    if w.shared_prefix % P:
        raise ValueError("shared prefix must be page aligned")
    if shared_pages and int(L.min()) < w.shared_prefix:
        raise ValueError("every request must contain the shared prefix")
    npages = [(-(-int(l) // P)) for l in L]
    private = [n - shared_pages for n in npages]
    n_unique = shared_pages + int(sum(private))
    NP = n_unique + w.decoys
    perm = rng.permutation(NP).astype(np.int32)

    page_table = np.full((B, MP), -1, dtype=np.int32)
    logical = shared_pages
    for b in range(B):
        page_table[b, :shared_pages] = perm[:shared_pages]
        page_table[b, shared_pages:npages[b]] = perm[logical:logical + private[b]]
        logical += private[b]

    vals = rng.standard_normal((n_unique, P, D), dtype=np.float32)
    vals *= np.float32(w.sigma)
    # slots past the end of each request's last (private) page
    tail = []
    logical = shared_pages
    for b in range(B):
        if private[b] > 0:
            used = int(L[b]) - (npages[b] - 1) * P
            tail.append((logical + private[b] - 1, used))
        logical += private[b]

    kv_scales = None
    if w.kv_dtype == "f32":
        kv = np.empty((NP, P, D), dtype=np.float32)
        kv[perm[:n_unique]] = vals
        if poison:
            kv[perm[n_unique:]] = np.nan
            for u, used in tail:
                kv[perm[u], used:] = np.nan
        else:
            kv[perm[n_unique:]] = 0
    elif w.kv_dtype == "bf16":
        kv = np.empty((NP, P, D), dtype=np.uint16)
        kv[perm[:n_unique]] = f32_to_bf16_bits_blocked(vals)
        fill = BF16_NAN_BITS if poison else 0
        kv[perm[n_unique:]] = fill
        if poison:
            for u, used in tail:
                kv[perm[u], used:] = fill
    elif w.kv_dtype == "fp8":
        codes, scales = quantize_rows_e4m3(vals)
        kv = np.empty((NP, P, D), dtype=np.uint8)
        kv_scales = np.empty((NP, P), dtype=np.float32)
        kv[perm[:n_unique]] = codes
        kv_scales[perm[:n_unique]] = scales
        if poison:
            kv[perm[n_unique:]] = E4M3_NAN_CODE
            kv_scales[perm[n_unique:]] = np.nan
            for u, used in tail:
                kv[perm[u], used:] = E4M3_NAN_CODE
                kv_scales[perm[u], used:] = np.nan
        else:
            kv[perm[n_unique:]] = 0
            kv_scales[perm[n_unique:]] = 1.0
    else:
        raise ValueError(w.kv_dtype)
    del vals

    q_abs = rng.standard_normal((B, T, H, Dc), dtype=np.float32) * np.float32(w.sigma)
    q_rope = rng.standard_normal((B, T, H, Dr), dtype=np.float32) * np.float32(w.sigma)
    if w.q_dtype == "bf16":
        q_abs = f32_to_bf16_bits(q_abs)
        q_rope = f32_to_bf16_bits(q_rope)
    elif w.q_dtype != "f32":
        raise ValueError(w.q_dtype)
    return {
        "workload": w, "seq_lens": L, "page_table": page_table, "kv": kv,
        "kv_scales": kv_scales, "q_abs": q_abs, "q_rope": q_rope,
        "scale": np.float32(w.scale), "num_pages": NP,
    }


def chunk_count_hint(w):
    """Number of page-aligned chunks a request of max length is cut into when splits are forced."""
    return w.num_splits


# Shapes of the per-head projections on either side of the attention for the
# DeepSeek-style workloads: d_nope = 128 (the score scale 1/sqrt(192) covers
# 128 non-rope + 64 rope query dims) and d_v = d_nope.
PROJ_D_NOPE = 128
PROJ_D_V = 128


def make_projection_inputs(M, G, K, N, seed, sigma_x=0.5):
    """Seeded bf16 inputs of one per-head projection: x [M, G, K] ~ N(0,1) * sigma_x
    and random synthetic weights w [G, N, K] ~ N(0,1) / sqrt(K), drawn in fp32
    (x first, then w) and rounded once to bf16.  Returns (x_bits, w_bits) as
    uint16 arrays of bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, G, K), dtype=np.float32) * np.float32(sigma_x)).astype(np.float32)
    w = (rng.standard_normal((G, N, K), dtype=np.float32) * np.float32(1.0 / math.sqrt(K))).astype(np.float32)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)
