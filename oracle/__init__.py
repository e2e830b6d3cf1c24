"""CPU oracle for MLA decode over a paged latent KV cache (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
fp64, built by ``oracle/build.py`` with gcc) and never touches the GPU path:
the two share no code, and inputs come from the ``synth`` generator only.

The computation is documented in ``mla_oracle.c``; in short, for every query
row it forms z_j = scale * (q_abs . c_j + q_rope . k_j) over the visible
tokens, takes an exact three-pass softmax and returns o = sum_j p_j c_j and
lse = m + ln l in fp64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ORC_F32, ORC_BF16, ORC_E4M3 = 0, 1, 2
_DT = {"f32": ORC_F32, "bf16": ORC_BF16, "fp8": ORC_E4M3}
_ERR = {-1: "bad argument", -2: "page id out of range", -3: "out of memory"}


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_heads", "d_latent", "d_rope", "page_size", "num_pages",
        "max_pages_per_seq", "q_dtype", "kv_dtype", "causal")]


_lib = None


def load(rebuild=False):
    """Load liboracle.so, building it first if it is missing (or on request)."""
    global _lib
    if _lib is not None and not rebuild:
        return _lib
    if rebuild or not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.orc_attend.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, ctypes.c_float, i32,
                               P, P, P, P, P, i32]
    lib.orc_attend.restype = ctypes.c_int
    lib.orc_probs.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, ctypes.c_float, i32,
                              i32, i32, P]
    lib.orc_probs.restype = ctypes.c_int
    lib.orc_chunk_bounds.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.orc_chunk_bounds.restype = None
    lib.orc_combine.argtypes = [i32, i32, i32, P, P, P, P]
    lib.orc_combine.restype = ctypes.c_int
    lib.orc_gather_rows.argtypes = [ctypes.POINTER(Problem), P, P, i32, P, P, P]
    lib.orc_gather_rows.restype = ctypes.c_int
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_append_rows.argtypes = [i32, i32, i32, P, P, i32, i32, i32, P, i32, P, P]
    lib.orc_append_rows.restype = ctypes.c_int
    lib.orc_project.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.orc_project.restype = ctypes.c_int
    lib.orc_verify_greedy.argtypes = [i32, i32, i32, P, P, P, P, P]
    lib.orc_verify_greedy.restype = ctypes.c_int
    lib.orc_e4m3_code.argtypes = [ctypes.c_float]
    lib.orc_e4m3_code.restype = ctypes.c_uint8
    lib.orc_bf16_bits.argtypes = [ctypes.c_float]
    lib.orc_bf16_bits.restype = ctypes.c_uint16
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what}: {_ERR.get(rc, rc)}")


def problem(inp):
    w = inp["workload"]
    pt = inp["page_table"]
    return Problem(w.batch, w.q_len, w.heads, w.d_latent, w.d_rope, w.page_size,
                   int(inp["kv"].shape[0]), int(pt.shape[1]), _DT[w.q_dtype], _DT[w.kv_dtype],
                   1 if w.causal else 0)


def _arrays(inp):
    c = np.ascontiguousarray
    kv_scales = inp.get("kv_scales")
    return (c(inp["q_abs"]), c(inp["q_rope"]), c(inp["kv"]),
            None if kv_scales is None else c(kv_scales, dtype=np.float32),
            c(inp["page_table"], dtype=np.int32), c(inp["seq_lens"], dtype=np.int32))


def attend(inp, req_ids=None, tok_begin=None, tok_end=None, threads=0):
    """fp64 outputs for the listed requests: (o [n, T, H, Dc], lse [n, T, H])."""
    lib = load()
    w = inp["workload"]
    pr = problem(inp)
    qa, qr, kv, sc, pt, sl = _arrays(inp)
    if req_ids is None:
        n = w.batch
        rid = None
    else:
        rid = np.ascontiguousarray(req_ids, dtype=np.int32)
        n = int(rid.size)
    tb = None if tok_begin is None else np.ascontiguousarray(tok_begin, dtype=np.int32)
    te = None if tok_end is None else np.ascontiguousarray(tok_end, dtype=np.int32)
    out = np.zeros((n, w.q_len, w.heads, w.d_latent), dtype=np.float64)
    lse = np.zeros((n, w.q_len, w.heads), dtype=np.float64)
    rc = lib.orc_attend(ctypes.byref(pr), _ptr(qa), _ptr(qr), _ptr(kv), _ptr(sc), _ptr(pt),
                        _ptr(sl), ctypes.c_float(float(inp["scale"])), n, _ptr(rid), _ptr(tb),
                        _ptr(te), _ptr(out), _ptr(lse), int(threads))
    _check(rc, "attend")
    return out, lse


def probs(inp, b, t, h):
    """Softmax probabilities of one query row over its request's tokens (fp64 [L_b])."""
    lib = load()
    pr = problem(inp)
    qa, qr, kv, sc, pt, sl = _arrays(inp)
    p = np.zeros(max(int(sl[b]), 1), dtype=np.float64)
    rc = lib.orc_probs(ctypes.byref(pr), _ptr(qa), _ptr(qr), _ptr(kv), _ptr(sc), _ptr(pt),
                       _ptr(sl), ctypes.c_float(float(inp["scale"])), int(b), int(t), int(h),
                       _ptr(p))
    _check(rc, "probs")
    return p[:int(sl[b])]


def chunk_bounds(L, S, P, k):
    lib = load()
    b = ctypes.c_int32()
    e = ctypes.c_int32()
    lib.orc_chunk_bounds(int(L), int(S), int(P), int(k), ctypes.byref(b), ctypes.byref(e))
    return b.value, e.value


def combine(o_parts, lse_parts):
    """Merge chunk results: o_parts [n, S, Dc], lse_parts [n, S] -> (o [n, Dc], lse [n])."""
    lib = load()
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, S, Dc = o_parts.shape
    out = np.zeros((n, Dc), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    _check(lib.orc_combine(n, S, Dc, _ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse)),
           "combine")
    return out, lse


def split_attend(inp, S, req_ids=None, threads=0):
    """Per-chunk results for S page-aligned chunks: (o [n, S, T, H, Dc], lse [n, S, T, H])."""
    w = inp["workload"]
    sl = inp["seq_lens"]
    ids = np.arange(w.batch) if req_ids is None else np.asarray(req_ids)
    os_, ls_ = [], []
    for k in range(S):
        bounds = [chunk_bounds(int(sl[b]), S, w.page_size, k) for b in ids]
        o, l = attend(inp, ids, [x[0] for x in bounds], [x[1] for x in bounds], threads)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_, axis=1), np.stack(ls_, axis=1)


def gather_rows(inp, b, j):
    """Raw stored bytes of rows (b[i], j[i]): uint8 [n, D * element size]."""
    lib = load()
    pr = problem(inp)
    kv = np.ascontiguousarray(inp["kv"])
    pt = np.ascontiguousarray(inp["page_table"], dtype=np.int32)
    b = np.ascontiguousarray(b, dtype=np.int32)
    j = np.ascontiguousarray(j, dtype=np.int32)
    rb = kv.itemsize * kv.shape[-1]
    out = np.zeros((b.size, rb), dtype=np.uint8)
    _check(lib.orc_gather_rows(ctypes.byref(pr), _ptr(kv), _ptr(pt), int(b.size), _ptr(b),
                               _ptr(j), _ptr(out)), "gather_rows")
    return out


def bf16_value(bits):
    return load().orc_bf16_value(int(bits))


def e4m3_value(code):
    return load().orc_e4m3_value(int(code))


def max_threads():
    return load().orc_max_threads()


def append_rows(src, page_table, pos0, kv, kv_scales=None, dst="fp8"):
    """Paged KV append (see orc_append_rows): src [n_req, T, D] float32 exact
    source values; writes rows into kv [NP, P, D] (uint8 codes / uint16 bf16
    bits / float32) and, for fp8, per-token scales into kv_scales [NP, P]."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    n_req, T, D = src.shape
    NP, P = kv.shape[0], kv.shape[1]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    assert kv.flags.c_contiguous and (kv_scales is None or kv_scales.flags.c_contiguous)
    rc = load().orc_append_rows(n_req, T, D, _ptr(src), _ptr(pt), pt.shape[1], P, NP, _ptr(p0),
                                _DT[dst], _ptr(kv), None if kv_scales is None else _ptr(kv_scales))
    _check(rc, "orc_append_rows")


def e4m3_code(q):
    return int(load().orc_e4m3_code(float(q)))


def bf16_bits(v):
    return int(load().orc_bf16_bits(float(v)))


def verify_greedy(logits, draft):
    """Greedy linear-chain verification (see orc_verify_greedy).  logits
    [B, T, V] (any real dtype; compared as exact fp64 values), draft [B, T-1]
    int32.  Returns (argmax [B, T], accept_len [B], out_tokens [B, T])."""
    lg = np.ascontiguousarray(logits, dtype=np.float64)
    B, T, V = lg.shape
    d = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, max(T - 1, 0))
    am = np.zeros((B, T), dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, T), dtype=np.int32)
    _check(load().orc_verify_greedy(B, T, V, _ptr(lg), _ptr(d) if d.size else None, _ptr(am), _ptr(n),
                                    _ptr(out)), "orc_verify_greedy")
    return am, n, out


def project(x, w):
    """Per-head projection out[m, g, n] = sum_k w[g, n, k] x[m, g, k] in fp64
    (see orc_project).  x [M, G, K], w [G, N, K] (any real dtype, exact values)."""
    xx = np.ascontiguousarray(x, dtype=np.float64)
    ww = np.ascontiguousarray(w, dtype=np.float64)
    M, G, K = xx.shape
    G2, N, K2 = ww.shape
    assert G2 == G and K2 == K
    out = np.zeros((M, G, N), dtype=np.float64)
    _check(load().orc_project(M, G, K, N, _ptr(xx), _ptr(ww), _ptr(out)), "orc_project")
    return out
