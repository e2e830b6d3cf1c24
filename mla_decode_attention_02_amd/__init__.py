"""MI355X (gfx950) MLA decode over a paged, prefix-shared latent KV cache.

Thin Python binding over the C ABI in ``include/mla.h`` (libmla_decode.so,
built in-tree by ``mla_decode_attention_02_amd/build.py``).  This module only
marshals arguments: it checks dtypes, shapes and devices, allocates outputs
and workspace with torch when the caller does not pass them, and calls the
library on ``torch.cuda.current_stream()``.  Every step of the decode runs in
the library's HIP kernels; there is no other code path.  If the library is
missing, importing the binding still works but every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_DTYPE_F32, MLA_DTYPE_BF16, MLA_DTYPE_FP8_E4M3 = 0, 1, 2
MLA_OK = 0
MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE = -1, -2, -3
MLA_ERR_HIP, MLA_ERR_CHECK, MLA_ERR_SCRATCH = -4, -5, -6
STATIC_SCRATCH_BYTES = 72 << 20  # MLA_STATIC_SCRATCH_BYTES

EXPORTS = ("mla_num_splits", "mla_workspace_size", "mla_decode", "mla_decode_split",
           "mla_combine", "mla_balanced_workgroups",
           "mla_decode_split_balanced", "mla_combine_balanced", "mla_cascade_workspace_size",
           "mla_decode_cascade", "mla_append_kv", "mla_verify_greedy",
           "mla_project", "mla_gather_rows", "mla_stream_read",
           "mla_check_tables", "mla_decode_no_alloc", "mla_status_string")

BALANCED_ROWS = 128  # rows per unit of the balanced work list
BALANCED_START_COST = 4  # positions the balanced work list charges for starting a unit


class MLAError(RuntimeError):
    def __init__(self, what, status, message):
        super().__init__(f"{what}: {message} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ``mla_problem`` in include/mla.h."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_heads", "d_latent", "d_rope", "page_size", "num_pages",
        "max_pages_per_seq", "max_seq_len", "q_dtype", "kv_dtype", "out_dtype", "causal",
        "num_splits")]


_lib = None


def library():
    """The loaded libmla_decode.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mla_decode_attention_02_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PP = ctypes.POINTER(Problem)
    lib.mla_num_splits.argtypes = [PP, ctypes.POINTER(i32)]
    lib.mla_workspace_size.argtypes = [PP, ctypes.POINTER(sz)]
    lib.mla_decode.argtypes = [PP, P, P, P, P, P, P, ctypes.c_float, P, P, P, sz, P]
    lib.mla_decode_split.argtypes = [PP, P, P, P, P, P, P, ctypes.c_float, i32, P, P, P]
    lib.mla_combine.argtypes = [i32, i32, i32, i32, P, P, i32, P, P, P]
    lib.mla_balanced_workgroups.argtypes = [ctypes.POINTER(i32)]
    lib.mla_decode_split_balanced.argtypes = [PP, P, P, P, P, P, P, ctypes.c_float, i32, P, P, P,
                                              P, P, P]
    lib.mla_combine_balanced.argtypes = [PP, i32, P, P, P, P, P, P]
    lib.mla_cascade_workspace_size.argtypes = [PP, i32, ctypes.POINTER(sz)]
    lib.mla_decode_cascade.argtypes = [PP, P, P, P, P, P, P, ctypes.c_float, i32, P, P, P, sz, P]
    lib.mla_append_kv.argtypes = [PP, P, i32, P, P, P, P, P]
    lib.mla_verify_greedy.argtypes = [i32, i32, i32, P, i32, P, P, P, P, P]
    lib.mla_project.argtypes = [i32, i32, i32, i32, P, P, i32, P, P]
    lib.mla_gather_rows.argtypes = [PP, P, P, i32, P, P, P, P]
    lib.mla_stream_read.argtypes = [P, sz, P, i32, P]
    lib.mla_check_tables.argtypes = [PP, P, P]
    lib.mla_decode_no_alloc.argtypes = [PP, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status):
    return library().mla_status_string(int(status)).decode()


def _check(status, what):
    if status != MLA_OK:
        raise MLAError(what, status, status_string(status))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MLA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code):
    return {MLA_DTYPE_F32: torch.float32, MLA_DTYPE_BF16: torch.bfloat16}[code]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require(t, name, device, dtype=None, ndim=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def make_problem(q_abs, q_rope, kv_pages, page_table, *, causal=False, num_splits=0,
                 max_seq_len=0, out_dtype=None):
    """Build an ``mla_problem`` from tensor shapes (q_abs [B,T,H,Dc], kv_pages [NP,P,Dc+Dr])."""
    B, T, H, Dc = q_abs.shape
    Dr = q_rope.shape[-1] if q_rope is not None else 0
    NP, P, D = kv_pages.shape
    if D != Dc + Dr:
        raise ValueError(f"kv row width {D} != d_latent {Dc} + d_rope {Dr}")
    if out_dtype is None:
        out_dtype = torch.float32 if q_abs.dtype == torch.float32 else torch.bfloat16
    return Problem(B, T, H, Dc, Dr, P, NP, page_table.shape[1], int(max_seq_len),
                   _dtype_code(q_abs), _dtype_code(kv_pages), _dtype_code(torch.empty(0, dtype=out_dtype)),
                   1 if causal else 0, int(num_splits))


def num_splits(problem):
    s = ctypes.c_int32()
    _check(library().mla_num_splits(ctypes.byref(problem), ctypes.byref(s)), "mla_num_splits")
    return s.value


def workspace_size(problem):
    n = ctypes.c_size_t()
    _check(library().mla_workspace_size(ctypes.byref(problem), ctypes.byref(n)),
           "mla_workspace_size")
    return n.value


def _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales):
    dev = q_abs.device
    _require(q_abs, "q_abs", dev, ndim=4)
    if q_rope is not None:
        _require(q_rope, "q_rope", dev, dtype=q_abs.dtype, ndim=4)
        if q_rope.shape[:3] != q_abs.shape[:3]:
            raise ValueError("q_rope and q_abs disagree on [B, T, H]")
    _require(kv_pages, "kv_pages", dev, ndim=3)
    _require(page_table, "page_table", dev, dtype=torch.int32, ndim=2)
    _require(seq_lens, "seq_lens", dev, dtype=torch.int32, ndim=1)
    if page_table.shape[0] != q_abs.shape[0] or seq_lens.shape[0] != q_abs.shape[0]:
        raise ValueError("page_table / seq_lens batch size differs from q_abs")
    if kv_scales is not None:
        _require(kv_scales, "kv_scales", dev, dtype=torch.float32, ndim=2)
        if tuple(kv_scales.shape) != tuple(kv_pages.shape[:2]):
            raise ValueError("kv_scales must be [num_pages, page_size]")


def _outputs(pr, q_abs, out, lse):
    """The caller's out [B,T,H,Dc] and lse [B,T,H] after checks of device,
    dtype, contiguity and size, or new tensors where they are None."""
    dev = q_abs.device
    B, T, H, Dc = q_abs.shape
    if out is None:
        out = torch.empty((B, T, H, Dc), dtype=_torch_dtype(pr.out_dtype), device=dev)
    else:
        _require(out, "out", dev, dtype=_torch_dtype(pr.out_dtype))
        if out.numel() != B * T * H * Dc:
            raise ValueError(f"out must hold [B, T, H, Dc] = {(B, T, H, Dc)} elements")
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    else:
        _require(lse, "lse", dev, dtype=torch.float32)
        if lse.numel() != B * T * H:
            raise ValueError(f"lse must hold [B, T, H] = {(B, T, H)} elements")
    return out, lse


def decode(q_abs, q_rope, kv_pages, page_table, seq_lens, scale, *, kv_scales=None,
           causal=False, num_splits=0, max_seq_len=0, out=None, lse=None, workspace=None,
           out_dtype=None):
    """MLA decode (split stage + merge) through ``mla_decode``.  Returns (out, lse)."""
    _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales)
    pr = make_problem(q_abs, q_rope, kv_pages, page_table, causal=causal,
                      num_splits=num_splits, max_seq_len=max_seq_len, out_dtype=out_dtype)
    dev = q_abs.device
    out, lse = _outputs(pr, q_abs, out, lse)
    need = workspace_size(pr)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace is not None:
        _require(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().mla_decode(ctypes.byref(pr), _ptr(q_abs), _ptr(q_rope), _ptr(kv_pages),
                                _ptr(kv_scales), _ptr(page_table), _ptr(seq_lens),
                                ctypes.c_float(float(scale)), _ptr(out), _ptr(lse),
                                _ptr(workspace), ws_bytes, _stream()), "mla_decode")
    return out, lse


def decode_no_alloc(q_abs, q_rope, kv_pages, page_table, seq_lens, scale, *, kv_scales=None,
                    causal=False, num_splits=0, max_seq_len=0, out=None, lse=None, out_dtype=None):
    """mla_decode with the library's static device scratch as its workspace
    (``mla_decode_no_alloc``): no workspace is allocated for the call.
    Returns (out, lse); out/lse are allocated here only when not given."""
    _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales)
    pr = make_problem(q_abs, q_rope, kv_pages, page_table, causal=causal,
                      num_splits=num_splits, max_seq_len=max_seq_len, out_dtype=out_dtype)
    out, lse = _outputs(pr, q_abs, out, lse)
    _check(library().mla_decode_no_alloc(ctypes.byref(pr), _ptr(q_abs), _ptr(q_rope), _ptr(kv_pages),
                                         _ptr(kv_scales), _ptr(page_table), _ptr(seq_lens),
                                         ctypes.c_float(float(scale)), _ptr(out), _ptr(lse), _stream()),
           "mla_decode_no_alloc")
    return out, lse


def decode_cascade(q_abs, q_rope, kv_pages, page_table, seq_lens, scale, prefix_len, *, kv_scales=None,
                   causal=False, max_seq_len=0, out=None, lse=None, workspace=None, out_dtype=None):
    """Cascade decode over a shared prefix of prefix_len tokens (mla_decode_cascade).
    Returns (out, lse)."""
    _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales)
    pr = make_problem(q_abs, q_rope, kv_pages, page_table, causal=causal, max_seq_len=max_seq_len,
                      out_dtype=out_dtype)
    dev = q_abs.device
    out, lse = _outputs(pr, q_abs, out, lse)
    need = ctypes.c_size_t(0)
    _check(library().mla_cascade_workspace_size(ctypes.byref(pr), int(prefix_len), ctypes.byref(need)),
           "mla_cascade_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(1, need.value), dtype=torch.uint8, device=dev)
    else:
        _require(workspace, "workspace", dev)
    _check(library().mla_decode_cascade(ctypes.byref(pr), _ptr(q_abs), _ptr(q_rope), _ptr(kv_pages),
                                        _ptr(kv_scales), _ptr(page_table), _ptr(seq_lens),
                                        ctypes.c_float(float(scale)), int(prefix_len), _ptr(out), _ptr(lse),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream()),
           "mla_decode_cascade")
    return out, lse


def decode_split(q_abs, q_rope, kv_pages, page_table, seq_lens, scale, num_splits, *,
                 kv_scales=None, causal=False, partial_o=None, partial_lse=None):
    """Split stage only: returns (partial_o [B,S,T*H,Dc] fp32, partial_lse [B,S,T*H] fp32)."""
    _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales)
    pr = make_problem(q_abs, q_rope, kv_pages, page_table, causal=causal)
    dev = q_abs.device
    B, T, H, Dc = q_abs.shape
    S = int(num_splits)
    if partial_o is None:
        partial_o = torch.empty((B, S, T * H, Dc), dtype=torch.float32, device=dev)
    if partial_lse is None:
        partial_lse = torch.empty((B, S, T * H), dtype=torch.float32, device=dev)
    _require(partial_o, "partial_o", dev, dtype=torch.float32)
    _require(partial_lse, "partial_lse", dev, dtype=torch.float32)
    if partial_o.numel() < B * S * T * H * Dc or partial_lse.numel() < B * S * T * H:
        raise ValueError("partial buffers too small")
    _check(library().mla_decode_split(ctypes.byref(pr), _ptr(q_abs), _ptr(q_rope),
                                      _ptr(kv_pages), _ptr(kv_scales), _ptr(page_table),
                                      _ptr(seq_lens), ctypes.c_float(float(scale)), S,
                                      _ptr(partial_o), _ptr(partial_lse), _stream()),
           "mla_decode_split")
    return partial_o, partial_lse


def balanced_workgroups():
    """Workgroups of the balanced work list on the current device."""
    n = ctypes.c_int32(0)
    _check(library().mla_balanced_workgroups(ctypes.byref(n)), "mla_balanced_workgroups")
    return int(n.value)


def decode_split_balanced(problem, q_abs, q_rope, kv_pages, page_table, seq_lens, scale,
                          num_workgroups, tile_prefix, out, lse, slot_o, slot_lse, *,
                          kv_scales=None):
    """Split stage of the balanced work list: writes tile_prefix [U + 1], whole units
    to out/lse and other segments to slot_o [2 nw, 128, Dc] bf16 / slot_lse [2 nw, 128] fp32."""
    _validate(q_abs, q_rope, kv_pages, page_table, seq_lens, kv_scales)
    dev = q_abs.device
    nw = int(num_workgroups)
    _require(tile_prefix, "tile_prefix", dev, dtype=torch.int32)
    groups = -(-problem.q_len * problem.num_heads // BALANCED_ROWS)
    if tile_prefix.numel() < problem.batch * groups + 1:
        raise ValueError("tile_prefix too small")
    _require(out, "out", dev, dtype=_torch_dtype(problem.out_dtype))
    if lse is not None:  # the C ABI takes NULL: no lse output
        _require(lse, "lse", dev, dtype=torch.float32)
    _require(slot_o, "slot_o", dev, dtype=torch.bfloat16)
    _require(slot_lse, "slot_lse", dev, dtype=torch.float32)
    if (slot_o.numel() < 2 * nw * BALANCED_ROWS * problem.d_latent
            or slot_lse.numel() < 2 * nw * BALANCED_ROWS):
        raise ValueError("slot buffers too small")
    _check(library().mla_decode_split_balanced(
        ctypes.byref(problem), _ptr(q_abs), _ptr(q_rope), _ptr(kv_pages), _ptr(kv_scales),
        _ptr(page_table), _ptr(seq_lens), ctypes.c_float(float(scale)), nw, _ptr(tile_prefix),
        _ptr(out), _ptr(lse), _ptr(slot_o), _ptr(slot_lse), _stream()),
        "mla_decode_split_balanced")


def combine_balanced(problem, num_workgroups, tile_prefix, slot_o, slot_lse, out, lse):
    """Merge stage of the balanced work list into out/lse."""
    dev = out.device
    _require(tile_prefix, "tile_prefix", dev, dtype=torch.int32)
    _require(slot_o, "slot_o", dev, dtype=torch.bfloat16)
    _require(slot_lse, "slot_lse", dev, dtype=torch.float32)
    if lse is not None:  # the C ABI takes NULL: no lse output
        _require(lse, "lse", dev, dtype=torch.float32)
    _require(out, "out", dev, dtype=_torch_dtype(problem.out_dtype))
    nw = int(num_workgroups)
    groups = -(-problem.q_len * problem.num_heads // BALANCED_ROWS)
    if (tile_prefix.numel() < problem.batch * groups + 1
            or slot_o.numel() < 2 * nw * BALANCED_ROWS * problem.d_latent
            or slot_lse.numel() < 2 * nw * BALANCED_ROWS):
        raise ValueError("tile_prefix or slot buffers too small")
    rows = problem.batch * problem.q_len * problem.num_heads
    if out.numel() < rows * problem.d_latent or (lse is not None and lse.numel() < rows):
        raise ValueError("out or lse too small")
    _check(library().mla_combine_balanced(ctypes.byref(problem), int(num_workgroups),
                                          _ptr(tile_prefix), _ptr(slot_o), _ptr(slot_lse),
                                          _ptr(out), _ptr(lse), _stream()),
           "mla_combine_balanced")


def combine(partial_o, partial_lse, *, out_dtype=torch.bfloat16, out=None, lse=None):
    """Merge split partials: partial_o [B,S,R,Dc], partial_lse [B,S,R] -> (out [B,R,Dc], lse [B,R])."""
    dev = partial_o.device
    _require(partial_o, "partial_o", dev, dtype=torch.float32, ndim=4)
    _require(partial_lse, "partial_lse", dev, dtype=torch.float32, ndim=3)
    B, S, R, Dc = partial_o.shape
    if tuple(partial_lse.shape) != (B, S, R):
        raise ValueError("partial_lse must be [B, S, rows]")
    code = _dtype_code(torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((B, R, Dc), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, R), dtype=torch.float32, device=dev)
    _require(out, "out", dev, dtype=out_dtype)
    _require(lse, "lse", dev, dtype=torch.float32)
    _check(library().mla_combine(B, S, R, Dc, _ptr(partial_o), _ptr(partial_lse), code,
                                 _ptr(out), _ptr(lse), _stream()), "mla_combine")
    return out, lse


def append_kv(rows, page_table, positions, kv_pages, *, kv_scales=None, d_latent=None):
    """Paged KV append with packing through ``mla_append_kv``: rows [B, T, D]
    (float32 or bfloat16) into kv_pages [NP, P, D] (float32, bfloat16 or uint8
    E4M3 codes with kv_scales [NP, P] float32) at positions[b] + t."""
    dev = rows.device
    _require(rows, "rows", dev, ndim=3)
    _require(page_table, "page_table", dev, dtype=torch.int32, ndim=2)
    _require(positions, "positions", dev, dtype=torch.int32, ndim=1)
    _require(kv_pages, "kv_pages", dev, ndim=3)
    B, T, D = rows.shape
    NP, P, Dk = kv_pages.shape
    if Dk != D or page_table.shape[0] != B or positions.numel() != B:
        raise ValueError("inconsistent shapes")
    if (kv_scales is None) != (_dtype_code(kv_pages) != MLA_DTYPE_FP8_E4M3):
        raise ValueError("kv_scales goes with E4M3 pages only")
    if kv_scales is not None:
        _require(kv_scales, "kv_scales", dev, dtype=torch.float32)
    dl = D if d_latent is None else int(d_latent)
    pr = Problem(B, T, 1, dl, D - dl, P, NP, page_table.shape[1], 0, MLA_DTYPE_BF16,
                 _dtype_code(kv_pages), MLA_DTYPE_BF16, 0, 0)
    _check(library().mla_append_kv(ctypes.byref(pr), _ptr(rows), _dtype_code(rows), _ptr(page_table),
                                   _ptr(positions), _ptr(kv_pages), _ptr(kv_scales), _stream()),
           "mla_append_kv")


def verify_greedy(logits, draft=None):
    """Greedy linear-chain verification through ``mla_verify_greedy``: logits
    [B, T, V] (float32 or bfloat16), draft [B, T-1] int32.  Returns
    (argmax [B, T], accept_len [B], out_tokens [B, T]) int32 tensors."""
    dev = logits.device
    _require(logits, "logits", dev, ndim=3)
    B, T, V = logits.shape
    if T > 1:
        _require(draft, "draft", dev, dtype=torch.int32, ndim=2)
        if tuple(draft.shape) != (B, T - 1):
            raise ValueError("draft must be [B, T-1]")
    am = torch.empty((B, T), dtype=torch.int32, device=dev)
    n = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, T), dtype=torch.int32, device=dev)
    _check(library().mla_verify_greedy(B, T, V, _ptr(logits), _dtype_code(logits),
                                       _ptr(draft) if T > 1 else None, _ptr(am), _ptr(n), _ptr(out),
                                       _stream()), "mla_verify_greedy")
    return am, n, out


def project(x, w, *, out_dtype=torch.bfloat16, out=None):
    """Per-head projection through ``mla_project``: x [M, G, K] and w [G, N, K]
    bfloat16 -> out [M, G, N] with out[m, g, n] = sum_k w[g, n, k] x[m, g, k].
    Query side: x = q_nope, w = W_UK transposed per head ([G, d_latent, d_nope]);
    value side: x = the attention output, w = W_UV ([G, d_v, d_latent])."""
    dev = x.device
    _require(x, "x", dev, dtype=torch.bfloat16, ndim=3)
    _require(w, "w", dev, dtype=torch.bfloat16, ndim=3)
    M, G, K = x.shape
    if w.shape[0] != G or w.shape[2] != K:
        raise ValueError(f"w must be [{G}, N, {K}], got {tuple(w.shape)}")
    N = w.shape[1]
    if out is None:
        out = torch.empty((M, G, N), dtype=out_dtype, device=dev)
    else:
        _require(out, "out", dev, dtype=out_dtype, ndim=3)
        if tuple(out.shape) != (M, G, N):
            raise ValueError("out must be [M, G, N]")
    _check(library().mla_project(M, G, K, N, _ptr(x), _ptr(w), _dtype_code(out), _ptr(out), _stream()),
           "mla_project")
    return out


def gather_rows(kv_pages, page_table, req, tok, *, d_latent, d_rope=None):
    """Test hook: raw stored rows of (req[i], tok[i]) through the page table -> [n, D] (kv dtype)."""
    dev = kv_pages.device
    _require(kv_pages, "kv_pages", dev, ndim=3)
    _require(page_table, "page_table", dev, dtype=torch.int32, ndim=2)
    _require(req, "req", dev, dtype=torch.int32, ndim=1)
    _require(tok, "tok", dev, dtype=torch.int32, ndim=1)
    NP, P, D = kv_pages.shape
    if d_rope is None:
        d_rope = D - d_latent
    pr = Problem(page_table.shape[0], 1, 1, d_latent, d_rope, P, NP, page_table.shape[1], 0,
                 MLA_DTYPE_BF16, _dtype_code(kv_pages), MLA_DTYPE_BF16, 0, 0)
    out = torch.empty((req.numel(), D), dtype=kv_pages.dtype, device=dev)
    _check(library().mla_gather_rows(ctypes.byref(pr), _ptr(kv_pages), _ptr(page_table),
                                     req.numel(), _ptr(req), _ptr(tok), _ptr(out), _stream()),
           "mla_gather_rows")
    return out


def stream_read(src, sink):
    """Measurement hook: read the bytes of the contiguous device tensor `src`
    once; sink (int32 device tensor, one entry per workgroup) receives the
    XOR of the 32-bit words each workgroup read."""
    dev = src.device
    _require(src, "src", dev)
    _require(sink, "sink", dev, dtype=torch.int32, ndim=1)
    nbytes = src.numel() * src.element_size()
    _check(library().mla_stream_read(_ptr(src), nbytes, _ptr(sink), sink.numel(), _stream()),
           "mla_stream_read")
    return sink


def check_tables(problem, page_table_host, seq_lens_host):
    """Host-side table check (numpy int32 arrays); returns the status code."""
    import numpy as np
    pt = np.ascontiguousarray(page_table_host, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    return library().mla_check_tables(ctypes.byref(problem), pt.ctypes.data_as(ctypes.c_void_p),
                                      sl.ctypes.data_as(ctypes.c_void_p))
