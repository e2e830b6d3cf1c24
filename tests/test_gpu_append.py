"""GPU parity of the paged KV append with packing (mla_append_kv) against the
oracle: the whole cache, written slots and untouched ones, must be equal byte
for byte (codes, bf16 bits, fp32 values and per-row scales)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_attention_02_amd as m
    m.library()
    return m


def _rows(rng, B, T, D, src):
    x = (rng.standard_normal((B, T, D)) * 0.5).astype(np.float32)
    x[0, 0] = 0.0                                           # all-zero row
    x[0, -1, :8] = [-0.0, 1e-30, -1e-30, 1e-40, -3e-41, 7.0, -7.0, 0.0]
    if B > 1:
        x[1, 0] *= 1e30                                     # huge row
        x[1, -1] *= 1e-30                                   # tiny row
    if B > 2:
        x[2, 0, 3] = np.nan                                  # NaN element
    if src == "bf16":  # values the bf16 source can hold
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x


def _case(seed, B, T, D, P, MP, NP, src, dst):
    rng = np.random.default_rng(seed)
    x = _rows(rng, B, T, D, src)
    pt = rng.permutation(NP)[: B * MP].reshape(B, MP).astype(np.int32)
    pos = rng.integers(0, MP * P - T + 1, size=B).astype(np.int32)
    pos[0] = P - 1  # first request crosses a page boundary
    elt = {"fp8": np.uint8, "bf16": np.uint16, "f32": np.float32}[dst]
    kv = rng.integers(0, 255, size=(NP, P, D)).astype(np.uint8).view(np.uint8)
    kv = np.frombuffer(rng.bytes(NP * P * D * np.dtype(elt).itemsize), dtype=elt).reshape(NP, P, D).copy()
    sc = rng.standard_normal((NP, P)).astype(np.float32) if dst == "fp8" else None
    return x, pt, pos, kv, sc


def _run(mla, x, pt, pos, kv, sc, src, dst):
    dev = "cuda"
    # the bf16 source bits are made once, on the host, so that both sides see
    # the same bits (a device-side cast may pick another NaN payload)
    rows = torch.from_numpy(x)
    if src == "bf16":
        rows = rows.to(torch.bfloat16)
    rows = rows.to(dev)
    tdt = {"fp8": torch.uint8, "bf16": torch.bfloat16, "f32": torch.float32}[dst]
    kv_t = torch.from_numpy(kv.view(np.int16) if dst == "bf16" else kv).to(dev)
    if dst == "bf16":
        kv_t = kv_t.view(torch.bfloat16)
    sc_t = None if sc is None else torch.from_numpy(sc).to(dev)
    mla.append_kv(rows, torch.from_numpy(pt).to(dev), torch.from_numpy(pos).to(dev), kv_t,
                  kv_scales=sc_t)
    torch.cuda.synchronize()
    out = kv_t.view(torch.int16).cpu().numpy().view(np.uint16) if dst == "bf16" else kv_t.cpu().numpy()
    return out, None if sc_t is None else sc_t.cpu().numpy()


@pytest.mark.parametrize("src,dst", [("bf16", "fp8"), ("f32", "fp8"), ("f32", "bf16"),
                                     ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("D", [576, 80, 81])
def test_append_bitwise_equals_oracle(mla, src, dst, D):
    x, pt, pos, kv, sc = _case(31 + D, B=4, T=5, D=D, P=16, MP=6, NP=30, src=src, dst=dst)
    got, got_sc = _run(mla, x, pt, pos, kv.copy(), None if sc is None else sc.copy(), src, dst)
    ref, ref_sc = kv.copy(), None if sc is None else sc.copy()
    oracle.append_rows(x, pt, pos, ref, ref_sc, dst=dst)
    assert got.tobytes() == ref.tobytes()
    if sc is not None:
        assert got_sc.tobytes() == ref_sc.tobytes()


def test_append_decode_shaped_batch(mla):
    """A decode step's append at the FP8 workload's shape: 128 requests, one
    576-wide token each, 64-token pages."""
    x, pt, pos, kv, sc = _case(37, B=128, T=1, D=576, P=64, MP=8, NP=1100, src="bf16", dst="fp8")
    got, got_sc = _run(mla, x, pt, pos, kv.copy(), sc.copy(), "bf16", "fp8")
    ref, ref_sc = kv.copy(), sc.copy()
    oracle.append_rows(x, pt, pos, ref, ref_sc, dst="fp8")
    assert got.tobytes() == ref.tobytes() and got_sc.tobytes() == ref_sc.tobytes()


@pytest.mark.parametrize("B,T", [(3, 3), (1, 1), (2, 7)])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_append_fp8_partial_row_groups(mla, B, T, src):
    """Row counts that leave the last group of rows per wavefront partly empty
    (rows are packed several per wavefront); only the appended slots change."""
    x, pt, pos, kv, sc = _case(53 + 7 * B + T, B=B, T=T, D=576, P=16, MP=6, NP=30, src=src, dst="fp8")
    got, got_sc = _run(mla, x, pt, pos, kv.copy(), sc.copy(), src, "fp8")
    ref, ref_sc = kv.copy(), sc.copy()
    oracle.append_rows(x, pt, pos, ref, ref_sc, dst="fp8")
    assert got.tobytes() == ref.tobytes() and got_sc.tobytes() == ref_sc.tobytes()
