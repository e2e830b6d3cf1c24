"""GPU parity of the per-head projection (mla_project) against the oracle.

Inputs are bf16 (exact in fp64), so the oracle's fp64 result is the exact
value.  fp32 outputs: every bf16 x bf16 product is exact in fp32 and the K
products are summed in fp32, so |out - exact| <= K * 2^-24 * sum_k |w x|
(the standard bound for K-term recursive summation, with margin for the order
the hardware picks).  bf16 outputs add one rounding to nearest:
<= 2^-8 |exact| more (8 significant bits); they must also meet the decode's bf16 tolerance
(max-abs 2e-2, mean-relative 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_attention_02_amd as m
    m.library()
    return m


def _bf16_tensor(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def _case(M, G, K, N, seed):
    xb, wb = synth.make_projection_inputs(M, G, K, N, seed)
    x = synth.bf16_bits_to_f32(xb).astype(np.float64)
    w = synth.bf16_bits_to_f32(wb).astype(np.float64)
    return xb, wb, x, w


def _check(got, x, w, rows, out_dtype):
    """got [len(rows), G, N] from the GPU; the oracle on the sampled rows."""
    xs = x[rows]
    ref = oracle.project(xs, w)
    mag = oracle.project(np.abs(xs), np.abs(w))           # sum_k |w x| per output
    K = x.shape[2]
    bound = K * 2.0 ** -24 * mag + 1e-30
    if out_dtype == torch.bfloat16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), (err - bound).max()
    if out_dtype == torch.bfloat16:
        assert err.max() <= 2e-2
        assert err.sum() <= 1e-2 * np.abs(ref).sum()


CASES = [
    # (M, G, K, N): ragged m and n tiles, k = 8 (one piece), k with a half-chunk
    # tail, k shorter than one chunk per wave, both DeepSeek-side k/n roles;
    # k not a multiple of 64 takes the register-direct form
    (5, 3, 64, 72),
    (37, 4, 128, 512),
    (33, 2, 512, 128),
    (1, 1, 8, 8),
    (70, 3, 520, 40),
    (32, 5, 40, 64),
    (64, 2, 1056, 136),
    # the staged form (k a multiple of 64): tails in m and n, n below one tile;
    # more than 64 rows with k <= 128 take 128-row tiles
    (3, 2, 192, 8),
    (130, 3, 640, 200),
    (200, 2, 128, 72),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,G,K,N", CASES)
def test_project_matches_oracle(mla, M, G, K, N, out_dtype):
    xb, wb, x, w = _case(M, G, K, N, seed=M * 7 + K + N)
    out = mla.project(_bf16_tensor(xb).cuda(), _bf16_tensor(wb).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(out.float().cpu().numpy().astype(np.float64), x, w, np.arange(M), out_dtype)


@pytest.mark.parametrize("side", ["query", "value"])
@pytest.mark.parametrize("M,G", [(64, 128), (1024, 64)], ids=["deepseek_b64", "spec_b256_t4"])
def test_project_full_size_sampled_rows(mla, side, M, G):
    """DeepSeek-style sizes (d_nope = d_v = 128, d_latent = 512) in the launch
    the benchmark times; the oracle checks every output of 24 sampled rows."""
    K, N = (synth.PROJ_D_NOPE, 512) if side == "query" else (512, synth.PROJ_D_V)
    xb, wb, x, w = _case(M, G, K, N, seed=99 + M + K)
    out = mla.project(_bf16_tensor(xb).cuda(), _bf16_tensor(wb).cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(M, size=24, replace=False))
    rows[0], rows[-1] = 0, M - 1
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    _check(got, x, w, rows, torch.bfloat16)


def test_project_no_rows_and_rejected_shapes(mla):
    dev = torch.device("cuda:0")
    w = torch.zeros((2, 16, 16), dtype=torch.bfloat16, device=dev)
    out = mla.project(torch.zeros((0, 2, 16), dtype=torch.bfloat16, device=dev), w)
    assert out.shape == (0, 2, 16)
    with pytest.raises(mla.MLAError) as e:                     # in_dim not a multiple of 8
        mla.project(torch.zeros((3, 2, 12), dtype=torch.bfloat16, device=dev),
                    torch.zeros((2, 16, 12), dtype=torch.bfloat16, device=dev))
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED
    base = torch.zeros((3 * 2 * 16 + 1,), dtype=torch.bfloat16, device=dev)
    x = base[1:].view(3, 2, 16)                                 # 2-byte aligned only
    with pytest.raises(mla.MLAError) as e:
        mla.project(x, w)
    assert e.value.status == mla.MLA_ERR_INVALID_ARG


def test_project_chain_around_decode_matches_oracle(mla):
    """q_nope -> mla_project -> mla_decode -> mla_project, against the oracle's
    projections and attention on the same inputs (DeepSeek-shaped, small batch)."""
    from helpers import small, to_device
    w_ = small(1, batch=3, seq_lens=("uniform", 70, 200))
    inp = dict(synth.make_inputs(w_, seed=17))
    B, H, Dc = w_.batch, w_.heads, w_.d_latent
    qb, wkb = synth.make_projection_inputs(B, H, synth.PROJ_D_NOPE, Dc, seed=18)
    _, wvb = synth.make_projection_inputs(1, H, Dc, synth.PROJ_D_V, seed=19)
    q_nope = synth.bf16_bits_to_f32(qb).astype(np.float64)
    w_uk_t = synth.bf16_bits_to_f32(wkb).astype(np.float64)
    w_uv = synth.bf16_bits_to_f32(wvb).astype(np.float64)
    dev = torch.device("cuda:0")
    q_abs = mla.project(_bf16_tensor(qb).to(dev), _bf16_tensor(wkb).to(dev))
    torch.cuda.synchronize()
    # query side against the oracle's projection
    got_q = q_abs.float().cpu().numpy().astype(np.float64)
    _check(got_q, q_nope, w_uk_t, np.arange(B), torch.bfloat16)
    # the oracle attends with the bf16 query the decode reads
    inp["q_abs"] = q_abs.cpu().view(torch.int16).numpy().view(np.uint16).reshape(B, 1, H, Dc)
    o_ref, _ = oracle.attend(inp)
    v_ref = oracle.project(o_ref.reshape(B, H, Dc), w_uv)
    d = to_device(inp)
    d["q_abs"] = q_abs.view(B, 1, H, Dc)
    o, _ = mla.decode(d["q_abs"], d["q_rope"], d["kv"], d["page_table"], d["seq_lens"],
                      float(inp["scale"]), kv_scales=d["kv_scales"], max_seq_len=w_.max_seq_len,
                      out_dtype=torch.bfloat16)
    v = mla.project(o.reshape(B, H, Dc), _bf16_tensor(wvb).to(dev))
    torch.cuda.synchronize()
    got = v.float().cpu().numpy().astype(np.float64)
    assert np.abs(got - v_ref).max() <= 2e-2
    assert np.abs(got - v_ref).sum() <= 1e-2 * np.abs(v_ref).sum()
