"""GPU parity of the greedy chain verification (mla_verify_greedy) against the
oracle: argmax, accepted lengths and emitted tokens must be identical
(integer results; the argmax compares the stored logit values exactly)."""
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


def _inputs(seed, B, T, V, dtype):
    rng = np.random.default_rng(seed)
    lg = torch.from_numpy(rng.standard_normal((B, T, V)).astype(np.float32))
    if dtype == "bf16":
        lg = lg.to(torch.bfloat16)                 # frequent exact ties
    vals = lg.float().numpy()
    if B > 2:
        r = vals[1, 0]
        r[[5, V - 2]] = r.max() + 1.0               # a planted tie: the smaller index wins
        vals[2, T - 1, ::3] = np.nan                 # NaN never wins
        if B > 3:
            vals[3, 0, :] = -np.inf                  # all -inf: the first index
        if B > 4:
            vals[4, 0, :] = np.nan                   # all NaN: 0
        lg = torch.from_numpy(vals).to(lg.dtype)
        vals = lg.float().numpy()
    p = np.nan_to_num(vals, nan=-np.inf).argmax(axis=2)
    draft = p[:, : T - 1].astype(np.int32).copy()
    for b in range(B):                               # a mismatch planted at k = b mod T
        k = b % T
        if k < T - 1:
            draft[b, k] = (p[b, k] + 1) % V
    return lg, vals, draft


@pytest.mark.parametrize("dtype,V", [("bf16", 129280), ("bf16", 1001), ("f32", 1000), ("f32", 1001)])
@pytest.mark.parametrize("T", [1, 4])
def test_verify_equals_oracle(mla, dtype, V, T):
    lg, vals, draft = _inputs(41 + V + T, B=12, T=T, V=V, dtype=dtype)
    am, n, out = mla.verify_greedy(lg.cuda(), torch.from_numpy(draft).cuda() if T > 1 else None)
    torch.cuda.synchronize()
    ram, rn, rout = oracle.verify_greedy(vals, draft)
    assert np.array_equal(am.cpu().numpy(), ram)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(out.cpu().numpy(), rout)
