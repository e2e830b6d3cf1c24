"""Pins for the CPU oracle: each check ties it to something other than itself.

* absorption identity: attention over the latent rows with the key
  up-projection folded into the query equals explicit multi-head attention
  over decompressed keys/values (numpy, independent gather), after applying
  the value up-projection to the oracle's latent output;
* a pure-Python brute force with its own gather and its own format decoding
  (torch's bf16/e4m3 casts) on tiny inputs of every dtype;
* softmax rows sum to one; lse equals scipy's logsumexp;
* paged == contiguous storage and page-permutation invariance, bit for bit;
* split + merge == unsplit; empty splits; the chunk plan partitions [0, L);
* causal rows reduce to shorter single-token requests;
* special cases: L = 1, identical rows, q = 0, empty visible set;
* the FP8 E4M3 table and bf16 decoding against torch's CPU casts, and the
  pages' printed facts in tests/golden/page_facts.json.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    base = synth.workload(0)
    return base.with_(**kw) if kw else base


def small_ds(**kw):
    """A small DeepSeek-shaped bf16 case: several pages and a ragged tail."""
    w = synth.workload(1).with_(batch=3, heads=8, seq_lens=("fixed", (130, 64, 201)), decoys=3,
                                index=11)
    return w.with_(**kw) if kw else w


def stored_values(inp, which):
    """Exact values of a stored tensor, decoded independently of the oracle (torch casts)."""
    w = inp["workload"]
    a = inp[which]
    if which == "kv":
        if w.kv_dtype == "f32":
            return a.astype(np.float64)
        if w.kv_dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
        codes = torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
        return codes * inp["kv_scales"].astype(np.float64)[..., None]
    if w.q_dtype == "f32":
        return a.astype(np.float64)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()


def contiguous_rows(inp, b):
    """Rows of request b in logical order via numpy fancy indexing of the block table."""
    w = inp["workload"]
    L = int(inp["seq_lens"][b])
    kv = stored_values(inp, "kv")
    j = np.arange(L)
    pages = inp["page_table"][b, j // w.page_size]
    return kv[pages, j % w.page_size]


# ---------------------------------------------------------------- absorption

def _absorbed_case(w, seed):
    """Inputs whose q_abs = W_UK^T q_nope is exact in the storage dtype (dyadic values)."""
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(seed)
    dn = dv = 64
    H, T, Dc = w.heads, w.q_len, w.d_latent
    W_UK = rng.integers(-1, 2, size=(H, dn, Dc)).astype(np.float64) / 16.0
    W_UV = rng.standard_normal((H, dv, Dc))
    q_nope = rng.integers(-2, 3, size=(w.batch, T, H, dn)).astype(np.float64)
    q_abs = np.einsum("bthn,hnc->bthc", q_nope, W_UK)
    if w.q_dtype == "f32":
        stored = q_abs.astype(np.float32)
        assert np.array_equal(stored.astype(np.float64), q_abs)
        inp["q_abs"] = stored
    else:
        bits = synth.f32_to_bf16_bits(q_abs.astype(np.float32))
        back = synth.bf16_bits_to_f32(bits).astype(np.float64)
        assert np.array_equal(back, q_abs), "q_abs must be exact in bf16 for this pin"
        inp["q_abs"] = bits
    return inp, W_UK, W_UV, q_nope


def _expanded_mha(inp, W_UK, W_UV, q_nope):
    """Plain multi-head attention over decompressed K = [W_UK c ; k] and V = W_UV c."""
    w = inp["workload"]
    Dc = w.d_latent
    q_rope = stored_values(inp, "q_rope")
    out = np.zeros((w.batch, w.q_len, w.heads, W_UV.shape[1]))
    for b in range(w.batch):
        rows = contiguous_rows(inp, b)
        L = rows.shape[0]
        c, k = rows[:, :Dc], rows[:, Dc:]
        for h in range(w.heads):
            K = np.concatenate([c @ W_UK[h].T, k], axis=1)        # [L, dn + Dr]
            V = c @ W_UV[h].T                                     # [L, dv]
            for t in range(w.q_len):
                nvis = L - w.q_len + 1 + t if w.causal else L
                Q = np.concatenate([q_nope[b, t, h], q_rope[b, t, h]])
                s = (K[:nvis] @ Q) * float(inp["scale"])
                p = scipy.special.softmax(s)
                out[b, t, h] = p @ V[:nvis]
    return out


@pytest.mark.parametrize("w", [tiny(), small_ds(), small_ds(q_len=3, causal=True, heads=4)],
                         ids=["tiny_f32", "ds_bf16", "ds_bf16_causal"])
def test_absorption_identity_vs_expanded_mha(w):
    inp, W_UK, W_UV, q_nope = _absorbed_case(w, seed=7)
    o, _ = oracle.attend(inp)
    got = np.einsum("hvc,bthc->bthv", W_UV, o)
    ref = _expanded_mha(inp, W_UK, W_UV, q_nope)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= 1e-10, err


def test_absorption_identity_catches_rope_in_value():
    """Negative control: treating the whole 576-wide row as the value breaks the identity."""
    w = small_ds(batch=1, heads=2)
    inp, W_UK, W_UV, q_nope = _absorbed_case(w, seed=3)
    ref = _expanded_mha(inp, W_UK, W_UV, q_nope)
    o, _ = oracle.attend(inp)
    rows = contiguous_rows(inp, 0)
    shifted = o.copy()
    shifted[0, 0, :, :w.d_rope] += 1e-3 * rows[:, w.d_latent:].mean(axis=0)
    got = np.einsum("hvc,bthc->bthv", W_UV, shifted)
    assert np.abs(got - ref).max() / np.abs(ref).max() > 1e-8


# --------------------------------------------------------------- brute force

def _brute(inp):
    """Pure-Python loops; its own gather and decoding (via torch casts)."""
    w = inp["workload"]
    kv = stored_values(inp, "kv")
    qa = stored_values(inp, "q_abs")
    qr = stored_values(inp, "q_rope")
    sc = float(inp["scale"])
    P, Dc = w.page_size, w.d_latent
    o = np.zeros((w.batch, w.q_len, w.heads, Dc))
    lse = np.full((w.batch, w.q_len, w.heads), -math.inf)
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        for t in range(w.q_len):
            n = L - w.q_len + 1 + t if w.causal else L
            for h in range(w.heads):
                zs, rows = [], []
                for j in range(max(n, 0)):
                    row = kv[inp["page_table"][b][j // P]][j % P]
                    z = 0.0
                    for d in range(Dc):
                        z += qa[b, t, h, d] * row[d]
                    for e in range(w.d_rope):
                        z += qr[b, t, h, e] * row[Dc + e]
                    zs.append(sc * z)
                    rows.append(row)
                if not zs:
                    continue
                m = max(zs)
                ws = [math.exp(z - m) for z in zs]
                tot = math.fsum(ws)
                for wj, row in zip(ws, rows):
                    for d in range(Dc):
                        o[b, t, h, d] += (wj / tot) * row[d]
                lse[b, t, h] = m + math.log(tot)
    return o, lse


@pytest.mark.parametrize("kv_dtype,q_dtype,causal,T", [
    ("f32", "f32", False, 1), ("bf16", "bf16", False, 1), ("fp8", "bf16", False, 1),
    ("bf16", "bf16", True, 3), ("fp8", "bf16", True, 2)])
def test_bruteforce_python_loops(kv_dtype, q_dtype, causal, T):
    w = tiny(batch=3, heads=3, d_latent=8, d_rope=4, page_size=4, q_len=T, causal=causal,
             seq_lens=("fixed", (1, 9, 14)), kv_dtype=kv_dtype, q_dtype=q_dtype, decoys=2,
             scale=0.37, out_dtype="f32")
    inp = synth.make_inputs(w, seed=123)
    o, lse = oracle.attend(inp)
    ob, lb = _brute(inp)
    assert np.abs(o - ob).max() <= 1e-12 * max(1.0, np.abs(ob).max())
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lb[fin]).max() <= 1e-12 * max(1.0, np.abs(lb[fin]).max())


# ------------------------------------------------------- softmax invariants

def test_probabilities_sum_to_one_and_lse_matches_logsumexp():
    w = small_ds(q_len=2, causal=True)
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    for b in range(w.batch):
        rows = contiguous_rows(inp, b)
        L = rows.shape[0]
        for t in range(w.q_len):
            for h in (0, w.heads - 1):
                p = oracle.probs(inp, b, t, h)
                nvis = L - w.q_len + 1 + t
                assert abs(p.sum() - 1.0) <= 1e-12
                assert (p >= 0).all() and (p[nvis:] == 0).all()
                qa = stored_values(inp, "q_abs")[b, t, h]
                qr = stored_values(inp, "q_rope")[b, t, h]
                z = (rows[:nvis] @ np.concatenate([qa, qr])) * float(inp["scale"])
                assert abs(lse[b, t, h] - scipy.special.logsumexp(z)) <= 1e-12 * abs(lse[b, t, h])
                # the output is the probability-weighted latent rows
                assert np.abs(o[b, t, h] - p[:nvis] @ rows[:nvis, :w.d_latent]).max() <= 1e-12


# ----------------------------------------------------------------- paging

def _relayout(inp, table_fn, P_new):
    """Copy the stored rows into a new pool/page table built by table_fn."""
    w = inp["workload"]
    B = w.batch
    L = inp["seq_lens"]
    kv = inp["kv"]
    sc = inp["kv_scales"]
    MPn = max(1, -(-int(L.max()) // P_new))
    npages = [-(-int(l) // P_new) for l in L]
    total = sum(npages)
    order = table_fn(total)
    kvn = np.zeros((total, P_new) + kv.shape[2:], dtype=kv.dtype)
    scn = None if sc is None else np.ones((total, P_new), dtype=np.float32)
    pt = np.full((B, MPn), -1, dtype=np.int32)
    u = 0
    for b in range(B):
        for e in range(npages[b]):
            phys = int(order[u])
            pt[b, e] = phys
            for s in range(P_new):
                j = e * P_new + s
                if j >= L[b]:
                    break
                op = inp["page_table"][b, j // w.page_size]
                kvn[phys, s] = kv[op, j % w.page_size]
                if sc is not None:
                    scn[phys, s] = sc[op, j % w.page_size]
            u += 1
    out = dict(inp)
    out.update(kv=kvn, kv_scales=scn, page_table=pt,
               workload=w.with_(page_size=P_new, seq_lens=("fixed", tuple(int(x) for x in L))))
    return out


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "f32"])
def test_paged_equals_contiguous_bitwise(kv_dtype):
    w = small_ds(kv_dtype=kv_dtype, q_dtype="f32" if kv_dtype == "f32" else "bf16")
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    Lmax = int(inp["seq_lens"].max())
    contig = _relayout(inp, lambda n: np.arange(n), Lmax)   # one page per request, identity
    o2, lse2 = oracle.attend(contig)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_page_permutation_invariance_bitwise():
    w = small_ds(q_len=2, causal=True)
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    rng = np.random.default_rng(5)
    for P_new in (16, 64):
        other = _relayout(inp, lambda n: rng.permutation(n), P_new)
        o2, lse2 = oracle.attend(other)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_bad_page_id_is_rejected():
    inp = synth.make_inputs(tiny())
    inp["page_table"] = inp["page_table"].copy()
    inp["page_table"][0, 0] = inp["num_pages"]
    with pytest.raises(RuntimeError, match="page id"):
        oracle.attend(inp)


def test_gather_rows_matches_block_table_indexing():
    for w in (tiny(), small_ds(), small_ds(kv_dtype="fp8")):
        inp = synth.make_inputs(w)
        b = np.repeat(np.arange(w.batch), 5)
        j = np.concatenate([np.linspace(0, l - 1, 5).astype(int) for l in inp["seq_lens"]])
        got = oracle.gather_rows(inp, b, j)
        kv = inp["kv"]
        ref = np.stack([kv[inp["page_table"][bb, jj // w.page_size], jj % w.page_size]
                        for bb, jj in zip(b, j)])
        assert np.array_equal(got, ref.reshape(len(b), -1).view(np.uint8))


# ------------------------------------------------------------ split-KV merge

@pytest.mark.parametrize("L,S,P", [(100, 4, 16), (37, 16, 16), (0, 3, 64), (64, 1, 64),
                                   (8192, 16, 64), (4097, 7, 64), (1, 2, 64)])
def test_chunk_plan_partitions_sequence(L, S, P):
    spans = [oracle.chunk_bounds(L, S, P, k) for k in range(S)]
    assert spans[0][0] == 0 and spans[-1][1] == L
    for (b0, e0), (b1, e1) in zip(spans, spans[1:]):
        assert e0 == b1
    for b0, e0 in spans:
        assert 0 <= b0 <= e0 <= L
        assert b0 % P == 0 or b0 == L
    C = P * math.ceil(math.ceil(L / S) / P)
    assert spans == [(min(k * C, L), min((k + 1) * C, L)) for k in range(S)]


@pytest.mark.parametrize("S", [1, 2, 3, 16])
def test_split_and_merge_equals_unsplit(S):
    w = small_ds(q_len=2, causal=True, page_size=16)
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    op, lp = oracle.split_attend(inp, S)
    n, S_, T, H, Dc = op.shape
    rows_o = op.transpose(0, 2, 3, 1, 4).reshape(n * T * H, S, Dc)
    rows_l = lp.transpose(0, 2, 3, 1).reshape(n * T * H, S)
    m, ml = oracle.combine(rows_o, rows_l)
    assert np.abs(m.reshape(o.shape) - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(ml.reshape(lse.shape) - lse).max() <= 1e-12 * np.abs(lse).max()


def test_merge_with_empty_splits():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((3, 4, 8))
    lse = rng.standard_normal((3, 4))
    lse[0, 1:] = -np.inf                 # one live split: merge returns it unchanged
    lse[1, :] = -np.inf                  # nothing live: zeros and -inf
    m, ml = oracle.combine(o, lse)
    assert np.array_equal(m[0], o[0, 0]) and ml[0] == lse[0, 0]
    assert (m[1] == 0).all() and ml[1] == -np.inf
    w = np.exp(lse[2] - lse[2].max())
    assert np.abs(m[2] - (w @ o[2]) / w.sum()).max() <= 1e-14
    assert abs(ml[2] - scipy.special.logsumexp(lse[2])) <= 1e-14


# --------------------------------------------------------------- causal rows

def test_causal_row_equals_shorter_request():
    w = small_ds(q_len=4, causal=True, heads=4)
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    for t in range(w.q_len):
        sub = dict(inp)
        sub["seq_lens"] = inp["seq_lens"] - w.q_len + 1 + t
        sub["q_abs"] = np.ascontiguousarray(inp["q_abs"][:, t:t + 1])
        sub["q_rope"] = np.ascontiguousarray(inp["q_rope"][:, t:t + 1])
        sub["workload"] = w.with_(q_len=1, causal=False)
        o1, l1 = oracle.attend(sub)
        assert np.array_equal(o1[:, 0], o[:, t]) and np.array_equal(l1[:, 0], lse[:, t])


def test_empty_visible_sets():
    w = tiny(q_len=3, causal=True, seq_lens=("fixed", (0, 2)))
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    assert (o[0] == 0).all() and (lse[0] == -np.inf).all()     # L = 0
    assert (o[1, 0] == 0).all() and (lse[1, 0] == -np.inf).all()  # L - T + 1 + 0 = 0
    assert np.isfinite(lse[1, 1:]).all()


# ------------------------------------------------------------ special cases

def test_single_token_returns_its_latent_row_exactly():
    w = small_ds(seq_lens=("fixed", (1, 1, 1)))
    inp = synth.make_inputs(w)
    o, lse = oracle.attend(inp)
    for b in range(w.batch):
        c0 = contiguous_rows(inp, b)[0, :w.d_latent]
        assert np.array_equal(o[b, 0], np.broadcast_to(c0, o[b, 0].shape))


def test_identical_rows_and_zero_query():
    w = small_ds()
    inp = synth.make_inputs(w, poison=False)
    # zero query: uniform weights, output = mean of latent rows, lse = ln L
    inp0 = dict(inp, q_abs=np.zeros_like(inp["q_abs"]), q_rope=np.zeros_like(inp["q_rope"]))
    o, lse = oracle.attend(inp0)
    for b in range(w.batch):
        rows = contiguous_rows(inp, b)
        assert np.abs(o[b, 0] - rows[:, :w.d_latent].mean(axis=0)).max() <= 1e-13
        assert abs(lse[b, 0, 0] - math.log(rows.shape[0])) <= 1e-13
    # identical rows: output = that row whatever the query
    kv = inp["kv"].copy()
    kv[:] = kv[inp["page_table"][0, 0], 0]
    o, _ = oracle.attend(dict(inp, kv=kv))
    row = stored_values(dict(inp, kv=kv), "kv")[0, 0, :w.d_latent]
    assert np.abs(o - row).max() <= 1e-13


# ----------------------------------------------------------------- formats

def test_e4m3_table_against_torch_and_pages():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["fp8_formats"]["e4m3"]
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == facts["max_finite"]
    assert np.nanmin(got[got > 0]) == 2.0 ** -9
    assert len(np.unique(got[~nan & (got > 0)])) == 2 ** (facts["exponent_bits"] +
                                                           facts["mantissa_bits"]) - 2


def test_bf16_value_against_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and np.array_equal(got[~nan], ref[~nan])


def test_generator_encoders_match_torch_casts():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(200000) * 50, rng.uniform(-448, 448, 200000),
                        rng.standard_normal(10000) * 1e-3,
                        [0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 240.0, 232.0,
                         464.0 - 1e-3]]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.f32_to_e4m3_codes(x), ref)
    y = (rng.standard_normal(100000) * 10).astype(np.float32)
    refb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(y), refb)


def test_fp8_row_scale_is_absmax_over_448():
    x = (np.random.default_rng(2).standard_normal((50, 576)) * 0.5).astype(np.float32)
    x[3] = 0
    codes, scale = synth.quantize_rows_e4m3(x)
    ref = np.abs(x).max(axis=1) / np.float32(448)
    ref[3] = 1.0
    assert np.array_equal(scale, ref.astype(np.float32))
    back = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * scale[:, None]
    assert np.abs(back).max(axis=1)[np.arange(50) != 3].min() > 0
    assert (np.abs(back - x) <= np.abs(x) * 2 ** -4 + 2 ** -9 * scale[:, None]).all()


def test_workload_rows_follow_the_pages():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    for w in synth.WORKLOADS[1:]:
        assert w.d_latent == facts["latent_row"]["d_latent"]
        assert w.d_rope == facts["latent_row"]["d_rope"]
    assert synth.WORKLOADS[0].page_size == facts["paged_block"]["example_block_size"]


# ------------------------------------------------ paged KV append (FP8 pack)

def _e4m3_all_finite():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    keep = np.isfinite(vals)
    return codes[keep], vals[keep]


def test_e4m3_encoder_against_torch_cast():
    """The oracle's E4M3 encoder (from the format definition) against torch's
    float8_e4m3fn cast, an independent implementation: every finite code, every
    midpoint between neighbours (ties to even), one fp32 step either side of
    each midpoint, and random values in range."""
    codes, vals = _e4m3_all_finite()
    pos = np.unique(np.abs(vals))
    mids = (pos[:-1].astype(np.float64) + pos[1:]) / 2
    probe = [vals.astype(np.float32)]
    for m in mids:
        f = np.float32(m)
        probe.append(np.array([f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9)),
                               -f], dtype=np.float32))
    rng = np.random.default_rng(5)
    probe.append((rng.uniform(-448, 448, 4000)).astype(np.float32))
    probe.append((rng.standard_normal(4000) * np.float32(0.02)).astype(np.float32))
    x = np.concatenate(probe)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_code(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encoder_saturates_at_the_pages_maximum():
    fmt = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["fp8_formats"]["e4m3"]
    top = oracle.e4m3_code(fmt["max_finite"])
    assert oracle.e4m3_value(top) == fmt["max_finite"]
    for v in (448.5, 479.9, 480.0, 1e6, 3e38, float("inf")):
        assert oracle.e4m3_code(v) == top and oracle.e4m3_code(-v) == top | 0x80
    assert oracle.e4m3_code(float("nan")) & 0x7F == 0x7F


def test_bf16_encoder_against_torch_cast():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32),
                        rng.uniform(-1e30, 1e30, 500).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0, np.inf, -np.inf], dtype=np.float32)])
    # exact ties: bf16 values plus half a bf16 step
    b = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    x = np.concatenate([x, (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_bits(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _append_case(seed, n_req=3, T=2, D=80, P=16, MP=6, NP=24, dst="fp8"):
    rng = np.random.default_rng(seed)
    src = (rng.standard_normal((n_req, T, D)) * 0.5).astype(np.float32)
    src[0, 0] = 0.0                      # all-zero row: scale 1, codes of +0
    src[0, 1, :5] = [-0.0, 1e-30, -1e-30, 3.0, -3.0]
    pt = rng.permutation(NP)[: n_req * MP].reshape(n_req, MP).astype(np.int32)
    pos0 = np.array([0, 15, 2 * P + 7], dtype=np.int32)[:n_req]   # one append crosses a page
    elt = {"fp8": np.uint8, "bf16": np.uint16, "f32": np.float32}[dst]
    kv = np.full((NP, P, D), 0x5A if dst == "fp8" else 0x7FC0 if dst == "bf16" else np.nan, dtype=elt)
    sc = np.full((NP, P), np.nan, dtype=np.float32) if dst == "fp8" else None
    return src, pt, pos0, kv, sc


@pytest.mark.parametrize("dst", ["fp8", "bf16", "f32"])
def test_append_paged_equals_contiguous(dst):
    """Appending through a permuted page table and through one contiguous page
    per request store the same rows, read back by logical position with the
    (separately pinned) page-table gather; untouched slots keep their poison."""
    src, pt, pos0, kv, sc = _append_case(11, dst=dst)
    fresh = kv.copy()
    n_req, T, D = src.shape
    P, MP = kv.shape[1], pt.shape[1]
    oracle.append_rows(src, pt, pos0, kv, sc, dst=dst)
    kvc = np.zeros((n_req, MP * P, D), dtype=kv.dtype)
    scc = None if sc is None else np.zeros((n_req, MP * P), dtype=np.float32)
    oracle.append_rows(src, np.arange(n_req, dtype=np.int32)[:, None], pos0, kvc, scc, dst=dst)
    written = set()
    for b in range(n_req):
        for t in range(T):
            pos = int(pos0[b]) + t
            page, slot = pt[b, pos // P], pos % P
            written.add((page, slot))
            assert kv[page, slot].tobytes() == kvc[b, pos].tobytes()
            if sc is not None:
                assert sc[page, slot] == scc[b, pos]
    untouched = [(p, s) for p in range(kv.shape[0]) for s in range(P) if (p, s) not in written]
    for p, s in untouched:
        assert kv[p, s].tobytes() == fresh[p, s].tobytes()


def test_append_fp8_rows_meet_the_format_error_bound():
    """Each stored value decodes (code x scale) to within half a step of E4M3
    around the source: relative 2^-4 above 2^-6 s, absolute 2^-10 s below; the
    row's largest magnitude lands on the largest finite code."""
    src, pt, pos0, kv, sc = _append_case(12, n_req=3, T=4, D=576, P=16, MP=8, NP=30)
    oracle.append_rows(src, pt, pos0, kv, sc, dst="fp8")
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    for b in range(src.shape[0]):
        for t in range(src.shape[1]):
            pos = int(pos0[b]) + t
            page, slot = pt[b, pos // 16], pos % 16
            s = float(sc[page, slot])
            x = src[b, t].astype(np.float64)
            amax = np.abs(x).max()
            assert s == (np.float32(amax) / np.float32(448) if amax > 0 else 1.0)
            dec = table[kv[page, slot]] * s
            tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
            assert np.all(np.abs(dec - x) <= tol)
            if amax > 0:
                assert kv[page, slot][np.argmax(np.abs(x))] & 0x7F == 0x7E


def test_append_fp8_matches_generator_encoder():
    """The generator's row quantiser (written separately, used to build the FP8
    workload) and the oracle's append agree bit for bit."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((1, 40, 576)) * 0.5).astype(np.float32)
    kv = np.zeros((3, 16, 576), dtype=np.uint8)
    sc = np.zeros((3, 16), dtype=np.float32)
    oracle.append_rows(x, np.array([[2, 0, 1]], dtype=np.int32), np.array([0], dtype=np.int32), kv, sc)
    codes, scales = synth.formats.quantize_rows_e4m3(x[0])
    order = [(2, s) for s in range(16)] + [(0, s) for s in range(16)] + [(1, s) for s in range(8)]
    for t, (pg, sl) in enumerate(order):
        assert np.array_equal(kv[pg, sl], codes[t]) and sc[pg, sl] == scales[t]


# -------------------------------------------------- greedy chain verification

def test_verify_argmax_matches_numpy_first_occurrence():
    """p_t against numpy's argmax (first index among equal maxima), with ties
    made frequent by rounding the logits to bf16 and by planting copies."""
    rng = np.random.default_rng(21)
    lg = torch.from_numpy(rng.standard_normal((6, 4, 3000)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    lg[0, 0, 100] = lg[0, 0, 2000] = lg[0, 0].max() + 1.0   # an exact tie, smaller index wins
    lg[1, 2, :] = 0.5                                        # all equal: index 0
    am, _, _ = oracle.verify_greedy(lg, np.zeros((6, 3), dtype=np.int32))
    assert np.array_equal(am, lg.argmax(axis=2))
    assert am[0, 0] == 100 and am[1, 2] == 0


def test_verify_nan_never_wins():
    lg = np.array([[[np.nan, 1.0, 3.0, np.nan, 2.0]]])
    am, n, out = oracle.verify_greedy(lg, np.zeros((1, 0), dtype=np.int32))
    assert am[0, 0] == 2 and n[0] == 0 and out[0, 0] == 2


@pytest.mark.parametrize("T", [1, 2, 4, 7])
def test_verify_acceptance_is_the_run_of_leading_matches(T):
    """Drafts built from the target's own predictions with one planted
    mismatch at k: exactly k drafts pass (later matches do not count), the
    output is those drafts, then p_k, then -1."""
    rng = np.random.default_rng(22 + T)
    B, V = 3 * T, 50
    lg = rng.standard_normal((B, T, V))
    p = lg.argmax(axis=2)
    draft = p[:, : T - 1].astype(np.int32).copy()
    planted = []
    for b in range(B):
        k = b % T  # k = T - 1: no mismatch, every draft passes and p_{T-1} is the bonus
        if k < T - 1:
            draft[b, k] = (p[b, k] + 1) % V
        planted.append(k)
    am, n, out = oracle.verify_greedy(lg, draft)
    assert np.array_equal(am, p)
    for b in range(B):
        k = planted[b]
        assert n[b] == k
        assert list(out[b, :k]) == list(draft[b, :k]) and out[b, k] == p[b, k]
        assert (out[b, k + 1:] == -1).all()


# ---------------------------------------------------------------- projections

@pytest.mark.parametrize("w", [tiny(), small_ds(q_len=2, causal=True, heads=4)], ids=["tiny", "ds_causal"])
def test_projections_around_the_oracle_equal_expanded_mha(w):
    """Query side: project(q_nope, W_UK^T per head) is the absorbed query (the
    dyadic case makes it exact); value side: project(o, W_UV) equals attention
    over decompressed keys and values, computed without any projection call."""
    inp, W_UK, W_UV, q_nope = _absorbed_case(w, seed=11)
    B, T, H = w.batch, w.q_len, w.heads
    q_abs = oracle.project(q_nope.reshape(B * T, H, -1), W_UK.transpose(0, 2, 1))
    assert np.array_equal(q_abs.reshape(B, T, H, -1), stored_values(inp, "q_abs"))
    o, _ = oracle.attend(inp)
    got = oracle.project(o.reshape(B * T, H, -1), W_UV).reshape(B, T, H, -1)
    ref = _expanded_mha(inp, W_UK, W_UV, q_nope)
    assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


def test_projection_one_hot_weights_pick_one_input_column():
    """w[g] with a single 1 at (n_g, k_g), different per head, copies x[:, g, k_g]
    to out[:, g, n_g] and leaves every other output zero (index roles)."""
    M, G, K, N = 5, 3, 6, 6
    rng = np.random.default_rng(2)
    x = rng.standard_normal((M, G, K))
    w = np.zeros((G, N, K))
    picks = [(1, 4), (5, 0), (2, 3)]
    for g, (n, k) in enumerate(picks):
        w[g, n, k] = 1.0
    out = oracle.project(x, w)
    expect = np.zeros((M, G, N))
    for g, (n, k) in enumerate(picks):
        expect[:, g, n] = x[:, g, k]
    assert np.array_equal(out, expect)


def test_projection_matches_matmul_per_head():
    M, G, K, N = 7, 4, 24, 16
    xb, wb = synth.make_projection_inputs(M, G, K, N, seed=5)
    x, w = synth.bf16_bits_to_f32(xb).astype(np.float64), synth.bf16_bits_to_f32(wb).astype(np.float64)
    out = oracle.project(x, w)
    for g in range(G):
        ref = x[:, g, :] @ w[g].T
        assert np.abs(out[:, g, :] - ref).max() <= 1e-13 * np.abs(ref).max()


def test_projection_of_no_rows():
    assert oracle.project(np.zeros((0, 2, 8)), np.ones((2, 3, 8))).shape == (0, 2, 3)
