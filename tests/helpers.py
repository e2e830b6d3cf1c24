"""Shared helpers for the GPU parity tests: move synth inputs to the device,
run the HIP path through the C-ABI binding, and compare with the oracle."""
import numpy as np
import torch

import synth

# Parity bars (max-abs and mean-relative = sum|g - r| / sum|r|): bf16 outputs
# 2e-2 / 1e-2, fp8 KV 5e-2 / 1e-2; the fp32 path is held to 1e-4 / 1e-5.
TOL = {"bf16": (2e-2, 1e-2), "fp8": (5e-2, 1e-2), "f32": (1e-4, 1e-5)}


def tolerance(w):
    if w.kv_dtype == "fp8":
        return TOL["fp8"]
    return TOL["f32"] if w.out_dtype == "f32" else TOL["bf16"]


def bf16_tensor(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(inp, device="cuda"):
    w = inp["workload"]
    d = {}
    if w.q_dtype == "bf16":
        d["q_abs"] = bf16_tensor(inp["q_abs"], device)
        d["q_rope"] = bf16_tensor(inp["q_rope"], device)
    else:
        d["q_abs"] = torch.from_numpy(inp["q_abs"]).to(device)
        d["q_rope"] = torch.from_numpy(inp["q_rope"]).to(device)
    if w.kv_dtype == "bf16":
        d["kv"] = bf16_tensor(inp["kv"], device)
    elif w.kv_dtype == "fp8":
        d["kv"] = torch.from_numpy(inp["kv"]).to(device)
    else:
        d["kv"] = torch.from_numpy(inp["kv"]).to(device)
    d["kv_scales"] = None if inp["kv_scales"] is None else torch.from_numpy(inp["kv_scales"]).to(device)
    d["page_table"] = torch.from_numpy(inp["page_table"]).to(device)
    d["seq_lens"] = torch.from_numpy(inp["seq_lens"]).to(device)
    return d


def run_decode(mla, inp, dev=None, num_splits=0, out_dtype=None):
    """Run mla_decode on the inputs; returns (out float64 numpy [B,T,H,Dc], lse numpy)."""
    w = inp["workload"]
    if dev is None:
        dev = to_device(inp)
    od = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype or w.out_dtype]
    out, lse = mla.decode(dev["q_abs"], dev["q_rope"], dev["kv"], dev["page_table"],
                          dev["seq_lens"], float(inp["scale"]), kv_scales=dev["kv_scales"],
                          causal=w.causal, num_splits=num_splits, max_seq_len=w.max_seq_len,
                          out_dtype=od)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def metrics(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    diff = np.abs(g - r)
    max_abs = float(diff.max()) if diff.size else 0.0
    denom = float(np.abs(r).sum())
    mean_rel = float(diff.sum() / denom) if denom > 0 else float(diff.sum())
    return max_abs, mean_rel


def assert_close(g, r, tol, what=""):
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    max_abs, mean_rel = metrics(g, r)
    assert max_abs <= tol[0] and mean_rel <= tol[1], \
        f"{what}: max_abs {max_abs:.3e} (bar {tol[0]:.0e}), mean_rel {mean_rel:.3e} (bar {tol[1]:.0e})"
    return max_abs, mean_rel


def small(which, **kw):
    """A scaled-down copy of workload `which` that the oracle finishes in seconds."""
    return synth.workload(which).with_(**kw)
