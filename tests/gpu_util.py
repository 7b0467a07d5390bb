"""Helpers for GPU parity tests: device transfer, oracle comparison and error reports."""
from __future__ import annotations

import numpy as np

BF16_TOL = (2e-2, 2e-2)     # |err| <= atol + rtol * |ref| for bf16 inputs, fp32 accumulation
F32_TOL = (1e-5, 1e-5)      # fp32 inputs
LSE_TOL = 1e-3              # absolute on finite LSE; -inf must match exactly

# Gradient bounds above the standard one, each for the workloads of one test only, and each
# the maximum that the rounding model (tests/rounding_model.py: bf16 P / dS operands, D from
# the stored output, bf16 outputs) needs on those workloads at rtol 2e-2, rounded up by 10 %
# (tests/test_tolerance_derivation.py derives and checks them on the CPU):
#   64 query heads over one K/V head (the deep-GQA limit test): dK, dV;
#   the dropout backward's ragged edge workloads: dQ, dK, dV.
GQA64_GRAD_TOL = (3.4e-2, 2e-2)
DROPOUT_GRAD_TOL = (3.7e-2, 2e-2)


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_device(w):
    """Workload arrays -> contiguous GPU tensors (exact: arrays hold representable values)."""
    import torch
    dt = torch_dtype(w)
    dev = torch.device("cuda:0")
    t = {
        "q": torch.from_numpy(w.q).to(dev).to(dt).contiguous(),
        "k": torch.from_numpy(w.k).to(dev).to(dt).contiguous(),
        "v": torch.from_numpy(w.v).to(dev).to(dt).contiguous(),
        "cu_q": torch.from_numpy(w.cu_q.astype(np.int32)).to(dev),
        "cu_k": torch.from_numpy(w.cu_k.astype(np.int32)).to(dev),
    }
    if w.dout is not None:
        t["dout"] = torch.from_numpy(w.dout).to(dev).to(dt).contiguous()
    return t


def run_fwd(w, t=None, path=0, num_splits=0):
    import exact_attention_tiled_amd as eat
    t = t or to_device(w)
    out, lse = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                            w.max_seqlen_k, w.scale, w.mask_mode, w.window, path=path,
                            num_splits=num_splits)
    return out, lse


def to_np(x):
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def tol_for(w):
    return BF16_TOL if w.dtype == "bf16" else F32_TOL


def assert_close(got, ref, atol, rtol, what, coords=None):
    """Elementwise |got - ref| <= atol + rtol |ref|; NaN in ref marks entries not checked.
    Reports max abs / rel error, mean abs error, violation count, first failing
    coordinates, and requires finite values wherever the reference is finite."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    chk = ~np.isnan(ref)
    fin = chk & np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{what}: non-finite values where the reference is finite"
    inf_ref = chk & np.isinf(ref)
    assert np.array_equal(got[inf_ref], ref[inf_ref]), f"{what}: infinities differ"
    err = np.abs(got[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    bad = err > bound
    if bad.any():
        idx = np.argwhere(fin)[bad][:10]
        rel = err / np.maximum(np.abs(ref[fin]), 1e-30)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max abs {err.max():.3e}, "
            f"max rel {rel.max():.3e}, mean abs {err.mean():.3e}; first failing coords "
            f"{idx.tolist()} got {got[tuple(idx.T)].tolist()} ref {ref[tuple(idx.T)].tolist()}")
    return float(err.max()) if err.size else 0.0


def check_fwd(w, out, lse, ref_o, ref_lse, what=""):
    atol, rtol = tol_for(w)
    assert_close(to_np(out), ref_o, atol, rtol, f"{what} O")
    assert_close(to_np(lse), ref_lse, LSE_TOL, 0.0, f"{what} LSE")

