"""attn_fwd_no_workspace (the forward for callers that cannot allocate) against attn_fwd:
two calls in a row on the fixed device scratch, the second with a smaller input, for the
split-K decode (partials in the scratch) and for a ragged prefill (tile order in the
scratch). Outputs must be bitwise equal to attn_fwd's with its own workspace (same plan,
same kernels) and within tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import exact_attention_tiled_amd as eat
import oracle
import workloads as wl
from gpu_util import check_fwd, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    eat.load()


def _cases():
    big_dec = wl.random_workload(71, [16] * 4, [4096] * 4, 32, 8, 128, "bf16",
                                 wl.MASK_CAUSAL_BOTTOM_RIGHT, name="decode_nq16")
    small_dec = wl.random_workload(72, [4] * 2, [2048, 1500], 32, 8, 128, "bf16",
                                   wl.MASK_CAUSAL_BOTTOM_RIGHT, name="decode_nq4")
    big_pre = wl.random_workload(73, [300, 129, 0, 700], [300, 129, 5, 700], 8, 2, 128, "bf16",
                                 wl.MASK_CAUSAL_TOP_LEFT, name="ragged_prefill")
    small_pre = wl.random_workload(74, [65, 3], [65, 40], 4, 2, 64, "bf16",
                                   wl.MASK_CAUSAL_BOTTOM_RIGHT, window=17, name="ragged_small")
    return [(big_dec, small_dec), (big_pre, small_pre)]


@pytest.mark.parametrize("pair", [0, 1], ids=["splitk_decode", "ragged_prefill"])
def test_no_workspace_matches_attn_fwd(pair):
    for w in _cases()[pair]:
        print(f"no-workspace case {w.name}", flush=True)
        t = to_device(w)
        plan = eat.attn_describe_plan(t["q"], t["k"], t["cu_q"], w.max_seqlen_q, w.max_seqlen_k,
                                      w.mask_mode, w.window)
        need = eat.attn_fwd_workspace_size(t["q"], t["k"], t["cu_q"], w.max_seqlen_q,
                                           w.max_seqlen_k, w.mask_mode, w.window)
        assert 0 < need <= (16 << 20), (w.name, plan, need)
        out = torch.full_like(t["q"], 7.0)
        lse = torch.full((w.hq, w.total_q), 7.0, dtype=torch.float32, device=t["q"].device)
        eat.attn_fwd_no_workspace(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                  w.max_seqlen_k, w.scale, w.mask_mode, w.window, out=out,
                                  lse=lse)
        ref_out, ref_lse = eat.attn_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"],
                                        w.max_seqlen_q, w.max_seqlen_k, w.scale, w.mask_mode,
                                        w.window)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), (w.name, plan)
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), (w.name, plan)
        ro, rl = oracle.attention(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.mask_mode, w.window)
        check_fwd(w, out, lse, ro, rl, what=f"no-workspace {w.name}")
