"""attn_check_seqlens on the GPU: well-formed packings give 0, each malformation its bit.

The cumulative-length arrays locate each sequence's segment of the packed tensors ("Causal
Mask and Ragged Sequence Layouts", section 1); the entry points trust them, and this call is
how a caller finds out whether they can. The expected words are the definitions of the
header's bits evaluated on the host, bit for bit.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import exact_attention_tiled_amd as eat
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    eat.load()


def expected_word(cu_q, cu_k, total_q, total_k, max_q, max_k):
    word = 0
    for bit0, cu, total, mx in ((1, cu_q, total_q, max_q), (16, cu_k, total_k, max_k)):
        lens = np.diff(np.asarray(cu, dtype=np.int64))
        if cu[0] != 0:
            word |= bit0
        if np.any(lens < 0):
            word |= 2 * bit0
        if cu[-1] != total:
            word |= 4 * bit0
        if np.any(lens > mx):
            word |= 8 * bit0
    return word


def check(cu_q, cu_k, total_q, total_k, max_q, max_k):
    import torch
    import exact_attention_tiled_amd as eat
    cq = torch.tensor(np.asarray(cu_q, dtype=np.int32), device="cuda")
    ck = torch.tensor(np.asarray(cu_k, dtype=np.int32), device="cuda")
    print(f"check_seqlens num_seqs={len(cu_q) - 1} totals=({total_q},{total_k}) "
          f"max=({max_q},{max_k})", flush=True)
    got = eat.attn_check_seqlens(cq, ck, total_q, total_k, max_q, max_k)
    want = expected_word(cu_q, cu_k, total_q, total_k, max_q, max_k)
    assert got == want, (got, want, [eat.SEQLENS_ERRORS[b] for b in eat.SEQLENS_ERRORS if got & b])
    return got


def _cu(lengths):
    return [int(x) for x in wl.cu_from_lengths(lengths)]


@pytest.mark.parametrize("lq,lk", [
    (wl.ragged_lengths(3), None),                     # the ragged GQA packing
    ([2048] * 4, None),                               # dense, equal lengths
    ([16] * 16, [32768] * 16),                        # decode, Nq = 16
    ([127, 128, 129, 1, 0, 5], [127, 128, 129, 1, 3, 0]),
    ([], []),                                         # empty batch: cu = [0]
    ([3] * 1000, [5] * 1000),                         # more sequences than threads
])
def test_well_formed_packings_pass(lq, lk):
    lk = lq if lk is None else lk
    cu_q, cu_k = _cu(lq), _cu(lk)
    assert check(cu_q, cu_k, cu_q[-1], cu_k[-1], max(lq, default=0), max(lk, default=0)) == 0


def test_each_malformation_sets_its_bit():
    lq, lk = [3] * 700, [5] * 700
    cu_q, cu_k = _cu(lq), _cu(lk)
    tq, tk = cu_q[-1], cu_k[-1]
    # start not at zero (every length stays valid)
    assert check([1] + cu_q[1:], cu_k, tq, tk, 3, 5) == 1
    assert check(cu_q, [1] + cu_k[1:], tq, tk, 3, 5) == 16
    # a decreasing step deep in the array (sequence 600, past the first 256 threads)
    bad = list(cu_q)
    bad[601] = bad[600] - 1
    assert check(bad, cu_k, tq, tk, 3, 5) & 2
    bad = list(cu_k)
    bad[301] = bad[300] - 2
    assert check(cu_q, bad, tq, tk, 3, 5) & 32
    # last entry not the token count
    assert check(cu_q, cu_k, tq + 1, tk, 3, 5) == 4
    assert check(cu_q, cu_k, tq, tk - 1, 3, 5) == 64
    # a length above the host's bound (equal-length batches trust it for their geometry)
    assert check(cu_q, cu_k, tq, tk, 2, 5) == 8
    assert check(cu_q, cu_k, tq, tk, 3, 4) == 128
    # the plain-reading mistake of passing a packing with unequal lengths as uniform
    uneven = _cu([100, 8092])
    assert check(uneven, uneven, 8192, 8192, 4096, 4096) == 8 | 128
    # several at once, and an empty batch whose single entry is not zero
    assert check([5], [0], 0, 0, 0, 0) == 1 | 4
    assert check([2] + cu_q[1:], [0] + cu_k[1:-1] + [tk + 9], tq, tk, 1, 5) == 1 | 8 | 64 | 128
