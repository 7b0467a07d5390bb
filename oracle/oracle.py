"""Plain float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module; only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares
no code with the HIP library and does not import it.

What it computes is the textbook definition, written out with no tiling, no online
recurrence and no fusion, so that it cannot share the tiled kernel's bugs:

  * "Efficient Attention: Formal Correctness" page, section "The FlashAttention Proof":
    the optimised kernel is held equal to a naive attention specification, and the online
    recurrence computes exactly the recomputed softmax. The oracle *is* that naive
    specification: O = softmax(scale * Q K^T restricted to allowed keys) V.
  * "Causal Mask and Ragged Sequence Layouts" page: every query and key carries a sequence
    id and an in-sequence position (first section); padding and out-of-range lanes are an
    exclusion rule applied before the maximum and the denominator (second section);
    top-left (j <= i) and bottom-right (j <= i + Nk - Nq) causal alignment (third section);
    all-masked rows give zero output (fourth section); backward rebuilds the same mask
    (sixth section).
  * "Attention Algorithm Error and Complexity Tests" page, third section: GQA shares one
    K/V head among a group of query heads and the group's gradients are summed.

Readings taken where the pages are silent:
  * window: width W > 0 admits the W most recent keys up to the aligned diagonal,
    pos_k in (pos_q + off - W, pos_q + off]; only with a causal alignment.
  * LSE of an all-masked row is -inf; LSE is the natural log-sum-exp of the scaled logits,
    stored [Hq, total_q].
  * GQA grouping is consecutive: query head h reads K/V head h // (Hq // Hkv).
  * Dropout ("Attention Algorithm Error and Complexity Tests" page, first and fourth
    sections; "Causal Mask and Ragged Sequence Layouts" page, sixth section: replay must
    follow logical indices): inverted dropout on the normalised weights,
    O = (P * keep / (1 - p)) V, with the LSE of the undropped softmax. The keep flag of
    (sequence index, query head, in-sequence query position, in-sequence key position)
    comes from Philox4x32-10 (dropout_keep below); p is rounded to a multiple of 1/256.

All arithmetic is float64 (numpy). Inputs may be any float dtype; they are upcast exactly.
Every function is pinned by tests in tests/test_oracle_*.py (closed forms, invariants,
finite differences, brute force and a library special case).
"""
from __future__ import annotations

import numpy as np

MASK_NONE = 0
MASK_CAUSAL_TOP_LEFT = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2

_ROW_CHUNK = 512


# ----------------------------------------------------------------------------------------
# Metadata and the explicit mask ("Causal Mask and Ragged Sequence Layouts", sections 1-4)
# ----------------------------------------------------------------------------------------

def token_metadata(cu):
    """Per-token sequence id and in-sequence position, and per-sequence lengths.

    The cumulative-length array only locates each segment; the position of token t is its
    offset from the start of its own segment, never the global index t.
    """
    cu = np.asarray(cu, dtype=np.int64)
    total = int(cu[-1])
    t = np.arange(total, dtype=np.int64)
    # side='right' - 1 maps t to the last segment whose start is <= t, which skips
    # zero-length segments (their start equals the next segment's start).
    seq = np.searchsorted(cu, t, side="right") - 1
    pos = t - cu[seq]
    lengths = np.diff(cu)
    return seq, pos, lengths


def allowed(seq_q, pos_q, seq_k, pos_k, len_q, len_k, mask_mode, window):
    """Elementwise allowed-pair predicate (broadcasting numpy arrays).

    seq_*/pos_* are sequence ids and in-sequence positions; len_q/len_k are the lengths of
    the *query's* sequence (the only one a pair can be allowed in).
    """
    same = seq_q == seq_k
    if mask_mode == MASK_NONE:
        if window > 0:
            raise ValueError("a window needs a causal alignment")
        return same & np.ones_like(pos_k, dtype=bool)
    if mask_mode == MASK_CAUSAL_TOP_LEFT:
        diag = pos_q                              # key j allowed iff j <= i
    elif mask_mode == MASK_CAUSAL_BOTTOM_RIGHT:
        diag = pos_q + (len_k - len_q)            # key j allowed iff j <= i + Nk - Nq
    else:
        raise ValueError(f"unknown mask mode {mask_mode}")
    ok = same & (pos_k <= diag)
    if window > 0:
        ok = ok & (pos_k > diag - window)
    return ok


def explicit_mask(cu_q, cu_k, mask_mode, window=0):
    """Full boolean [total_q, total_k] mask from sequence ids and positions (small cases)."""
    sq, pq, lq = token_metadata(cu_q)
    sk, pk, lk = token_metadata(cu_k)
    return allowed(sq[:, None], pq[:, None], sk[None, :], pk[None, :],
                   lq[sq][:, None], lk[sq][:, None], mask_mode, window)


# ----------------------------------------------------------------------------------------
# Forward: the naive specification on an explicit mask
# ----------------------------------------------------------------------------------------

def _softmax_rows(s, a):
    """Masked softmax pieces for logits s and allowed flags a (both [rows, keys]).

    Disallowed entries are excluded before the maximum and the denominator. Rows with no
    allowed entry give p = 0 and lse = -inf.
    """
    n = a.sum(axis=1)
    m = np.where(a, s, -np.inf).max(axis=1, initial=-np.inf)
    m_safe = np.where(n > 0, m, 0.0)
    e = np.where(a, np.exp(np.where(a, s, 0.0) - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(n > 0, l, 1.0)
    p = e / l_safe[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(n > 0, m_safe + np.log(l_safe), -np.inf)
    return p, lse


def attention_explicit(q, k, v, mask, scale):
    """O, LSE for a given boolean mask [total_q, total_k] shared by all heads.

    q: [Tq, Hq, d]; k, v: [Tk, Hkv, d]. Query head h uses K/V head h // (Hq // Hkv).
    Returns O [Tq, Hq, d] and LSE [Hq, Tq], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    o = np.zeros((tq, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((hq, tq), -np.inf, dtype=np.float64)
    for h in range(hq):
        kh, vh = k[:, h // g, :], v[:, h // g, :]
        for r0 in range(0, tq, _ROW_CHUNK):
            r1 = min(tq, r0 + _ROW_CHUNK)
            s = scale * (q[r0:r1, h, :] @ kh.T)
            p, lse[h, r0:r1] = _softmax_rows(s, mask[r0:r1])
            o[r0:r1, h, :] = p @ vh
    return o, lse


def attention(q, k, v, cu_q, cu_k, scale, mask_mode, window=0, seqs=None, heads=None,
              dropout_p=0.0, seed=0):
    """Varlen GQA attention: O [Tq, Hq, d], LSE [Hq, Tq] in float64.

    With dropout_p > 0 the weights that reach V are P * keep / (1 - t/256) with the keep
    flags of ``dropout_keep`` (t = ``dropout_threshold(dropout_p)``); the LSE stays that of
    the undropped softmax.

    The mask of every query row is built from sequence ids and in-sequence positions. A
    pair can only be allowed inside one sequence, so each sequence's rows are evaluated
    against that sequence's key segment (every other key fails the same-sequence test);
    the same-sequence test is still applied explicitly.

    ``seqs`` / ``heads`` restrict the evaluation to some sequences / query heads; rows not
    evaluated are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = hq // hkv
    sq, pq, lq = token_metadata(cu_q)
    sk, pk, lk = token_metadata(cu_k)
    nseq = len(lq)
    if len(lk) != nseq:
        raise ValueError("cu_seqlens_q and cu_seqlens_k describe different batch sizes")
    restricted = seqs is not None or heads is not None
    fill = np.nan if restricted else 0.0
    o = np.full((tq, hq, v.shape[2]), fill, dtype=np.float64)
    lse = np.full((hq, tq), np.nan if restricted else -np.inf, dtype=np.float64)
    seqs = range(nseq) if seqs is None else seqs
    heads = range(hq) if heads is None else heads
    thr = dropout_threshold(dropout_p)
    for s in seqs:
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        for r0 in range(qa, qb, _ROW_CHUNK):
            r1 = min(qb, r0 + _ROW_CHUNK)
            a = allowed(sq[r0:r1, None], pq[r0:r1, None], sk[None, ka:kb], pk[None, ka:kb],
                        lq[s], lk[s], mask_mode, window)
            for h in heads:
                g = h // grp
                sc = scale * (q[r0:r1, h, :] @ k[ka:kb, g, :].T)
                p, lse[h, r0:r1] = _softmax_rows(sc, a)
                if thr > 0:
                    p = p * _dropout_factor(seed, s, h, pq[r0:r1], pk[ka:kb], thr)
                o[r0:r1, h, :] = p @ v[ka:kb, g, :]
    return o, lse


def _dropout_factor(seed, s, h, pos_q, pos_k, thr):
    """keep / (1 - t/256) for rows pos_q and columns pos_k of sequence s, head h."""
    keep = dropout_keep(seed, s, h, pos_q[:, None], pos_k[None, :], thr)
    return np.where(keep, 256.0 / (256.0 - thr), 0.0)


def attention_per_sequence(q, k, v, cu_q, cu_k, scale, mask_mode, window=0):
    """Same operator evaluated one sequence at a time with purely local indices.

    Each sequence is cut out, given its own explicit mask built from 0-based positions
    (a one-sequence cu array), and run through ``attention_explicit``; the results are
    scattered back. Used to pin that packing reproduces per-sequence results.
    """
    q = np.asarray(q, dtype=np.float64)
    tq, hq, d = q.shape
    o = np.zeros((tq, hq, np.asarray(v).shape[2]), dtype=np.float64)
    lse = np.full((hq, tq), -np.inf, dtype=np.float64)
    for s in range(len(cu_q) - 1):
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        m = explicit_mask([0, qb - qa], [0, kb - ka], mask_mode, window)
        os_, ls_ = attention_explicit(q[qa:qb], np.asarray(k)[ka:kb], np.asarray(v)[ka:kb],
                                      m, scale)
        o[qa:qb] = os_
        lse[:, qa:qb] = ls_
    return o, lse


# ----------------------------------------------------------------------------------------
# Dropout: a counter-based generator keyed by logical indices
# ----------------------------------------------------------------------------------------

_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
    as easy as 1, 2, 3", SC'11, section 3: the Philox S-box and its key schedule).

    Each round multiplies counter words 0 and 2 by the two Philox multipliers (full 64-bit
    products), and the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key is advanced by the two Weyl constants before every round but the
    first. Counters broadcast as numpy arrays; returns four uint32 arrays.
    """
    m0, m1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
    w0, w1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
    c = [np.asarray(x).astype(np.uint64) & _M32 for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + w0) & _M32
            k1 = (k1 + w1) & _M32
        p0 = m0 * c[0]  # < 2^64: exact in uint64
        p1 = m1 * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _M32, (p0 >> np.uint64(32)) ^ c[3] ^ k1,
             p0 & _M32]
    return [x.astype(np.uint32) for x in c]


def dropout_threshold(p):
    """Byte threshold t = round(256 p) of a dropout probability given as float32: an element
    is dropped iff its random byte is below t, so the realised probability is t / 256.
    t must be at most 255 (p < 255.5 / 256)."""
    p32 = float(np.float32(p))
    t = int(np.floor(p32 * 256.0 + 0.5))
    if not (p32 >= 0.0 and t <= 255):
        raise ValueError("dropout probability must lie in [0, 255.5/256)")
    return t


def dropout_keep(seed, seq, head, pos_q, pos_k, thr):
    """Keep flags [n, m] of (sequence index, query head) for query positions pos_q (shape
    [n, 1]) against key positions pos_k (shape [1, m]). One generator call covers the 4 x 4
    patch of query positions 4 (pos_q // 4) + 0..3 and key positions 4 (pos_k // 4) + 0..3:
    counter (pos_q // 4, pos_k // 4, head, seq), key (low, high 32 bits of the 64-bit
    seed); the element takes byte pos_k % 4 of output word pos_q % 4. Storage offsets never
    enter, so the realisation replays across packings and in the backward."""
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    if pos_q.ndim != 2 or pos_k.ndim != 2 or pos_q.shape[1] != 1 or pos_k.shape[0] != 1:
        raise ValueError("pos_q must be [n, 1] and pos_k [1, m]")
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    qp, iq = np.unique(pos_q[:, 0] // 4, return_inverse=True)
    kp, ik = np.unique(pos_k[0, :] // 4, return_inverse=True)
    words = np.stack(philox4x32_10(qp[:, None], kp[None, :], int(head), int(seq),
                                   seed & 0xFFFFFFFF, seed >> 32))        # [4, patches_q, patches_k]
    word = words[(pos_q % 4), iq[:, None], ik[None, :]]
    byte = (word >> (8 * (pos_k % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= np.uint32(thr)


# ----------------------------------------------------------------------------------------
# Backward: gradients of the same naive specification with the same mask
# ----------------------------------------------------------------------------------------

def _bwd_rows(qh, kg, vg, doh, a, scale, zf=None, oh=None):
    """Gradients for one block of rows of one query head (all in float64).

    P is recomputed from the logits and the mask; D = rowsum(dO * O) with O = P V;
    dP = dO V^T; dS = P * (dP - D); dQ = scale dS K; dK = scale dS^T Q; dV = P^T dO.
    With dropout factors zf (keep / (1 - p)): Z = P * zf, O = Z V, dZ = dO V^T,
    dP = dZ * zf, dS = P * (dP - D) with D = rowsum(dO * O) = rowsum(P * dP), dV = Z^T dO.
    With a stored output oh, D = rowsum(dO * oh) instead.
    """
    s = scale * (qh @ kg.T)
    p, _ = _softmax_rows(s, a)
    z = p if zf is None else p * zf
    o = z @ vg if oh is None else oh
    dd = (doh * o).sum(axis=1)
    dp = doh @ vg.T
    if zf is not None:
        dp = dp * zf
    ds = p * (dp - dd[:, None])
    return scale * (ds @ kg), scale * (ds.T @ qh), z.T @ doh


def attention_bwd(q, k, v, dout, cu_q, cu_k, scale, mask_mode, window=0,
                  seqs=None, kv_heads=None, dropout_p=0.0, seed=0, out=None):
    """dQ [Tq,Hq,d], dK and dV [Tk,Hkv,d] (float64) of sum(dout * O).

    dK/dV of a K/V head are summed over every query head of its group. ``seqs`` /
    ``kv_heads`` restrict the evaluation (other entries NaN). ``dropout_p`` / ``seed``
    replay the forward's dropout realisation (the same keep flags).

    ``out`` ([Tq, Hq, d], optional): the stored forward output the backward is given (the
    library's backward receives the forward's output as an input); D = rowsum(dout * out)
    is then formed from it instead of from the oracle's own float64 output. Everything else
    is unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    out = None if out is None else np.asarray(out, dtype=np.float64)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = hq // hkv
    sq, pq, lq = token_metadata(cu_q)
    sk, pk, lk = token_metadata(cu_k)
    restricted = seqs is not None or kv_heads is not None
    fill = np.nan if restricted else 0.0
    dq = np.full(q.shape, fill)
    dk = np.full(k.shape, fill)
    dv = np.full(v.shape, fill)
    seqs = range(len(lq)) if seqs is None else seqs
    kv_heads = range(hkv) if kv_heads is None else kv_heads
    thr = dropout_threshold(dropout_p)
    for s in seqs:
        qa, qb = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        for g in kv_heads:
            dk_acc = np.zeros((kb - ka, d))
            dv_acc = np.zeros((kb - ka, v.shape[2]))
            for h in range(g * grp, (g + 1) * grp):
                for r0 in range(qa, qb, _ROW_CHUNK):
                    r1 = min(qb, r0 + _ROW_CHUNK)
                    a = allowed(sq[r0:r1, None], pq[r0:r1, None], sk[None, ka:kb],
                                pk[None, ka:kb], lq[s], lk[s], mask_mode, window)
                    zf = (_dropout_factor(seed, s, h, pq[r0:r1], pk[ka:kb], thr)
                          if thr > 0 else None)
                    gq, gk, gv = _bwd_rows(q[r0:r1, h], k[ka:kb, g], v[ka:kb, g],
                                           dout[r0:r1, h], a, scale, zf,
                                           None if out is None else out[r0:r1, h])
                    dq[r0:r1, h] = gq
                    dk_acc += gk
                    dv_acc += gv
            dk[ka:kb, g] = dk_acc
            dv[ka:kb, g] = dv_acc
    return dq, dk, dv


def attention_explicit_bwd(q, k, v, dout, mask, scale):
    """Backward of ``attention_explicit`` for a given [Tq, Tk] mask."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h // grp
        gq, gk, gv = _bwd_rows(q[:, h], k[:, g], v[:, g], dout[:, h], mask, scale)
        dq[:, h] = gq
        dk[:, g] += gk
        dv[:, g] += gv
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Key-range partials and their log-sum-exp combination (decode split over the key axis)
# ----------------------------------------------------------------------------------------

def lse_combine(parts):
    """Combine (O_i, LSE_i) computed over disjoint key subsets into (O, LSE).

    LSE = log sum_i exp(LSE_i); O = sum_i exp(LSE_i - LSE) O_i. A row whose every part is
    empty (LSE_i = -inf for all i) gives O = 0 and LSE = -inf.
    O_i: [Tq, Hq, d], LSE_i: [Hq, Tq].
    """
    lses = np.stack([p[1] for p in parts])                 # [n, Hq, Tq]
    outs = np.stack([p[0] for p in parts])                 # [n, Tq, Hq, d]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe[None]), 0.0)   # [n, Hq, Tq]
    tot = w.sum(axis=0)
    tot_safe = np.where(finite, tot, 1.0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(tot_safe), -np.inf)
    wn = w / tot_safe[None]                                  # [n, Hq, Tq]
    o = np.einsum("nht,nthd->thd", wn, outs)
    return o, lse


def attention_key_range(q, k, v, cu_q, cu_k, scale, mask_mode, window, key_lo, key_hi):
    """Attention restricted to keys whose in-sequence position lies in [key_lo, key_hi).

    The restriction is one more exclusion applied with the mask; positions and alignment
    stay those of the full sequence.
    """
    sq, pq, lq = token_metadata(cu_q)
    sk, pk, lk = token_metadata(cu_k)
    full = explicit_mask(cu_q, cu_k, mask_mode, window)
    in_range = (pk >= key_lo) & (pk < key_hi)
    return attention_explicit(q, k, v, full & in_range[None, :], scale)
