"""CPU model of the roundings the bf16 kernels prescribe, applied to exact (float64) values.

Test infrastructure for deriving gradient tolerances: it is neither the oracle nor the HIP
path. Every value is first computed exactly (float64), then rounded to bf16 (round to
nearest even) at exactly the points where the kernels hold bf16 data:
  forward  O = (sum_j bf16(p_j) v_j) / sum_j p_j, stored as bf16 (the PV contraction takes
           the unnormalised weights as bf16 operands, the denominator sums them unrounded;
           each p_j is taken at the running exponent offset the kernel holds for its stage,
           which the later rescales of the accumulator undo exactly);
  backward P rebuilt from the LSE, D = rowsum(dO * O_stored) (without dropout), the exact
           D = sum_j P dP (the dropout path's own D pass) or D from the stored output plus
           its rounding residual, dS = P (dP - D) and the dV operand
           (P, or Z = P * keep / (1 - p) with dropout) rounded to bf16 before the
           contractions; dQ, dK, dV accumulated exactly and stored as bf16.
The fp32 accumulations of the kernels (products of bf16 values are exact in fp32; sums carry
relative errors near 2^-24) are left exact here: they are orders of magnitude below the
bf16 roundings.

The tolerance a kernel output needs, as atol at rtol 2e-2 (|err| <= atol + 2e-2 |ref|), is
then what this model needs on the same inputs.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as wl

RTOL = 2e-2


def bf16(x):
    return wl.round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def required_atol(got, ref):
    """Smallest atol with |got - ref| <= atol + RTOL |ref| everywhere (0 if none needed)."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    return float(max(0.0, (err - RTOL * np.abs(ref)).max())) if err.size else 0.0


def stage_offsets_of(logits2, stage=64, threshold=8.0):
    """Per pair, the running exponent offset (log2 units) the prefill kernels hold when they
    round that pair's weight 2^(logit - offset) to bf16. logits2: [rows, keys] scaled logits
    in log2 units (-inf where excluded). Keys are visited in stages of `stage` from key 0; a
    row's offset starts at -inf and becomes a stage's maximum when that exceeds the offset by
    more than `threshold`. Excluded pairs get their row's maximum (0 for empty rows)."""
    nq, nk = logits2.shape
    rowmax = logits2.max(axis=1, initial=-np.inf)
    rowmax = np.where(np.isfinite(rowmax), rowmax, 0.0)
    off = np.repeat(rowmax[:, None], nk, axis=1)
    m = np.full(nq, -np.inf)
    for k0 in range(0, nk, stage):
        blk = logits2[:, k0:k0 + stage]
        mt = blk.max(axis=1)
        m = np.where(mt > m + threshold, mt, m)
        off[:, k0:k0 + stage] = np.where(np.isfinite(blk), m[:, None], off[:, k0:k0 + stage])
    return off


def fp32_dot_sigma(qh, kg, chunk=16):
    """Standard deviation of the fp32 accumulation error of every dot product q_i . k_j:
    the matrix cores sum `chunk` exact bf16 products per instruction and round each partial
    sum into the fp32 accumulator once (error uniform within half an ulp of that partial
    sum, standard deviation ulp / sqrt(12))."""
    prod = qh[:, None, :] * kg[None, :, :]
    parts = np.cumsum(prod.reshape(prod.shape[0], prod.shape[1], -1, chunk).sum(axis=3), axis=2)
    ulp = np.spacing(np.abs(parts).astype(np.float32)).astype(np.float64)
    return np.sqrt((ulp ** 2).sum(axis=2) / 12.0)


def model_backward(w, dropout_p=0.0, seed=0, residual=False, stage_offsets=True,
                   logit_noise=None):
    """(dQ, dK, dV) of the rounding model for workload w (bf16 inputs, any mask, GQA). With
    residual=True (with or without dropout) D is formed from the stored output plus its bf16
    rounding residual; the forward that writes the residual splits each weight Z into
    bf16(Z) + bf16(Z - bf16(Z)) and accumulates both against V, so its unrounded output is
    the exact one to about 2^-16. Otherwise D is exact with dropout and formed from the
    stored output without. The forward's weights are rounded relative to the row maximum,
    or with stage_offsets at the running offset the prefill kernels use (stage_offsets_of):
    where one weight dominates a row (large |scale|) its rounding is exact at the row
    maximum but not at another offset, and the stored output's rounding grows.
    With logit_noise (a seed) the dot products also carry a draw of the fp32 accumulation
    error (fp32_dot_sigma): one draw for the forward's weights and another for the
    backward's recomputed P, normalised with the forward's LSE. Multiplied by a large
    |scale| that error moves some weights across a bf16 rounding boundary, so the rows whose
    stored output rounds differently vary from draw to draw; the kernel's need is then one
    sample of the model's distribution over draws."""
    q, k, v, do = (np.asarray(a, np.float64) for a in (w.q, w.k, w.v, w.dout))
    thr = oracle.dropout_threshold(dropout_p)
    zscale = float(np.float32(256.0 / (256 - thr))) if thr > 0 else 1.0
    hq, hkv = q.shape[1], k.shape[1]
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    sq, pq, lq = oracle.token_metadata(w.cu_q)
    sk, pk, lk = oracle.token_metadata(w.cu_k)
    rng = np.random.default_rng(logit_noise) if logit_noise is not None else None
    for s in range(len(lq)):
        qa, qb, ka, kb = (int(x) for x in (w.cu_q[s], w.cu_q[s + 1], w.cu_k[s], w.cu_k[s + 1]))
        if qa == qb or ka == kb:
            continue
        a = oracle.allowed(sq[qa:qb, None], pq[qa:qb, None], sk[None, ka:kb], pk[None, ka:kb],
                           lq[s], lk[s], w.mask_mode, w.window)
        rows = a.any(axis=1)
        for h in range(hq):
            g = h // grp
            dots = q[qa:qb, h] @ k[ka:kb, g].T
            dots_b = dots
            if rng is not None:
                sig = fp32_dot_sigma(q[qa:qb, h], k[ka:kb, g])
                dots = dots + rng.standard_normal(dots.shape) * sig
                dots_b = dots_b + rng.standard_normal(dots.shape) * sig
            logits = np.where(a, w.scale * dots, -np.inf)
            m = np.where(rows, logits.max(axis=1, initial=-np.inf), 0.0)[:, None]
            pt = np.where(a, np.exp(logits - m), 0.0)
            if stage_offsets:
                # the kernel's weight at its running offset, and the exact rescale of that
                # offset to the row maximum (the accumulator's later alpha factors)
                l2 = logits * np.log2(np.e)
                off = stage_offsets_of(l2)
                wk = np.where(a, np.exp2(np.where(a, l2, 0.0) - off), 0.0)
                back = np.exp2(off - m * np.log2(np.e))
            else:
                wk, back = pt, 1.0
            l = pt.sum(axis=1, keepdims=True)
            l1 = np.where(l > 0, l, 1.0)
            if rng is not None:
                lse = m + np.log(l1)
                p = np.where(a, np.exp(np.where(a, w.scale * dots_b, 0.0) - lse), 0.0)
            else:
                p = pt / l1
            if thr > 0:
                keep = oracle.dropout_keep(seed, s, h, pq[qa:qb, None], pk[None, ka:kb], thr)
                zf = np.where(keep, zscale, 0.0)
            else:
                zf = 1.0
            dp = (do[qa:qb, h] @ v[ka:kb, g].T) * zf
            if residual:
                z_hi = bf16(wk * zf)
                z_lo = bf16(wk * zf - z_hi)
                of = ((z_hi + z_lo) * back) @ v[ka:kb, g] / l1       # the forward's fp32 O
                o = bf16(of) + bf16(of - bf16(of))              # stored output + residual
                dd = (do[qa:qb, h] * o).sum(axis=1)
            elif thr > 0:
                dd = (p * dp).sum(axis=1)                       # the dropout path's exact D
            else:
                o = bf16((bf16(wk) * back) @ v[ka:kb, g] / l1)    # the stored output
                dd = (do[qa:qb, h] * o).sum(axis=1)
            ds = bf16(p * (dp - dd[:, None]))
            z = bf16(p * zf)
            dq[qa:qb, h] = w.scale * ds @ k[ka:kb, g]
            dk[ka:kb, g] += w.scale * ds.T @ q[qa:qb, h]
            dv[ka:kb, g] += z.T @ do[qa:qb, h]
    return bf16(dq), bf16(dk), bf16(dv)
