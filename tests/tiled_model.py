"""A small float64 CPU model of the tiled online-softmax schedule, with switchable mutants.

This is test infrastructure: it lets the tests show that the pins in pins.py are strong
enough to catch the mistakes a tiled kernel typically makes. With no mutant it must agree
with the oracle; with any mutant at least one pin must fail.

Schedule modelled (the shape of the HIP forward, not its code): for each sequence and query
head, query tiles of ``bm`` rows start at the sequence's first token; key tiles of ``bn``
keys start at the sequence's first key and step through the *packed* key array, so the last
tile of a sequence may overrun into the next sequence (or past the end of the array).
Per tile: logits, exclusion of disallowed / out-of-range lanes, running max, rescale of the
denominator and accumulator by exp(m_old - m_new), accumulation, and at the end a division
by the denominator ("Efficient Attention: Formal Correctness" page, section "The
FlashAttention Proof": online softmax recurrence; "Causal Mask and Ragged Sequence Layouts"
page, second section: out-of-range lanes are excluded).

Mutants:
  no_l_rescale      denominator not rescaled when the max moves
  no_acc_rescale    accumulator not rescaled when the max moves
  mask_after_max    running max taken over all lanes, exclusion applied after it
  swap_alignment    top-left and bottom-right exchanged
  global_position   the packed (global) index used as the causal position
  include_oob_lanes lanes beyond the sequence end take part
  head_map_mod      query head h reads K/V head h % Hkv instead of h // (Hq/Hkv)
  bwd_missing_d     backward drops the D = rowsum(dO * O) term
  bwd_no_scale_dk   backward forgets the logit scale on dK
"""
from __future__ import annotations

import numpy as np

NONE, TL, BR = 0, 1, 2

FWD_MUTANTS = ("no_l_rescale", "no_acc_rescale", "mask_after_max", "swap_alignment",
               "global_position", "include_oob_lanes", "head_map_mod")
BWD_MUTANTS = ("bwd_missing_d", "bwd_no_scale_dk")


def _rule(pos_q, pos_k, len_q, len_k, mode, window):
    if mode == NONE:
        return np.ones(np.broadcast(pos_q, pos_k).shape, dtype=bool)
    end = pos_q if mode == TL else pos_q + (len_k - len_q)
    ok = pos_k <= end
    if window > 0:
        ok &= pos_k > end - window
    return ok


class TiledModel:
    def __init__(self, bm=2, bn=3, mutants=(), invariant_log=None):
        self.bm, self.bn = bm, bn
        self.mut = set(mutants)
        self.invariant_log = invariant_log

    # -- shared tile geometry --------------------------------------------------------------
    def _kv_head(self, h, hq, hkv):
        return h % hkv if "head_map_mod" in self.mut else h // (hq // hkv)

    def _tile_allowed(self, rows, keys, s, cu_q, cu_k, tk, mode, window):
        """Allowed flags for query rows x key lanes of one tile (global indices)."""
        lq = int(cu_q[s + 1] - cu_q[s])
        lk = int(cu_k[s + 1] - cu_k[s])
        if "swap_alignment" in self.mut and mode != NONE:
            mode = TL if mode == BR else BR
        if "global_position" in self.mut:
            pq, pk = rows[:, None], keys[None, :]
        else:
            pq, pk = rows[:, None] - cu_q[s], keys[None, :] - cu_k[s]
        end_k = tk if "include_oob_lanes" in self.mut else int(cu_k[s + 1])
        in_range = (keys < end_k)[None, :]
        return in_range & _rule(pq, pk, lq, lk, mode, window)

    # -- forward ----------------------------------------------------------------------------
    def forward(self, q, k, v, cu_q, cu_k, scale, mode, window):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        cu_q, cu_k = np.asarray(cu_q), np.asarray(cu_k)
        tq, hq, d = q.shape
        tk, hkv, _ = k.shape
        o = np.zeros((tq, hq, v.shape[2]))
        lse = np.full((hq, tq), -np.inf)
        for s in range(len(cu_q) - 1):
            for h in range(hq):
                g = self._kv_head(h, hq, hkv)
                for r0 in range(int(cu_q[s]), int(cu_q[s + 1]), self.bm):
                    rows = np.arange(r0, min(r0 + self.bm, int(cu_q[s + 1])))
                    m = np.full(len(rows), -np.inf)
                    l = np.zeros(len(rows))
                    acc = np.zeros((len(rows), v.shape[2]))
                    seen = []
                    for u0 in range(int(cu_k[s]), int(cu_k[s + 1]), self.bn):
                        keys = np.arange(u0, min(u0 + self.bn, tk))
                        a = self._tile_allowed(rows, keys, s, cu_q, cu_k, tk, mode, window)
                        sc = scale * (q[rows, h] @ k[keys, g].T)
                        masked = np.where(a, sc, -np.inf)
                        tile_max = (sc if "mask_after_max" in self.mut else masked).max(axis=1)
                        m_new = np.maximum(m, tile_max)
                        base = np.where(np.isfinite(m_new), m_new, 0.0)
                        alpha = np.exp(m - base)          # exp(-inf) = 0 when m is -inf
                        p = np.where(a, np.exp(masked - base[:, None]), 0.0)
                        l = (l if "no_l_rescale" in self.mut else alpha * l) + p.sum(axis=1)
                        acc = (acc if "no_acc_rescale" in self.mut else alpha[:, None] * acc) \
                            + p @ v[keys, g]
                        m = m_new
                        seen.append(masked)
                        if self.invariant_log is not None:
                            allm = np.concatenate(seen, axis=1)
                            want = np.where(np.isfinite(allm), np.exp(allm - base[:, None]), 0.0)
                            self.invariant_log.append(np.abs(l - want.sum(axis=1)).max()
                                                      / max(1.0, np.abs(l).max()))
                    nz = l > 0
                    o[rows[nz], h] = acc[nz] / l[nz, None]
                    lse[h, rows[nz]] = m[nz] + np.log(l[nz])
        return o, lse

    # -- backward (recomputes P from the saved LSE, tile by tile over keys) -------------------
    def backward(self, q, k, v, dout, cu_q, cu_k, scale, mode, window):
        q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        o, lse = self.forward(q, k, v, cu_q, cu_k, scale, mode, window)
        tq, hq, d = q.shape
        tk, hkv, _ = k.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        dd = (dout * o).sum(axis=2)                       # [Tq, Hq]
        if "bwd_missing_d" in self.mut:
            dd = np.zeros_like(dd)
        for s in range(len(cu_q) - 1):
            rows = np.arange(int(cu_q[s]), int(cu_q[s + 1]))
            if len(rows) == 0:
                continue
            for u0 in range(int(cu_k[s]), int(cu_k[s + 1]), self.bn):
                keys = np.arange(u0, min(u0 + self.bn, tk))
                a = self._tile_allowed(rows, keys, s, cu_q, cu_k, tk, mode, window)
                for h in range(hq):
                    g = self._kv_head(h, hq, hkv)
                    sc = scale * (q[rows, h] @ k[keys, g].T)
                    fin = np.isfinite(lse[h, rows])[:, None]
                    p = np.where(a & fin, np.exp(sc - np.where(fin, lse[h, rows][:, None], 0)), 0)
                    dv[keys, g] += p.T @ dout[rows, h]
                    dp = dout[rows, h] @ v[keys, g].T
                    ds = p * (dp - dd[rows, h][:, None])
                    kscale = 1.0 if "bwd_no_scale_dk" in self.mut else scale
                    dk[keys, g] += kscale * (ds.T @ q[rows, h])
                    dq[rows, h] += scale * (ds @ k[keys, g])
        return dq, dk, dv

    def fwd_fn(self):
        return lambda q, k, v, cu_q, cu_k, scale, mode, window: self.forward(
            q, k, v, cu_q, cu_k, scale, mode, window)

    def bwd_fn(self):
        return lambda q, k, v, do, cu_q, cu_k, scale, mode, window: self.backward(
            q, k, v, do, cu_q, cu_k, scale, mode, window)


def two_tile_value(values, mutants=()):
    """The recurrence over two one-key tiles with logits 0 and ln 3 (exact-rational fixture)."""
    q = np.array([[[np.log(3.0)]]])
    k = np.array([[[0.0]], [[1.0]]])
    v = np.array([[[float(values[0])]], [[float(values[1])]]])
    o, _ = TiledModel(bm=1, bn=1, mutants=mutants).forward(q, k, v, [0, 1], [0, 2], 1.0, NONE, 0)
    return float(o[0, 0, 0])
