"""Seeded synthetic attention inputs, shared by the tests, the bench and the oracle's callers.

This module only draws numbers and lays them out; it contains none of the attention
arithmetic (no logits, masks, softmax or reductions), so that the oracle and the HIP path
can both be fed from it without sharing any of the method.

Layout is THD: q is [total_q, Hq, d], k and v are [total_k, Hkv, d], contiguous, d fastest.
cu_seqlens arrays are int32 of length num_seqs + 1 with cu[0] = 0 ("Causal Mask and Ragged
Sequence Layouts", first section: a cumulative-length array locates each sequence's segment).

bf16 workloads are drawn in float32 and rounded to bfloat16 with round-to-nearest-even;
the float32 arrays returned here hold exactly the rounded values, so the oracle (which
upcasts them to float64) sees the same numbers as the device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

MASK_NONE = 0
MASK_CAUSAL_TOP_LEFT = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2

MASK_NAMES = {MASK_NONE: "none", MASK_CAUSAL_TOP_LEFT: "top_left",
              MASK_CAUSAL_BOTTOM_RIGHT: "bottom_right"}

# Lengths forced into the ragged pack: just below, at and just above 64- and 128-token
# tile edges ("Causal Mask and Ragged Sequence Layouts", fifth section).
FORCED_RAGGED_LENGTHS = (63, 64, 65, 127, 128, 129)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Inputs are finite normal draws, so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "bf16" or "f32": the element type of q, k, v, out (and grads)
    q: np.ndarray              # [total_q, Hq, d] float32 (bf16-representable when dtype == bf16)
    k: np.ndarray              # [total_k, Hkv, d]
    v: np.ndarray              # [total_k, Hkv, d]
    cu_q: np.ndarray           # [num_seqs + 1] int32
    cu_k: np.ndarray           # [num_seqs + 1] int32
    scale: float
    mask_mode: int
    window: int = 0
    dout: Optional[np.ndarray] = None   # [total_q, Hq, d], only for backward workloads
    seed: object = None

    @property
    def num_seqs(self) -> int:
        return int(self.cu_q.shape[0] - 1)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def total_k(self) -> int:
        return int(self.k.shape[0])

    @property
    def hq(self) -> int:
        return int(self.q.shape[1])

    @property
    def hkv(self) -> int:
        return int(self.k.shape[1])

    @property
    def d(self) -> int:
        return int(self.q.shape[2])

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_q).max()) if self.num_seqs > 0 else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(np.diff(self.cu_k).max()) if self.num_seqs > 0 else 0

    def with_mask(self, mask_mode: int, window: int = 0, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, mask_mode=mask_mode, window=window,
                                   name=name or self.name)

    def describe(self) -> dict:
        return {
            "workload": self.name, "dtype": self.dtype, "num_seqs": self.num_seqs,
            "total_q": self.total_q, "total_k": self.total_k, "hq": self.hq, "hkv": self.hkv,
            "d": self.d, "mask": MASK_NAMES[self.mask_mode], "window": self.window,
            "max_seqlen_q": self.max_seqlen_q, "max_seqlen_k": self.max_seqlen_k,
            "seed": repr(self.seed),
        }


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    assert cu[-1] < 2 ** 31
    return cu.astype(np.int32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def random_workload(seed, lengths_q, lengths_k, hq: int, hkv: int, d: int, dtype: str,
                    mask_mode: int, window: int = 0, with_dout: bool = False,
                    name: str = "custom", scale: Optional[float] = None,
                    v_offsets: bool = False) -> Workload:
    """Generic seeded generator; draw order q, k, v, dout (each standard normal float32).

    With ``v_offsets`` the values of sequence s become v * (s + 1) + 10 * s before rounding,
    so that a leak from one packed sequence into another shifts outputs far beyond tolerance
    ("Causal Mask and Ragged Sequence Layouts", fifth section: deliberately different value
    ranges).
    """
    rng = np.random.default_rng(seed)
    cu_q = cu_from_lengths(lengths_q)
    cu_k = cu_from_lengths(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _normal(rng, (tq, hq, d), dtype)
    k = _normal(rng, (tk, hkv, d), dtype)
    v = rng.standard_normal((tk, hkv, d), dtype=np.float32)
    if v_offsets:
        for s in range(len(lengths_k)):
            a, b = int(cu_k[s]), int(cu_k[s + 1])
            v[a:b] = v[a:b] * np.float32(s + 1) + np.float32(10 * s)
    if dtype == "bf16":
        v = round_to_bf16(v)
    dout = _normal(rng, (tq, hq, d), dtype) if with_dout else None
    return Workload(name=name, dtype=dtype, q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
                    mask_mode=mask_mode, window=window, dout=dout, seed=seed)


def ragged_lengths(seed: int, total: int = 16384, low: int = 1, high: int = 4096,
                   forced=FORCED_RAGGED_LENGTHS) -> list:
    """Lengths drawn uniformly from [low, high] until the pack holds ``total`` tokens.

    The forced lengths are reserved first; draws continue until they fill the rest, the last
    draw is cut to fit exactly, then the forced lengths are appended and the order permuted.
    """
    rng = np.random.default_rng(seed)
    budget = total - int(sum(forced))
    drawn = []
    while budget > 0:
        x = int(rng.integers(low, high + 1))
        x = min(x, budget)
        drawn.append(x)
        budget -= x
    lengths = np.array(drawn + list(forced), dtype=np.int64)
    return [int(x) for x in lengths[rng.permutation(len(lengths))]]


# ----------------------------------------------------------------------------------------
# The five named workloads (tiny fp32, dense bf16 prefill, ragged GQA, cached decode,
# forward+backward training shape).
# ----------------------------------------------------------------------------------------

def tiny_f32(mask_mode: int = MASK_CAUSAL_BOTTOM_RIGHT) -> Workload:
    """B=2, Hq=Hkv=2, Nq=Nk=128, d=64, fp32 inputs."""
    return random_workload(1, [128, 128], [128, 128], 2, 2, 64, "f32", mask_mode,
                           name="tiny_f32_b2_h2_n128_d64")


def dense_bf16(batch: int = 4, seqlen: int = 2048, heads: int = 16, d: int = 128,
               mask_mode: int = MASK_CAUSAL_TOP_LEFT, seed=2) -> Workload:
    """B=4, Hq=Hkv=16, N=2048, d=128, bf16, causal top-left."""
    lens = [seqlen] * batch
    return random_workload(seed, lens, lens, heads, heads, d, "bf16", mask_mode,
                           name=f"dense_bf16_b{batch}_h{heads}_n{seqlen}_d{d}")


def ragged_gqa(seed: int = 3, total: int = 16384, with_dout: bool = False,
               v_offsets: bool = True) -> Workload:
    """Packed ragged GQA: 16384 tokens, lengths U[1,4096] + forced, Hq=32, Hkv=8, d=128.

    ``with_dout`` adds the loss gradient (drawn after q, k, v, which stay the same);
    ``v_offsets=False`` keeps the values standard normal (the backward's variant)."""
    lens = ragged_lengths(seed, total=total)
    return random_workload((seed, 1), lens, lens, 32, 8, 128, "bf16", MASK_CAUSAL_TOP_LEFT,
                           v_offsets=v_offsets, with_dout=with_dout,
                           name=f"ragged_gqa_t{total}_hq32_hkv8_d128")


def decode(nq: int, nk: int = 32768, batch: int = 16) -> Workload:
    """Cached decode: B=16, Hq=32, Hkv=8, d=128, bf16, Nq query rows at the end of Nk keys."""
    return random_workload((4, nq, nk), [nq] * batch, [nk] * batch, 32, 8, 128, "bf16",
                           MASK_CAUSAL_BOTTOM_RIGHT,
                           name=f"decode_bf16_b{batch}_hq32_hkv8_nq{nq}_nk{nk}_d128")


def train_bf16(window: int = 0, seqlen: int = 8192, batch: int = 2, hq: int = 32, hkv: int = 8,
               d: int = 128) -> Workload:
    """Forward+backward: B=2, Hq=32, Hkv=8, N=8192, d=128, bf16, causal TL (+ window)."""
    lens = [seqlen] * batch
    tag = f"_w{window}" if window > 0 else ""
    return random_workload(5, lens, lens, hq, hkv, d, "bf16", MASK_CAUSAL_TOP_LEFT,
                           window=window, with_dout=True,
                           name=f"train_bf16_b{batch}_hq{hq}_hkv{hkv}_n{seqlen}_d{d}{tag}")
