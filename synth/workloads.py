"""Seeded synthetic inputs for the W4A16 MoE expert GEMM.

This module is the only code shared by the CPU oracle and the HIP path.  It
holds none of the method's arithmetic: it draws random numbers, rounds the
drawn activations and scales to bfloat16 with torch's own conversion (a
library round-to-nearest-even), runs a router to pick top-k experts, and
arranges rows into the grouped layouts.  Nothing here dequantises, multiplies
or combines.

Shapes and distributions follow the workloads the Chord W4A16 MoE post
(vLLM x Novita AI, "Chord ... INT4 MoE for Kimi K2.x") measures: Kimi K2.x
hidden size 7168, MoE intermediate 2048, 384 routed experts, top-8, as an
EP8 share (48 local experts) or a TP8 share (all 384 experts, intermediate
sliced by 8); the grouped contiguous and masked layouts follow that post's
"Grouped SM90 kernels" section (Figure 3).

Every tensor gets its own child seed from one root seed, so each tensor is
reproducible on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

GROUP = 32  # scale group along K (the post's "group-32")

# tensor tags -> child-seed index; fixed so adding a tensor never shifts others
_TAGS = {
    "logits": 0, "zipf_rank": 1, "zero_experts": 2, "x": 3, "a": 4,
    "w1_codes": 5, "w1_scales": 6, "w2_codes": 7, "w2_scales": 8,
    "w1_mx_codes": 9, "w1_mx_scales": 10, "w2_mx_codes": 11, "w2_mx_scales": 12,
}


def child_rng(root_seed: int, tag: str) -> np.random.Generator:
    ss = np.random.SeedSequence(root_seed)
    kids = ss.spawn(len(_TAGS))
    return np.random.Generator(np.random.PCG64(kids[_TAGS[tag]]))


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's library conversion and
    return the raw uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(root_seed: int, tag: str, rows: int, K: int) -> np.ndarray:
    """bf16 bit patterns of N(0, 1) draws, shape [rows, K]."""
    rng = child_rng(root_seed, tag)
    return to_bf16_bits(rng.standard_normal((rows, K), dtype=np.float32))


def weight_codes(root_seed: int, tag: str, E: int, N: int, K: int) -> np.ndarray:
    """Unsigned INT4 codes, uniform on 0..15, one code per byte, [E, N, K]."""
    rng = child_rng(root_seed, tag)
    return rng.integers(0, 16, size=(E, N, K), dtype=np.uint8)


def weight_scales(root_seed: int, tag: str, E: int, N: int, K: int,
                  lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    """bf16 bit patterns of U[lo, hi] group scales, [E, N, K/32]."""
    assert K % GROUP == 0
    rng = child_rng(root_seed, tag)
    return to_bf16_bits(rng.uniform(lo, hi, size=(E, N, K // GROUP)).astype(np.float32))


def mx_weight_codes(root_seed: int, tag: str, E: int, N: int, K: int) -> np.ndarray:
    """MXFP4 weight codes, every 4-bit E2M1 code uniform on 0..15, stored two
    per byte: uniform bytes [E, N, K/2]."""
    rng = child_rng(root_seed, tag)
    return rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)


def mx_weight_scales(root_seed: int, tag: str, E: int, N: int, K: int,
                     lo: int = 120, hi: int = 123) -> np.ndarray:
    """E8M0 scale codes uniform on [lo, hi) (2^-7 .. 2^-5 by default: weights
    of magnitude up to about 0.19, like the INT4 weights' range), [E, N, K/32]."""
    assert K % GROUP == 0
    rng = child_rng(root_seed, tag)
    return rng.integers(lo, hi, size=(E, N, K // GROUP), dtype=np.uint8)


def route(root_seed: int, T: int, E_glob: int, topk: int,
          zipf_s: Optional[float] = None,
          zero_experts: Sequence[int] = ()) -> tuple[np.ndarray, np.ndarray]:
    """Router: logits ~ N(0,1) per (token, expert); optional Zipf expert bias
    rank^(-s) with rank a seeded permutation of 1..E_glob; experts listed in
    `zero_experts` never chosen.  Top-k by logit (ties -> lower expert id),
    weights = softmax over the k chosen logits (softmax top-k, renormalised).
    Returns topk_ids int32 [T, k] and topk_weights float32 [T, k]."""
    rng = child_rng(root_seed, "logits")
    logits = rng.standard_normal((T, E_glob))
    if zipf_s is not None:
        rank = child_rng(root_seed, "zipf_rank").permutation(E_glob) + 1
        logits = logits + rank.astype(np.float64) ** (-zipf_s)
    if len(zero_experts):
        logits[:, np.asarray(zero_experts, dtype=np.int64)] = -np.inf
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    chosen = np.take_along_axis(logits, order, axis=1)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def local_slot_lists(topk_ids: np.ndarray, first: int, E_loc: int) -> list[np.ndarray]:
    """For each local expert, the slot ids (t*k + j) routed to it, ascending."""
    flat = topk_ids.reshape(-1).astype(np.int64)
    out = []
    for e in range(E_loc):
        out.append(np.nonzero(flat == first + e)[0])
    return out


def contiguous_layout(topk_ids: np.ndarray, x_bits: np.ndarray, first: int, E_loc: int,
                      pad: int = 128, pad_fill: int = 0) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Grouped contiguous layout: each local expert's rows (its tokens, in slot
    order) concatenated, each expert padded to a multiple of `pad` rows; padding
    rows hold `pad_fill` (bf16 bits) and m_indices -1 there.
    Returns A bits [M, K], m_indices int32 [M], and the slot id of each row
    (-1 on padding)."""
    k = topk_ids.shape[1]
    K = x_bits.shape[1]
    lists = local_slot_lists(topk_ids, first, E_loc)
    rows, mids, slots = [], [], []
    for e, sl in enumerate(lists):
        n = len(sl)
        if n == 0:
            continue
        P = -(-n // pad) * pad
        blk = np.full((P, K), pad_fill, dtype=np.uint16)
        blk[:n] = x_bits[sl // k]
        rows.append(blk)
        mids.append(np.concatenate([np.full(n, e, np.int32), np.full(P - n, -1, np.int32)]))
        slots.append(np.concatenate([sl, np.full(P - n, -1, np.int64)]))
    if not rows:
        return (np.zeros((0, K), np.uint16), np.zeros(0, np.int32), np.zeros(0, np.int64))
    return np.concatenate(rows), np.concatenate(mids), np.concatenate(slots)


def masked_layout(topk_ids: np.ndarray, x_bits: np.ndarray, first: int, E_loc: int,
                  max_m: int, pad_fill: int = 0) -> tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """Grouped masked layout: A [E_loc, max_m, K]; row r of group g is the r-th
    slot (ascending) routed to local expert g, for r < masked_m[g] =
    min(count, max_m); the rest hold `pad_fill`.  Slots beyond max_m are
    dropped.  Returns A bits, masked_m int32 [E_loc], slot ids [E_loc, max_m]
    (-1 where unused), and the number of dropped slots."""
    k = topk_ids.shape[1]
    K = x_bits.shape[1]
    A = np.full((E_loc, max_m, K), pad_fill, dtype=np.uint16)
    mm = np.zeros(E_loc, np.int32)
    slots = np.full((E_loc, max_m), -1, np.int64)
    dropped = 0
    for e, sl in enumerate(local_slot_lists(topk_ids, first, E_loc)):
        n = min(len(sl), max_m)
        dropped += len(sl) - n
        mm[e] = n
        A[e, :n] = x_bits[sl[:n] // k]
        slots[e, :n] = sl[:n]
    return A, mm, slots, dropped


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """One projection pair of a MoE layer share on one GPU."""
    name: str
    E_glob: int      # routed experts in the model
    E_loc: int       # experts held by this GPU: [first, first + E_loc)
    first: int
    topk: int
    T: int           # tokens
    K1: int          # gate/up reduction (hidden)
    N1: int          # gate/up output (2 x intermediate share)
    K2: int          # down reduction (intermediate share)
    N2: int          # down output (hidden)
    zipf_s: Optional[float] = None
    n_zero_experts: int = 0
    max_m: int = 0   # masked layout row budget (grouped workload only)
    seed: int = 0


def _cfg(i: int, **kw) -> MoEShape:
    return MoEShape(seed=20261202 + i, **kw)


# The five synthetic workloads (sizes of the Kimi K2.x shares described above).
WORKLOADS = {
    "tiny": _cfg(0, name="tiny", E_glob=8, E_loc=8, first=0, topk=2, T=64,
                 K1=256, N1=512, K2=256, N2=256),
    "ep8_decode": _cfg(1, name="ep8_decode", E_glob=384, E_loc=48, first=0, topk=8, T=576,
                       K1=7168, N1=4096, K2=2048, N2=7168),
    "ep8_prefill": _cfg(2, name="ep8_prefill", E_glob=384, E_loc=48, first=0, topk=8, T=8192,
                        K1=7168, N1=4096, K2=2048, N2=7168, zipf_s=1.0),
    "grouped_skewed": _cfg(4, name="grouped_skewed", E_glob=384, E_loc=48, first=0, topk=8,
                           T=16384, K1=7168, N1=4096, K2=2048, N2=7168, zipf_s=1.2,
                           n_zero_experts=4, max_m=512),
}
TP8_TOKENS = (1, 16, 128, 1024, 4096)
for _t in TP8_TOKENS:
    WORKLOADS[f"tp8_t{_t}"] = _cfg(3, name=f"tp8_t{_t}", E_glob=384, E_loc=384, first=0,
                                   topk=8, T=_t, K1=7168, N1=512, K2=256, N2=7168)

# Second workloads on the same kernels: the EP16 and EP32 shares of the same
# layer (24 and 12 local experts; the Chord post's grouped tables cover EP8,
# EP16 and EP32), and a Kimi-K3-like routing shape (16 of 896 experts per
# token, AMD's Kimi-K3 post) on the K2.x projection shapes, since that post
# gives the routing but not the projection sizes.
for _i, (_name, _eloc, _T, _zipf) in enumerate((("ep16_decode", 24, 576, None), ("ep32_decode", 12, 576, None),
                                                ("ep16_prefill", 24, 8192, 1.0), ("ep32_prefill", 12, 8192, 1.0))):
    WORKLOADS[_name] = _cfg(5 + _i, name=_name, E_glob=384, E_loc=_eloc, first=0, topk=8, T=_T,
                            K1=7168, N1=4096, K2=2048, N2=7168, zipf_s=_zipf)
WORKLOADS["k3_decode"] = _cfg(9, name="k3_decode", E_glob=896, E_loc=112, first=0, topk=16, T=576,
                              K1=7168, N1=4096, K2=2048, N2=7168)


def zero_expert_ids(shape: MoEShape) -> np.ndarray:
    """Seeded choice of local experts that receive no rows."""
    if shape.n_zero_experts == 0:
        return np.zeros(0, np.int64)
    rng = child_rng(shape.seed, "zero_experts")
    return shape.first + rng.choice(shape.E_loc, size=shape.n_zero_experts, replace=False)


def routing_for(shape: MoEShape, T: Optional[int] = None):
    T = shape.T if T is None else T
    return route(shape.seed, T, shape.E_glob, shape.topk, shape.zipf_s, zero_expert_ids(shape))


def scaled(shape: MoEShape, **changes) -> MoEShape:
    """Same workload recipe at other sizes (for parity cases that the oracle
    finishes in seconds)."""
    return dataclasses.replace(shape, **changes)
