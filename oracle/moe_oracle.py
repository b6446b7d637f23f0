"""CPU oracle for the W4A16 INT4 MoE expert GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

It is a plain, slow, obviously correct restatement of what the method
computes, written from the Chord W4A16 MoE post ("vLLM x Novita AI: Chord,
a faster INT4 MoE for Kimi K2.x"):

* BF16 activations times INT4 weights with BF16 group-32 scales
  (post summary); weights are unsigned INT4 codes [G, N, K] with BF16 scales
  [G, N, K/32] (section "Grouped SM90 kernels", operator entry listing).
* Dequantisation is subtract-then-scale, rounded to BF16 the way the unfused
  form rounds it (section "H200 and Blackwell indexed decode"); the group
  scale is applied while dequantising, before the matrix product (section
  "H200 prefill and TP8", main-loop sketch: "dequant + group scale").
* Accumulation is FP32 or better: the FP16-accumulate option is not
  implemented by either backend (section "vLLM integration").
* Indexed routing consumes sorted_ids / expert_ids / num_tokens_padded, whose
  padding lives in sentinel index values; activations are not padded
  (section "Two kernel families"; "Grouped SM90 kernels", Figure 3).
* Grouped contiguous: rows concatenated per expert, padded to 128-row
  boundaries, m_indices = -1 on padding; output [m, N].  Grouped masked:
  fixed per-expert row budget, masked_m holds the valid counts, output flat
  [G*max_m, N] with rows past the count ignored (section "Grouped SM90
  kernels").

Where the post leaves a step open, the plainest reading is taken:
* zero point 8 for the unsigned codes, group axis K, group index kk // 32;
* one BF16 round-to-nearest-even of each output element;
* the top-k weights are applied in the down projection, summed over a
  token's local slots in full precision, then rounded once; weights are not
  renormalised over local experts; a token with no local slot gives 0;
* moe_align pads each local expert's segment to a multiple of block_m with
  the sentinel T*k, keeps slot ids ascending inside a segment, writes -1 into
  expert_ids past the padded total and the sentinel into the tail of
  sorted_ids.

Precision: dequantised weights are exact BF16 values held in float64;
products and sums are float64 (a library dgemm serves as the matrix product
step); the single BF16 rounding is done directly from float64, so there is no
double rounding.  The `*_fp32` functions are the same steps with float32
sums (library sgemm): they are the timed CPU baseline, not the parity
reference.

All BF16 tensors are passed as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
ZERO_POINT = 8


# ---------------------------------------------------------------- bf16 helpers

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even) directly,
    returning bit patterns.  bf16 keeps 8 significant bits, 8 exponent bits;
    below 2**-126 the spacing is fixed at 2**-133 (subnormals); values that
    round past the largest finite bf16 become infinity; NaN stays NaN."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    a = np.abs(v)
    small = a < 2.0 ** -126
    # normal range: keep 8 significant bits of the float64 significand (52
    # stored bits -> drop the low 45), ties to even, carry may bump exponent
    u = v.view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64(1) << np.uint64(44)
    lsb = (u >> drop) & np.uint64(1)
    r = (u + (half - np.uint64(1)) + lsb) & ~((np.uint64(1) << drop) - np.uint64(1))
    out[:] = r.view(np.float64)
    # subnormal range: multiples of 2**-133, np.round is ties-to-even
    if small.any():
        q = 2.0 ** -133
        out[small] = np.round(v[small] / q) * q
    nan = np.isnan(v)
    out[nan] = np.nan
    # anything at or beyond 2**128 after rounding is infinity in bf16
    big = np.abs(out) >= 2.0 ** 128
    out[big & ~nan] = np.copysign(np.inf, v[big & ~nan])
    f32 = out.astype(np.float32)  # exact: <= 8 significant bits, in range
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) -> bit patterns (fp32 baseline)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(v, dtype=np.float32))
    r[nan] = 0x7FC0
    return r


# ---------------------------------------------------------------- dequantise

def dequant(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """W[..., n, kk] = bf16_RNE((q - 8) * s[..., n, kk // 32]) as float64.

    Subtract-then-scale with one BF16 rounding (post, "H200 and Blackwell
    indexed decode": the fused dequant keeps the unfused BF16 rounding order).
    (q - 8) * s is exact in float64, so one rounding from float64 is that
    order."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    assert K % GROUP == 0 and scale_bits.shape[-1] == K // GROUP
    s = bf16_to_f64(scale_bits)
    s_full = np.repeat(s, GROUP, axis=-1)
    exact = (codes.astype(np.float64) - ZERO_POINT) * s_full
    return bf16_to_f64(f64_to_bf16(exact))


def dequant_rows(codes_e: np.ndarray, scale_bits_e: np.ndarray, rows=None) -> np.ndarray:
    """Dequantise one expert's [N, K] weight, optionally only output rows
    `rows` (used for sampled checks at full size)."""
    if rows is not None:
        codes_e = codes_e[rows]
        scale_bits_e = scale_bits_e[rows]
    return dequant(codes_e, scale_bits_e)


# ---------------------------------------------------------------- routing align

def align_capacity(T: int, k: int, E_loc: int, block_m: int) -> int:
    """Worst-case padded length: every slot local and every expert segment
    padded by block_m - 1 (over-allocation, post section "vLLM integration":
    the fast path consumes over-allocated buffers without a host readback)."""
    n = T * k + E_loc * (block_m - 1)
    return -(-n // block_m) * block_m


def moe_align(topk_ids: np.ndarray, E_glob: int, first: int, E_loc: int,
              block_m: int, capacity: int | None = None):
    """Counting sort of slots by local expert (post, "Two kernel families":
    the indexed family consumes sorted_ids / expert_ids / num_tokens_padded;
    Figure 3: padding lives in index sentinels).

    slot id s = t*k + j.  Local expert e = topk_ids[t, j] - first when that is
    in [0, E_loc); other slots (other GPUs' experts, or ids outside
    [0, E_glob)) are dropped.  n_e = slots of e; P_e = ceil(n_e / bm) * bm;
    segment of e starts at sum of P_e' for e' < e; inside it the slot ids of e
    ascending, then the sentinel T*k.  expert_ids[b] = e for the blocks of
    e's segment, -1 after.  num_tokens_padded = sum P_e.
    Returns (sorted_ids int32 [cap], expert_ids int32 [cap / bm], ntp int)."""
    T, k = topk_ids.shape
    cap = align_capacity(T, k, E_loc, block_m) if capacity is None else capacity
    sentinel = T * k
    flat = topk_ids.reshape(-1).astype(np.int64)
    sorted_ids = np.full(cap, sentinel, dtype=np.int32)
    expert_ids = np.full(cap // block_m, -1, dtype=np.int32)
    pos = 0
    for e in range(E_loc):
        g = first + e
        if g < 0 or g >= E_glob:
            continue
        slots = np.nonzero(flat == g)[0]          # ascending slot ids of expert g
        n = len(slots)
        P = -(-n // block_m) * block_m
        assert pos + P <= cap, "capacity too small"
        sorted_ids[pos:pos + n] = slots
        expert_ids[pos // block_m:(pos + P) // block_m] = e
        pos += P
    return sorted_ids, expert_ids, pos


# ---------------------------------------------------------------- GEMMs (fp64)

def _local(topk_ids: np.ndarray, first: int, E_loc: int, E_glob: int | None = None):
    g = topk_ids.astype(np.int64)
    e = g - first
    ok = (e >= 0) & (e < E_loc)
    if E_glob is not None:
        ok &= (g >= 0) & (g < E_glob)
    return e, ok


def indexed_gate_up(x_bits: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray,
                    topk_ids: np.ndarray, first: int, E_loc: int,
                    slots=None, cols=None):
    """Per-slot projection h[t*k + j, :] = bf16(x[t] . W[e]^T) for every local
    slot (t, j) with expert e (gate/up call of the indexed family; output
    per routed slot, non-local slots not produced).

    x_bits [T, K] bf16; codes [E_loc, N, K] u8; scale_bits [E_loc, N, K/32].
    `slots` / `cols` restrict the computation to a sample (full-size checks).
    Returns (out bits [len(slots), len(cols)], written mask [len(slots)])."""
    T, k = topk_ids.shape
    N = codes.shape[1]
    slots = np.arange(T * k) if slots is None else np.asarray(slots, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    e_all, ok_all = _local(topk_ids.reshape(-1), first, E_loc)
    e_s, ok_s = e_all[slots], ok_all[slots]
    out = np.zeros((len(slots), len(cols)), dtype=np.uint16)
    for e in np.unique(e_s[ok_s]):
        idx = np.nonzero(ok_s & (e_s == e))[0]
        W = dequant_rows(codes[e], scale_bits[e], cols)           # [len(cols), K]
        X = bf16_to_f64(x_bits[slots[idx] // k])                  # [n, K]
        out[idx] = f64_to_bf16(X @ W.T)
    return out, ok_s


def indexed_down_combine(a_bits: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray,
                         topk_ids: np.ndarray, topk_weights: np.ndarray, first: int,
                         E_loc: int, tokens=None, cols=None) -> np.ndarray:
    """Down projection with top-k-weighted combine:
    out[t, :] = bf16( sum over local j of w[t, j] * (a[t*k + j] . Wd[e]^T) ),
    one rounding after the full-precision weighted sum; weights used as
    given (not renormalised over local experts); no local slot -> 0.

    a_bits [T*k, K] bf16 (one row per slot); topk_weights float32 [T, k]."""
    T, k = topk_ids.shape
    N = codes.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    acc = np.zeros((len(tokens), len(cols)), dtype=np.float64)
    e_tk, ok_tk = _local(topk_ids[tokens], first, E_loc)
    w = topk_weights[tokens].astype(np.float64)
    for e in np.unique(e_tk[ok_tk]):
        ti, jj = np.nonzero(ok_tk & (e_tk == e))
        W = dequant_rows(codes[e], scale_bits[e], cols)
        A = bf16_to_f64(a_bits[tokens[ti] * k + jj])
        contrib = (A @ W.T) * w[ti, jj][:, None]
        np.add.at(acc, ti, contrib)
    return f64_to_bf16(acc)


def grouped_contiguous(a_bits: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray,
                       m_indices: np.ndarray, rows=None, cols=None):
    """Grouped contiguous call: out[r] = bf16(A[r] . W[m_indices[r]]^T) for
    rows with m_indices[r] >= 0; other rows are not defined (post, "Grouped
    SM90 kernels", contiguous prefill bullet and operator listing).
    Returns (out bits [rows, cols], valid mask)."""
    M = a_bits.shape[0]
    N = codes.shape[1]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    mi = np.asarray(m_indices, dtype=np.int64)[rows]
    out = np.zeros((len(rows), len(cols)), dtype=np.uint16)
    for e in np.unique(mi[mi >= 0]):
        idx = np.nonzero(mi == e)[0]
        W = dequant_rows(codes[e], scale_bits[e], cols)
        out[idx] = f64_to_bf16(bf16_to_f64(a_bits[rows[idx]]) @ W.T)
    return out, mi >= 0


def grouped_masked(a_bits: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray,
                   masked_m: np.ndarray, groups=None, cols=None):
    """Grouped masked call: A [G, max_m, K]; out flat [G*max_m, N] with
    out[g*max_m + r] = bf16(A[g, r] . W[g]^T) for r < masked_m[g]; rows past
    the count are ignored by consumers (post, "Grouped SM90 kernels", masked
    decode bullet and the note under the operator listing).
    Returns (out bits [len(groups)*max_m, cols], valid mask)."""
    G, max_m, K = a_bits.shape
    N = codes.shape[1]
    groups = np.arange(G) if groups is None else np.asarray(groups, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    out = np.zeros((len(groups) * max_m, len(cols)), dtype=np.uint16)
    valid = np.zeros(len(groups) * max_m, dtype=bool)
    for i, g in enumerate(groups):
        n = int(masked_m[g])
        if n == 0:
            continue
        W = dequant_rows(codes[g], scale_bits[g], cols)
        out[i * max_m:i * max_m + n] = f64_to_bf16(bf16_to_f64(a_bits[g, :n]) @ W.T)
        valid[i * max_m:i * max_m + n] = True
    return out, valid


def silu_mul(h_bits: np.ndarray) -> np.ndarray:
    """Activation between the two projections for chained checks only (not
    on the measured path; the post's layer numbers exclude it):
    bf16(silu(gate) * up) with gate = first half of the columns."""
    h = bf16_to_f64(h_bits)
    n = h.shape[-1] // 2
    g, u = h[..., :n], h[..., n:]
    return f64_to_bf16(g / (1.0 + np.exp(-g)) * u)


def gate_up_silu_sorted(h_bits: np.ndarray, sorted_ids: np.ndarray, sentinel: int):
    """The activation between the projections, placed in sorted order: for
    each sorted position p holding a slot s (sorted_ids[p] < sentinel),
    out[p] = silu_mul(h[s]), h the per-slot gate/up output.  Padding
    positions are not defined (mask False).  (The post excludes this step
    from its layer numbers, section "Measurement"; gate = first half of the
    gate/up columns.)
    Returns (out uint16 [len(sorted_ids), N/2], valid bool [len(sorted_ids)])."""
    sid = np.asarray(sorted_ids).astype(np.int64)
    valid = sid < sentinel
    out = np.zeros((len(sid), h_bits.shape[1] // 2), dtype=np.uint16)
    out[valid] = silu_mul(h_bits[sid[valid]])
    return out, valid


# ---------------------------------------------------------------- fp32 baseline

def indexed_gate_up_fp32(x_bits, codes, scale_bits, topk_ids, first, E_loc):
    """Timed CPU baseline: the same steps with float32 sums (sgemm)."""
    T, k = topk_ids.shape
    N = codes.shape[1]
    out = np.zeros((T * k, N), dtype=np.uint16)
    e_all, ok = _local(topk_ids.reshape(-1), first, E_loc)
    xf = bf16_to_f64(x_bits).astype(np.float32)
    for e in np.unique(e_all[ok]):
        idx = np.nonzero(ok & (e_all == e))[0]
        W = dequant(codes[e], scale_bits[e]).astype(np.float32)
        out[idx] = f32_to_bf16(xf[idx // k] @ W.T)
    return out


def indexed_down_combine_fp32(a_bits, codes, scale_bits, topk_ids, topk_weights, first, E_loc):
    T, k = topk_ids.shape
    N = codes.shape[1]
    acc = np.zeros((T, N), dtype=np.float32)
    e_tk, ok = _local(topk_ids, first, E_loc)
    for e in np.unique(e_tk[ok]):
        ti, jj = np.nonzero(ok & (e_tk == e))
        W = dequant(codes[e], scale_bits[e]).astype(np.float32)
        A = bf16_to_f64(a_bits[ti * k + jj]).astype(np.float32)
        np.add.at(acc, ti, (A @ W.T) * topk_weights[ti, jj][:, None])
    return f32_to_bf16(acc)


# ---------------------------------------------------------------- tolerance

def tolerance(ref_bits: np.ndarray, rel_rms: float = 1e-2) -> np.ndarray:
    """Per-element bound: rel_rms * RMS(reference) + one bf16 ulp at the
    reference value (spacing 2**(floor(log2|ref|) - 7); zero at ref = 0)."""
    ref = bf16_to_f64(ref_bits)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    a = np.abs(ref)
    ulp = np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 0.0)
    return rel_rms * rms + ulp
