"""CPU oracle for the A4W4 (MXFP4 x MXFP4) MoE expert GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
never calls it, and this module imports nothing from the product path.

What the pages fix:
* The AMD Kimi K3 post ("Blick hinter die Kulissen der Kimi-K3-Optimierung",
  technical note "Experten-Routing und Praezision") describes A4W4 as taking
  the MoE activations from eight to four bits while the weights stay 4-bit;
  the same post serves the model with MXFP4 weights (section "MLA", table
  note) and quotes the MI355X dense peak for MXFP4 (introduction).
* Routing is the indexed form of the W4A16 path (sorted_ids / expert_ids /
  num_tokens_padded, sentinel padding), so per-slot outputs and the top-k
  combine are those of `moe_oracle`.

Where the pages are silent, the plainest reading is taken: MXFP4 is the
OCP Microscaling v1.0 format -- blocks of 32 consecutive K elements in FP4
E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; no inf or NaN)
sharing one E8M0 scale 2^(c - 127) (c = 255 is NaN) -- and activations are
quantised per row and per block of 32 K the way that specification converts
a vector:
  shared exponent  = floor(log2(max |v|)) - 2   (2 = exponent of E2M1's
                     largest normal, 6 = 1.5 * 2^2), clamped to [-127, 127];
                     a block of zeros takes code 0;
  element          = v / 2^shared rounded to the nearest E2M1 value, ties to
                     the even mantissa, magnitudes past 6 clamp to 6; the
                     sign bit is the input's sign bit (so -0 and negative
                     values that round to zero give code 8).
Products and sums are float64; each output is rounded once to BF16.

Codes are uint8 arrays holding one 4-bit code per element; scales are uint8
E8M0 codes; BF16 tensors are uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from oracle.moe_oracle import bf16_to_f64, f64_to_bf16

BLOCK = 32          # elements per shared scale
EMAX_ELEM = 2       # exponent of E2M1's largest normal value


# ------------------------------------------------------------ element format

def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 code -> value: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (mantissa * 0.5)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return sign * mag


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale code -> 2^(c - 127); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    v = np.ldexp(1.0, (c - 127).astype(np.int32))
    return np.where(c == 255, np.nan, v)


_MAG_CODES = np.arange(8)


def f64_to_e2m1(y: np.ndarray, negative: np.ndarray | None = None) -> np.ndarray:
    """Nearest E2M1 code to y (ties to the even mantissa bit, i.e. the even
    code; beyond 6 the nearest finite value is 6).  `negative` gives the sign
    bit where y itself is zero or its sign is not the input's."""
    y = np.asarray(y, dtype=np.float64)
    mags = e2m1_to_f64(_MAG_CODES)                       # 0, .5, 1, 1.5, 2, 3, 4, 6
    d = np.abs(np.abs(y)[..., None] - mags)              # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    tied = d == best
    # among the nearest magnitudes prefer an even code (mantissa bit 0)
    even_pref = np.where(tied & (_MAG_CODES % 2 == 0), 1, 0) + np.where(tied, 1, 0)
    code = np.argmax(even_pref, axis=-1)
    neg = np.signbit(y) if negative is None else np.asarray(negative, dtype=bool)
    return (code | np.where(neg, 8, 0)).astype(np.uint8)


# ------------------------------------------------------------ quantisation

def mx_quantize(x_bits: np.ndarray, rows_per_slice: int = 2048):
    """BF16 rows [R, K] (K % 32 == 0) -> (codes uint8 [R, K], scales uint8
    [R, K/32]) by the per-block conversion in the module docstring.  Rows are
    independent; they are converted a slice at a time to bound memory."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    assert K % BLOCK == 0
    if R > rows_per_slice:
        parts = [_mx_quantize_rows(x_bits[i:i + rows_per_slice]) for i in range(0, R, rows_per_slice)]
        return np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts])
    return _mx_quantize_rows(x_bits)


def _mx_quantize_rows(x_bits: np.ndarray):
    R, K = x_bits.shape
    v = bf16_to_f64(x_bits).reshape(R, K // BLOCK, BLOCK)
    negative = ((x_bits >> 15) & 1).astype(bool).reshape(R, K // BLOCK, BLOCK)
    amax = np.abs(v).max(axis=-1)
    mant, ex = np.frexp(amax)                           # amax = mant * 2^ex, mant in [0.5, 1)
    floor_log2 = ex.astype(np.int64) - 1
    shared = np.clip(floor_log2 - EMAX_ELEM, -127, 127)
    scale = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    y = v / e8m0_to_f64(scale)[..., None]
    codes = f64_to_e2m1(y, negative)
    return codes.reshape(R, K), scale


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., K] and scales [..., K/32] -> float64 values [..., K]."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    s = np.repeat(e8m0_to_f64(scales), BLOCK, axis=-1)[..., :K]
    return e2m1_to_f64(codes) * s


# ------------------------------------------------------------ MoE GEMMs

def _local_slots(topk_ids: np.ndarray, first: int, E_loc: int):
    flat = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    e = flat - first
    ok = (flat >= 0) & (e >= 0) & (e < E_loc)
    return e, ok


def mx_indexed_gate_up(a_codes, a_scales, w_codes, w_scales, topk_ids, first, E_loc):
    """Per-slot output h[t*k + j] = bf16(A[t] . W[e]^T) for local slots,
    activation row = token; other rows are left 0 with valid = False.
    A: codes [T, K] + scales [T, K/32]; W: codes [E, N, K] + scales [E, N, K/32]."""
    T, k = np.asarray(topk_ids).shape
    N = w_codes.shape[1]
    A = mx_dequant(a_codes, a_scales)
    e, ok = _local_slots(topk_ids, first, E_loc)
    out = np.zeros((T * k, N), np.uint16)
    for ex in range(E_loc):
        slots = np.nonzero(ok & (e == ex))[0]
        if len(slots) == 0:
            continue
        W = mx_dequant(w_codes[ex], w_scales[ex])
        out[slots] = f64_to_bf16(A[slots // k] @ W.T)
    return out, ok


def mx_indexed_down_combine(a_codes, a_scales, w_codes, w_scales, topk_ids, topk_weights, first, E_loc):
    """out[t] = bf16(sum over local j, of w[t, j] * (A[t*k + j] . W[e]^T)),
    activation row = slot; tokens with no local slot give 0."""
    T, k = np.asarray(topk_ids).shape
    N = w_codes.shape[1]
    A = mx_dequant(a_codes, a_scales)
    e, ok = _local_slots(topk_ids, first, E_loc)
    wt = np.asarray(topk_weights, dtype=np.float64).reshape(-1)
    acc = np.zeros((T * k, N), np.float64)
    for ex in range(E_loc):
        slots = np.nonzero(ok & (e == ex))[0]
        if len(slots) == 0:
            continue
        W = mx_dequant(w_codes[ex], w_scales[ex])
        acc[slots] = (A[slots] @ W.T) * wt[slots, None]
    return f64_to_bf16(acc.reshape(T, k, N).sum(axis=1))


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """One code per byte [..., K] -> two per byte [..., K/2], element 2i in
    the low nibble (the usual MXFP4 storage order)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out
