"""Pins for the MXFP4 (A4W4) oracle, independent of its own code.

* the E2M1 value table and E8M0 scale values as the OCP Microscaling v1.0
  specification lists them (literal tables here, not the oracle's formula);
* round-to-nearest-even at every E2M1 tie and clamping past the largest
  normal, hand-computed;
* brute force: the nearest code by trying all sixteen, with exact rationals;
* closed forms: blocks of representable values survive quantisation
  unchanged; one-hot activations read back weight values exactly;
  power-of-two scale changes scale the output exactly;
* a scalar exact-rational triple loop against the vectorised GEMM oracle,
  and the dense special case against a library matmul.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import mx_oracle as X

# E2M1 magnitudes for codes 0..7 as the MX specification tabulates them
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32_bits_to_bf16(vals):
    """float values exactly representable in bf16 -> bit patterns."""
    f = np.asarray(vals, dtype=np.float32)
    assert np.all(f.view(np.uint32) & 0xFFFF == 0), "not exact in bf16"
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_e2m1_table():
    v = X.e2m1_to_f64(np.arange(16))
    assert list(v[:8]) == E2M1_TABLE
    assert list(v[8:]) == [-t for t in E2M1_TABLE]
    assert np.signbit(v[8]) and not np.signbit(v[0])          # code 8 is -0


def test_e8m0_values():
    got = X.e8m0_to_f64(np.array([0, 1, 126, 127, 128, 254, 255]))
    want = [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert list(got[:6]) == want and np.isnan(got[6])


@pytest.mark.parametrize("y,code", [
    (0.0, 0), (0.24, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.75, 2), (0.9, 2), (1.25, 2),
    (1.2500001, 3), (1.5, 3), (1.75, 4), (2.5, 4), (2.5000001, 5), (3.0, 5), (3.5, 6), (4.0, 6),
    (5.0, 6), (5.0000001, 7), (6.0, 7), (7.0, 7), (7.99, 7)])
def test_e2m1_rounding_ties_and_clamp(y, code):
    assert int(X.f64_to_e2m1(np.array(y))) == code
    assert int(X.f64_to_e2m1(np.array(-y))) == code | 8


def _nearest_brute(y: Fraction) -> int:
    best = None
    for c in range(16):
        v = Fraction(E2M1_TABLE[c & 7]) * (-1 if c & 8 else 1)
        if (c & 8) != (8 if y < 0 else 0):
            continue                                           # keep the input's sign
        d = abs(v - y)
        key = (d, (c & 1))                                     # nearest, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e2m1_nearest_brute_force():
    rng = np.random.default_rng(3)
    ys = np.concatenate([rng.uniform(-8, 8, 3000), np.arange(-31, 32) / 4.0])
    got = X.f64_to_e2m1(ys)
    for y, g in zip(ys, got):
        if y == 0:
            continue
        assert int(g) == _nearest_brute(Fraction(float(y))), y


def test_quantize_representable_blocks_roundtrip():
    rng = np.random.default_rng(4)
    R, K = 6, 128
    codes = rng.integers(0, 16, (R, K)).astype(np.uint8)
    k = rng.integers(-20, 20, (R, K // 32))
    # every block holds a +-4 or +-6 so its max |v| has floor(log2) = 2
    codes[:, ::32] = rng.choice([6, 7, 14, 15], (R, K // 32))
    vals = np.array([E2M1_TABLE[c & 7] * (-1 if c & 8 else 1) for c in codes.ravel()]).reshape(R, K)
    vals = vals * np.repeat(2.0 ** k, 32, axis=1)
    xb = f32_bits_to_bf16(vals)
    xb = np.where(codes == 8, np.uint16(0x8000), xb)           # -0 keeps its sign bit
    qc, qs = X.mx_quantize(xb)
    np.testing.assert_array_equal(qs, (k + 127).astype(np.uint8))
    np.testing.assert_array_equal(qc, codes)


def test_quantize_known_blocks():
    def one(block):
        qc, qs = X.mx_quantize(f32_bits_to_bf16(np.array(block, np.float32))[None])
        return list(qc[0]), int(qs[0, 0])
    z = [0.0] * 31
    assert one([1.0] + z) == ([6] + [0] * 31, 125)             # 1 = 4 * 2^-2
    assert one([0.0] * 32) == ([0] * 32, 0)                    # all zero: code 0
    assert one([7.0] + z) == ([7] + [0] * 31, 127)             # 7 / 1 clamps to 6
    assert one([0.75, -0.75] + [0.0] * 30) == ([7, 15] + [0] * 30, 124)   # 0.75 = 6 * 2^-3
    # X = 0.5: 3 -> 6; 0.375 -> 0.75, a tie between 0.5 and 1 -> 1 (even);
    # -0.125 -> -0.25, a tie between 0 and 0.5 -> -0 (code 8)
    assert one([3.0, 0.375, -0.125] + [0.0] * 29) == ([7, 2, 8] + [0] * 29, 126)
    tiny = float(np.float32(2.0 ** -130))                       # bf16 subnormal
    assert one([tiny] + z) == ([0] * 32, 0)                    # shared exponent clamps at -127


def test_quantize_error_bound():
    rng = np.random.default_rng(5)
    x = O.f64_to_bf16(rng.standard_normal((64, 256)) * np.repeat(2.0 ** rng.integers(-8, 8, (64, 8)), 32, 1))
    qc, qs = X.mx_quantize(x)
    v = O.bf16_to_f64(x)
    scale = np.repeat(X.e8m0_to_f64(qs), 32, axis=1)
    y = np.abs(v) / scale
    err = np.abs(X.mx_dequant(qc, qs) - v) / scale
    half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    assert np.all((err <= half_step) | (y > 6))
    assert np.all(err[y > 6] < 2.0) and np.all(y < 8)


def test_nibble_packing_order():
    assert X.pack_nibbles(np.array([1, 2, 15, 0], np.uint8)).tolist() == [0x21, 0x0F]
    c = np.random.default_rng(6).integers(0, 16, (3, 64)).astype(np.uint8)
    np.testing.assert_array_equal(X.unpack_nibbles(X.pack_nibbles(c)), c)


# ------------------------------------------------------------ GEMM pins

def _rand_mx(rng, shape_rows, K, scale_lo=120, scale_hi=130):
    codes = rng.integers(0, 16, shape_rows + (K,)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi, shape_rows + (K // 32,)).astype(np.uint8)
    return codes, scales


def test_gemm_one_hot_reads_weights():
    rng = np.random.default_rng(7)
    E, N, K, T, k = 3, 16, 64, 8, 2
    wc, ws = _rand_mx(rng, (E, N), K)
    cols = rng.integers(0, K, T)
    x = np.zeros((T, K), np.float32)
    x[np.arange(T), cols] = 1.0
    ac, as_ = X.mx_quantize(f32_bits_to_bf16(x))
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    h, ok = X.mx_indexed_gate_up(ac, as_, wc, ws, ids, 0, E)
    assert ok.all()
    for s in range(T * k):
        e, t = ids.reshape(-1)[s], s // k
        c = cols[t]
        want = [E2M1_TABLE[q & 7] * (-1 if q & 8 else 1) * 2.0 ** (int(sc) - 127)
                for q, sc in zip(wc[e, :, c], ws[e, :, c // 32])]
        np.testing.assert_array_equal(O.bf16_to_f64(h[s]), np.array(want))


def _exact_value(code, scale):
    return Fraction(E2M1_TABLE[code & 7]) * (-1 if code & 8 else 1) * Fraction(2) ** (int(scale) - 127)


def _rne_bf16(v: Fraction) -> float:
    """Exact rational -> nearest bf16 (ties to even), normal range."""
    if v == 0:
        return 0.0
    s = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    m = a * 128                                   # 8 significant bits
    fl = int(m)
    r = m - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(Fraction(fl, 128) * Fraction(2) ** e)


def test_gemm_brute_force_exact():
    rng = np.random.default_rng(8)
    E_glob, first, E, N, K, T, k = 5, 1, 3, 4, 64, 5, 2
    wc, ws = _rand_mx(rng, (E, N), K, 125, 129)
    ac, as_ = _rand_mx(rng, (T,), K, 125, 129)
    ids = rng.integers(0, E_glob, (T, k)).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    h, ok = X.mx_indexed_gate_up(ac, as_, wc, ws, ids, first, E)
    dc, ds = _rand_mx(rng, (T * k,), K, 125, 129)
    y = X.mx_indexed_down_combine(dc, ds, wc, ws, ids, tw, first, E)
    for t in range(T):
        tot = [Fraction(0)] * N
        for j in range(k):
            e = int(ids[t, j]) - first
            s = t * k + j
            if not (0 <= e < E):
                assert not ok[s]
                continue
            for n in range(N):
                g = sum(_exact_value(ac[t, kk], as_[t, kk // 32]) * _exact_value(wc[e, n, kk], ws[e, n, kk // 32])
                        for kk in range(K))
                assert float(O.bf16_to_f64(h[s, n])) == _rne_bf16(g)
                d = sum(_exact_value(dc[s, kk], ds[s, kk // 32]) * _exact_value(wc[e, n, kk], ws[e, n, kk // 32])
                        for kk in range(K))
                tot[n] += Fraction(float(tw[t, j])) * d
        for n in range(N):
            assert float(O.bf16_to_f64(y[t, n])) == _rne_bf16(tot[n])


def test_gemm_dense_special_case_matches_matmul():
    rng = np.random.default_rng(9)
    N, K, T = 48, 256, 24
    wc, ws = _rand_mx(rng, (1, N), K)
    ac, as_ = _rand_mx(rng, (T,), K)
    ids = np.zeros((T, 1), np.int32)
    h, _ = X.mx_indexed_gate_up(ac, as_, wc, ws, ids, 0, 1)
    a = torch.tensor([[float(_exact_value(c, as_[t, i // 32])) for i, c in enumerate(ac[t])] for t in range(T)],
                     dtype=torch.float64)
    w = torch.tensor([[float(_exact_value(c, ws[0, n, i // 32])) for i, c in enumerate(wc[0, n])] for n in range(N)],
                     dtype=torch.float64)
    ref = torch.matmul(a, w.T).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    # fp64 -> fp32 -> bf16 double rounding can differ by one ulp from the
    # direct rounding; compare within one bf16 ulp
    diff = np.abs(O.bf16_to_f64(h) - O.bf16_to_f64(ref))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(O.bf16_to_f64(ref)), 2.0 ** -120))) - 7)
    assert np.all(diff <= ulp)


def test_power_of_two_activation_scale():
    rng = np.random.default_rng(10)
    E, N, K, T, k = 2, 16, 128, 6, 2
    wc, ws = _rand_mx(rng, (E, N), K)
    ac, as_ = _rand_mx(rng, (T,), K)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    h1, _ = X.mx_indexed_gate_up(ac, as_, wc, ws, ids, 0, E)
    h2, _ = X.mx_indexed_gate_up(ac, as_ + 1, wc, ws, ids, 0, E)
    np.testing.assert_array_equal(O.bf16_to_f64(h2), 2 * O.bf16_to_f64(h1))
