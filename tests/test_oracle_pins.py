"""Pins for the CPU oracle, independent of the oracle's own code.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, double rounding, renormalised
weights) fails at least one of them:

* exact rational arithmetic (fractions.Fraction) with an exact rational
  round-to-nearest-even written here, on tiny shapes (brute force);
* torch's bfloat16 conversion (a library routine) on float32 inputs;
* the one worked rounding example the pages print (AMD Kimi-K3 post, KDA
  precision note: 256.5 -> 256 in BF16);
* closed forms (one-hot activations, zero codes, power-of-two scaling);
* invariants (token order, duplicate experts, non-local slots, sentinels).
"""
import itertools
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ exact helpers

def bits_to_fraction(b: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    return Fraction(f)


def rne_bf16_fraction(v: Fraction) -> int:
    """Exact RNE of a rational to bf16 (normal and subnormal range), bits."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # below 2^-126 spacing is 2^-133
    ulp = Fraction(2) ** (e - 7)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f32 = struct.unpack("<I", struct.pack("<f", float(val)))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", f32))[0]) == val
    return sign | (f32 >> 16)


def torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------ bf16 rounding

def test_golden_bf16_example_from_amd_post():
    g = json.load(open(os.path.join(GOLDEN, "bf16_rounding_amd_kimi_k3.json")))
    for x, y in g["round_to_bf16"]:
        assert O.bf16_to_f64(O.f64_to_bf16(np.array([x])))[0] == y
        assert O.bf16_to_f64(O.f32_to_bf16(np.array([x], np.float32)))[0] == y
    s = g["subtract_fp32"]
    a32, b32 = np.float32(s["a"]), np.float32(s["b"])
    assert float(a32 - b32) == s["keep_fp32_inputs"]
    ab = O.bf16_to_f64(O.f64_to_bf16(np.array([s["a"], s["b"]])))
    assert float(np.float32(ab[0]) - np.float32(ab[1])) == s["bf16_inputs_first"]


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # force exact ties: values with bit 15 set and low bits zero
    u = v.view(np.uint32).copy()
    u[:5000] = (u[:5000] & 0xFFFF0000) | 0x8000
    u[5000:10000] = (u[5000:10000] & 0xFFFF0000) | 0x7FFF
    u[10000:15000] = (u[10000:15000] & 0xFFFF0000) | 0x8001
    v = u.view(np.float32)
    ref = torch_bf16_bits(v)
    np.testing.assert_array_equal(O.f64_to_bf16(v.astype(np.float64)), ref)
    np.testing.assert_array_equal(O.f32_to_bf16(v), ref)


def test_bf16_rounding_no_double_rounding():
    # 1 + 2^-8 + 2^-40: above the tie, must round up; via fp32 it would become
    # the tie 1 + 2^-8 and round down to 1.0.
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8 + 2.0 ** -40),
                  1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    got = O.bf16_to_f64(O.f64_to_bf16(v))
    assert list(got) == [1 + 2.0 ** -7, -(1 + 2.0 ** -7), 1.0, 1 + 2.0 ** -6]


def test_bf16_rounding_exact_rational_random():
    rng = np.random.default_rng(2)
    mant = rng.integers(1, 2 ** 52, 3000)
    ex = rng.integers(-140, 130, 3000)
    sg = rng.choice([-1, 1], 3000)
    vals = [float(s * (1 + Fraction(int(m), 2 ** 52)) * Fraction(2) ** int(e))
            if -1074 < e < 1000 else 0.0 for s, m, e in zip(sg, mant, ex)]
    v = np.array(vals)
    got = O.f64_to_bf16(v)
    for i in range(len(vals)):
        assert int(got[i]) == rne_bf16_fraction(Fraction(vals[i])), (vals[i], hex(got[i]))


def test_bf16_special_values():
    v = np.array([2.0 ** -134, 3 * 2.0 ** -134, 1.5 * 2.0 ** -133 * 2, (2 - 2.0 ** -8) * 2.0 ** 127,
                  (2 - 2.0 ** -7) * 2.0 ** 127, np.inf, -np.inf])
    got = O.f64_to_bf16(v)
    assert got[0] == 0x0000                     # half of min subnormal, tie -> even (0)
    assert got[1] == 0x0002                     # 1.5 min subnormals -> 2 (even)
    assert got[3] == 0x7F80                     # tie above max finite -> inf
    assert got[4] == 0x7F7F                     # max finite stays
    assert got[5] == 0x7F80 and got[6] == 0xFF80
    assert np.isnan(O.bf16_to_f64(O.f64_to_bf16(np.array([np.nan]))))[0]


# ------------------------------------------------------------ dequantisation

def test_dequant_exact_rational_all_codes():
    rng = np.random.default_rng(3)
    s_bits = W.to_bf16_bits(rng.uniform(-3, 3, 64).astype(np.float32))
    s_bits[:4] = W.to_bf16_bits(np.array([0.0078125 * 1.0078125, 1e-30, 3e37, 0.01], np.float32))
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :].repeat(64, 0)  # [64, 32]
    got = O.f64_to_bf16(O.dequant(codes, s_bits[:, None]))
    for n in range(64):
        s = bits_to_fraction(s_bits[n])
        for kk in range(32):
            want = rne_bf16_fraction((int(codes[n, kk]) - 8) * s)
            assert int(got[n, kk]) & 0x7FFF == want & 0x7FFF
            if want & 0x7FFF:
                assert int(got[n, kk]) == want


def test_dequant_closed_forms_and_group_index():
    K, N = 256, 6
    rng = np.random.default_rng(4)
    s_bits = W.to_bf16_bits(rng.uniform(0.005, 0.02, (N, K // 32)).astype(np.float32))
    s = O.bf16_to_f64(s_bits)
    for q, mult in [(8, 0.0), (9, 1.0), (10, 2.0), (12, 4.0), (0, -8.0), (7, -1.0), (6, -2.0)]:
        codes = np.full((N, K), q, np.uint8)
        Wd = O.dequant(codes, s_bits)
        np.testing.assert_array_equal(Wd, mult * np.repeat(s, 32, axis=1))
    # group index is kk // 32 along K, per output row n (not n-major, not kk % groups)
    codes = np.full((N, K), 9, np.uint8)
    Wd = O.dequant(codes, s_bits)
    for n in range(N):
        for kk in range(K):
            assert Wd[n, kk] == s[n, kk // 32]


# ------------------------------------------------------------ routing align

def _check_align(topk_ids, E_glob, first, E_loc, bm, sorted_ids, expert_ids, ntp):
    T, k = topk_ids.shape
    sentinel = T * k
    flat = topk_ids.reshape(-1)
    local = {s: int(flat[s]) - first for s in range(T * k) if first <= flat[s] < first + E_loc}
    assert ntp % bm == 0
    assert all(sorted_ids[ntp:] == sentinel) and all(expert_ids[ntp // bm:] == -1)
    got = [int(s) for s in sorted_ids[:ntp] if s != sentinel]
    assert sorted(got) == sorted(local)
    pos, seen = 0, []
    while pos < ntp:
        e = int(expert_ids[pos // bm])
        assert 0 <= e < E_loc and e not in seen
        seen.append(e)
        seg_end = pos
        while seg_end < ntp and expert_ids[seg_end // bm] == e:
            seg_end += bm
        seg = [int(s) for s in sorted_ids[pos:seg_end]]
        valid = [s for s in seg if s != sentinel]
        assert seg[:len(valid)] == valid                         # sentinels only at the end
        assert valid == sorted(valid)                            # ascending slot ids
        assert all(local[s] == e for s in valid)
        assert len(valid) > seg_end - pos - bm                   # minimal padding
        pos = seg_end
    assert seen == sorted(seen)                                  # expert order
    assert set(seen) == set(local.values())


def test_align_brute_force_all_tiny_routings():
    n = 0
    for T, k, E_glob in [(1, 1, 3), (2, 1, 3), (3, 2, 3), (2, 2, 2)]:
        for ids in itertools.product(range(E_glob), repeat=T * k):
            topk = np.array(ids, dtype=np.int32).reshape(T, k)
            for first, E_loc in [(0, E_glob), (1, E_glob - 1), (0, 1)]:
                for bm in (1, 2, 4):
                    si, ei, ntp = O.moe_align(topk, E_glob, first, E_loc, bm)
                    assert len(si) == O.align_capacity(T, k, E_loc, bm)
                    _check_align(topk, E_glob, first, E_loc, bm, si, ei, ntp)
                    n += 1
    assert n > 1000


def test_align_worked_example():
    # T=3, k=2: slots 0..5 -> experts [2,0 | 0,1 | 2,2]; bm=2, all local
    topk = np.array([[2, 0], [0, 1], [2, 2]], np.int32)
    si, ei, ntp = O.moe_align(topk, 3, 0, 3, 2)
    S = 6
    assert ntp == 8
    assert list(si[:8]) == [1, 2, 3, S, 0, 4, 5, S]
    assert list(ei[:4]) == [0, 1, 2, 2]
    # EP share: experts 1..2 local (first=1)
    si, ei, ntp = O.moe_align(topk, 3, 1, 2, 2)
    assert ntp == 6 and list(si[:6]) == [3, S, 0, 4, 5, S] and list(ei[:3]) == [0, 1, 1]


# ------------------------------------------------------------ GEMM: exact brute force

def _tiny_problem(seed, T=3, k=2, E=3, N=5, K=64, integer_x=True):
    rng = np.random.default_rng(seed)
    if integer_x:   # small dyadic values: every fp64 sum below is exact
        x = W.to_bf16_bits((rng.integers(-4, 5, (T, K)) * 0.25).astype(np.float32))
    else:
        x = W.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    codes = rng.integers(0, 16, (E, N, K), dtype=np.uint8)
    sc = W.to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    return x, codes, sc, ids, w


def _exact_W(codes, sc, e, n, kk):
    return bits_to_fraction(rne_bf16_fraction((int(codes[e, n, kk]) - 8) * bits_to_fraction(sc[e, n, kk // 32])))


def test_gate_up_exact_brute_force():
    for seed in range(3):
        x, codes, sc, ids, _ = _tiny_problem(seed)
        T, k = ids.shape
        E, N, K = codes.shape
        out, ok = O.indexed_gate_up(x, codes, sc, ids, 0, E)
        assert ok.all()
        for t, j, n in itertools.product(range(T), range(k), range(N)):
            e = int(ids[t, j])
            acc = sum(bits_to_fraction(x[t, kk]) * _exact_W(codes, sc, e, n, kk) for kk in range(K))
            assert int(out[t * k + j, n]) == rne_bf16_fraction(acc), (t, j, n)


def test_down_combine_exact_brute_force():
    for seed in range(3):
        a_tok, codes, sc, ids, w = _tiny_problem(10 + seed, T=4, k=3, E=4, N=6, K=96)
        T, k = ids.shape
        E, N, K = codes.shape
        rng = np.random.default_rng(seed)
        a = W.to_bf16_bits((rng.integers(-4, 5, (T * k, K)) * 0.5).astype(np.float32))
        first, E_loc = 1, 2        # only experts 1, 2 are local; others dropped, no renormalising
        out = O.indexed_down_combine(a, codes[first:first + E_loc], sc[first:first + E_loc], ids, w, first, E_loc)
        for t, n in itertools.product(range(T), range(N)):
            acc = Fraction(0)
            for j in range(k):
                e = int(ids[t, j])
                if not first <= e < first + E_loc:
                    continue
                dot = sum(bits_to_fraction(a[t * k + j, kk]) * _exact_W(codes, sc, e, n, kk) for kk in range(K))
                acc += Fraction(float(w[t, j])) * dot
            assert int(out[t, n]) == rne_bf16_fraction(acc), (t, n)


def test_gate_up_random_normal_within_one_ulp_of_exact():
    x, codes, sc, ids, _ = _tiny_problem(7, T=2, k=2, E=2, N=4, K=128, integer_x=False)
    out, _ = O.indexed_gate_up(x, codes, sc, ids, 0, 2)
    for t, j, n in itertools.product(range(2), range(2), range(4)):
        e = int(ids[t, j])
        acc = sum(bits_to_fraction(x[t, kk]) * _exact_W(codes, sc, e, n, kk) for kk in range(128))
        want = rne_bf16_fraction(acc)
        assert abs(int(out[t * 2 + j, n]) - want) <= 1


# ------------------------------------------------------------ GEMM: closed forms and invariants

def test_one_hot_activation_returns_weight_column():
    E, N, K = 3, 40, 96          # N != K catches a transposed operand
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (E, N, K), dtype=np.uint8)
    sc = W.to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    T, k = K, 1
    x = W.to_bf16_bits(np.eye(K, dtype=np.float32))      # token t is one-hot at kk = t
    ids = (np.arange(T) % E).astype(np.int32)[:, None]
    out, _ = O.indexed_gate_up(x, codes, sc, ids, 0, E)
    for t in range(T):
        e = t % E
        for n in range(N):
            assert int(out[t, n]) == rne_bf16_fraction(_exact_W(codes, sc, e, n, t))


def test_code_eight_gives_zero_and_power_of_two_scaling():
    x, codes, sc, ids, w = _tiny_problem(8, T=5, k=2, E=3, N=8, K=64, integer_x=False)
    out0, _ = O.indexed_gate_up(x, np.full_like(codes, 8), sc, ids, 0, 3)
    assert not out0.any()
    out1, _ = O.indexed_gate_up(x, codes, sc, ids, 0, 3)
    x2 = W.to_bf16_bits((O.bf16_to_f64(x) * 4).astype(np.float32))
    out2, _ = O.indexed_gate_up(x2, codes, sc, ids, 0, 3)
    np.testing.assert_array_equal(O.bf16_to_f64(out2), 4 * O.bf16_to_f64(out1))
    sc2 = W.to_bf16_bits((O.bf16_to_f64(sc) * 0.5).astype(np.float32))
    out3, _ = O.indexed_gate_up(x, codes, sc2, ids, 0, 3)
    np.testing.assert_array_equal(O.bf16_to_f64(out3), 0.5 * O.bf16_to_f64(out1))
    a = W.to_bf16_bits(np.random.default_rng(0).standard_normal((10, 64)).astype(np.float32))
    d1 = O.indexed_down_combine(a, codes, sc, ids, w, 0, 3)
    d2 = O.indexed_down_combine(a, codes, sc, ids, w * np.float32(8), 0, 3)
    np.testing.assert_array_equal(O.bf16_to_f64(d2), 8 * O.bf16_to_f64(d1))


def test_token_order_invariance():
    x, codes, sc, ids, w = _tiny_problem(9, T=7, k=2, E=3, N=8, K=64, integer_x=False)
    a = W.to_bf16_bits(np.random.default_rng(1).standard_normal((14, 64)).astype(np.float32))
    perm = np.random.default_rng(2).permutation(7)
    h, _ = O.indexed_gate_up(x, codes, sc, ids, 0, 3)
    hp, _ = O.indexed_gate_up(x[perm], codes, sc, ids[perm], 0, 3)
    np.testing.assert_array_equal(hp.reshape(7, 2, -1), h.reshape(7, 2, -1)[perm])
    d = O.indexed_down_combine(a, codes, sc, ids, w, 0, 3)
    ap = a.reshape(7, 2, -1)[perm].reshape(14, -1)
    dp = O.indexed_down_combine(ap, codes, sc, ids[perm], w[perm], 0, 3)
    np.testing.assert_array_equal(dp, d[perm])


def test_routed_equals_dense_per_token_sum():
    """The routed combine equals a dense per-token loop over its top-k experts
    (each expert's full dense product, then the weighted sum)."""
    _, codes, sc, ids, w = _tiny_problem(11, T=6, k=3, E=4, N=8, K=64)
    rng = np.random.default_rng(3)
    a = W.to_bf16_bits(rng.standard_normal((18, 64)).astype(np.float32))
    d = O.indexed_down_combine(a, codes, sc, ids, w, 0, 4)
    Wall = [O.dequant(codes[e], sc[e]) for e in range(4)]
    A = O.bf16_to_f64(a)
    for t in range(6):
        dense = np.zeros(8)
        for j in range(3):
            dense += float(w[t, j]) * (Wall[ids[t, j]] @ A[t * 3 + j])
        np.testing.assert_array_equal(d[t], O.f64_to_bf16(dense))


def test_duplicate_expert_and_no_local_token():
    E, N, K = 2, 8, 64
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, (4, N, K), dtype=np.uint8)
    sc = W.to_bf16_bits(rng.uniform(0.005, 0.02, (4, N, K // 32)).astype(np.float32))
    ids = np.array([[1, 1], [0, 3], [2, 3]], np.int32)      # first=0, E_loc=2: token 2 has no local slot
    w = np.array([[0.5, 0.25], [0.25, 0.75], [0.5, 0.5]], np.float32)
    a = W.to_bf16_bits(rng.standard_normal((6, K)).astype(np.float32))
    a[1] = a[0]
    d = O.indexed_down_combine(a, codes[:2], sc[:2], ids, w, 0, 2)
    W1 = O.dequant(codes[1], sc[1])
    W0 = O.dequant(codes[0], sc[0])
    A = O.bf16_to_f64(a)
    np.testing.assert_array_equal(d[0], O.f64_to_bf16(0.75 * (W1 @ A[0])))   # both duplicate slots count
    np.testing.assert_array_equal(d[1], O.f64_to_bf16(0.25 * (W0 @ A[2])))   # weight not renormalised
    assert not d[2].any()                                                      # no local slot -> 0


def test_gate_up_skips_nonlocal_slots():
    x, codes, sc, ids, _ = _tiny_problem(13, T=6, k=2, E=5, N=8, K=64)
    out, ok = O.indexed_gate_up(x, codes[1:3], sc[1:3], ids, 1, 2)
    flat = ids.reshape(-1)
    np.testing.assert_array_equal(ok, (flat >= 1) & (flat < 3))
    full, _ = O.indexed_gate_up(x, codes, sc, ids, 0, 5)
    np.testing.assert_array_equal(out[ok], full[ok])


def test_grouped_layouts_agree_with_indexed():
    sh = W.scaled(W.WORKLOADS["grouped_skewed"], T=96, K1=64, N1=48, E_glob=16, E_loc=6, first=2, max_m=24)
    ids, _ = W.routing_for(sh)
    x = W.activations(sh.seed, "x", sh.T, sh.K1)
    codes = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
    sc = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
    h, ok = O.indexed_gate_up(x, codes, sc, ids, sh.first, sh.E_loc)
    A, mi, slots = W.contiguous_layout(ids, x, sh.first, sh.E_loc, pad=128)
    assert A.shape[0] % 128 == 0
    out, valid = O.grouped_contiguous(A, codes, sc, mi)
    np.testing.assert_array_equal(valid, slots >= 0)
    np.testing.assert_array_equal(out[valid], h[slots[valid]])
    A3, mm, sl3, dropped = W.masked_layout(ids, x, sh.first, sh.E_loc, sh.max_m)
    outm, vm = O.grouped_masked(A3, codes, sc, mm)
    s = sl3.reshape(-1)
    np.testing.assert_array_equal(vm, s >= 0)
    np.testing.assert_array_equal(outm[vm], h[s[vm]])
    assert dropped == int(ok.sum()) - int(mm.sum())


def test_silu_mul_closed_forms():
    h = W.to_bf16_bits(np.array([[0.0, 30.0, 2.0, -3.0]], np.float32))   # gate [0, 30], up [2, -3]
    out = O.bf16_to_f64(O.silu_mul(h))
    assert out[0, 0] == 0.0
    assert out[0, 1] == -90.0                     # silu(30) rounds to 30 in bf16 range; 30 * -3


def test_silu_mul_matches_library_logistic():
    """silu(g) * u against SciPy's logistic function (a separate library
    routine): bf16(g * expit(g) * u) for bf16 inputs."""
    from scipy.special import expit
    rng = np.random.default_rng(7)
    g = W.to_bf16_bits(rng.normal(0, 4, 20000).astype(np.float32))
    u = W.to_bf16_bits(rng.normal(0, 1, 20000).astype(np.float32))
    h = np.stack([g, u], axis=1)
    got = O.silu_mul(h)[:, 0]
    gf, uf = O.bf16_to_f64(g), O.bf16_to_f64(u)
    ref = O.f64_to_bf16(gf * expit(gf) * uf)
    assert np.array_equal(got, ref)
    # odd-part identity: silu(x) - silu(-x) = x (checked in fp64 before rounding)
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(x * expit(x) - (-x) * expit(-x), x, rtol=0, atol=1e-12)


def test_gate_up_silu_sorted_places_rows():
    """Each valid sorted position gets the activation of its slot's row;
    padding positions are masked out; the ordering is that of moe_align."""
    T, k, E = 6, 2, 3
    ids = np.array([[0, 2], [1, 0], [2, 2], [0, 1], [1, 1], [2, 0]], np.int32)
    sid, eid, ntp = O.moe_align(ids, E, 0, E, 16)
    h = W.to_bf16_bits(np.arange(T * k * 4, dtype=np.float32).reshape(T * k, 4) / 7.0 - 3.0)
    out, valid = O.gate_up_silu_sorted(h, sid, T * k)
    assert valid.sum() == T * k and not valid[ntp:].any()
    act = O.silu_mul(h)
    for p in np.nonzero(valid)[0]:
        assert np.array_equal(out[p], act[sid[p]])


def test_fp32_baseline_within_tolerance_of_fp64():
    sh = W.scaled(W.WORKLOADS["tiny"])
    ids, w = W.routing_for(sh)
    x = W.activations(sh.seed, "x", sh.T, sh.K1)
    a = W.activations(sh.seed, "a", sh.T * sh.topk, sh.K2)
    c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
    s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
    c2 = W.weight_codes(sh.seed, "w2_codes", sh.E_loc, sh.N2, sh.K2)
    s2 = W.weight_scales(sh.seed, "w2_scales", sh.E_loc, sh.N2, sh.K2)
    ref, _ = O.indexed_gate_up(x, c1, s1, ids, 0, sh.E_loc)
    got = O.indexed_gate_up_fp32(x, c1, s1, ids, 0, sh.E_loc)
    assert (np.abs(O.bf16_to_f64(got) - O.bf16_to_f64(ref)) <= O.tolerance(ref)).all()
    ref = O.indexed_down_combine(a, c2, s2, ids, w, 0, sh.E_loc)
    got = O.indexed_down_combine_fp32(a, c2, s2, ids, w, 0, sh.E_loc)
    assert (np.abs(O.bf16_to_f64(got) - O.bf16_to_f64(ref)) <= O.tolerance(ref)).all()


def test_tolerance_formula():
    ref = W.to_bf16_bits(np.array([1.0, -3.0, 0.0, 1000.0], np.float32))
    tol = O.tolerance(ref, rel_rms=0.0)
    assert list(tol) == [2.0 ** -7, 2.0 ** -6, 0.0, 2.0 ** 2]


def test_workload_recipes():
    sh = W.WORKLOADS["ep8_decode"]
    ids, w = W.routing_for(sh)
    assert ids.shape == (576, 8) and ids.dtype == np.int32
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    assert all(len(set(r)) == 8 for r in ids)
    cnt = np.bincount(ids.reshape(-1), minlength=384)[:48]
    assert 6 <= cnt.mean() <= 18
    sh4 = W.WORKLOADS["grouped_skewed"]
    z = W.zero_expert_ids(sh4)
    assert len(z) == 4 and all(0 <= e < 48 for e in z)
    ids4, _ = W.route(sh4.seed, 256, 384, 8, 1.2, z)
    assert not np.isin(ids4, z).any()


def test_gemm_sum_is_not_rounded_to_fp32_first():
    """x has ones at kk = 0, 32, 64; row 0 of W dequantises to 1, 2^-8, 2^-30 in
    those groups.  Exact sum 1 + 2^-8 + 2^-30 rounds up to 1 + 2^-7 in bf16; a
    float32 partial sum would land on the tie 1 + 2^-8 and round down to 1."""
    K, N = 96, 2
    x = np.zeros((1, K), np.float32)
    x[0, [0, 32, 64]] = 1.0
    xb = W.to_bf16_bits(x)
    codes = np.full((1, N, K), 8, np.uint8)
    codes[0, :, [0, 32, 64]] = 9
    sc = W.to_bf16_bits(np.array([[[1.0, 2.0 ** -8, 2.0 ** -30]] * N], np.float32))
    out, _ = O.indexed_gate_up(xb, codes, sc, np.zeros((1, 1), np.int32), 0, 1)
    assert out[0, 0] == 0x3F81
    d = O.indexed_down_combine(xb, codes, sc, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), 0, 1)
    assert d[0, 0] == 0x3F81
