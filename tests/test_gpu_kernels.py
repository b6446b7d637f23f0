"""GPU parity of the HIP kernels against the CPU oracle on small and ragged
shapes: routing align (bit-exact), weight packing (bit-exact round trip),
the indexed GEMM with per-slot and combined outputs, the grouped layouts, and
the invariants (padding contributes nothing, token order, tile configuration
does not change bits, zero-row experts, empty inputs)."""
import itertools

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import workloads as W
from tests.gpu_util import Problem, assert_close, bits, dev, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

import w4a16_int4_mixture_moe_amd as M  # noqa: E402  (fails loudly if the binding is broken)


# ------------------------------------------------------------ routing align

def _align_case(topk, E_glob, first, E_loc, bm):
    T, k = topk.shape
    r = M.moe_align(to_dev(topk.astype(np.int32)), E_glob, first, E_loc, bm)
    si, ei, ntp = O.moe_align(topk, E_glob, first, E_loc, bm)
    got_si = r.sorted_ids.cpu().numpy()
    got_ei = r.expert_ids.cpu().numpy()[: len(ei)]
    got_ntp = int(r.num_tokens_padded.cpu().item())
    assert got_ntp == ntp, (T, k, E_glob, first, E_loc, bm)
    np.testing.assert_array_equal(got_si, si)
    np.testing.assert_array_equal(got_ei, ei)


def test_align_bit_exact_small_random():
    rng = np.random.default_rng(0)
    n = 0
    for T, k, E_glob in [(1, 1, 1), (3, 2, 5), (37, 3, 11), (64, 2, 8), (200, 8, 64), (513, 6, 7)]:
        for (first, E_loc), bm in itertools.product([(0, E_glob), (E_glob // 3, max(1, E_glob // 2))],
                                                    (16, 32, 64, 128, 256)):
            topk = rng.integers(0, E_glob, (T, k)).astype(np.int32)
            _align_case(topk, E_glob, first, E_loc, bm)
            n += 1
    log(f"{n} align cases bit-exact")


def test_align_out_of_range_ids_are_not_local_and_validate_rejects():
    topk = np.array([[0, 5], [-1, 2], [9, 1]], np.int32)
    _align_case(topk, 4, 0, 4, 16)
    with pytest.raises(M.W4A16Error, match="ERR_ROUTING"):
        M.moe_align(to_dev(topk), 4, 0, 4, 16, validate=True)


def test_align_edge_cases():
    _align_case(np.zeros((0, 4), np.int32), 8, 0, 8, 16)                       # no tokens
    _align_case(np.full((50, 2), 7, np.int32), 8, 0, 4, 32)                   # no local slot
    _align_case(np.full((300, 2), 3, np.int32), 8, 0, 8, 16)                  # all to one expert
    _align_case(np.random.default_rng(1).integers(0, 1024, (256, 8)).astype(np.int32), 1024, 0, 1024, 16)
    # both sides of the 16-wave / 8-wave switch at 512 local experts, with a
    # slot count that ends mid-batch in the last wave's range
    g = np.random.default_rng(2)
    for E_loc in (512, 513, 777):
        _align_case(g.integers(0, 1000, (4099, 5)).astype(np.int32), 1000, 1000 - E_loc, E_loc, 32)


def test_align_several_workgroups_bit_exact():
    """From 16,384 slots the align splits its scatter over several
    workgroups (each counts every slot): slot counts on both sides of that
    switch and ending mid-tile, one to 777 local experts (ballot matching
    above 512), out-of-range ids, skewed routing, every block_m."""
    g = np.random.default_rng(3)
    cases = [(2048, 8, 64, 0, 64, 16), (2048, 8, 64, 0, 64, 128),       # 16,384: one workgroup
             (2049, 8, 64, 8, 40, 32),                                  # 16,392: three
             (4099, 5, 1000, 223, 777, 64),                             # 20,495 slots, 777 experts
             (8191, 8, 384, 0, 48, 128), (12000, 8, 96, 5, 1, 16)]      # up to 96,000 slots, one expert
    for T, k, E_glob, first, E_loc, bm in cases:
        ids = g.integers(-1, E_glob + 1, (T, k)).astype(np.int32)       # -1 and E_glob are not local
        _align_case(ids, E_glob, first, E_loc, bm)
    # skewed: most slots on a few experts
    p = 1.0 / np.arange(1, 65) ** 1.5
    ids = g.choice(64, size=(9000, 4), p=p / p.sum()).astype(np.int32)
    for bm in (16, 64, 128):
        _align_case(ids, 64, 0, 64, bm)


@pytest.mark.parametrize("name", ["ep8_decode", "ep8_prefill", "tp8_t1", "tp8_t4096", "grouped_skewed"])
def test_align_bit_exact_workloads(name):
    sh = W.WORKLOADS[name]
    topk, _ = W.routing_for(sh)
    for bm in (16, 32, 128):
        _align_case(topk, sh.E_glob, sh.first, sh.E_loc, bm)


# ------------------------------------------------------------ packing

def _unpack_cpu(w_bytes: np.ndarray, s_bytes: np.ndarray, E, N, K):
    """Read the packed layout as documented in w4a16_moe.h back into codes
    [E, N, K] and scales [E, N, K/32]."""
    KP = -(-K // 128) * 128
    KC, NT = KP // 128, N // 16
    words = w_bytes.view(np.uint32).reshape(E, NT, KC, 64, 4)
    codes = np.zeros((E, N, KP), np.uint8)
    for l, j, e in itertools.product(range(64), range(4), range(8)):
        g, i = divmod(l, 16)
        shift = 4 * (e // 2) + 16 * (e % 2)
        vals = (words[:, :, :, l, j] >> shift) & 0xF                     # [E, NT, KC]
        kk = np.arange(KC) * 128 + 32 * g + 8 * j + e
        codes[:, np.arange(NT)[:, None] * 16 + i, kk[None, :]] = vals
    KC2 = -(-KC // 2)
    words = s_bytes.view(np.uint32).reshape(E, NT, KC2, 64)
    sc = np.stack([words & 0xFFFF, words >> 16], axis=3).reshape(E, NT, 2 * KC2, 64).astype(np.uint16)
    scales = np.zeros((E, N, 8 * KC2), np.uint16)
    for l in range(64):
        g, i = divmod(l, 16)
        scales[:, (np.arange(NT) * 16 + i)[:, None], (4 * np.arange(2 * KC2) + g)[None, :]] = sc[:, :, :, l]
    return codes, scales


@pytest.mark.parametrize("E,N,K", [(3, 48, 96), (2, 32, 256), (1, 16, 7168)])
def test_pack_round_trip_bit_exact(E, N, K):
    rng = np.random.default_rng(E * N + K)
    codes = rng.integers(0, 16, (E, N, K), dtype=np.uint8)
    scales = rng.integers(0, 65536, (E, N, K // 32), dtype=np.uint16)
    p = M.pack_w4(to_dev(codes), to_dev_bf16(scales))
    c2, s2 = _unpack_cpu(p.w.cpu().numpy(), p.s.cpu().numpy(), E, N, K)
    np.testing.assert_array_equal(c2[:, :, :K], codes)
    assert (c2[:, :, K:] == 8).all()                       # K padding decodes to weight 0
    np.testing.assert_array_equal(s2[:, :, : K // 32], scales)
    assert (s2[:, :, K // 32:] == 0).all()


# ------------------------------------------------------------ indexed GEMM

def _run_indexed(P, bm, nr=None, first=None, stages=2, waves=4):
    sh = P.sh
    first = sh.first if first is None else first
    r = M.moe_align(P.d_ids, sh.E_glob, first, sh.E_loc, bm)
    cfg = M.config(bm, nr if nr else (4 if bm >= 64 else 2), waves=waves, stages=stages)
    h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=cfg)
    y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=cfg) if P.with_down else None
    torch.cuda.synchronize()
    return r, h, y


def _check_indexed(P, h, y, what):
    sh = P.sh
    ref_h, ok = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc)
    gh = bits(h)
    e1, x1 = assert_close(gh[ok], ref_h[ok], what + " gate/up")
    assert not gh[~ok].any(), "non-local slot rows were written"
    res = {"gate_up_max_err": e1, "gate_up_exact": x1}
    if y is not None:
        ref_y = O.indexed_down_combine(P.a, P.c2, P.s2, P.topk_ids, P.topk_w, sh.first, sh.E_loc)
        e2, x2 = assert_close(bits(y), ref_y, what + " down+combine")
        res.update(down_max_err=e2, down_exact=x2)
    log(what, res)
    return res


def test_tiny_workload_all_tile_configs_match_oracle_and_each_other():
    """Every built tile configuration, including the pipeline depth (2 or 4
    chunks of weights in flight), gives the same output bits."""
    P = Problem(W.WORKLOADS["tiny"]).upload()
    outs = {}
    combos = [(bm, nr, 2, 4) for bm, nr in itertools.product((16, 32, 64, 128), (2, 4))]
    combos += [(16, 2, 4, 4), (32, 2, 4, 4), (16, 2, 2, 8), (32, 2, 2, 8), (128, 2, 2, 8)]
    for bm, nr, st, nw in combos:
        _, h, y = _run_indexed(P, bm, nr, stages=st, waves=nw)
        _check_indexed(P, h, y, f"tiny bm={bm} nr={nr} stages={st} waves={nw}")
        outs[(bm, nr, st, nw)] = (bits(h), bits(y))
    base = outs[(16, 2, 2, 4)]
    for key, (h, y) in outs.items():          # tile configuration does not change bits
        np.testing.assert_array_equal(h, base[0], err_msg=str(key))
        np.testing.assert_array_equal(y, base[1], err_msg=str(key))


def test_ragged_shapes():
    """N not a multiple of the workgroup tile, K not a multiple of 128, odd T."""
    sh = W.MoEShape(name="ragged", E_glob=9, E_loc=5, first=2, topk=3, T=37, K1=96, N1=48,
                    K2=160, N2=80, seed=77)
    P = Problem(sh).upload()
    for bm in (16, 32, 128):
        _, h, y = _run_indexed(P, bm)
        _check_indexed(P, h, y, f"ragged bm={bm}")
    _, h, y = _run_indexed(P, 32, stages=4)
    _check_indexed(P, h, y, "ragged bm=32 stages=4")
    for bm in (16, 32, 128):
        _, h, y = _run_indexed(P, bm, 2, waves=8)
        _check_indexed(P, h, y, f"ragged bm={bm} waves=8")


def test_sparse_routing_launches_only_possible_tiles():
    """The launch grid covers the tiles that can hold routed rows (T * topk
    slots plus one rounding per expert with rows), not the over-allocated
    capacity: a few tokens over many experts (every slot its own expert, the
    most padding per row) at every block size, tiles dividing a 256-row
    routing, K slices and stream-K, against the oracle."""
    for T in (1, 3, 48):
        sh = W.MoEShape(name=f"sparse_t{T}", E_glob=384, E_loc=384, first=0, topk=8, T=T, K1=512, N1=64,
                        K2=512, N2=96, seed=600 + T)
        P = Problem(sh).upload()
        for bm in (16, 32, 64, 128):
            _, h, y = _run_indexed(P, bm)
            _check_indexed(P, h, y, f"sparse T={T} bm={bm}")
        r256 = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 256)
        _, h, y = _run_indexed(P, 16, nr=1, waves=8)
        _check_indexed(P, h, y, f"sparse T={T} bm=16 nr=1 (waves splitting K)")
        for c in (M.config(256, 2, 8), M.config(128, 4), M.config(64, 2), M.config(16, 2, split_k=2),
                  M.config(16, 2, split_k=0), M.config(16, 1, 8)):
            h = M.moe_w4a16_gemm(P.d_x, P.p1, r256, cfg=c)
            y = M.moe_w4a16_gemm(P.d_a, P.p2, r256, topk_weights=P.d_w, cfg=c)
            torch.cuda.synchronize()
            _check_indexed(P, h, y, f"sparse T={T} 256-row routing bm={c.block_m} split_k={c.split_k}")


def test_decode_xcd_groups_cover_every_tile():
    """Decode tiles of a block with 32 or more N tiles run in groups of 16 N
    tiles per XCD (the grid rounded up to whole rounds of eight groups;
    workgroups past the last block exit).  Gate/up N = 4096 on block_m 32,
    nr 2 (32 N tiles per block: grouped) gives the same bits as nr 4 (16 N
    tiles: block-major), whose outputs are summed in the same order, and
    matches the oracle; with a grid that needs idle groups and one that
    does not."""
    for T, seed in ((40, 31), (57, 32)):
        sh = W.MoEShape(name=f"xcd_t{T}", E_glob=8, E_loc=5, first=1, topk=2, T=T, K1=256, N1=4096,
                        K2=256, N2=64, seed=seed)
        P = Problem(sh, with_down=False).upload()
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 32)
        hg = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=M.config(32, 2))
        hb = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=M.config(32, 4))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(hg), bits(hb), err_msg=f"T={T}: grouped vs block-major")
        _check_indexed(P, hg, None, f"xcd groups T={T}")


def test_multi_chunk_k():
    """K spanning many 128-wide chunks (steady-state loop plus its tail, both
    prefetch depths), ragged and not, against the oracle; depths agree bit
    for bit."""
    for K1, K2 in ((1312, 1024), (2304, 1184)):
        sh = W.MoEShape(name=f"k{K1}", E_glob=8, E_loc=6, first=1, topk=2, T=40, K1=K1, N1=96,
                        K2=K2, N2=80, seed=91)
        P = Problem(sh).upload()
        outs = []
        for bm, st, nw in ((16, 2, 4), (32, 4, 4), (64, 2, 4), (16, 2, 8), (32, 2, 8), (128, 2, 8)):
            _, h, y = _run_indexed(P, bm, 2, stages=st, waves=nw)
            _check_indexed(P, h, y, f"K1={K1} K2={K2} bm={bm} stages={st} waves={nw}")
            outs.append((bits(h), bits(y)))
        for h, y in outs[1:]:
            np.testing.assert_array_equal(h, outs[0][0])
            np.testing.assert_array_equal(y, outs[0][1])


def test_one_hot_activations_return_dequantised_weights_bit_exact():
    E, N, K = 3, 64, 256
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (E, N, K), dtype=np.uint8)
    sc = W.to_bf16_bits(rng.uniform(0.005, 0.02, (E, N, K // 32)).astype(np.float32))
    x = W.to_bf16_bits(np.eye(K, dtype=np.float32))
    ids = (np.arange(K) % E).astype(np.int32)[:, None]
    p = M.pack_w4(to_dev(codes), to_dev_bf16(sc))
    r = M.moe_align(to_dev(ids), E, 0, E, 16)
    h = bits(M.moe_w4a16_gemm(to_dev_bf16(x), p, r))
    Wd = O.f64_to_bf16(O.dequant(codes, sc))                          # [E, N, K]
    want = np.stack([Wd[t % E, :, t] for t in range(K)])
    np.testing.assert_array_equal(h, want)


def test_zero_codes_give_zero_and_power_of_two_scaling_is_exact():
    P = Problem(W.WORKLOADS["tiny"])
    P.c1 = np.full_like(P.c1, 8)
    P.upload()
    _, h, _ = _run_indexed(P, 16)
    assert not bits(h).any()
    P = Problem(W.WORKLOADS["tiny"]).upload()
    _, h1, y1 = _run_indexed(P, 32)
    P.d_x = P.d_x * 4
    P.d_w = P.d_w * 2
    _, h2, y2 = _run_indexed(P, 32)
    np.testing.assert_array_equal(O.bf16_to_f64(bits(h2)), 4 * O.bf16_to_f64(bits(h1)))
    np.testing.assert_array_equal(O.bf16_to_f64(bits(y2)), 2 * O.bf16_to_f64(bits(y1)))


def test_padding_contributes_nothing():
    """Garbage past num_tokens_padded, canaries in non-local rows, NaN in
    activation rows that no slot references: outputs unchanged."""
    sh = W.scaled(W.WORKLOADS["tiny"], E_glob=16, E_loc=8, first=4)
    P = Problem(sh).upload()
    r, h, y = _run_indexed(P, 32)
    ntp = int(r.num_tokens_padded.item())
    r.sorted_ids[ntp:] = 3                     # valid-looking slot ids past the end
    r.expert_ids[ntp // 32:] = 1
    canary = torch.full_like(h, -7.0)
    h2 = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=M.config(32, 2), out=canary.clone())
    y2 = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=M.config(32, 2))
    torch.cuda.synchronize()
    ok = np.isin(P.topk_ids.reshape(-1), np.arange(4, 12))
    hb, h2b = bits(h), bits(h2)
    np.testing.assert_array_equal(h2b[ok], hb[ok])
    assert (O.bf16_to_f64(h2b[~ok]) == -7.0).all()
    np.testing.assert_array_equal(bits(y2), bits(y))
    # NaN in every down-input row of a non-local slot: never read
    a = P.a.copy()
    a[~ok] = 0x7FC0
    P.d_a = to_dev_bf16(a)
    _, _, y3 = _run_indexed(P, 32)
    np.testing.assert_array_equal(bits(y3), bits(y))


def test_token_order_invariance_bit_exact():
    P = Problem(W.WORKLOADS["tiny"]).upload()
    _, h, y = _run_indexed(P, 16)
    perm = np.random.default_rng(3).permutation(P.T)
    Q = Problem(W.WORKLOADS["tiny"])
    Q.topk_ids, Q.topk_w, Q.x = P.topk_ids[perm], P.topk_w[perm], P.x[perm]
    Q.a = P.a.reshape(P.T, -1, P.a.shape[1])[perm].reshape(P.a.shape)
    Q.upload()
    _, hq, yq = _run_indexed(Q, 16)
    k = P.sh.topk
    np.testing.assert_array_equal(bits(hq).reshape(P.T, k, -1), bits(h).reshape(P.T, k, -1)[perm])
    np.testing.assert_array_equal(bits(yq), bits(y)[perm])


def test_zero_row_experts_and_no_local_tokens():
    sh = W.scaled(W.WORKLOADS["tiny"], T=40)
    P = Problem(sh)
    P.topk_ids = np.where(P.topk_ids % 2 == 0, 1, 5).astype(np.int32)     # only experts 1, 5 used
    P.upload()
    _, h, y = _run_indexed(P, 16)
    _check_indexed(P, h, y, "two experts only")
    # EP share that receives nothing: ntp = 0, combine output all zero
    Q = Problem(sh)
    Q.topk_ids = np.full_like(Q.topk_ids, 7)
    Q.upload()
    r = M.moe_align(Q.d_ids, 8, 0, 7, 16)
    sh7 = r
    assert int(sh7.num_tokens_padded.item()) == 0
    p7 = M.pack_w4(to_dev(Q.c2[:7]), to_dev_bf16(Q.s2[:7]))
    y = M.moe_w4a16_gemm(Q.d_a, p7, r, topk_weights=Q.d_w, cfg=M.config(16, 2))
    torch.cuda.synchronize()
    assert not bits(y).any()


def test_duplicate_expert_in_one_token():
    sh = W.scaled(W.WORKLOADS["tiny"], T=24)
    P = Problem(sh)
    P.topk_ids[:, 1] = P.topk_ids[:, 0]
    P.upload()
    _, h, y = _run_indexed(P, 32)
    _check_indexed(P, h, y, "duplicate experts")


def test_empty_token_batch():
    sh = W.scaled(W.WORKLOADS["tiny"], T=0)
    p = M.pack_w4(torch.zeros((8, 512, 256), dtype=torch.uint8, device=dev()),
                  torch.zeros((8, 512, 8), dtype=torch.bfloat16, device=dev()))
    ids = torch.zeros((0, 2), dtype=torch.int32, device=dev())
    r = M.moe_align(ids, 8, 0, 8, 16)
    h = M.moe_w4a16_gemm(torch.zeros((0, 256), dtype=torch.bfloat16, device=dev()), p, r)
    torch.cuda.synchronize()
    assert h.shape == (0, 512)


def test_dense_special_case_matches_library_matmul():
    """E = 1, top-1, weight 1: the routed GEMM is a dense x . W^T; compare with
    torch.matmul (hipBLASLt) on the dequantised weight, at K = 7168, N = 4096."""
    T, N, K = 256, 4096, 7168
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (1, N, K), dtype=np.uint8)
    sc = W.to_bf16_bits(rng.uniform(0.005, 0.02, (1, N, K // 32)).astype(np.float32))
    x = W.activations(9, "x", T, K)
    dc, ds = to_dev(codes), to_dev_bf16(sc)
    p = M.pack_w4(dc, ds)
    r = M.moe_align(torch.zeros((T, 1), dtype=torch.int32, device=dev()), 1, 0, 1, 128)
    dx = to_dev_bf16(x)
    h = M.moe_w4a16_gemm(dx, p, r, cfg=M.config(128, 4))
    Wd = ((dc[0].float() - 8.0) * ds[0].float().repeat_interleave(32, dim=1)).to(torch.bfloat16)
    ref = torch.matmul(dx.float(), Wd.float().t().contiguous()).to(torch.bfloat16)
    torch.cuda.synchronize()
    e, x_exact = assert_close(bits(h), bits(ref), "dense vs torch.matmul")
    log("dense special case: max err", e, "bit-exact fraction", x_exact)


# ------------------------------------------------------------ grouped layouts

def test_grouped_contiguous_and_masked_small():
    sh = W.scaled(W.WORKLOADS["grouped_skewed"], T=300, K1=512, N1=96, E_glob=24, E_loc=6,
                  first=3, max_m=48, n_zero_experts=1)
    P = Problem(sh, with_down=False).upload()
    A, mi, slots = W.contiguous_layout(P.topk_ids, P.x, sh.first, sh.E_loc, pad=128, pad_fill=0x7FC0)
    ref, valid = O.grouped_contiguous(A, P.c1, P.s1, mi)
    for bm, nr, nw in ((16, 2, 4), (64, 4, 4), (128, 4, 4), (128, 2, 8), (32, 2, 8)):
        out = bits(M.grouped_contiguous(to_dev_bf16(A), P.p1, to_dev(mi),
                                        cfg=M.config(bm, nr, waves=nw, kind="contiguous")))
        assert_close(out[valid], ref[valid], f"contiguous bm={bm} nr={nr} waves={nw}")
    A3, mm, sl3, dropped = W.masked_layout(P.topk_ids, P.x, sh.first, sh.E_loc, sh.max_m, pad_fill=0x7FC0)
    log("masked dropped", dropped, "masked_m", mm.tolist())
    ref, valid = O.grouped_masked(A3, P.c1, P.s1, mm)
    for bm, nw in ((16, 4), (32, 4), (64, 4), (16, 8), (32, 8)):
        out = bits(M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), 32, cfg=M.config(bm, 2, waves=nw, kind="masked")))
        assert_close(out[valid], ref[valid], f"masked bm={bm} waves={nw}")
    out = bits(M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), expected_m=max(1, int(mm.mean()))))
    assert_close(out[valid], ref[valid], "masked auto config")
    # split K on the grouped layouts (K = 512: two slices of one chunk pair)
    out = bits(M.grouped_contiguous(to_dev_bf16(A), P.p1, to_dev(mi), cfg=M.config(32, 2, split_k=2, kind="contiguous")))
    ref_c, valid_c = O.grouped_contiguous(A, P.c1, P.s1, mi)
    assert_close(out[valid_c], ref_c[valid_c], "contiguous split_k=2")
    out = bits(M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), 32, cfg=M.config(16, 2, split_k=2, kind="masked")))
    assert_close(out[valid], ref[valid], "masked split_k=2")
    # grouped and indexed agree on the same rows
    h, ok = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc)
    s = sl3.reshape(-1)
    np.testing.assert_array_equal(ref[valid], h[s[valid]])


def test_hip_graph_capture_replays_match_eager():
    """align + gate/up + down+combine captured in one HIP graph: no host
    readback or allocation in the path, so replays reproduce the eager
    outputs bit for bit, also with other eager work between replays."""
    P = Problem(W.WORKLOADS["tiny"]).upload()
    sh = P.sh
    bm = 32
    cap = M.align_capacity(sh.T, sh.topk, sh.E_loc, bm)
    r = M.Routing(torch.empty(cap, dtype=torch.int32, device=dev()),
                  torch.empty(cap // bm, dtype=torch.int32, device=dev()),
                  torch.empty(1, dtype=torch.int32, device=dev()), bm, P.d_ids, sh.E_glob,
                  sh.first, sh.E_loc)
    h = torch.zeros(sh.T * sh.topk, sh.N1, dtype=torch.bfloat16, device=dev())
    y = torch.empty(sh.T, sh.N2, dtype=torch.bfloat16, device=dev())
    cfg = M.config(bm, 2, split_k=0)
    ws = torch.empty(M.workspace_bytes(P.p2, r, True, cfg), dtype=torch.uint8, device=dev())
    ws1 = torch.empty(max(16, M.workspace_bytes(P.p1, r, False, cfg)), dtype=torch.uint8, device=dev())

    def step():
        rr = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm, capacity=cap)
        r.sorted_ids.copy_(rr.sorted_ids)        # (eager reference path only)
        return rr

    ref_r = step()
    ref_h = bits(M.moe_w4a16_gemm(P.d_x, P.p1, ref_r, cfg=cfg))
    ref_y = bits(M.moe_w4a16_gemm(P.d_a, P.p2, ref_r, topk_weights=P.d_w, cfg=cfg))

    import ctypes
    L = M.load()

    def captured_step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        M._lib.check(L.w4a16_moe_align(P.d_ids.data_ptr(), sh.T, sh.topk, sh.E_glob, sh.first,
                                       sh.E_loc, bm, r.sorted_ids.data_ptr(), r.expert_ids.data_ptr(),
                                       r.num_tokens_padded.data_ptr(), cap, 0, s))
        M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=cfg, out=h, workspace=ws1)
        M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=cfg, out=y, workspace=ws)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured_step()
    for rep in range(4):
        r.sorted_ids.fill_(-5)
        h.fill_(0)
        y.fill_(1.0)
        ws.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(h), ref_h, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(bits(y), ref_y, err_msg=f"replay {rep}")
        _ = (P.d_x.float() @ P.d_x.float().t()).sum().item()   # unrelated eager work


@pytest.mark.parametrize("name,T", [("tiny", 64), ("ragged", 37), ("tiny", 300)])
def test_streamk_matches_oracle_and_is_deterministic(name, T):
    """Stream-K (split_k = 0) cuts tiles between persistent workgroups and
    finishes them from fp32 partials: results within tolerance of the oracle,
    identical across repeated calls, and within tolerance of the one-
    workgroup-per-tile schedule."""
    if name == "ragged":
        sh = W.MoEShape(name="ragged", E_glob=9, E_loc=5, first=2, topk=3, T=T, K1=96, N1=48,
                        K2=160, N2=80, seed=77)
    else:
        sh = W.scaled(W.WORKLOADS["tiny"], T=T)
    P = Problem(sh).upload()
    for bm in (16, 32, 128):
        nr = 4 if bm >= 64 else 2
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        outs = []
        for rep in range(2):
            cfg = M.config(bm, nr, split_k=0)
            h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=cfg)
            y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=cfg)
            torch.cuda.synchronize()
            outs.append((bits(h), bits(y)))
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
        _check_indexed(P, torch.from_numpy(outs[0][0].view(np.int16)).view(torch.bfloat16),
                       torch.from_numpy(outs[0][1].view(np.int16)).view(torch.bfloat16),
                       f"stream-K {name} T={T} bm={bm}")


# ------------------------------------------------------------ split K

def _split_shapes():
    # K slices are whole pairs of 128-K chunks: K of at least two pairs, and
    # ragged ones (a last chunk of 96 and of 32 columns)
    return [W.scaled(W.WORKLOADS["tiny"], K1=1024, K2=512),
            W.MoEShape(name="ragged", E_glob=9, E_loc=5, first=2, topk=3, T=37, K1=608, N1=48,
                       K2=672, N2=80, seed=77),
            W.MoEShape(name="k1312", E_glob=8, E_loc=6, first=1, topk=2, T=40, K1=1312, N1=96,
                       K2=1024, N2=80, seed=91)]


@pytest.mark.parametrize("shape", _split_shapes(), ids=lambda s: s.name)
def test_split_k_matches_oracle_is_deterministic_and_leaves_counters_zero(shape):
    """split_k = S: S workgroups per tile over equal shares of the pairs of
    K chunks, the last to finish summing the fp32 slices in slice order.
    Within tolerance of the oracle for every S the shape allows (at most one
    slice per chunk pair), bit-identical across repeated calls on one
    workspace (whichever workgroup finishes last), and the arrival counters
    are back at zero after every call."""
    P = Problem(shape).upload()
    sh = P.sh
    pairs = lambda K: -(-K // 256)
    for bm in (16, 32, 128):
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        for S in (2, 4, 8):
            if S > pairs(sh.K1) and S > pairs(sh.K2):
                continue
            outs = []
            c1 = M.config(bm, 2, split_k=S if S <= pairs(sh.K1) else 1)
            c2 = M.config(bm, 2, split_k=S if S <= pairs(sh.K2) else 1)
            ws1 = torch.zeros(max(16, M.workspace_bytes(P.p1, r, False, c1)), dtype=torch.uint8, device=dev())
            ws2 = torch.zeros(max(16, M.workspace_bytes(P.p2, r, True, c2)), dtype=torch.uint8, device=dev())
            for rep in range(3):
                h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c1, workspace=ws1)
                y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=c2, workspace=ws2)
                torch.cuda.synchronize()
                outs.append((bits(h), bits(y)))
            for k_ in (1, 2):
                np.testing.assert_array_equal(outs[0][0], outs[k_][0])
                np.testing.assert_array_equal(outs[0][1], outs[k_][1])
            for ws, c in ((ws1, c1), (ws2, c2)):
                if c.split_k > 1:   # counters: the first region, 4 bytes per splittable tile
                    assert not bool(ws[:256].any()), "split-K arrival counters not reset"
            _check_indexed(P, torch.from_numpy(outs[0][0].view(np.int16)).view(torch.bfloat16),
                           torch.from_numpy(outs[0][1].view(np.int16)).view(torch.bfloat16),
                           f"split {sh.name} bm={bm} S={S} (gate/up {c1.split_k}, down {c2.split_k})")


def test_split_k_past_the_tile_cap_runs_whole_tiles():
    """More tiles than the split slices are kept for (2048): tiles past the
    cap run whole in their first workgroup, the rest split; all within
    tolerance of the oracle."""
    sh = W.MoEShape(name="many_tiles", E_glob=96, E_loc=96, first=0, topk=4, T=900, K1=512, N1=2048,
                    K2=256, N2=64, seed=5)
    P = Problem(sh).upload()
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 16)
    n_tiles = 2048 // 16 // 8
    ntp = int(r.num_tokens_padded.item())
    assert ntp // 16 * n_tiles > 2048, "shape must exceed the split tile cap"
    c = M.config(16, 2, split_k=2)
    h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c)
    torch.cuda.synchronize()
    ref_h, ok = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc)
    assert_close(bits(h)[ok], ref_h[ok], "split past the tile cap")


def test_split_k_graph_replays_match_eager():
    """A split-K call captured in a HIP graph: every replay reproduces the
    eager bits (the counters it leaves at zero let the next replay split
    again), with eager work and poisoned outputs between replays."""
    P = Problem(W.scaled(W.WORKLOADS["tiny"], K1=2048, K2=1024)).upload()
    sh = P.sh
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 16)
    c1, c2 = M.config(16, 2, split_k=8), M.config(16, 2, split_k=4)
    ws1 = torch.zeros(M.workspace_bytes(P.p1, r, False, c1), dtype=torch.uint8, device=dev())
    ws2 = torch.zeros(M.workspace_bytes(P.p2, r, True, c2), dtype=torch.uint8, device=dev())
    h = torch.zeros(sh.T * sh.topk, sh.N1, dtype=torch.bfloat16, device=dev())
    y = torch.empty(sh.T, sh.N2, dtype=torch.bfloat16, device=dev())
    M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c1, out=h, workspace=ws1)
    M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=c2, out=y, workspace=ws2)
    torch.cuda.synchronize()
    ref_h, ref_y = bits(h).copy(), bits(y).copy()
    _check_indexed(P, h, y, "split graph eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c1, out=h, workspace=ws1)
        M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=c2, out=y, workspace=ws2)
    for rep in range(4):
        h.fill_(0)
        y.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(h), ref_h, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(bits(y), ref_y, err_msg=f"replay {rep}")
        _ = (P.d_x.float() @ P.d_x.float().t()).sum().item()   # unrelated eager work


# ------------------------------------------------------------ prefill tile

# (K of the gate/up, K of the down): chunk counts of 128 that leave 0, 1, 2
# and 3 chunks past the prefill tile's four-chunk steps, and counts below four
PREFILL_K = [(1152, 1024), (1280, 896), (384, 256), (512, 128)]


@pytest.mark.parametrize("K1,K2", PREFILL_K)
def test_prefill_tile_bit_identical_to_the_general_kernel(K1, K2):
    """The prefill tile (block_m 128, nr 4: LDS-DMA staging, K a multiple of
    128) sums every output in the same order as the general kernel's 128-row
    tiles, so their bits agree, for every chunk count modulo four (the tile's
    main loop takes four chunks a step), every active-tile count (skewed
    routing), a ragged last N tile, and every epilogue and row source; both
    within tolerance of the oracle.  So does the 256-row tile (nr 2, eight
    waves) on a 256-row routing, and so do 128- and 64-row tiles over that
    routing."""
    sh = W.MoEShape(name="prefill_tile", E_glob=12, E_loc=6, first=3, topk=4, T=400, K1=K1, N1=512,
                    K2=K2, N2=272, zipf_s=1.0, seed=4242)
    P = Problem(sh).upload()
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 128)
    flat = P.topk_ids.reshape(-1)
    counts = np.bincount(flat[(flat >= sh.first) & (flat < sh.first + sh.E_loc)] - sh.first, minlength=sh.E_loc)
    log(f"K1={K1} K2={K2} rows per local expert", counts.tolist())
    tiles = {"prefill": (4, 4), "general": (2, 4)}     # (nr, waves)
    out = {}
    for name, (nr, waves) in tiles.items():
        c = M.config(128, nr, waves)
        h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c)
        y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=c)
        torch.cuda.synchronize()
        out[name] = (bits(h), bits(y))
        if name == "prefill":
            _check_indexed(P, h, y, f"prefill tile check K1={K1} K2={K2}")
    # the 256-row tile (block_m 256, nr 2, eight waves) on its own routing
    r256 = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 256)
    wide = M.config(256, 2, 8)
    out["wide"] = (bits(M.moe_w4a16_gemm(P.d_x, P.p1, r256, cfg=wide)),
                   bits(M.moe_w4a16_gemm(P.d_a, P.p2, r256, topk_weights=P.d_w, cfg=wide)))
    for name in ("prefill", "wide"):
        np.testing.assert_array_equal(out[name][0], out["general"][0], err_msg=f"gate/up: {name} vs general kernel")
        np.testing.assert_array_equal(out[name][1], out["general"][1], err_msg=f"down+combine: {name} vs general kernel")
    # tiles of 128 and 64 rows over the 256-row routing (a tile looks its
    # expert up from the routed block it falls in; a tile of padding only
    # exits), as the down + combine runs after a 256-row gate/up
    for c in (M.config(128, 4), M.config(128, 2), M.config(64, 2)):
        tag = f"bm{c.block_m} nr{c.nr}"
        y = bits(M.moe_w4a16_gemm(P.d_a, P.p2, r256, topk_weights=P.d_w, cfg=c))
        np.testing.assert_array_equal(y, out["general"][1], err_msg=f"down+combine on the 256-row routing, {tag}")
        h = bits(M.moe_w4a16_gemm(P.d_x, P.p1, r256, cfg=c))
        np.testing.assert_array_equal(h, out["general"][0], err_msg=f"gate/up on the 256-row routing, {tag}")
    # the calls' own choice (cfg None: the 256-row tile, unsplit, for both
    # projections), bit-identical; K slices and stream-K over the 256-row
    # routing: within the oracle's tolerance
    h = M.moe_w4a16_gemm(P.d_x, P.p1, r256)
    y = M.moe_w4a16_gemm(P.d_a, P.p2, r256, topk_weights=P.d_w)
    np.testing.assert_array_equal(bits(h), out["general"][0], err_msg="gate/up on the 256-row routing, cfg None")
    np.testing.assert_array_equal(bits(y), out["general"][1], err_msg="down+combine on the 256-row routing, cfg None")
    _check_indexed(P, h, y, f"256-row routing, cfg None, K1={K1} K2={K2}")
    for c in ((M.config(64, 2, split_k=2),) if K2 >= 512 else ()) + (M.config(128, 2, split_k=0),):
        _check_indexed(P, M.moe_w4a16_gemm(P.d_x, P.p1, r256, cfg=c),
                       M.moe_w4a16_gemm(P.d_a, P.p2, r256, topk_weights=P.d_w, cfg=c),
                       f"256-row routing bm{c.block_m} split_k={c.split_k} K1={K1} K2={K2}")
    # fused SiLU epilogue on the interleaved gate/up weight
    p1g = M.pack_w4(to_dev(P.c1), to_dev_bf16(P.s1), gate_up=True)
    inter = {name: bits(M.moe_gate_up_silu(P.d_x, p1g, r, cfg=M.config(128, nr, waves)))
             for name, (nr, waves) in tiles.items()}
    valid = r.sorted_ids.cpu().numpy() < sh.T * sh.topk
    for name in ("prefill",):
        np.testing.assert_array_equal(inter[name][valid], inter["general"][valid], err_msg=f"fused SiLU: {name}")
    # fused SiLU on the 256-row routing (the 256-row tile, and 128-row tiles):
    # rows in that routing's sorted order, compared per slot
    s128, s256 = r.sorted_ids.cpu().numpy(), r256.sorted_ids.cpu().numpy()
    v256 = s256 < sh.T * sh.topk
    for c in (wide, M.config(128, 4), None):
        iw = bits(M.moe_gate_up_silu(P.d_x, p1g, r256, cfg=c))
        by_slot = np.zeros((sh.T * sh.topk, iw.shape[1]), iw.dtype)
        by_slot[s256[v256]] = iw[v256]
        np.testing.assert_array_equal(by_slot[s128[valid]], inter["general"][valid],
                                      err_msg=f"fused SiLU on the 256-row routing, {c}")
    # grouped row sources
    A, mi, _ = W.contiguous_layout(P.topk_ids, P.x, sh.first, sh.E_loc, pad=128, pad_fill=0x7FC0)
    oc = {name: bits(M.grouped_contiguous(to_dev_bf16(A), P.p1, to_dev(mi),
                                          cfg=M.config(128, nr, waves, kind="contiguous")))
          for name, (nr, waves) in tiles.items()}
    ok = mi >= 0
    ref, vr = O.grouped_contiguous(A, P.c1, P.s1, mi)
    A3, mm, _, _ = W.masked_layout(P.topk_ids, P.x, sh.first, sh.E_loc, 200, pad_fill=0x7FC0)
    om = {name: bits(M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), 100,
                                      cfg=M.config(128, nr, waves, kind="masked")))
          for name, (nr, waves) in tiles.items()}
    refm, vm = O.grouped_masked(A3, P.c1, P.s1, mm)
    om["wide"] = bits(M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), 100, cfg=M.config(256, 2, 8, kind="masked")))
    for name in ("prefill",):
        np.testing.assert_array_equal(oc[name][ok], oc["general"][ok], err_msg=f"contiguous: {name}")
    for name in ("prefill", "wide"):
        np.testing.assert_array_equal(om[name][vm], om["general"][vm], err_msg=f"masked: {name}")
    assert_close(oc["prefill"][vr], ref[vr], "contiguous prefill tile")
    assert_close(om["prefill"][vm], refm[vm], "masked prefill tile")


def test_combine_passes_bit_identical():
    """The down projection + combine over column passes (combine_cols) gives
    the same bits as one pass over all N: each pass runs the GEMM over its
    column range of the weights and combines those columns.  Pass widths
    that cut a workgroup tile, leave a ragged last pass, or take one 16-column
    tile; on the general kernel, the prefill tile, K slices and stream-K."""
    sh = W.MoEShape(name="combine_passes", E_glob=12, E_loc=6, first=3, topk=4, T=300, K1=256, N1=64,
                    K2=1024, N2=272, zipf_s=1.0, seed=515)
    P = Problem(sh).upload()
    ref = O.indexed_down_combine(P.a, P.c2, P.s2, P.topk_ids, P.topk_w, sh.first, sh.E_loc)
    for bm, nr, split in ((32, 2, 1), (128, 4, 1), (32, 2, 2), (64, 2, 0)):
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        one = bits(M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=M.config(bm, nr, split_k=split)))
        assert_close(one, ref, f"down+combine bm={bm} nr={nr} split={split}")
        for cols in (16, 64, 112, 256, 272):
            got = bits(M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w,
                                        cfg=M.config(bm, nr, split_k=split, combine_cols=cols)))
            np.testing.assert_array_equal(got, one, err_msg=f"bm={bm} nr={nr} split={split} combine_cols={cols}")
        log(f"bm={bm} nr={nr} split={split}: passes of 16..272 columns bit-identical to one pass")


def test_prefill_tile_n_tile_loop_bit_identical():
    """K of at most 256 on the prefill tile: when the grid is large enough a
    workgroup keeps its block's activation rows in LDS and runs several N
    tiles (here 445 routed-block slots x 7 N tiles: two tiles per workgroup,
    the last group one tile).  Bits equal the general kernel's for the per-slot
    store, the weighted combine, the fused SiLU epilogue and the contiguous
    layout; sampled outputs within tolerance of the oracle."""
    sh = W.MoEShape(name="pf_loop", E_glob=384, E_loc=384, first=0, topk=8, T=1024, K1=256, N1=1792,
                    K2=256, N2=1792, seed=4343)
    P = Problem(sh).upload()
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 128)
    assert r.capacity // 128 == 445
    out = {}
    for name, nr in (("prefill", 4), ("general", 2)):
        c = M.config(128, nr)
        h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=c)
        y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=c)
        torch.cuda.synchronize()
        out[name] = (bits(h), bits(y))
    np.testing.assert_array_equal(out["prefill"][0], out["general"][0], err_msg="gate/up: N-tile loop")
    np.testing.assert_array_equal(out["prefill"][1], out["general"][1], err_msg="down+combine: N-tile loop")
    rng = np.random.default_rng(7)
    flat = P.topk_ids.reshape(-1)
    slots = rng.choice(len(flat), 64, replace=False)
    cols = np.unique(np.concatenate([rng.choice(sh.N1, 64, replace=False), [0, sh.N1 - 1]]))
    ref, _ = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc, slots=slots, cols=cols)
    assert_close(out["prefill"][0][slots][:, cols], ref, "N-tile loop gate/up")
    toks = rng.choice(sh.T, 48, replace=False)
    ref2 = O.indexed_down_combine(P.a, P.c2, P.s2, P.topk_ids, P.topk_w, sh.first, sh.E_loc, tokens=toks, cols=cols)
    assert_close(out["prefill"][1][toks][:, cols], ref2, "N-tile loop down+combine")
    p1g = M.pack_w4(to_dev(P.c1), to_dev_bf16(P.s1), gate_up=True)
    inter = {nr: bits(M.moe_gate_up_silu(P.d_x, p1g, r, cfg=M.config(128, nr))) for nr in (4, 2)}
    valid = r.sorted_ids.cpu().numpy() < sh.T * sh.topk
    np.testing.assert_array_equal(inter[4][valid], inter[2][valid], err_msg="fused SiLU: N-tile loop")
    A, mi, _ = W.contiguous_layout(P.topk_ids, P.x, sh.first, sh.E_loc, pad=128, pad_fill=0x7FC0)
    dA, dmi = to_dev_bf16(A), to_dev(mi)
    oc = {nr: bits(M.grouped_contiguous(dA, P.p1, dmi, cfg=M.config(128, nr, kind="contiguous"))) for nr in (4, 2)}
    ok = mi >= 0
    np.testing.assert_array_equal(oc[4][ok], oc[2][ok], err_msg="contiguous: N-tile loop")
    log("N-tile loop: bit-identical to the general kernel; rows", int(ok.sum()))
