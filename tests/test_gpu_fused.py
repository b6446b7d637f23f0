"""GPU checks of the gate/up-interleaved packing, the fused SiLU gate/up call
and the down projection reading rows in sorted order.

* Interleaved packing changes only where tiles live: every call on it gives
  the same output bits as on the plain packing.
* The fused epilogue against the oracle's activation of the GPU's own
  per-slot gate/up output (identical bf16 inputs): at most one bf16 ulp
  apart (fp32 + exp on the GPU, fp64 in the oracle).
* Down on sorted rows is bit-identical to down on the same rows gathered
  per slot (same values, same accumulation).
* The whole chain (gate/up -> SiLU -> down + combine) against the oracle's
  chain within the stated tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import workloads as W
from tests.gpu_util import Problem, assert_close, bits, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

import w4a16_int4_mixture_moe_amd as M  # noqa: E402


def _gate_up_shapes():
    tiny = W.WORKLOADS["tiny"]                                        # K2 = N1 / 2 already
    ragged = W.MoEShape(name="ragged_gu", E_glob=9, E_loc=5, first=2, topk=3, T=37, K1=96, N1=64,
                        K2=32, N2=80, seed=78)
    deep = W.MoEShape(name="deep_gu", E_glob=8, E_loc=6, first=1, topk=2, T=40, K1=1312, N1=192,
                      K2=96, N2=96, seed=92)
    return [tiny, ragged, deep]


def _ulp(ref_bits):
    r = np.abs(O.bf16_to_f64(ref_bits))
    e = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    return np.where(r > 0, 2.0 ** (e - 7), 2.0 ** -133)


def test_interleaved_packing_keeps_outputs():
    P = Problem(W.WORKLOADS["tiny"]).upload()
    sh = P.sh
    p1g = M.pack_w4(to_dev(P.c1), to_dev_bf16(P.s1), gate_up=True)
    assert p1g.gate_up and not P.p1.gate_up
    for bm, nr, nw in ((16, 2, 4), (32, 4, 4), (128, 2, 8)):
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        cfg = M.config(bm, nr, waves=nw)
        h = M.moe_w4a16_gemm(P.d_x, P.p1, r, cfg=cfg)
        hg = M.moe_w4a16_gemm(P.d_x, p1g, r, cfg=cfg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(hg), bits(h), err_msg=f"bm={bm} nr={nr} waves={nw}")
    A, mi, _ = W.contiguous_layout(P.topk_ids, P.x, sh.first, sh.E_loc, pad=128)
    o = M.grouped_contiguous(to_dev_bf16(A), P.p1, to_dev(mi))
    og = M.grouped_contiguous(to_dev_bf16(A), p1g, to_dev(mi))
    torch.cuda.synchronize()
    valid = mi >= 0
    np.testing.assert_array_equal(bits(og)[valid], bits(o)[valid])


@pytest.mark.parametrize("shape", _gate_up_shapes(), ids=lambda s: s.name)
def test_fused_silu_and_sorted_down(shape):
    sh = shape
    assert sh.K2 == sh.N1 // 2
    P = Problem(sh).upload()
    T, k = P.T, sh.topk
    p1g = M.pack_w4(to_dev(P.c1), to_dev_bf16(P.s1), gate_up=True)
    # oracle chain: per-slot gate/up, activation, down + combine on slot rows
    h_ref, ok = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc)
    a_ref = np.zeros((T * k, sh.K2), np.uint16)
    a_ref[ok] = O.silu_mul(h_ref[ok])
    y_ref = O.indexed_down_combine(a_ref, P.c2, P.s2, P.topk_ids, P.topk_w, sh.first, sh.E_loc)
    # (16, 1, 8): one tile (a gate / up pair in the fused call) per workgroup,
    # waves splitting K, built for K a multiple of 128
    kw = ((16, 1, 8),) if sh.K1 % 128 == 0 and sh.K2 % 128 == 0 else ()
    for bm, nr, nw in ((16, 2, 4), (32, 2, 4), (64, 4, 4), (128, 2, 4), (32, 2, 8)) + kw:
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        cfg = M.config(bm, nr, waves=nw)
        h = M.moe_w4a16_gemm(P.d_x, p1g, r, cfg=cfg)
        inter = M.moe_gate_up_silu(P.d_x, p1g, r, cfg=cfg)
        torch.cuda.synchronize()
        sid = r.sorted_ids.cpu().numpy()
        ref_i, valid = O.gate_up_silu_sorted(bits(h), sid, T * k)
        got_i = bits(inter)[valid]
        err = np.abs(O.bf16_to_f64(got_i) - O.bf16_to_f64(ref_i[valid]))
        assert (err <= _ulp(ref_i[valid])).all(), f"bm={bm}: fused activation off by more than one ulp"
        # down on sorted rows == down on the same rows gathered per slot
        a_slot = torch.zeros(T * k, sh.K2, dtype=torch.bfloat16, device="cuda")
        vpos = torch.from_numpy(np.nonzero(valid)[0]).cuda()
        a_slot[torch.from_numpy(sid[valid].astype(np.int64)).cuda()] = inter[vpos]
        y_sorted = M.moe_w4a16_gemm(inter, P.p2, r, topk_weights=P.d_w, a_layout="sorted", cfg=cfg)
        y_slot = M.moe_w4a16_gemm(a_slot, P.p2, r, topk_weights=P.d_w, a_layout="slot", cfg=cfg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(y_sorted), bits(y_slot), err_msg=f"bm={bm}")
        e, x = assert_close(bits(y_sorted), y_ref, f"{sh.name} chain bm={bm} nr={nr} waves={nw}")
        log(sh.name, f"bm={bm} nr={nr} waves={nw}", dict(chain_max_err=e, chain_exact=x,
                                                           silu_exact=float(np.mean(err == 0))))


def test_fused_full_size_ep8_decode():
    """The selector's configuration at the EP8 decode size: fused activation
    against the oracle's activation of the GPU's per-slot output on sampled
    positions, and sorted-row down bit-identical to gathered-row down."""
    sh = W.WORKLOADS["ep8_decode"]
    P = Problem(sh).upload()
    T, k = P.T, sh.topk
    p1g = M.pack_w4(to_dev(P.c1), to_dev_bf16(P.s1), gate_up=True)
    cfg = M.select(T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    cfg.split_k = 1
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, cfg.block_m)
    h = M.moe_w4a16_gemm(P.d_x, p1g, r, cfg=cfg)
    inter = M.moe_gate_up_silu(P.d_x, p1g, r, cfg=cfg)
    torch.cuda.synchronize()
    sid = r.sorted_ids.cpu().numpy()
    ref_i, valid = O.gate_up_silu_sorted(bits(h), sid, T * k)
    got = bits(inter)
    err = np.abs(O.bf16_to_f64(got[valid]) - O.bf16_to_f64(ref_i[valid]))
    assert (err <= _ulp(ref_i[valid])).all()
    # gate/up on the interleaved packing equals the oracle on sampled slots
    rng = np.random.default_rng(5)
    flat = P.topk_ids.reshape(-1)
    loc = np.nonzero((flat >= sh.first) & (flat < sh.first + sh.E_loc))[0]
    slots = rng.choice(loc, 48, replace=False)
    cols = rng.choice(sh.N1, 64, replace=False)
    ref_h, _ = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc, slots=slots, cols=cols)
    assert_close(bits(h)[slots][:, cols], ref_h, "ep8 gate/up on interleaved packing")
    # the down projection on sorted rows needs K2 = N1 / 2 = 2048: that is this workload's down K
    assert sh.K2 == sh.N1 // 2
    a_slot = torch.zeros(T * k, sh.K2, dtype=torch.bfloat16, device="cuda")
    vpos = torch.from_numpy(np.nonzero(valid)[0]).cuda()
    a_slot[torch.from_numpy(sid[valid].astype(np.int64)).cuda()] = inter[vpos]
    y_sorted = M.moe_w4a16_gemm(inter, P.p2, r, topk_weights=P.d_w, a_layout="sorted", cfg=cfg)
    y_slot = M.moe_w4a16_gemm(a_slot, P.p2, r, topk_weights=P.d_w, a_layout="slot", cfg=cfg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y_sorted), bits(y_slot))
    log("ep8 fused", dict(silu_exact=float(np.mean(err == 0)), positions=int(valid.sum())))
