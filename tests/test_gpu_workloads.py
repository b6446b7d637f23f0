"""GPU parity at the full workload sizes, in the tile configuration the
selector picks (the one bench.py times): routed outputs on sampled rows and
columns against the oracle, plus whole-output properties checked on the GPU
(non-local slot rows untouched, combine rows finite)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import workloads as W
from tests.gpu_util import Problem, assert_close, bits, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

import w4a16_int4_mixture_moe_amd as M  # noqa: E402  (fails loudly if the binding is broken)


def _sample(rng, n, k):
    if n <= k:
        return np.arange(n)
    s = rng.choice(n, size=k, replace=False)
    return np.unique(np.concatenate([s, [0, n - 1]]))


def _indexed_full(P, name):
    sh = P.sh
    T, k = P.T, sh.topk
    cfg1 = M.select(T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, cfg1.block_m)
    canary = torch.full((T * k, sh.N1), -3.0, dtype=torch.bfloat16, device="cuda")
    # cfg=None: each projection runs the library's own choice for the routing
    # (block_m fixed by the routing; split_k per projection)
    h = M.moe_w4a16_gemm(P.d_x, P.p1, r, out=canary)
    y = M.moe_w4a16_gemm(P.d_a, P.p2, r, topk_weights=P.d_w)
    torch.cuda.synchronize()
    assert M.indexed_config(r, P.p1).split_k == cfg1.split_k
    log(name, "gate/up", M.indexed_config(r, P.p1), "down", M.indexed_config(r, P.p2),
        "ntp", int(r.num_tokens_padded.item()))
    flat = P.topk_ids.reshape(-1)
    ok = (flat >= sh.first) & (flat < sh.first + sh.E_loc)
    d_ok = torch.from_numpy(ok).cuda()
    assert bool((h[~d_ok].float() == -3.0).all()), "a non-local slot row was written"
    assert bool(torch.isfinite(h[d_ok].float()).all()) and bool(torch.isfinite(y.float()).all())
    rng = np.random.default_rng(123)
    loc = np.nonzero(ok)[0]
    slots = loc[_sample(rng, len(loc), 96)]
    cols = _sample(rng, sh.N1, 96)
    ref, _ = O.indexed_gate_up(P.x, P.c1, P.s1, P.topk_ids, sh.first, sh.E_loc, slots=slots, cols=cols)
    got = bits(h[torch.from_numpy(slots).cuda()][:, torch.from_numpy(cols).cuda()])
    e1, x1 = assert_close(got, ref, name + " gate/up")
    toks = _sample(rng, T, 64)
    cols2 = _sample(rng, sh.N2, 96)
    ref2 = O.indexed_down_combine(P.a, P.c2, P.s2, P.topk_ids, P.topk_w, sh.first, sh.E_loc,
                                  tokens=toks, cols=cols2)
    got2 = bits(y[torch.from_numpy(toks).cuda()][:, torch.from_numpy(cols2).cuda()])
    e2, x2 = assert_close(got2, ref2, name + " down+combine")
    log(name, dict(gate_up_max_err=e1, gate_up_exact=x1, down_max_err=e2, down_exact=x2))


@pytest.mark.parametrize("name", ["ep8_decode", "ep8_prefill", "ep16_decode", "ep32_decode", "ep16_prefill",
                                  "ep32_prefill", "k3_decode"])
def test_ep_full_size(name):
    log("generating", name)
    P = Problem(W.WORKLOADS[name]).upload()
    _indexed_full(P, name)


@pytest.fixture(scope="module")
def tp8_weights():
    sh = W.WORKLOADS["tp8_t1"]
    c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
    s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
    c2 = W.weight_codes(sh.seed, "w2_codes", sh.E_loc, sh.N2, sh.K2)
    s2 = W.weight_scales(sh.seed, "w2_scales", sh.E_loc, sh.N2, sh.K2)
    p1 = M.pack_w4(to_dev(c1), to_dev_bf16(s1))
    p2 = M.pack_w4(to_dev(c2), to_dev_bf16(s2))
    return c1, s1, c2, s2, p1, p2


@pytest.mark.parametrize("T", W.TP8_TOKENS)
def test_tp8_sweep_full_size(T, tp8_weights):
    sh = W.WORKLOADS[f"tp8_t{T}"]
    P = Problem.__new__(Problem)
    P.sh, P.T, P.with_down = sh, T, True
    P.topk_ids, P.topk_w = W.routing_for(sh)
    P.x = W.activations(sh.seed, "x", T, sh.K1)
    P.a = W.activations(sh.seed, "a", T * sh.topk, sh.K2)
    P.c1, P.s1, P.c2, P.s2, P.p1, P.p2 = tp8_weights
    P.d_ids, P.d_w = to_dev(P.topk_ids), to_dev(P.topk_w)
    P.d_x, P.d_a = to_dev_bf16(P.x), to_dev_bf16(P.a)
    _indexed_full(P, f"tp8_t{T}")


def test_grouped_full_size():
    sh = W.WORKLOADS["grouped_skewed"]
    log("generating grouped_skewed")
    P = Problem(sh, with_down=False).upload()
    rng = np.random.default_rng(7)
    A, mi, slots = W.contiguous_layout(P.topk_ids, P.x, sh.first, sh.E_loc, pad=128, pad_fill=0x7FC0)
    n_zero = int(sum(1 for e in range(sh.E_loc) if not (mi == e).any()))
    log("contiguous rows", A.shape[0], "zero-row experts", n_zero)
    assert n_zero >= 4
    out = M.grouped_contiguous(to_dev_bf16(A), P.p1, to_dev(mi))
    torch.cuda.synchronize()
    valid = np.nonzero(mi >= 0)[0]
    rows = valid[_sample(rng, len(valid), 128)]
    cols = _sample(rng, sh.N1, 96)
    ref, _ = O.grouped_contiguous(A, P.c1, P.s1, mi, rows=rows, cols=cols)
    got = bits(out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    log("contiguous", assert_close(got, ref, "contiguous"))
    d_valid = torch.from_numpy(mi >= 0).cuda()
    assert bool(torch.isfinite(out[d_valid].float()).all()), "NaN padding leaked into valid rows"

    A3, mm, sl3, dropped = W.masked_layout(P.topk_ids, P.x, sh.first, sh.E_loc, sh.max_m, pad_fill=0x7FC0)
    log("masked: max_m", sh.max_m, "dropped", dropped, "max count", int(mm.max()))
    expected_m = max(1, int(round(float(mm.mean()))))
    out3 = M.grouped_masked(to_dev_bf16(A3), P.p1, to_dev(mm), expected_m)
    torch.cuda.synchronize()
    groups = np.unique(np.concatenate([rng.choice(sh.E_loc, 6, replace=False), [int(np.argmax(mm))]]))
    cols = _sample(rng, sh.N1, 64)
    ref3, v3 = O.grouped_masked(A3, P.c1, P.s1, mm, groups=groups, cols=cols)
    rows3 = (groups[:, None] * sh.max_m + np.arange(sh.max_m)[None, :]).reshape(-1)
    got3 = bits(out3[torch.from_numpy(rows3).cuda()][:, torch.from_numpy(cols).cuda()])
    log("masked", assert_close(got3[v3], ref3[v3], "masked"))
