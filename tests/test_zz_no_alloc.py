"""The allocation-free entry point w4a16_moe_gemm_noalloc, called through the
C ABI: bit-identical to w4a16_moe_gemm with a caller workspace on the same
inputs and config, on two calls in a row (the second smaller), for the top-k
combine and for split-K (whose arrival counters live in the library's scratch
array), and a call needing more than the scratch array is refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import Problem, bits, dev, log

pytestmark = pytest.mark.gpu

import w4a16_int4_mixture_moe_amd as M  # noqa: E402
from w4a16_int4_mixture_moe_amd import _lib  # noqa: E402


def _call(fn, P, packed, a, a_layout, r, w, out, cfg, ws=None):
    L = M.load()
    rc = r.as_c()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    common = (ctypes.byref(packed.desc), packed.w.data_ptr(), packed.s.data_ptr(), a.data_ptr(), a.shape[0],
              a_layout, ctypes.byref(rc), None if w is None else w.data_ptr(), out.data_ptr(),
              None if cfg is None else ctypes.byref(cfg))
    if fn == "noalloc":
        return L.w4a16_moe_gemm_noalloc(*common, s)
    return L.w4a16_moe_gemm(*common, None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), s)


def _compare(P, T, cfg_gu, cfg_dn):
    """gate/up (per slot) and down + combine through both entry points."""
    sh = P.sh
    ids = P.d_ids[:T].contiguous()
    r = M.moe_align(ids, sh.E_glob, sh.first, sh.E_loc, cfg_gu.block_m)
    x, a, wts = P.d_x[:T].contiguous(), P.d_a[:T * sh.topk].contiguous(), P.d_w[:T].contiguous()
    res = {}
    for fn in ("noalloc", "workspace"):
        h = torch.full((T * sh.topk, sh.N1), -2.0, dtype=torch.bfloat16, device=dev())
        y = torch.full((T, sh.N2), 3.0, dtype=torch.bfloat16, device=dev())
        ws1 = torch.zeros(max(16, M.workspace_bytes(P.p1, r, False, cfg_gu)), dtype=torch.uint8, device=dev())
        ws2 = torch.zeros(max(16, M.workspace_bytes(P.p2, r, True, cfg_dn)), dtype=torch.uint8, device=dev())
        assert _call(fn, P, P.p1, x, _lib.A_TOKEN, r, None, h, cfg_gu, ws1) == 0, M.load().w4a16_last_error()
        assert _call(fn, P, P.p2, a, _lib.A_SLOT, r, wts, y, cfg_dn, ws2) == 0, M.load().w4a16_last_error()
        torch.cuda.synchronize()
        res[fn] = (bits(h).copy(), bits(y).copy())
    np.testing.assert_array_equal(res["noalloc"][0], res["workspace"][0], err_msg=f"gate/up T={T}")
    np.testing.assert_array_equal(res["noalloc"][1], res["workspace"][1], err_msg=f"down+combine T={T}")
    log("no-alloc matches the workspace entry point, T =", T, cfg_gu, cfg_dn)


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    sh = W.MoEShape(name="noalloc", E_glob=64, E_loc=16, first=8, topk=4, T=300, K1=2048, N1=256, K2=512,
                    N2=1024, seed=1234)
    P = Problem(sh).upload()
    plain = M.config(32, 2)
    split = M.config(32, 2, split_k=4)       # counters and slices in the scratch array
    _compare(P, 300, split, M.config(32, 2, split_k=2))
    _compare(P, 77, split, M.config(32, 2, split_k=2))   # second call, smaller input
    _compare(P, 300, plain, plain)
    _compare(P, 41, plain, plain)
    # a 256-row routing (the 256-row tile for both projections; 128-row down
    # tiles over it) and the tile whose waves split K
    _compare(P, 300, M.config(256, 2, 8), M.config(256, 2, 8))
    _compare(P, 300, M.config(256, 2, 8), M.config(128, 4))
    _compare(P, 41, M.config(16, 1, 8), M.config(16, 1, 8))


def test_noalloc_refuses_calls_beyond_its_scratch():
    sh = W.MoEShape(name="noalloc_big", E_glob=8, E_loc=8, first=0, topk=8, T=640, K1=256, N1=64, K2=256,
                    N2=7168, seed=99)
    P = Problem(sh).upload()
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 32)
    one_pass = M.config(32, 2, combine_cols=sh.N2)
    need = M.workspace_bytes(P.p2, r, True, one_pass)
    assert need > 128 << 20                 # 640 x 8 x 7168 x 4 bytes of combine partials in one pass
    y = torch.full((sh.T, sh.N2), 3.0, dtype=torch.bfloat16, device=dev())
    st = _call("noalloc", P, P.p2, P.d_a, _lib.A_SLOT, r, P.d_w, y, one_pass)
    assert st == -8 and b"scratch" in M.load().w4a16_last_error()
    torch.cuda.synchronize()
    assert bool((y.float() == 3.0).all()), "a refused call wrote its output"
    # the same combine in two passes of 3584 columns fits the scratch array:
    # same bits as the workspace call
    two_passes = M.config(32, 2, combine_cols=3584)
    assert M.workspace_bytes(P.p2, r, True, two_passes) == 640 * 8 * 3584 * 4 + 768   # + local-slot counts
    _compare(P, sh.T, M.config(32, 2), two_passes)
