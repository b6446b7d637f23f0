"""GPU parity of the A4W4 (MXFP4 x MXFP4) path against the CPU oracle.

* quantisation: codes and scales bit-exact against the oracle's conversion,
  on random rows and on blocks built to hit every rounding tie, clamping,
  zero, negative-zero and subnormal case;
* GEMM: per-slot gate/up and down + top-k combine within the stated
  tolerance on small and ragged shapes, over every built tile configuration,
  fed the oracle's own quantised rows (so the GEMM is checked on its own);
  output bits independent of the tile configuration; non-local rows left
  untouched;
* closed form: one-hot activation rows read back dequantised weights exactly;
* the chain GPU quantisation -> GPU GEMM against the oracle's chain;
* the EP8 decode share at full size on sampled output columns.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import mx_oracle as X
from synth import workloads as W
from tests.gpu_util import assert_close, bits, dev, log, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

import w4a16_int4_mixture_moe_amd as M  # noqa: E402

CONFIGS = [(16, 2), (16, 4), (32, 2), (32, 4), (64, 2), (64, 4), (128, 2), (128, 4)]


def _gpu_quant(x_bits):
    q = M.mxfp4_quant(to_dev_bf16(x_bits))
    torch.cuda.synchronize()
    return X.unpack_nibbles(q.codes.cpu().numpy()), q.scales.cpu().numpy()


def _mx_rows(codes, scales):
    return M.MXRows(to_dev(X.pack_nibbles(codes)), to_dev(np.ascontiguousarray(scales)))


# ------------------------------------------------------------ quantisation

def _special_rows():
    """Blocks of 32 that exercise every branch of the conversion."""
    rows = []
    z = [0.0] * 32
    rows.append(z)                                                  # zero block
    rows.append([-0.0] * 32)                                        # negative zeros
    for k in (-3, 0, 5):
        X_ = 2.0 ** k
        # amax 6X fixes the shared exponent at k; the rest sit on every tie
        ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.24, 0.26, 5.01, 6.0]
        blk = [6.0 * X_] + [t * X_ for t in ties] + [-t * X_ for t in ties]
        rows.append(blk + [0.0] * (32 - len(blk)))
    rows.append([7.0 * 2.0 ** 3] + [7.5 * 2.0 ** 3] + [-7.9 * 2.0 ** 3] + [0.0] * 29)   # clamp at 6
    rows.append([2.0 ** -130, -(2.0 ** -128), 2.0 ** -127] + [0.0] * 29)                # subnormals
    rows.append([2.0 ** 100, -(2.0 ** 99)] + [1.0] * 30)                               # large
    vals = np.array(rows, np.float32)
    out = W.to_bf16_bits(vals)
    out[1] = 0x8000
    return out


@pytest.mark.parametrize("K", [32, 96, 256, 7168])
def test_mx_quant_bit_exact(K):
    rng = np.random.default_rng(K)
    R = 96
    v = rng.standard_normal((R, K)).astype(np.float32)
    v *= np.repeat(2.0 ** rng.integers(-20, 20, (R, K // 32)), 32, axis=1).astype(np.float32)
    x = W.to_bf16_bits(v)
    if K >= 32:
        sp = _special_rows()
        x[: len(sp), :32] = sp
    gc, gs = _gpu_quant(x)
    oc, os_ = X.mx_quantize(x)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gc, oc)
    log(f"mx quant K={K}: {R} rows bit-exact")


def test_mx_quant_local_slots_converts_exactly_the_local_rows():
    """Per-slot rows: local slots' rows equal the oracle's conversion bit for
    bit; the rows of other slots (non-local ids, -1) keep their old bytes."""
    rng = np.random.default_rng(11)
    T, k, K, E_glob, first, E_loc = 37, 4, 256, 16, 5, 6
    ids = rng.integers(-1, E_glob, (T, k)).astype(np.int32)
    x = W.to_bf16_bits(rng.standard_normal((T * k, K)).astype(np.float32))
    r = M.moe_align(to_dev(ids), E_glob, first, E_loc, 16)
    out = M.MXRows(torch.full((T * k, K // 2), 0xA5, dtype=torch.uint8, device=dev()),
                   torch.full((T * k, K // 32), 0x5A, dtype=torch.uint8, device=dev()))
    M.mxfp4_quant_local_slots(to_dev_bf16(x), r, out=out)
    torch.cuda.synchronize()
    gc, gs = X.unpack_nibbles(out.codes.cpu().numpy()), out.scales.cpu().numpy()
    local = ((ids >= first) & (ids < first + E_loc)).reshape(-1)
    oc, os_ = X.mx_quantize(x[local])
    np.testing.assert_array_equal(gc[local], oc)
    np.testing.assert_array_equal(gs[local], os_)
    assert (out.codes.cpu().numpy()[~local] == 0xA5).all() and (gs[~local] == 0x5A).all()
    log(f"mx local-slot quant: {int(local.sum())} of {T * k} rows converted, others untouched")


# ------------------------------------------------------------ GEMM

class MxProblem:
    def __init__(self, sh, T=None):
        self.sh = sh
        self.T = sh.T if T is None else T
        self.topk_ids, self.topk_w = W.routing_for(sh, self.T)
        x = W.activations(sh.seed, "x", self.T, sh.K1)
        a = W.activations(sh.seed, "a", self.T * sh.topk, sh.K2)
        self.xq = X.mx_quantize(x)                     # oracle's quantised rows
        self.aq = X.mx_quantize(a)
        self.x_bits, self.a_bits = x, a
        self.w1 = W.mx_weight_codes(sh.seed, "w1_mx_codes", sh.E_loc, sh.N1, sh.K1)
        self.s1 = W.mx_weight_scales(sh.seed, "w1_mx_scales", sh.E_loc, sh.N1, sh.K1)
        self.w2 = W.mx_weight_codes(sh.seed, "w2_mx_codes", sh.E_loc, sh.N2, sh.K2)
        self.s2 = W.mx_weight_scales(sh.seed, "w2_mx_scales", sh.E_loc, sh.N2, sh.K2)

    def upload(self):
        self.p1 = M.pack_mxfp4(to_dev(self.w1), to_dev(self.s1))
        self.p2 = M.pack_mxfp4(to_dev(self.w2), to_dev(self.s2))
        self.d_ids = to_dev(self.topk_ids)
        self.d_w = to_dev(self.topk_w)
        self.d_x = _mx_rows(*self.xq)
        self.d_a = _mx_rows(*self.aq)
        torch.cuda.synchronize()
        return self


def _shapes():
    tiny = W.WORKLOADS["tiny"]
    ragged = W.MoEShape(name="ragged_mx", E_glob=9, E_loc=5, first=2, topk=3, T=37, K1=384, N1=80,
                        K2=128, N2=48, seed=81)
    deep = W.MoEShape(name="deep_mx", E_glob=8, E_loc=6, first=1, topk=2, T=70, K1=1408, N1=96,
                      K2=256, N2=64, seed=93)
    return [tiny, ragged, deep]


@pytest.mark.parametrize("shape", _shapes(), ids=lambda s: s.name)
def test_mx_gemm_vs_oracle(shape):
    sh = shape
    P = MxProblem(sh).upload()
    T, k = P.T, sh.topk
    h_ref, ok = X.mx_indexed_gate_up(*P.xq, X.unpack_nibbles(P.w1), P.s1, P.topk_ids, sh.first, sh.E_loc)
    y_ref = X.mx_indexed_down_combine(*P.aq, X.unpack_nibbles(P.w2), P.s2, P.topk_ids, P.topk_w,
                                      sh.first, sh.E_loc)
    first_bits = None
    for bm, nr in CONFIGS:
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        cfg = M.mxfp4_config(bm, nr)
        canary = torch.full((T * k, sh.N1), 0x7F81, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        h = M.moe_mxfp4_gemm(P.d_x, P.p1, r, cfg=cfg, out=canary)
        y = M.moe_mxfp4_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=cfg)
        torch.cuda.synchronize()
        hb, yb = bits(h), bits(y)
        assert (hb[~ok] == 0x7F81).all(), "non-local per-slot rows were written"
        e1, x1 = assert_close(hb[ok], h_ref[ok], f"{sh.name} gate/up bm={bm} nr={nr}")
        e2, x2 = assert_close(yb, y_ref, f"{sh.name} down+combine bm={bm} nr={nr}")
        if first_bits is None:
            first_bits = (hb, yb)
        else:
            np.testing.assert_array_equal(hb[ok], first_bits[0][ok], err_msg=f"bits depend on config bm={bm} nr={nr}")
            np.testing.assert_array_equal(yb, first_bits[1], err_msg=f"bits depend on config bm={bm} nr={nr}")
        log(sh.name, f"bm={bm} nr={nr}", dict(gu_err=e1, gu_exact=x1, dn_err=e2, dn_exact=x2))


def test_mx_kwave_tile_vs_oracle():
    """The A4W4 K-split tile (block_m 16, nr 1: eight waves share a 16-row
    weight tile's K chunks and sum in wave order): within tolerance of the
    oracle for the per-slot store and the top-k combine, with two batches of
    chunks per wave (K = 10240: ten chunks each), one or two chunks per wave
    (K = 1152, 640), and waves without chunks (K = 256); non-local rows
    untouched; and the call's own choice on a 16-row routing."""
    for K1, K2, seed in ((10240, 256, 61), (1152, 640, 62)):
        sh = W.MoEShape(name=f"mx_kwave_{K1}", E_glob=8, E_loc=5, first=2, topk=2, T=21, K1=K1, N1=64,
                        K2=K2, N2=48, seed=seed)
        P = MxProblem(sh).upload()
        T, k = P.T, sh.topk
        h_ref, ok = X.mx_indexed_gate_up(*P.xq, X.unpack_nibbles(P.w1), P.s1, P.topk_ids, sh.first, sh.E_loc)
        y_ref = X.mx_indexed_down_combine(*P.aq, X.unpack_nibbles(P.w2), P.s2, P.topk_ids, P.topk_w,
                                          sh.first, sh.E_loc)
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 16)
        for cfg in (M.mxfp4_config(16, 1), None):
            canary = torch.full((T * k, sh.N1), 0x7F81, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            h = M.moe_mxfp4_gemm(P.d_x, P.p1, r, cfg=cfg, out=canary)
            y = M.moe_mxfp4_gemm(P.d_a, P.p2, r, topk_weights=P.d_w, cfg=cfg)
            torch.cuda.synchronize()
            hb, yb = bits(h), bits(y)
            what = f"{sh.name} {'nr 1' if cfg is not None else 'cfg None'}"
            assert (hb[~ok] == 0x7F81).all(), "non-local per-slot rows were written"
            e1, x1 = assert_close(hb[ok], h_ref[ok], what + " gate/up")
            e2, x2 = assert_close(yb, y_ref, what + " down+combine")
            log(what, dict(gu_err=e1, gu_exact=x1, dn_err=e2, dn_exact=x2))


def test_mx_one_hot_reads_weights_exactly():
    sh = W.MoEShape(name="onehot_mx", E_glob=6, E_loc=4, first=1, topk=2, T=40, K1=512, N1=64,
                    K2=128, N2=32, seed=55)
    P = MxProblem(sh)
    rng = np.random.default_rng(2)
    cols = rng.integers(0, sh.K1, P.T)
    x = np.zeros((P.T, sh.K1), np.float32)
    x[np.arange(P.T), cols] = 1.0
    P.xq = X.mx_quantize(W.to_bf16_bits(x))
    P.upload()
    w_val = X.mx_dequant(X.unpack_nibbles(P.w1), P.s1)                 # [E, N, K] exact
    for bm, nr in ((16, 4), (64, 2), (128, 4)):
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        h = bits(M.moe_mxfp4_gemm(P.d_x, P.p1, r, cfg=M.mxfp4_config(bm, nr)))
        flat = P.topk_ids.reshape(-1)
        for s in range(P.T * sh.topk):
            e = int(flat[s]) - sh.first
            if 0 <= e < sh.E_loc:
                # values, so -0 (weight code 8) equals the +0 the fp32
                # accumulation starting from +0 produces
                want = O.bf16_to_f64(O.f64_to_bf16(w_val[e, :, cols[s // sh.topk]]))
                np.testing.assert_array_equal(O.bf16_to_f64(h[s]), want, err_msg=f"slot {s} bm={bm}")


def test_mx_chain_gpu_quant_then_gemm():
    sh = W.WORKLOADS["tiny"]
    P = MxProblem(sh).upload()
    # the GEMM fed by the device quantiser equals the oracle's chain
    q = M.mxfp4_quant(to_dev_bf16(P.x_bits))
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, 32)
    h = bits(M.moe_mxfp4_gemm(q, P.p1, r))
    h_ref, ok = X.mx_indexed_gate_up(*X.mx_quantize(P.x_bits), X.unpack_nibbles(P.w1), P.s1, P.topk_ids,
                                     sh.first, sh.E_loc)
    assert_close(h[ok], h_ref[ok], "quant -> gemm chain")


def test_mx_no_local_slots_and_empty():
    sh = W.WORKLOADS["tiny"]
    P = MxProblem(sh).upload()
    d_ids = to_dev(np.full_like(P.topk_ids, -1, dtype=np.int32))       # no slot is local
    r = M.moe_align(d_ids, sh.E_glob, sh.first, sh.E_loc, 32)
    y = M.moe_mxfp4_gemm(P.d_a, P.p2, r, topk_weights=P.d_w)
    torch.cuda.synchronize()
    assert (bits(y) == 0).all()
    e = torch.zeros((0, sh.topk), dtype=torch.int32, device="cuda")
    r0 = M.moe_align(e, sh.E_glob, sh.first, sh.E_loc, 32)
    q0 = M.mxfp4_quant(torch.zeros((0, sh.K1), dtype=torch.bfloat16, device="cuda"))
    out = M.moe_mxfp4_gemm(q0, P.p1, r0)
    torch.cuda.synchronize()
    assert out.shape == (0, sh.N1)


@pytest.mark.parametrize("name", ["ep8_decode", "k3_decode", "ep8_prefill"])
def test_mx_full_size(name):
    """Full-size shares (EP8 decode and prefill: 48 experts, N 4096, K 7168
    and the down projection; the K3-like routing), with the selector's
    block_m: all slots, 64 sampled output columns, against the oracle."""
    log("generating", name)
    sh = W.WORKLOADS[name]
    P = MxProblem(sh).upload()
    T, k = P.T, sh.topk
    cfg0 = M.select(T, k, sh.E_glob, sh.E_loc, sh.N1, sh.K1)
    r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, cfg0.block_m)
    h = bits(M.moe_mxfp4_gemm(P.d_x, P.p1, r))
    y = bits(M.moe_mxfp4_gemm(P.d_a, P.p2, r, topk_weights=P.d_w))
    rng = np.random.default_rng(11)
    c1 = np.sort(rng.choice(sh.N1, 64, replace=False))
    c2 = np.sort(rng.choice(sh.N2, 64, replace=False))
    h_ref, ok = X.mx_indexed_gate_up(*P.xq, X.unpack_nibbles(P.w1[:, c1]), P.s1[:, c1], P.topk_ids,
                                     sh.first, sh.E_loc)
    y_ref = X.mx_indexed_down_combine(*P.aq, X.unpack_nibbles(P.w2[:, c2]), P.s2[:, c2], P.topk_ids,
                                      P.topk_w, sh.first, sh.E_loc)
    e1, x1 = assert_close(h[ok][:, c1], h_ref[ok], f"{name} mx gate/up")
    e2, x2 = assert_close(y[:, c2], y_ref, f"{name} mx down+combine")
    log(name, "mx full size", dict(block_m=cfg0.block_m, gu_err=e1, gu_exact=x1, dn_err=e2, dn_exact=x2))


# ------------------------------------------------------------ fused A4W4 chain

def _fused_shapes():
    tiny = W.WORKLOADS["tiny"]                                         # K2 = N1 / 2
    ragged = W.MoEShape(name="ragged_mxf", E_glob=9, E_loc=5, first=2, topk=3, T=37, K1=384, N1=256,
                        K2=128, N2=48, seed=83)
    deep = W.MoEShape(name="deep_mxf", E_glob=8, E_loc=6, first=1, topk=2, T=70, K1=1408, N1=512,
                      K2=256, N2=64, seed=95)
    return [tiny, ragged, deep]


@pytest.mark.parametrize("shape", _fused_shapes(), ids=lambda s: s.name)
def test_mx_fused_silu_quant_and_sorted_down(shape):
    """Fused A4W4 gate/up (activation + MXFP4 quantisation in sorted order)
    against the oracle's activation and quantiser applied to the GPU's own
    per-slot gate/up output; the down projection on the sorted rows
    bit-identical to the same rows gathered per slot; the chain against the
    oracle's chain."""
    sh = shape
    assert sh.K2 == sh.N1 // 2
    P = MxProblem(sh).upload()
    T, k = P.T, sh.topk
    p1g = M.pack_mxfp4(to_dev(P.w1), to_dev(P.s1), gate_up=True)
    # oracle chain: per-slot gate/up, activation, MXFP4, down + combine
    h_ref, ok = X.mx_indexed_gate_up(*P.xq, X.unpack_nibbles(P.w1), P.s1, P.topk_ids, sh.first, sh.E_loc)
    a_ref = np.zeros((T * k, sh.K2), np.uint16)
    a_ref[ok] = O.silu_mul(h_ref[ok])
    y_ref = X.mx_indexed_down_combine(*X.mx_quantize(a_ref), X.unpack_nibbles(P.w2), P.s2, P.topk_ids, P.topk_w,
                                      sh.first, sh.E_loc)
    # nr 1: the K-split tile (four packed tiles per workgroup in the fused call)
    for bm, nr in ((16, 4), (32, 4), (64, 4), (128, 4), (16, 1)):
        r = M.moe_align(P.d_ids, sh.E_glob, sh.first, sh.E_loc, bm)
        cfg = M.mxfp4_config(bm, nr)
        h = M.moe_mxfp4_gemm(P.d_x, P.p1, r, cfg=cfg)
        hg = M.moe_mxfp4_gemm(P.d_x, p1g, r, cfg=cfg)
        inter = M.moe_mxfp4_gate_up_silu(P.d_x, p1g, r, cfg=cfg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(hg), bits(h), err_msg=f"interleaved packing changed bits, bm={bm} nr={nr}")
        sid = r.sorted_ids.cpu().numpy()
        valid = sid < T * k
        # the oracle's activation and quantiser on the GPU's per-slot values
        hb = bits(h)
        act = O.silu_mul(hb[sid[valid]])
        rc, rs = X.mx_quantize(act)
        gc = X.unpack_nibbles(inter.codes.cpu().numpy())[valid]
        gs = inter.scales.cpu().numpy()[valid]
        same_s = gs == rs
        same_c = gc == rc
        got_v = X.mx_dequant(gc, gs)
        ref_v = X.mx_dequant(rc, rs)
        # a one-ulp difference in the bf16 activation (fp32 exp on the GPU,
        # fp64 in the oracle) can move a code by one step or the block scale
        # by one binade: at most one step of the coarser E2M1 spacing (2 X)
        bound = 2.0 * np.repeat(np.maximum(X.e8m0_to_f64(gs), X.e8m0_to_f64(rs)), 32, axis=1)
        assert np.all(np.abs(got_v - ref_v) <= bound), f"bm={bm} nr={nr}"
        assert same_s.mean() > 0.99 and same_c.mean() > 0.99, (same_s.mean(), same_c.mean())
        # down on sorted rows == down on the same rows gathered per slot
        slot_rows = M.MXRows(torch.zeros(T * k, sh.K2 // 2, dtype=torch.uint8, device="cuda"),
                             torch.zeros(T * k, sh.K2 // 32, dtype=torch.uint8, device="cuda"))
        vpos = torch.from_numpy(np.nonzero(valid)[0]).cuda()
        vslot = torch.from_numpy(sid[valid].astype(np.int64)).cuda()
        slot_rows.codes[vslot] = inter.codes[vpos]
        slot_rows.scales[vslot] = inter.scales[vpos]
        y_sorted = M.moe_mxfp4_gemm(inter, P.p2, r, topk_weights=P.d_w, a_layout="sorted", cfg=cfg)
        y_slot = M.moe_mxfp4_gemm(slot_rows, P.p2, r, topk_weights=P.d_w, a_layout="slot", cfg=cfg)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(y_sorted), bits(y_slot), err_msg=f"bm={bm} nr={nr}")
        e, x_ = assert_close(bits(y_sorted), y_ref, f"{sh.name} A4W4 chain bm={bm} nr={nr}")
        log(sh.name, f"bm={bm} nr={nr}", dict(chain_err=e, chain_exact=x_, codes_exact=float(same_c.mean()),
                                      scales_exact=float(same_s.mean())))


def test_mx_graph_capture_replays_match_eager():
    """The fused A4W4 step (align, quantise x, fused gate/up, sorted-row down
    + combine) captured in one HIP graph: replays reproduce the eager outputs
    bit for bit, with other eager work and poisoned buffers between them."""
    sh = W.WORKLOADS["tiny"]
    P = MxProblem(sh).upload()
    T, k = P.T, sh.topk
    p1g = M.pack_mxfp4(to_dev(P.w1), to_dev(P.s1), gate_up=True)
    bm = 32
    x = to_dev_bf16(P.x_bits)
    cap = M.align_capacity(T, k, sh.E_loc, bm)
    r = M.Routing(torch.empty(cap, dtype=torch.int32, device="cuda"),
                  torch.empty(cap // bm, dtype=torch.int32, device="cuda"),
                  torch.empty(1, dtype=torch.int32, device="cuda"), bm, P.d_ids, sh.E_glob, sh.first, sh.E_loc)
    q = M.MXRows(torch.empty(T, sh.K1 // 2, dtype=torch.uint8, device="cuda"),
                 torch.empty(T, sh.K1 // 32, dtype=torch.uint8, device="cuda"))
    inter = M.MXRows(torch.zeros(cap, sh.K2 // 2, dtype=torch.uint8, device="cuda"),
                     torch.zeros(cap, sh.K2 // 32, dtype=torch.uint8, device="cuda"))
    y = torch.empty(T, sh.N2, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(M.mxfp4_workspace_bytes(P.p2, T, k, True), dtype=torch.uint8, device="cuda")
    cfg = M.mxfp4_config(bm, 4)
    L = M.load()
    import ctypes

    def step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        M._lib.check(L.w4a16_moe_align(P.d_ids.data_ptr(), T, k, sh.E_glob, sh.first, sh.E_loc, bm,
                                       r.sorted_ids.data_ptr(), r.expert_ids.data_ptr(),
                                       r.num_tokens_padded.data_ptr(), cap, 0, s))
        M.mxfp4_quant(x, out=q)
        M.moe_mxfp4_gate_up_silu(q, p1g, r, cfg=cfg, out=inter)
        M.moe_mxfp4_gemm(inter, P.p2, r, topk_weights=P.d_w, a_layout="sorted", cfg=cfg, out=y, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_y = bits(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        r.sorted_ids.fill_(-5)
        q.codes.fill_(0xFF)
        y.fill_(1.0)
        ws.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(y), ref_y, err_msg=f"replay {rep}")
        _ = (x.float() @ x.float().t()).sum().item()                  # unrelated eager work
