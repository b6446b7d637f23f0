"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/w4a16_moe.h declares, and rejects bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

import w4a16_int4_mixture_moe_amd as W
from w4a16_int4_mixture_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16_moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(W.lib_path()):
        pytest.skip("library not built")
    return W.load()


def test_every_declared_function_is_exported_and_bound(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def test_struct_layouts_match_header():
    assert ctypes.sizeof(_lib.WeightDesc) == 64
    assert _lib.WeightDesc.flags.offset == 32 and _lib.WeightDesc.w_bytes.offset == 40
    assert ctypes.sizeof(_lib.Config) == 28 and _lib.Config.kind.offset == 20 and _lib.Config.combine_cols.offset == 24
    assert ctypes.sizeof(_lib.IndexedRouting) == 72 and _lib.IndexedRouting.E_glob.offset == 64
    assert _lib.IndexedRouting.capacity.offset == 24


def test_header_compiles_as_c_and_matches_the_binding(tmp_path):
    """The header is plain C (gcc -std=c99 -Wall -Werror), and the struct
    sizes and field offsets the C compiler gives agree with the ctypes
    mirrors the binding passes to the library, as do the constants."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"w4a16_weight_desc": _lib.WeightDesc, "w4a16_config": _lib.Config,
               "w4a16_indexed_routing": _lib.IndexedRouting}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "w4a16_moe.h"', "int main(void) {"]
    for cname, ct in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in ct._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    for const in ("W4A16_ABI_VERSION", "W4A16_DESC_GATE_UP", "W4A16_DESC_MXFP4", "W4A16_A_TOKEN", "W4A16_A_SLOT",
                  "W4A16_A_SORTED", "W4A16_ROUTE_INDEXED", "W4A16_ROUTE_CONTIGUOUS", "W4A16_ROUTE_MASKED"):
        lines.append(f'  printf("const {const} %d\\n", (int)({const}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        *key, val = line.split()
        got[tuple(key)] = int(val)
    for cname, ct in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(ct), cname
        for f, _ in ct._fields_:
            assert got[(cname, f)] == getattr(ct, f).offset, (cname, f)
    assert got[("const", "W4A16_DESC_GATE_UP")] == _lib.DESC_GATE_UP
    assert got[("const", "W4A16_DESC_MXFP4")] == _lib.DESC_MXFP4
    assert (got[("const", "W4A16_A_TOKEN")], got[("const", "W4A16_A_SLOT")],
            got[("const", "W4A16_A_SORTED")]) == (_lib.A_TOKEN, _lib.A_SLOT, _lib.A_SORTED)
    assert (got[("const", "W4A16_ROUTE_INDEXED")], got[("const", "W4A16_ROUTE_CONTIGUOUS")],
            got[("const", "W4A16_ROUTE_MASKED")]) == (_lib.ROUTE_INDEXED, _lib.ROUTE_CONTIGUOUS, _lib.ROUTE_MASKED)
    assert got[("const", "W4A16_ABI_VERSION")] == 8


def test_version_and_desc(L):
    assert L.w4a16_abi_version() == 8
    d = W.weight_desc(48, 4096, 7168)
    assert (d.K_pad, d.chunks, d.group) == (7168, 56, 32)
    assert d.w_bytes == 48 * 4096 * 7168 // 2
    assert d.s_bytes == 48 * 256 * 28 * 64 * 4
    d = W.weight_desc(2, 32, 96)                         # ragged K: padded to one chunk
    assert (d.K_pad, d.chunks) == (128, 1)


@pytest.mark.parametrize("E,N,K,code", [(0, 16, 32, -1), (1, 16, 33, -2), (1, 24, 32, -2), (1, 16, -32, -1)])
def test_desc_rejects_bad_shapes(L, E, N, K, code):
    d = _lib.WeightDesc()
    assert L.w4a16_weight_desc_init(E, N, K, ctypes.byref(d)) == code
    assert L.w4a16_last_error()


def test_gate_up_descriptor(L):
    d = W.weight_desc(4, 64, 256, gate_up=True)
    assert d.flags == _lib.DESC_GATE_UP and d.w_bytes == W.weight_desc(4, 64, 256).w_bytes
    e = _lib.WeightDesc()
    assert L.w4a16_weight_desc_init_gate_up(4, 48, 256, ctypes.byref(e)) == -2       # N % 32
    d.flags = 2                                                                      # unknown flag
    assert L.w4a16_pack_w4(16, 16, ctypes.byref(d), 16, 16, None) == -3


def test_corrupted_descriptor_is_rejected(L):
    d = W.weight_desc(4, 64, 256)
    d.N = 128                                           # shape changed after packing
    st = L.w4a16_grouped_contiguous(ctypes.byref(d), 16, 16, 16, 128, 16, 16, None, None, 0, None)
    assert st == -3 and b"checksum" in L.w4a16_last_error()
    d = W.weight_desc(4, 64, 256)
    d.magic = 0
    assert L.w4a16_pack_w4(16, 16, ctypes.byref(d), 16, 16, None) == -3


def _routing(T, topk, E_loc, block_m, E_glob=384, P=16, capacity=None):
    cap = W.align_capacity(T, topk, E_loc, block_m) if capacity is None else capacity
    return _lib.IndexedRouting(P, P, P, cap, block_m, T, topk, P, 0, E_loc, E_glob)


def _ws(desc, r, combine, cfg=None):
    return L_().w4a16_moe_gemm_workspace_bytes(ctypes.byref(desc), ctypes.byref(r), int(combine),
                                               None if cfg is None else ctypes.byref(cfg))


def L_():
    return W.load()


def test_capacity_and_workspace(L):
    assert W.align_capacity(576, 8, 48, 32) == ((4608 + 48 * 31 + 31) // 32) * 32
    assert L.w4a16_align_capacity(4, 2, 3, 24) == -1
    d = W.weight_desc(4, 7168, 2048)
    r = _routing(10, 8, 4, 32)
    one_wg_per_tile = W.config(32, 2, split_k=1)
    tok = 256                                          # local-slot counts of the 10 tokens, one 256-byte region
    assert _ws(d, r, True, one_wg_per_tile) == 10 * 8 * 7168 * 4 + tok
    assert _ws(d, r, False, one_wg_per_tile) == 0
    assert _ws(d, r, True, W.config(32, 3)) == 0                     # unsupported config
    assert _ws(d, r, True, W.config(32, 2, stages=4)) == 10 * 8 * 7168 * 4 + tok
    assert _ws(d, r, True, W.config(64, 4, stages=4)) == 0           # not built
    assert _ws(d, r, True, W.config(32, 2, stages=3)) == 0           # odd depth: not built
    assert _ws(d, r, True, W.config(32, 2, kind="masked")) == 0      # config of another routing kind
    # split K: arrival counters + slices for every tile that can exist (routed
    # blocks bounded by min(capacity / block_m, T*topk / block_m + E_loc)),
    # then the combine's partials
    blocks = min(r.capacity // 32, -(-80 // 32) + 4)
    tiles = blocks * (7168 // 16 // 8)
    al = lambda v: -(-v // 256) * 256
    slices = tiles * 4 * (2 * 2 * 256 * 16)
    assert _ws(d, r, True, W.config(32, 2, split_k=4)) == al(tiles * 4) + al(slices) + 10 * 8 * 7168 * 4 + tok
    assert _ws(d, r, True, W.config(32, 2, split_k=32)) == 0         # not a split count
    # cfg NULL: the selector's config for the routing's block_m
    c = _lib.Config()
    assert L.w4a16_indexed_config(10, 8, 384, 4, 7168, 2048, 32, ctypes.byref(c)) == 0
    assert (c.block_m, c.nr, c.waves, c.stages, c.kind) == (32, 2, 4, 2, 0)
    assert _ws(d, r, True) == _ws(d, r, True, c)
    assert c.combine_cols == 0


def test_wide_tile_selection(L):
    """From 128 routed rows per expert (K a multiple of 128) the selector
    aligns the routing to 256 rows: both projections run the 256-row tile
    (nr 2, eight waves, unsplit), the down projection with the combine on a
    workspace sized for that tile."""
    ep8 = W.select(8192, 8, 384, 48, 4096, 7168)
    assert (ep8.block_m, ep8.nr, ep8.waves, ep8.split_k) == (256, 2, 8, 1)
    assert W.select(4096, 8, 384, 384, 512, 7168).block_m == 128        # 85 rows per expert
    # the padded-rows fit: 127.1 rows fit one 128-row block, 130 need 144 rows -> the 256-row tile;
    # 300 rows fit two blocks of 160 (-> 256), as do 512 (two of 256)
    assert W.select(6100, 8, 384, 48, 4096, 7168).block_m == 128
    assert W.select(6240, 8, 384, 48, 4096, 7168).block_m == 256
    assert W.select(14400, 8, 384, 48, 4096, 7168).block_m == 256
    assert W.select(24576, 8, 384, 48, 4096, 7168).block_m == 256
    assert W.select(8192, 8, 384, 48, 4096, 7000).block_m == 128        # K not a multiple of 128
    assert W.mxfp4_select(8192, 8, 384, 48, 4096, 7168).block_m == 64   # the A4W4 rule is unchanged
    c = _lib.Config()
    assert L.w4a16_indexed_config(8192, 8, 384, 48, 4096, 7168, 256, ctypes.byref(c)) == 0
    assert (c.block_m, c.nr, c.waves, c.split_k) == (256, 2, 8, 1)
    assert L.w4a16_indexed_config(8192, 8, 384, 48, 7168, 2048, 256, ctypes.byref(c)) == 0
    assert (c.block_m, c.nr, c.waves, c.split_k) == (256, 2, 8, 1)
    assert L.w4a16_indexed_config(8192, 8, 384, 48, 7168, 2000, 256, ctypes.byref(c)) == 0
    assert c.block_m == 128                                             # K not a multiple of 128
    d = W.weight_desc(48, 7168, 2048)
    r = _routing(8192, 8, 48, 256)
    assert _ws(d, r, True) == _ws(d, r, True, W.config(256, 2, 8))
    assert _ws(d, r, False) == 0


def test_combine_passes_size_the_workspace(L):
    """The combine's workspace holds one pass of fp32 per-slot partials:
    T * topk * cols * 4 bytes, cols = the config's combine_cols or the
    library's choice (all of N while the expected local partials fit 128 MB,
    else the fewest passes that do, in whole workgroup tiles)."""
    d = W.weight_desc(4, 7168, 2048)
    r = _routing(10, 8, 4, 32)
    tok = 256                                          # local-slot counts per token, rounded to 256 bytes
    assert _ws(d, r, True, W.config(32, 2, combine_cols=1024)) == 10 * 8 * 1024 * 4 + tok
    assert _ws(d, r, True, W.config(32, 2, combine_cols=16)) == -(-(10 * 8 * 16 * 4) // 256) * 256 + tok
    assert _ws(d, r, True, W.config(32, 2, combine_cols=8192)) == 10 * 8 * 7168 * 4 + tok   # capped at N
    assert _ws(d, r, True, W.config(32, 2, combine_cols=24)) == 0       # not a multiple of 16
    assert _ws(d, r, True, W.config(32, 2, combine_cols=-16)) == 0
    assert _ws(d, r, False, W.config(32, 2, combine_cols=1024)) == 0    # no combine, no partials
    # TP8-like down projection, every expert local: T = 4096, top-8, N = 7168
    # -> 940 MB of partials in one pass; the library's choice is 4 passes of
    # 1792 columns (7 workgroup tiles of 256)
    d2 = W.weight_desc(384, 7168, 256)
    r2 = _lib.IndexedRouting(None, None, None, 40960, 128, 4096, 8, None, 0, 384, 384)
    assert _ws(d2, r2, True, W.config(128, 4)) == 4096 * 8 * 1792 * 4 + 4096
    # T = 1024: 235 MB fits one pass
    r4 = _lib.IndexedRouting(None, None, None, 10240, 32, 1024, 8, None, 0, 384, 384)
    assert _ws(d2, r4, True, W.config(32, 2)) == 1024 * 8 * 7168 * 4 + 1024
    # an EP8 share (1 in 8 slots local) of T = 576 stays one pass
    d3 = W.weight_desc(48, 7168, 2048)
    r3 = _lib.IndexedRouting(None, None, None, 6144, 32, 576, 8, None, 0, 48, 384)
    assert _ws(d3, r3, True, W.config(32, 2)) == 576 * 8 * 7168 * 4 + 768


def test_align_argument_errors(L):
    P = 16  # fake, aligned, never dereferenced: every case fails validation first
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 16, None, P, P, 1024, 0, None) == -1
    assert L.w4a16_moe_align(P, 4, 2, 8, 4, 8, 16, P, P, P, 1024, 0, None) == -1     # range past E_glob
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 24, P, P, P, 1024, 0, None) == -2     # block_m
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 16, P, P, P, 64, 0, None) == -5       # capacity
    assert L.w4a16_moe_align(P, 4, 2, 2000, 0, 1500, 16, P, P, P, 1 << 20, 0, None) == -2


def test_gemm_argument_errors(L, monkeypatch):
    P = 16
    d = W.weight_desc(8, 64, 256)
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8, 64)
    cfg = W.config(32, 2)
    call = lambda **kw: L.w4a16_moe_gemm(ctypes.byref(kw.get("d", d)), P, P, kw.get("a", P), kw.get("rows", 64),
                                         kw.get("layout", 0), ctypes.byref(kw.get("r", r)), kw.get("w"), P,
                                         kw.get("cfg", ctypes.byref(cfg)), kw.get("ws"),
                                         kw.get("wsb", 0), None)
    assert call(a=P + 2) == -1                                           # misaligned activations
    assert call(rows=10) == -2                                           # too few activation rows
    assert call(cfg=ctypes.byref(W.config(64, 2))) == -3                 # block_m does not divide the routing's
    assert call(cfg=ctypes.byref(W.config(32, 3))) == -4                 # tile config not built
    assert call(w=P) == -8                                               # combine without workspace
    assert call(cfg=ctypes.byref(W.config(32, 2, split_k=3))) == -4     # not a split count
    # slices are whole pairs of 128-K chunks: K = 256 has one pair, K = 512 two
    assert call(cfg=ctypes.byref(W.config(32, 2, split_k=2))) == -4     # more slices than the 1 chunk pair
    d4 = W.weight_desc(8, 64, 512)
    assert call(d=d4, cfg=ctypes.byref(W.config(32, 2, split_k=4))) == -4   # more slices than the 2 pairs
    assert call(d=d4, cfg=ctypes.byref(W.config(32, 2, split_k=2))) == -8   # split needs workspace
    assert call(cfg=ctypes.byref(W.config(32, 2, kind="contiguous"))) == -1   # config of another kind
    assert call(cfg=ctypes.byref(W.config(32, 2, combine_cols=40)), w=P) == -1  # pass width not a multiple of 16
    # nr 1 (waves splitting K): block_m 16, eight waves, split_k 1, K a multiple of 128
    assert call(cfg=ctypes.byref(W.config(16, 1, 8, split_k=2))) == -4
    assert call(cfg=ctypes.byref(W.config(16, 1, 4))) == -4
    assert call(cfg=ctypes.byref(W.config(32, 1, 8))) == -4
    assert call(d=W.weight_desc(8, 64, 224), cfg=ctypes.byref(W.config(16, 1, 8))) == -4
    bad = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 4, 64)
    assert call(r=bad) == -3                                             # E_loc != weight experts
    no_eg = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8, 0)
    assert call(r=no_eg, cfg=None) == -1                                 # NULL cfg needs E_glob to select
    gated = W.weight_desc(8, 64, 256, gate_up=True)
    assert call(d=gated, w=P) == -3                                      # combine on a gate/up weight
    # activations are addressed with 32-bit byte offsets: no call may read past 4 GiB
    big = W.weight_desc(8, 64, 7168)
    rb = _lib.IndexedRouting(P, P, P, 320128, 32, 40000, 8, P, 0, 8, 64)
    assert call(d=big, r=rb, rows=320000, layout=_lib.A_SLOT) == -2      # 320000 x 7168 x 2 B > 4 GiB
    gm = lambda max_m, em, cfg=None, d_=d: L.w4a16_grouped_masked(ctypes.byref(d_), P, P, P, max_m, P, em, P,
                                                                 cfg, None, 0, None)
    assert gm(0, 4) == -1
    assert gm(32, 0) == -1
    assert gm(32, 4, ctypes.byref(W.config(32, 2))) == -1                # indexed config on a grouped call
    assert gm(37500, 4, None, W.weight_desc(8, 64, 7168)) == -2          # 8 x 37500 rows x 14 KB > 4 GiB
    gc = lambda rows, cfg=None, d_=d: L.w4a16_grouped_contiguous(ctypes.byref(d_), P, P, P, rows, P, P, cfg,
                                                                None, 0, None)
    assert gc(100) == -2
    assert gc(128, ctypes.byref(W.config(64, 2))) == -1                  # indexed config on a grouped call
    assert gc(256, ctypes.byref(W.config(256, 2, 8, kind="contiguous"))) == -4   # 256-row blocks straddle 128-row segments
    assert gc(300032, None, W.weight_desc(8, 64, 7168)) == -2            # 300032 x 7168 x 2 B > 4 GiB
    # tuning overrides belong to indexed routing: grouped calls and grouped selection refuse them
    monkeypatch.setenv("W4A16_BLOCK_M", "64")
    assert gc(128) == -1 and b"W4A16_BLOCK_M" in L.w4a16_last_error()
    with pytest.raises(W.W4A16Error):
        W.select(512, 1, 1, 8, 64, 256, kind="masked", expected_m=30)
    assert W.select(576, 8, 384, 48, 4096, 7168).block_m == 64          # indexed selection takes the override
    monkeypatch.delenv("W4A16_BLOCK_M")
    lay = lambda layout, rows: L.w4a16_moe_gemm(ctypes.byref(d), P, P, P, rows, layout, ctypes.byref(r), None, P,
                                                ctypes.byref(cfg), None, 0, None)
    assert lay(3, 4096) == -1                                            # unknown activation layout
    assert lay(_lib.A_SLOT, 64) == -2                                    # slot rows: needs T * topk = 128
    assert lay(_lib.A_SORTED, 128) == -2                                 # sorted rows: needs capacity = 1024


def test_gate_up_silu_argument_errors(L):
    P = 16
    plain = W.weight_desc(8, 64, 256)
    gated = W.weight_desc(8, 64, 256, gate_up=True)
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8, 64)
    call = lambda d, cfg: L.w4a16_moe_gate_up_silu(ctypes.byref(d), P, P, P, 64, ctypes.byref(r), P,
                                                   ctypes.byref(cfg), None)
    assert call(plain, W.config(32, 2)) == -3                            # weight not gate/up packed
    assert call(gated, W.config(32, 2, split_k=0)) == -4                 # one workgroup per tile only
    assert call(gated, W.config(32, 2, split_k=2)) == -4
    assert call(gated, W.config(32, 3)) == -4                            # odd nr other than 1
    assert call(gated, W.config(64, 2)) == -3                            # block_m does not divide the routing's
    assert call(gated, W.config(32, 2, kind="masked")) == -1             # config of another kind


def test_mxfp4_selector_halves_large_prefill_blocks(L):
    """A4W4 takes 64-row blocks where the W4A16 rule gives 128 or 256 at >= 128
    rows per expert, keeps 128 below that, follows the W4A16 block_m elsewhere,
    and uses one workgroup per tile with four weight tiles per wave, or its
    K-split tile where the W4A16 rule takes one."""
    pre = W.mxfp4_select(8192, 8, 384, 48, 4096, 7168)          # ~171 rows/expert
    assert W.select(8192, 8, 384, 48, 4096, 7168).block_m == 256
    assert (pre.block_m, pre.nr, pre.waves, pre.split_k, pre.stages) == (64, 4, 4, 1, 2)
    tp = W.mxfp4_select(4096, 8, 384, 384, 512, 7168)           # ~85 rows/expert
    assert W.select(4096, 8, 384, 384, 512, 7168).block_m == 128 and tp.block_m == 128
    for args in ((576, 8, 384, 48, 4096, 7168), (16, 8, 384, 384, 512, 7168), (1024, 8, 384, 384, 512, 7168)):
        c, w = W.mxfp4_select(*args), W.select(*args)
        assert c.block_m == w.block_m and c.split_k == 1 and c.nr == 4
        assert c.stages == (4 if c.block_m <= 32 else 2)
    # where the W4A16 rule takes the tile whose waves split K (TP8 T = 1
    # gate/up), A4W4 takes its own K-split tile; the short-K down keeps nr 4
    t1, w1 = W.mxfp4_select(1, 8, 384, 384, 512, 7168), W.select(1, 8, 384, 384, 512, 7168)
    assert w1.nr == 1 and (t1.block_m, t1.nr, t1.waves, t1.split_k) == (16, 1, 8, 1)
    d1 = W.mxfp4_select(1, 8, 384, 384, 7168, 256)
    assert (d1.block_m, d1.nr, d1.waves) == (16, 4, 4)
    with pytest.raises(W.W4A16Error):
        W.mxfp4_select(16, 0, 384, 48, 4096, 7168)


def test_selector_follows_tokens_per_expert(L):
    dec = W.select(576, 8, 384, 48, 4096, 7168)            # ~12 rows/expert
    assert dec.block_m == 32 and dec.nr == 2 and dec.kind == 0
    one = W.select(16, 8, 384, 384, 512, 7168)             # ~0.3 rows/expert
    assert one.block_m == 16
    pre = W.select(8192, 8, 384, 48, 4096, 7168)           # ~171 rows/expert
    assert pre.block_m == 256 and pre.nr == 2 and pre.waves == 8   # the 256-row tile (K % 128 == 0)
    mid = W.select(4096, 8, 384, 48, 4096, 7168)           # ~85 rows/expert
    assert mid.block_m == 128 and mid.nr == 4                  # the 128-row prefill tile
    ragged = W.select(8192, 8, 384, 48, 4096, 7200)           # ragged K: the general kernel
    assert ragged.block_m == 128 and ragged.nr == 2
    # tok_e, not total tokens: same T, 8x more experts -> decode side
    assert W.select(8192, 8, 3072, 48, 4096, 7168).block_m < 128
    assert W.select(576, 8, 384, 48, 4096, 7168).block_m == dec.block_m   # memoised, stable


def test_selector_splits_k_only_for_underfilled_grids(L):
    """split_k doubles while the doubled grid (sampled routed blocks x N tiles x
    split_k x 2) stays within 4/5 of one round of resident workgroups (256 CUs
    x 4 for 16/32-row blocks) and each slice keeps >= 4 chunks of 128 K."""
    assert W.select(576, 8, 384, 48, 4096, 7168).split_k == 1     # EP8 decode: 48 x 32 tiles fill the machine
    assert W.select(576, 8, 384, 24, 4096, 7168).split_k == 1     # EP16 decode: 768 tiles
    assert W.select(576, 8, 384, 12, 4096, 7168).split_k == 2     # EP32 decode: 384 tiles
    assert W.select(16, 8, 384, 384, 512, 7168).split_k == 2      # TP8 T=16: ~400 sampled tiles
    t1 = W.select(1, 8, 384, 384, 512, 7168)                      # TP8 T=1: 8 blocks x 4 tiles
    # it would split 8 ways (56 chunks: 7 per slice); the waves split K instead
    assert (t1.block_m, t1.nr, t1.waves, t1.split_k) == (16, 1, 8, 1)
    assert W.select(1, 8, 384, 384, 512, 7000).split_k == 8       # K not a multiple of 128: K slices
    assert W.select(1, 8, 384, 384, 7168, 256).split_k == 1       # its down projection: K = 256, 2 chunks
    # 16-row blocks over K = 256 take four weight tiles per wave while the grid keeps 2 per CU
    assert W.select(1, 8, 384, 384, 7168, 256).nr == 2            # 9 blocks x 28 tiles: too few
    assert W.select(16, 8, 384, 384, 7168, 256).nr == 4
    assert W.select(128, 8, 384, 384, 7168, 256).nr == 4
    assert W.select(1024, 8, 384, 384, 7168, 256).nr == 2         # 32-row blocks
    assert W.select(4096, 8, 384, 384, 512, 7168).split_k == 1    # prefill-side grids fill the machine
    assert W.select(8192, 8, 384, 48, 4096, 7168).split_k == 1


def test_grouped_selection_follows_the_grouped_rules(L):
    """Masked: deep K covers ~1.3 x expected_m rows, short K ceil(1.25 x
    expected_m, 8), rounded up to a built block; contiguous: 128-row blocks
    when their grid fills the machine, 64 for small problems."""
    m = lambda em, K, N=4096: W.select(512, 1, 1, 48, N, K, kind="masked", expected_m=em)
    assert m(12, 7168).block_m == 16 and m(13, 7168).block_m == 32      # 1.3 x 12 = 15.6; 1.3 x 13 = 16.9
    assert m(24, 7168).block_m == 32 and m(25, 7168).block_m == 64      # 31.2 -> 32; 32.5 -> 64
    assert m(25, 2048).block_m == 32                                     # ceil(31.25, 8) = 32
    assert m(315, 7168).block_m == 128
    assert m(12, 7168).stages == 4 and m(315, 7168).stages == 2          # ~512 buffered K for decode tiles
    assert m(12, 7168).kind == 2
    c = lambda rows, E=48: W.select(rows, 1, 1, E, 4096, 7168, kind="contiguous")
    assert c(17024).block_m == 128 and c(17024).kind == 1                # 133 blocks x 32 N tiles
    assert c(1024, 8).block_m == 64                                      # 8 x 32 tiles < one round: BM64
    with pytest.raises(W.W4A16Error):
        W.select(512, 1, 1, 48, 4096, 7168, kind="masked", expected_m=0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib._build, "lib_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(_lib.W4A16Error):
        _lib.load()


def test_mxfp4_descriptor_and_errors(L):
    d = W.mxfp4_weight_desc(48, 4096, 7168)
    assert d.flags == _lib.DESC_MXFP4 and d.chunks == 56
    assert d.w_bytes == 48 * 4096 * 7168 // 2 and d.s_bytes == 48 * 4096 * 7168 // 32
    e = _lib.WeightDesc()
    assert L.w4a16_mxfp4_weight_desc_init(2, 32, 96, ctypes.byref(e)) == -2           # K % 128
    P = 16
    plain = W.weight_desc(8, 64, 256)
    mx = W.mxfp4_weight_desc(8, 64, 256)
    # each family's calls reject the other family's weights
    assert L.w4a16_mxfp4_pack(P, P, ctypes.byref(plain), P, P, None) == -3
    assert L.w4a16_pack_w4(P, P, ctypes.byref(mx), P, P, None) == -3
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8)
    cfg = W.mxfp4_config(32, 4)
    call = lambda d=mx, layout=_lib.A_TOKEN, rows=64, c=cfg, w=None, ws=None, wsb=0: L.w4a16_mxfp4_moe_gemm(
        ctypes.byref(d), P, P, P, P, rows, layout, ctypes.byref(r), w, P, ctypes.byref(c), ws, wsb, None)
    assert call(d=plain) == -3                                           # not an MXFP4 weight
    assert L.w4a16_moe_gemm(ctypes.byref(mx), P, P, P, 64, 0, ctypes.byref(r), None, P,
                            ctypes.byref(W.config(32, 2)), None, 0, None) == -3
    assert call(layout=3) == -1                                          # unknown activation layout
    assert call(layout=_lib.A_SORTED) == -2                              # sorted rows: needs capacity = 1024
    assert call(rows=10) == -2                                           # too few rows
    assert call(c=W.mxfp4_config(32, 3)) == -4                           # not built
    assert call(c=W.config(32, 4, split_k=0, stages=4)) == -4            # one workgroup per tile
    assert call(c=W.mxfp4_config(64, 4)) == -3                           # block_m does not divide the routing's
    assert call(w=P) == -8                                               # combine without workspace
    assert L.w4a16_mxfp4_moe_gemm_workspace_bytes(ctypes.byref(mx), 10, 8, 1) == 10 * 8 * 64 * 4
    assert L.w4a16_mxfp4_quant(P, 4, 48, P, P, None) == -2               # K % 32
    assert L.w4a16_mxfp4_quant(P + 4, 4, 64, P, P, None) == -1           # misaligned rows
    q = L.w4a16_mxfp4_quant_local_slots
    assert q(P, None, 4, 8, 0, 48, 64, P, P, None) == -1                 # topk_ids NULL
    assert q(P, P, 4, 8, 0, 48, 48, P, P, None) == -2                    # K % 32
    assert q(P, P, 4, 0, 0, 48, 64, P, P, None) == -1                    # topk 0
    assert q(P, P, 4, 8, 0, 0, 64, P, P, None) == -1                     # no local experts
    assert q(None, None, 0, 8, 0, 48, 64, None, None, None) == 0         # no tokens: nothing to do


def test_mxfp4_gate_up_silu_errors(L):
    P = 16
    plain = W.mxfp4_weight_desc(8, 128, 256)
    gated = W.mxfp4_weight_desc(8, 128, 256, gate_up=True)
    assert gated.flags == _lib.DESC_MXFP4 | _lib.DESC_GATE_UP
    e = _lib.WeightDesc()
    assert L.w4a16_mxfp4_weight_desc_init_gate_up(8, 96, 256, ctypes.byref(e)) == -2   # N % 64
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8)
    call = lambda d, cfg: L.w4a16_mxfp4_gate_up_silu(ctypes.byref(d), P, P, P, P, 64, ctypes.byref(r), P, P,
                                                     ctypes.byref(cfg), None)
    assert call(plain, W.mxfp4_config(32, 4)) == -3                      # not a gate/up MXFP4 weight
    assert call(W.weight_desc(8, 128, 256, gate_up=True), W.mxfp4_config(32, 4)) == -3   # INT4 weight
    assert call(gated, W.mxfp4_config(32, 2)) == -4                      # nr must be 4 or 1
    assert call(gated, W.mxfp4_config(32, 1)) == -4                      # nr 1 only on block_m 16
    assert call(gated, W.mxfp4_config(64, 4)) == -3                      # block_m does not divide the routing's
    # the INT4 calls reject the combined flags too
    assert L.w4a16_pack_w4(P, P, ctypes.byref(gated), P, P, None) == -3
