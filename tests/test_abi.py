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
    assert ctypes.sizeof(_lib.Config) == 20
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
                  "W4A16_A_SORTED"):
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
    assert got[("const", "W4A16_ABI_VERSION")] == 4


def test_version_and_desc(L):
    assert L.w4a16_abi_version() == 4
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
    st = L.w4a16_grouped_contiguous(ctypes.byref(d), 16, 16, 16, 128, 16, 16, None, None)
    assert st == -3 and b"checksum" in L.w4a16_last_error()
    d = W.weight_desc(4, 64, 256)
    d.magic = 0
    assert L.w4a16_pack_w4(16, 16, ctypes.byref(d), 16, 16, None) == -3


def test_capacity_and_workspace(L):
    assert W.align_capacity(576, 8, 48, 32) == ((4608 + 48 * 31 + 31) // 32) * 32
    assert L.w4a16_align_capacity(4, 2, 3, 24) == -1
    p = W.PackedW4(W.weight_desc(4, 7168, 2048), None, None)
    one_wg_per_tile = W.config(32, 2, split_k=1)
    assert W.workspace_bytes(p, 10, 8, True, one_wg_per_tile) == 10 * 8 * 7168 * 4
    assert W.workspace_bytes(p, 10, 8, False, one_wg_per_tile) == 0
    assert W.workspace_bytes(p, 10, 8, True, W.config(32, 3)) == 0          # unsupported config
    d = W.indexed_config(64)
    assert (d.block_m, d.nr, d.waves, d.split_k, d.stages) == (64, 2, 4, 1, 2)
    assert W.workspace_bytes(p, 10, 8, True, W.config(32, 2, stages=4)) == 10 * 8 * 7168 * 4
    assert W.workspace_bytes(p, 10, 8, True, W.config(64, 4, stages=4)) == 0   # not built
    assert W.workspace_bytes(p, 10, 8, True, W.config(32, 2, stages=3)) == 0   # odd depth: not built


def test_align_argument_errors(L):
    P = 16  # fake, aligned, never dereferenced: every case fails validation first
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 16, None, P, P, 1024, 0, None) == -1
    assert L.w4a16_moe_align(P, 4, 2, 8, 4, 8, 16, P, P, P, 1024, 0, None) == -1     # range past E_glob
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 24, P, P, P, 1024, 0, None) == -2     # block_m
    assert L.w4a16_moe_align(P, 4, 2, 8, 0, 8, 16, P, P, P, 64, 0, None) == -5       # capacity
    assert L.w4a16_moe_align(P, 4, 2, 2000, 0, 1500, 16, P, P, P, 1 << 20, 0, None) == -2


def test_gemm_argument_errors(L):
    P = 16
    d = W.weight_desc(8, 64, 256)
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8)
    cfg = W.config(32, 2)
    call = lambda **kw: L.w4a16_moe_gemm(ctypes.byref(d), P, P, kw.get("a", P), kw.get("rows", 64), 0,
                                         ctypes.byref(kw.get("r", r)), kw.get("w"), P,
                                         kw.get("cfg", ctypes.byref(cfg)), kw.get("ws"),
                                         kw.get("wsb", 0), None)
    assert call(a=P + 2) == -1                                           # misaligned activations
    assert call(rows=10) == -2                                           # too few activation rows
    assert call(cfg=ctypes.byref(W.config(64, 2))) == -3                 # block_m disagrees with routing
    assert call(cfg=ctypes.byref(W.config(32, 3))) == -4                 # tile config not built
    assert call(w=P) == -8                                               # combine without workspace
    assert call(cfg=ctypes.byref(W.config(32, 2, split_k=2))) == -4      # split_k must be 0 or 1
    bad = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 4)
    assert call(r=bad) == -3                                             # E_loc != weight experts
    assert L.w4a16_grouped_masked(ctypes.byref(d), P, P, P, 0, P, 4, P, None, None) == -1
    assert L.w4a16_grouped_masked(ctypes.byref(d), P, P, P, 32, P, 0, P, None, None) == -1
    assert L.w4a16_grouped_contiguous(ctypes.byref(d), P, P, P, 100, P, P, None, None) == -2
    lay = lambda layout, rows: L.w4a16_moe_gemm(ctypes.byref(d), P, P, P, rows, layout, ctypes.byref(r), None, P,
                                                ctypes.byref(cfg), None, 0, None)
    assert lay(3, 4096) == -1                                            # unknown activation layout
    assert lay(_lib.A_SLOT, 64) == -2                                    # slot rows: needs T * topk = 128
    assert lay(_lib.A_SORTED, 128) == -2                                 # sorted rows: needs capacity = 1024


def test_gate_up_silu_argument_errors(L):
    P = 16
    plain = W.weight_desc(8, 64, 256)
    gated = W.weight_desc(8, 64, 256, gate_up=True)
    r = _lib.IndexedRouting(P, P, P, 1024, 32, 64, 2, P, 0, 8)
    call = lambda d, cfg: L.w4a16_moe_gate_up_silu(ctypes.byref(d), P, P, P, 64, ctypes.byref(r), P,
                                                   ctypes.byref(cfg), None)
    assert call(plain, W.config(32, 2)) == -3                            # weight not gate/up packed
    assert call(gated, W.config(32, 2, split_k=0)) == -4                 # one workgroup per tile only
    assert call(gated, W.config(16, 2)) == -3                            # block_m disagrees with routing


def test_mxfp4_selector_halves_large_prefill_blocks(L):
    """A4W4 takes 64-row blocks where the W4A16 rule gives 128 at >= 128 rows
    per expert, keeps 128 below that, follows the W4A16 block_m elsewhere,
    and always uses one workgroup per tile with four weight tiles per wave."""
    pre = W.mxfp4_select(8192, 8, 384, 48, 4096, 7168)          # ~171 rows/expert
    assert W.select(8192, 8, 384, 48, 4096, 7168).block_m == 128
    assert (pre.block_m, pre.nr, pre.waves, pre.split_k, pre.stages) == (64, 4, 4, 1, 2)
    tp = W.mxfp4_select(4096, 8, 384, 384, 512, 7168)           # ~85 rows/expert
    assert W.select(4096, 8, 384, 384, 512, 7168).block_m == 128 and tp.block_m == 128
    for args in ((576, 8, 384, 48, 4096, 7168), (16, 8, 384, 384, 512, 7168), (1024, 8, 384, 384, 512, 7168)):
        c, w = W.mxfp4_select(*args), W.select(*args)
        assert c.block_m == w.block_m and c.split_k == 1 and c.nr == 4
        assert c.stages == (4 if c.block_m <= 32 else 2)
    with pytest.raises(W.W4A16Error):
        W.mxfp4_select(16, 0, 384, 48, 4096, 7168)


def test_selector_follows_tokens_per_expert(L):
    dec = W.select(576, 8, 384, 48, 4096, 7168)            # ~12 rows/expert
    assert dec.block_m == 32 and dec.nr == 2
    one = W.select(16, 8, 384, 384, 512, 7168)             # ~0.3 rows/expert
    assert one.block_m == 16
    assert dec.split_k == 1 and one.split_k == 1            # stream-K only when asked for
    pre = W.select(8192, 8, 384, 48, 4096, 7168)           # ~171 rows/expert
    assert pre.block_m == 128 and pre.nr == 2
    # tok_e, not total tokens: same T, 8x more experts -> decode side
    assert W.select(8192, 8, 3072, 48, 4096, 7168).block_m < 128
    assert W.select(576, 8, 384, 48, 4096, 7168).block_m == dec.block_m   # memoised, stable


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
    assert call(c=W.mxfp4_config(64, 4)) == -3                           # block_m disagrees with routing
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
    assert call(gated, W.mxfp4_config(32, 2)) == -4                      # nr must be 4
    assert call(gated, W.mxfp4_config(64, 4)) == -3                      # block_m disagrees with routing
    # the INT4 calls reject the combined flags too
    assert L.w4a16_pack_w4(P, P, ctypes.byref(gated), P, P, None) == -3
