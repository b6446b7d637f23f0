"""Python binding of the W4A16 MoE C ABI: torch tensors in, device pointers and
torch's current HIP stream out.  Argument marshalling only -- every step of
the computation runs in the HIP library's kernels.

    packed = pack_w4(codes_u8[E, N, K], scales_bf16[E, N, K/32])
    routing = moe_align(topk_ids[T, k], E_glob, first_expert, E_loc, block_m)
    h = moe_w4a16_gemm(x[T, K], packed, routing)                     # per slot
    y = moe_w4a16_gemm(a[T*k, K2], packed2, routing, topk_weights)   # combined
    # chained layer: fused SiLU gate/up in sorted order, down reads it as is
    p1 = pack_w4(codes1, scales1, gate_up=True)
    inter = moe_gate_up_silu(x, p1, routing)                         # [capacity, N/2]
    y = moe_w4a16_gemm(inter, packed2, routing, topk_weights, a_layout="sorted")
    out = grouped_contiguous(a2[m, K], packed, m_indices)
    out = grouped_masked(a3[E, max_m, K], packed, masked_m, expected_m)
    # A4W4: MXFP4 weights, activations quantised to MXFP4 on the device
    pm = pack_mxfp4(codes_u8[E, N, K/2], scales_e8m0[E, N, K/32])
    q = mxfp4_quant(x[T, K])                                         # MXFP4 rows
    h = moe_mxfp4_gemm(q, pm, routing)                               # per slot
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from ._lib import (A_SLOT, A_SORTED, A_TOKEN, DESC_GATE_UP, DESC_MXFP4, ROUTE_CONTIGUOUS, ROUTE_INDEXED,
                   ROUTE_MASKED, Config, IndexedRouting, W4A16Error, WeightDesc, check, load)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16)


@dataclasses.dataclass
class PackedW4:
    desc: WeightDesc
    w: torch.Tensor      # uint8 [w_bytes]
    s: torch.Tensor      # uint8 [s_bytes]

    @property
    def E(self):
        return self.desc.E

    @property
    def N(self):
        return self.desc.N

    @property
    def K(self):
        return self.desc.K

    @property
    def gate_up(self):
        return self.desc.flags == DESC_GATE_UP


def weight_desc(E: int, N: int, K: int, gate_up: bool = False) -> WeightDesc:
    d = WeightDesc()
    init = load().w4a16_weight_desc_init_gate_up if gate_up else load().w4a16_weight_desc_init
    check(init(E, N, K, ctypes.byref(d)))
    return d


def pack_w4(codes: torch.Tensor, scales: torch.Tensor, gate_up: bool = False) -> PackedW4:
    """codes uint8 [E, N, K] (0..15), scales bf16 [E, N, K/32] -> packed weight.
    gate_up: rows [0, N/2) are the gate and [N/2, N) the up projection; their
    tiles are interleaved (needed by moe_gate_up_silu; every call still sees
    the logical column order)."""
    _need(codes, "codes", (torch.uint8,), 3)
    _need(scales, "scales", _BF16, 3)
    E, N, K = codes.shape
    if tuple(scales.shape) != (E, N, K // 32) or K % 32:
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
    d = weight_desc(E, N, K, gate_up)
    w = torch.empty(d.w_bytes, dtype=torch.uint8, device=codes.device)
    s = torch.empty(d.s_bytes, dtype=torch.uint8, device=codes.device)
    check(load().w4a16_pack_w4(codes.data_ptr(), scales.data_ptr(), ctypes.byref(d), w.data_ptr(),
                               s.data_ptr(), _stream(codes.device)))
    return PackedW4(d, w, s)


@dataclasses.dataclass
class Routing:
    sorted_ids: torch.Tensor          # int32 [capacity]
    expert_ids: torch.Tensor          # int32 [capacity / block_m]
    num_tokens_padded: torch.Tensor   # int32 [1]
    block_m: int
    topk_ids: torch.Tensor            # int32 [T, k]
    E_glob: int
    first_expert: int
    E_loc: int

    @property
    def T(self):
        return self.topk_ids.shape[0]

    @property
    def topk(self):
        return self.topk_ids.shape[1]

    @property
    def capacity(self):
        return self.sorted_ids.numel()

    def as_c(self) -> IndexedRouting:
        return IndexedRouting(self.sorted_ids.data_ptr(), self.expert_ids.data_ptr(),
                              self.num_tokens_padded.data_ptr(), self.capacity, self.block_m,
                              self.T, self.topk, self.topk_ids.data_ptr(), self.first_expert,
                              self.E_loc, self.E_glob)


def align_capacity(T: int, topk: int, E_loc: int, block_m: int) -> int:
    c = load().w4a16_align_capacity(T, topk, E_loc, block_m)
    if c < 0:
        raise ValueError("bad arguments for align_capacity")
    return int(c)


def moe_align(topk_ids: torch.Tensor, E_glob: int, first_expert: int, E_loc: int, block_m: int,
              validate: bool = False, capacity: Optional[int] = None) -> Routing:
    """topk_ids int32 [T, k] -> sorted_ids / expert_ids / num_tokens_padded."""
    _need(topk_ids, "topk_ids", (torch.int32,), 2)
    T, k = topk_ids.shape
    cap = align_capacity(T, k, E_loc, block_m) if capacity is None else int(capacity)
    dev = topk_ids.device
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    ntp = torch.empty(1, dtype=torch.int32, device=dev)
    check(load().w4a16_moe_align(topk_ids.data_ptr(), T, k, E_glob, first_expert, E_loc, block_m,
                                 sorted_ids.data_ptr(), expert_ids.data_ptr(), ntp.data_ptr(), cap,
                                 int(bool(validate)), _stream(dev)))
    return Routing(sorted_ids, expert_ids, ntp, block_m, topk_ids, E_glob, first_expert, E_loc)


_KINDS = {"indexed": ROUTE_INDEXED, "contiguous": ROUTE_CONTIGUOUS, "masked": ROUTE_MASKED}


def select(T: int, topk: int, E_glob: int, E_loc: int, N: int, K: int, kind: str = "indexed",
           expected_m: int = 0) -> Config:
    """The library's tile choice (w4a16_select).  kind "indexed": T tokens,
    top-k of E_glob experts, E_loc local; "contiguous": T = rows of the
    layout, E_loc experts; "masked": T = max_m, E_loc groups, expected_m."""
    c = Config()
    check(load().w4a16_select(T, topk, E_glob, E_loc, N, K, _KINDS[kind], expected_m, ctypes.byref(c)))
    return c


def config(block_m: int, nr: int, waves: int = 4, split_k: int = 1, stages: int = 2,
           kind: str = "indexed", combine_cols: int = 0) -> Config:
    """split_k = 1: one workgroup per tile; 2, 4, 8, 16: K slices per tile,
    reduced in slice order; 0: stream-K over resident workgroups.
    stages: K chunks of weights in flight per wave (2, or 4 for small tiles).
    combine_cols: output columns per GEMM + combine pass of a top-k combine
    (0: the library's choice; else a multiple of 16)."""
    return Config(block_m, nr, waves, split_k, stages, _KINDS[kind], combine_cols)


def indexed_config(routing: "Routing", packed: PackedW4) -> Config:
    """The config moe_w4a16_gemm and moe_gate_up_silu use when cfg is None:
    the selector's choice for the routing's shape with the routing's
    block_m."""
    c = Config()
    check(load().w4a16_indexed_config(routing.T, routing.topk, routing.E_glob, routing.E_loc, packed.N, packed.K,
                                      routing.block_m, ctypes.byref(c)))
    return c


def workspace_bytes(packed: PackedW4, routing: "Routing", combine: bool, cfg: Optional[Config] = None) -> int:
    """Workspace bytes of moe_w4a16_gemm (zero-fill it once before first use)."""
    r = routing.as_c()
    return int(load().w4a16_moe_gemm_workspace_bytes(
        ctypes.byref(packed.desc), ctypes.byref(r), int(bool(combine)),
        None if cfg is None else ctypes.byref(cfg)))


def grouped_workspace_bytes(packed: PackedW4, kind: str, rows: int, expected_m: int = 0,
                            cfg: Optional[Config] = None) -> int:
    """Workspace bytes of a grouped call ("contiguous": rows = m_rows;
    "masked": rows = max_m, with its expected_m)."""
    return int(load().w4a16_grouped_workspace_bytes(ctypes.byref(packed.desc), _KINDS[kind], rows, expected_m,
                                                    None if cfg is None else ctypes.byref(cfg)))


def _workspace(nbytes: int, dev: torch.device) -> Optional[torch.Tensor]:
    # zero-filled: split-K arrival counters start at zero (calls leave them so)
    return torch.zeros(nbytes, dtype=torch.uint8, device=dev) if nbytes else None


_A_LAYOUTS = {"token": A_TOKEN, "slot": A_SLOT, "sorted": A_SORTED}


def moe_w4a16_gemm(a: torch.Tensor, packed: PackedW4, routing: Routing,
                   topk_weights: Optional[torch.Tensor] = None, a_layout: Optional[str] = None,
                   cfg: Optional[Config] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexed MoE GEMM.  Without topk_weights: out[T*k, N] per routed slot
    (only local slots written).  With topk_weights float32 [T, k]: out[T, N]
    top-k-weighted combine.  a_layout: "token" (a[T, K]), "slot" (a[T*k, K])
    or "sorted" (a[capacity, K], row p for sorted position p, as written by
    moe_gate_up_silu); default "slot" with topk_weights, else "token"."""
    _need(a, "a", _BF16, 2)
    T, k = routing.T, routing.topk
    if a_layout is None:
        a_layout = "slot" if topk_weights is not None else "token"
    if a_layout not in _A_LAYOUTS:
        raise ValueError(f"a_layout must be one of {sorted(_A_LAYOUTS)}")
    if a.shape[1] != packed.K:
        raise ValueError(f"a has K={a.shape[1]}, weight has K={packed.K}")
    dev = a.device
    combine = topk_weights is not None
    if combine:
        _need(topk_weights, "topk_weights", (torch.float32,), 2)
        rows = T
    else:
        rows = T * k
    if out is None:
        out = (torch.zeros if not combine else torch.empty)(rows, packed.N, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", _BF16, 2)
        if out.shape[0] < rows or out.shape[1] != packed.N:
            raise ValueError(f"out must be [{rows}, {packed.N}]")
    if workspace is None:
        workspace = _workspace(workspace_bytes(packed, routing, combine, cfg), dev)
    r = routing.as_c()
    check(load().w4a16_moe_gemm(ctypes.byref(packed.desc), packed.w.data_ptr(), packed.s.data_ptr(),
                                a.data_ptr(), a.shape[0], _A_LAYOUTS[a_layout], ctypes.byref(r),
                                _ptr(topk_weights), out.data_ptr(),
                                None if cfg is None else ctypes.byref(cfg),
                                _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                _stream(dev)))
    return out


def moe_gate_up_silu(x: torch.Tensor, packed: PackedW4, routing: Routing,
                     cfg: Optional[Config] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused gate/up + SiLU(gate) * up for a gate_up-packed weight [E, 2I, K]:
    out bf16 [capacity, I], row p = sorted position p (rows of local slots
    written, padding rows left as they are)."""
    _need(x, "x", _BF16, 2)
    if not packed.gate_up:
        raise ValueError("moe_gate_up_silu needs a weight packed with gate_up=True")
    if x.shape[1] != packed.K:
        raise ValueError(f"x has K={x.shape[1]}, weight has K={packed.K}")
    if out is None:
        out = torch.empty(routing.capacity, packed.N // 2, dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, "out", _BF16, 2)
        if out.shape[0] < routing.capacity or out.shape[1] != packed.N // 2:
            raise ValueError(f"out must be [{routing.capacity}, {packed.N // 2}]")
    r = routing.as_c()
    check(load().w4a16_moe_gate_up_silu(ctypes.byref(packed.desc), packed.w.data_ptr(), packed.s.data_ptr(),
                                        x.data_ptr(), x.shape[0], ctypes.byref(r), out.data_ptr(),
                                        None if cfg is None else ctypes.byref(cfg), _stream(x.device)))
    return out


def grouped_contiguous(a: torch.Tensor, packed: PackedW4, m_indices: torch.Tensor,
                       cfg: Optional[Config] = None, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """a [m, K] (experts' rows back to back, 128-row aligned segments),
    m_indices int32 [m] (-1 on padding) -> out [m, N].  cfg: None (the
    call's own selection) or select(..., kind="contiguous")."""
    _need(a, "a", _BF16, 2)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m = a.shape[0]
    if m_indices.shape[0] != m or a.shape[1] != packed.K:
        raise ValueError("a / m_indices / weight shapes disagree")
    if out is None:
        out = torch.zeros(m, packed.N, dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        workspace = _workspace(grouped_workspace_bytes(packed, "contiguous", m, 0, cfg), a.device)
    check(load().w4a16_grouped_contiguous(ctypes.byref(packed.desc), packed.w.data_ptr(),
                                          packed.s.data_ptr(), a.data_ptr(), m, m_indices.data_ptr(),
                                          out.data_ptr(), None if cfg is None else ctypes.byref(cfg),
                                          _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                          _stream(a.device)))
    return out


def grouped_masked(a: torch.Tensor, packed: PackedW4, masked_m: torch.Tensor, expected_m: int,
                   cfg: Optional[Config] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """a [E, max_m, K], masked_m int32 [E] -> out flat [E * max_m, N].
    cfg: None (the call's own selection from expected_m) or
    select(..., kind="masked")."""
    _need(a, "a", _BF16, 3)
    _need(masked_m, "masked_m", (torch.int32,), 1)
    G, max_m, K = a.shape
    if G != packed.E or K != packed.K or masked_m.shape[0] != G:
        raise ValueError("a / masked_m / weight shapes disagree")
    if out is None:
        out = torch.zeros(G * max_m, packed.N, dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        workspace = _workspace(grouped_workspace_bytes(packed, "masked", max_m, int(expected_m), cfg), a.device)
    check(load().w4a16_grouped_masked(ctypes.byref(packed.desc), packed.w.data_ptr(),
                                      packed.s.data_ptr(), a.data_ptr(), max_m, masked_m.data_ptr(),
                                      int(expected_m), out.data_ptr(),
                                      None if cfg is None else ctypes.byref(cfg),
                                      _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                      _stream(a.device)))
    return out


__all__ = [
    "W4A16Error", "PackedW4", "Routing", "Config", "weight_desc", "pack_w4", "align_capacity",
    "moe_align", "select", "config", "indexed_config", "workspace_bytes", "grouped_workspace_bytes", "moe_w4a16_gemm",
    "moe_gate_up_silu",
    "grouped_contiguous",
    "grouped_masked",
]


# ------------------------------------------------------------ A4W4 (MXFP4)

@dataclasses.dataclass
class MXRows:
    """MXFP4 rows: codes uint8 [rows, K/2] (two E2M1 codes per byte, element
    2i in the low nibble) and E8M0 scales uint8 [rows, K/32]."""
    codes: torch.Tensor
    scales: torch.Tensor

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def K(self):
        return 2 * self.codes.shape[1]


def mxfp4_weight_desc(E: int, N: int, K: int, gate_up: bool = False) -> WeightDesc:
    d = WeightDesc()
    init = load().w4a16_mxfp4_weight_desc_init_gate_up if gate_up else load().w4a16_mxfp4_weight_desc_init
    check(init(E, N, K, ctypes.byref(d)))
    return d


def pack_mxfp4(codes: torch.Tensor, scales: torch.Tensor, gate_up: bool = False) -> PackedW4:
    """MXFP4 weight: codes uint8 [E, N, K/2] (two per byte), E8M0 scales
    uint8 [E, N, K/32] -> packed weight (K % 128 == 0).  gate_up: rows
    [0, N/2) gate, [N/2, N) up, tiles interleaved (moe_mxfp4_gate_up_silu)."""
    _need(codes, "codes", (torch.uint8,), 3)
    _need(scales, "scales", (torch.uint8,), 3)
    E, N, K2 = codes.shape
    K = 2 * K2
    if tuple(scales.shape) != (E, N, K // 32):
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
    d = mxfp4_weight_desc(E, N, K, gate_up)
    w = torch.empty(d.w_bytes, dtype=torch.uint8, device=codes.device)
    s = torch.empty(d.s_bytes, dtype=torch.uint8, device=codes.device)
    check(load().w4a16_mxfp4_pack(codes.data_ptr(), scales.data_ptr(), ctypes.byref(d), w.data_ptr(),
                                  s.data_ptr(), _stream(codes.device)))
    return PackedW4(d, w, s)


def mxfp4_quant(x: torch.Tensor, out: Optional[MXRows] = None) -> MXRows:
    """bf16 [rows, K] -> MXFP4 rows (per row and block of 32: shared exponent
    floor(log2 max|v|) - 2, nearest-even E2M1 elements clamped at 6)."""
    _need(x, "x", _BF16, 2)
    R, K = x.shape
    if out is None:
        out = MXRows(torch.empty(R, K // 2, dtype=torch.uint8, device=x.device),
                     torch.empty(R, K // 32, dtype=torch.uint8, device=x.device))
    elif out.rows < R or out.K != K:
        raise ValueError(f"out must hold [{R}, {K}] MXFP4 rows")
    check(load().w4a16_mxfp4_quant(x.data_ptr(), R, K, out.codes.data_ptr(), out.scales.data_ptr(),
                                   _stream(x.device)))
    return out


def mxfp4_quant_local_slots(x: torch.Tensor, routing: Routing, out: Optional[MXRows] = None) -> MXRows:
    """mxfp4_quant on per-slot rows x [T * topk, K], converting only the rows
    of slots routed to the routing's local experts (the rows the down GEMM
    reads); other rows of `out` are left as they are."""
    _need(x, "x", _BF16, 2)
    R, K = x.shape
    T, k = routing.T, routing.topk
    if R != T * k:
        raise ValueError(f"x must hold T * topk = {T * k} rows")
    if out is None:
        out = MXRows(torch.empty(R, K // 2, dtype=torch.uint8, device=x.device),
                     torch.empty(R, K // 32, dtype=torch.uint8, device=x.device))
    elif out.rows < R or out.K != K:
        raise ValueError(f"out must hold [{R}, {K}] MXFP4 rows")
    check(load().w4a16_mxfp4_quant_local_slots(x.data_ptr(), routing.topk_ids.data_ptr(), T, k,
                                               routing.first_expert, routing.E_loc, K, out.codes.data_ptr(),
                                               out.scales.data_ptr(), _stream(x.device)))
    return out


def mxfp4_workspace_bytes(packed: PackedW4, T: int, topk: int, combine: bool) -> int:
    """Workspace moe_mxfp4_gemm needs (the top-k combine's fp32 partials)."""
    return int(load().w4a16_mxfp4_moe_gemm_workspace_bytes(ctypes.byref(packed.desc), T, topk, int(bool(combine))))


def mxfp4_select(T: int, topk: int, E_glob: int, E_loc: int, N: int, K: int) -> Config:
    """The library's A4W4 tile choice (block_m decides the routing alignment)."""
    c = Config()
    check(load().w4a16_mxfp4_select(T, topk, E_glob, E_loc, N, K, ctypes.byref(c)))
    return c


def mxfp4_config(block_m: int, nr: int = 4, stages: Optional[int] = None) -> Config:
    """An A4W4 tile config: nr 2 or 4 weight tiles per wave on four waves, or
    nr 1 (block_m 16): the K-split tile, whose eight waves split K."""
    return config(block_m, nr, waves=8 if nr == 1 else 4, split_k=1,
                  stages=(4 if block_m <= 32 else 2) if stages is None else stages)


def moe_mxfp4_gemm(a: MXRows, packed: PackedW4, routing: Routing,
                   topk_weights: Optional[torch.Tensor] = None, a_layout: Optional[str] = None,
                   cfg: Optional[Config] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexed A4W4 MoE GEMM on MXFP4 rows and an MXFP4 weight; outputs as
    moe_w4a16_gemm (per slot, or the top-k combine with topk_weights).
    a_layout: "token", "slot" (default with topk_weights) or "sorted" (the
    rows moe_mxfp4_gate_up_silu writes)."""
    if not packed.desc.flags & DESC_MXFP4:
        raise ValueError("moe_mxfp4_gemm needs a weight from pack_mxfp4")
    _need(a.codes, "a.codes", (torch.uint8,), 2)
    _need(a.scales, "a.scales", (torch.uint8,), 2)
    T, k = routing.T, routing.topk
    if a_layout is None:
        a_layout = "slot" if topk_weights is not None else "token"
    if a_layout not in _A_LAYOUTS:
        raise ValueError(f"a_layout must be one of {sorted(_A_LAYOUTS)}")
    if a.K != packed.K or a.scales.shape[1] != packed.K // 32:
        raise ValueError(f"activations have K={a.K}, weight has K={packed.K}")
    dev = a.codes.device
    combine = topk_weights is not None
    if combine:
        _need(topk_weights, "topk_weights", (torch.float32,), 2)
    rows = T if combine else T * k
    if out is None:
        out = (torch.zeros if not combine else torch.empty)(rows, packed.N, dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", _BF16, 2)
        if out.shape[0] < rows or out.shape[1] != packed.N:
            raise ValueError(f"out must be [{rows}, {packed.N}]")
    if workspace is None:
        nws = mxfp4_workspace_bytes(packed, T, k, combine)
        if nws:
            workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    r = routing.as_c()
    check(load().w4a16_mxfp4_moe_gemm(ctypes.byref(packed.desc), packed.w.data_ptr(), packed.s.data_ptr(),
                                      a.codes.data_ptr(), a.scales.data_ptr(), a.rows, _A_LAYOUTS[a_layout],
                                      ctypes.byref(r), _ptr(topk_weights), out.data_ptr(),
                                      None if cfg is None else ctypes.byref(cfg),
                                      _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                      _stream(dev)))
    return out


def moe_mxfp4_gate_up_silu(x: MXRows, packed: PackedW4, routing: Routing, cfg: Optional[Config] = None,
                           out: Optional[MXRows] = None) -> MXRows:
    """Fused A4W4 gate/up for a gate/up-interleaved MXFP4 weight [E, 2I, K]:
    MXFP4 rows of bf16(silu(g) * u) at sorted positions, [capacity, I]
    (padding positions unwritten); the down projection reads them with
    a_layout="sorted"."""
    if packed.desc.flags != (DESC_MXFP4 | DESC_GATE_UP):
        raise ValueError("moe_mxfp4_gate_up_silu needs a weight from pack_mxfp4(..., gate_up=True)")
    _need(x.codes, "x.codes", (torch.uint8,), 2)
    _need(x.scales, "x.scales", (torch.uint8,), 2)
    if x.K != packed.K:
        raise ValueError(f"activations have K={x.K}, weight has K={packed.K}")
    I = packed.N // 2
    cap = routing.capacity
    dev = x.codes.device
    if out is None:
        out = MXRows(torch.zeros(cap, I // 2, dtype=torch.uint8, device=dev),
                     torch.zeros(cap, I // 32, dtype=torch.uint8, device=dev))
    elif out.rows < cap or out.K != I:
        raise ValueError(f"out must hold [{cap}, {I}] MXFP4 rows")
    r = routing.as_c()
    check(load().w4a16_mxfp4_gate_up_silu(ctypes.byref(packed.desc), packed.w.data_ptr(), packed.s.data_ptr(),
                                          x.codes.data_ptr(), x.scales.data_ptr(), x.rows, ctypes.byref(r),
                                          out.codes.data_ptr(), out.scales.data_ptr(),
                                          None if cfg is None else ctypes.byref(cfg), _stream(dev)))
    return out
