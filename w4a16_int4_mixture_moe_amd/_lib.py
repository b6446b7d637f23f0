"""ctypes view of the C ABI in include/w4a16_moe.h.

Loading fails loudly when the HIP library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

W4A16_OK = 0
STATUS_NAMES = {
    0: "OK", -1: "ERR_ARG", -2: "ERR_SHAPE", -3: "ERR_LAYOUT", -4: "ERR_UNSUPPORTED",
    -5: "ERR_CAPACITY", -6: "ERR_ROUTING", -7: "ERR_HIP", -8: "ERR_WORKSPACE",
}


class W4A16Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class WeightDesc(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("K_pad", ctypes.c_int32), ("chunks", ctypes.c_int32), ("group", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("w_bytes", ctypes.c_uint64), ("s_bytes", ctypes.c_uint64), ("check", ctypes.c_uint64),
    ]


DESC_GATE_UP = 1            # W4A16_DESC_GATE_UP
DESC_MXFP4 = 2              # W4A16_DESC_MXFP4
A_TOKEN, A_SLOT, A_SORTED = 0, 1, 2   # W4A16_A_TOKEN / _SLOT / _SORTED
ROUTE_INDEXED, ROUTE_CONTIGUOUS, ROUTE_MASKED = 0, 1, 2   # W4A16_ROUTE_*


class Config(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("nr", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("split_k", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("combine_cols", ctypes.c_int32)]

    def __repr__(self):
        return (f"Config(block_m={self.block_m}, nr={self.nr}, waves={self.waves}, "
                f"split_k={self.split_k}, stages={self.stages}, kind={self.kind}, "
                f"combine_cols={self.combine_cols})")


class IndexedRouting(ctypes.Structure):
    _fields_ = [
        ("sorted_ids", ctypes.c_void_p), ("expert_ids", ctypes.c_void_p),
        ("num_tokens_padded", ctypes.c_void_p), ("capacity", ctypes.c_int64),
        ("block_m", ctypes.c_int32), ("T", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("topk_ids", ctypes.c_void_p), ("first_expert", ctypes.c_int32), ("E_loc", ctypes.c_int32),
        ("E_glob", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every function the header declares
SIGNATURES = {
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_abi_version": (_I32, []),
    "w4a16_weight_desc_init": (_I32, [_I32, _I32, _I32, ctypes.POINTER(WeightDesc)]),
    "w4a16_weight_desc_init_gate_up": (_I32, [_I32, _I32, _I32, ctypes.POINTER(WeightDesc)]),
    "w4a16_pack_w4": (_I32, [_P, _P, ctypes.POINTER(WeightDesc), _P, _P, _P]),
    "w4a16_align_capacity": (_I64, [_I32, _I32, _I32, _I32]),
    "w4a16_moe_align": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _I32, _P]),
    "w4a16_select": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Config)]),
    "w4a16_mxfp4_select": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Config)]),
    "w4a16_indexed_config": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Config)]),
    "w4a16_moe_gemm_workspace_bytes": (_SZ, [ctypes.POINTER(WeightDesc), ctypes.POINTER(IndexedRouting), _I32,
                                             ctypes.POINTER(Config)]),
    "w4a16_moe_gemm": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _I64, _I32,
                              ctypes.POINTER(IndexedRouting), _P, _P, ctypes.POINTER(Config),
                              _P, _SZ, _P]),
    "w4a16_moe_gemm_noalloc": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _I64, _I32,
                                      ctypes.POINTER(IndexedRouting), _P, _P, ctypes.POINTER(Config), _P]),
    "w4a16_moe_gate_up_silu": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _I64,
                                      ctypes.POINTER(IndexedRouting), _P, ctypes.POINTER(Config), _P]),
    "w4a16_grouped_contiguous": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _I64, _P, _P,
                                        ctypes.POINTER(Config), _P, _SZ, _P]),
    "w4a16_grouped_masked": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _I32, _P, _I32, _P,
                                    ctypes.POINTER(Config), _P, _SZ, _P]),
    "w4a16_grouped_workspace_bytes": (_SZ, [ctypes.POINTER(WeightDesc), _I32, _I64, _I32, ctypes.POINTER(Config)]),
    "w4a16_mxfp4_weight_desc_init": (_I32, [_I32, _I32, _I32, ctypes.POINTER(WeightDesc)]),
    "w4a16_mxfp4_weight_desc_init_gate_up": (_I32, [_I32, _I32, _I32, ctypes.POINTER(WeightDesc)]),
    "w4a16_mxfp4_gate_up_silu": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _P, _I64,
                                        ctypes.POINTER(IndexedRouting), _P, _P, ctypes.POINTER(Config), _P]),
    "w4a16_mxfp4_pack": (_I32, [_P, _P, ctypes.POINTER(WeightDesc), _P, _P, _P]),
    "w4a16_mxfp4_quant": (_I32, [_P, _I64, _I32, _P, _P, _P]),
    "w4a16_mxfp4_quant_local_slots": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "w4a16_mxfp4_moe_gemm_workspace_bytes": (_SZ, [ctypes.POINTER(WeightDesc), _I32, _I32, _I32]),
    "w4a16_mxfp4_moe_gemm": (_I32, [ctypes.POINTER(WeightDesc), _P, _P, _P, _P, _I64, _I32,
                                    ctypes.POINTER(IndexedRouting), _P, _P, ctypes.POINTER(Config),
                                    _P, _SZ, _P]),
}

_lib = None


def lib_path() -> str:
    return _build.lib_path()


def load() -> ctypes.CDLL:
    """Load the built HIP library (raises if it is missing)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise W4A16Error(-7, f"HIP library not built ({path}); run "
                                 "`python -m w4a16_int4_mixture_moe_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != W4A16_OK:
        msg = load().w4a16_last_error()
        raise W4A16Error(status, msg.decode() if msg else "")
