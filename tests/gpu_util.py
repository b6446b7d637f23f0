"""Helpers for the GPU parity tests: host <-> device copies of the seeded
inputs and the element-wise comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda", 0)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "", rel_rms: float = 1e-2):
    """max |got - ref| <= rel_rms * RMS(ref) + 1 bf16 ulp(ref), element-wise
    (the stated output tolerance).  Returns (max abs err, fraction bit-exact)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = O.bf16_to_f64(got)
    r = O.bf16_to_f64(ref)
    tol = O.tolerance(ref, rel_rms)
    err = np.abs(g - r)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"first at {idx.tolist()}: got {g[tuple(idx[0])]}, ref {r[tuple(idx[0])]}, "
                             f"tol {tol[tuple(idx[0])]}")
    exact = float(np.mean(got == ref)) if got.size else 1.0
    return float(err.max()) if err.size else 0.0, exact


class Problem:
    """Seeded inputs of one workload (host copies) plus their device copies."""

    def __init__(self, shape, with_down=True, T=None):
        from synth import workloads as W
        self.sh = shape
        sh = shape
        self.T = sh.T if T is None else T
        self.topk_ids, self.topk_w = W.routing_for(sh, self.T)
        self.x = W.activations(sh.seed, "x", self.T, sh.K1)
        self.c1 = W.weight_codes(sh.seed, "w1_codes", sh.E_loc, sh.N1, sh.K1)
        self.s1 = W.weight_scales(sh.seed, "w1_scales", sh.E_loc, sh.N1, sh.K1)
        if with_down:
            self.a = W.activations(sh.seed, "a", self.T * sh.topk, sh.K2)
            self.c2 = W.weight_codes(sh.seed, "w2_codes", sh.E_loc, sh.N2, sh.K2)
            self.s2 = W.weight_scales(sh.seed, "w2_scales", sh.E_loc, sh.N2, sh.K2)
        self.with_down = with_down

    def upload(self):
        import w4a16_int4_mixture_moe_amd as M
        self.d_ids = to_dev(self.topk_ids)
        self.d_w = to_dev(self.topk_w)
        self.d_x = to_dev_bf16(self.x)
        self.p1 = M.pack_w4(to_dev(self.c1), to_dev_bf16(self.s1))
        if self.with_down:
            self.d_a = to_dev_bf16(self.a)
            self.p2 = M.pack_w4(to_dev(self.c2), to_dev_bf16(self.s2))
        torch.cuda.synchronize()
        return self
