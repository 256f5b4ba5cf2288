"""Shared helpers of the test suite: device transfer of seeded inputs,
lazily decoded bf16 weight arrays for the oracle, tolerance checks, and a
process pool that runs the oracle's own MXFP8 quantizer on slices of large
weight tensors in parallel.

Holds none of the layer's arithmetic."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import bf16_bits_to_f32  # noqa: E402

# Tolerances of the acceptance bar: max |err| <= tol * max |ref| per tensor.
TOL_BF16 = 2e-2
TOL_MXFP8 = 6e-2


class Bf16Array:
    """Read-only view of a bf16 bit-pattern array that decodes to float64 on
    indexing (so the oracle never holds a whole decoded weight tensor)."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return bf16_bits_to_f32(np.asarray(self.bits[idx])).astype(np.float64)

    def full(self) -> np.ndarray:
        return bf16_bits_to_f32(self.bits).astype(np.float64)

    def __array__(self, dtype=None, copy=None):
        a = self.full()
        return a if dtype is None else a.astype(dtype)


def f64(bits):
    return None if bits is None else bf16_bits_to_f32(bits).astype(np.float64)


def to_dev(inp: dict, device="cuda"):
    """Seeded numpy inputs -> device tensors (bf16 bit patterns reinterpreted)."""
    import torch

    def bf(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    out = dict(x=bf(inp["x"]), top_experts=torch.from_numpy(inp["top_experts"]).to(device),
               router_weights=torch.from_numpy(inp["router_weights"]).to(device),
               grad_out=bf(inp.get("grad_out")))
    out["weights"] = {"routed_gate": bf(inp["w_gate"]), "routed_up": bf(inp["w_up"]),
                      "routed_down": bf(inp["w_down"])}
    if inp.get("s_gate") is not None:
        out["weights"].update(shared_gate=bf(inp["s_gate"]), shared_up=bf(inp["s_up"]),
                              shared_down=bf(inp["s_down"]))
    return out


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").float().numpy().astype(np.float64) if t.dtype != torch.float32 else \
        t.detach().cpu().numpy().astype(np.float64)


def assert_close_inf(got: np.ndarray, ref: np.ndarray, tol: float, what: str = ""):
    """max |got - ref| <= tol * max |ref| (the acceptance bar)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= tol * max(scale, 1e-30), f"{what}: max|err| {err:.4g} > {tol} * {scale:.4g}"
    return err, scale


# ---------------------------------------------------------------------------
# The oracle's quantizer on slices of a large tensor, in worker processes
# ---------------------------------------------------------------------------

def _qdq_chunk(args):
    from oracle import mxfp8
    v, axis = args
    return mxfp8.qdq(v, axis)


_POOL = None


def _pool():
    # spawned (not forked) workers: the parent may hold a GPU context
    global _POOL
    if _POOL is None:
        import multiprocessing as mp
        n = max(1, min(16, os.cpu_count() or 1))
        _POOL = mp.get_context("spawn").Pool(n)
    return _POOL


def par_qdq(v, axis):
    """``oracle.mxfp8.qdq(v, axis)``, computed on slices of ``v`` along
    another axis in worker processes. Blocks of 32 run along ``axis`` only,
    so no block crosses a slice and the values are those of one call."""
    from oracle import mxfp8
    v = np.ascontiguousarray(v, np.float64)
    axis %= v.ndim
    split = 0 if axis != 0 else 1
    n = v.shape[split]
    if v.size < (1 << 22) or n < 2:
        return mxfp8.qdq(v, axis)
    pieces = min(n, 64)
    bounds = [n * i // pieces for i in range(pieces + 1)]
    sl = lambda lo, hi: tuple(slice(lo, hi) if d == split else slice(None) for d in range(v.ndim))  # noqa: E731
    outs = _pool().map(_qdq_chunk, [(v[sl(lo, hi)], axis) for lo, hi in zip(bounds[:-1], bounds[1:])],
                       chunksize=1)
    return np.concatenate(outs, axis=split)


def oracle_qweights(inp: dict, for_backward: bool = False) -> dict:
    """``oracle.moe.quantize_weights_mxfp8`` of a workload's weights, with
    the quantizer run in parallel (``par_qdq``)."""
    from oracle import moe as omoe
    return omoe.quantize_weights_mxfp8(f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]),
                                       f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]),
                                       for_backward=for_backward, qfun=par_qdq)
