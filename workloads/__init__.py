"""Seeded synthetic inputs for the MoE layer: the one module shared by the
CPU oracle's tests and the GPU path's tests and benchmark.

It draws inputs only. It holds none of the layer's arithmetic (no schedule,
no expert MLP, no combine, no MXFP8 rounding): the router that produces
``top_experts`` and ``router_weights`` lives outside the layer on the pages
("Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
§"Where MoK is the wrong tool": the router is the caller's), so drawing the
routing here is part of making the input, not of the method.

Recipe: ``numpy.random.SeedSequence(seed).spawn(9)`` gives one independent
PCG64 stream per tensor, in this order: x, router logits, W_gate, W_up,
W_down, S_gate, S_up, S_down, grad_out (so shrinking one tensor's shape never
changes another tensor's values, e.g. the routing). Floats are drawn in float32 and rounded to bfloat16 (round to
nearest even) and kept as raw uint16 bit patterns, so the same bytes feed
the oracle and the GPU. Top-k is the k largest logits per token (stable
order: descending logit, ties by lower expert id); router weights are the
softmax over the k selected logits in float32.

Tensor layouts follow the NeMo AutoModel page ("mok_experts",
``_MoKRuntime.forward`` parameters): x [T,H]; top_experts int64 [T,k];
router_weights fp32 [T,k]; routed gate/up [E,I,H]; routed down [E,H,I];
shared gate/up [I_s,H]; shared down [H,I_s]. All contiguous.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["MoEShape", "CONFIGS", "make_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """One workload: shapes, routing recipe, capacity and seed."""
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    I_s: int
    seed: int
    mode: str = "bf16"            # "bf16" or "mxfp8"
    passes: str = "fwd"           # "fwd" or "fwd+bwd"
    routing: str = "normal"       # "normal" or "zipf"
    zipf_s: float = 1.2
    capacity_multiplier: float = 1.0
    expert_pad: int = 32
    x_std: float = 1.0
    w_std: float = 0.02

    def with_(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)

    def fwd_flops(self, kept_assignments: int | None = None, shared_rows: int | None = None) -> float:
        """Algorithmic forward FLOPs: 6*H*I per kept routed assignment
        (gate, up and down GEMMs) plus 6*H*I_s per token for the shared
        expert. Padding rows and capacity slack are not counted."""
        R = self.T * self.k if kept_assignments is None else kept_assignments
        Ts = self.T if shared_rows is None else shared_rows
        return 6.0 * self.H * (R * self.I + (Ts * self.I_s if self.I_s else 0))


# The five workloads, plus a labelled sixth (MXFP8 forward+backward at the
# 8192-token shape) that exercises the MXFP8 backward.
CONFIGS: dict[str, MoEShape] = {
    "tiny_bf16_fwd": MoEShape("tiny_bf16_fwd", T=256, H=128, I=64, E=8, k=2, I_s=0, seed=1000),
    "t8192_bf16_fwd": MoEShape("t8192_bf16_fwd", T=8192, H=2048, I=768, E=128, k=8, I_s=768, seed=1001),
    "skew_bf16_fwd": MoEShape("skew_bf16_fwd", T=16384, H=4096, I=1536, E=32, k=4, I_s=1536, seed=1002,
                              routing="zipf"),
    "t8192_mxfp8_fwd": MoEShape("t8192_mxfp8_fwd", T=8192, H=2048, I=768, E=128, k=8, I_s=768, seed=1003,
                                mode="mxfp8"),
    "t32768_bf16_fwdbwd": MoEShape("t32768_bf16_fwdbwd", T=32768, H=7168, I=2048, E=32, k=8, I_s=2048,
                                   seed=1004, passes="fwd+bwd"),
    "t8192_mxfp8_fwdbwd": MoEShape("t8192_mxfp8_fwdbwd", T=8192, H=2048, I=768, E=128, k=8, I_s=768,
                                   seed=1005, mode="mxfp8", passes="fwd+bwd"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs are finite (drawn from normals)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    n = flat.size
    chunk = 1 << 24
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[s:s + m] = f32_to_bf16_bits(v)
    return out


def _route(logits: np.ndarray, k: int):
    """Top-k (descending logit, ties to the lower expert id) and the softmax
    of the selected logits, renormalised over the k, in float32."""
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int64)
    sel = np.take_along_axis(logits, idx, axis=1).astype(np.float32)
    sel = sel - sel.max(axis=1, keepdims=True)
    e = np.exp(sel, dtype=np.float32)
    w = (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def make_inputs(cfg: MoEShape, *, with_grad: bool | None = None, T: int | None = None) -> dict:
    """Draw every input of one workload. Returns a dict of numpy arrays:
    x, grad_out (uint16 bf16 bits), top_experts (int64), router_weights
    (float32), w_gate, w_up, w_down, s_gate, s_up, s_down (uint16 bf16 bits;
    shared ones are None when I_s == 0), plus 'logits' (float32)."""
    T = cfg.T if T is None else T
    H, I, E, k, I_s = cfg.H, cfg.I, cfg.E, cfg.k, cfg.I_s
    if with_grad is None:
        with_grad = cfg.passes != "fwd"
    streams = [np.random.default_rng(s) for s in np.random.SeedSequence(cfg.seed).spawn(9)]
    x = _normal_bf16(streams[0], (T, H), cfg.x_std)
    logits = streams[1].standard_normal((T, E), dtype=np.float32)
    if cfg.routing == "zipf":
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-cfg.zipf_s)
        p /= p.sum()
        logits = (logits + np.log(p).astype(np.float32)).astype(np.float32)
    top, w = _route(logits, k)
    wg = _normal_bf16(streams[2], (E, I, H), cfg.w_std)
    wu = _normal_bf16(streams[3], (E, I, H), cfg.w_std)
    wd = _normal_bf16(streams[4], (E, H, I), cfg.w_std)
    if I_s:
        sg = _normal_bf16(streams[5], (I_s, H), cfg.w_std)
        su = _normal_bf16(streams[6], (I_s, H), cfg.w_std)
        sd = _normal_bf16(streams[7], (H, I_s), cfg.w_std)
    else:
        sg = su = sd = None
    g = _normal_bf16(streams[8], (T, H), 1.0) if with_grad else None
    return dict(x=x, logits=logits, top_experts=top, router_weights=w,
                w_gate=wg, w_up=wu, w_down=wd, s_gate=sg, s_up=su, s_down=sd, grad_out=g)

