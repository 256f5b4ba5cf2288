"""PyTorch autograd over the C ABI: the layer as a differentiable function
and a module holding the routed experts' parameters.

This follows the integration layer of the pages ([A]
"nemo_automodel.components.moe.mok_experts": ``_MoKAutogradFunction``,
``_MoKRuntime``, ``GroupedExpertsMoK``, ``_flatten_mok_tensor_dataclass``),
read for one GPU:

- ``MoKRuntime`` owns one layer's configuration, its precision mode and the
  cached workspace of that configuration (one workspace serves every layer
  of the same shape, [R] "The two API layers and the schedule object").
- ``MoKAutogradFunction.forward`` builds the schedule, runs the fused
  forward and keeps its activation context; ``backward`` hands the same
  schedule and context to the fused backward and returns a gradient for
  every float input (none for the runtime and the integer expert ids).
- The schedule and the context are each one flat byte tensor, and both go
  through ``ctx.save_for_backward``: saved-tensor hooks (activation
  checkpointing, CPU offload) see them, and nothing else on ``ctx`` holds a
  tensor, so a layer's context lives only as long as autograd keeps it.
- In MXFP8 mode the parameters stay BF16; the forward takes them quantized
  by ``mxfp8_quantize`` along H (gate, up) and I (down), the backward
  transposed and quantized along each backward GEMM's contraction by
  ``mxfp8_quantize_transposed`` ([R] "Tuning the five hyperparameters
  before production": MXFP8 takes pre-quantized weights). Each quantized
  copy is kept per parameter and made again whenever the parameter's
  in-place version counter moves (an optimizer step, a ``copy_``), so a
  step never runs on stale codes.

Every step of the layer runs in the library's HIP kernels; tensors on the
CPU are rejected.
"""
from __future__ import annotations

import dataclasses
import weakref

import torch

from . import (MOK_MODE_BF16, MOK_MODE_MXFP8, MoKConfig, backward, build_schedule, context_bytes, forward,
               get_workspace, mxfp8_quantize, mxfp8_quantize_transposed)

__all__ = ["MoKRuntime", "MoKAutogradFunction", "MoKExperts", "moe_layer"]

_WEIGHT_NAMES = ("shared_gate", "shared_up", "shared_down", "routed_gate", "routed_up", "routed_down")


class MoKRuntime:
    """One layer's configuration, precision mode and SwiGLU input limit
    ([A] ``_MoKRuntime(mok_config, swiglu_limit)``; None keeps the config's
    own ``swiglu_limit``). The workspace comes from the per-(device, config)
    cache, so layers of one shape and limit share it."""

    def __init__(self, cfg: MoKConfig, mode: int = MOK_MODE_BF16, swiglu_limit: float | None = None):
        if mode not in (MOK_MODE_BF16, MOK_MODE_MXFP8):
            raise ValueError("mode must be MOK_MODE_BF16 or MOK_MODE_MXFP8")
        if swiglu_limit is not None:
            cfg = dataclasses.replace(cfg, swiglu_limit=float(swiglu_limit))
        self.cfg = cfg
        self.mode = mode
        # name -> (weak reference to the weight, its version, its address, codes, scales)
        self._q: dict = {}

    def workspace(self, device: torch.device):
        if device.type != "cuda":
            raise ValueError("the MoE layer runs on the GPU only: inputs must be CUDA tensors")
        return get_workspace(self.cfg, device.index if device.index is not None else torch.cuda.current_device())

    def quantized(self, name: str, w: torch.Tensor, transposed: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
        """MXFP8 codes and scales of a BF16 weight along its last dimension
        (the forward's form), or transposed and quantized along its
        second-to-last (the backward's form), made again when the weight
        changed since they were made."""
        key = (name, transposed)
        hit = self._q.get(key)
        if hit is not None:
            ref, version, ptr, codes, sc = hit
            if ref() is w and version == w._version and ptr == w.data_ptr():
                return codes, sc
        if transposed:
            codes, sc = mxfp8_quantize_transposed(w.detach())
        else:
            codes, sc = mxfp8_quantize(w.detach().reshape(-1, w.shape[-1]), axis=1)
            codes = codes.view(w.shape)
        self._q[key] = (weakref.ref(w), w._version, w.data_ptr(), codes, sc)
        return codes, sc

    def forward_weights(self, w: dict) -> dict:
        if self.mode == MOK_MODE_BF16:
            return w
        q = {}
        for name, t in w.items():
            if t is None:
                continue
            q[name], q[name + "_scale"] = self.quantized(name, t)
        return q

    def backward_weights(self, w: dict) -> dict:
        """MXFP8: the weights transposed and quantized for the backward's
        GEMMs, kept like the forward's codes until the weight changes."""
        if self.mode == MOK_MODE_BF16:
            return w
        q = {}
        for name, t in w.items():
            if t is None:
                continue
            q[name], q[name + "_scale"] = self.quantized(name, t, transposed=True)
        return q


def _check(name: str, t: torch.Tensor | None, dtype: torch.dtype, shape: tuple) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _run_forward(runtime: MoKRuntime, keep: bool, x, router_weights, top_experts, shared_gate, shared_up,
                 shared_down, routed_gate, routed_up, routed_down):
    """Validate, build the schedule and run the fused forward; the context
    is allocated and filled only when ``keep``. Returns (out, schedule,
    context or None, weights by name)."""
    cfg = runtime.cfg
    if x is None or x.dim() != 2:
        raise ValueError("x must be a [tokens, hidden] tensor")
    T = x.shape[0]
    H, I, Is, E, k = cfg.hidden, cfg.intermediate, cfg.shared_intermediate, cfg.num_experts, cfg.topk
    _check("x", x, torch.bfloat16, (T, H))
    _check("router_weights", router_weights, torch.float32, (T, k))
    _check("top_experts", top_experts, torch.int64, (T, k))
    _check("routed_gate", routed_gate, torch.bfloat16, (E, I, H))
    _check("routed_up", routed_up, torch.bfloat16, (E, I, H))
    _check("routed_down", routed_down, torch.bfloat16, (E, H, I))
    if Is:
        _check("shared_gate", shared_gate, torch.bfloat16, (Is, H))
        _check("shared_up", shared_up, torch.bfloat16, (Is, H))
        _check("shared_down", shared_down, torch.bfloat16, (H, Is))
    elif any(t is not None for t in (shared_gate, shared_up, shared_down)):
        raise ValueError("shared expert weights given but the config has shared_intermediate = 0")
    if T > cfg.max_tokens:
        raise ValueError(f"{T} tokens exceed the config's max_tokens {cfg.max_tokens}")
    w = dict(shared_gate=shared_gate, shared_up=shared_up, shared_down=shared_down,
             routed_gate=routed_gate, routed_up=routed_up, routed_down=routed_down)
    for name, t in [("x", x), ("router_weights", router_weights), ("top_experts", top_experts)] + list(w.items()):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}: every input must be on one GPU")
    ws = runtime.workspace(x.device)
    sched = build_schedule(ws, top_experts)
    context = torch.empty(context_bytes(cfg, runtime.mode), dtype=torch.uint8, device=x.device) if keep else None
    out = forward(ws, sched, x, router_weights, runtime.forward_weights(w), mode=runtime.mode, context=context)
    return out, sched, context, w


class MoKAutogradFunction(torch.autograd.Function):
    """out = MoE layer (schedule, gathered SwiGLU experts, shared expert,
    combine), differentiable in x, router_weights and every weight."""

    @staticmethod
    def forward(ctx, runtime: MoKRuntime, x, router_weights, top_experts, shared_gate, shared_up, shared_down,
                routed_gate, routed_up, routed_down):
        keep = any(ctx.needs_input_grad[1:])
        out, sched, context, w = _run_forward(runtime, keep, x, router_weights, top_experts, shared_gate,
                                              shared_up, shared_down, routed_gate, routed_up, routed_down)
        ctx.runtime = runtime
        if keep:
            ctx.save_for_backward(sched, context, x, router_weights, *[w[n] for n in _WEIGHT_NAMES])
        return out

    @staticmethod
    def backward(ctx, grad_out):
        runtime = ctx.runtime
        sched, context, x, router_weights, *wl = ctx.saved_tensors
        w = dict(zip(_WEIGHT_NAMES, wl))
        if grad_out.dtype != torch.bfloat16:
            grad_out = grad_out.to(torch.bfloat16)
        grad_out = grad_out.contiguous()
        ws = runtime.workspace(x.device)
        g = backward(ws, sched, context, grad_out, x, router_weights, runtime.backward_weights(w), mode=runtime.mode)
        need = ctx.needs_input_grad

        def pick(i, name):
            return g.get(name) if need[i] else None

        return (None, pick(1, "dx"), pick(2, "d_router_weights"), None,
                pick(4, "d_shared_gate"), pick(5, "d_shared_up"), pick(6, "d_shared_down"),
                pick(7, "d_routed_gate"), pick(8, "d_routed_up"), pick(9, "d_routed_down"))


def moe_layer(runtime: MoKRuntime, x, router_weights, top_experts, shared_gate, shared_up, shared_down,
              routed_gate, routed_up, routed_down) -> torch.Tensor:
    """Functional form of the differentiable layer (argument order of [A]
    ``_MoKAutogradFunction.forward``). When no gradient is wanted (grad mode
    off, or no input requires one) the forward runs without keeping a
    context."""
    args = (x, router_weights, top_experts, shared_gate, shared_up, shared_down, routed_gate, routed_up,
            routed_down)
    if torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in args):
        return MoKAutogradFunction.apply(runtime, *args)
    with torch.no_grad():
        return _run_forward(runtime, False, *args)[0]


class MoKExperts(torch.nn.Module):
    """Routed expert parameters in the library's native layouts (gate and
    up [E, I, H], down [E, H, I], bf16), run by the fused layer. As in [A]
    ``GroupedExpertsMoK``, the router stays outside: forward takes the
    router's weights and expert ids, plus the shared expert's weights, and
    there is no expert bias."""

    def __init__(self, hidden: int, intermediate: int, num_experts: int, topk: int, max_tokens: int,
                 shared_intermediate: int = 0, capacity_multiplier: float = 1.0, expert_pad: int = 32,
                 mode: int = MOK_MODE_BF16, device=None):
        super().__init__()
        self.runtime = MoKRuntime(MoKConfig(hidden=hidden, intermediate=intermediate, num_experts=num_experts,
                                            topk=topk, max_tokens=max_tokens,
                                            shared_intermediate=shared_intermediate,
                                            capacity_multiplier=capacity_multiplier, expert_pad=expert_pad), mode)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.routed_gate_weights = torch.nn.Parameter(torch.empty(num_experts, intermediate, hidden, **bf))
        self.routed_up_weights = torch.nn.Parameter(torch.empty(num_experts, intermediate, hidden, **bf))
        self.routed_down_weights = torch.nn.Parameter(torch.empty(num_experts, hidden, intermediate, **bf))

    @torch.no_grad()
    def init_weights(self, init_std: float = 0.02, generator: torch.Generator | None = None) -> None:
        """Normal(0, init_std) draws, rounded to bf16."""
        for p in (self.routed_gate_weights, self.routed_up_weights, self.routed_down_weights):
            p.copy_(torch.randn(p.shape, generator=generator, dtype=torch.float32).mul_(init_std))

    def forward(self, x, weights, indices, shared_gate_weights=None, shared_up_weights=None,
                shared_down_weights=None) -> torch.Tensor:
        """x bf16 [T, H], weights fp32 [T, k], indices int64 [T, k] -> bf16
        [T, H]: the routed experts' weighted SwiGLU outputs plus the shared
        expert's."""
        return moe_layer(self.runtime, x, weights, indices, shared_gate_weights, shared_up_weights,
                         shared_down_weights, self.routed_gate_weights, self.routed_up_weights,
                         self.routed_down_weights)

    def extra_repr(self) -> str:
        c = self.runtime.cfg
        mode = "mxfp8" if self.runtime.mode == MOK_MODE_MXFP8 else "bf16"
        return (f"hidden={c.hidden}, intermediate={c.intermediate}, experts={c.num_experts}, topk={c.topk}, "
                f"shared_intermediate={c.shared_intermediate}, max_tokens={c.max_tokens}, mode={mode}")

