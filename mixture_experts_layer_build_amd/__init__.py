"""MI355X-native MoE layer hot path: Python binding of libmok.so.

Thin argument marshalling over the C ABI in ``include/mok.h``: every step of
the path (schedule, MXFP8 quantization, gather, grouped SwiGLU GEMMs,
combine, backward) runs in the library's HIP kernels. PyTorch provides device
memory and the current stream only. There is no CPU fallback: the calls raise
when the library or a GPU is missing.

The names follow the pages' API ("Mixture-of-Kittens: a deterministic MoE
megakernel for NVL72 racks", section "The two API layers and the schedule
object"): a workspace is created once and reused across layers
(``create_workspace`` / ``get_workspace`` / ``clear_workspace_cache``), a
schedule is built once per layer and step (``build_schedule``) and passed to
``forward`` and ``backward``; ``mxfp8_quantize`` pre-quantizes weights.
"""
from __future__ import annotations

import ctypes as C
import dataclasses

import torch

from . import _lib
from ._lib import (MOK_MODE_BF16, MOK_MODE_MXFP8, HDR_FIELDS, TILE_BMS, MokError)

__all__ = ["MoKConfig", "Workspace", "create_workspace", "get_workspace", "clear_workspace_cache",
           "build_schedule", "forward", "forward_static", "backward", "mxfp8_quantize",
           "mxfp8_quantize_transposed", "mxfp8_backward_weights", "schedule_fields",
           "schedule_bytes", "context_bytes", "workspace_bytes", "MokError", "MOK_MODE_BF16", "MOK_MODE_MXFP8", "lib"]


def lib():
    return _lib.load()


@dataclasses.dataclass(frozen=True)
class MoKConfig:
    """Single-GPU reading of the pages' MoKConfig (see include/mok.h)."""
    hidden: int
    intermediate: int
    num_experts: int
    topk: int
    max_tokens: int
    shared_intermediate: int = 0
    capacity_multiplier: float = 1.0
    expert_pad: int = 32
    minibatch_size: int = 0
    num_mover_wgs: int = 0
    swiglu_limit: float = 0.0     # 0 = no limit (see include/mok.h)
    macrobatch_size: int = 0      # tokens per pass of the forward's token ring; 0 = one pass
    forward_only: int = 0         # 1 = inference workspace (no backward scratch)

    def c(self) -> _lib.MokConfig:
        return _lib.MokConfig(C.sizeof(_lib.MokConfig), self.hidden, self.intermediate, self.num_experts,
                              self.topk, self.shared_intermediate, self.max_tokens,
                              float(self.capacity_multiplier), self.expert_pad, self.minibatch_size,
                              self.num_mover_wgs, float(self.swiglu_limit), self.macrobatch_size,
                              self.forward_only)


def schedule_bytes(cfg: MoKConfig) -> int:
    c = cfg.c()
    n = lib().mok_schedule_bytes(C.byref(c))
    if n == 0:
        _lib.check("mok_schedule_bytes", lib().mok_validate_config(C.byref(c)))
    return n


def context_bytes(cfg: MoKConfig, mode: int = MOK_MODE_BF16) -> int:
    c = cfg.c()
    n = lib().mok_context_bytes(C.byref(c), mode)
    if n == 0:
        _lib.check("mok_context_bytes", lib().mok_validate_config(C.byref(c)))
    return n


def workspace_bytes(cfg: MoKConfig) -> int:
    """Device bytes a workspace of this configuration allocates."""
    c = cfg.c()
    n = lib().mok_workspace_bytes(C.byref(c))
    if n == 0:
        _lib.check("mok_workspace_bytes", lib().mok_validate_config(C.byref(c)))
    return n


def schedule_layout(cfg: MoKConfig) -> _lib.MokScheduleLayout:
    c = cfg.c()
    out = _lib.MokScheduleLayout()
    _lib.check("mok_schedule_layout_query", lib().mok_schedule_layout_query(C.byref(c), C.byref(out)))
    return out


def _stream() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


_PLACEHOLDER: dict = {}


def _ptr(t) -> C.c_void_p | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if t.numel() == 0:
        # An empty batch: torch gives no storage (pointer 0), which the
        # library rejects. The kernels read T = 0 from the schedule and never
        # touch these buffers, so a small placeholder of the device stands in.
        dev = t.device.index if t.device.index is not None else torch.cuda.current_device()
        if dev not in _PLACEHOLDER:
            _PLACEHOLDER[dev] = torch.zeros(64, dtype=torch.int32, device=t.device)
        return C.c_void_p(_PLACEHOLDER[dev].data_ptr())
    return C.c_void_p(t.data_ptr())


class Workspace:
    """Device scratch for one config on one device, reused across layers
    and steps. One stream at a time."""

    def __init__(self, cfg: MoKConfig, device: int | None = None):
        if device is None:
            device = torch.cuda.current_device()
        self.cfg = cfg
        self.device = int(device)
        self._c = cfg.c()
        h = C.c_void_p()
        _lib.check("mok_workspace_create", lib().mok_workspace_create(C.byref(self._c), self.device, C.byref(h)))
        self.handle = h
        self.layout = schedule_layout(cfg)

    def close(self) -> None:
        if getattr(self, "handle", None):
            _lib.check("mok_workspace_destroy", lib().mok_workspace_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # per-kernel event timing (diagnostics)
    def set_timing(self, on: bool, kernels=None) -> None:
        """Time every kernel (on), none (off), or only the named ones
        (kernels: names as mok_kernel_name gives them, e.g. "gate_up")."""
        if kernels is None or not on:
            _lib.check("mok_workspace_set_timing", lib().mok_workspace_set_timing(self.handle, int(on)))
            return
        ids = {lib().mok_kernel_name(i).decode(): i for i in range(_lib.KERNEL_COUNT)}
        mask = 0
        for name in kernels:
            if name not in ids:
                raise ValueError(f"unknown kernel name {name!r}")
            mask |= 1 << ids[name]
        _lib.check("mok_workspace_set_timing_mask", lib().mok_workspace_set_timing_mask(self.handle, mask))

    def read_timing(self) -> dict:
        n = _lib.KERNEL_COUNT
        ms = (C.c_float * n)()
        cnt = (C.c_int64 * n)()
        _lib.check("mok_workspace_read_timing", lib().mok_workspace_read_timing(self.handle, ms, cnt, n))
        return {lib().mok_kernel_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(n) if cnt[i]}

    def read_status(self) -> tuple[int, int]:
        """(mover waits of the minibatch pipeline that ran out of time,
        launches given a schedule of another configuration) since the last
        call, both 0 in normal operation; synchronises the device. Does not
        raise on a mismatch: the count says it."""
        v, m = C.c_int32(0), C.c_int32(0)
        st = lib().mok_workspace_read_status(self.handle, C.byref(v), C.byref(m))
        if st not in (_lib.MOK_OK, _lib.MOK_ERR_CONFIG_MISMATCH):
            _lib.check("mok_workspace_read_status", st)
        return int(v.value), int(m.value)


def create_workspace(cfg: MoKConfig, device: int | None = None) -> Workspace:
    """A new workspace owned by the caller (not cached)."""
    return Workspace(cfg, device)


_CACHE: dict = {}


def get_workspace(cfg: MoKConfig, device: int | None = None) -> Workspace:
    """A workspace cached by (device, config): one per model, reused."""
    dev = torch.cuda.current_device() if device is None else int(device)
    key = (dev, cfg)
    ws = _CACHE.get(key)
    if ws is None:
        ws = _CACHE[key] = Workspace(cfg, dev)
    return ws


def clear_workspace_cache() -> None:
    for ws in list(_CACHE.values()):
        ws.close()
    _CACHE.clear()


def build_schedule(ws: Workspace, top_experts: torch.Tensor, schedule: torch.Tensor | None = None) -> torch.Tensor:
    """Schedule bytes (uint8 device tensor) for top_experts int64 [T, k]."""
    if top_experts.dtype != torch.int64 or top_experts.dim() != 2 or top_experts.shape[1] != ws.cfg.topk:
        raise ValueError("top_experts must be int64 [T, topk]")
    nb = ws.layout.total_bytes
    if schedule is None:
        schedule = torch.empty(nb, dtype=torch.uint8, device=top_experts.device)
    T = top_experts.shape[0]
    _lib.check("mok_build_schedule", lib().mok_build_schedule(
        ws.handle, _ptr(top_experts) if T else None, T, _ptr(schedule), schedule.numel(), _stream()))
    return schedule


def schedule_fields(ws: Workspace, schedule: torch.Tensor) -> dict:
    """Views of the schedule's int32 fields (device tensors)."""
    L, cfg = ws.layout, ws.cfg
    E = cfg.num_experts
    s32 = schedule.view(torch.int32)

    def f(off, n):
        return s32[off // 4: off // 4 + n]

    return dict(header=f(L.header, 16), counts=f(L.counts, E), kept=f(L.kept, E),
                offsets=f(L.offsets, E + 1), mb_offsets=f(L.mb_offsets, (L.n_mb_max + 1) * E),
                row_src=f(L.row_src, L.rows_cap_max), slot_row=f(L.slot_row, cfg.max_tokens * cfg.topk),
                tiles=f(L.tiles, len(TILE_BMS) * (E + 2)))


def _weights(w: dict) -> _lib.MokWeights:
    s = _lib.MokWeights()
    for name in ("routed_gate", "routed_up", "routed_down", "shared_gate", "shared_up", "shared_down"):
        setattr(s, name, _ptr(w.get(name)))
        setattr(s, name + "_scale", _ptr(w.get(name + "_scale")))
    return s


def forward(ws: Workspace, schedule: torch.Tensor, x: torch.Tensor, router_weights: torch.Tensor, weights: dict,
            mode: int = MOK_MODE_BF16, out: torch.Tensor | None = None, context: torch.Tensor | None = None
            ) -> torch.Tensor:
    """out bf16 [T, H]. ``weights``: routed_gate/up [E,I,H], routed_down
    [E,H,I], shared_* (bf16; or MXFP8 bytes with *_scale entries). Pass a
    ``context`` (uint8, context_bytes) to keep activations for backward."""
    if x.dtype != torch.bfloat16 or router_weights.dtype != torch.float32:
        raise ValueError("x must be bf16 and router_weights fp32")
    if out is None:
        out = torch.empty_like(x)
    ws_w = _weights(weights)
    _lib.check("mok_forward", lib().mok_forward(
        ws.handle, mode, _ptr(schedule), schedule.numel(), _ptr(x), _ptr(router_weights), C.byref(ws_w),
        _ptr(out), _ptr(context), 0 if context is None else context.numel(), _stream()))
    return out


def forward_static(cfg: MoKConfig, schedule: torch.Tensor, x: torch.Tensor, router_weights: torch.Tensor,
                   weights: dict, mode: int = MOK_MODE_BF16, out: torch.Tensor | None = None) -> torch.Tensor:
    """The inference forward (no context) of ``forward`` without a
    workspace: its scratch is the library's fixed device array (128 MiB per
    GPU), so nothing is allocated on the device. Runs on the current device;
    ``schedule`` comes from ``build_schedule`` with a workspace of the same
    config. Raises MokError (MOK_ERR_UNSUPPORTED) when the config needs more
    scratch than the array holds. Calls that overlap on one GPU race."""
    if x.dtype != torch.bfloat16 or router_weights.dtype != torch.float32:
        raise ValueError("x must be bf16 and router_weights fp32")
    if out is None:
        out = torch.empty_like(x)
    c = cfg.c()
    ws_w = _weights(weights)
    _lib.check("mok_forward_static", lib().mok_forward_static(
        C.byref(c), mode, _ptr(schedule), schedule.numel(), _ptr(x), _ptr(router_weights), C.byref(ws_w),
        _ptr(out), _stream()))
    return out


def backward(ws: Workspace, schedule: torch.Tensor, context: torch.Tensor, grad_out: torch.Tensor,
             x: torch.Tensor, router_weights: torch.Tensor, weights: dict, mode: int = MOK_MODE_BF16,
             grads: dict | None = None) -> dict:
    """Gradients: dx, d_router_weights, d_routed_gate/up/down, d_shared_*."""
    cfg = ws.cfg
    E, H, I, Is, k = cfg.num_experts, cfg.hidden, cfg.intermediate, cfg.shared_intermediate, cfg.topk
    T = x.shape[0]
    dev = x.device
    if grads is None:
        bf = dict(dtype=torch.bfloat16, device=dev)
        grads = dict(dx=torch.empty(T, H, **bf),
                     d_router_weights=torch.empty(T, k, dtype=torch.float32, device=dev),
                     d_routed_gate=torch.empty(E, I, H, **bf), d_routed_up=torch.empty(E, I, H, **bf),
                     d_routed_down=torch.empty(E, H, I, **bf))
        if Is:
            grads.update(d_shared_gate=torch.empty(Is, H, **bf), d_shared_up=torch.empty(Is, H, **bf),
                         d_shared_down=torch.empty(H, Is, **bf))
    g = _lib.MokGrads()
    for name, _ in _lib.MokGrads._fields_:
        setattr(g, name, _ptr(grads.get(name)))
    ws_w = _weights(weights)
    _lib.check("mok_backward", lib().mok_backward(
        ws.handle, mode, _ptr(schedule), schedule.numel(), _ptr(context), context.numel(), _ptr(grad_out),
        _ptr(x), _ptr(router_weights), C.byref(ws_w), C.byref(g), _stream()))
    return grads


def mxfp8_quantize(src: torch.Tensor, axis: int = 1, out: torch.Tensor | None = None,
                   scale: torch.Tensor | None = None):
    """MXFP8-quantize a 2-D (or flattened-to-2-D) bf16/fp32 device tensor in
    blocks of 32 along ``axis`` (1: along a row, 0: down a column).
    Returns (E4M3 codes uint8 with src's shape, E8M0 scales uint8)."""
    if src.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("src must be bf16 or fp32")
    shape = src.shape
    s2 = src.reshape(-1, shape[-1])
    rows, cols = s2.shape
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=src.device)
    if scale is None:
        sshape = (rows, cols // 32) if axis == 1 else (rows // 32, cols)
        scale = torch.empty(sshape, dtype=torch.uint8, device=src.device)
    _lib.check("mok_mxfp8_quantize", lib().mok_mxfp8_quantize(
        _ptr(s2), int(src.dtype == torch.float32), rows, cols, cols, axis, _ptr(out), cols, _ptr(scale), _stream()))
    return out, scale


def mxfp8_quantize_transposed(src: torch.Tensor, out: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """Transpose the last two dimensions of a bf16 device tensor [..., R, C]
    (a weight, or a batch of them) and MXFP8-quantize it along the new rows
    (blocks of 32 along R). Returns (codes uint8 [..., C, R], scales uint8
    [..., C, R/32])."""
    if src.dtype != torch.bfloat16:
        raise ValueError("src must be bf16")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    R, Cc = src.shape[-2], src.shape[-1]
    B = src.numel() // (R * Cc) if src.numel() else 0
    lead = tuple(src.shape[:-2])
    if out is None:
        out = torch.empty(lead + (Cc, R), dtype=torch.uint8, device=src.device)
    if scale is None:
        scale = torch.empty(lead + (Cc, R // 32), dtype=torch.uint8, device=src.device)
    _lib.check("mok_mxfp8_quantize_transposed", lib().mok_mxfp8_quantize_transposed(
        _ptr(src), B, R, Cc, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def mxfp8_backward_weights(weights: dict) -> dict:
    """The BF16 weights in the form the MXFP8 backward takes them
    pre-quantized (see include/mok.h, mok_backward): each transposed and
    quantized along the backward GEMM's contraction, with *_scale entries."""
    q = {}
    for name, t in weights.items():
        if t is None or name.endswith("_scale"):
            continue
        q[name], q[name + "_scale"] = mxfp8_quantize_transposed(t)
    return q
