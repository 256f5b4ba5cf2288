"""The autograd layer (``mixture_experts_layer_build_amd.autograd``) on the
GPU.

Its outputs and gradients are the library's: bit-identical to calling
mok_build_schedule / mok_forward / mok_backward directly. Those calls are
themselves checked against the oracle in test_gpu_forward*.py and
test_gpu_backward*.py, and one case here also goes to the oracle directly.
What is specific to the wrapper:
- every float input gets its gradient, and the integer ids none;
- inference (no grad) keeps no context, and its output is the same;
- activation checkpointing (recompute in backward) and CPU offload of the
  saved tensors give the same bits, since the layer is deterministic and the
  schedule and context go through the saved-tensor hooks;
- two stacked layers share one cached workspace between their forwards and
  backwards;
- in MXFP8 mode the quantized weights are reused until a parameter changes in
  place, and made again after;
- an empty batch gives empty outputs and all-zero weight gradients;
- a training step (forward and backward) captured in one graph replays to
  the eager step's bits."""
import numpy as np
import pytest

from mokutil import TOL_BF16, assert_close_inf, f64, to_dev

from oracle import moe as omoe
from workloads import CONFIGS, MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402
from mixture_experts_layer_build_amd.autograd import MoKExperts, MoKRuntime, moe_layer  # noqa: E402

NAMES = ("shared_gate", "shared_up", "shared_down", "routed_gate", "routed_up", "routed_down")


def bits(t):
    return t.detach().contiguous().view(torch.uint8)


def same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(bits(a), bits(b)), what


def leaves(d: dict, grad: bool = True) -> dict:
    w = {n: (d["weights"].get(n).clone().requires_grad_(grad) if d["weights"].get(n) is not None else None)
         for n in NAMES}
    return dict(x=d["x"].clone().requires_grad_(grad), rw=d["router_weights"].clone().requires_grad_(grad),
                top=d["top_experts"], w=w)


def run_layer(rt: MoKRuntime, L: dict):
    w = L["w"]
    return moe_layer(rt, L["x"], L["rw"], L["top"], *[w[n] for n in NAMES])


def grads_of(L: dict) -> dict:
    g = dict(dx=L["x"].grad, d_router_weights=L["rw"].grad)
    for n in NAMES:
        if L["w"][n] is not None:
            g["d_" + n] = L["w"][n].grad
    return g


def direct(cfg: mok.MoKConfig, d: dict, mode: int):
    """The same layer through the binding's direct calls (no autograd)."""
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.empty(mok.context_bytes(cfg, mode), dtype=torch.uint8, device="cuda")
    w = d["weights"]
    wf = w
    if mode == mok.MOK_MODE_MXFP8:
        wf = {}
        for n, t in w.items():
            codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
            wf[n], wf[n + "_scale"] = codes.view(t.shape), sc
    out = mok.forward(ws, sched, d["x"], d["router_weights"], wf, mode=mode, context=ctx)
    g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], w, mode=mode)
    torch.cuda.synchronize()
    return out, g


def shape_cfg(c: MoEShape, mult: float = 1.0) -> mok.MoKConfig:
    return mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                         shared_intermediate=c.I_s, capacity_multiplier=mult)


CASES = [
    # name, T, H, I, E, k, I_s, mult, mxfp8
    ("bf16_ragged", 300, 256, 256, 5, 3, 128, 1.0, False),
    ("bf16_drops_no_shared", 257, 384, 192, 4, 2, 0, 0.4, False),
    ("mxfp8_ragged", 300, 256, 256, 5, 3, 128, 1.0, True),
    ("mxfp8_many_experts", 513, 128, 128, 40, 4, 128, 1.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_autograd_matches_direct_calls(case):
    name, T, H, I, E, k, Is, mult, mx = case
    mode = mok.MOK_MODE_MXFP8 if mx else mok.MOK_MODE_BF16
    c = MoEShape(name, T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=131, w_std=0.05, passes="fwd+bwd",
                 mode="mxfp8" if mx else "bf16")
    d = to_dev(make_inputs(c))
    print(f"autograd vs direct {name}", flush=True)
    cfg = shape_cfg(c, mult)
    ref_out, ref_g = direct(cfg, d, mode)
    L = leaves(d)
    out = run_layer(MoKRuntime(cfg, mode), L)
    out.backward(d["grad_out"])
    torch.cuda.synchronize()
    same(out, ref_out, "out")
    g = grads_of(L)
    assert set(g) == set(ref_g), (set(g), set(ref_g))
    for n in ref_g:
        same(g[n], ref_g[n], n)
    assert L["top"].grad is None


def test_autograd_bf16_against_oracle():
    # one case straight to the float64 oracle as well (forward and backward)
    c = MoEShape("oracle", T=300, H=256, I=192, E=5, k=3, I_s=128, seed=133, w_std=0.05, passes="fwd+bwd")
    inp = make_inputs(c)
    d = to_dev(inp)
    L = leaves(d)
    out = run_layer(MoKRuntime(shape_cfg(c)), L)
    out.backward(d["grad_out"])
    torch.cuda.synchronize()
    a = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
         f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    ref_out = omoe.forward(*a)
    assert_close_inf(out.detach().float().cpu().numpy().astype(np.float64), ref_out, TOL_BF16, "out")
    ref = omoe.backward(f64(inp["grad_out"]), *a)
    g = grads_of(L)
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"), ("d_shared_gate", "d_s_gate"),
                         ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
        assert_close_inf(g[gname].float().cpu().numpy().astype(np.float64), ref[rname], TOL_BF16, gname)


def test_autograd_saves_flat_tensors_only():
    c = MoEShape("saved", T=200, H=256, I=128, E=4, k=2, I_s=64, seed=135, w_std=0.05, passes="fwd+bwd")
    d = to_dev(make_inputs(c))
    cfg = shape_cfg(c)
    L = leaves(d)
    out = run_layer(MoKRuntime(cfg), L)
    fn = out.grad_fn
    # nothing but saved tensors holds a tensor on the autograd context
    assert not any(isinstance(v, torch.Tensor) for v in vars(fn).values())
    saved = fn.saved_tensors
    assert saved[0].dtype == torch.uint8 and saved[0].numel() == mok.schedule_bytes(cfg)
    assert saved[1].dtype == torch.uint8 and saved[1].numel() == mok.context_bytes(cfg)
    out.backward(d["grad_out"])


def test_autograd_inference_and_partial_grads():
    c = MoEShape("partial", T=300, H=256, I=192, E=5, k=3, I_s=128, seed=137, w_std=0.05, passes="fwd+bwd")
    d = to_dev(make_inputs(c))
    cfg = shape_cfg(c)
    rt = MoKRuntime(cfg)
    ref_out, ref_g = direct(cfg, d, mok.MOK_MODE_BF16)
    # no grad at all: no context kept, same output
    with torch.no_grad():
        out = run_layer(rt, leaves(d))
    assert out.grad_fn is None
    same(out, ref_out, "inference out")
    L = leaves(d, grad=False)
    out = run_layer(rt, L)
    assert out.grad_fn is None
    same(out, ref_out, "no-requires-grad out")
    # only x needs a gradient
    L = leaves(d, grad=False)
    L["x"].requires_grad_(True)
    out = run_layer(rt, L)
    out.backward(d["grad_out"])
    same(L["x"].grad, ref_g["dx"], "dx")
    assert all(L["w"][n].grad is None for n in NAMES) and L["rw"].grad is None
    # a float32 loss upstream: grad_out arrives as bf16 of the same values
    L = leaves(d)
    out = run_layer(rt, L)
    (out.float() * d["grad_out"].float()).sum().backward()
    g = grads_of(L)
    for n in ref_g:
        same(g[n], ref_g[n], "via float loss: " + n)


def test_autograd_checkpoint_and_cpu_offload():
    c = MoEShape("ckpt", T=300, H=256, I=192, E=5, k=3, I_s=128, seed=139, w_std=0.05, passes="fwd+bwd")
    d = to_dev(make_inputs(c))
    rt = MoKRuntime(shape_cfg(c))

    def plain():
        L = leaves(d)
        out = run_layer(rt, L)
        out.backward(d["grad_out"])
        return out.detach(), grads_of(L)

    ref_out, ref_g = plain()
    # activation checkpointing: the forward runs again inside backward
    L = leaves(d)
    w = L["w"]
    out = torch.utils.checkpoint.checkpoint(lambda x, rw, *ws: moe_layer(rt, x, rw, L["top"], *ws),
                                            L["x"], L["rw"], *[w[n] for n in NAMES], use_reentrant=False)
    out.backward(d["grad_out"])
    same(out, ref_out, "checkpoint out")
    g = grads_of(L)
    for n in ref_g:
        same(g[n], ref_g[n], "checkpoint " + n)
    # the saved schedule and context go through saved-tensor hooks: offload
    # them to host memory and back
    packed = []

    def pack(t):
        packed.append((t.dtype, t.numel()))
        return t.to("cpu")

    def unpack(t):
        return t.to("cuda")

    L = leaves(d)
    with torch.autograd.graph.saved_tensors_hooks(pack, unpack):
        out = run_layer(rt, L)
    out.backward(d["grad_out"])
    g = grads_of(L)
    for n in ref_g:
        same(g[n], ref_g[n], "offload " + n)
    cfg = rt.cfg
    assert (torch.uint8, mok.schedule_bytes(cfg)) in packed
    assert (torch.uint8, mok.context_bytes(cfg)) in packed


def test_autograd_two_layers_share_the_workspace():
    # two layers of one shape: both forwards run before both backwards on the
    # one cached workspace; the result equals each layer run on its own
    c = MoEShape("stack", T=300, H=256, I=192, E=5, k=3, I_s=128, seed=141, w_std=0.05, passes="fwd+bwd")
    d1 = to_dev(make_inputs(c))
    d2 = to_dev(make_inputs(c.with_(seed=142)))
    cfg = shape_cfg(c)
    rt1, rt2 = MoKRuntime(cfg), MoKRuntime(cfg)
    assert rt1.workspace(d1["x"].device) is rt2.workspace(d1["x"].device)
    L1, L2 = leaves(d1), leaves(d2)
    y1 = run_layer(rt1, L1)
    L2["x"] = y1
    y2 = run_layer(rt2, L2)
    y2.backward(d2["grad_out"])
    torch.cuda.synchronize()
    # layer 2 on its own, fed layer 1's output; then layer 1 fed layer 2's dx
    e2 = dict(d2, x=y1.detach())
    o2, g2 = direct(cfg, e2, mok.MOK_MODE_BF16)
    same(y2, o2, "layer 2 out")
    e1 = dict(d1, grad_out=g2["dx"])
    o1, g1 = direct(cfg, e1, mok.MOK_MODE_BF16)
    same(y1, o1, "layer 1 out")
    for n in g1:
        if n == "dx":
            same(L1["x"].grad, g1["dx"], "layer 1 dx")
        elif n == "d_router_weights":
            same(L1["rw"].grad, g1[n], "layer 1 d_router_weights")
            same(L2["rw"].grad, g2[n], "layer 2 d_router_weights")
        else:
            same(L1["w"][n[2:]].grad, g1[n], "layer 1 " + n)
            same(L2["w"][n[2:]].grad, g2[n], "layer 2 " + n)


def test_autograd_mxfp8_requantizes_changed_weights():
    c = MoEShape("requant", T=300, H=256, I=256, E=5, k=3, I_s=128, seed=143, w_std=0.05, passes="fwd+bwd",
                 mode="mxfp8")
    d = to_dev(make_inputs(c))
    cfg = shape_cfg(c)
    rt = MoKRuntime(cfg, mok.MOK_MODE_MXFP8)
    L = leaves(d)
    out1 = run_layer(rt, L)
    out1.backward(d["grad_out"])  # also makes the backward's transposed codes
    codes1 = {n: rt._q[n][3] for n in rt._q}  # keyed (name, transposed)
    assert {n for n, _ in codes1} == set(NAMES) and {t for _, t in codes1} == {False, True}
    out1b = run_layer(rt, L)
    out1b.backward(d["grad_out"])
    # unchanged weights: the cached codes are reused
    assert all(rt._q[n][3] is codes1[n] for n in codes1)
    same(out1b, out1, "repeat")
    for t in [L["x"], L["rw"]] + [L["w"][n] for n in NAMES]:
        t.grad = None
    # an optimizer-like in-place step on two weights: their codes are made again
    with torch.no_grad():
        L["w"]["routed_up"].mul_(0.5)
        L["w"]["shared_down"].add_(0.01)
    out2 = run_layer(rt, L)
    # the forward's codes are made again for the changed weights only
    assert rt._q[("routed_up", False)][3] is not codes1[("routed_up", False)]
    assert rt._q[("shared_down", False)][3] is not codes1[("shared_down", False)]
    assert rt._q[("routed_gate", False)][3] is codes1[("routed_gate", False)]
    e = dict(d, weights={n: L["w"][n].detach() for n in NAMES})
    ref_out, ref_g = direct(cfg, e, mok.MOK_MODE_MXFP8)
    same(out2, ref_out, "after the step")
    out2.backward(d["grad_out"])
    # the backward's transposed codes are made again for the changed weights only
    assert rt._q[("routed_up", True)][3] is not codes1[("routed_up", True)]
    assert rt._q[("shared_down", True)][3] is not codes1[("shared_down", True)]
    assert rt._q[("routed_gate", True)][3] is codes1[("routed_gate", True)]
    g = grads_of(L)
    # the gradients of this call only (the earlier ones were cleared)
    for n in ref_g:
        same(g[n], ref_g[n], "after the step " + n)


def test_autograd_empty_batch():
    c = MoEShape("empty", T=64, H=256, I=128, E=4, k=2, I_s=64, seed=145, w_std=0.05, passes="fwd+bwd")
    d = to_dev(make_inputs(c))
    rt = MoKRuntime(shape_cfg(c))
    L = leaves(d)
    L["x"] = L["x"].detach()[:0].clone().requires_grad_(True)
    L["rw"] = L["rw"].detach()[:0].clone().requires_grad_(True)
    L["top"] = L["top"][:0].clone()
    out = run_layer(rt, L)
    assert out.shape == (0, c.H)
    out.backward(torch.zeros(0, c.H, dtype=torch.bfloat16, device="cuda"))
    assert L["x"].grad.shape == (0, c.H) and L["rw"].grad.shape == (0, c.k)
    for n in NAMES:
        assert torch.count_nonzero(L["w"][n].grad) == 0, n


def test_experts_module_8192_tokens_mxfp8():
    # the module at the 8192-token MXFP8 training shape (128 experts, top-8,
    # shared expert): output and every gradient equal the direct calls'
    c = CONFIGS["t8192_mxfp8_fwdbwd"]
    d = to_dev(make_inputs(c))
    print("8192-token module inputs ready", flush=True)
    m = MoKExperts(c.H, c.I, c.E, c.k, c.T, shared_intermediate=c.I_s, mode=mok.MOK_MODE_MXFP8, device="cuda")
    with torch.no_grad():
        m.routed_gate_weights.copy_(d["weights"]["routed_gate"])
        m.routed_up_weights.copy_(d["weights"]["routed_up"])
        m.routed_down_weights.copy_(d["weights"]["routed_down"])
    x = d["x"].clone().requires_grad_(True)
    rw = d["router_weights"].clone().requires_grad_(True)
    sw = {n: d["weights"][n].clone().requires_grad_(True) for n in ("shared_gate", "shared_up", "shared_down")}
    out = m(x, rw, d["top_experts"], sw["shared_gate"], sw["shared_up"], sw["shared_down"])
    out.backward(d["grad_out"])
    torch.cuda.synchronize()
    ref_out, ref_g = direct(shape_cfg(c), d, mok.MOK_MODE_MXFP8)
    same(out, ref_out, "out")
    same(x.grad, ref_g["dx"], "dx")
    same(rw.grad, ref_g["d_router_weights"], "d_router_weights")
    same(m.routed_gate_weights.grad, ref_g["d_routed_gate"], "d_routed_gate")
    same(m.routed_up_weights.grad, ref_g["d_routed_up"], "d_routed_up")
    same(m.routed_down_weights.grad, ref_g["d_routed_down"], "d_routed_down")
    for n in sw:
        same(sw[n].grad, ref_g["d_" + n], "d_" + n)


def test_autograd_training_step_graph_replay():
    # forward and backward captured in one graph (warm-up on a side stream
    # first, as whole-network capture needs); every replay, with eager steps
    # and synchronisations between replays, gives the eager step's bits
    c = MoEShape("graph", T=300, H=256, I=256, E=5, k=3, I_s=128, seed=151, w_std=0.05, passes="fwd+bwd")
    d = to_dev(make_inputs(c))
    rt = MoKRuntime(shape_cfg(c))
    L = leaves(d)
    params = [L["x"], L["rw"]] + [L["w"][n] for n in NAMES]

    def step():
        for t in params:
            t.grad = None
        y = run_layer(rt, L)
        y.backward(d["grad_out"])
        return y

    ref_y = step().detach().clone()
    ref_g = {n: g.clone() for n, g in grads_of(L).items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for t in params:
        t.grad = None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_static = run_layer(rt, L)
        y_static.backward(d["grad_out"])
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        same(y_static, ref_y, f"replay {rep} out")
        for n, gr in grads_of(L).items():
            same(gr, ref_g[n], f"replay {rep} {n}")
        # eager work between replays (its own gradients are set aside)
        saved = [t.grad for t in params]
        eager = run_layer(rt, leaves(d, grad=False))
        torch.cuda.synchronize()
        same(eager, ref_y, f"eager between replays {rep}")
        for t, gr in zip(params, saved):
            t.grad = gr
