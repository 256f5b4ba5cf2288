"""GPU parity of mok_backward (BF16) against the float64 oracle: every
gradient within max|err| <= 2e-2 * max|ref| of its tensor. The backward
reuses the schedule and the context saved by mok_forward.

Small cases are compared element by element over whole tensors (several
tiles, ragged expert segments, drops and invalid ids, a shared expert of
another width). The 32768-token workload runs at full size: its forward
output, dx and router-weight gradients of 1024 sampled tokens, and the whole
weight gradients of four routed experts and of the shared expert, against
the expert-grouped oracle restricted to those tokens and experts."""
import numpy as np
import pytest

from mokutil import TOL_BF16, Bf16Array, assert_close_inf, f64, to_dev

from oracle import moe as omoe
from oracle.schedule import build_schedule as oracle_schedule
from workloads import CONFIGS, MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def gpu_fwd_bwd(c: MoEShape, inp: dict, mult: float):
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s, capacity_multiplier=mult)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.empty(mok.context_bytes(cfg), dtype=torch.uint8, device="cuda")
    out = mok.forward(ws, sched, d["x"], d["router_weights"], d["weights"], context=ctx)
    g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"])
    torch.cuda.synchronize()
    return out, g, (ws, sched, ctx, d)


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


SMALL = [
    ("ragged", 300, 256, 256, 5, 3, 128, 1.0, False),
    ("drops_invalid", 300, 256, 192, 5, 3, 128, 0.3, True),
    ("no_shared", 200, 384, 320, 3, 2, 0, 1.0, False),
    ("many_experts", 513, 128, 64, 40, 4, 64, 1.0, True),
    ("deep", 130, 1024, 256, 4, 2, 512, 0.6, False),
    ("deep_experts", 1100, 512, 192, 2, 2, 64, 1.0, False),  # grouped tile order
]


@pytest.mark.parametrize("case", SMALL, ids=[s[0] for s in SMALL])
def test_backward_bf16_small(case):
    name, T, H, I, E, k, Is, mult, invalid = case
    c = MoEShape(name, T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=79, w_std=0.05, passes="fwd+bwd")
    inp = make_inputs(c)
    if invalid:
        top = inp["top_experts"].copy()
        top[::7, 0] = -1
        top[3::11, -1] = E + 3
        inp["top_experts"] = top
    print(f"backward small {name}", flush=True)
    _, g, _ = gpu_fwd_bwd(c, inp, mult)
    ref = omoe.backward(f64(inp["grad_out"]), f64(inp["x"]), inp["top_experts"], inp["router_weights"],
                        f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]),
                        f64(inp["s_up"]), f64(inp["s_down"]), capacity_multiplier=mult)
    pairs = [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
             ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down")]
    if Is:
        pairs += [("d_shared_gate", "d_s_gate"), ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]
    for gname, rname in pairs:
        err, scale = assert_close_inf(np64(g[gname]), ref[rname], TOL_BF16, f"{name}:{gname}")
        print(f"  {gname}: max err {err:.3g} of max {scale:.3g}")
    # dropped and invalid assignments get exactly zero router-weight gradient
    sched = oracle_schedule(inp["top_experts"], E, mult, 32)
    not_kept = sched["slot_row"].reshape(T, k) < 0
    assert np.all(np64(g["d_router_weights"])[not_kept] == 0.0)


def test_backward_bf16_tiny_workload():
    c = CONFIGS["tiny_bf16_fwd"].with_(passes="fwd+bwd")
    inp = make_inputs(c)
    _, g, _ = gpu_fwd_bwd(c, inp, 1.0)
    ref = omoe.backward(f64(inp["grad_out"]), f64(inp["x"]), inp["top_experts"], inp["router_weights"],
                        f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]))
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down")]:
        assert_close_inf(np64(g[gname]), ref[rname], TOL_BF16, gname)


def test_backward_bf16_deterministic():
    c = MoEShape("det", T=400, H=256, I=192, E=6, k=3, I_s=64, seed=12, w_std=0.05, passes="fwd+bwd")
    inp = make_inputs(c)
    _, g1, (ws, sched, ctx, d) = gpu_fwd_bwd(c, inp, 1.0)
    g1 = {k_: v.clone() for k_, v in g1.items()}
    g2 = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"])
    torch.cuda.synchronize()
    for k_ in g1:
        assert torch.equal(g1[k_].view(torch.uint8), g2[k_].view(torch.uint8)), k_


def test_backward_bf16_32768_tokens_full_size():
    """The 32768-token workload at full size: the forward output and the
    dx and router-weight gradients of 1024 sampled tokens, and the whole
    weight gradients of four routed experts and of the shared expert,
    against the expert-grouped float64 oracle (restricted to those tokens
    and experts, its schedule the whole batch's)."""
    c = CONFIGS["t32768_bf16_fwdbwd"]
    inp = make_inputs(c)
    print("generated 32768-token inputs", flush=True)
    out, g, _ = gpu_fwd_bwd(c, inp, c.capacity_multiplier)
    print("gpu forward+backward done", flush=True)
    rng = np.random.default_rng(4)
    toks = np.unique(np.concatenate([[0, c.T - 1], rng.choice(c.T, size=1022, replace=False)]))
    experts = [0, 11, 22, c.E - 1]
    wg, wu, wd = Bf16Array(inp["w_gate"]), Bf16Array(inp["w_up"]), Bf16Array(inp["w_down"])
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], wg, wu, wd,
            f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    ref_out = omoe.forward(*args, tokens=toks)
    err, scale = assert_close_inf(np64(out[toks]), ref_out[toks], TOL_BF16, "out")
    print(f"  out ({toks.size} tokens): max err {err:.3g} of max {scale:.3g}", flush=True)
    ref = omoe.backward(f64(inp["grad_out"]), *args, tokens=toks, dw_experts=experts + ["shared"])
    print("oracle backward done", flush=True)

    def check(got, want, name):
        err, scale = assert_close_inf(got, want, TOL_BF16, name)
        print(f"  {name}: max err {err:.3g} of max {scale:.3g}", flush=True)

    check(np64(g["dx"][toks]), ref["dx"][toks], f"dx ({toks.size} tokens)")
    check(np64(g["d_router_weights"][toks]), ref["d_router_weights"][toks], "d_router_weights")
    for gname, rname in (("d_routed_gate", "d_w_gate"), ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down")):
        check(np.stack([np64(g[gname][e]) for e in experts]), ref[rname][experts], f"{gname} experts {experts}")
    for gname, rname in (("d_shared_gate", "d_s_gate"), ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")):
        check(np64(g[gname]), ref[rname], gname)
    for k_, v in g.items():
        assert torch.isfinite(v.float()).all(), k_
