"""Edge cases of the whole path against the oracle: a batch smaller than the
workspace's max_tokens (BF16 and MXFP8, forward and backward), an empty
batch (no tokens: empty outputs, every weight gradient exactly zero),
router weights of zero (the output is the shared expert alone), and expert
paddings that do not divide the 256-row GEMM tile (96, 160) or exceed it
(512)."""
import numpy as np
import pytest

from mokutil import TOL_BF16, TOL_MXFP8, assert_close_inf, f64, to_dev

from oracle import moe as omoe
from workloads import MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def quantize_weights(wdev: dict) -> dict:
    q = {}
    for name, t in wdev.items():
        codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
        q[name] = codes.view(t.shape)
        q[name + "_scale"] = sc
    return q


def run(c: MoEShape, inp: dict, T_max: int, mxfp8: bool, expert_pad: int = 32):
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=T_max,
                        shared_intermediate=c.I_s, expert_pad=expert_pad)
    ws = mok.Workspace(cfg)
    mode = mok.MOK_MODE_MXFP8 if mxfp8 else mok.MOK_MODE_BF16
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.empty(mok.context_bytes(cfg, mode), dtype=torch.uint8, device="cuda")
    w_fwd = quantize_weights(d["weights"]) if mxfp8 else d["weights"]
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w_fwd, mode=mode, context=ctx)
    g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"], mode=mode)
    torch.cuda.synchronize()
    return out, g


@pytest.mark.parametrize("mxfp8", [False, True], ids=["bf16", "mxfp8"])
def test_batch_smaller_than_max_tokens(mxfp8):
    # 37 tokens in a workspace sized for 1000
    c = MoEShape("small_batch", T=37, H=256, I=128, E=5, k=2, I_s=128, seed=41, w_std=0.05,
                 mode="mxfp8" if mxfp8 else "bf16", passes="fwd+bwd")
    inp = make_inputs(c)
    out, g = run(c, inp, 1000, mxfp8)
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
            f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    tol = TOL_MXFP8 if mxfp8 else TOL_BF16
    ref_out = omoe.forward_mxfp8(*args) if mxfp8 else omoe.forward(*args)
    assert_close_inf(np64(out), ref_out, tol, "out")
    ref = omoe.backward_mxfp8(f64(inp["grad_out"]), *args) if mxfp8 else omoe.backward(f64(inp["grad_out"]), *args)
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"), ("d_shared_gate", "d_s_gate"),
                         ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
        assert_close_inf(np64(g[gname]), ref[rname], tol, gname)


@pytest.mark.parametrize("mxfp8", [False, True], ids=["bf16", "mxfp8"])
def test_empty_batch(mxfp8):
    H, I, E, k, Is = 256, 128, 4, 2, 128
    rng = np.random.default_rng(3)
    dev = "cuda"
    cfg = mok.MoKConfig(hidden=H, intermediate=I, num_experts=E, topk=k, max_tokens=64, shared_intermediate=Is)
    ws = mok.Workspace(cfg)
    mode = mok.MOK_MODE_MXFP8 if mxfp8 else mok.MOK_MODE_BF16
    w = {"routed_gate": torch.from_numpy(rng.normal(0, 0.05, (E, I, H)).astype(np.float32)),
         "routed_up": torch.from_numpy(rng.normal(0, 0.05, (E, I, H)).astype(np.float32)),
         "routed_down": torch.from_numpy(rng.normal(0, 0.05, (E, H, I)).astype(np.float32)),
         "shared_gate": torch.from_numpy(rng.normal(0, 0.05, (Is, H)).astype(np.float32)),
         "shared_up": torch.from_numpy(rng.normal(0, 0.05, (Is, H)).astype(np.float32)),
         "shared_down": torch.from_numpy(rng.normal(0, 0.05, (H, Is)).astype(np.float32))}
    w = {n: t.to(torch.bfloat16).to(dev) for n, t in w.items()}
    x = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    top = torch.empty((0, k), dtype=torch.int64, device=dev)
    rw = torch.empty((0, k), dtype=torch.float32, device=dev)
    go = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    sched = mok.build_schedule(ws, top)
    ctx = torch.empty(mok.context_bytes(cfg, mode), dtype=torch.uint8, device=dev)
    out = mok.forward(ws, sched, x, rw, quantize_weights(w) if mxfp8 else w, mode=mode, context=ctx)
    # gradient buffers start non-zero: the backward must write every element
    grads = {"dx": torch.empty((0, H), dtype=torch.bfloat16, device=dev),
             "d_router_weights": torch.empty((0, k), dtype=torch.float32, device=dev)}
    for n, t in w.items():
        grads["d_" + n] = torch.full_like(t, 7.0)
    g = mok.backward(ws, sched, ctx, go, x, rw, w, mode=mode, grads=grads)
    torch.cuda.synchronize()
    assert out.shape == (0, H) and g["dx"].shape == (0, H) and g["d_router_weights"].shape == (0, k)
    for n in w:
        assert not torch.any(g["d_" + n] != 0), n


def test_zero_router_weights_leave_the_shared_expert():
    c = MoEShape("zero_w", T=300, H=256, I=128, E=6, k=3, I_s=128, seed=42, w_std=0.05)
    inp = make_inputs(c)
    inp["router_weights"] = np.zeros_like(inp["router_weights"])
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    out = mok.forward(ws, sched, d["x"], d["router_weights"], d["weights"])
    torch.cuda.synchronize()
    ref = omoe.forward(f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]),
                       f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]),
                       f64(inp["s_down"]))
    assert_close_inf(np64(out), ref, TOL_BF16, "out")
    shared_only = omoe.forward(f64(inp["x"]), np.full_like(inp["top_experts"], -1), inp["router_weights"],
                               f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]),
                               f64(inp["s_up"]), f64(inp["s_down"]))
    assert_close_inf(np64(out), shared_only, TOL_BF16, "shared only")


@pytest.mark.parametrize("E", [300, 1024])
@pytest.mark.parametrize("mode", ["bf16", "mxfp8"])
def test_more_experts_than_the_lds_tables_hold(mode, E):
    # 300 and 1024 experts (the largest a workspace takes): the grouped GEMM
    # reads its tile tables from global memory
    # (natural tile order) instead of LDS; forward and backward in both
    # modes against the oracle
    c = MoEShape("many", T=2 * E, H=128, I=128, E=E, k=2, I_s=128, seed=161, w_std=0.05, passes="fwd+bwd",
                 mode=mode)
    inp = make_inputs(c)
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s)
    ws = mok.Workspace(cfg)
    m = mok.MOK_MODE_MXFP8 if mode == "mxfp8" else mok.MOK_MODE_BF16
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.empty(mok.context_bytes(cfg, m), dtype=torch.uint8, device="cuda")
    w = d["weights"]
    if mode == "mxfp8":
        q = {}
        for n, t in w.items():
            codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
            q[n], q[n + "_scale"] = codes.view(t.shape), sc
        w = q
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=m, context=ctx)
    torch.cuda.synchronize()
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
            f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    ref = omoe.forward_mxfp8(*args) if mode == "mxfp8" else omoe.forward(*args)
    assert_close_inf(np64(out), ref, TOL_MXFP8 if mode == "mxfp8" else TOL_BF16, f"E={E} {mode} out")
    g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"], mode=m)
    torch.cuda.synchronize()
    if mode == "mxfp8":
        rg = omoe.backward_mxfp8(f64(inp["grad_out"]), *args)
    else:
        rg = omoe.backward(f64(inp["grad_out"]), *args)
    tol = TOL_MXFP8 if mode == "mxfp8" else TOL_BF16
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"),
                         ("d_shared_gate", "d_s_gate"), ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
        assert_close_inf(np64(g[gname]), rg[rname], tol, f"E={E} {mode} {gname}")


@pytest.mark.parametrize("pad", [96, 160, 512])
@pytest.mark.parametrize("mxfp8", [False, True], ids=["bf16", "mxfp8"])
def test_expert_pad_not_dividing_the_tile(mxfp8, pad):
    # Expert 0 gets exactly 250 rows and expert 1 exactly 260: with P = 96
    # their segments are padded to 288 rows, past one 256-row tile while the
    # kept rows of expert 0 fit in one; P = 512 pads every segment past two
    # tiles. Forward and backward against the oracle with the same padding.
    T, H, I, E, k, Is = 640, 256, 128, 4, 2, 128
    c = MoEShape("pad", T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=97, w_std=0.05,
                 mode="mxfp8" if mxfp8 else "bf16", passes="fwd+bwd")
    inp = make_inputs(c)
    top = np.empty((T, k), np.int64)
    top[:, 0] = np.where(np.arange(T) < 250, 0, 2)
    top[:, 1] = np.where(np.arange(T) < 260, 1, 3)
    inp["top_experts"] = top
    print(f"expert pad {pad} {'mxfp8' if mxfp8 else 'bf16'}", flush=True)
    out, g = run(c, inp, T, mxfp8, expert_pad=pad)
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
            f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    tol = TOL_MXFP8 if mxfp8 else TOL_BF16
    ref_out = (omoe.forward_mxfp8 if mxfp8 else omoe.forward)(*args, expert_pad=pad)
    assert_close_inf(np64(out), ref_out, tol, "out")
    ref = (omoe.backward_mxfp8 if mxfp8 else omoe.backward)(f64(inp["grad_out"]), *args, expert_pad=pad)
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"), ("d_shared_gate", "d_s_gate"),
                         ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
        assert_close_inf(np64(g[gname]), ref[rname], tol, f"pad {pad} {gname}")


def _limit_in_a_gap(target: float, inp: dict, mult: float, mxfp8: bool) -> tuple[float, float]:
    """A limit near ``target`` with no gate or up value of the batch within
    the widest margin found: the clamp is a decision the kernel takes on fp32
    accumulations and the oracle on float64, so a value within rounding of L
    could be clamped on one side only. Returns (limit, margin)."""
    from oracle import mxfp8 as omx
    from oracle.schedule import build_schedule
    q = (lambda v, a: omx.qdq(v, a)) if mxfp8 else (lambda v, a: v)  # noqa: E731
    x = q(f64(inp["x"]), 1)
    E = inp["w_gate"].shape[0]
    s = build_schedule(inp["top_experts"], E, mult, 32)
    vals = []
    for e in range(E):
        rows, _, t = omoe.segment_rows(s, e)
        vals += [(x[t] @ q(f64(inp["w_gate"][e]), 1).T).ravel(), np.abs(x[t] @ q(f64(inp["w_up"][e]), 1).T).ravel()]
    if inp.get("s_gate") is not None:
        vals += [(x @ q(f64(inp["s_gate"]), 1).T).ravel(), np.abs(x @ q(f64(inp["s_up"]), 1).T).ravel()]
    v = np.sort(np.concatenate(vals))
    cand = np.linspace(0.9 * target, 1.1 * target, 4001)
    idx = np.clip(np.searchsorted(v, cand), 1, v.size - 1)
    margin = np.minimum(np.abs(v[idx] - cand), np.abs(v[idx - 1] - cand))
    best = int(np.argmax(margin))
    return float(np.float32(cand[best])), float(margin[best])


@pytest.mark.parametrize("limit", [0.35, 1.0])
@pytest.mark.parametrize("mxfp8", [False, True], ids=["bf16", "mxfp8"])
def test_swiglu_limit(mxfp8, limit):
    # h = silu(min(g, L)) * clamp(u, -L, L); gradients blocked where a clamp
    # is active. With L = 0.35 about a quarter of the gate values and half of
    # the up values are clamped (both have a spread of ~0.56 here), with
    # L = 1.0 4 % and 7 %. Each limit is moved to a gap of the batch's gate
    # and up values (within 10 %), so no clamp decision hangs on rounding.
    c = MoEShape("limit", T=160, H=256, I=256, E=4, k=2, I_s=128, seed=99, w_std=0.035,
                 mode="mxfp8" if mxfp8 else "bf16", passes="fwd+bwd")
    inp = make_inputs(c)
    limit, margin = _limit_in_a_gap(limit, inp, 1.0, mxfp8)
    assert margin > 1e-5, margin  # far above fp32 accumulation error (~1e-6) at these sizes
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s, swiglu_limit=limit)
    ws = mok.Workspace(cfg)
    mode = mok.MOK_MODE_MXFP8 if mxfp8 else mok.MOK_MODE_BF16
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.empty(mok.context_bytes(cfg, mode), dtype=torch.uint8, device="cuda")
    w_fwd = quantize_weights(d["weights"]) if mxfp8 else d["weights"]
    print(f"swiglu limit {limit} (margin {margin:.2e}) {'mxfp8' if mxfp8 else 'bf16'}", flush=True)
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w_fwd, mode=mode, context=ctx)
    g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"], mode=mode)
    torch.cuda.synchronize()
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
            f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    tol = TOL_MXFP8 if mxfp8 else TOL_BF16
    ref_out = (omoe.forward_mxfp8 if mxfp8 else omoe.forward)(*args, swiglu_limit=limit)
    assert_close_inf(np64(out), ref_out, tol, "out")
    # the limit changes the result well beyond the tolerance
    free = (omoe.forward_mxfp8 if mxfp8 else omoe.forward)(*args)
    assert np.max(np.abs(free - ref_out)) > 4 * tol * np.max(np.abs(ref_out))
    ref = (omoe.backward_mxfp8 if mxfp8 else omoe.backward)(f64(inp["grad_out"]), *args, swiglu_limit=limit)
    for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                         ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"), ("d_shared_gate", "d_s_gate"),
                         ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
        err, scale = assert_close_inf(np64(g[gname]), ref[rname], tol, f"limit {limit} {gname}")
        print(f"  {gname}: max err {err:.3g} of max {scale:.3g}", flush=True)


def test_schedule_of_another_configuration_is_refused_on_the_device():
    # Two configs with the same buffer sizes but different capacity
    # multipliers: a schedule built by one and handed to the other's forward
    # carries the other hash, so every launch of that forward does nothing
    # (the output keeps its sentinel) and the workspace counts the mismatches.
    c = MoEShape("hash", T=1000, H=256, I=128, E=4, k=2, I_s=128, seed=171, w_std=0.05)
    d = to_dev(make_inputs(c))
    base = dict(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T, shared_intermediate=c.I_s)
    ws_a = mok.Workspace(mok.MoKConfig(capacity_multiplier=1.0, **base))
    ws_b = mok.Workspace(mok.MoKConfig(capacity_multiplier=0.9, **base))
    assert ws_a.layout.total_bytes == ws_b.layout.total_bytes
    sched = mok.build_schedule(ws_a, d["top_experts"])
    out = torch.full_like(d["x"], 3.0)
    mok.forward(ws_b, sched, d["x"], d["router_weights"], d["weights"], out=out)
    timeouts, mismatches = ws_b.read_status()
    assert timeouts == 0 and mismatches >= 3  # gate/up, down, combine
    assert torch.all(out == 3.0)
    assert ws_b.read_status() == (0, 0)  # the counts were reset
    # the matching workspace runs it, and its status stays clean
    mok.forward(ws_a, sched, d["x"], d["router_weights"], d["weights"], out=out)
    assert ws_a.read_status() == (0, 0)
    assert not torch.all(out == 3.0)
