"""The forward's minibatch pipeline (one launch: compute workgroups run the
down tiles minibatch by minibatch, mover workgroups combine minibatch b once
all of its tiles are counted) gives the same bits as the single-pass forward, for ragged minibatches,
minibatches past the batch (T below max_tokens), no shared expert, many
experts, MXFP8 mode, and with a context kept for the backward; at 8192
tokens the pipelined output is also compared with the oracle on every
token."""
import numpy as np
import pytest

from mokutil import TOL_BF16, assert_close_inf, f64, to_dev
from oracle import moe as omoe
from workloads import CONFIGS, MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def run_forward(c: MoEShape, d: dict, T_max: int, mode: int, minibatch: int, movers: int, with_context: bool):
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=T_max,
                        shared_intermediate=c.I_s, capacity_multiplier=c.capacity_multiplier,
                        minibatch_size=minibatch, num_mover_wgs=movers)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    ctx = torch.zeros(mok.context_bytes(cfg, mode), dtype=torch.uint8, device="cuda") if with_context else None
    w = d["weights"]
    if mode == mok.MOK_MODE_MXFP8:
        q = {}
        for n, t in w.items():
            codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
            q[n] = codes.view(t.shape)
            q[n + "_scale"] = sc
        w = q
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=mode, context=ctx)
    out2 = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=mode, context=ctx)  # reuse the workspace
    torch.cuda.synchronize()
    assert ws.read_status() == (0, 0)  # no mover wait ran out of time; the schedule matched
    return out, out2, ctx


CASES = [
    # name, T, T_max, H, I, E, k, I_s, minibatch, movers, mxfp8, context
    ("ragged", 1000, 1000, 256, 256, 6, 3, 128, 300, 16, False, False),
    ("t_below_max", 500, 1000, 256, 256, 6, 3, 128, 256, 8, False, True),
    ("no_shared", 777, 777, 384, 256, 5, 2, 0, 200, 32, False, False),
    ("many_experts_mxfp8", 700, 700, 256, 256, 40, 4, 128, 128, 16, True, True),
    ("one_token_minibatches", 40, 40, 128, 128, 4, 2, 128, 1, 8, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_minibatch_pipeline_matches_single_pass(case):
    name, T, T_max, H, I, E, k, Is, mb, movers, mx, with_ctx = case
    c = MoEShape(name, T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=91, w_std=0.05, mode="mxfp8" if mx else "bf16")
    d = to_dev(make_inputs(c))
    mode = mok.MOK_MODE_MXFP8 if mx else mok.MOK_MODE_BF16
    print(f"minibatch pipeline {name}", flush=True)
    ref, _, ctx_ref = run_forward(c, d, T_max, mode, 0, 0, with_ctx)
    got, got2, ctx_got = run_forward(c, d, T_max, mode, mb, movers, with_ctx)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))
    if with_ctx:
        assert torch.equal(ctx_got, ctx_ref)


def test_minibatch_pipeline_8192_tokens():
    # bit-identical to the single pass, and every token against the oracle
    c = CONFIGS["t8192_bf16_fwd"]
    inp = make_inputs(c)
    d = to_dev(inp)
    ref, _, _ = run_forward(c, d, c.T, mok.MOK_MODE_BF16, 0, 0, False)
    got, got2, _ = run_forward(c, d, c.T, mok.MOK_MODE_BF16, 2048, 16, False)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))
    want = omoe.forward(f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]),
                        f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]),
                        f64(inp["s_down"]), capacity_multiplier=c.capacity_multiplier)
    err, scale = assert_close_inf(got.float().cpu().numpy().astype(np.float64), want, TOL_BF16, "pipeline out")
    print(f"pipeline at 8192 tokens: max err {err:.3g} of max {scale:.3g}", flush=True)


def test_minibatch_pipeline_graph_replay():
    # the pipelined forward captured in a graph: every replay (eager work and
    # synchronisations between them) matches the single-pass result
    c = MoEShape("graph", T=900, H=256, I=256, E=6, k=3, I_s=128, seed=17, w_std=0.05)
    d = to_dev(make_inputs(c))
    ref, _, _ = run_forward(c, d, c.T, mok.MOK_MODE_BF16, 0, 0, False)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s, minibatch_size=256, num_mover_wgs=16)
    ws = mok.Workspace(cfg)
    mok.build_schedule(ws, d["top_experts"])
    out = torch.zeros_like(ref)
    sbuf = torch.zeros(ws.layout.total_bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mok.build_schedule(ws, d["top_experts"], sbuf)
            mok.forward(ws, sbuf, d["x"], d["router_weights"], d["weights"], out=out)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        # eager work between replays
        eager, _, _ = run_forward(c, d, c.T, mok.MOK_MODE_BF16, 256, 16, False)
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))
    assert ws.read_status() == (0, 0)
