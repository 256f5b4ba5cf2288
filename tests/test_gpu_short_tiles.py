"""Segments whose last M tile has at most 64 rows run the gate/up K loop on
a three-stage ring of compact stages. Here the routing is chosen so that
segment sizes sit on both sides of that boundary (1, 31, 32, 33, 63, 64,
65, 127, 128, 129, 256, 262, 320, 321 rows) and the shared expert's last tile
has 40 rows. Outputs (and, in BF16, every gradient, which reads the G and U
the gate/up epilogue saved) are compared with the float64 oracle at H = 128,
the fewest K steps the contract allows (2 in BF16, 1 in MXFP8), and at
H = 384."""
import numpy as np
import pytest

from mokutil import TOL_BF16, TOL_MXFP8, assert_close_inf, f64, to_dev

from oracle import moe as omoe
from workloads import MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402

COUNTS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 256, 320, 321, 262]  # sum 1832 = 7 * 256 + 40


def crafted_inputs(H: int, I: int, mode: str, seed: int) -> tuple[MoEShape, dict]:
    T, E = sum(COUNTS), len(COUNTS)
    c = MoEShape("short", T=T, H=H, I=I, E=E, k=1, I_s=128, seed=seed, w_std=0.05, mode=mode, passes="fwd+bwd")
    inp = make_inputs(c)
    rng = np.random.default_rng(seed)
    ids = np.repeat(np.arange(E, dtype=np.int64), COUNTS)
    rng.shuffle(ids)  # each expert's rows are scattered tokens
    inp["top_experts"] = ids.reshape(T, 1)
    inp["router_weights"] = rng.uniform(0.25, 1.0, size=(T, 1)).astype(np.float32)
    return c, inp


def quantized(w: dict) -> dict:
    q = {}
    for n, t in w.items():
        codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
        q[n], q[n + "_scale"] = codes.view(t.shape), sc
    return q


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("H", [128, 384])
@pytest.mark.parametrize("mode", ["bf16", "mxfp8"])
def test_short_tile_boundaries(H, mode):
    c, inp = crafted_inputs(H, 128, mode, seed=200 + H)
    d = to_dev(inp)
    print(f"short tiles H={H} {mode}", flush=True)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=1, max_tokens=c.T,
                        shared_intermediate=c.I_s)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    kept = mok.schedule_fields(ws, sched)["kept"].cpu().numpy()
    assert list(kept) == COUNTS
    m = mok.MOK_MODE_MXFP8 if mode == "mxfp8" else mok.MOK_MODE_BF16
    ctx = torch.empty(mok.context_bytes(cfg, m), dtype=torch.uint8, device="cuda")
    w = quantized(d["weights"]) if mode == "mxfp8" else d["weights"]
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=m, context=ctx)
    torch.cuda.synchronize()
    args = (f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]), f64(inp["w_up"]),
            f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]), f64(inp["s_down"]))
    ref = omoe.forward_mxfp8(*args) if mode == "mxfp8" else omoe.forward(*args)
    assert_close_inf(np64(out), ref, TOL_MXFP8 if mode == "mxfp8" else TOL_BF16, f"out H={H} {mode}")
    if mode == "bf16":
        g = mok.backward(ws, sched, ctx, d["grad_out"], d["x"], d["router_weights"], d["weights"])
        torch.cuda.synchronize()
        rg = omoe.backward(f64(inp["grad_out"]), *args)
        for gname, rname in [("dx", "dx"), ("d_router_weights", "d_router_weights"), ("d_routed_gate", "d_w_gate"),
                             ("d_routed_up", "d_w_up"), ("d_routed_down", "d_w_down"),
                             ("d_shared_gate", "d_s_gate"), ("d_shared_up", "d_s_up"), ("d_shared_down", "d_s_down")]:
            assert_close_inf(np64(g[gname]), rg[rname], TOL_BF16, f"{gname} H={H}")
