"""The forward's token ring (macrobatch_size < max_tokens, an inference
workspace): the batch streams through scratch sized for one macrobatch, pass
by pass, each pass running on a schedule cut out of the whole batch's. The
output is bit-identical to the one-pass forward for ragged last passes, a
batch shorter than max_tokens (passes with no tokens), capacity drops, no
shared expert, many experts, minibatch sub-offsets, MXFP8 mode and an empty
batch; the full-size workloads are compared with the one-pass forward and,
at 8192 tokens, every token with the oracle."""
import numpy as np
import pytest

from mokutil import TOL_BF16, assert_close_inf, f64, to_dev
from oracle import moe as omoe
from workloads import CONFIGS, MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def quantized(w: dict) -> dict:
    q = {}
    for n, t in w.items():
        codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
        q[n] = codes.view(t.shape)
        q[n + "_scale"] = sc
    return q


def run(c: MoEShape, d: dict, T_max: int, mode: int, macro: int, minibatch: int = 0, forward_only: int = 1):
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=T_max,
                        shared_intermediate=c.I_s, capacity_multiplier=c.capacity_multiplier,
                        minibatch_size=minibatch, num_mover_wgs=16 if minibatch else 0,
                        macrobatch_size=macro, forward_only=forward_only)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    w = quantized(d["weights"]) if mode == mok.MOK_MODE_MXFP8 else d["weights"]
    out = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=mode)
    out2 = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=mode)  # reuse the workspace
    torch.cuda.synchronize()
    assert ws.read_status() == (0, 0)
    return out, out2, sched, ws


CASES = [
    # name, T, T_max, H, I, E, k, I_s, capacity, macrobatch, minibatch, mxfp8
    ("ragged_last_pass", 2000, 2000, 256, 256, 6, 3, 128, 1.0, 768, 0, False),
    ("t_below_max", 1000, 2000, 256, 256, 6, 3, 128, 1.0, 768, 0, False),
    ("drops", 1500, 1500, 256, 256, 8, 2, 128, 0.3, 512, 0, False),
    ("no_shared", 777, 777, 384, 256, 5, 2, 0, 1.0, 200, 0, False),
    ("many_experts", 900, 900, 256, 256, 40, 4, 128, 0.6, 256, 0, False),
    ("minibatches", 1100, 1100, 256, 256, 6, 3, 128, 1.0, 512, 128, False),
    ("one_token_passes", 40, 40, 128, 128, 4, 2, 128, 1.0, 1, 0, False),
    ("mxfp8", 1300, 1300, 256, 256, 8, 4, 128, 0.8, 384, 0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_token_ring_matches_one_pass(case):
    name, T, T_max, H, I, E, k, Is, cap, macro, mb, mx = case
    c = MoEShape(name, T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=93, w_std=0.05, capacity_multiplier=cap,
                 mode="mxfp8" if mx else "bf16")
    d = to_dev(make_inputs(c))
    mode = mok.MOK_MODE_MXFP8 if mx else mok.MOK_MODE_BF16
    print(f"token ring {name}", flush=True)
    ref, _, _, _ = run(c, d, T_max, mode, 0, forward_only=0)
    got, got2, _, _ = run(c, d, T_max, mode, macro, mb)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))


def test_token_ring_empty_batch():
    c = MoEShape("empty", T=0, H=128, I=128, E=4, k=2, I_s=128, seed=5, w_std=0.05)
    d = to_dev(make_inputs(c))
    out, _, _, ws = run(c, d, 512, mok.MOK_MODE_BF16, 128)
    assert out.shape == (0, 128)


def test_token_ring_refuses_backward_context_and_foreign_schedule():
    c = MoEShape("refuse", T=600, H=128, I=128, E=4, k=2, I_s=128, seed=6, w_std=0.05)
    d = to_dev(make_inputs(c))
    _, _, sched, ws = run(c, d, 600, mok.MOK_MODE_BF16, 256)
    ctx = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(mok.MokError) as e:
        mok.forward(ws, sched, d["x"], d["router_weights"], d["weights"], context=ctx)
    assert e.value.status == mok._lib.MOK_ERR_UNSUPPORTED
    with pytest.raises(mok.MokError) as e:
        mok.backward(ws, sched, ctx, torch.zeros_like(d["x"]), d["x"], d["router_weights"], d["weights"])
    assert e.value.status == mok._lib.MOK_ERR_UNSUPPORTED
    # a schedule of the one-pass configuration: every pass's launches return
    # without writing, and the mismatch is counted
    cfg1 = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=600,
                         shared_intermediate=c.I_s)
    foreign = torch.zeros(ws.layout.total_bytes, dtype=torch.uint8, device="cuda")
    mok.build_schedule(mok.Workspace(cfg1), d["top_experts"], foreign)
    out = torch.full_like(d["x"], 7)
    mok.forward(ws, foreign, d["x"], d["router_weights"], d["weights"], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7)
    timeouts, mismatches = ws.read_status()
    assert timeouts == 0 and mismatches > 0


@pytest.mark.parametrize("name,macro", [("t8192_bf16_fwd", 2048), ("skew_bf16_fwd", 3000),
                                        ("t8192_mxfp8_fwd", 3000)])
def test_token_ring_full_size(name, macro):
    # bit-identical to the one pass; at 8192 tokens in BF16 also every token
    # against the oracle
    c = CONFIGS[name]
    inp = make_inputs(c)
    d = to_dev(inp)
    mode = mok.MOK_MODE_MXFP8 if c.mode == "mxfp8" else mok.MOK_MODE_BF16
    print(f"token ring {name} macrobatch {macro}", flush=True)
    ref, _, _, _ = run(c, d, c.T, mode, 0, forward_only=1)
    got, got2, _, _ = run(c, d, c.T, mode, macro)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))
    if name != "t8192_bf16_fwd":
        return
    want = omoe.forward(f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]),
                        f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]),
                        f64(inp["s_down"]), capacity_multiplier=c.capacity_multiplier)
    err, scale = assert_close_inf(got.float().cpu().numpy().astype(np.float64), want, TOL_BF16, "ring out")
    print(f"token ring at 8192 tokens: max err {err:.3g} of max {scale:.3g}", flush=True)
