"""GPU parity of mok_forward in MXFP8 mode against the oracle's MXFP8
emulation: max|err| <= 6e-2 * max|ref|. x is quantized on the device inside
the call; the weights are pre-quantized with mok_mxfp8_quantize (checked
bit-exact against the oracle quantizer here too). Small cases and the
8192-token workload at full size are compared over every token (the
oracle's weight quantization runs on slices in worker processes)."""
import numpy as np
import pytest

from mokutil import TOL_MXFP8, assert_close_inf, f64, oracle_qweights, to_dev

from oracle import moe as omoe
from oracle import mxfp8 as omx
from workloads import CONFIGS, MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402


def quantize_weights(wdev: dict, check_bits: dict | None = None) -> dict:
    """MXFP8 codes + scales of every weight along its last (contraction) dim."""
    q = {}
    for name, t in wdev.items():
        codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
        q[name] = codes.view(t.shape)
        q[name + "_scale"] = sc
        if check_bits is not None and name in check_bits:
            bits = check_bits[name]
            rc, rs = omx.quantize(f64(bits).reshape(-1, bits.shape[-1]), axis=1)
            np.testing.assert_array_equal(codes.cpu().numpy(), rc, err_msg=name)
            np.testing.assert_array_equal(sc.cpu().numpy(), rs, err_msg=name)
    return q


def gpu_forward_mxfp8(c: MoEShape, inp: dict, mult: float, check_bits=False):
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s, capacity_multiplier=mult)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    names = {"routed_gate": "w_gate", "routed_up": "w_up", "routed_down": "w_down",
             "shared_gate": "s_gate", "shared_up": "s_up", "shared_down": "s_down"}
    chk = {n: inp[names[n]] for n in d["weights"]} if check_bits else None
    wq = quantize_weights(d["weights"], chk)
    out = mok.forward(ws, sched, d["x"], d["router_weights"], wq, mode=mok.MOK_MODE_MXFP8)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


SMALL = [
    ("ragged", 300, 256, 256, 5, 3, 128, 1.0),
    ("drops_wide", 260, 384, 384, 4, 2, 0, 0.4),
    ("many_experts", 513, 128, 128, 40, 4, 128, 1.0),
    ("deep_k", 130, 1024, 256, 4, 2, 512, 1.0),
    ("deep_experts", 1100, 512, 256, 2, 2, 128, 1.0),  # grouped tile order
]


@pytest.mark.parametrize("case", SMALL, ids=[s[0] for s in SMALL])
def test_forward_mxfp8_small(case):
    name, T, H, I, E, k, Is, mult = case
    c = MoEShape(name, T=T, H=H, I=I, E=E, k=k, I_s=Is, seed=78, w_std=0.05, mode="mxfp8")
    inp = make_inputs(c)
    print(f"mxfp8 small {name}", flush=True)
    got = gpu_forward_mxfp8(c, inp, mult, check_bits=True)
    ref = omoe.forward_mxfp8(f64(inp["x"]), inp["top_experts"], inp["router_weights"], f64(inp["w_gate"]),
                             f64(inp["w_up"]), f64(inp["w_down"]), f64(inp["s_gate"]), f64(inp["s_up"]),
                             f64(inp["s_down"]), capacity_multiplier=mult)
    err, scale = assert_close_inf(got, ref, TOL_MXFP8, name)
    # the quantization is visible: the BF16-exact oracle differs from the MXFP8 one
    print(f"{name}: max err {err:.3g} of max {scale:.3g}")


def test_forward_mxfp8_8192_tokens_every_token():
    c = CONFIGS["t8192_mxfp8_fwd"]
    inp = make_inputs(c)
    got = gpu_forward_mxfp8(c, inp, c.capacity_multiplier)
    print("gpu forward done", flush=True)
    qw = oracle_qweights(inp)
    print("oracle weights quantized", flush=True)
    ref = omoe.forward_mxfp8(f64(inp["x"]), inp["top_experts"], inp["router_weights"], None, None, None,
                             qweights=qw, capacity_multiplier=c.capacity_multiplier,
                             s_gate=f64(inp["s_gate"]), s_up=f64(inp["s_up"]), s_down=f64(inp["s_down"]))
    err, scale = assert_close_inf(got, ref, TOL_MXFP8, c.name)
    print(f"{c.name}: all {c.T} tokens, max err {err:.3g} of max {scale:.3g}", flush=True)


def test_forward_mxfp8_rejects_unsupported_shapes():
    c = MoEShape("bad", T=64, H=128, I=64, E=2, k=1, I_s=0, seed=1)  # I % 128 != 0
    inp = make_inputs(c)
    d = to_dev(inp)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T)
    ws = mok.Workspace(cfg)
    sched = mok.build_schedule(ws, d["top_experts"])
    wq = quantize_weights(d["weights"])
    with pytest.raises(mok.MokError):
        mok.forward(ws, sched, d["x"], d["router_weights"], wq, mode=mok.MOK_MODE_MXFP8)
    w = dict(wq)
    del w["routed_gate_scale"]
    cfg2 = mok.MoKConfig(hidden=128, intermediate=128, num_experts=2, topk=1, max_tokens=64)
    ws2 = mok.Workspace(cfg2)
    with pytest.raises(mok.MokError):
        mok.forward(ws2, mok.build_schedule(ws2, d["top_experts"]), d["x"], d["router_weights"], w,
                    mode=mok.MOK_MODE_MXFP8)
