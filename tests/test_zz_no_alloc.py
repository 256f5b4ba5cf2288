"""mok_forward_static (the allocation-free forward: its scratch is the
library's fixed device array) against mok_forward with a workspace, through
the C ABI: bit-identical outputs on two calls in a row, the second with a
smaller batch, in BF16 and MXFP8; configs that need more scratch than the
array holds are rejected before anything runs."""
import numpy as np
import pytest

from mokutil import to_dev
from workloads import MoEShape, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402
from mixture_experts_layer_build_amd._lib import MOK_ERR_UNSUPPORTED  # noqa: E402


def quantize_weights(wdev: dict) -> dict:
    q = {}
    for name, t in wdev.items():
        codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
        q[name] = codes.view(t.shape)
        q[name + "_scale"] = sc
    return q


@pytest.mark.parametrize("mxfp8", [False, True], ids=["bf16", "mxfp8"])
def test_forward_static_matches_the_workspace_forward(mxfp8):
    # 1024 tokens of an 8192-token-shaped layer (H = 2048, I = I_s = 768,
    # 128 experts, top-8): 71 MiB of scratch in BF16, 64 MiB in MXFP8, under
    # the 128 MiB array
    T_max = 1024
    cfg = mok.MoKConfig(hidden=2048, intermediate=768, num_experts=128, topk=8, max_tokens=T_max,
                        shared_intermediate=768)
    ws = mok.Workspace(cfg)
    mode = mok.MOK_MODE_MXFP8 if mxfp8 else mok.MOK_MODE_BF16
    for call, T in enumerate((T_max, 300)):  # the second call with a smaller batch
        c = MoEShape("static", T=T, H=2048, I=768, E=128, k=8, I_s=768, seed=120 + call,
                     mode="mxfp8" if mxfp8 else "bf16")
        d = to_dev(make_inputs(c))
        w = quantize_weights(d["weights"]) if mxfp8 else d["weights"]
        sched = mok.build_schedule(ws, d["top_experts"])
        print(f"static forward call {call}: T={T} {'mxfp8' if mxfp8 else 'bf16'}", flush=True)
        want = mok.forward(ws, sched, d["x"], d["router_weights"], w, mode=mode)
        got = mok.forward_static(cfg, sched, d["x"], d["router_weights"], w, mode=mode)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {call}"


def test_forward_static_rejects_configs_beyond_its_scratch():
    cfg = mok.MoKConfig(hidden=2048, intermediate=768, num_experts=128, topk=8, max_tokens=8192,
                        shared_intermediate=768)
    x = torch.zeros((8192, 2048), dtype=torch.bfloat16, device="cuda")
    rw = torch.zeros((8192, 8), dtype=torch.float32, device="cuda")
    w = {"routed_gate": torch.zeros((128, 768, 2048), dtype=torch.bfloat16, device="cuda"),
         "routed_up": torch.zeros((128, 768, 2048), dtype=torch.bfloat16, device="cuda"),
         "routed_down": torch.zeros((128, 2048, 768), dtype=torch.bfloat16, device="cuda"),
         "shared_gate": torch.zeros((768, 2048), dtype=torch.bfloat16, device="cuda"),
         "shared_up": torch.zeros((768, 2048), dtype=torch.bfloat16, device="cuda"),
         "shared_down": torch.zeros((2048, 768), dtype=torch.bfloat16, device="cuda")}
    sched = torch.zeros(mok.schedule_bytes(cfg), dtype=torch.uint8, device="cuda")
    with pytest.raises(mok.MokError) as ei:
        mok.forward_static(cfg, sched, x, rw, w)
    assert ei.value.status == MOK_ERR_UNSUPPORTED
