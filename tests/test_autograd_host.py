"""Host-side checks of the autograd layer: it imports and builds without a
GPU, rejects tensors on the CPU (there is no CPU fallback) and bad shapes,
dtypes and modes before touching the device."""
import pytest

torch = pytest.importorskip("torch")
import mixture_experts_layer_build_amd as mok  # noqa: E402
from mixture_experts_layer_build_amd.autograd import MoKExperts, MoKRuntime, moe_layer  # noqa: E402

H, I, E, K, IS, T = 64, 32, 4, 2, 32, 16


def inputs(**over):
    d = dict(x=torch.zeros(T, H, dtype=torch.bfloat16), rw=torch.full((T, K), 0.5),
             top=torch.zeros(T, K, dtype=torch.int64),
             sg=torch.zeros(IS, H, dtype=torch.bfloat16), su=torch.zeros(IS, H, dtype=torch.bfloat16),
             sd=torch.zeros(H, IS, dtype=torch.bfloat16))
    d.update(over)
    return d


def test_module_builds_on_the_host():
    m = MoKExperts(H, I, E, K, max_tokens=T, shared_intermediate=IS)
    m.init_weights(0.02, generator=torch.Generator().manual_seed(3))
    assert m.routed_gate_weights.shape == (E, I, H) and m.routed_down_weights.shape == (E, H, I)
    assert m.routed_gate_weights.dtype == torch.bfloat16
    std = float(m.routed_up_weights.float().std())
    assert 0.015 < std < 0.025
    assert "experts=4" in repr(m)
    assert [n for n, _ in m.named_parameters()] == ["routed_gate_weights", "routed_up_weights",
                                                    "routed_down_weights"]


@pytest.mark.parametrize("grad", [False, True])
def test_cpu_tensors_are_rejected(grad):
    m = MoKExperts(H, I, E, K, max_tokens=T, shared_intermediate=IS)
    d = inputs()
    x = d["x"].requires_grad_(grad)
    with pytest.raises(ValueError, match="CUDA"):
        m(x, d["rw"], d["top"], d["sg"], d["su"], d["sd"])


def test_bad_arguments_are_rejected_before_the_device():
    rt = MoKRuntime(mok.MoKConfig(hidden=H, intermediate=I, num_experts=E, topk=K, max_tokens=T,
                                  shared_intermediate=IS))
    m = MoKExperts(H, I, E, K, max_tokens=T, shared_intermediate=IS)
    w = (m.routed_gate_weights, m.routed_up_weights, m.routed_down_weights)
    d = inputs()
    with pytest.raises(ValueError, match="bfloat16"):
        moe_layer(rt, d["x"].float(), d["rw"], d["top"], d["sg"], d["su"], d["sd"], *w)
    with pytest.raises(ValueError, match="shape"):
        moe_layer(rt, d["x"], d["rw"][:, :1].contiguous(), d["top"], d["sg"], d["su"], d["sd"], *w)
    with pytest.raises(ValueError, match=r"\[tokens, hidden\]"):
        moe_layer(rt, d["x"].unsqueeze(0), d["rw"], d["top"], d["sg"], d["su"], d["sd"], *w)
    with pytest.raises(ValueError, match="int64"):
        moe_layer(rt, d["x"], d["rw"], d["top"].int(), d["sg"], d["su"], d["sd"], *w)
    with pytest.raises(ValueError, match="required"):
        moe_layer(rt, d["x"], d["rw"], d["top"], None, d["su"], d["sd"], *w)
    rt0 = MoKRuntime(mok.MoKConfig(hidden=H, intermediate=I, num_experts=E, topk=K, max_tokens=T))
    with pytest.raises(ValueError, match="shared_intermediate = 0"):
        moe_layer(rt0, d["x"], d["rw"], d["top"], d["sg"], d["su"], d["sd"], *w)
    with pytest.raises(ValueError, match="must be one of|MOK_MODE"):
        MoKRuntime(rt.cfg, mode=7)
