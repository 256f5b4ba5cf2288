"""Pins for oracle.moe: dense-MLP special case via torch, two formulations,
equivariance, linearity, autograd and finite differences for the backward,
and structural checks of the MXFP8 emulation."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import moe, mxfp8
from oracle.schedule import build_schedule


def rand_case(seed, T=12, H=8, I=6, E=4, k=2, I_s=5, id_lo=0, id_hi=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    top = rng.integers(id_lo, E if id_hi is None else id_hi, size=(T, k)).astype(np.int64)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    Wg = rng.standard_normal((E, I, H)) * 0.5
    Wu = rng.standard_normal((E, I, H)) * 0.5
    Wd = rng.standard_normal((E, H, I)) * 0.5
    sh = (rng.standard_normal((I_s, H)) * 0.5, rng.standard_normal((I_s, H)) * 0.5,
          rng.standard_normal((H, I_s)) * 0.5) if I_s else (None, None, None)
    return x, top, w, Wg, Wu, Wd, sh


def test_single_expert_equals_dense_swiglu_mlp_torch():
    rng = np.random.default_rng(0)
    T, H, I = 9, 16, 12
    x = rng.standard_normal((T, H))
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((1, I, H), (1, I, H), (1, H, I)))
    top = np.zeros((T, 1), np.int64)
    w = np.ones((T, 1))
    out = moe.forward(x, top, w, Wg, Wu, Wd)
    xt = torch.from_numpy(x)
    ref = F.linear(F.silu(F.linear(xt, torch.from_numpy(Wg[0]))) * F.linear(xt, torch.from_numpy(Wu[0])),
                   torch.from_numpy(Wd[0])).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_shared_only_equals_dense_mlp_torch():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(1)
    out = moe.forward(x, top, np.zeros_like(w), Wg, Wu, Wd, Sg, Su, Sd)
    xt = torch.from_numpy(x)
    ref = F.linear(F.silu(F.linear(xt, torch.from_numpy(Sg))) * F.linear(xt, torch.from_numpy(Su)),
                   torch.from_numpy(Sd)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mult", [1.0, 0.3])
def test_grouped_equals_per_token_loop(seed, mult):
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(seed, id_lo=-1, id_hi=5)
    s = build_schedule(top, 4, mult, 4)
    a = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    b = moe.forward_per_token(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    c = moe.forward_tokens(range(x.shape[0]), x, top, w, Wg, Wu, Wd, Sg, Su, Sd, slot_row=s["slot_row"])
    np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-12)


def test_token_permutation_equivariance():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(3, T=20)
    perm = np.random.default_rng(9).permutation(20)
    a = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd)
    b = moe.forward(x[perm], top[perm], w[perm], Wg, Wu, Wd, Sg, Su, Sd)
    np.testing.assert_allclose(a[perm], b, rtol=1e-12, atol=1e-12)


def test_linearity_in_router_weights():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(4)
    shared = moe.forward(x, top, np.zeros_like(w), Wg, Wu, Wd, Sg, Su, Sd)
    a = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd) - shared
    b = moe.forward(x, top, 2.5 * w, Wg, Wu, Wd, Sg, Su, Sd) - shared
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-12, atol=1e-12)


def test_dropped_assignments_contribute_nothing():
    x, top, w, Wg, Wu, Wd, _ = rand_case(5, T=30, E=3)
    s = build_schedule(top, 3, 0.2, 2)
    assert s["dropped"] > 0
    w2 = w.copy().reshape(-1)
    w2[s["slot_row"] < 0] = 123.0          # weights of dropped slots must not matter
    a = moe.forward(x, top, w, Wg, Wu, Wd, sched=s)
    b = moe.forward(x, top, w2.reshape(w.shape), Wg, Wu, Wd, sched=s)
    np.testing.assert_array_equal(a, b)


def torch_forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, keep):
    """The layer written directly in torch ops (float64) for autograd."""
    T, k = top.shape
    out = torch.zeros_like(x)
    for j in range(k):
        for e in range(Wg.shape[0]):
            m = torch.from_numpy((top[:, j] == e) & keep[:, j])
            if not m.any():
                continue
            xs = x[m]
            h = F.silu(xs @ Wg[e].T) * (xs @ Wu[e].T)
            out = out.index_add(0, torch.nonzero(m)[:, 0], w[m, j:j + 1] * (h @ Wd[e].T))
    if Sg is not None:
        out = out + (F.silu(x @ Sg.T) * (x @ Su.T)) @ Sd.T
    return out


@pytest.mark.parametrize("mult", [1.0, 0.4])
def test_backward_matches_torch_autograd(mult):
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(6, T=16, id_lo=-1, id_hi=5)
    s = build_schedule(top, 4, mult, 4)
    keep = (s["slot_row"] >= 0).reshape(top.shape)
    rng = np.random.default_rng(11)
    dO = rng.standard_normal(x.shape)
    tens = [torch.tensor(a, requires_grad=True) for a in (x, w, Wg, Wu, Wd, Sg, Su, Sd)]
    out = torch_forward(tens[0], top, *tens[1:], keep)
    np.testing.assert_allclose(out.detach().numpy(), moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s),
                               rtol=1e-12, atol=1e-12)
    (out * torch.from_numpy(dO)).sum().backward()
    g = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    names = ["dx", "d_router_weights", "d_w_gate", "d_w_up", "d_w_down", "d_s_gate", "d_s_up", "d_s_down"]
    for n, t in zip(names, tens):
        np.testing.assert_allclose(g[n], t.grad.numpy(), rtol=1e-10, atol=1e-10, err_msg=n)


def test_backward_finite_differences():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(7, T=6, H=5, I=4, E=3, k=2, I_s=3)
    s = build_schedule(top, 3, 1.0, 2)
    dO = np.random.default_rng(12).standard_normal(x.shape)
    g = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    args = dict(x=x, w=w, Wg=Wg, Wu=Wu, Wd=Wd, Sg=Sg, Su=Su, Sd=Sd)
    gname = dict(x="dx", w="d_router_weights", Wg="d_w_gate", Wu="d_w_up", Wd="d_w_down",
                 Sg="d_s_gate", Su="d_s_up", Sd="d_s_down")

    def loss(a):
        return float(np.sum(dO * moe.forward(a["x"], top, a["w"], a["Wg"], a["Wu"], a["Wd"],
                                             a["Sg"], a["Su"], a["Sd"], sched=s)))
    rng = np.random.default_rng(13)
    eps = 1e-6
    for name, arr in args.items():
        for _ in range(4):
            idx = tuple(rng.integers(n) for n in arr.shape)
            p = {kk: vv.copy() for kk, vv in args.items()}
            m = {kk: vv.copy() for kk, vv in args.items()}
            p[name][idx] += eps
            m[name][idx] -= eps
            fd = (loss(p) - loss(m)) / (2 * eps)
            assert abs(fd - g[gname[name]][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


def _on_grid(v, axis):
    return mxfp8.qdq(v, axis)


def test_mxfp8_forward_reduces_to_forward_on_grid_inputs():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(8, T=10, H=64, I=32, E=3, k=2, I_s=32)
    x = _on_grid(x, 1)
    Wg, Wu, Wd = _on_grid(Wg, 2), _on_grid(Wu, 2), _on_grid(Wd, 2)
    Sg, Su, Sd = _on_grid(Sg, 1), _on_grid(Su, 1), _on_grid(Sd, 1)
    a = moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, quantize_h=False)
    b = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    # with h quantized the result moves, but only by h's rounding
    c = moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd)
    assert np.max(np.abs(c - b)) <= 0.1 * np.max(np.abs(b))


def test_mxfp8_backward_structure_with_identity_quantizer():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(9, T=10, H=64, I=32, E=3, k=2, I_s=32)
    s = build_schedule(top, 3, 1.0, 32)
    dO = np.random.default_rng(14).standard_normal(x.shape)
    ident = lambda v, axis=-1: np.asarray(v, np.float64)
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qfun=ident, saved=None)
    b = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    for n in b:
        np.testing.assert_allclose(a[n], b[n], rtol=1e-11, atol=1e-11, err_msg=n)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("mult", [1.0, 0.4])
def test_forward_tokens_mxfp8_equals_forward_mxfp8(seed, mult):
    rng = np.random.default_rng(100 + seed)
    T, H, I, E, k, Is = 10, 64, 32, 3, 2, 32
    x = rng.standard_normal((T, H))
    top = rng.integers(-1, E + 1, size=(T, k)).astype(np.int64)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    Wg, Wu = rng.standard_normal((E, I, H)) * 0.3, rng.standard_normal((E, I, H)) * 0.3
    Wd = rng.standard_normal((E, H, I)) * 0.3
    Sg, Su, Sd = rng.standard_normal((Is, H)) * 0.3, rng.standard_normal((Is, H)) * 0.3, rng.standard_normal((H, Is)) * 0.3
    s = build_schedule(top, E, mult, 32)
    a = moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    b = moe.forward_tokens_mxfp8(range(T), x, top, w, Wg, Wu, Wd, Sg, Su, Sd, slot_row=s["slot_row"])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("mult", [1.0, 0.4])
def test_backward_slices_equal_backward(seed, mult):
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(200 + seed, T=11, H=7, I=5, E=3, k=2, I_s=4, id_lo=-1, id_hi=4)
    dO = np.random.default_rng(300 + seed).standard_normal(x.shape)
    s = build_schedule(top, 3, mult, 32)
    full = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    cols = [(e, i) for e in range(3) for i in range(5)]
    sl = moe.backward_slices(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, slot_row=s["slot_row"],
                             tokens=range(11), expert_cols=cols, shared_cols=range(4))
    for t in range(11):
        np.testing.assert_allclose(sl["dx"][t], full["dx"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sl["d_router_weights"][t], full["d_router_weights"][t], rtol=1e-12, atol=1e-12)
    for (e, i) in cols:
        np.testing.assert_allclose(sl["d_w_gate_rows"][(e, i)], full["d_w_gate"][e][i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sl["d_w_up_rows"][(e, i)], full["d_w_up"][e][i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sl["d_w_down_cols"][(e, i)], full["d_w_down"][e][:, i], rtol=1e-12, atol=1e-12)
    for i in range(4):
        np.testing.assert_allclose(sl["d_s_gate_rows"][i], full["d_s_gate"][i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sl["d_s_up_rows"][i], full["d_s_up"][i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sl["d_s_down_cols"][i], full["d_s_down"][:, i], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("mult", [1.0, 0.4])
def test_backward_slices_mxfp8_equal_backward_mxfp8(seed, mult):
    # 70 tokens x top-2 over 3 experts: segments of more than one 32-row block;
    # I = 64 puts sampled columns in both 32-column blocks of h
    rng = np.random.default_rng(400 + seed)
    T, H, I, E, k, Is = 70, 64, 64, 3, 2, 32
    x = rng.standard_normal((T, H))
    top = rng.integers(-1, E + 1, size=(T, k)).astype(np.int64)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    Wg, Wu = rng.standard_normal((E, I, H)) * 0.3, rng.standard_normal((E, I, H)) * 0.3
    Wd = rng.standard_normal((E, H, I)) * 0.3
    Sg, Su, Sd = rng.standard_normal((Is, H)) * 0.3, rng.standard_normal((Is, H)) * 0.3, rng.standard_normal((H, Is)) * 0.3
    dO = rng.standard_normal((T, H))
    s = build_schedule(top, E, mult, 32)
    full = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    cols = [(e, i) for e in range(E) for i in (0, 31, 32, 63)]
    sl = moe.backward_slices_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, slot_row=s["slot_row"],
                                   tokens=range(T), expert_cols=cols, shared_cols=(0, 17, 31))
    tol = dict(rtol=1e-10, atol=1e-10)
    for t in range(T):
        np.testing.assert_allclose(sl["dx"][t], full["dx"][t], **tol)
        np.testing.assert_allclose(sl["d_router_weights"][t], full["d_router_weights"][t], **tol)
    for (e, i) in cols:
        np.testing.assert_allclose(sl["d_w_gate_rows"][(e, i)], full["d_w_gate"][e][i], **tol)
        np.testing.assert_allclose(sl["d_w_up_rows"][(e, i)], full["d_w_up"][e][i], **tol)
        np.testing.assert_allclose(sl["d_w_down_cols"][(e, i)], full["d_w_down"][e][:, i], **tol)
    for i in (0, 17, 31):
        np.testing.assert_allclose(sl["d_s_gate_rows"][i], full["d_s_gate"][i], **tol)
        np.testing.assert_allclose(sl["d_s_up_rows"][i], full["d_s_up"][i], **tol)
        np.testing.assert_allclose(sl["d_s_down_cols"][i], full["d_s_down"][:, i], **tol)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(21)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, size=100000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0, 1e-40]])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = moe.bf16_round(v)
    np.testing.assert_array_equal(got, ref)
    assert np.signbit(got[v.size - 5])


def test_mxfp8_backward_saved_context_rounding_only_touches_swiglu_derivative():
    # with an identity quantizer, rounding the saved g, u changes the result by
    # the bf16 rounding only (relative 2^-8), and saved=None gives backward()
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(19, T=10, H=64, I=32, E=3, k=2, I_s=32)
    s = build_schedule(top, 3, 1.0, 32)
    dO = np.random.default_rng(15).standard_normal(x.shape)
    ident = lambda v, axis=-1: np.asarray(v, np.float64)
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qfun=ident)
    b = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    for n in b:
        scale = np.max(np.abs(b[n]))
        assert np.max(np.abs(a[n] - b[n])) <= 2.0 ** -6 * scale, n
    # d_router_weights and dW_down do not use the derivative: unchanged
    np.testing.assert_allclose(a["d_router_weights"], b["d_router_weights"], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(a["d_w_down"], b["d_w_down"], rtol=1e-11, atol=1e-11)
