"""Pins for oracle.moe: dense-MLP special case via torch, two formulations,
equivariance, linearity, autograd and finite differences for the backward,
and checks of the MXFP8 emulation: its GEMM structure (identity quantizer),
the blocking axis of every quantized operand (a table of each GEMM's
contraction dimension), and properties that hold only when every operand is
blocked along its own GEMM's contraction dimension (per-token locality,
dead-row perturbations, exact power-of-two equivariance)."""
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


def torch_forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, keep, limit=None):
    """The layer written directly in torch ops (float64) for autograd; with
    a limit, SwiGLU's inputs go through torch.clamp."""
    def act(g, u):
        if limit is None:
            return F.silu(g) * u
        return F.silu(torch.clamp(g, max=limit)) * torch.clamp(u, -limit, limit)
    T, k = top.shape
    out = torch.zeros_like(x)
    for j in range(k):
        for e in range(Wg.shape[0]):
            m = torch.from_numpy((top[:, j] == e) & keep[:, j])
            if not m.any():
                continue
            xs = x[m]
            h = act(xs @ Wg[e].T, xs @ Wu[e].T)
            out = out.index_add(0, torch.nonzero(m)[:, 0], w[m, j:j + 1] * (h @ Wd[e].T))
    if Sg is not None:
        out = out + act(x @ Sg.T, x @ Su.T) @ Sd.T
    return out


@pytest.mark.parametrize("mult,limit", [(1.0, None), (0.4, None), (1.0, 0.8), (0.4, 1.5)])
def test_backward_matches_torch_autograd(mult, limit):
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(6, T=16, id_lo=-1, id_hi=5)
    s = build_schedule(top, 4, mult, 4)
    keep = (s["slot_row"] >= 0).reshape(top.shape)
    rng = np.random.default_rng(11)
    dO = rng.standard_normal(x.shape)
    tens = [torch.tensor(a, requires_grad=True) for a in (x, w, Wg, Wu, Wd, Sg, Su, Sd)]
    out = torch_forward(tens[0], top, *tens[1:], keep, limit=limit)
    np.testing.assert_allclose(out.detach().numpy(),
                               moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, swiglu_limit=limit),
                               rtol=1e-12, atol=1e-12)
    if limit is not None:  # the limit is active on a good share of the inputs
        g_all = np.concatenate([(x @ Wg[e].T).ravel() for e in range(4)])
        u_all = np.concatenate([(x @ Wu[e].T).ravel() for e in range(4)])
        assert np.mean(g_all > limit) > 0.1 and np.mean(np.abs(u_all) > limit) > 0.1
    (out * torch.from_numpy(dO)).sum().backward()
    g = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, swiglu_limit=limit)
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
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qfun=ident)
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



# ---------------------------------------------------------------------------
# MXFP8: every operand blocked along its own GEMM's contraction dimension
# ---------------------------------------------------------------------------

def _axis_case(seed=31):
    # distinct sizes (H = 64, I = 96, I_s = 160) and kept counts that are not
    # multiples of 32, so that every (shape, blocked axis) pair names one
    # operand class
    rng = np.random.default_rng(seed)
    T, H, I, E, k, Is = 45, 64, 96, 3, 2, 160
    x = rng.standard_normal((T, H))
    top = np.stack([np.arange(T) % 3, (np.arange(T) + 1) % 3], axis=1).astype(np.int64)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    Wg, Wu = rng.standard_normal((E, I, H)) * 0.3, rng.standard_normal((E, I, H)) * 0.3
    Wd = rng.standard_normal((E, H, I)) * 0.3
    Sg, Su = rng.standard_normal((Is, H)) * 0.3, rng.standard_normal((Is, H)) * 0.3
    Sd = rng.standard_normal((H, Is)) * 0.3
    dO = rng.standard_normal((T, H))
    return (T, H, I, E, k, Is), x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO


def _recording_qdq():
    calls = []

    def q(v, axis):
        v = np.asarray(v, np.float64)
        calls.append((tuple(v.shape), axis % v.ndim))
        return mxfp8.qdq(v, axis)
    return q, calls


def test_mxfp8_every_operand_blocked_along_its_contraction_dimension():
    """The blocked axis of every quantizer call, against a table written from
    the rule "each GEMM's operands are blocked along that GEMM's contraction
    dimension": gate/up contracts over H, down over I, dh over H, dA over I,
    the weight gradients over an expert's rows (32-row blocks of its
    zero-padded segment). A swapped axis anywhere changes the multiset."""
    from collections import Counter
    (T, H, I, E, k, Is), x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO = _axis_case()
    s = build_schedule(top, E, 1.0, 32)
    n = [int(v) for v in s["kept"]]
    assert all(v % 32 for v in n) and T % 32
    pad = lambda m: -(-m // 32) * 32  # noqa: E731
    want = Counter()
    # forward GEMMs (recomputed inside the backward): gate/up over H, down over I
    want[((T, H), 1)] += 1                  # x, gate/up A operand
    want[((E, I, H), 2)] += 2               # W_g, W_u, gate/up B operands
    want[((Is, H), 1)] += 2                 # S_g, S_u
    for ne in n:
        want[((ne, I), 1)] += 1             # h of the routed rows (down's A operand)
    want[((T, Is), 1)] += 1                 # h of the shared expert
    # dh = grad_out rows . W_d, over H
    want[((E, H, I), 1)] += 1               # W_d blocked along H
    want[((H, Is), 0)] += 1                 # S_d blocked along H
    for ne in n:
        want[((ne, H), 1)] += 1             # grad_out rows of the expert
    want[((T, H), 1)] += 1                  # grad_out rows of the shared expert
    # dA = dG . W_g + dU . W_u, over I
    want[((E, I, H), 1)] += 2               # W_g, W_u blocked along I
    want[((Is, H), 0)] += 2                 # S_g, S_u blocked along I_s
    for ne in n:
        want[((ne, I), 1)] += 2             # dG, dU rows
    want[((T, Is), 1)] += 2
    # weight gradients, over the rows of each (padded) segment
    for ne in n:
        want[((pad(ne), H), 0)] += 2        # w * grad_out rows (dW_down), x rows (dW_gate, dW_up)
        want[((pad(ne), I), 0)] += 3        # h (dW_down), dG (dW_gate), dU (dW_up)
    want[((pad(T), H), 0)] += 2
    want[((pad(T), Is), 0)] += 3
    q, calls = _recording_qdq()
    moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qfun=q)
    assert Counter(calls) == want, (Counter(calls) - want, want - Counter(calls))


def _fwd_mx(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, s):
    return moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)


def test_mxfp8_forward_token_locality():
    """out[t] depends on x only through x[t]: x is blocked along H and h
    along I, both inside one token's row. Blocks of 32 rows would couple the
    tokens sharing a block (the 45 tokens span two such blocks)."""
    _, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, _ = _axis_case(32)
    s = build_schedule(top, 3, 1.0, 32)
    a = _fwd_mx(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, s)
    for t0 in (0, 7, 40):
        x2 = x.copy()
        x2[t0] *= 37.0  # moves every block maximum of that row
        b = _fwd_mx(x2, top, w, Wg, Wu, Wd, Sg, Su, Sd, s)
        others = np.arange(x.shape[0]) != t0
        np.testing.assert_array_equal(a[others], b[others])
        assert np.max(np.abs(a[t0] - b[t0])) > 0


def test_mxfp8_forward_weight_rows_are_blocked_along_h_and_down_rows_along_i():
    """Gate/up weights blocked along H: with W_u[e, i] = 0 (so h_i = 0
    whatever g_i is), rescaling W_g[e, i] by a non-power of two leaves the
    output unchanged, and likewise W_u[e, i] with W_g[e, i] = 0; blocked along I, the other rows of its 32-row block
    would be requantized. Down weights blocked along I: rescaling row h' of
    W_d[e] moves only output column h'."""
    _, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, _ = _axis_case(33)
    s = build_schedule(top, 3, 1.0, 32)
    Wu = Wu.copy()
    Wu[1, 5] = 0.0
    Su = Su.copy()
    Su[70] = 0.0
    a = _fwd_mx(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, s)
    Wg2, Sg2 = Wg.copy(), Sg.copy()
    Wg2[1, 5] *= 23.0
    Sg2[70] *= 23.0
    np.testing.assert_array_equal(a, _fwd_mx(x, top, w, Wg2, Wu, Wd, Sg2, Su, Sd, s))
    # and the other way round: W_g[e, i] = 0 (g_i = 0, so h_i = 0), W_u[e, i] rescaled
    Wg3, Sg3 = Wg.copy(), Sg.copy()
    Wg3[2, 50] = 0.0
    Sg3[3] = 0.0
    a3 = _fwd_mx(x, top, w, Wg3, Wu, Wd, Sg3, Su, Sd, s)
    Wu3, Su3 = Wu.copy(), Su.copy()
    Wu3[2, 50] *= 23.0
    Su3[3] *= 23.0
    np.testing.assert_array_equal(a3, _fwd_mx(x, top, w, Wg3, Wu3, Wd, Sg3, Su3, Sd, s))
    Wd2, Sd2 = Wd.copy(), Sd.copy()
    Wd2[2, 9] *= 23.0
    Sd2[9] *= 23.0
    b = _fwd_mx(x, top, w, Wg, Wu, Wd2, Sg, Su, Sd2, s)
    cols = np.arange(x.shape[1]) != 9
    np.testing.assert_array_equal(a[:, cols], b[:, cols])
    assert np.max(np.abs(a[:, 9] - b[:, 9])) > 0


def test_mxfp8_backward_token_locality():
    """dx[t] and the router-weight gradients of t depend on grad_out only
    through grad_out[t]: grad_out rows are blocked along H and dG, dU along
    I. 32-row blocks of either would couple tokens."""
    _, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO = _axis_case(34)
    s = build_schedule(top, 3, 1.0, 32)
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    for t0 in (3, 33):
        d2 = dO.copy()
        d2[t0] *= 37.0
        b = moe.backward_mxfp8(d2, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
        others = np.arange(x.shape[0]) != t0
        for n in ("dx", "d_router_weights"):
            np.testing.assert_array_equal(a[n][others], b[n][others])
            assert np.max(np.abs(a[n][t0] - b[n][t0])) > 0


def test_mxfp8_backward_down_weight_columns_are_blocked_along_h():
    """dh = grad_out rows . W_d contracts over H, so W_d is blocked along H
    (within one column i). With row i of W_g and W_u zero (g_i = u_i = 0,
    hence h_i = dG_i = dU_i = 0 whatever dh_i is), rescaling column i of
    W_d[e] leaves dx and the router-weight gradients unchanged; blocked
    along I, the rest of its row block would be requantized."""
    _, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO = _axis_case(35)
    s = build_schedule(top, 3, 1.0, 32)
    Wg, Wu, Sg, Su = Wg.copy(), Wu.copy(), Sg.copy(), Su.copy()
    Wg[0, 40] = Wu[0, 40] = 0.0
    Sg[100] = Su[100] = 0.0
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    Wd2, Sd2 = Wd.copy(), Sd.copy()
    Wd2[0, :, 40] *= 23.0
    Sd2[:, 100] *= 23.0
    b = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd2, Sg, Su, Sd2, sched=s)
    for n in ("dx", "d_router_weights", "d_w_gate", "d_w_up", "d_s_gate", "d_s_up"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def test_mxfp8_backward_down_weight_gradient_rows_scale_with_grad_out_columns():
    """dW_down = Q_r(w * grad_out rows)^T Q_r(h) contracts over rows: the
    blocks of the grad_out operand run down one column. Doubling column h' of
    grad_out (a power of two: quantization commutes exactly) doubles row h'
    of every dW_down and leaves the other rows bit-identical; blocks along H
    would requantize the rest of the row block."""
    _, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO = _axis_case(36)
    s = build_schedule(top, 3, 1.0, 32)
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    d2 = dO.copy()
    d2[:, 17] *= 2.0
    b = moe.backward_mxfp8(d2, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    rows = np.arange(x.shape[1]) != 17
    np.testing.assert_array_equal(a["d_w_down"][:, rows], b["d_w_down"][:, rows])
    np.testing.assert_array_equal(2.0 * a["d_w_down"][:, 17], b["d_w_down"][:, 17])
    np.testing.assert_array_equal(a["d_s_down"][rows], b["d_s_down"][rows])
    np.testing.assert_array_equal(2.0 * a["d_s_down"][17], b["d_s_down"][17])


# ---------------------------------------------------------------------------
# Restricted forms used by the full-size GPU checks
# ---------------------------------------------------------------------------

def test_token_and_expert_restrictions_equal_the_whole_computation():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(41, T=40, H=6, I=5, E=4, k=2, I_s=3, id_lo=-1, id_hi=5)
    dO = np.random.default_rng(42).standard_normal(x.shape)
    s = build_schedule(top, 4, 0.4, 2)
    toks = [0, 3, 17, 39]
    full = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    part = moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, tokens=toks)
    np.testing.assert_allclose(part[toks], full[toks], rtol=1e-12, atol=1e-12)
    assert not np.any(np.delete(part, toks, axis=0))
    fb = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    pb = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, tokens=toks, dw_experts=[1, "shared"])
    for n in ("dx", "d_router_weights"):
        np.testing.assert_allclose(pb[n][toks], fb[n][toks], rtol=1e-12, atol=1e-12)
    for n in ("d_w_gate", "d_w_up", "d_w_down"):
        np.testing.assert_allclose(pb[n][1], fb[n][1], rtol=1e-12, atol=1e-12)
    for n in ("d_s_gate", "d_s_up", "d_s_down"):
        np.testing.assert_allclose(pb[n], fb[n], rtol=1e-12, atol=1e-12)


def test_mxfp8_restrictions_and_prequantized_weights_equal_the_whole_computation():
    (T, H, I, E, k, Is), x, top, w, Wg, Wu, Wd, Sg, Su, Sd, dO = _axis_case(43)
    s = build_schedule(top, E, 0.5, 32)
    toks = [1, 2, 30, 44]
    full = moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    qf = moe.quantize_weights_mxfp8(Wg, Wu, Wd, Sg, Su, Sd)
    part = moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qweights=qf, tokens=toks)
    np.testing.assert_array_equal(part[toks], full[toks])
    np.testing.assert_array_equal(moe.forward_mxfp8(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qweights=qf), full)
    fb = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s)
    qb = moe.quantize_weights_mxfp8(Wg, Wu, Wd, Sg, Su, Sd, for_backward=True)
    pb = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qweights=qb, tokens=toks,
                            dw_experts=[2, "shared"])
    for n in ("dx", "d_router_weights"):
        np.testing.assert_array_equal(pb[n][toks], fb[n][toks])
    for n in ("d_w_gate", "d_w_up", "d_w_down"):
        np.testing.assert_array_equal(pb[n][2], fb[n][2])
    for n in ("d_s_gate", "d_s_up", "d_s_down"):
        np.testing.assert_array_equal(pb[n], fb[n])


def test_parallel_quantizer_equals_one_call():
    from mokutil import par_qdq
    rng = np.random.default_rng(44)
    for shape, axis in (((3, 64, 1 << 15), 2), ((3, 1 << 15, 64), 1), ((1 << 17, 64), 0), ((64, 1 << 17), 1)):
        v = rng.standard_normal(shape) * 10.0 ** rng.integers(-3, 3, size=shape[-1])
        np.testing.assert_array_equal(par_qdq(v, axis), mxfp8.qdq(v, axis))



# ---------------------------------------------------------------------------
# SwiGLU input limit
# ---------------------------------------------------------------------------

def test_swiglu_limit_dense_mlp_matches_torch_clamp():
    rng = np.random.default_rng(50)
    T, H, I, L = 9, 16, 12, 0.7
    x = rng.standard_normal((T, H))
    Wg, Wu, Wd = (rng.standard_normal(s) for s in ((1, I, H), (1, I, H), (1, H, I)))
    out = moe.forward(x, np.zeros((T, 1), np.int64), np.ones((T, 1)), Wg, Wu, Wd, swiglu_limit=L)
    xt = torch.from_numpy(x)
    g = torch.clamp(F.linear(xt, torch.from_numpy(Wg[0])), max=L)
    u = torch.clamp(F.linear(xt, torch.from_numpy(Wu[0])), -L, L)
    ref = F.linear(F.silu(g) * u, torch.from_numpy(Wd[0])).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_swiglu_limit_above_every_input_changes_nothing():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(51)
    dO = np.random.default_rng(52).standard_normal(x.shape)
    big = 1e6
    np.testing.assert_array_equal(moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, swiglu_limit=big),
                                  moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd))
    a = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, swiglu_limit=big)
    b = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd)
    for n in b:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    for off in (None, 0.0, np.inf):
        np.testing.assert_array_equal(moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd, swiglu_limit=off),
                                      moe.forward(x, top, w, Wg, Wu, Wd, Sg, Su, Sd))


def test_swiglu_limit_backward_finite_differences():
    # central differences at points where no input sits within 1e-3 of a limit
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(53, T=6, H=5, I=4, E=3, k=2, I_s=3)
    L = 0.6
    s = build_schedule(top, 3, 1.0, 2)
    dO = np.random.default_rng(54).standard_normal(x.shape)
    g = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, swiglu_limit=L)
    args = dict(x=x, w=w, Wg=Wg, Wu=Wu, Wd=Wd, Sg=Sg, Su=Su, Sd=Sd)
    gname = dict(x="dx", w="d_router_weights", Wg="d_w_gate", Wu="d_w_up", Wd="d_w_down",
                 Sg="d_s_gate", Su="d_s_up", Sd="d_s_down")

    def loss(a):
        return float(np.sum(dO * moe.forward(a["x"], top, a["w"], a["Wg"], a["Wu"], a["Wd"], a["Sg"], a["Su"],
                                             a["Sd"], sched=s, swiglu_limit=L)))
    pre = np.concatenate([(x @ W.T).ravel() for W in list(Wg) + list(Wu) + [Sg, Su]])
    assert np.min(np.abs(np.abs(pre) - L)) > 1e-3 and np.mean(np.abs(pre) > L) > 0.1
    rng = np.random.default_rng(55)
    eps = 1e-7
    for name, arr in args.items():
        for _ in range(4):
            idx = tuple(rng.integers(n) for n in arr.shape)
            p = {kk: vv.copy() for kk, vv in args.items()}
            m = {kk: vv.copy() for kk, vv in args.items()}
            p[name][idx] += eps
            m[name][idx] -= eps
            fd = (loss(p) - loss(m)) / (2 * eps)
            assert abs(fd - g[gname[name]][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


def test_swiglu_limit_mxfp8_structure_with_identity_quantizer():
    x, top, w, Wg, Wu, Wd, (Sg, Su, Sd) = rand_case(56, T=10, H=64, I=32, E=3, k=2, I_s=32)
    s = build_schedule(top, 3, 1.0, 32)
    dO = np.random.default_rng(57).standard_normal(x.shape)
    ident = lambda v, axis=-1: np.asarray(v, np.float64)  # noqa: E731
    a = moe.backward_mxfp8(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, qfun=ident, swiglu_limit=0.9)
    b = moe.backward(dO, x, top, w, Wg, Wu, Wd, Sg, Su, Sd, sched=s, swiglu_limit=0.9)
    for n in b:
        np.testing.assert_allclose(a[n], b[n], rtol=1e-11, atol=1e-11, err_msg=n)
