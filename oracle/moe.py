"""Oracle: MoE layer forward and backward in float64. TEST INFRASTRUCTURE ONLY.

What the layer computes, from the pages:
  * [A] "nemo_automodel.components.moe.mok_experts", ``GroupedExpertsMoK.forward``:
    fused shared and routed SwiGLU experts; x [T,H] BF16, router weights
    [T,k], int64 expert ids [T,k], shared gate/up [I_s,H] and down [H,I_s];
    routed gate/up [E,I,H] and down [E,H,I] (``_MoKRuntime.forward``); no
    expert bias (``down_proj_bias`` / ``gate_up_proj_bias`` are None).
  * [A] ``_MoKRuntime.backward``: gradients for x, the router weights, the
    three routed and the three shared weight tensors, reusing the forward's
    schedule; the integer ids get none.
  * [R] "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
    §"The two API layers and the schedule object": one schedule drives both
    dispatch and combine, and is reused by backward.

Formula (weights in the nn.Linear [out, in] layout, so y = W a):
  for each kept assignment (t, j) with expert e = top[t, j] and weight w[t, j]:
      g = W_g[e] x_t,  u = W_u[e] x_t,  h = silu(g) * u,  y = W_d[e] h
  out[t] = sum_j w[t, j] * y_(t, j) + S_d (silu(S_g x_t) * (S_u x_t))
with silu(z) = z * sigmoid(z). Dropped or invalid assignments contribute 0.

Readings taken where the pages leave a step open: SwiGLU is silu(gate) * up; the shared
expert has weight 1 and is always on; router weights are used as given (the
router is outside the layer, [R] §"Where MoK is the wrong tool"); the weight
is applied to the expert output (equal to applying it to h by linearity).

All arithmetic is float64. Inputs are float arrays (bf16 already decoded).
"""
from __future__ import annotations

import numpy as np

from . import mxfp8
from .schedule import build_schedule


__all__ = ["sigmoid", "silu", "swiglu", "swiglu_backward", "forward", "forward_per_token", "forward_tokens",
           "backward", "backward_slices", "quantize_weights_mxfp8", "forward_mxfp8", "forward_tokens_mxfp8",
           "backward_mxfp8", "backward_slices_mxfp8", "segment_rows"]


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def segment_rows(sched: dict, e: int):
    """Kept rows of expert e: (row ids, flat assignment ids, token ids)."""
    lo = sched["offsets"][e]
    rows = np.arange(lo, lo + sched["kept"][e], dtype=np.int64)
    a = sched["row_src"][rows]
    return rows, a, a // sched["k"]


def swiglu(g, u, limit=None):
    """h = silu(g) * u. With a limit L > 0 (the ``swiglu_limit`` of [A]
    ``_MoKRuntime``, which the pages name without a formula; the reading
    taken: a limit on SwiGLU's two inputs) h = silu(min(g, L)) *
    clamp(u, -L, L). None, 0 or inf: no limit.

    Pins (tests/test_oracle_moe.py): a dense torch MLP with torch.clamp, and
    a limit above every input equal to no limit."""
    if limit is None or not (0 < limit < np.inf):
        return silu(g) * u
    return silu(np.minimum(g, limit)) * np.clip(u, -limit, limit)


def swiglu_backward(g, u, dh, limit=None):
    """(dg, du) for h = swiglu(g, u, limit) and the gradient dh of h:
    dg = dh * u_c * s (1 + g_c (1 - s)) with s = sigmoid(g_c), du = dh *
    silu(g_c), where g_c, u_c are the limited inputs, and no gradient
    through an active limit (g > L; |u| > L), as a clamp's derivative.

    Pins (tests/test_oracle_moe.py): torch.autograd through torch.clamp, and
    central finite differences away from the limit."""
    if limit is None or not (0 < limit < np.inf):
        s = sigmoid(g)
        return dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    s = sigmoid(gc)
    dg = np.where(g <= limit, dh * uc * s * (1.0 + gc * (1.0 - s)), 0.0)
    du = np.where(np.abs(u) <= limit, dh * gc * s, 0.0)
    return dg, du


def _token_set(T, tokens):
    """Boolean mask over the T tokens (all True for tokens=None)."""
    if tokens is None:
        return np.ones(T, bool)
    m = np.zeros(T, bool)
    m[np.asarray(list(tokens), np.int64)] = True
    return m


def _expert_mlp(A, Wg, Wu, Wd, limit=None):
    g = A @ Wg.T
    u = A @ Wu.T
    h = swiglu(g, u, limit)
    return g, u, h, h @ Wd.T


def forward(x, top_experts, router_weights, w_gate, w_up, w_down,
            s_gate=None, s_up=None, s_down=None, sched=None,
            capacity_multiplier=1.0, expert_pad=32, return_parts=False, tokens=None, swiglu_limit=None):
    """Layer output [T,H] in float64, expert-grouped formulation: each
    expert's kept rows are gathered, run through its SwiGLU MLP, weighted and
    added back at their tokens. ``swiglu_limit``: see ``swiglu``.

    ``tokens`` (optional) restricts the work to the rows of those tokens (for
    checks at full size; the schedule is still the whole batch's): their
    output rows are exact, every other row is left 0.

    Pins (tests/test_oracle_moe.py): with E=1, k=1, w=1 and no shared expert
    it equals a dense SwiGLU MLP written with torch CPU ops; it equals the
    per-token loop ``forward_per_token``; permuting tokens permutes the output
    (no drops); it is linear in the router weights; w = 0 leaves only the
    shared expert."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    if sched is None:
        sched = build_schedule(top_experts, E, capacity_multiplier, expert_pad)
    wflat = np.asarray(router_weights, np.float64).reshape(-1)
    sel = _token_set(T, tokens)
    out = np.zeros((T, H))
    parts = {}
    for e in range(E):
        rows, a, t = segment_rows(sched, e)
        keep = sel[t]
        rows, a, t = rows[keep], a[keep], t[keep]
        if rows.size == 0:
            continue
        g, u, h, y = _expert_mlp(x[t], np.asarray(w_gate[e], np.float64), np.asarray(w_up[e], np.float64),
                                 np.asarray(w_down[e], np.float64), swiglu_limit)
        np.add.at(out, t, wflat[a][:, None] * y)
        if return_parts:
            parts[e] = dict(rows=rows, a=a, t=t, g=g, u=u, h=h, y=y)
    if s_gate is not None:
        ts = np.flatnonzero(sel)
        g, u, h, y = _expert_mlp(x[ts], np.asarray(s_gate, np.float64), np.asarray(s_up, np.float64),
                                 np.asarray(s_down, np.float64), swiglu_limit)
        out[ts] += y
        if return_parts:
            parts["shared"] = dict(g=g, u=u, h=h, y=y)
    if return_parts:
        return out, sched, parts
    return out


def forward_per_token(x, top_experts, router_weights, w_gate, w_up, w_down,
                      s_gate=None, s_up=None, s_down=None, sched=None,
                      capacity_multiplier=1.0, expert_pad=32):
    """The same output by a scalar-style loop over tokens and slots, reading
    the keep/drop decision from the schedule's slot map. Used at tiny sizes
    as an independent formulation of ``forward``."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    if sched is None:
        sched = build_schedule(top_experts, E, capacity_multiplier, expert_pad)
    out = np.zeros((T, H))
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            if sched["slot_row"][t * k + j] < 0:
                continue
            e = int(top_experts[t, j])
            h = silu(w_gate[e] @ x[t]) * (w_up[e] @ x[t])
            acc += float(router_weights[t, j]) * (w_down[e] @ h)
        if s_gate is not None:
            acc += s_down @ (silu(s_gate @ x[t]) * (s_up @ x[t]))
        out[t] = acc
    return out


def forward_tokens(tokens, x, top_experts, router_weights, w_gate, w_up, w_down,
                   s_gate=None, s_up=None, s_down=None, slot_row=None):
    """Output rows for a subset of tokens only, each computed on its own
    (used for sampled checks at full sizes). ``slot_row`` ([T*k], -1 where an
    assignment was not kept) comes from the oracle schedule of the whole
    batch; None means every valid assignment is kept."""
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    outs = []
    for t in tokens:
        xt = np.asarray(x[t], np.float64)
        acc = np.zeros(xt.shape[0])
        for j in range(k):
            e = int(top_experts[t, j])
            kept = (0 <= e < E) if slot_row is None else slot_row[t * k + j] >= 0
            if not kept:
                continue
            Wg, Wu, Wd = (np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))
            h = silu(Wg @ xt) * (Wu @ xt)
            acc += float(router_weights[t, j]) * (Wd @ h)
        if s_gate is not None:
            acc += np.asarray(s_down, np.float64) @ (silu(np.asarray(s_gate, np.float64) @ xt)
                                                     * (np.asarray(s_up, np.float64) @ xt))
        outs.append(acc)
    return np.stack(outs) if outs else np.zeros((0, x.shape[1]))


def backward(grad_out, x, top_experts, router_weights, w_gate, w_up, w_down,
             s_gate=None, s_up=None, s_down=None, sched=None,
             capacity_multiplier=1.0, expert_pad=32, tokens=None, dw_experts=None, swiglu_limit=None):
    """Gradients of sum(grad_out * out) with respect to every float input
    (``swiglu_limit``: see ``swiglu`` and ``swiglu_backward``).

    ``tokens`` and ``dw_experts`` (optional) restrict the work for checks at
    full size: dx and d_router_weights are exact for the listed tokens, the
    weight gradients for the listed experts (the string "shared" names the
    shared expert); entries outside them are unspecified.

    Returns dict: dx [T,H], d_router_weights [T,k], d_w_gate, d_w_up
    [E,I,H], d_w_down [E,H,I], d_s_gate, d_s_up [I_s,H], d_s_down [H,I_s]
    (None without a shared expert). Dropped or invalid assignments get a zero
    router-weight gradient and add nothing anywhere.

    Per kept row r (token t, expert e, weight w), with y the unweighted
    expert output:
      dw     = <grad_out[t], y>
      dy     = w * grad_out[t];    dh = W_d[e]^T dy
      dg     = dh * u * s * (1 + g (1 - s)),  s = sigmoid(g);   du = dh * silu(g)
      dW_d  += dy h^T;   dW_g += dg x_t^T;   dW_u += du x_t^T
      dx[t] += W_g[e]^T dg + W_u[e]^T du
    and the same for the shared expert with w = 1.

    Pins (tests/test_oracle_moe.py): central finite differences in float64
    for every input on tiny shapes, and torch.autograd (CPU, float64) through
    a torch-written forward.
    """
    dO = np.asarray(grad_out, np.float64)
    x = np.asarray(x, np.float64)
    T, H = x.shape
    k = top_experts.shape[1]
    E, I, _ = w_gate.shape
    if sched is None:
        sched = build_schedule(top_experts, E, capacity_multiplier, expert_pad)
    wflat = np.asarray(router_weights, np.float64).reshape(-1)
    sel = _token_set(T, tokens)
    want_dw = (lambda e: True) if dw_experts is None else (lambda e: e in dw_experts)  # noqa: E731
    dx = np.zeros((T, H))
    dwr = np.zeros(T * k)
    dWg = np.zeros((E, I, H))
    dWu = np.zeros((E, I, H))
    dWd = np.zeros((E, H, I))
    for e in range(E):
        rows, a, t = segment_rows(sched, e)
        if not want_dw(e):  # the weight gradients need every row; dx and dw only the listed tokens'
            keep = sel[t]
            rows, a, t = rows[keep], a[keep], t[keep]
        if rows.size == 0:
            continue
        Wg_e, Wu_e, Wd_e = (np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))
        A = x[t]
        g, u, h, y = _expert_mlp(A, Wg_e, Wu_e, Wd_e, swiglu_limit)
        dOt = dO[t]
        dwr[a] = np.sum(dOt * y, axis=1)
        dy = wflat[a][:, None] * dOt
        dh = dy @ Wd_e
        dg, du = swiglu_backward(g, u, dh, swiglu_limit)
        if want_dw(e):
            dWd[e] = dy.T @ h
            dWg[e] = dg.T @ A
            dWu[e] = du.T @ A
        np.add.at(dx, t, dg @ Wg_e + du @ Wu_e)
    res = dict(dx=dx, d_router_weights=dwr.reshape(T, k), d_w_gate=dWg, d_w_up=dWu,
               d_w_down=dWd, d_s_gate=None, d_s_up=None, d_s_down=None)
    if s_gate is not None:
        Sg, Su, Sd = (np.asarray(w, np.float64) for w in (s_gate, s_up, s_down))
        ts = np.arange(T) if want_dw("shared") else np.flatnonzero(sel)
        xs, dOs = x[ts], dO[ts]
        g, u, h, y = _expert_mlp(xs, Sg, Su, Sd, swiglu_limit)
        dh = dOs @ Sd
        dg, du = swiglu_backward(g, u, dh, swiglu_limit)
        if want_dw("shared"):
            res["d_s_down"] = dOs.T @ h
            res["d_s_gate"] = dg.T @ xs
            res["d_s_up"] = du.T @ xs
        dx[ts] += dg @ Sg + du @ Su
    return res


def backward_slices(grad_out, x, top_experts, router_weights, w_gate, w_up, w_down,
                    s_gate=None, s_up=None, s_down=None, slot_row=None, tokens=(), expert_cols=(),
                    shared_cols=()):
    """Slices of ``backward`` computed on their own (for sampled checks at
    full sizes), from the same per-row formulas:
      dx[t] and d_router_weights[t, :] for t in ``tokens``;
      for (e, i) in ``expert_cols``: dW_g[e][i, :], dW_u[e][i, :] and
      dW_d[e][:, i] (sums over the kept rows of expert e in any order);
      for i in ``shared_cols``: the same slices of the shared expert's
      gradients (rows = every token).
    ``slot_row`` ([T*k], -1 where an assignment was not kept) comes from
    the oracle schedule of the whole batch. Weight and activation arguments
    may be indexable objects decoding rows lazily (``w[e]`` -> float
    matrix, ``x[t]`` -> float row).

    Pin (tests/test_oracle_moe.py): every slice equals ``backward`` on
    random small cases with drops and invalid ids."""
    T = top_experts.shape[0]
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    f = lambda a: np.asarray(a, np.float64)  # noqa: E731

    def kept(t, j):
        e = int(top_experts[t, j])
        return (0 <= e < E) if slot_row is None else slot_row[t * k + j] >= 0

    def row_terms(xt, dOt, w, Wg, Wu, Wd):
        g = Wg @ xt
        u = Wu @ xt
        s = sigmoid(g)
        h = g * s * u
        dh_hat = Wd.T @ dOt
        dh = w * dh_hat
        dg = dh * u * s * (1.0 + g * (1.0 - s))
        du = dh * g * s
        return h, dh_hat, dg, du

    res = dict(dx={}, d_router_weights={}, d_w_gate_rows={}, d_w_up_rows={}, d_w_down_cols={},
               d_s_gate_rows={}, d_s_up_rows={}, d_s_down_cols={})
    for t in tokens:
        xt, dOt = f(x[t]), f(grad_out[t])
        dx = np.zeros(xt.shape[0])
        dwr = np.zeros(k)
        for j in range(k):
            if not kept(t, j):
                continue
            e = int(top_experts[t, j])
            Wg, Wu, Wd = f(w_gate[e]), f(w_up[e]), f(w_down[e])
            h, dh_hat, dg, du = row_terms(xt, dOt, float(router_weights[t, j]), Wg, Wu, Wd)
            dwr[j] = dh_hat @ h
            dx += Wg.T @ dg + Wu.T @ du
        if s_gate is not None:
            h, dh_hat, dg, du = row_terms(xt, dOt, 1.0, f(s_gate), f(s_up), f(s_down))
            dx += f(s_gate).T @ dg + f(s_up).T @ du
        res["dx"][t] = dx
        res["d_router_weights"][t] = dwr
    for (e, i) in expert_cols:
        Wg, Wu, Wd = f(w_gate[e]), f(w_up[e]), f(w_down[e])
        H = Wg.shape[1]
        dWg = np.zeros(H)
        dWu = np.zeros(H)
        dWd = np.zeros(Wd.shape[0])
        for t in range(T):
            for j in range(k):
                if int(top_experts[t, j]) != e or not kept(t, j):
                    continue
                xt, dOt, w = f(x[t]), f(grad_out[t]), float(router_weights[t, j])
                g, u = Wg[i] @ xt, Wu[i] @ xt
                s = sigmoid(g)
                dh = w * (Wd[:, i] @ dOt)
                dWg += dh * u * s * (1.0 + g * (1.0 - s)) * xt
                dWu += dh * g * s * xt
                dWd += w * (g * s * u) * dOt
        res["d_w_gate_rows"][(e, i)] = dWg
        res["d_w_up_rows"][(e, i)] = dWu
        res["d_w_down_cols"][(e, i)] = dWd
    if s_gate is not None:
        for i in shared_cols:
            Sg, Su, Sd = f(s_gate), f(s_up), f(s_down)
            dWg = np.zeros(Sg.shape[1])
            dWu = np.zeros(Sg.shape[1])
            dWd = np.zeros(Sd.shape[0])
            for t in range(T):
                xt, dOt = f(x[t]), f(grad_out[t])
                g, u = Sg[i] @ xt, Su[i] @ xt
                s = sigmoid(g)
                dh = Sd[:, i] @ dOt
                dWg += dh * u * s * (1.0 + g * (1.0 - s)) * xt
                dWu += dh * g * s * xt
                dWd += (g * s * u) * dOt
            res["d_s_gate_rows"][i] = dWg
            res["d_s_up_rows"][i] = dWu
            res["d_s_down_cols"][i] = dWd
    return res


# ---------------------------------------------------------------------------
# MXFP8 emulation
# ---------------------------------------------------------------------------

def quantize_weights_mxfp8(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
                           for_backward=False, qfun=None):
    """The weights as the MXFP8 GEMMs read them: dequantize(quantize(.)) in
    blocks of 32 along the contraction dimension of the GEMM that reads them.
      forward:  gate/up blocked along H (W_g, W_u [E,I,H] axis 2; S_g, S_u
                [I_s,H] axis 1), down along I (W_d [E,H,I] axis 2; S_d
                [H,I_s] axis 1): keys Wg_f, Wu_f, Wd_f (Sg_f, Su_f, Sd_f);
      backward: gate/up along H again (the forward is recomputed), down along
                H (dh contracts over H: W_d axis 1, S_d axis 0) and gate/up
                along I (dA contracts over I: W_g, W_u axis 1, S_g, S_u axis
                0): keys Wg_f, Wu_f, Wd_b, Wg_b, Wu_b (Sg_f, Su_f, Sd_b, Sg_b,
                Su_b).
    The shared keys are absent without a shared expert. ``qfun`` replaces
    the quantizer (signature of ``mxfp8.qdq``); the test suite passes one that
    records its calls, or one that runs ``mxfp8.qdq`` on slices in parallel
    (the blocks never cross the slices, so the values are the same)."""
    q = mxfp8.qdq if qfun is None else qfun
    f = lambda a: np.asarray(a, np.float64)  # noqa: E731
    r = dict(Wg_f=q(f(w_gate), axis=2), Wu_f=q(f(w_up), axis=2))
    if for_backward:
        r.update(Wd_b=q(f(w_down), axis=1), Wg_b=q(f(w_gate), axis=1), Wu_b=q(f(w_up), axis=1))
    else:
        r.update(Wd_f=q(f(w_down), axis=2))
    if s_gate is not None:
        r.update(Sg_f=q(f(s_gate), axis=1), Su_f=q(f(s_up), axis=1))
        if for_backward:
            r.update(Sd_b=q(f(s_down), axis=0), Sg_b=q(f(s_gate), axis=0), Su_b=q(f(s_up), axis=0))
        else:
            r.update(Sd_f=q(f(s_down), axis=1))
    return r


def forward_mxfp8(x, top_experts, router_weights, w_gate, w_up, w_down,
                  s_gate=None, s_up=None, s_down=None, sched=None,
                  capacity_multiplier=1.0, expert_pad=32, return_parts=False,
                  quantize_h=True, qweights=None, tokens=None, swiglu_limit=None):
    """MXFP8 forward: x, W_g, W_u (blocks along H) and W_d (blocks along I),
    shared weights included, are replaced by dequantize(quantize(.)); h is
    computed in float64 from those and itself quantized along I before the
    down projection. SwiGLU, the weighting and the combine stay in float64.

    Reading: [R] §"Tuning the five hyperparameters before production" keeps
    activations in BF16 at the interface and quantizes weights beforehand;
    the quantization of x and h along the contraction dimension inside the
    layer is the plain reading of "MXFP8 forward" (blocks along K).

    ``qweights`` (optional): the result of ``quantize_weights_mxfp8`` for
    these weights, computed beforehand. ``tokens`` (optional) restricts the
    work to those tokens' rows as in ``forward`` (other rows are left 0).
    ``swiglu_limit``: see ``swiglu``.

    Pin (tests/test_oracle_moe.py): when x and every weight already sit on
    the MX grid, the only difference to ``forward`` is h's quantization, so
    replacing the h step by the identity must reproduce ``forward`` exactly.
    """
    q = mxfp8.qdq
    qh = mxfp8.qdq if quantize_h else (lambda v, axis: v)
    if qweights is None:
        qweights = quantize_weights_mxfp8(w_gate, w_up, w_down, s_gate, s_up, s_down)
    Wg, Wu, Wd = qweights["Wg_f"], qweights["Wu_f"], qweights["Wd_f"]
    T, H = np.shape(x)
    sel = _token_set(T, tokens)
    xq = np.zeros((T, H))
    xq[sel] = q(np.asarray(x, np.float64)[sel], axis=1)  # blocks along H: rows are independent
    E = Wg.shape[0]
    if sched is None:
        sched = build_schedule(top_experts, E, capacity_multiplier, expert_pad)
    wflat = np.asarray(router_weights, np.float64).reshape(-1)
    out = np.zeros((T, H))
    parts = {}
    for e in range(E):
        rows, a, t = segment_rows(sched, e)
        keep = sel[t]
        rows, a, t = rows[keep], a[keep], t[keep]
        if rows.size == 0:
            continue
        A = xq[t]
        g = A @ Wg[e].T
        u = A @ Wu[e].T
        h = qh(swiglu(g, u, swiglu_limit), axis=1)
        y = h @ Wd[e].T
        np.add.at(out, t, wflat[a][:, None] * y)
        if return_parts:
            parts[e] = dict(rows=rows, a=a, t=t, g=g, u=u, hq=h, y=y)
    if s_gate is not None:
        ts = np.flatnonzero(sel)
        g = xq[ts] @ qweights["Sg_f"].T
        u = xq[ts] @ qweights["Su_f"].T
        h = qh(swiglu(g, u, swiglu_limit), axis=1)
        out[ts] += h @ qweights["Sd_f"].T
        if return_parts:
            parts["shared"] = dict(g=g, u=u, hq=h)
    if return_parts:
        return out, sched, parts
    return out


def forward_tokens_mxfp8(tokens, x, top_experts, router_weights, w_gate, w_up, w_down,
                         s_gate=None, s_up=None, s_down=None, slot_row=None):
    """``forward_mxfp8`` for a subset of tokens, each computed on its own
    (for sampled checks at full sizes): x_t quantized along H; the gate/up
    weights of each expert it uses along H, the down weights along I; h
    computed in float64 and quantized along I; weighted sum in float64.
    ``slot_row`` as in ``forward_tokens``. Weight arguments may be any
    indexable of float rows per expert (decoded lazily).

    Pin (tests/test_oracle_moe.py): over all tokens of random small cases it
    equals ``forward_mxfp8`` (with drops and invalid ids)."""
    q = mxfp8.qdq
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = (q(np.asarray(w_gate[e], np.float64), axis=1), q(np.asarray(w_up[e], np.float64), axis=1),
                        q(np.asarray(w_down[e], np.float64), axis=1))
        return cache[e]

    if s_gate is not None:
        Sg = q(np.asarray(s_gate, np.float64), axis=1)
        Su = q(np.asarray(s_up, np.float64), axis=1)
        Sd = q(np.asarray(s_down, np.float64), axis=1)
    outs = []
    for t in tokens:
        xt = q(np.asarray(x[t], np.float64)[None, :], axis=1)[0]
        acc = np.zeros(xt.shape[0])
        for j in range(k):
            e = int(top_experts[t, j])
            kept = (0 <= e < E) if slot_row is None else slot_row[t * k + j] >= 0
            if not kept:
                continue
            Wg, Wu, Wd = expert(e)
            h = q((silu(Wg @ xt) * (Wu @ xt))[None, :], axis=1)[0]
            acc += float(router_weights[t, j]) * (Wd @ h)
        if s_gate is not None:
            h = q((silu(Sg @ xt) * (Su @ xt))[None, :], axis=1)[0]
            acc += Sd @ h
        outs.append(acc)
    return np.stack(outs) if outs else np.zeros((0, x.shape[1]))


def _qdq_rows_in_segment(v, q, block=32):
    """Quantize [n, C] along rows in 32-row blocks, the rows being one
    expert's kept rows followed by zero padding up to a multiple of 32."""
    n = v.shape[0]
    npad = -(-n // block) * block
    vp = np.zeros((npad,) + v.shape[1:])
    vp[:n] = v
    return q(vp, axis=0)[:n]


def backward_mxfp8(grad_out, x, top_experts, router_weights, w_gate, w_up, w_down,
                   s_gate=None, s_up=None, s_down=None, sched=None,
                   capacity_multiplier=1.0, expert_pad=32, qfun=None, qweights=None,
                   tokens=None, dw_experts=None, swiglu_limit=None):
    """MXFP8 backward: every backward GEMM operand is quantized along that
    GEMM's contraction dimension, the forward activations being the MXFP8
    forward's (g, u from quantized x and weights; h quantized along I).

      dh   = Q_H(grad_out rows) @ Q_H(W_d)              (contraction over H)
      dA   = Q_I(dg) @ Q_I(W_g) + Q_I(du) @ Q_I(W_u)   (contraction over I)
      dW_d = Q_r(dy)^T @ Q_r(h)                        (contraction over rows)
      dW_g = Q_r(dg)^T @ Q_r(x rows);  dW_u likewise
    where Q_r works in 32-row blocks inside each expert's zero-padded segment.
    The router-weight gradient is <dh_unweighted, h> (equal to <grad_out, y>).
    Reading: the pages give the MXFP8 backward only by name; quantizing each
    operand along its own contraction dimension is the plain reading of
    "MXFP8" (blocks along K) for a GEMM whose K differs from the forward's.
    Everything between the quantizers is exact (float64): g and u are the
    MXFP8 forward's own, so this is the gradient of ``forward_mxfp8`` with
    each backward GEMM's operands quantized.

    ``qweights`` (optional): ``quantize_weights_mxfp8(..., for_backward=True)``
    of these weights, computed beforehand. ``tokens`` and ``dw_experts``
    restrict the work as in ``backward`` (a listed expert's weight gradients
    use all of its rows, as its 32-row blocks need). ``swiglu_limit``: see
    ``swiglu`` and ``swiglu_backward``.

    Pins (tests/test_oracle_moe.py): with ``qfun`` the identity this must equal
    ``backward`` (checks which operand goes where); a recording ``qfun`` checks
    that every operand is blocked along its GEMM's contraction dimension;
    per-token locality (a token's dx and router-weight gradients do not move
    when another token's grad_out does) and exact power-of-two equivariance
    of dW_down rows pin the blocking semantically; the quantizer itself is
    pinned in tests/test_oracle_mxfp8.py.
    """
    q = mxfp8.qdq if qfun is None else qfun
    if qweights is None:
        qweights = quantize_weights_mxfp8(w_gate, w_up, w_down, s_gate, s_up, s_down, for_backward=True, qfun=q)
    Wg_f, Wu_f, Wd_b, Wg_b, Wu_b = (qweights[n] for n in ("Wg_f", "Wu_f", "Wd_b", "Wg_b", "Wu_b"))
    dO = np.asarray(grad_out, np.float64)
    xraw = np.asarray(x, np.float64)
    T, H = xraw.shape
    sel = _token_set(T, tokens)
    want_dw = (lambda e: True) if dw_experts is None else (lambda e: e in dw_experts)  # noqa: E731
    xq = q(xraw, axis=1)
    k = top_experts.shape[1]
    E, I, _ = Wg_f.shape
    if sched is None:
        sched = build_schedule(top_experts, E, capacity_multiplier, expert_pad)
    wflat = np.asarray(router_weights, np.float64).reshape(-1)
    dx = np.zeros((T, H))
    dwr = np.zeros(T * k)
    dWg = np.zeros((E, I, H))
    dWu = np.zeros((E, I, H))
    dWd = np.zeros((E, H, I))
    for e in range(E):
        rows, a, t = segment_rows(sched, e)
        if not want_dw(e):  # the weight gradients need every row; dx and dw only the listed tokens'
            keep = sel[t]
            rows, a, t = rows[keep], a[keep], t[keep]
        if rows.size == 0:
            continue
        A = xq[t]
        g = A @ Wg_f[e].T
        u = A @ Wu_f[e].T
        hq = q(swiglu(g, u, swiglu_limit), axis=1)
        dOq = q(dO[t], axis=1)
        dh_un = dOq @ Wd_b[e]
        dwr[a] = np.sum(dh_un * hq, axis=1)
        w = wflat[a][:, None]
        dh = w * dh_un
        dg, du = swiglu_backward(g, u, dh, swiglu_limit)
        dx_rows = q(dg, axis=1) @ Wg_b[e] + q(du, axis=1) @ Wu_b[e]
        np.add.at(dx, t, dx_rows)
        if want_dw(e):
            dy = w * dO[t]
            dWd[e] = _qdq_rows_in_segment(dy, q).T @ _qdq_rows_in_segment(hq, q)
            xr = _qdq_rows_in_segment(xraw[t], q)
            dWg[e] = _qdq_rows_in_segment(dg, q).T @ xr
            dWu[e] = _qdq_rows_in_segment(du, q).T @ xr
    res = dict(dx=dx, d_router_weights=dwr.reshape(T, k), d_w_gate=dWg, d_w_up=dWu,
               d_w_down=dWd, d_s_gate=None, d_s_up=None, d_s_down=None)
    if s_gate is not None:
        ts = np.arange(T) if want_dw("shared") else np.flatnonzero(sel)
        g = xq[ts] @ qweights["Sg_f"].T
        u = xq[ts] @ qweights["Su_f"].T
        hq = q(swiglu(g, u, swiglu_limit), axis=1)
        dh = q(dO[ts], axis=1) @ qweights["Sd_b"]
        dg, du = swiglu_backward(g, u, dh, swiglu_limit)
        dx[ts] += q(dg, axis=1) @ qweights["Sg_b"] + q(du, axis=1) @ qweights["Su_b"]
        if want_dw("shared"):
            res["d_s_down"] = _qdq_rows_in_segment(dO, q).T @ _qdq_rows_in_segment(hq, q)
            xr = _qdq_rows_in_segment(xraw, q)
            res["d_s_gate"] = _qdq_rows_in_segment(dg, q).T @ xr
            res["d_s_up"] = _qdq_rows_in_segment(du, q).T @ xr
    return res


def backward_slices_mxfp8(grad_out, x, top_experts, router_weights, w_gate, w_up, w_down,
                          s_gate=None, s_up=None, s_down=None, slot_row=None, tokens=(), expert_cols=(),
                          shared_cols=()):
    """Slices of ``backward_mxfp8`` computed on their own (for sampled checks
    at full sizes), with the same quantization of every operand:
      dx[t] and d_router_weights[t, :] for t in ``tokens``;
      for (e, i) in ``expert_cols``: dW_g[e][i, :], dW_u[e][i, :] and
      dW_d[e][:, i]; for i in ``shared_cols`` the shared expert's slices.
    ``slot_row`` ([T*k], -1 where an assignment was not kept) is the oracle
    schedule's; an expert's rows are its kept assignments in ascending flat
    index, which is the row order the 32-row blocks of Q_r follow. Weight
    and activation arguments may decode rows lazily (``w[e]``, ``x[t]``).

    Pin (tests/test_oracle_moe.py): every slice equals ``backward_mxfp8`` on
    random small cases with drops and invalid ids."""
    q = mxfp8.qdq
    T = top_experts.shape[0]
    k = top_experts.shape[1]
    E = w_gate.shape[0]
    f = lambda a: np.asarray(a, np.float64)  # noqa: E731
    cache = {}

    def expert(e):
        # forward operands along H (gate/up) and I (down); backward operands
        # along each backward GEMM's contraction: down along H, gate/up along I
        if e not in cache:
            Wg, Wu, Wd = f(w_gate[e]), f(w_up[e]), f(w_down[e])
            cache[e] = dict(Wg_f=q(Wg, axis=1), Wu_f=q(Wu, axis=1), Wd_b=q(Wd, axis=0),
                            Wg_b=q(Wg, axis=0), Wu_b=q(Wu, axis=0))
        return cache[e]

    if s_gate is not None:
        Sg, Su, Sd = f(s_gate), f(s_up), f(s_down)
        shared = dict(Wg_f=q(Sg, axis=1), Wu_f=q(Su, axis=1), Wd_b=q(Sd, axis=0), Wg_b=q(Sg, axis=0),
                      Wu_b=q(Su, axis=0))

    def kept(t, j):
        e = int(top_experts[t, j])
        return (0 <= e < E) if slot_row is None else slot_row[t * k + j] >= 0

    def qrow(v):
        return q(np.asarray(v, np.float64)[None, :], axis=1)[0]

    res = dict(dx={}, d_router_weights={}, d_w_gate_rows={}, d_w_up_rows={}, d_w_down_cols={},
               d_s_gate_rows={}, d_s_up_rows={}, d_s_down_cols={})
    for t in tokens:
        xq = qrow(x[t])
        dOq = qrow(grad_out[t])
        dx = np.zeros(xq.shape[0])
        dwr = np.zeros(k)
        terms = [(j, float(router_weights[t, j]), expert(int(top_experts[t, j]))) for j in range(k) if kept(t, j)]
        if s_gate is not None:
            terms.append((None, 1.0, shared))
        for j, w, m in terms:
            g = m["Wg_f"] @ xq
            u = m["Wu_f"] @ xq
            hq = qrow(silu(g) * u)
            dh_un = dOq @ m["Wd_b"]
            if j is not None:
                dwr[j] = dh_un @ hq
            dh = w * dh_un
            s = sigmoid(g)
            dg = dh * u * s * (1.0 + g * (1.0 - s))
            du = dh * g * s
            dx += qrow(dg) @ m["Wg_b"] + qrow(du) @ m["Wu_b"]
        res["dx"][t] = dx
        res["d_router_weights"][t] = dwr

    def column_slices(m, X, dO, w, i):
        """dW_g[i, :], dW_u[i, :], dW_d[:, i] over one segment's rows."""
        xq = q(X, axis=1)
        b0 = (i // 32) * 32
        g = xq @ m["Wg_f"][b0:b0 + 32].T
        u = xq @ m["Wu_f"][b0:b0 + 32].T
        hq_i = q(silu(g) * u, axis=1)[:, i - b0]
        dOq = q(dO, axis=1)
        dh = w * (dOq @ m["Wd_b"][:, i])
        gi, ui = g[:, i - b0], u[:, i - b0]
        s = sigmoid(gi)
        dg = dh * ui * s * (1.0 + gi * (1.0 - s))
        du = dh * gi * s
        xr = _qdq_rows_in_segment(X, q)
        dWg = _qdq_rows_in_segment(dg[:, None], q)[:, 0] @ xr
        dWu = _qdq_rows_in_segment(du[:, None], q)[:, 0] @ xr
        dy = _qdq_rows_in_segment(w[:, None] * dO, q)
        dWd = dy.T @ _qdq_rows_in_segment(hq_i[:, None], q)[:, 0]
        return dWg, dWu, dWd

    for (e, i) in expert_cols:
        rows = [(t, j) for t in range(T) for j in range(k) if int(top_experts[t, j]) == e and kept(t, j)]
        m = expert(e)
        H = m["Wg_f"].shape[1]
        if not rows:
            res["d_w_gate_rows"][(e, i)] = np.zeros(H)
            res["d_w_up_rows"][(e, i)] = np.zeros(H)
            res["d_w_down_cols"][(e, i)] = np.zeros(m["Wd_b"].shape[0])
            continue
        X = np.stack([f(x[t]) for t, _ in rows])
        dO = np.stack([f(grad_out[t]) for t, _ in rows])
        w = np.array([float(router_weights[t, j]) for t, j in rows])
        dWg, dWu, dWd = column_slices(m, X, dO, w, i)
        res["d_w_gate_rows"][(e, i)] = dWg
        res["d_w_up_rows"][(e, i)] = dWu
        res["d_w_down_cols"][(e, i)] = dWd
    if s_gate is not None and len(shared_cols):
        X = np.stack([f(x[t]) for t in range(T)])
        dO = np.stack([f(grad_out[t]) for t in range(T)])
        w = np.ones(T)
        for i in shared_cols:
            dWg, dWu, dWd = column_slices(shared, X, dO, w, i)
            res["d_s_gate_rows"][i] = dWg
            res["d_s_up_rows"][i] = dWu
            res["d_s_down_cols"][i] = dWd
    return res
