"""fp64 CPU oracle of the Mixture-of-Experts FFN layer backward.

TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module; the library path
never calls it and it shares no code with the HIP kernels. It differentiates
exactly the forward that oracle/moe_ref.py defines, in float64, for a loss whose
gradient with respect to the layer output y is dy, plus optionally the
load-balancing loss coef * E * sum_e f_e P_e ([RO] How It Works 1; [FS] Why MoE
breaks naive fine-tuning) with f treated as a constant (counts are not
differentiable).

The routing decision is piecewise constant: gradients reach the router through
the gates of the selected experts (and through P when the balancing term is on),
never through the choice itself ([MT] Noisy top-k gating: non-top-k entries are
-inf before the softmax, so they carry no gradient). A selection bias only moves
the choice, so it gets no gradient ([RO] How It Works 2 updates it by the sign
rule instead). Assignments dropped by expert capacity contribute nothing forward,
so nothing flows back through them.

Chain rule per piece (row vectors; Linear weights stored [out, in]):
  expert, GELU:    z = X W1^T + b1, h = gelu(z), Y = h W2^T + b2
                   dh = dY W2, dW2 = dY^T h, db2 = sum dY, dz = dh * gelu'(z),
                   dW1 = dz^T X, db1 = sum dz, dX = dz W1,  gelu'(z) = Phi(z) + z phi(z)
  expert, SwiGLU:  a = X Wg^T, u = X Wu^T, h = silu(a) * u, Y = h Wd^T
                   dh = dY Wd, dWd = dY^T h, da = dh * u * silu'(a), du = dh * silu(a),
                   dWg = da^T X, dWu = du^T X, dX = da Wg + du Wu,
                   silu'(a) = sig(a) (1 + a (1 - sig(a)))
  combine:         dg[t, j] = <dy[t], Y(t, j)>, dY(t, j) = g[t, j] dy[t]
  gates:           softmax over the selected logits: dl_S = g * (dg - <g, dg>)
                   full-softmax probabilities: dl = p * (dp - <p, dp>), dp = dg at the selection
                   sigmoid normalised over the selection: ds = (dg - <g, dg>) / sum_S s,
                   dl_S = ds * s (1 - s)
  router:          dW_r = dl^T x, dx += dl W_r
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
from scipy.special import erf

from oracle import moe_ref as R


def silu_grad(a: np.ndarray) -> np.ndarray:
    s = R.sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def gelu_grad(z: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def expert_backward(X, w_in, b_in, w_out, b_out, act: str, dY):
    """Gradients of one expert FFN on rows X given dY: (dX, dw_in, db_in, dw_out, db_out)."""
    if act == "gelu":
        z = X @ w_in.T
        if b_in is not None:
            z = z + b_in[None, :]
        h = R.gelu(z)
        dh = dY @ w_out
        dz = dh * gelu_grad(z)
        dw_in = dz.T @ X
        db_in = dz.sum(axis=0) if b_in is not None else None
        dX = dz @ w_in
    elif act == "swiglu":
        F = w_in.shape[0] // 2
        a = X @ w_in[:F].T
        u = X @ w_in[F:].T
        h = R.silu(a) * u
        dh = dY @ w_out
        da = dh * u * silu_grad(a)
        du = dh * R.silu(a)
        dw_in = np.concatenate([da.T @ X, du.T @ X], axis=0)
        db_in = None
        dX = da @ w_in[:F] + du @ w_in[F:]
    else:
        raise ValueError(act)
    dw_out = dY.T @ h
    db_out = dY.sum(axis=0) if b_out is not None else None
    return dX, dw_in, db_in, dw_out, db_out


def gate_backward(l: np.ndarray, idx: np.ndarray, score: str, renorm: bool, dg: np.ndarray) -> np.ndarray:
    """Gradient of the router logits from the gate gradients dg [T, k] (see the module notes)."""
    T, E = l.shape
    dl = np.zeros((T, E))
    sel = np.take_along_axis(l, idx, axis=-1)
    if score == "softmax" and renorm:
        g = R.softmax(sel)
        dsel = g * (dg - np.sum(g * dg, axis=-1, keepdims=True))
        np.put_along_axis(dl, idx, dsel, axis=-1)
    elif score == "softmax":
        p = R.softmax(l)
        dp = np.zeros((T, E))
        np.put_along_axis(dp, idx, dg, axis=-1)
        dl = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    else:
        s = R.sigmoid(sel)
        Z = s.sum(axis=-1, keepdims=True)
        g = s / Z
        ds = (dg - np.sum(g * dg, axis=-1, keepdims=True)) / Z
        np.put_along_axis(dl, idx, ds * s * (1.0 - s), axis=-1)
    return dl


def aux_backward(l: np.ndarray, idx: np.ndarray, score: str, coef: float) -> np.ndarray:
    """Gradient of coef * E * sum_e f_e P_e with f = counts / T held constant and
    P_e = mean_t p[t, e] (p the balance distribution of route_stats)."""
    T, E = l.shape
    f = R.expert_counts(idx, E) / T
    dp = np.broadcast_to(coef * E * f / T, (T, E))
    if score == "softmax":
        p = R.softmax(l)
        return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    s = R.sigmoid(l)
    Z = s.sum(axis=-1, keepdims=True)
    p = s / Z
    ds = (dp - np.sum(p * dp, axis=-1, keepdims=True)) / Z
    return ds * s * (1.0 - s)


@dataclasses.dataclass
class BackwardResult:
    dx: np.ndarray  # [T, d]
    dw_r: np.ndarray  # [E, d]
    dw_in: np.ndarray  # [E, n_in, d]
    db_in: Optional[np.ndarray]  # [E, F]
    dw_out: np.ndarray  # [E, d, F]
    db_out: Optional[np.ndarray]  # [E, d]
    dws_in: Optional[np.ndarray]  # [2 Fs, d]
    dws_out: Optional[np.ndarray]  # [d, Fs]
    dl: np.ndarray  # [T, E] router logit gradient
    dg: np.ndarray  # [T, k] gate gradient
    y: np.ndarray  # the forward output, for reference


def layer_backward(x, w_r, get_expert, k: int, act: str, score: str, renorm: bool, sel_bias, ws_in, ws_out, dy,
                   forced_idx: Optional[np.ndarray] = None, capacity: int = 0,
                   aux_coef: float = 0.0) -> BackwardResult:
    """All gradients of the layer for output gradient dy (see the module notes)."""
    x, dy = R.f64(x), R.f64(dy)
    w_r = R.f64(w_r)
    fwd = R.layer_forward(x, w_r, get_expert, k, act, score, renorm, sel_bias, ws_in, ws_out, forced_idx,
                          capacity)
    r = fwd.route
    T, d = x.shape
    E = w_r.shape[0]
    idx, g = r.idx, r.gates
    inv = fwd.inv_pos.reshape(T, k)
    # combine
    dg = np.zeros((T, k))
    dYp = np.zeros_like(fwd.y_perm)
    for j in range(k):
        kept = inv[:, j] >= 0
        rows = inv[kept, j]
        dg[kept, j] = np.sum(dy[kept] * fwd.y_perm[rows], axis=1)
        dYp[rows] = g[kept, j:j + 1] * dy[kept]
    # experts on their rows
    w0 = get_expert(0)
    n_in, F = w0[0].shape[0], w0[2].shape[1]
    dw_in = np.zeros((E, n_in, d))
    dw_out = np.zeros((E, d, F))
    db_in = np.zeros((E, F)) if w0[1] is not None else None
    db_out = np.zeros((E, d)) if w0[3] is not None else None
    dXp = np.zeros_like(fwd.x_perm)
    for e in range(E):
        r0, r1 = int(fwd.offsets[e]), int(fwd.offsets[e + 1])
        if r1 == r0:
            continue
        wi, bi, wo, bo = get_expert(e)
        dX, dwi, dbi, dwo, dbo = expert_backward(fwd.x_perm[r0:r1], wi, bi, wo, bo, act, dYp[r0:r1])
        dXp[r0:r1] = dX
        dw_in[e], dw_out[e] = dwi, dwo
        if db_in is not None:
            db_in[e] = dbi
        if db_out is not None:
            db_out[e] = dbo
    dx = np.zeros((T, d))
    for j in range(k):
        kept = inv[:, j] >= 0
        dx[kept] += dXp[inv[kept, j]]
    # shared expert, gate 1
    dws_in = dws_out = None
    if ws_in is not None:
        dXs, dws_in, _, dws_out, _ = expert_backward(x, R.f64(ws_in), None, R.f64(ws_out), None, "swiglu", dy)
        dx = dx + dXs
    # router
    dl = gate_backward(r.logits, idx, score, renorm, dg)
    if aux_coef:
        dl = dl + aux_backward(r.logits, idx, score, aux_coef)
    dw_r = dl.T @ x
    dx = dx + dl @ w_r
    return BackwardResult(dx, dw_r, dw_in, db_in, dw_out, db_out, dws_in, dws_out, dl, dg, fwd.y)


def tokens_backward(x_rows, w_r, idx_rows: np.ndarray, logits_rows: np.ndarray, get_expert, act: str, score: str,
                    renorm: bool, ws_in, ws_out, dy_rows, dl_extra: Optional[np.ndarray] = None,
                    return_term_ssq: bool = False):
    """dx and the router-logit gradient of a subset of tokens, given their selection and logits.

    Without capacity and with the balancing term's f held constant, token t's gradients depend only
    on its own x, dy and routing, so sampled tokens of a large layer are evaluated directly: for each
    expert the sample uses, the FFN and its backward on the sampled rows routed to it (one expert
    converted to float64 at a time). dl_extra [S, E] is added to the logit gradient before it
    reaches dx (the balancing term's rows, which need the whole layer's counts).

    return_term_ssq: also return, per token, the sum of the squared norms of the terms dx adds up
    (one per selected expert, the shared expert's, the router's) -- the scale of a sum whose terms
    may cancel. The gradients themselves are the same either way."""
    x_rows, dy_rows, w_r = R.f64(x_rows), R.f64(dy_rows), R.f64(w_r)
    S, k = idx_rows.shape
    g = R.gates(logits_rows, idx_rows, score, renorm)
    dg = np.zeros((S, k))
    dx = np.zeros(x_rows.shape)
    ssq = np.zeros(S)
    for e in np.unique(idx_rows):
        rows, slots = np.nonzero(idx_rows == e)
        wi, bi, wo, bo = get_expert(int(e))
        Y = R.expert_ffn(x_rows[rows], wi, bi, wo, bo, act)
        dg[rows, slots] = np.sum(dy_rows[rows] * Y, axis=1)
        dX = expert_backward(x_rows[rows], wi, bi, wo, bo, act, g[rows, slots][:, None] * dy_rows[rows])[0]
        np.add.at(dx, rows, dX)
        np.add.at(ssq, rows, np.sum(dX * dX, axis=1))
    if ws_in is not None:
        dXs = expert_backward(x_rows, R.f64(ws_in), None, R.f64(ws_out), None, "swiglu", dy_rows)[0]
        dx = dx + dXs
        ssq = ssq + np.sum(dXs * dXs, axis=1)
    dl = gate_backward(logits_rows, idx_rows, score, renorm, dg)
    if dl_extra is not None:
        dl = dl + dl_extra
    dr = dl @ w_r
    if return_term_ssq:
        return dx + dr, dl, ssq + np.sum(dr * dr, axis=1)
    return dx + dr, dl


def expert_backward_features(X, w_in, b_in, w_out, b_out, act: str, dY, feats: np.ndarray):
    """expert_backward's weight gradients restricted to the hidden features `feats`.

    Hidden feature f enters the expert only through row f of W1 (rows f and F + f of [Wg; Wu]),
    b1[f] and column f of W2, so the gradients of those entries need only that feature's
    pre-activation over the expert's rows. Returns (dw_in rows: [len(feats), d] for GELU, gate rows
    then up rows [2 len(feats), d] for SwiGLU; db_in[feats] or None; dw_out[:, feats])."""
    X, dY = R.f64(X), R.f64(dY)
    feats = np.asarray(feats)
    if act == "gelu":
        z = X @ w_in[feats].T
        if b_in is not None:
            z = z + b_in[feats][None, :]
        h = R.gelu(z)
        dz = (dY @ w_out[:, feats]) * gelu_grad(z)
        dw_in = dz.T @ X
        db_in = dz.sum(axis=0) if b_in is not None else None
    elif act == "swiglu":
        F = w_in.shape[0] // 2
        a = X @ w_in[feats].T
        u = X @ w_in[F + feats].T
        h = R.silu(a) * u
        dh = dY @ w_out[:, feats]
        da = dh * u * silu_grad(a)
        du = dh * R.silu(a)
        dw_in = np.concatenate([da.T @ X, du.T @ X], axis=0)
        db_in = None
    else:
        raise ValueError(act)
    return dw_in, db_in, dY.T @ h
