"""Checks that pin the float64 backward oracle (oracle/moe_grad.py) to things other than itself:
  * central finite differences of the forward oracle on tiny layers, every parameter, for the loss
    <dy, y> (+ the balancing term), skipping coordinates whose perturbation would change the routing;
  * torch autograd through a forward written here from torch operations (float64 on the CPU),
    independent of the oracle's numpy code, including the gate, capacity and balancing parts.
Each check takes the backward module so that a deliberately broken copy can be passed in.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import moe_ref as R
from tests.oracle_pins import tiny_case

CONFIGS = [
    dict(act="swiglu", score="softmax", renorm=True, bias=False, shared=False),
    dict(act="gelu", score="softmax", renorm=True, bias=True, shared=False),
    dict(act="swiglu", score="softmax", renorm=False, bias=False, shared=True),
    dict(act="gelu", score="sigmoid", renorm=True, bias=True, shared=True),
    dict(act="swiglu", score="sigmoid", renorm=True, bias=False, shared=False),
]


def _case(i, seed_base=5000):
    kw = CONFIGS[i % len(CONFIGS)]
    c = tiny_case(seed_base + i, T=5, d=3, F=2, E=3, k=2, **kw)
    c["dy"] = np.random.default_rng(seed_base + 100 + i).standard_normal((5, 3))
    return c


def _getter(c):
    return R.stacked_experts(c["w_in"], c["b_in"], c["w_out"], c["b_out"])


def _loss(c, capacity, aux_coef, counts0):
    r = R.layer_forward(c["x"], c["w_r"], _getter(c), c["k"], c["act"], c["score"], c["renorm"], c["sel_bias"],
                        c["ws_in"], c["ws_out"], capacity=capacity)
    L = float(np.sum(c["dy"] * r.y))
    if aux_coef:
        p = R.balance_probs(r.route.logits, c["score"])
        E = c["w_r"].shape[0]
        L += aux_coef * E * float(np.sum(counts0 / c["T"] * p.mean(axis=0)))
    return L, r.route.idx


def check_finite_differences(G, cases=range(10), eps=1e-6, tol=2e-6):
    for i in cases:
        c = _case(i)
        capacity = 3 if i % 3 == 2 else 0
        aux = 0.01 if i % 2 else 0.0
        base = R.layer_forward(c["x"], c["w_r"], _getter(c), c["k"], c["act"], c["score"], c["renorm"],
                               c["sel_bias"], c["ws_in"], c["ws_out"], capacity=capacity)
        counts0 = R.expert_counts(base.route.idx, c["w_r"].shape[0])
        g = G.layer_backward(c["x"], c["w_r"], _getter(c), c["k"], c["act"], c["score"], c["renorm"], c["sel_bias"],
                             c["ws_in"], c["ws_out"], c["dy"], capacity=capacity, aux_coef=aux)
        names = [("x", g.dx), ("w_r", g.dw_r), ("w_in", g.dw_in), ("w_out", g.dw_out)]
        if c["b_in"] is not None:
            names += [("b_in", g.db_in), ("b_out", g.db_out)]
        if c["ws_in"] is not None:
            names += [("ws_in", g.dws_in), ("ws_out", g.dws_out)]
        for name, grad in names:
            arr = c[name]
            for pos in np.ndindex(arr.shape):
                old = arr[pos]
                arr[pos] = old + eps
                lp, ip = _loss(c, capacity, aux, counts0)
                arr[pos] = old - eps
                lm, im = _loss(c, capacity, aux, counts0)
                arr[pos] = old
                if not (np.array_equal(ip, base.route.idx) and np.array_equal(im, base.route.idx)):
                    continue  # the routing is not differentiable across a change of choice
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - grad[pos]) <= tol * (1.0 + abs(fd)), (i, name, pos, fd, grad[pos])


def _torch_layer(c, idx, capacity, aux_coef, params, keep=None):
    """The layer forward in torch ops for a fixed selection idx [T, k]; returns the loss (keep, if
    given, receives the logits with their gradient retained)."""
    x, w_r, w_in, w_out = params["x"], params["w_r"], params["w_in"], params["w_out"]
    b_in, b_out = params.get("b_in"), params.get("b_out")
    T, k = idx.shape
    E = w_r.shape[0]
    l = x @ w_r.T
    if keep is not None:
        l.retain_grad()
        keep["l"] = l
    sel = torch.gather(l, 1, torch.as_tensor(idx))
    if c["score"] == "softmax" and c["renorm"]:
        gts = torch.softmax(sel, dim=1)
    elif c["score"] == "softmax":
        gts = torch.gather(torch.softmax(l, dim=1), 1, torch.as_tensor(idx))
    else:
        s = torch.sigmoid(sel)
        gts = s / s.sum(dim=1, keepdim=True)
    seen = [0] * E
    y = torch.zeros_like(x)
    rows = []
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            kept = capacity == 0 or seen[e] < capacity
            seen[e] += 1
            if not kept:
                continue
            xt = x[t]
            if c["act"] == "gelu":
                z = w_in[e] @ xt + (b_in[e] if b_in is not None else 0.0)
                h = 0.5 * z * (1.0 + torch.erf(z / math.sqrt(2.0)))
            else:
                F = w_in.shape[1] // 2
                a, u = w_in[e, :F] @ xt, w_in[e, F:] @ xt
                h = a * torch.sigmoid(a) * u
            out = w_out[e] @ h + (b_out[e] if b_out is not None else 0.0)
            rows.append((t, gts[t, j] * out))
    for t, v in rows:
        y = y + torch.nn.functional.one_hot(torch.tensor(t), T).to(x.dtype)[:, None] * v[None, :]
    if params.get("ws_in") is not None:
        wsi, wso = params["ws_in"], params["ws_out"]
        F = wsi.shape[0] // 2
        a, u = x @ wsi[:F].T, x @ wsi[F:].T
        y = y + (a * torch.sigmoid(a) * u) @ wso.T
    loss = (torch.as_tensor(c["dy"]) * y).sum()
    if aux_coef:
        f = torch.as_tensor(np.bincount(idx.ravel(), minlength=E) / T)
        if c["score"] == "softmax":
            p = torch.softmax(l, dim=1)
        else:
            s = torch.sigmoid(l)
            p = s / s.sum(dim=1, keepdim=True)
        loss = loss + aux_coef * E * (f * p.mean(dim=0)).sum()
    return loss


def check_autograd(G, cases=range(12)):
    for i in cases:
        c = _case(i, seed_base=6000)
        capacity = 2 if i % 4 == 3 else 0
        aux = 0.05 if i % 3 == 1 else 0.0
        g = G.layer_backward(c["x"], c["w_r"], _getter(c), c["k"], c["act"], c["score"], c["renorm"], c["sel_bias"],
                             c["ws_in"], c["ws_out"], c["dy"], capacity=capacity, aux_coef=aux)
        idx = R.route(c["x"], c["w_r"], c["k"], c["score"], c["renorm"], c["sel_bias"]).idx
        keys = ["x", "w_r", "w_in", "w_out"] + (["b_in", "b_out"] if c["b_in"] is not None else []) + \
            (["ws_in", "ws_out"] if c["ws_in"] is not None else [])
        params = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in keys}
        loss = _torch_layer(c, idx, capacity, aux, params)
        loss.backward()
        mine = {"x": g.dx, "w_r": g.dw_r, "w_in": g.dw_in, "w_out": g.dw_out, "b_in": g.db_in, "b_out": g.db_out,
                "ws_in": g.dws_in, "ws_out": g.dws_out}
        for n in keys:
            ref = params[n].grad.numpy()
            err = np.max(np.abs(mine[n] - ref))
            assert err <= 1e-12 * (1.0 + np.max(np.abs(ref))), (i, n, err)


def check_sampled_restrictions(G, cases=range(10)):
    """tokens_backward on a subset of tokens and expert_backward_features on a subset of hidden
    features against torch autograd of the whole (dropless) layer: the token rows of dx and of the
    logit gradient, and the matching rows / columns of each expert's weight gradients."""
    for i in cases:
        c = _case(i, seed_base=7000)
        r = R.route(c["x"], c["w_r"], c["k"], c["score"], c["renorm"], c["sel_bias"])
        idx, logits = r.idx, r.logits
        keys = ["x", "w_r", "w_in", "w_out"] + (["b_in", "b_out"] if c["b_in"] is not None else []) + \
            (["ws_in", "ws_out"] if c["ws_in"] is not None else [])
        params = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in keys}
        keep = {}
        _torch_layer(c, idx, 0, 0.0, params, keep).backward()
        S = np.array([i % 5, (i + 2) % 5, 4])
        S = np.unique(S)
        dx, dl = G.tokens_backward(c["x"][S], c["w_r"], idx[S], logits[S], _getter(c), c["act"], c["score"],
                                   c["renorm"], c["ws_in"], c["ws_out"], c["dy"][S])
        for what, mine, ref in (("dx", dx, params["x"].grad.numpy()[S]), ("dl", dl, keep["l"].grad.numpy()[S])):
            err = np.max(np.abs(mine - ref))
            assert err <= 1e-12 * (1.0 + np.max(np.abs(ref))), (i, what, err)
        g = R.gates(logits, idx, c["score"], c["renorm"])
        F = c["w_out"].shape[2]
        feats = np.array([i % F])
        for e in range(c["w_r"].shape[0]):
            rows, slots = np.nonzero(idx == e)
            if rows.size == 0:
                continue
            wi, bi, wo, bo = _getter(c)(e)
            dwi, dbi, dwo = G.expert_backward_features(c["x"][rows], wi, bi, wo, bo, c["act"],
                                                       g[rows, slots][:, None] * c["dy"][rows], feats)
            gi = params["w_in"].grad.numpy()[e]
            want_in = gi[feats] if c["act"] == "gelu" else np.concatenate([gi[feats], gi[F + feats]], axis=0)
            pairs = [("dw_in", dwi, want_in), ("dw_out", dwo, params["w_out"].grad.numpy()[e][:, feats])]
            if bi is not None:
                pairs.append(("db_in", dbi, params["b_in"].grad.numpy()[e][feats]))
            for what, mine, ref in pairs:
                err = np.max(np.abs(mine - ref))
                assert err <= 1e-12 * (1.0 + np.max(np.abs(ref))), (i, e, what, err)


def check_term_ssq(G, cases=range(8)):
    """tokens_backward's optional per-token sum of squared term norms: asking for it leaves dx and
    the logit gradient unchanged; with one expert, k = 1 and no shared expert the gate is constantly 1,
    so the logit gradient is zero and dx is the single expert term (ssq = ||dx||^2 exactly); and in
    general the Cauchy-Schwarz bound ||dx||^2 <= (terms) * ssq holds (k experts, shared, router)."""
    for i in cases:
        c = _case(i, seed_base=9000)
        r = R.route(c["x"], c["w_r"], c["k"], c["score"], c["renorm"], c["sel_bias"])
        args = (c["x"], c["w_r"], r.idx, r.logits, _getter(c), c["act"], c["score"], c["renorm"], c["ws_in"],
                c["ws_out"], c["dy"])
        dx0, dl0 = G.tokens_backward(*args)
        dx, dl, ssq = G.tokens_backward(*args, return_term_ssq=True)
        assert np.array_equal(dx, dx0) and np.array_equal(dl, dl0), i
        n_terms = c["k"] + 1 + (1 if c["ws_in"] is not None else 0)
        assert (np.sum(dx * dx, axis=1) <= n_terms * ssq * (1 + 1e-12)).all(), i
        assert (ssq >= 0).all()
    for act in ("gelu", "swiglu"):
        c = tiny_case(9100, T=6, d=4, F=3, E=1, k=1, act=act, score="softmax", renorm=True, bias=False, shared=False)
        dy = np.random.default_rng(9101).standard_normal((6, 4))
        r = R.route(c["x"], c["w_r"], 1, "softmax", True)
        dx, dl, ssq = G.tokens_backward(c["x"], c["w_r"], r.idx, r.logits, _getter(c), act, "softmax", True, None,
                                        None, dy, return_term_ssq=True)
        assert np.abs(dl).max() == 0.0
        assert np.allclose(ssq, np.sum(dx * dx, axis=1), rtol=1e-14, atol=0), act


ALL_GRAD_CHECKS = [
    ("finite_differences", check_finite_differences),
    ("autograd", check_autograd),
    ("sampled_restrictions", check_sampled_restrictions),
    ("term_ssq", check_term_ssq),
]
