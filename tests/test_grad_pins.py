"""The backward oracle against finite differences and torch autograd (tests/grad_pins.py), and
plausible mistakes planted in private copies of it, each of which some pin must catch."""
import importlib.util
import os
import sys

import numpy as np
import pytest

from tests import grad_pins as pins

GRAD_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_grad.py")


@pytest.mark.parametrize("name,check", pins.ALL_GRAD_CHECKS, ids=[n for n, _ in pins.ALL_GRAD_CHECKS])
def test_grad_pin(name, check):
    from oracle import moe_grad

    check(moe_grad)


def fresh(tag):
    name = f"moe_grad_mutant_{tag}"
    spec = importlib.util.spec_from_file_location(name, GRAD_PATH)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


MUTANTS = {
    "silu_grad_sigmoid_only": lambda m: setattr(m, "silu_grad", lambda a: m.R.sigmoid(a)),
    "gelu_grad_without_density": lambda m: setattr(m, "gelu_grad", lambda z: 0.5 * (1.0 + m.erf(z / np.sqrt(2.0)))),
    "gate_grad_without_centering": lambda m: setattr(m, "gate_backward", _no_centering(m)),
    "aux_grad_ignored": lambda m: setattr(m, "aux_backward", lambda l, idx, score, coef: np.zeros_like(l)),
    "expert_dw_out_from_pre_activation": lambda m: setattr(m, "expert_backward", _dw_out_wrong(m)),
    "feature_gate_and_up_rows_swapped": lambda m: setattr(m, "expert_backward_features", _feats_swapped(m)),
    "tokens_shared_expert_dropped": lambda m: setattr(m, "tokens_backward", _tokens_no_shared(m)),
}


def _feats_swapped(m):
    orig = m.expert_backward_features

    def f(X, w_in, b_in, w_out, b_out, act, dY, feats):
        dwi, dbi, dwo = orig(X, w_in, b_in, w_out, b_out, act, dY, feats)
        n = len(feats)
        if act == "swiglu":
            dwi = np.concatenate([dwi[n:], dwi[:n]], axis=0)
        return dwi, dbi, dwo
    return f


def _tokens_no_shared(m):
    orig = m.tokens_backward

    def f(x_rows, w_r, idx_rows, logits_rows, get_expert, act, score, renorm, ws_in, ws_out, dy_rows,
          dl_extra=None):
        return orig(x_rows, w_r, idx_rows, logits_rows, get_expert, act, score, renorm, None, None, dy_rows, dl_extra)
    return f


def _no_centering(m):
    def gb(l, idx, score, renorm, dg):
        T, E = l.shape
        dl = np.zeros((T, E))
        sel = np.take_along_axis(l, idx, axis=-1)
        g = m.R.softmax(sel) if score == "softmax" else m.R.sigmoid(sel) / m.R.sigmoid(sel).sum(-1, keepdims=True)
        np.put_along_axis(dl, idx, g * dg, axis=-1)
        return dl
    return gb


def _dw_out_wrong(m):
    orig = m.expert_backward

    def eb(X, w_in, b_in, w_out, b_out, act, dY):
        dX, dwi, dbi, dwo, dbo = orig(X, w_in, b_in, w_out, b_out, act, dY)
        return dX, dwi, dbi, dwo * 0.5, dbo
    return eb


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_grad_mutant_is_caught(name):
    mod = fresh(name)
    MUTANTS[name](mod)
    caught = []
    for cname, check in pins.ALL_GRAD_CHECKS:
        try:
            check(mod)
        except Exception as exc:  # noqa: BLE001
            caught.append((cname, type(exc).__name__))
    assert caught, f"mutant {name} passed every backward pin"
