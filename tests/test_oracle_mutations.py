"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and require that at least
one pin catches each -- evidence that the pins constrain every step, not just the happy path."""
import importlib.util
import math
import os
import sys

import numpy as np
import pytest

from tests import oracle_pins as pins

REF_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_ref.py")


def fresh_oracle(tag: str):
    name = f"moe_ref_mutant_{tag}"
    spec = importlib.util.spec_from_file_location(name, REF_PATH)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod  # dataclasses resolve string annotations through sys.modules
    spec.loader.exec_module(mod)
    return mod


def _ties_to_higher_index(key, k):
    E = key.shape[1]
    order = np.argsort(-key[:, ::-1], axis=-1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int64)


def _mut_gates_full_softmax(m):
    orig = m.gates

    def g(l, idx, score, renorm):
        return orig(l, idx, score, False) if score == "softmax" else orig(l, idx, score, renorm)
    return g


def _mut_sigmoid_unnormalised(m):
    orig = m.gates

    def g(l, idx, score, renorm):
        if score == "sigmoid":
            return m.sigmoid(np.take_along_axis(l, idx, axis=-1))
        return orig(l, idx, score, renorm)
    return g


def _mut_gates_from_biased(m):
    """Gates computed from the biased key instead of the raw logits."""
    orig_route = m.route

    def route(x, w_r, k, score="softmax", renorm=True, sel_bias=None):
        r = orig_route(x, w_r, k, score, renorm, sel_bias)
        if sel_bias is not None and score == "softmax":
            r.gates = m.gates(r.key, r.idx, score, renorm)
        return r
    return route


def _mut_swiglu_swapped(m):
    orig = m.expert_ffn

    def ffn(X, w_in, b_in, w_out, b_out, act):
        if act == "swiglu":
            F = w_in.shape[0] // 2
            w_in = np.concatenate([w_in[F:], w_in[:F]], axis=0)
        return orig(X, w_in, b_in, w_out, b_out, act)
    return ffn


def _mut_drop_out_bias(m):
    orig = m.expert_ffn
    return lambda X, w_in, b_in, w_out, b_out, act: orig(X, w_in, b_in, w_out, None, act)


def _gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def _mut_permute_descending(m):
    orig = m.permute

    def permute(idx, E, capacity=0):
        T, k = idx.shape
        offsets, st, inv = orig(idx, E, capacity)
        st2, inv2 = st.copy(), inv.copy()
        for e in range(E):
            r0, r1 = offsets[e], offsets[e + 1]
            st2[r0:r1] = st[r0:r1][::-1]
        for a in range(T * k):
            e = idx.reshape(-1)[a]
            if inv[a] >= 0:
                inv2[a] = offsets[e] + offsets[e + 1] - 1 - (inv[a] - offsets[e]) - offsets[e]
        return offsets, st2, inv2
    return permute


def _mut_inclusive_offsets(m):
    orig = m.permute

    def permute(idx, E, capacity=0):
        offsets, st, inv = orig(idx, E, capacity)
        counts = np.bincount(idx.ravel(), minlength=E)
        off2 = offsets.copy()
        off2[:E] = offsets[:E] + counts  # inclusive instead of exclusive
        return off2, st, inv
    return permute


def _mut_f_over_assignments(m):
    orig = m.route_stats

    def stats(l, idx, E, score):
        f, P, aux, ent = orig(l, idx, E, score)
        k = idx.shape[1]
        return f / k, P, aux / k, ent
    return stats


def _mut_entropy_bits(m):
    orig = m.route_stats

    def stats(l, idx, E, score):
        f, P, aux, ent = orig(l, idx, E, score)
        return f, P, aux, ent / math.log(2.0)
    return stats


def _mut_P_selected_only(m):
    orig = m.route_stats

    def stats(l, idx, E, score):
        f, P, aux, ent = orig(l, idx, E, score)
        mask = np.zeros_like(l)
        np.put_along_axis(mask, idx, 1.0, axis=-1)
        p = m.balance_probs(l, score) * mask
        P2 = p.mean(axis=0)
        return f, P2, E * float(np.sum(f * P2)), ent
    return stats


def _mut_combine_sorted_token(m):
    def combine(y_perm, inv_pos, g, y_shared=None):
        T, k = g.shape
        y = np.zeros((T, y_perm.shape[1]))
        for j in range(k):
            y += g[:, j:j + 1] * y_perm[np.arange(T) * k + j]  # ignores the permutation
        return y if y_shared is None else y + y_shared
    return combine


def _mut_drop_shared(m):
    orig = m.combine
    return lambda y_perm, inv_pos, g, y_shared=None: orig(y_perm, inv_pos, g, None)


def _mut_router_transposed_bias(m):
    """Bias added after the sigmoid is replaced by bias added to the logit before it."""
    def key(l, score, sel_bias):
        base = l + (0 if sel_bias is None else sel_bias[None, :])
        return m.sigmoid(base) if score == "sigmoid" else base
    return key


def _mut_capacity_keeps_last(m):
    """Keeps the last C assignments of an overloaded expert instead of the first C."""
    def permute(idx, E, capacity=0):
        if capacity <= 0:
            return m.__dict__["_orig_permute"](idx, E, 0)
        T, k = idx.shape
        rev = idx[::-1, ::-1].copy()
        off, st, inv = m.__dict__["_orig_permute"](rev, E, capacity)
        inv2 = inv[::-1].copy()
        # rows of each expert back in ascending token order
        st2 = st.copy()
        for e in range(E):
            r0, r1 = off[e], off[e + 1]
            st2[r0:r1] = (T - 1 - st[r0:r1])[::-1]
        for a in range(T * k):
            if inv2[a] >= 0:
                e = idx.reshape(-1)[a]
                inv2[a] = off[e] + off[e + 1] - 1 - (inv2[a] - off[e]) - off[e] + off[e]
        return off, st2, inv2
    return permute


def _mut_capacity_off_by_one(m):
    orig = m.permute
    return lambda idx, E, capacity=0: orig(idx, E, capacity + 1 if capacity > 0 else 0)


def _mut_capacity_renormalises(m):
    """Renormalises the kept gates of a token whose assignment was dropped."""
    orig = m.combine

    def combine(y_perm, inv_pos, g, y_shared=None):
        T, k = g.shape
        pos = inv_pos.reshape(T, k)
        g2 = np.where(pos >= 0, g, 0.0)
        s = g2.sum(axis=1, keepdims=True)
        g2 = np.where(s > 0, g2 / np.where(s > 0, s, 1.0) * g.sum(axis=1, keepdims=True), g2)
        return orig(y_perm, inv_pos, g2, y_shared)
    return combine


def _mut_bias_sign_flipped(m):
    orig = m.update_bias
    return lambda bias, counts, T, k, gamma: orig(bias, counts, T, k, -gamma)


def _mut_bias_target_per_token(m):
    """Uniform load taken as T/E (tokens) instead of T*k/E (assignments)."""
    orig = m.update_bias
    return lambda bias, counts, T, k, gamma: orig(bias, counts, T, 1, gamma) if k > 1 else orig(bias, np.asarray(counts) + 1, T, k, gamma)


def _mut_noise_unscaled(m):
    """Noise added without the learned softplus scale."""
    return lambda x, w_r, w_noise, noise: m.router_logits(x, w_r) + m.f64(noise)


def _mut_softplus_as_exp(m):
    return lambda z: np.exp(z)


def _mut_tokens_gate_of_slot0(m):
    """Every slot weighted by the gate of slot 0."""
    orig = m.tokens_forward
    return lambda x_rows, idx_rows, gates_rows, get_expert, act, ws_in=None, ws_out=None: orig(
        x_rows, idx_rows, np.repeat(np.asarray(gates_rows)[:, :1], gates_rows.shape[1], axis=1), get_expert, act,
        ws_in, ws_out)


def _mut_tokens_gates_reversed(m):
    """Slot j weighted by the gate of slot k-1-j."""
    orig = m.tokens_forward
    return lambda x_rows, idx_rows, gates_rows, get_expert, act, ws_in=None, ws_out=None: orig(
        x_rows, idx_rows, np.asarray(gates_rows)[:, ::-1].copy(), get_expert, act, ws_in, ws_out)


def _mut_tokens_shared_twice(m):
    orig = m.tokens_forward

    def tf(x_rows, idx_rows, gates_rows, get_expert, act, ws_in=None, ws_out=None):
        y = orig(x_rows, idx_rows, gates_rows, get_expert, act, ws_in, ws_out)
        if ws_in is not None:
            y = y + m.shared_ffn(m.f64(x_rows), m.f64(ws_in), m.f64(ws_out))
        return y
    return tf


def _mut_rel_l2_axis0(m):
    def rel(a, ref):
        a, ref = m.f64(a), m.f64(ref)
        num = np.linalg.norm(a - ref, axis=0)
        den = np.linalg.norm(ref, axis=0)
        floor = 1e-6 * math.sqrt(float(np.mean(den ** 2))) if den.size else 0.0
        return num / np.maximum(den, max(floor, 1e-300))
    return rel


def _mut_rel_l2_big_floor(m):
    def rel(a, ref):
        a, ref = m.f64(a), m.f64(ref)
        num = np.linalg.norm(a - ref, axis=1)
        den = np.linalg.norm(ref, axis=1)
        floor = 1e-2 * math.sqrt(float(np.mean(den ** 2))) if den.size else 0.0
        return num / np.maximum(den, max(floor, 1e-300))
    return rel


def _mut_rel_l2_over_result(m):
    """Denominator taken from the compared values instead of the reference."""
    orig = m.rel_l2_per_row
    return lambda a, ref: orig(a, ref) * np.linalg.norm(m.f64(ref), axis=1) / np.maximum(
        np.linalg.norm(m.f64(a), axis=1), 1e-300)


def _install_keeps_last(m):
    m._orig_permute = m.permute
    m.permute = _mut_capacity_keeps_last(m)


MUTANTS = {
    "ties_to_higher_index": lambda m: setattr(m, "topk", _ties_to_higher_index),
    "gates_full_softmax": lambda m: setattr(m, "gates", _mut_gates_full_softmax(m)),
    "sigmoid_gates_unnormalised": lambda m: setattr(m, "gates", _mut_sigmoid_unnormalised(m)),
    "gates_from_biased_key": lambda m: setattr(m, "route", _mut_gates_from_biased(m)),
    "swiglu_gate_up_swapped": lambda m: setattr(m, "expert_ffn", _mut_swiglu_swapped(m)),
    "dropped_output_bias": lambda m: setattr(m, "expert_ffn", _mut_drop_out_bias(m)),
    "gelu_tanh_approx": lambda m: setattr(m, "gelu", _gelu_tanh),
    "silu_as_sigmoid": lambda m: setattr(m, "silu", lambda z: 1.0 / (1.0 + np.exp(-z))),
    "permute_descending_tokens": lambda m: setattr(m, "permute", _mut_permute_descending(m)),
    "inclusive_offsets": lambda m: setattr(m, "permute", _mut_inclusive_offsets(m)),
    "f_over_assignments": lambda m: setattr(m, "route_stats", _mut_f_over_assignments(m)),
    "entropy_in_bits": lambda m: setattr(m, "route_stats", _mut_entropy_bits(m)),
    "P_selected_only": lambda m: setattr(m, "route_stats", _mut_P_selected_only(m)),
    "combine_ignores_permutation": lambda m: setattr(m, "combine", _mut_combine_sorted_token(m)),
    "shared_expert_dropped": lambda m: setattr(m, "combine", _mut_drop_shared(m)),
    "bias_inside_sigmoid": lambda m: setattr(m, "selection_key", _mut_router_transposed_bias(m)),
    "softmax_without_normalisation": lambda m: setattr(m, "softmax", lambda l: np.exp(l - l.max(axis=-1, keepdims=True))),
    "logits_sign_flipped": lambda m: setattr(m, "router_logits", lambda x, w: -(x @ w.T)),
    "capacity_keeps_last": _install_keeps_last,
    "capacity_off_by_one": lambda m: setattr(m, "permute", _mut_capacity_off_by_one(m)),
    "capacity_renormalises_gates": lambda m: setattr(m, "combine", _mut_capacity_renormalises(m)),
    "bias_update_sign_flipped": lambda m: setattr(m, "update_bias", _mut_bias_sign_flipped(m)),
    "bias_target_per_token": lambda m: setattr(m, "update_bias", _mut_bias_target_per_token(m)),
    "noise_unscaled": lambda m: setattr(m, "noisy_logits", _mut_noise_unscaled(m)),
    "softplus_as_exp": lambda m: setattr(m, "softplus", _mut_softplus_as_exp(m)),
    "tokens_gate_of_slot0": lambda m: setattr(m, "tokens_forward", _mut_tokens_gate_of_slot0(m)),
    "tokens_gates_reversed": lambda m: setattr(m, "tokens_forward", _mut_tokens_gates_reversed(m)),
    "tokens_shared_twice": lambda m: setattr(m, "tokens_forward", _mut_tokens_shared_twice(m)),
    "rel_l2_wrong_axis": lambda m: setattr(m, "rel_l2_per_row", _mut_rel_l2_axis0(m)),
    "rel_l2_floor_swamps": lambda m: setattr(m, "rel_l2_per_row", _mut_rel_l2_big_floor(m)),
    "rel_l2_over_result": lambda m: setattr(m, "rel_l2_per_row", _mut_rel_l2_over_result(m)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, page_values):
    mod = fresh_oracle(name)
    MUTANTS[name](mod)
    caught = []
    for check_name, check in pins.ALL_CHECKS:
        try:
            check(mod, page_values)
        except Exception as exc:  # noqa: BLE001 -- any failure counts as caught
            caught.append((check_name, type(exc).__name__))
    assert caught, f"mutant {name} passed every pin"
