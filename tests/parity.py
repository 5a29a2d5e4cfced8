"""GPU-vs-oracle comparison protocol (used by the gpu-marked tests and the smoke check).

Route: the oracle flags a token ambiguous when its k-th and (k+1)-th selection keys differ by
<= 1e-4 (float64). On every other token the GPU's expert set must equal the oracle's, and the slot
order must match wherever adjacent keys differ by more than 1e-4; on ambiguous tokens the GPU's
set must be a valid top-k within that margin. Logits within 5e-5 absolute (half the margin),
gates within 1e-5 absolute, counts exactly the histogram of the GPU's selection, f/P/aux/entropy
within 1e-5 relative.
Permute: offsets, sorted_token, inv_pos and x_perm bit-exact against the oracle's permutation of
the GPU's selection.
FFN and layer: per-row relative L2 error, maximum over rows, <= 1e-4 (fp32 layers) or 2e-2
(bf16 layers), with the oracle re-run on the GPU's selection (so ambiguous tokens compare like
with like).
Backward: each gradient is cut into blocks (a token's row of dx and dlogits, an expert's slice of
the weight gradients); a block's L2 error must be <= the same tolerance times the larger of its own
norm and the median block norm. The median floor covers blocks whose value is a small difference
of large terms (a token whose two gate gradients nearly cancel): their error scales with the terms,
not with the difference. Blocks the oracle makes exactly zero (an expert without rows) must be
exactly zero.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_ref as R

MARGIN = R.AMBIGUITY_MARGIN
LOGIT_ATOL = 5e-5
GATE_ATOL = 1e-5
STAT_RTOL = 1e-5


def tol_for(cfg) -> float:
    return 1e-4 if cfg.dtype == "f32" else 2e-2


def np64(t):
    return R.f64(t)


def check_route(cfg, L, ref: "R.RouteResult", logits=True):
    """Returns the number of ambiguous tokens; raises AssertionError on a mismatch."""
    T, k, E = L.T, cfg.k, cfg.E
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    gw = L.topk_w.cpu().numpy().astype(np.float64)
    assert idx.shape == (T, k)
    assert ((idx >= 0) & (idx < E)).all(), "expert index out of range"
    for t in range(T):
        assert len(set(idx[t].tolist())) == k, f"token {t}: repeated expert {idx[t]}"
    if logits:
        lg = L.logits.cpu().numpy().astype(np.float64)
        err = np.max(np.abs(lg - ref.logits))
        assert err <= LOGIT_ATOL, f"logits max abs err {err:.3g}"
    amb = ref.ambiguous
    key = ref.key
    unamb = ~amb
    # same set on unambiguous tokens
    same_set = np.array([set(idx[t]) == set(ref.idx[t]) for t in range(T)])
    bad = np.nonzero(unamb & ~same_set)[0]
    assert bad.size == 0, f"selection differs on unambiguous tokens {bad[:10]}"
    # slot order where adjacent keys are separated
    for t in np.nonzero(unamb)[0]:
        kk = key[t, idx[t]]
        for j in range(k - 1):
            if abs(kk[j] - kk[j + 1]) > MARGIN:
                assert kk[j] > kk[j + 1], f"token {t}: slot order {idx[t]} keys {kk}"
    # ambiguous tokens: a valid top-k within the margin
    for t in np.nonzero(amb)[0]:
        kth = -np.sort(-key[t])[k - 1]
        chosen = np.zeros(E, bool)
        chosen[idx[t]] = True
        assert (key[t, chosen] >= kth - MARGIN).all() and (key[t, ~chosen] <= kth + MARGIN).all(), t
    # gates: the oracle's gates for the GPU's selection (identical on unambiguous tokens)
    want = R.gates(ref.logits, idx, cfg.score, cfg.renorm)
    gerr = np.max(np.abs(gw - want))
    assert gerr <= GATE_ATOL, f"gates max abs err {gerr:.3g}"
    counts = L.counts.cpu().numpy().astype(np.int64)
    assert (counts == np.bincount(idx.ravel(), minlength=E)).all(), "counts != histogram of topk_idx"
    st = L.stats.cpu().numpy().astype(np.float64)
    f, P, aux, ent = R.route_stats(ref.logits, idx, E, cfg.score)

    def rel(a, b, what):
        err = np.max(np.abs(np.asarray(a) - np.asarray(b)) / np.maximum(np.abs(np.asarray(b)), 1e-3))
        assert err <= STAT_RTOL, f"{what} rel err {err:.3g}"

    rel(st[:E], f, "f")
    rel(st[E:2 * E], P, "P")
    rel(st[2 * E], aux, "aux")
    rel(st[2 * E + 1], ent, "entropy")
    return int(amb.sum())


def check_permute(cfg, L, x_host64):
    """GPU permutation of the GPU's own selection vs the oracle's permutation of it (bit-exact),
    with the layer's expert capacity (rows past offsets[E] are not compared)."""
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    cap = getattr(L, "capacity", 0)
    off, st, inv = R.permute(idx, cfg.E, cap)
    n = int(off[-1])
    assert (L.offsets.cpu().numpy() == off).all(), "offsets"
    assert (L.sorted_token.cpu().numpy()[:n] == st).all(), "sorted_token"
    assert (L.inv_pos.cpu().numpy() == inv).all(), "inv_pos"
    xp = L.x_perm.cpu()[:n]
    want = L.t["x"].cpu()[torch.from_numpy(st)]
    assert torch.equal(xp.view(torch.int16) if xp.dtype == torch.bfloat16 else xp.view(torch.int32),
                       want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), "x_perm"
    return off, st, inv


def get_expert_fn(L):
    t = L.t
    return R.stacked_experts(t["w_in"], t["b_in"], t["w_out"], t["b_out"])


def check_ffn(cfg, L, off, x_perm64, e_range=None):
    y_ref = R.experts_on_rows(x_perm64, off, get_expert_fn(L), cfg.act, e_range)
    y = np64(L.y_perm)[:y_ref.shape[0]]  # with a capacity only the kept rows exist
    rows = ~np.isnan(y_ref[:, 0])
    if rows.any():
        err = R.rel_l2_per_row(y[rows], y_ref[rows])
        assert err.max() <= tol_for(cfg), f"y_perm max rel-L2 {err.max():.3g}"
        return float(err.max())
    return 0.0


def oracle_layer_on_gpu_routing(cfg, L):
    """The oracle layer with the GPU's selection forced (its gates follow from that selection)."""
    t = L.t
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    return R.layer_forward(t["x"], np64(t["w_r"]), get_expert_fn(L), cfg.k, cfg.act, cfg.score, cfg.renorm,
                           None if t["sel_bias"] is None else np64(t["sel_bias"]), t["ws_in"], t["ws_out"],
                           forced_idx=idx, capacity=getattr(L, "capacity", 0))


def check_layer(cfg, y_gpu, y_ref):
    err = R.rel_l2_per_row(np64(y_gpu), y_ref)
    assert err.max() <= tol_for(cfg), f"layer max per-token rel-L2 {err.max():.3g}"
    return float(err.max())


def sum_rel_l2(got, ref, term_ssq) -> np.ndarray:
    """Per-row ||got - ref|| / max(||ref||, sqrt(term_ssq)): the relative error of a row that is a
    sum of terms, measured against the larger of the sum and the root-sum-square of its terms."""
    g, r = np64(got), np64(ref)
    assert np.isfinite(g).all(), "non-finite values"
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), np.sqrt(np.asarray(term_ssq, dtype=np.float64)))
    return num / np.maximum(den, 1e-300)


def grad_err(got, ref, blocks: int, what: str, tol: float) -> float:
    """Block-wise gradient comparison (see the module notes); returns the largest block error."""
    g = np64(got).reshape(blocks, -1)
    r = np64(ref).reshape(blocks, -1)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    zero = den == 0.0
    assert (num[zero] == 0.0).all(), f"{what}: blocks {np.nonzero(zero & (num > 0))[0][:8]} must be exactly zero"
    if zero.all():
        return 0.0
    floor = float(np.median(den[~zero]))
    err = num / np.maximum(den, floor)
    worst = int(np.argmax(err))
    assert err.max() <= tol, f"{what}: block {worst} rel err {err.max():.3g} (tol {tol})"
    return float(err.max())
