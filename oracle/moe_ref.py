"""fp64 CPU oracle of the Mixture-of-Experts FFN layer forward.

TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module. The library path
never calls it, and it shares no code with the HIP kernels or their host
layer: it is a plain, slow, obviously correct restatement of what the layer
computes, in float64 on the exact stored input values (bf16 and fp32 inputs
convert to float64 exactly). It does not emulate any bf16 intermediate of
the GPU path.

Sources (cited by page title and section):
  [VI]  Vector Institute, "Mixture-of-Experts: From sparse routing to multimodal
        deployment" -- router score and softmax, top-k, Eq. (moe-output) and the
        renormalisation paragraph after it, load balancing, shared experts,
        routing audit (gating entropy, in nats).
  [RO]  "Fine-Tuning Mixture of Experts (MoE) Models: Router Optimization
        Techniques" -- What Is It? (router logits, TopK, Softmax(TopK), layer
        output; SwiGLU expert), How It Works 1 (f_i, P_i, L_aux) and 2
        (selection-only bias), Fine-Tuning Strategies 1 (dynamic-bias router).
  [FS]  "Fine-tuning and serving MoE models" -- How an MoE layer actually
        works (MoEFeedForward: router Linear without bias, top-k on logits, fp32
        softmax over the selected logits, loop over experts with gather and
        index_add), Why MoE breaks naive fine-tuning (load-balancing loss),
        Utilization is a first-class metric (per-expert counts).
  [MT]  "Mixture of Experts" tutorial -- A router and a panel of specialists
        (weighted-ensemble output), The whole point: most G(x)_i are zero
        (top-k then renormalise), Noisy top-k gating (-inf masking makes
        unselected gates exactly zero), Selective precision (fp32 router).

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of the repository):
  * the router has no bias; scores are its logits ([RO] What Is It?, [FS]);
  * selection is on a per-token key: the logit (softmax scoring), the logit plus
    a per-expert bias when a bias is given ([RO] How It Works 2), or the sigmoid
    score plus the bias (sigmoid scoring);
  * ties in the key go to the lower expert index; slots are in descending key
    order, ties by ascending index;
  * gates: softmax renormalised over the selected k (equal to softmax of the
    selected logits), or the raw full-softmax probability (renorm off), or for
    sigmoid scoring the selected unbiased scores divided by their sum;
  * f_e = count_e / T (so sum f = k), P_e = mean over tokens of the full-softmax
    probability (sigmoid: of s / sum s), aux = E * sum f_e P_e (the caller applies
    alpha), entropy = mean over tokens of -sum p ln p, in nats;
  * GELU is the exact erf form; SwiGLU is (SiLU(x Wg^T) * (x Wu^T)) Wd^T with no
    biases; a shared expert has gate 1 and is added after the routed sum;
  * capacity: C = ceil(c * T * k / E) rows per expert; an expert keeps its first C
    assignments in (t, j) order; a dropped assignment contributes nothing (it reaches
    the next layer through the residual, outside this layer); kept gates unchanged;
  * bias update: b_e <- b_e - gamma * sign(count_e - T*k/E), sign(0) = 0, in float32;
  * noisy top-k: H = x W_r^T + n * softplus(x W_noise^T) with caller-supplied noise n,
    then H replaces the logits everywhere (key, gates, statistics).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional, Tuple

import numpy as np
from scipy.special import erf

AMBIGUITY_MARGIN = 1e-4  # key_(k) - key_(k+1) at or below this marks a token ambiguous


def f64(a) -> np.ndarray:
    """Exact conversion of a numpy array or a (CPU or GPU) torch tensor to float64 numpy."""
    if hasattr(a, "detach"):
        import torch

        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------------------
# Route
# --------------------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] W_r[e, i] -- one score per expert, no bias ([RO] What Is It?; [FS])."""
    return x @ w_r.T


def softmax(l: np.ndarray) -> np.ndarray:
    """Probability over experts, max-subtracted ([VI] router softmax; [MT] How does the router decide?)."""
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def sigmoid(l: np.ndarray) -> np.ndarray:
    """Per-expert sigmoid score 1 / (1 + e^-l) (sigmoid-scored routing)."""
    return 1.0 / (1.0 + np.exp(-l))


def selection_key(l: np.ndarray, score: str, sel_bias: Optional[np.ndarray]) -> np.ndarray:
    """The value top-k ranks experts by.

    softmax: the logit itself (softmax is monotone, so this is the same order as the
    probabilities), plus the bias if one is given ([RO] How It Works 2: the bias
    enters the TopK argument only). sigmoid: the sigmoid score plus the bias.
    """
    if score == "softmax":
        key = l.copy()
    elif score == "sigmoid":
        key = sigmoid(l)
    else:
        raise ValueError(score)
    if sel_bias is not None:
        key = key + sel_bias[None, :]
    return key


def topk(key: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest key: descending key, ties to the lower index.

    A stable sort of -key keeps equal keys in ascending index order, which is
    exactly the (key descending, index ascending) total order.
    """
    order = np.argsort(-key, axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def gates(l: np.ndarray, idx: np.ndarray, score: str, renorm: bool) -> np.ndarray:
    """Combination weights of the selected experts ([VI] Eq. (moe-output) and renormalisation;
    [RO] What Is It?: Softmax(TopK(h)); [FS]: softmax over the selected logits).

    softmax + renorm: softmax over the selected logits (= full softmax renormalised over them);
    softmax, no renorm: the full-softmax probability at each selected index;
    sigmoid: the selected (unbiased) sigmoid scores divided by their sum.
    """
    sel = np.take_along_axis(l, idx, axis=-1)
    if score == "softmax":
        if renorm:
            return softmax(sel)
        return np.take_along_axis(softmax(l), idx, axis=-1)
    s = sigmoid(sel)
    return s / s.sum(axis=-1, keepdims=True)


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, slot) assignments per expert ([FS] utilisation tally; [RO] bincount)."""
    return np.bincount(idx.ravel(), minlength=E).astype(np.int64)


def balance_probs(l: np.ndarray, score: str) -> np.ndarray:
    """Per-token distribution over experts that P_e averages and the entropy measures.

    softmax: the full router softmax ([RO] How It Works 1, P_i). sigmoid: the scores
    normalised to sum to 1 over experts (reading for sigmoid routing).
    """
    if score == "softmax":
        return softmax(l)
    s = sigmoid(l)
    return s / s.sum(axis=-1, keepdims=True)


def route_stats(l: np.ndarray, idx: np.ndarray, E: int, score: str):
    """(f, P, aux, entropy): f_e = count_e / T, P_e = mean_t p[t, e], aux = E sum f P
    ([RO] How It Works 1; [FS] load_balancing_loss), entropy = mean_t -sum_e p ln p in nats
    ([VI] routing audit, gating entropy; [RO] best practice 6)."""
    T = l.shape[0]
    p = balance_probs(l, score)
    counts = expert_counts(idx, E)
    f = counts / T
    P = p.mean(axis=0)
    aux = E * float(np.sum(f * P))
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    entropy = float(np.mean(-plogp.sum(axis=-1)))
    return f, P, aux, entropy


def ambiguous_tokens(key: np.ndarray, k: int, margin: float = AMBIGUITY_MARGIN) -> np.ndarray:
    """True where the k-th and (k+1)-th largest keys are within `margin` (k = E: never)."""
    E = key.shape[1]
    if k >= E:
        return np.zeros(key.shape[0], dtype=bool)
    srt = -np.sort(-key, axis=-1)
    return (srt[:, k - 1] - srt[:, k]) <= margin


@dataclasses.dataclass
class RouteResult:
    logits: np.ndarray  # [T, E]
    key: np.ndarray  # [T, E]
    idx: np.ndarray  # [T, k] int64
    gates: np.ndarray  # [T, k]
    counts: np.ndarray  # [E] int64
    f: np.ndarray  # [E]
    P: np.ndarray  # [E]
    aux: float
    entropy: float
    ambiguous: np.ndarray  # [T] bool


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + e^z), evaluated as max(z, 0) + log1p(e^-|z|)."""
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def noisy_logits(x: np.ndarray, w_r: np.ndarray, w_noise: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """Noisy top-k gating ([MT] Noisy top-k gating): the router logits plus Gaussian noise scaled
    per token and expert by a second learned projection of x, H = x W_r^T + n * softplus(x W_noise^T).
    The page names the recipe and its two parts but its formula was lost; the scale is kept
    positive with softplus as in the published recipe. The noise n [T, E] is supplied by the
    caller (it is the only randomness); every later step uses H as the logits."""
    return router_logits(x, w_r) + f64(noise) * softplus(router_logits(x, f64(w_noise)))


def route(x, w_r, k: int, score: str = "softmax", renorm: bool = True,
          sel_bias: Optional[np.ndarray] = None, w_noise=None, noise=None) -> RouteResult:
    """The routing stage: logits, key, top-k, gates, counts and load-balance statistics. With
    w_noise and noise, the logits are the noisy ones (noisy_logits)."""
    x, w_r = f64(x), f64(w_r)
    if sel_bias is not None:
        sel_bias = f64(sel_bias)
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(w_r))
    E = w_r.shape[0]
    l = router_logits(x, w_r) if w_noise is None else noisy_logits(x, w_r, w_noise, noise)
    key = selection_key(l, score, sel_bias)
    idx = topk(key, k)
    g = gates(l, idx, score, renorm)
    f, P, aux, ent = route_stats(l, idx, E, score)
    return RouteResult(l, key, idx, g, expert_counts(idx, E), f, P, aux, ent,
                       ambiguous_tokens(key, k))


# --------------------------------------------------------------------------------------
# Permute
# --------------------------------------------------------------------------------------


def permute(idx: np.ndarray, E: int, capacity: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Expert-contiguous order of the T*k assignments.

    offsets[e] = sum of the row counts of experts below e. Within expert e, its
    assignments (t, j) appear in ascending t*k + j -- the order a per-expert
    nonzero() over the [T, k] index matrix yields ([FS] loop over experts) --
    packed into one contiguous buffer ([RO] What Most Articles Miss 2).

    capacity > 0 caps every expert at that many rows ([RO] Why It Matters 3 and
    FAQ 6; [VI] capacity factor; [MT] The capacity factor formula): an expert
    keeps the first `capacity` of its assignments in that order, and the rest
    are dropped -- they pass the layer untouched through the residual, so they
    get no row (inv_pos = -1). capacity = 0 keeps everything (dropless).

    Returns (offsets [E+1], sorted_token [offsets[E]] (row -> token),
    inv_pos [T*k] ((t, j) -> row, or -1 when dropped)).
    """
    T, k = idx.shape
    flat = idx.reshape(-1)
    offsets = np.zeros(E + 1, dtype=np.int64)
    sorted_token = np.empty(T * k, dtype=np.int64)
    inv_pos = np.full(T * k, -1, dtype=np.int64)
    row = 0
    for e in range(E):
        offsets[e] = row
        for n, a in enumerate(np.nonzero(flat == e)[0]):  # ascending assignment index a = t*k + j
            if capacity > 0 and n >= capacity:
                break
            sorted_token[row] = a // k
            inv_pos[a] = row
            row += 1
    offsets[E] = row
    assert capacity > 0 or row == T * k
    return offsets, sorted_token[:row], inv_pos


def capacity_rows(T: int, k: int, E: int, factor: float) -> int:
    """Expert capacity in rows: ceil(factor * T * k / E) ([RO] Why It Matters 3 and FAQ 6 state it
    as (tokens * k / experts) * capacity factor; rounding up keeps factor 1 exactly balanced)."""
    return int(math.ceil(factor * T * k / E))


def update_bias(bias: np.ndarray, counts: np.ndarray, T: int, k: int, gamma: float) -> np.ndarray:
    """Aux-loss-free balancing step ([RO] How It Works 2 and Fine-Tuning Strategies 1): an expert
    above the uniform load T*k/E lowers its selection bias by gamma, one below raises it by gamma,
    one exactly at it keeps it. The bias is stored in float32, so the step is one float32
    subtraction; the comparison with T*k/E is exact (counts * E against T * k in integers)."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    s = np.sign(counts * E - T * k).astype(np.float32)
    return (np.asarray(bias, dtype=np.float32) - np.float32(gamma) * s).astype(np.float32)


# --------------------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------------------


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU, z * Phi(z) = z/2 (1 + erf(z / sqrt 2)) (nn.GELU() default in [FS])."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU, z * sigmoid(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(X: np.ndarray, w_in: np.ndarray, b_in: Optional[np.ndarray], w_out: np.ndarray,
               b_out: Optional[np.ndarray], act: str) -> np.ndarray:
    """One expert FFN on rows X [n, d]; weights in Linear [out, in] layout.

    gelu:   gelu(X w_in^T + b_in) w_out^T + b_out        ([FS] Linear + GELU + Linear)
    swiglu: (silu(X Wg^T) * (X Wu^T)) w_out^T, where w_in = [Wg; Wu] stacked on rows
            ([RO] What Is It?, experts with W_gate, W_up, W_down)
    """
    if act == "gelu":
        h = X @ w_in.T
        if b_in is not None:
            h = h + b_in[None, :]
        h = gelu(h)
    elif act == "swiglu":
        F = w_in.shape[0] // 2
        h = silu(X @ w_in[:F].T) * (X @ w_in[F:].T)
    else:
        raise ValueError(act)
    y = h @ w_out.T
    if b_out is not None:
        y = y + b_out[None, :]
    return y


def shared_ffn(x: np.ndarray, ws_in: np.ndarray, ws_out: np.ndarray) -> np.ndarray:
    """Always-on shared SwiGLU expert, gate 1 ([VI] shared experts; [RO] lesson 2)."""
    return expert_ffn(x, ws_in, None, ws_out, None, "swiglu")


# --------------------------------------------------------------------------------------
# Layer
# --------------------------------------------------------------------------------------

ExpertGetter = Callable[[int], Tuple[np.ndarray, Optional[np.ndarray], np.ndarray, Optional[np.ndarray]]]


def stacked_experts(w_in, b_in, w_out, b_out) -> ExpertGetter:
    """Getter for stacked expert weights [E, ...]; converts one expert to float64 at a time."""

    def get(e: int):
        return (f64(w_in[e]), None if b_in is None else f64(b_in[e]),
                f64(w_out[e]), None if b_out is None else f64(b_out[e]))

    return get


def experts_on_rows(x_perm: np.ndarray, offsets: np.ndarray, get_expert: ExpertGetter, act: str,
                    e_range: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """y_perm: for each expert e, its FFN applied to its contiguous rows (an explicit per-expert
    loop, as in [FS]; empty experts are skipped). Rows outside e_range stay NaN."""
    E = offsets.shape[0] - 1
    e0, e1 = (0, E) if e_range is None else e_range
    out = np.full(x_perm.shape, np.nan)  # the expert output width is d_model
    for e in range(e0, e1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        w_in, b_in, w_out, b_out = get_expert(e)
        out[r0:r1] = expert_ffn(x_perm[r0:r1], w_in, b_in, w_out, b_out, act)
    return out


def combine(y_perm: np.ndarray, inv_pos: np.ndarray, g: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum_j g[t, j] y_perm[inv_pos[t*k + j]] (+ shared[t]) ([VI] Eq. (moe-output);
    [RO] MoE Layer Output; [FS] index_add of gate-scaled expert outputs)."""
    T, k = g.shape
    y = np.zeros((T, y_perm.shape[1]))
    pos = inv_pos.reshape(T, k)
    for j in range(k):
        kept = pos[:, j] >= 0  # a dropped assignment (capacity) contributes nothing
        y[kept] += g[kept, j:j + 1] * y_perm[pos[kept, j]]
    if y_shared is not None:
        y = y + y_shared
    return y


@dataclasses.dataclass
class LayerResult:
    route: RouteResult
    offsets: np.ndarray
    sorted_token: np.ndarray
    inv_pos: np.ndarray
    x_perm: np.ndarray
    y_perm: np.ndarray
    y_shared: Optional[np.ndarray]
    y: np.ndarray


def layer_forward(x, w_r, get_expert: ExpertGetter, k: int, act: str, score: str = "softmax",
                  renorm: bool = True, sel_bias=None, ws_in=None, ws_out=None,
                  forced_idx: Optional[np.ndarray] = None, capacity: int = 0) -> LayerResult:
    """The whole layer: y[t] = sum over the selected e of g_e(t) FFN_e(x[t]) (+ shared(x[t])).

    forced_idx replaces the oracle's own selection (used to re-run the expert and
    combine steps on another implementation's routing of ambiguous tokens); the
    gates are then those of the forced selection. capacity > 0 drops the
    assignments beyond each expert's first `capacity` (see permute); the gates of
    the kept ones are unchanged.
    """
    x = f64(x)
    E = w_r.shape[0]
    r = route(x, w_r, k, score, renorm, sel_bias)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int64)
        r = dataclasses.replace(r, idx=idx, gates=gates(r.logits, idx, score, renorm),
                                counts=expert_counts(idx, E))
    offsets, sorted_token, inv_pos = permute(r.idx, E, capacity)
    x_perm = x[sorted_token]
    y_perm = experts_on_rows(x_perm, offsets, get_expert, act)
    ys = shared_ffn(x, f64(ws_in), f64(ws_out)) if ws_in is not None else None
    y = combine(y_perm, inv_pos, r.gates, ys)
    return LayerResult(r, offsets, sorted_token, inv_pos, x_perm, y_perm, ys, y)


def tokens_forward(x_rows, idx_rows: np.ndarray, gates_rows: np.ndarray, get_expert: ExpertGetter,
                   act: str, ws_in=None, ws_out=None) -> np.ndarray:
    """The layer output for a subset of tokens, given their selection and gates.

    y[t] depends only on x[t] and its routing, so sampled tokens of a large layer are
    evaluated directly: for each expert used by the sample, its FFN on the sampled
    rows routed to it (one expert converted to float64 at a time)."""
    x_rows = f64(x_rows)
    out = np.zeros(x_rows.shape)
    for e in np.unique(idx_rows):
        rows, slots = np.nonzero(idx_rows == e)
        w_in, b_in, w_out, b_out = get_expert(int(e))
        Y = expert_ffn(x_rows[rows], w_in, b_in, w_out, b_out, act)
        out[rows] += gates_rows[rows, slots][:, None] * Y
    if ws_in is not None:
        out = out + shared_ffn(x_rows, f64(ws_in), f64(ws_out))
    return out


def rel_l2_per_row(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||a[t] - ref[t]||_2 / max(||ref[t]||_2, 1e-6 * rms row norm of ref), per row."""
    a, ref = f64(a), f64(ref)
    num = np.linalg.norm(a - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    floor = 1e-6 * math.sqrt(float(np.mean(den ** 2))) if den.size else 0.0
    return num / np.maximum(den, max(floor, 1e-300))
