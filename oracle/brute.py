"""Pure-Python brute force of the MoE-FFN layer for tiny inputs.

TEST INFRASTRUCTURE (same import rule as moe_ref). It shares no code with
moe_ref: it restates the layer a second way, with Python floats, loops and
the standard library only, so that the vectorised oracle can be pinned to
something other than itself.

* Selection: every k-subset of experts is enumerated; the chosen set is the
  one with the largest exact (Fraction) key sum, ties broken by the
  lexicographically smallest sorted index tuple. This is equivalent to
  "k largest keys, ties to the lower index" without relying on any sort.
* Output: the dense weighted ensemble over ALL experts ([MT] A router and a
  panel of specialists), with unselected gates forced to exactly zero by -inf
  masking before the softmax ([MT] Noisy top-k gating), so every expert runs
  on every token and only the gates decide.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import List, Optional, Sequence

Vec = List[float]
Mat = List[List[float]]


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def _matvec(W: Mat, v: Sequence[float]) -> Vec:
    """W [out][in] applied to v [in]."""
    return [_dot(row, v) for row in W]


def logits(x: Vec, w_r: Mat) -> Vec:
    return _matvec(w_r, x)


def key_of(l: Vec, score: str, sel_bias: Optional[Vec]) -> Vec:
    base = [1.0 / (1.0 + math.exp(-v)) for v in l] if score == "sigmoid" else list(l)
    if sel_bias is not None:
        base = [b + s for b, s in zip(base, sel_bias)]
    return base


def select(key: Vec, k: int) -> List[int]:
    """Chosen experts, slot order = descending key, ties ascending index."""
    E = len(key)
    best = None
    best_sum = None
    for subset in itertools.combinations(range(E), k):  # ascending tuples, lexicographic order
        s = sum((Fraction(key[e]) for e in subset), Fraction(0))
        if best_sum is None or s > best_sum:  # strict: an equal sum keeps the earlier tuple
            best, best_sum = subset, s
    # slot order: repeatedly take the largest remaining key, lowest index on ties
    remaining = list(best)
    ordered = []
    while remaining:
        top = remaining[0]
        for e in remaining[1:]:
            if key[e] > key[top]:
                top = e
        ordered.append(top)
        remaining.remove(top)
    return ordered


def masked_gates(l: Vec, chosen: List[int], score: str, renorm: bool) -> Vec:
    """Gate of every expert (0 for the unselected).

    softmax + renorm: softmax over logits with unselected entries set to -inf (their
    exp is exactly 0). softmax without renorm: plain full softmax, then zeroed off the
    selection. sigmoid: selected scores over their sum.
    """
    E = len(l)
    if score == "softmax":
        if renorm:
            masked = [l[e] if e in chosen else -math.inf for e in range(E)]
        else:
            masked = list(l)
        m = max(masked)
        ex = [math.exp(v - m) if v != -math.inf else 0.0 for v in masked]
        z = math.fsum(ex)
        g = [v / z for v in ex]
        return [g[e] if e in chosen else 0.0 for e in range(E)]
    s = [1.0 / (1.0 + math.exp(-v)) for v in l]
    z = math.fsum(s[e] for e in chosen)
    return [s[e] / z if e in chosen else 0.0 for e in range(E)]


def gelu(z: float) -> float:
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def expert(x: Vec, w_in: Mat, b_in: Optional[Vec], w_out: Mat, b_out: Optional[Vec], act: str) -> Vec:
    if act == "gelu":
        h = _matvec(w_in, x)
        if b_in is not None:
            h = [v + b for v, b in zip(h, b_in)]
        h = [gelu(v) for v in h]
    else:
        F = len(w_in) // 2
        g = _matvec(w_in[:F], x)
        u = _matvec(w_in[F:], x)
        h = [silu(a) * b for a, b in zip(g, u)]
    y = _matvec(w_out, h)
    if b_out is not None:
        y = [v + b for v, b in zip(y, b_out)]
    return y


def layer(x: Mat, w_r: Mat, w_in, b_in, w_out, b_out, k: int, act: str, score: str = "softmax",
          renorm: bool = True, sel_bias: Optional[Vec] = None, ws_in=None, ws_out=None):
    """Returns (idx [T][k], gates [T][k], counts [E], y [T][d]) by the dense masked ensemble."""
    E = len(w_r)
    idx, gts, ys = [], [], []
    counts = [0] * E
    for xt in x:
        l = logits(xt, w_r)
        chosen = select(key_of(l, score, sel_bias), k)
        g_all = masked_gates(l, chosen, score, renorm)
        acc = [0.0] * len(xt)
        for e in range(E):  # every expert runs; unselected ones are multiplied by exactly 0
            out = expert(xt, w_in[e], None if b_in is None else b_in[e], w_out[e],
                         None if b_out is None else b_out[e], act)
            acc = [a + g_all[e] * o for a, o in zip(acc, out)]
        if ws_in is not None:
            sh = expert(xt, ws_in, None, ws_out, None, "swiglu")
            acc = [a + s for a, s in zip(acc, sh)]
        for e in chosen:
            counts[e] += 1
        idx.append(chosen)
        gts.append([g_all[e] for e in chosen])
        ys.append(acc)
    return idx, gts, counts, ys


def permutation(idx: List[List[int]], E: int):
    """(offsets, sorted_token, inv_pos) by counting: for each assignment (t, j), its row is the
    number of assignments to lower experts plus the number of earlier assignments
    (smaller t*k + j) to the same expert."""
    T = len(idx)
    k = len(idx[0]) if T else 0
    flat = [e for row in idx for e in row]
    offsets = [sum(1 for v in flat if v < e) for e in range(E + 1)]
    inv_pos = [0] * len(flat)
    sorted_token = [0] * len(flat)
    for a, e in enumerate(flat):
        row = offsets[e] + sum(1 for b in range(a) if flat[b] == e)
        inv_pos[a] = row
        sorted_token[row] = a // k
    return offsets, sorted_token, inv_pos


def stats(x: Mat, w_r: Mat, idx: List[List[int]], score: str):
    """(f, P, aux, entropy) with explicit sums."""
    E, T = len(w_r), len(x)
    P = [0.0] * E
    ent = 0.0
    for xt in x:
        l = logits(xt, w_r)
        if score == "softmax":
            m = max(l)
            ex = [math.exp(v - m) for v in l]
        else:
            ex = [1.0 / (1.0 + math.exp(-v)) for v in l]
        z = math.fsum(ex)
        p = [v / z for v in ex]
        for e in range(E):
            P[e] += p[e] / T
        ent += -math.fsum(v * math.log(v) for v in p if v > 0) / T
    f = [sum(row.count(e) for row in idx) / T for e in range(E)]
    aux = E * math.fsum(a * b for a, b in zip(f, P))
    return f, P, aux, ent


def permutation_capacity(idx: List[List[int]], E: int, cap: int):
    """(offsets, sorted_token, inv_pos) with at most `cap` rows per expert, by counting: an
    assignment (t, j) to expert e is kept when fewer than `cap` assignments to e precede it in
    t*k + j order; its row is the kept total of lower experts plus that number; a dropped one has
    row -1."""
    T = len(idx)
    k = len(idx[0]) if T else 0
    flat = [e for row in idx for e in row]
    kept = [min(cap, sum(1 for v in flat if v == e)) for e in range(E)]
    offsets = [sum(kept[:e]) for e in range(E + 1)]
    inv_pos = [-1] * len(flat)
    sorted_token = [0] * offsets[E]
    for a, e in enumerate(flat):
        n = sum(1 for b in range(a) if flat[b] == e)
        if n < cap:
            inv_pos[a] = offsets[e] + n
            sorted_token[offsets[e] + n] = a // k
    return offsets, sorted_token, inv_pos


def layer_capacity(x: Mat, w_r: Mat, w_in, b_in, w_out, b_out, k: int, act: str, cap: int,
                   score: str = "softmax", renorm: bool = True, sel_bias: Optional[Vec] = None,
                   ws_in=None, ws_out=None):
    """The dense masked ensemble with expert capacity: the gate of a dropped assignment (one with
    `cap` or more earlier assignments, in token order, to the same expert) is multiplied by 0."""
    E = len(w_r)
    choices = []
    for xt in x:
        l = logits(xt, w_r)
        choices.append((l, select(key_of(l, score, sel_bias), k)))
    seen = [0] * E
    ys = []
    for xt, (l, chosen) in zip(x, choices):
        g_all = masked_gates(l, chosen, score, renorm)
        for e in chosen:  # slot order j = 0..k-1 within the token
            if seen[e] >= cap:
                g_all[e] = 0.0
            seen[e] += 1
        acc = [0.0] * len(xt)
        for e in range(E):
            out = expert(xt, w_in[e], None if b_in is None else b_in[e], w_out[e],
                         None if b_out is None else b_out[e], act)
            acc = [a + g_all[e] * o for a, o in zip(acc, out)]
        if ws_in is not None:
            sh = expert(xt, ws_in, None, ws_out, None, "swiglu")
            acc = [a + v for a, v in zip(acc, sh)]
        ys.append(acc)
    return [c for _, c in choices], ys


def noisy_route(x: Mat, w_r: Mat, w_noise: Mat, noise: Mat, k: int, score: str = "softmax",
                renorm: bool = True, sel_bias: Optional[Vec] = None):
    """Noisy top-k by explicit sums: H_e = l_e + n_e * log(1 + exp(s_e)) with s = x . W_noise,
    then the same exact-subset selection and masked gates as the plain router.
    Returns (H [T][E], idx [T][k], gates [T][k])."""
    Hs, idx, gts = [], [], []
    for t, xt in enumerate(x):
        l = logits(xt, w_r)
        sn = logits(xt, w_noise)
        H = [l[e] + noise[t][e] * math.log1p(math.exp(sn[e])) for e in range(len(l))]
        chosen = select(key_of(H, score, sel_bias), k)
        g_all = masked_gates(H, chosen, score, renorm)
        Hs.append(H)
        idx.append(chosen)
        gts.append([g_all[e] for e in chosen])
    return Hs, idx, gts

