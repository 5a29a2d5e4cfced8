"""Checks that pin the float64 oracle to things other than itself.

Each `check_*` takes the oracle module (so a deliberately broken copy can be
passed in by tests/test_oracle_mutations.py) and raises AssertionError when
the oracle disagrees with:
  * the pure-Python brute force (oracle/brute.py) on tiny random layers,
  * closed forms (zero router: uniform probabilities, entropy ln E, the
    lower-index tie rule; GELU at +-1 equals +-Phi(+-1); silu(z) - silu(-z) = z),
  * values the pages print (tests/golden/page_values.txt),
  * library routines (torch.nn.functional in float64 for the E = 1, k = 1 dense FFN),
  * invariants (gate sums, count sums, permutation identity, relabelling and
    token-order equivariance, identical experts, selection-only bias).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import brute

PHI_1 = 0.8413447460685429  # standard normal CDF at 1 (textbook value)


# ------------------------------------------------------------------ random tiny layers


def tiny_case(seed: int, T=None, d=None, F=None, E=None, k=None, act=None, score=None, renorm=None,
              bias=None, shared=None):
    rng = np.random.default_rng(seed)
    T = T if T is not None else int(rng.integers(1, 7))
    d = d if d is not None else int(rng.integers(2, 5))
    F = F if F is not None else int(rng.integers(2, 4))
    E = E if E is not None else int(rng.integers(1, 6))
    k = k if k is not None else int(rng.integers(1, E + 1))
    act = act or ("gelu" if rng.random() < 0.5 else "swiglu")
    score = score or ("softmax" if rng.random() < 0.6 else "sigmoid")
    renorm = True if score == "sigmoid" else (renorm if renorm is not None else bool(rng.random() < 0.7))
    bias = bias if bias is not None else bool(rng.random() < 0.5)
    shared = shared if shared is not None else bool(rng.random() < 0.4)
    n_in = 2 * F if act == "swiglu" else F
    c = dict(
        T=T, d=d, F=F, E=E, k=k, act=act, score=score, renorm=renorm,
        x=rng.standard_normal((T, d)),
        w_r=rng.standard_normal((E, d)),
        sel_bias=rng.standard_normal(E) * 0.3 if bias else None,
        w_in=rng.standard_normal((E, n_in, d)) / math.sqrt(d),
        b_in=rng.standard_normal((E, F)) * 0.5 if act == "gelu" else None,
        w_out=rng.standard_normal((E, d, F)) / math.sqrt(F),
        b_out=rng.standard_normal((E, d)) * 0.5 if act == "gelu" else None,
        ws_in=rng.standard_normal((2 * F, d)) / math.sqrt(d) if shared else None,
        ws_out=rng.standard_normal((d, F)) / math.sqrt(F) if shared else None,
    )
    return c


def _L(a):
    return None if a is None else a.tolist()


def run_ref(ref, c, **kw):
    return ref.layer_forward(c["x"], c["w_r"], ref.stacked_experts(c["w_in"], c["b_in"], c["w_out"], c["b_out"]),
                             c["k"], c["act"], c["score"], c["renorm"], c["sel_bias"], c["ws_in"], c["ws_out"], **kw)


def run_brute(c):
    return brute.layer(_L(c["x"]), _L(c["w_r"]), _L(c["w_in"]), _L(c["b_in"]), _L(c["w_out"]), _L(c["b_out"]),
                       c["k"], c["act"], c["score"], c["renorm"], _L(c["sel_bias"]), _L(c["ws_in"]),
                       _L(c["ws_out"]))


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max err {err:.3g} > {tol}"


# ------------------------------------------------------------------ brute-force pins


def check_against_brute(ref, seeds=range(40)):
    for s in seeds:
        c = tiny_case(s)
        r = run_ref(ref, c)
        b_idx, b_g, b_cnt, b_y = run_brute(c)
        assert r.route.idx.tolist() == b_idx, (s, r.route.idx.tolist(), b_idx)
        _close(r.route.gates, b_g, 1e-12, f"gates seed {s}")
        assert r.route.counts.tolist() == b_cnt, s
        _close(r.y, b_y, 1e-10, f"y seed {s}")
        f, P, aux, ent = brute.stats(_L(c["x"]), _L(c["w_r"]), b_idx, c["score"])
        _close(r.route.f, f, 1e-12, "f")
        _close(r.route.P, P, 1e-12, "P")
        _close(r.route.aux, aux, 1e-12, "aux")
        _close(r.route.entropy, ent, 1e-12, "entropy")
        off, st, inv = brute.permutation(b_idx, c["E"])
        assert r.offsets.tolist() == off and r.sorted_token.tolist() == st and r.inv_pos.tolist() == inv, s


def check_permute_brute(ref, seeds=range(30)):
    for s in seeds:
        rng = np.random.default_rng(1000 + s)
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(0, 12))
        # distinct experts per token, as a selection produces
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int64).reshape(T, k)
        off, st, inv = ref.permute(idx, E)
        b_off, b_st, b_inv = brute.permutation(idx.tolist(), E) if T else ([0] * (E + 1), [], [])
        assert off.tolist() == b_off and st.tolist() == b_st and inv.tolist() == b_inv, s


# ------------------------------------------------------------------ closed forms / page values


def check_zero_router(ref, page_values=None):
    """W_r = 0: every logit is exactly 0, so p = 1/E, entropy = ln E, every token picks 0..k-1."""
    rng = np.random.default_rng(7)
    for E, k in [(4, 2), (8, 2), (60, 4), (128, 8), (256, 8), (5, 5)]:
        x = rng.standard_normal((9, 16))
        r = ref.route(x, np.zeros((E, 16)), k)
        assert (r.idx == np.arange(k)[None, :]).all(), (E, k, r.idx[0])
        _close(r.P, np.full(E, 1.0 / E), 1e-14, "P uniform")
        _close(r.entropy, math.log(E), 1e-13, "entropy ln E")
        _close(r.gates, np.full((9, k), 1.0 / k), 1e-14, "gates 1/k")
        _close(r.aux, float(k), 1e-12, "aux = k")  # f = 1 on experts 0..k-1, P = 1/E
        if E == 128 and page_values:
            assert round(r.entropy, 2) == page_values["max_entropy_nats_E128"]
        if E == 60 and page_values:
            assert round(r.entropy / math.log(2.0), 2) == page_values["max_entropy_bits_E60"]
        # sigmoid: s = 1/2 everywhere, gates 1/k, normalised s uniform
        rs = ref.route(x, np.zeros((E, 16)), k, score="sigmoid")
        assert (rs.idx == np.arange(k)[None, :]).all()
        _close(rs.gates, np.full((9, k), 1.0 / k), 1e-14, "sigmoid gates")
        _close(rs.entropy, math.log(E), 1e-13, "sigmoid entropy")


def check_aux_pages(ref, page_values):
    """Uniform top-1 routing gives L_aux = 1; collapse onto one expert gives L_aux = N."""
    for E in (2, 4, 8, 16):
        x = np.eye(E)  # token t points at expert t
        r = ref.route(x, 3.0 * np.eye(E), 1)
        assert (r.idx[:, 0] == np.arange(E)).all()
        _close(r.aux, page_values["aux_uniform_top1"], 1e-12, "uniform aux")
        # collapse: every token's logit for expert 0 dominates by 60 -> P_0 = 1 - O(e^-60)
        xc = np.ones((5, 3))
        w = np.zeros((E, 3))
        w[0] = 20.0
        rc = ref.route(xc, w, 1)
        assert (rc.idx == 0).all()
        _close(rc.aux, page_values["aux_collapse_equals_num_experts"] * E, 1e-12, "collapsed aux")


def check_probe_arithmetic(ref, page_values):
    """384 selections over 60 experts with top-4: the counts sum to T*k and average 6.4."""
    k, E = int(page_values["probe_topk"]), int(page_values["probe_experts"])
    T = int(page_values["probe_selections"]) // k
    rng = np.random.default_rng(3)
    r = ref.route(rng.standard_normal((T, 24)), rng.standard_normal((E, 24)), k)
    assert r.counts.sum() == page_values["probe_selections"]
    _close(r.counts.mean(), page_values["probe_uniform_per_expert"], 1e-12, "mean per expert")
    _close(r.f.sum(), float(k), 1e-12, "sum f = k")
    _close(r.P.sum(), 1.0, 1e-12, "sum P = 1")


def check_router_example_shape(ref, page_values):
    B, L = int(page_values["router_example_batch"]), int(page_values["router_example_seq"])
    E, k = int(page_values["router_example_experts"]), int(page_values["router_example_topk"])
    rng = np.random.default_rng(4)
    r = ref.route(rng.standard_normal((B * L, 8)), rng.standard_normal((E, 8)), k)
    assert r.idx.shape == (page_values["router_example_rows"], k) and r.gates.shape == r.idx.shape


def check_activations(ref):
    _close(ref.gelu(np.array([1.0, -1.0, 0.0])), [PHI_1, -(1.0 - PHI_1), 0.0], 1e-15, "gelu(+-1)")
    z = np.linspace(-6, 6, 41)
    _close(ref.silu(z) - ref.silu(-z), z, 1e-14, "silu(z) - silu(-z) = z")
    _close(ref.silu(np.array([0.0])), [0.0], 0, "silu(0)")
    # large |z|: gelu -> z (z >> 0) and -> 0 (z << 0)
    _close(ref.gelu(np.array([12.0, -12.0])), [12.0, 0.0], 1e-15, "gelu tails")


# ------------------------------------------------------------------ library routine: dense FFN


def check_dense_ffn(ref):
    """E = 1, k = 1: gate 1 on the only expert, so the layer is one dense FFN (torch, float64)."""
    import torch
    import torch.nn.functional as Fn

    for act in ("gelu", "swiglu"):
        for score in ("softmax", "sigmoid"):
            c = tiny_case(11, T=6, d=5, F=4, E=1, k=1, act=act, score=score, bias=False, shared=False)
            r = run_ref(ref, c)
            x = torch.tensor(c["x"])
            wi, wo = torch.tensor(c["w_in"][0]), torch.tensor(c["w_out"][0])
            if act == "gelu":
                h = Fn.gelu(Fn.linear(x, wi, torch.tensor(c["b_in"][0])))
                y = Fn.linear(h, wo, torch.tensor(c["b_out"][0]))
            else:
                h = Fn.silu(Fn.linear(x, wi[:4])) * Fn.linear(x, wi[4:])
                y = Fn.linear(h, wo)
            _close(r.y, y.numpy(), 1e-13, f"dense ffn {act} {score}")
            _close(r.route.gates, np.ones((6, 1)), 0, "gate 1")


# ------------------------------------------------------------------ invariants


def check_invariants(ref, seeds=range(20)):
    for s in seeds:
        c = tiny_case(500 + s, T=9, E=5, k=int(np.random.default_rng(s).integers(1, 6)))
        r = run_ref(ref, c)
        T, k = c["T"], c["k"]
        assert r.route.counts.sum() == T * k
        _close(r.route.f.sum(), float(k), 1e-12, "sum f")
        _close(r.route.P.sum(), 1.0, 1e-12, "sum P")
        if c["renorm"] or c["score"] == "sigmoid":
            _close(r.route.gates.sum(axis=1), np.ones(T), 1e-13, "sum gates")
        if k == 1 and (c["renorm"] or c["score"] == "sigmoid"):
            _close(r.route.gates, np.ones((T, 1)), 1e-15, "k=1 gate")
        # permutation identity and ordering
        assert r.offsets[0] == 0 and r.offsets[-1] == T * k
        assert (np.diff(r.offsets) == r.route.counts).all()
        for a in range(T * k):
            assert r.sorted_token[r.inv_pos[a]] == a // k
            assert np.array_equal(r.x_perm[r.inv_pos[a]], c["x"][a // k])
        for e in range(c["E"]):
            seg = r.sorted_token[r.offsets[e]:r.offsets[e + 1]]
            assert (np.diff(seg) > 0).all()  # a token picks an expert at most once
            assert (r.route.idx[seg] == e).any(axis=1).all()


def check_identical_experts(ref):
    """All experts equal: the output is the (gate-sum scaled) dense FFN, whatever the routing."""
    for act in ("gelu", "swiglu"):
        for score, renorm in (("softmax", True), ("softmax", False), ("sigmoid", True)):
            c = tiny_case(21, T=7, d=4, F=3, E=5, k=2, act=act, score=score, renorm=renorm, bias=True,
                          shared=False)
            for key in ("w_in", "b_in", "w_out", "b_out"):
                if c[key] is not None:
                    c[key] = np.repeat(c[key][:1], 5, axis=0)
            r = run_ref(ref, c)
            dense = ref.expert_ffn(c["x"], c["w_in"][0], None if c["b_in"] is None else c["b_in"][0],
                                   c["w_out"][0], None if c["b_out"] is None else c["b_out"][0], act)
            gsum = r.route.gates.sum(axis=1, keepdims=True)
            _close(r.y, gsum * dense, 1e-12, f"identical experts {act} {score} {renorm}")


def check_relabel_and_token_order(ref, seeds=range(10)):
    for s in seeds:
        c = tiny_case(700 + s, T=8, E=5, k=2)
        r = run_ref(ref, c)
        rng = np.random.default_rng(s)
        pi = rng.permutation(c["E"])  # new expert q is old expert pi[q]
        c2 = dict(c)
        for key in ("w_r", "sel_bias", "w_in", "b_in", "w_out", "b_out"):
            if c[key] is not None:
                c2[key] = c[key][pi]
        r2 = run_ref(ref, c2)
        _close(r2.y, r.y, 1e-12, "relabel y")
        assert (pi[r2.route.idx] == r.route.idx).all()
        sig = rng.permutation(c["T"])
        c3 = dict(c)
        c3["x"] = c["x"][sig]
        r3 = run_ref(ref, c3)
        _close(r3.y, r.y[sig], 1e-12, "token order")


def check_bias_split(ref):
    """A large selection bias forces an expert into every token's top-k without touching its gate."""
    for score in ("softmax", "sigmoid"):
        c = tiny_case(31, T=8, d=4, F=3, E=6, k=2, score=score, renorm=True, bias=True, shared=False)
        c["sel_bias"] = np.zeros(6)
        c["sel_bias"][4] = 10.0
        r = run_ref(ref, c)
        assert (r.route.idx[:, 0] == 4).all()
        l = c["x"] @ c["w_r"].T
        for t in range(8):
            chosen = [int(e) for e in r.route.idx[t]]
            want = brute.masked_gates(l[t].tolist(), chosen, score, True)
            _close(r.route.gates[t], [want[e] for e in chosen], 1e-13, "bias-free gates")
        # zero bias: same selection as no bias, which for sigmoid is the logit top-k (monotone)
        c["sel_bias"] = np.zeros(6)
        r0 = run_ref(ref, c)
        c["sel_bias"] = None
        r1 = run_ref(ref, c)
        assert (r0.route.idx == r1.route.idx).all()
        assert (r1.route.idx == ref.topk(l, 2)).all()


def check_ambiguity(ref):
    key = np.array([[3.0, 2.0, 2.0 + 5e-5, 0.0], [3.0, 2.0, 1.0, 0.0], [1.0, 1.0, 1.0, 1.0]])
    amb = ref.ambiguous_tokens(key, 2)
    assert amb.tolist() == [True, False, True]
    assert not ref.ambiguous_tokens(key, 4).any()


# ------------------------------------------------------------------ capacity and bias update


def check_capacity_brute(ref, seeds=range(30)):
    """Capacity permutation and layer against counting / the masked dense ensemble."""
    for s in seeds:
        c = tiny_case(2000 + s, T=int(np.random.default_rng(s).integers(2, 9)))
        for cap in (1, 2, 3):
            r = run_ref(ref, c, capacity=cap)
            b_idx, b_y = brute.layer_capacity(_L(c["x"]), _L(c["w_r"]), _L(c["w_in"]), _L(c["b_in"]),
                                              _L(c["w_out"]), _L(c["b_out"]), c["k"], c["act"], cap, c["score"],
                                              c["renorm"], _L(c["sel_bias"]), _L(c["ws_in"]), _L(c["ws_out"]))
            assert r.route.idx.tolist() == b_idx, s
            off, st, inv = brute.permutation_capacity(b_idx, c["E"], cap)
            assert r.offsets.tolist() == off and r.sorted_token.tolist() == st and r.inv_pos.tolist() == inv, (s, cap)
            _close(r.y, b_y, 1e-10, f"capacity y seed {s} cap {cap}")


def check_capacity_limits(ref, seeds=range(10)):
    """A capacity at or above every expert's load changes nothing; kept rows = min(count, C); the
    output lost to capacity is exactly the gate-weighted expert output of the dropped assignments."""
    for s in seeds:
        c = tiny_case(3000 + s, T=8, E=3, k=2)
        full = run_ref(ref, c)
        big = run_ref(ref, c, capacity=int(full.route.counts.max()))
        assert np.array_equal(big.inv_pos, full.inv_pos) and np.array_equal(big.offsets, full.offsets)
        assert np.array_equal(big.y, full.y)
        for cap in (1, 2, 4):
            r = run_ref(ref, c, capacity=cap)
            kept = np.diff(r.offsets)
            assert kept.tolist() == np.minimum(full.route.counts, cap).tolist(), (s, cap)
            assert int((r.inv_pos >= 0).sum()) == int(r.offsets[-1])
            lost = np.zeros_like(full.y)
            flat = full.route.idx.reshape(-1)
            for a in np.nonzero(r.inv_pos < 0)[0]:
                t, j = divmod(int(a), c["k"])
                e = int(flat[a])
                Y = ref.expert_ffn(c["x"][t:t + 1], c["w_in"][e], None if c["b_in"] is None else c["b_in"][e],
                                   c["w_out"][e], None if c["b_out"] is None else c["b_out"][e], c["act"])
                lost[t] += full.route.gates[t, j] * Y[0]
            _close(full.y - r.y, lost, 1e-10, f"dropped contribution seed {s} cap {cap}")


def check_capacity_formula(ref):
    """ceil(c * T * k / E): a factor of 1 gives exactly the uniform load when it divides."""
    assert ref.capacity_rows(4096, 2, 16, 1.0) == 512
    assert ref.capacity_rows(4096, 2, 16, 1.25) == 640
    assert ref.capacity_rows(8192, 2, 8, 1.0) == 2048
    assert ref.capacity_rows(10, 1, 3, 1.0) == 4  # 10/3 rounded up
    assert ref.capacity_rows(64, 8, 128, 1.5) == 6


def check_bias_update(ref):
    """Sign rule of the dynamic-bias router, against the pages' float formulation
    (bias - rate * sign(counts - T*k/E), evaluated here with Python floats rounded to float32)."""
    import struct

    def f32(v):
        return struct.unpack("f", struct.pack("f", v))[0]

    gamma = 0.001
    rng = np.random.default_rng(7)
    for T, k, E in ((6, 2, 4), (10, 1, 3), (4096, 8, 256), (64, 2, 8)):
        counts = rng.multinomial(T * k, np.ones(E) / E)
        if T == 6:
            counts = np.array([5, 3, 1, 3])  # target 3: one over, two at, one under
        bias = (rng.integers(-50, 51, E) * gamma).astype(np.float32)
        got = ref.update_bias(bias, counts, T, k, gamma)
        for e in range(E):
            err = float(counts[e]) - (T * k) / E
            sgn = (err > 0) - (err < 0)
            want = f32(float(bias[e]) - f32(gamma) * sgn)
            assert got[e] == np.float32(want), (T, k, E, e, got[e], want)
        if T == 6:
            assert got[0] < bias[0] and got[1] == bias[1] and got[2] > bias[2] and got[3] == bias[3]
    # repeated steps stay on the gamma grid (up to float32 rounding)
    b = np.zeros(5, dtype=np.float32)
    for it in range(40):  # T*k/E = 4: one expert over, two under, two exactly at the target
        b = ref.update_bias(b, np.array([9, 1, 2, 4, 4]), 10, 2, gamma)
    assert np.allclose(b, np.array([-40, 40, 40, 0, 0]) * gamma, atol=1e-6), b


# ------------------------------------------------------------------ noisy top-k


def check_noisy_brute(ref, seeds=range(25)):
    for s in seeds:
        c = tiny_case(4000 + s)
        rng = np.random.default_rng(4000 + s)
        w_n = rng.standard_normal((c["E"], c["d"]))
        n = rng.standard_normal((c["T"], c["E"]))
        r = ref.route(c["x"], c["w_r"], c["k"], c["score"], c["renorm"], c["sel_bias"], w_n, n)
        H, b_idx, b_g = brute.noisy_route(_L(c["x"]), _L(c["w_r"]), _L(w_n), _L(n), c["k"], c["score"], c["renorm"],
                                          _L(c["sel_bias"]))
        _close(r.logits, H, 1e-12, f"noisy logits seed {s}")
        assert r.idx.tolist() == b_idx, s
        _close(r.gates, b_g, 1e-12, f"noisy gates seed {s}")


def check_noisy_limits(ref):
    """Zero noise reduces to the plain router; softplus closed forms; noise can flip a choice."""
    c = tiny_case(77, T=5, E=4, k=2, score="softmax")
    rng = np.random.default_rng(77)
    w_n = rng.standard_normal((4, c["d"]))
    plain = ref.route(c["x"], c["w_r"], 2, "softmax", c["renorm"], c["sel_bias"])
    quiet = ref.route(c["x"], c["w_r"], 2, "softmax", c["renorm"], c["sel_bias"], w_n, np.zeros((5, 4)))
    assert np.array_equal(plain.logits, quiet.logits) and np.array_equal(plain.idx, quiet.idx)
    assert abs(ref.softplus(np.array([0.0]))[0] - math.log(2.0)) < 1e-15
    z = np.linspace(-30, 30, 61)
    assert np.allclose(ref.softplus(z) - ref.softplus(-z), z, atol=1e-12, rtol=0)
    # one token, two experts with equal logits; a positive draw on expert 1 must select it
    x = np.array([[1.0, 0.0]])
    w = np.array([[1.0, 0.0], [1.0, 0.0]])
    wn = np.array([[0.0, 0.0], [0.0, 0.0]])  # softplus(0) = ln 2 scales both draws
    r = ref.route(x, w, 1, "softmax", True, None, wn, np.array([[0.0, 0.5]]))
    assert r.idx.tolist() == [[1]] and abs(r.logits[0, 1] - (1.0 + 0.5 * math.log(2.0))) < 1e-15


# ------------------------------------------------------------------ sampled-token layer and the error measure


def check_tokens_forward(ref, seeds=range(16)):
    """tokens_forward on a subset of rows (any order, repeats allowed) equals the brute-force layer's
    rows when given the brute force's own selection and gates; with arbitrary gates it equals the
    gate-weighted sum of the selected experts' outputs plus the shared expert, token by token
    ([VI] Eq. (moe-output); [FS] How an MoE layer actually works)."""
    for s in seeds:
        rng = np.random.default_rng(900 + s)
        c = tiny_case(900 + s, T=7, shared=bool(s % 2), renorm=bool(s % 3))
        b_idx, b_g, _, b_y = run_brute(c)
        rows = rng.choice(c["T"], size=5, replace=True)
        get = ref.stacked_experts(c["w_in"], c["b_in"], c["w_out"], c["b_out"])
        idx = np.array(b_idx, dtype=np.int64)
        g = np.array(b_g, dtype=np.float64)
        got = ref.tokens_forward(c["x"][rows], idx[rows], g[rows], get, c["act"], c["ws_in"], c["ws_out"])
        _close(got, np.array(b_y)[rows], 1e-10, f"tokens_forward seed {s}")
        # arbitrary gates (not a softmax of anything), so each slot's own gate must scale its own expert
        g2 = rng.standard_normal(idx.shape)
        got2 = ref.tokens_forward(c["x"][rows], idx[rows], g2[rows], get, c["act"], c["ws_in"], c["ws_out"])
        want2 = []
        for t in rows:
            xt = c["x"][t].tolist()
            acc = [0.0] * c["d"]
            for j, e in enumerate(idx[t]):
                out = brute.expert(xt, _L(c["w_in"][e]), None if c["b_in"] is None else _L(c["b_in"][e]),
                                   _L(c["w_out"][e]), None if c["b_out"] is None else _L(c["b_out"][e]), c["act"])
                acc = [a + g2[t, j] * o for a, o in zip(acc, out)]
            if c["ws_in"] is not None:
                sh = brute.expert(xt, _L(c["ws_in"]), None, _L(c["ws_out"]), None, "swiglu")
                acc = [a + v for a, v in zip(acc, sh)]
            want2.append(acc)
        _close(got2, want2, 1e-10, f"tokens_forward arbitrary gates seed {s}")


def check_rel_l2(ref):
    """Per-row relative L2 with the floor 1e-6 x (rms row norm of the reference), on values worked
    out by hand: reference rows of norms 0, 2, 2, 2*sqrt(2) (rms 2, so the floor is 2e-6)."""
    r = np.array([[0.0, 0.0], [2.0, 0.0], [0.0, 2.0], [2.0, 2.0]])
    a = np.array([[1e-6, 0.0], [2.0, 0.0], [0.0, 3.0], [2.3, 2.4]])
    got = ref.rel_l2_per_row(a, r)
    want = np.array([0.5, 0.0, 0.5, math.sqrt(2.0) / 8.0])  # 1e-6/2e-6, 0, 1/2, 0.5/(2 sqrt 2)
    assert got.shape == (4,), got.shape
    assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)
    # scale-free: both sides times 1000 give the same errors
    assert np.allclose(ref.rel_l2_per_row(1e3 * a, 1e3 * r), want, rtol=1e-12, atol=0)
    # equal inputs give exactly zero, including an all-zero reference
    assert (ref.rel_l2_per_row(r, r) == 0).all()
    assert (ref.rel_l2_per_row(np.zeros((3, 5)), np.zeros((3, 5))) == 0).all()
    # a wide row: one element off by 0.01 over a row of norm 1 is 1e-2
    w = np.zeros((1, 64))
    w[0, 7] = 1.0
    w2 = w.copy()
    w2[0, 40] = 0.01
    assert abs(ref.rel_l2_per_row(w2, w)[0] - 1e-2) < 1e-15


ALL_CHECKS = [
    ("brute", lambda ref, pv: check_against_brute(ref)),
    ("permute_brute", lambda ref, pv: check_permute_brute(ref)),
    ("zero_router", lambda ref, pv: check_zero_router(ref, pv)),
    ("aux_pages", lambda ref, pv: check_aux_pages(ref, pv)),
    ("probe", lambda ref, pv: check_probe_arithmetic(ref, pv)),
    ("router_shape", lambda ref, pv: check_router_example_shape(ref, pv)),
    ("activations", lambda ref, pv: check_activations(ref)),
    ("dense_ffn", lambda ref, pv: check_dense_ffn(ref)),
    ("invariants", lambda ref, pv: check_invariants(ref)),
    ("identical_experts", lambda ref, pv: check_identical_experts(ref)),
    ("relabel_token_order", lambda ref, pv: check_relabel_and_token_order(ref)),
    ("bias_split", lambda ref, pv: check_bias_split(ref)),
    ("ambiguity", lambda ref, pv: check_ambiguity(ref)),
    ("capacity_brute", lambda ref, pv: check_capacity_brute(ref)),
    ("capacity_limits", lambda ref, pv: check_capacity_limits(ref)),
    ("capacity_formula", lambda ref, pv: check_capacity_formula(ref)),
    ("bias_update", lambda ref, pv: check_bias_update(ref)),
    ("noisy_brute", lambda ref, pv: check_noisy_brute(ref)),
    ("noisy_limits", lambda ref, pv: check_noisy_limits(ref)),
    ("tokens_forward", lambda ref, pv: check_tokens_forward(ref)),
    ("rel_l2", lambda ref, pv: check_rel_l2(ref)),
]
