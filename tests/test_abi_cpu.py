"""The C-ABI library on the CPU: it loads, exports every symbol include/moe.h declares, and rejects
invalid calls on the host before any HIP call (so nothing here touches a GPU; every call below
is one the library must refuse, or a T = 0 no-op)."""
import ctypes
import os
import re

import pytest

from sparse_routing_expert_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned address; never dereferenced because every call is rejected first
MISALIGNED = FAKE + 4


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoe.so is not built (run `python -m sparse_routing_expert_amd.build`)")
    return L.lib()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert declared == sorted(L.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_exports_probes(lib):
    src = open(os.path.join(ROOT, "include", "moe_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert declared == sorted(L.PROBES)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.moe_probe_copy(None, FAKE, 16, 1, None) == -1
    assert lib.moe_probe_copy(FAKE, FAKE, 17, 1, None) == -1
    assert lib.moe_probe_mfma(0, 1, FAKE, None) == -1
    assert lib.moe_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 8 * 32 * 32 * 16 * 2


def test_status_strings(lib):
    assert L.status_name(0) == "MOE_OK"
    assert L.status_name(-3) == "MOE_ERR_WORKSPACE"
    assert L.status_name(123) == "MOE_ERR_UNKNOWN"


def good_shape(**kw):
    args = dict(T=128, d_model=256, d_ff=128, E=8, k=2, dtype="bf16", act="swiglu", score="softmax", renorm=True)
    args.update(kw)
    return L.make_shape(**args)


def ws_bytes(shape, stage):
    out = ctypes.c_size_t(0)
    rc = L.lib().moe_workspace_bytes(ctypes.byref(shape), stage, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("kw,want", [
    (dict(T=-1), L.MOE_ERR_INVALID_ARG),
    (dict(E=0), L.MOE_ERR_INVALID_ARG),
    (dict(E=1025), L.MOE_ERR_INVALID_ARG),
    (dict(k=0), L.MOE_ERR_INVALID_ARG),
    (dict(k=9), L.MOE_ERR_INVALID_ARG),  # k > E
    (dict(E=64, k=33), L.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), L.MOE_ERR_INVALID_ARG),
    # bf16 rows are 16-byte vectors of 8 elements, fp32 ones of 4
    (dict(d_model=72), L.MOE_OK),
    (dict(d_ff=200), L.MOE_OK),
    (dict(d_model=72, d_ff=200, d_ff_shared=40), L.MOE_OK),
    (dict(d_model=100), L.MOE_ERR_INVALID_ARG),
    (dict(d_ff=100), L.MOE_ERR_INVALID_ARG),
    (dict(d_ff_shared=12), L.MOE_ERR_INVALID_ARG),
    (dict(dtype="f32", d_model=6), L.MOE_ERR_INVALID_ARG),
    (dict(dtype="f32", d_model=12, d_ff=20), L.MOE_OK),
    (dict(score="sigmoid", renorm=False), L.MOE_ERR_UNSUPPORTED),
    (dict(T=2**31, k=2), L.MOE_ERR_INVALID_ARG),  # T*k overflows int32
    # widths up to MOE_MAX_WIDTH = 2^18 (32-bit DMA offsets in the matrix kernels)
    (dict(T=16, d_ff=2**18), L.MOE_OK),
    (dict(T=16, d_ff=2**18 + 8), L.MOE_ERR_UNSUPPORTED),
    (dict(T=16, d_model=2**18 + 8), L.MOE_ERR_UNSUPPORTED),
    (dict(T=16, d_ff_shared=2**18 + 8), L.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(lib, kw, want):
    rc, _ = ws_bytes(good_shape(**kw), L.MOE_STAGE_FORWARD)
    assert rc == want


def test_bad_enums_and_stage(lib):
    s = good_shape()
    s.dtype = 7
    assert ws_bytes(s, 0)[0] == L.MOE_ERR_INVALID_ARG
    s = good_shape()
    s.act = 5
    assert ws_bytes(s, 0)[0] == L.MOE_ERR_INVALID_ARG
    s = good_shape()
    s.score = 2
    assert ws_bytes(s, 0)[0] == L.MOE_ERR_INVALID_ARG
    s = good_shape()
    s.renorm = 3
    assert ws_bytes(s, 0)[0] == L.MOE_ERR_INVALID_ARG
    assert ws_bytes(good_shape(), 9)[0] == L.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_bytes(None, 0, None) == L.MOE_ERR_INVALID_ARG


def test_workspace_sizes_monotone(lib):
    small = [ws_bytes(good_shape(T=64), st)[1] for st in range(6)]
    big = [ws_bytes(good_shape(T=4096), st)[1] for st in range(6)]
    assert all(b >= a for a, b in zip(small, big))
    assert big[L.MOE_STAGE_FFN] >= 4096 * 2 * 128 * 2  # h = [T*k, d_ff] bf16
    rc, n = ws_bytes(good_shape(d_ff_shared=0), L.MOE_STAGE_SHARED)
    assert rc == 0 and n == 0
    # bf16 grouped GEMMs keep one fp32 256 x 256 partial tile per block (at least 8 blocks)
    rc, n = ws_bytes(good_shape(), L.MOE_STAGE_EXPERT)
    assert rc == 0 and n >= 8 * 256 * 256 * 4
    assert ws_bytes(good_shape(), L.MOE_STAGE_FFN)[1] >= n
    rc, n = ws_bytes(good_shape(dtype="f32"), L.MOE_STAGE_EXPERT)
    assert rc == 0 and n == 0


def test_capacity_and_bias_rejections(lib):
    s = good_shape(capacity=-1)
    assert ws_bytes(s, L.MOE_STAGE_PERMUTE)[0] == L.MOE_ERR_INVALID_ARG
    ok = good_shape(capacity=64)
    assert ws_bytes(ok, L.MOE_STAGE_PERMUTE)[0] == L.MOE_OK
    ub = lib.moe_update_bias
    assert ub(ctypes.byref(ok), None, 1e-3, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(ok), FAKE, 1e-3, None, None) == L.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(ok), FAKE, 1e-3, MISALIGNED, None) == L.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(ok), FAKE, float("nan"), FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(ok), FAKE, float("inf"), FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(good_shape(capacity=-5)), FAKE, 1e-3, FAKE, None) == L.MOE_ERR_INVALID_ARG


def test_route_noisy_rejections(lib):
    s = good_shape()
    rc, n = ws_bytes(s, L.MOE_STAGE_ROUTE_NOISY)
    assert rc == 0 and n > ws_bytes(s, L.MOE_STAGE_ROUTE)[1]
    f = lib.moe_route_noisy
    good = [ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, n, None]
    for i in (1, 2, 3, 4, 7, 8, 9):  # required pointers
        bad = list(good)
        bad[i] = None
        assert f(*bad) == L.MOE_ERR_INVALID_ARG, i
    bad = list(good)
    bad[4] = MISALIGNED
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[12] = n - 1
    assert f(*bad) == L.MOE_ERR_WORKSPACE
    z = list(good)
    z[0] = ctypes.byref(good_shape(T=0))
    assert f(*z) == L.MOE_OK


def test_route_rejections(lib):
    s = good_shape()
    r = lib.moe_route
    n = ws_bytes(s, L.MOE_STAGE_ROUTE)[1]
    args = [ctypes.byref(s), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, n, None]
    for i in (1, 2, 5, 6, 7):  # required pointers
        bad = list(args)
        bad[i] = None
        assert r(*bad) == L.MOE_ERR_INVALID_ARG
        bad[i] = MISALIGNED
        assert r(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[10] = n - 1
    assert r(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[3] = MISALIGNED  # optional pointer, misaligned
    assert r(*bad) == L.MOE_ERR_INVALID_ARG
    # T = 0 is a successful no-op (no launch)
    s0 = good_shape(T=0)
    assert r(ctypes.byref(s0), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, n, None) == L.MOE_OK


def test_permute_combine_rejections(lib):
    s = good_shape()
    n = ws_bytes(s, L.MOE_STAGE_PERMUTE)[1]
    p = lib.moe_permute
    good = [ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n, None]
    for i in range(1, 6):
        bad = list(good)
        bad[i] = None
        assert p(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[6] = MISALIGNED  # x_perm may be NULL (positions only) but not misaligned
    assert p(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[8] = 0
    assert p(*bad) == L.MOE_ERR_WORKSPACE
    c = lib.moe_combine
    assert c(ctypes.byref(s), None, FAKE, FAKE, None, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert c(ctypes.byref(s), FAKE, FAKE, FAKE, MISALIGNED, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert c(ctypes.byref(good_shape(T=0)), FAKE, FAKE, FAKE, None, FAKE, None) == L.MOE_OK


def test_permute_noalloc_rejections(lib):
    """The no-allocation permute checks everything on the host before any HIP call: pointers, the
    shape, and that the permute's scratch fits the library's fixed array."""
    s = good_shape()
    p = lib.moe_permute_noalloc
    good = [ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    for i in range(1, 7):
        bad = list(good)
        if i < 6:  # x_perm (6) may be NULL: positions only
            bad[i] = None
            assert p(*bad) == L.MOE_ERR_INVALID_ARG
        bad[i] = MISALIGNED
        assert p(*bad) == L.MOE_ERR_INVALID_ARG
    assert p(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert p(ctypes.byref(good_shape(k=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op that touches nothing (so it succeeds here, without a GPU)
    assert p(ctypes.byref(good_shape(T=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_OK
    # the largest permute workspace the fixed array holds, and one tile more
    E, k = 1024, 1
    per_tile = 2 * E * 4
    ntiles = L.MOE_NOALLOC_SCRATCH_BYTES // per_tile
    fits = good_shape(T=ntiles * 1024, E=E, k=k)
    assert ws_bytes(fits, L.MOE_STAGE_PERMUTE)[1] <= L.MOE_NOALLOC_SCRATCH_BYTES
    over = good_shape(T=ntiles * 1024 + 1, E=E, k=k)
    assert ws_bytes(over, L.MOE_STAGE_PERMUTE)[1] > L.MOE_NOALLOC_SCRATCH_BYTES
    assert p(ctypes.byref(over), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_WORKSPACE


def test_ffn_rejections(lib):
    s = good_shape()
    n = ws_bytes(s, L.MOE_STAGE_FFN)[1]
    f = lib.moe_grouped_ffn
    good = [ctypes.byref(s), 0, 8, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, n, None]
    for eb, ee in ((-1, 8), (3, 2), (0, 9)):
        bad = list(good)
        bad[1], bad[2] = eb, ee
        assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[6] = FAKE  # bias given to a SwiGLU layer
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[11] = n - 256
    assert f(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(good)
    bad[1], bad[2] = 4, 4  # empty expert range: no-op
    assert f(*bad) == L.MOE_OK
    # the two one-projection entry points: range, bias and workspace checks come before any launch
    ne = ws_bytes(s, L.MOE_STAGE_EXPERT)[1]
    for fn in (lib.moe_expert_up, lib.moe_expert_down):
        good = [ctypes.byref(s), 0, 8, FAKE, FAKE, FAKE, None, FAKE, FAKE, ne, None]
        bad = list(good)
        bad[1], bad[2] = 0, 9
        assert fn(*bad) == L.MOE_ERR_INVALID_ARG
        bad = list(good)
        bad[6] = FAKE  # bias given to a SwiGLU layer
        assert fn(*bad) == L.MOE_ERR_INVALID_ARG
        bad = list(good)
        bad[9] = ne - 256
        assert fn(*bad) == L.MOE_ERR_WORKSPACE
        bad = list(good)
        bad[8], bad[9] = None, 0
        assert fn(*bad) == L.MOE_ERR_WORKSPACE
        bad = list(good)
        bad[1], bad[2] = 4, 4  # empty expert range: no-op
        assert fn(*bad) == L.MOE_OK
    sh = lib.moe_shared_ffn
    assert sh(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == L.MOE_ERR_INVALID_ARG  # no shared


def test_forward_rejections(lib):
    s = good_shape(d_ff_shared=128)
    n = ws_bytes(s, L.MOE_STAGE_FORWARD)[1]
    fw = lib.moe_forward
    good = [ctypes.byref(s), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, None, None, None, None,
            FAKE, n, None]
    bad = list(good)
    bad[8] = None  # shared weights missing
    assert fw(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[16] = n - 1
    assert fw(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(good)
    bad[15] = None
    assert fw(*bad) == L.MOE_ERR_WORKSPACE
    s2 = good_shape()
    n2 = ws_bytes(s2, L.MOE_STAGE_FORWARD)[1]
    assert fw(ctypes.byref(s2), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, None, None, None,
              None, FAKE, n2, None) == L.MOE_ERR_INVALID_ARG  # shared weights without a shared expert


def test_backward_rejections(lib):
    s = good_shape()
    rc, n = ws_bytes(s, L.MOE_STAGE_BACKWARD)
    # at least dY, the recomputed pre-activation [T*k, 2F], h, dh (fp32) and dX (fp32)
    A = 128 * 2
    assert rc == 0 and n >= A * (256 * 2 + 256 * 2 + 128 * 2 + 128 * 4 + 256 * 4)
    f = lib.moe_backward
    # shape, x, w_r, w_in, b_in, w_out, b_out, ws_in, ws_out, logits, idx, topk_w, counts, offsets, inv_pos,
    # x_perm, y_perm, dy, aux_coef, dx, dw_r, dw_in, db_in, dw_out, db_out, dws_in, dws_out, dlogits, ws, bytes, st
    good = [ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, FAKE, FAKE, None, FAKE, FAKE,
            FAKE, FAKE, FAKE, 0.0, FAKE, FAKE, FAKE, None, FAKE, None, None, None, None, FAKE, n, None]
    # bf16 widths that are not multiples of 64: the forward takes them, the backward does not
    rag = good_shape(d_model=72)
    bad = list(good)
    bad[0] = ctypes.byref(rag)
    bad[-2] = ws_bytes(rag, L.MOE_STAGE_BACKWARD)[1]
    assert f(*bad) == L.MOE_ERR_UNSUPPORTED
    for i in (1, 2, 3, 5, 9, 10, 11, 13, 14, 15, 16, 17, 19, 20, 21, 23):  # required pointers
        bad = list(good)
        bad[i] = None
        assert f(*bad) == L.MOE_ERR_INVALID_ARG, i
    for i in (1, 17, 27):
        bad = list(good)
        bad[i] = MISALIGNED
        assert f(*bad) == L.MOE_ERR_INVALID_ARG, i
    bad = list(good)
    bad[18] = 0.01  # balancing term without counts
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad[18] = float("nan")
    bad[12] = FAKE
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[4] = FAKE  # SwiGLU has no biases
    bad[22] = FAKE
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[22] = FAKE  # a bias gradient without the bias
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[25] = FAKE  # shared gradients without a shared expert
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(good)
    bad[29] = n - 1
    assert f(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(good)
    bad[28] = None
    assert f(*bad) == L.MOE_ERR_WORKSPACE
    # GELU layer: biases and their gradients go together
    g = good_shape(act="gelu")
    ng = ws_bytes(g, L.MOE_STAGE_BACKWARD)[1]
    gg = list(good)
    gg[0], gg[29] = ctypes.byref(g), ng
    gg[4] = FAKE  # b_in without db_in
    assert f(*gg) == L.MOE_ERR_INVALID_ARG
    # shared expert: its weights and gradients are required
    sh = good_shape(d_ff_shared=128)
    nsh = ws_bytes(sh, L.MOE_STAGE_BACKWARD)[1]
    assert nsh > n
    gs = list(good)
    gs[0], gs[29] = ctypes.byref(sh), nsh
    gs[7], gs[8], gs[25] = FAKE, FAKE, FAKE  # dws_out missing
    assert f(*gs) == L.MOE_ERR_INVALID_ARG
    z = list(good)
    z[0] = ctypes.byref(good_shape(T=0))
    z[29] = ws_bytes(good_shape(T=0), L.MOE_STAGE_BACKWARD)[1]
    assert f(*z) == L.MOE_OK


def test_binding_raises_on_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(L.MoeLibraryMissing):
        L.lib()
