"""The C ABI without a GPU: the library loads, exports every function that
include/ckl.h declares, and rejects bad arguments on the host before any
device work (every call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from chunked_kl_loss_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckl.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from chunked_kl_loss_amd import build
        build.build()
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ckl_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ckl_version() >> 16 == 1


def test_status_strings(lib):
    for s in range(6):
        assert lib.ckl_status_string(s)
    assert lib.ckl_status_string(99) == b"unknown status"


def _prob(**kw):
    base = dict(T=256, d=128, V=2048, K=16, chunk=64, in_dtype=B.CKL_F32)
    base.update(kw)
    return B.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), B.CKL_ERR_INVALID_ARG),
    (dict(d=12), B.CKL_ERR_INVALID_ARG),
    (dict(d=0), B.CKL_ERR_INVALID_ARG),
    (dict(V=0), B.CKL_ERR_INVALID_ARG),
    (dict(K=0), B.CKL_ERR_INVALID_ARG),
    (dict(K=4097, V=10000), B.CKL_ERR_UNSUPPORTED),
    (dict(K=3000, V=2048), B.CKL_ERR_INVALID_ARG),
    (dict(chunk=0), B.CKL_ERR_INVALID_ARG),
    (dict(in_dtype=7), B.CKL_ERR_INVALID_ARG),
    (dict(d=131072), B.CKL_ERR_UNSUPPORTED),
    (dict(T=4000001), B.CKL_ERR_UNSUPPORTED),
    (dict(teacher_form=2), B.CKL_ERR_INVALID_ARG),
    (dict(v_offset=-1), B.CKL_ERR_INVALID_ARG),
    (dict(v_offset=10, v_total=2050), B.CKL_ERR_INVALID_ARG),   # shard past the vocabulary end
    (dict(v_total=1 << 31), B.CKL_ERR_UNSUPPORTED),
    (dict(K=3000, V=2048, v_total=2048), B.CKL_ERR_INVALID_ARG),
    (dict(teacher_form=-1), B.CKL_ERR_INVALID_ARG),
    (dict(V=4000001), B.CKL_ERR_UNSUPPORTED),
])
def test_problem_validation(lib, kw, status):
    p = _prob(**kw)
    out = ctypes.c_size_t()
    assert lib.ckl_workspace_size(ctypes.byref(p), 0, ctypes.byref(out)) == status
    assert lib.ckl_last_error()


def test_workspace_query_and_plan(lib):
    p = _prob()
    for which in range(4):
        assert B.workspace_size(p, which) > 0
    with pytest.raises(B.CklError):
        B.workspace_size(p, 4)
    plan = B.backward_plan(p)
    assert plan["Tc"] % 128 == 0 and plan["Vc"] % 128 == 0  # fp32 tiles are 128 x 128
    assert plan["nT"] * plan["Tc"] >= 256 and plan["nV"] * plan["Vc"] >= 2048


def test_null_and_alignment_rejected(lib):
    p = _prob()
    fake = 0x10000  # never dereferenced: every call below fails validation
    st = lib.ckl_forward(None, fake, fake, fake, fake, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    st = lib.ckl_forward(ctypes.byref(p), None, fake, fake, fake, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    st = lib.ckl_forward(ctypes.byref(p), fake + 2, fake, fake, fake, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    st = lib.ckl_backward(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, None, fake, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    # fused call: dW missing, then a misaligned lse
    st = lib.ckl_forward_backward(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake, None, fake, None,
                                  fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    st = lib.ckl_forward_backward(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake + 2, None, fake,
                                  fake, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG


def test_workspace_too_small_rejected(lib):
    p = _prob()
    fake = 0x10000
    need = B.workspace_size(p, 0)
    st = lib.ckl_forward(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None, fake, need - 1, None)
    assert st == B.CKL_ERR_WORKSPACE
    st = lib.ckl_forward(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None, None, need, None)
    assert st == B.CKL_ERR_WORKSPACE
    needb = B.workspace_size(p, 1)
    st = lib.ckl_backward(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, fake, fake, fake, needb - 1,
                          None)
    assert st == B.CKL_ERR_WORKSPACE
    needf = B.workspace_size(p, 2)
    st = lib.ckl_forward_backward(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake, None, fake, fake,
                                  fake, needf - 1, None)
    assert st == B.CKL_ERR_WORKSPACE


def test_workspace_linear_in_rows(lib):
    # peak memory must grow linearly in T: the workspace beyond the T-independent
    # part (W^T and the G block) grows proportionally to T.
    def ws(T):
        prob = B.make_problem(T, 2880, 201088, 100, 2048)
        q = B.backward_plan(prob)
        g_block = q["n_buffers"] * q["Tc"] * (q["Vc"] + 128) * 2  # G per buffer, bf16 (no G^T)
        assert g_block <= 2048 * 201088 * 2 * 1.01 / 2             # bounded by the chunk budget
        return B.workspace_size(prob, 1) - g_block
    a, b, c = ws(32768), ws(65536), ws(131072)
    assert c - b == pytest.approx(2 * (b - a), rel=1e-4)
    # and never approaches a T x V tensor
    assert B.workspace_size(B.make_problem(131072, 2880, 201088, 100, 2048), 1) < 131072 * 201088 * 2 / 4


def test_plan_respects_budget(lib):
    for T, V, chunk in [(32768, 201088, 2048), (262144, 201088, 512), (4096, 32000, 1024), (1000, 1000, 1)]:
        q = B.backward_plan(B.make_problem(T, 2880, V, 100, chunk))
        tile = 256  # bf16 logit tile: 256 vocabulary x 256 token rows
        assert q["Tc"] % tile == 0 and q["Vc"] % tile == 0
        assert q["n_buffers"] * q["Tc"] * q["Vc"] <= max(chunk * V // 2, tile * tile) or q["Tc"] == tile
        assert q["nT"] * q["Tc"] >= T and q["nV"] * q["Vc"] >= V


def test_fused_plan_and_workspace(lib):
    # chunks: `chunk` rounded up to 256 rows, covering every row; the dH
    # split-k parts cover the padded vocabulary in 256-multiples
    for T, V, chunk in [(32768, 201088, 2048), (262144, 201088, 512), (4096, 32000, 1024), (257, 2048, 64),
                        (1000, 1000, 100000)]:
        prob = B.make_problem(T, 2880, V, 100, chunk)
        f = B.fused_plan(prob)
        assert f["rows"] % 256 == 0 and f["rows"] >= min(chunk, T)
        assert f["rows"] <= max(256, -(-chunk // 256) * 256)
        assert f["chunks"] * f["rows"] >= T and (f["chunks"] - 1) * f["rows"] < T
        Vp = -(-V // 256) * 256
        assert f["part_cols"] % 256 == 0 and f["dh_parts"] * f["part_cols"] >= Vp
        assert (f["dh_parts"] - 1) * f["part_cols"] < Vp
    # beyond the part linear in T, u of one chunk (rows x V, bf16) and the
    # per-chunk partials grow with chunk; G of the dW group is bounded by
    # 16384 rows whatever the chunk
    def ws(T, chunk):
        return B.workspace_size(B.make_problem(T, 2880, 201088, 100, chunk), 2)
    a, b, c = ws(32768, 2048), ws(65536, 2048), ws(131072, 2048)
    assert c - b == pytest.approx(2 * (b - a), rel=1e-3)
    u_row = 201216 * 2
    g2k, g4k, g8k = ws(32768, 2048), ws(32768, 4096), ws(32768, 8192)
    assert 1.0 * 2048 * u_row <= g4k - g2k <= 1.4 * 2048 * u_row
    assert 1.0 * 4096 * u_row <= g8k - g4k <= 1.4 * 4096 * u_row
    # short sequences keep G of only the chunks they have
    one, two = ws(2048, 2048), ws(4096, 2048)
    assert two - one == pytest.approx(2048 * (201216 + 128) * 2, rel=0.05)


def test_shard_entry_points_reject_misuse(lib):
    fake = 0x10000
    shard = _prob(V=1000, v_offset=1000, v_total=2048)
    # the whole-vocabulary entry points refuse a shard
    st = lib.ckl_forward(ctypes.byref(shard), fake, fake, fake, fake, None, fake, fake, None, fake, 1 << 30, None)
    assert st == B.CKL_ERR_UNSUPPORTED
    st = lib.ckl_forward_backward(ctypes.byref(shard), fake, fake, fake, fake, None, None, fake, fake, None, fake,
                                  fake, fake, 1 << 30, None)
    assert st == B.CKL_ERR_UNSUPPORTED
    # K may exceed the shard's rows as long as it fits the whole vocabulary
    assert B.workspace_size(_prob(V=8, K=16, v_total=2048), 0) > 0
    # shard forward: missing output, short workspace
    st = lib.ckl_shard_forward(ctypes.byref(shard), fake, fake, fake, fake, None, fake, fake, 1 << 30, None)
    assert st == B.CKL_ERR_INVALID_ARG
    need = B.workspace_size(shard, 0)
    st = lib.ckl_shard_forward(ctypes.byref(shard), fake, fake, fake, fake, fake, fake, fake, need - 1, None)
    assert st == B.CKL_ERR_WORKSPACE
    # combine: no shards
    st = lib.ckl_shard_combine(ctypes.byref(shard), 0, fake, fake, fake, fake, None, fake, fake, None, fake, 1 << 30,
                               None)
    assert st == B.CKL_ERR_INVALID_ARG
