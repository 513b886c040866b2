"""The C ABI without a GPU: the library loads, exports every function that
include/ckl.h declares, and rejects bad arguments on the host before any
device work (every call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import numpy as np
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
    assert lib.ckl_version() >> 16 == 2


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
    (dict(dw_group_rows=-1), B.CKL_ERR_INVALID_ARG),
    (dict(compact_mask=2), B.CKL_ERR_INVALID_ARG),
])
def test_problem_validation(lib, kw, status):
    raw = {k: kw.pop(k) for k in ("compact_mask",) if k in kw}  # make_problem would coerce it to 0/1
    p = _prob(**kw)
    for k, v in raw.items():
        setattr(p, k, v)
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
    # peak memory must grow linearly in T: the workspace beyond the plan-sized
    # part (the G block and W^T of one vocabulary block) grows proportionally to T.
    def ws(T):
        prob = B.make_problem(T, 2880, 201088, 100, 2048)
        q = B.backward_plan(prob)
        g_block = q["n_buffers"] * q["Tc"] * (q["Vc"] + 128) * 2  # G per buffer, bf16 (no G^T)
        assert g_block <= 2048 * 201088 * 2 * 1.01 / 2             # bounded by the chunk budget
        wt_block = 2880 * (q["Vc"] + 128) * 2                      # W^T of one vocabulary block
        return B.workspace_size(prob, 1) - g_block - wt_block
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
    # the default dW group is at most eight chunks, so a smaller chunk holds less
    assert ws(32768, 512) < ws(32768, 2048) < ws(32768, 2048) + 1
    assert B.fused_plan(B.make_problem(32768, 2880, 201088, 100, 512))["dw_group_chunks"] == 8
    assert B.fused_plan(B.make_problem(32768, 2880, 201088, 100, 2048))["dw_group_chunks"] == 8
    assert B.fused_plan(B.make_problem(32768, 2880, 201088, 100, 8192))["dw_group_chunks"] == 2


def test_fused_dw_group_budget(lib):
    # dw_group_rows bounds the logit gradients kept per dW update: one chunk's
    # worth keeps G of one chunk, saving the other seven chunks' rows
    def prob(rows):
        return B.make_problem(32768, 2880, 201088, 100, 2048, dw_group_rows=rows)
    assert B.fused_plan(prob(2048))["dw_group_chunks"] == 1
    assert B.fused_plan(prob(5000))["dw_group_chunks"] == 2       # rounded down to whole chunks
    assert B.fused_plan(prob(1))["dw_group_chunks"] == 1          # at least one chunk
    assert B.fused_plan(prob(1 << 20))["dw_group_chunks"] == 16   # at most every chunk
    saved = B.workspace_size(prob(0), 2) - B.workspace_size(prob(2048), 2)
    # seven chunks fewer of G rows and of H^T columns (both staged per group)
    assert saved == pytest.approx(7 * 2048 * ((201216 + 128) + 2880) * 2, rel=1e-3)
    # at one chunk per group the one-call path holds u and G of one chunk, W^T and
    # the per-row arrays (H^T, the dH split partials, teacher lists)
    chunk_v = 2048 * (201216 + 128) * 2
    w_t = 2880 * (201216 + 128) * 2
    assert B.workspace_size(prob(2048), 2) < 2 * chunk_v + w_t + 0.6e9


def test_packed_rows_workspace(lib):
    # compact_mask adds the packed copy of H (T x d) and a few per-row arrays
    for which in (0, 1, 2):
        plain = B.workspace_size(B.make_problem(32768, 2880, 201088, 100, 2048), which)
        packed = B.workspace_size(B.make_problem(32768, 2880, 201088, 100, 2048, compact_mask=True), which)
        extra = packed - plain
        if which == 1:  # the backward also accumulates dH in fp32 for the scatter (bf16 dH has it anyway)
            assert extra == pytest.approx(32768 * 2880 * 2 + 16 * 32768, rel=0.01)
        else:
            assert extra == pytest.approx(32768 * 2880 * 2 + 16 * 32768, rel=0.01)
    f32 = dict(dh_dtype=B.CKL_F32)
    extra = (B.workspace_size(B.make_problem(32768, 2880, 201088, 100, 2048, compact_mask=True, **f32), 1)
             - B.workspace_size(B.make_problem(32768, 2880, 201088, 100, 2048, **f32), 1))
    assert extra == pytest.approx(32768 * 2880 * (2 + 4) + 16 * 32768, rel=0.01)


def test_scale_cast_rejects_misuse(lib):
    fake = 0x10000
    assert lib.ckl_scale_cast(None, fake, 16, B.CKL_F32, None, None) == B.CKL_ERR_INVALID_ARG
    assert lib.ckl_scale_cast(fake, fake + 0x1000, 6, B.CKL_F32, None, None) == B.CKL_ERR_INVALID_ARG  # n % 4
    assert lib.ckl_scale_cast(fake, fake + 0x1000, 16, 5, None, None) == B.CKL_ERR_INVALID_ARG
    assert lib.ckl_scale_cast(fake + 4, fake + 0x1000, 16, B.CKL_F32, None, None) == B.CKL_ERR_INVALID_ARG
    assert lib.ckl_scale_cast(fake, fake + 0x1000, 16, B.CKL_F32, fake + 2, None) == B.CKL_ERR_INVALID_ARG
    # a bf16 destination may not overlap the fp32 source
    assert lib.ckl_scale_cast(fake, fake + 16, 16, B.CKL_BF16, None, None) == B.CKL_ERR_INVALID_ARG


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


def test_noalloc_forward_refusals(lib):
    # refused on the host before any device work: a workspace beyond the
    # 64 MiB device scratch array, and index validation (it synchronises)
    fake = 0x10000
    too_big = B.make_problem(200000, 2880, 201088, 100, 2048)
    assert B.workspace_size(too_big, 0) > 64 << 20
    st = lib.ckl_forward_noalloc(ctypes.byref(too_big), fake, fake, fake, fake, None, fake, fake, None, None)
    assert st == B.CKL_ERR_UNSUPPORTED
    val = B.make_problem(100, 64, 1000, 8, 64, validate=True)
    st = lib.ckl_forward_noalloc(ctypes.byref(val), fake, fake, fake, fake, None, fake, fake, None, None)
    assert st == B.CKL_ERR_UNSUPPORTED
    # the headline forward fits
    assert B.workspace_size(B.make_problem(32768, 2880, 201088, 100, 2048), 0) <= 64 << 20


def test_plans_stay_inside_their_buffers(lib):
    # host-side plan invariants over drawn problems, both dtypes: the dH split
    # parts of the one-call path tile the padded vocabulary without reaching
    # past it (a part wider than the padding would read unwritten row padding
    # of G and W^T), chunks tile the padded rows, dW groups hold whole chunks,
    # and the backward's G blocks tile the padded rows and vocabulary
    rng = np.random.default_rng(11)
    for _ in range(400):
        bf16 = bool(rng.random() < 0.5)
        tile_v, tile_t = (256, 256) if bf16 else (128, 128)
        T = int(rng.integers(1, 300000))
        V = int(rng.integers(1, 300000))
        d = 8 * int(rng.integers(1, 600))
        K = int(rng.integers(1, min(V, 4096) + 1))
        chunk = int(rng.integers(1, 20000))
        code = B.CKL_BF16 if bf16 else B.CKL_F32
        prob = B.make_problem(T, d, V, K, chunk, code, dw_group_rows=int(rng.choice([0, 1, 5000, 10 ** 6])))
        vp = -(-V // tile_v) * tile_v
        tp = -(-T // tile_t) * tile_t
        f = B.fused_plan(prob)
        assert f["part_cols"] <= vp and f["part_cols"] % 8 == 0
        assert (f["dh_parts"] - 1) * f["part_cols"] < vp <= f["dh_parts"] * f["part_cols"]
        assert f["rows"] % 256 == 0 and (f["chunks"] - 1) * f["rows"] < tp <= f["chunks"] * f["rows"]
        assert 1 <= f["dw_group_chunks"] <= f["chunks"]
        b = B.backward_plan(prob)
        assert b["Tc"] % tile_t == 0 and b["Vc"] % tile_v == 0
        assert (b["nT"] - 1) * b["Tc"] < tp <= b["nT"] * b["Tc"]
        assert (b["nV"] - 1) * b["Vc"] < vp <= b["nV"] * b["Vc"]


def test_binding_refuses_host_tensors():
    # the binding hands only device pointers to the library: host tensors are refused before any call
    import torch

    import chunked_kl_loss_amd as ckl
    H = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(6, 8, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    tl = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        ckl.forward(H, W, idx, tl)
    with pytest.raises(ValueError):
        ckl.forward_backward(H, W, idx, tl)
    with pytest.raises(ValueError):
        ckl.backward(H, W, idx, tl, None, torch.zeros(4))
    with pytest.raises(ValueError):
        ckl.shard_combine(torch.zeros(2, 4), torch.zeros(2, 4), idx, tl, v_total=6, d=8)


def test_loss_function_refuses_mismatched_batch_shapes():
    # leading dimensions of H, idx, tlogit and mask must agree: refused before any call
    import torch

    import chunked_kl_loss_amd as ckl
    H, W = torch.zeros(2, 3, 8), torch.zeros(5, 8)
    with pytest.raises(ValueError):
        ckl.chunked_kl_loss(H, W, torch.zeros(2, 4, 2, dtype=torch.int32), torch.zeros(2, 4, 2))
    with pytest.raises(ValueError):
        ckl.chunked_kl_loss(H, W, torch.zeros(2, 3, 2, dtype=torch.int32), torch.zeros(2, 3, 3))
    with pytest.raises(ValueError):
        ckl.chunked_kl_loss(H, W, torch.zeros(2, 3, 2, dtype=torch.int32), torch.zeros(2, 3, 2),
                            torch.ones(6, dtype=torch.uint8))


def test_aliased_buffers_rejected(lib):
    # an output that overlaps an input, another output or the workspace is refused on the host
    p = _prob()
    need_f, need_b, need_fb = (B.workspace_size(p, w) for w in (0, 1, 2))
    far = 1 << 34  # 16 GiB apart: larger than any buffer of this problem
    H, W, idx, tl, mask, lse, loss, dH, dW, ws = ((1 << 40) + i * far for i in range(10))
    P = ctypes.byref(p)

    def err():
        return lib.ckl_last_error().decode()

    # forward: lse written over W, the workspace over the teacher values, loss inside lse
    assert lib.ckl_forward(P, H, W, idx, tl, mask, loss, W + 256, None, ws, need_f, None) == B.CKL_ERR_INVALID_ARG
    assert "lse overlaps W" in err()
    assert lib.ckl_forward(P, H, W, idx, tl, mask, loss, lse, None, tl - 64, need_f, None) == B.CKL_ERR_INVALID_ARG
    assert "ws overlaps tlogit" in err()
    assert lib.ckl_forward(P, H, W, idx, tl, mask, lse + 16, lse, None, ws, need_f, None) == B.CKL_ERR_INVALID_ARG
    assert "overlap" in err()
    # backward: dH in place of H, dW over the LSE input
    assert lib.ckl_backward(P, H, W, idx, tl, mask, lse, None, H, dW, ws, need_b, None) == B.CKL_ERR_INVALID_ARG
    assert "dH overlaps H" in err()
    assert lib.ckl_backward(P, H, W, idx, tl, mask, lse, None, dH, lse, ws, need_b, None) == B.CKL_ERR_INVALID_ARG
    assert "dW overlaps lse" in err()
    # one call: dH and dW sharing memory, the workspace over the mask
    assert lib.ckl_forward_backward(P, H, W, idx, tl, mask, None, loss, lse, None, dH, dH + 16, ws, need_fb,
                                    None) == B.CKL_ERR_INVALID_ARG
    assert "dH and dW overlap" in err()
    assert lib.ckl_forward_backward(P, H, W, idx, tl, mask, None, loss, lse, None, dH, dW, mask, need_fb,
                                    None) == B.CKL_ERR_INVALID_ARG
    assert "ws overlaps mask" in err()
    # shards: a partial written over the hidden states; the combined LSE over the partials
    shard = _prob(V=1000, v_offset=1000, v_total=2048)
    need_s = B.workspace_size(shard, 0)
    assert lib.ckl_shard_forward(ctypes.byref(shard), H, W, idx, tl, H + 32, lse, ws, need_s,
                                 None) == B.CKL_ERR_INVALID_ARG
    assert "lse_part overlaps H" in err()
    need_c = B.workspace_size(shard, 3)
    assert lib.ckl_shard_combine(ctypes.byref(shard), 2, dH, dW, idx, tl, None, loss, dH + 16, None, ws, need_c,
                                 None) == B.CKL_ERR_INVALID_ARG
    assert "lse overlaps lse_parts" in err()
