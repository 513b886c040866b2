"""GPU test of ckl_forward_noalloc, the forward entry point that takes its
workspace from the library's device scratch array instead of a caller's
buffer.  Called through the C ABI and compared with ckl_forward (a caller's
workspace) on the same inputs: the same kernels in the same order, so the
results agree bit for bit; two calls in a row, the second smaller, so the
scratch array's leftovers from the first call must not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

from chunked_kl_loss_amd import _binding as B
from synth import make_inputs
from tests.gpu_harness import say, to_device

pytestmark = pytest.mark.gpu


def _both(x, chunk, packed=False):
    lib = B.load_library()
    H, W, idx, tl, m = to_device(x)
    T, d, V, K = x.T, x.d, x.V, x.K
    code = B.CKL_BF16 if x.dtype == "bf16" else B.CKL_F32
    prob = B.make_problem(T, d, V, K, chunk, code, compact_mask=packed and m is not None)
    st = torch.cuda.current_stream().cuda_stream
    mp = None if m is None else m.data_ptr()
    out = []
    for use_scratch in (True, False):
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
        rl = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
        if use_scratch:
            status = lib.ckl_forward_noalloc(ctypes.byref(prob), H.data_ptr(), W.data_ptr(), idx.data_ptr(),
                                             tl.data_ptr(), mp, loss.data_ptr(), lse.data_ptr(), rl.data_ptr(), st)
        else:
            ws = torch.full((B.workspace_size(prob, 0),), 0xFF, dtype=torch.uint8, device="cuda")
            status = lib.ckl_forward(ctypes.byref(prob), H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(),
                                     mp, loss.data_ptr(), lse.data_ptr(), rl.data_ptr(), ws.data_ptr(), ws.numel(),
                                     st)
        B.check(status, lib)
        torch.cuda.synchronize()
        out.append((loss.cpu().numpy(), lse.cpu().numpy(), rl.cpu().numpy()))
    return out


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_forward_matches_workspace_forward(packed):
    big = make_inputs(4, seed=3, T=1800)    # 201,088-token vocabulary, packed-document mask
    small = make_inputs(4, seed=4, T=700)
    for x, chunk in ((big, 512), (small, 256)):   # the second call is smaller
        say(f"case no-alloc forward T={x.T} chunk={chunk} packed={packed}")
        (l0, s0, r0), (l1, s1, r1) = _both(x, chunk, packed)
        assert np.isfinite(l0).all() and np.isfinite(s0).all() and np.isfinite(r0).all()
        assert np.array_equal(l0, l1) and np.array_equal(s0, s1) and np.array_equal(r0, r1)


@pytest.mark.parametrize("seed", range(6))
def test_noalloc_forward_drawn(seed):
    # drawn problems (dtype, shapes, chunk, mask with or without packing)
    import dataclasses

    from tests.test_parity_gpu import _custom
    from tests.test_random_shapes_gpu import draw
    c = draw(seed + 300)
    x = dataclasses.replace(_custom(c["T"], c["d"], c["V"], c["K"], c["dtype"], seed=seed), mask=c["mask"])
    say(f"case no-alloc forward drawn seed={seed} T={x.T} d={x.d} V={x.V} K={x.K} chunk={c['chunk']} "
        f"{x.dtype} masked={x.mask is not None} packed={c['compact']}")
    (l0, s0, r0), (l1, s1, r1) = _both(x, c["chunk"], c["compact"])
    assert np.isfinite(l0).all() and np.isfinite(s0).all() and np.isfinite(r0).all()
    assert np.array_equal(l0, l1) and np.array_equal(s0, s1) and np.array_equal(r0, r1)


def test_noalloc_forward_unmasked_fp32():
    x = make_inputs(0, seed=1)
    say("case no-alloc forward fp32 tiny")
    (l0, s0, r0), (l1, s1, r1) = _both(x, 64)
    assert np.array_equal(l0, l1) and np.array_equal(s0, s1) and np.array_equal(r0, r1)


def test_noalloc_forward_limits():
    lib = B.load_library()
    fake = 0x10000  # never dereferenced: each call below is refused before any launch
    too_big = B.make_problem(200000, 2880, 201088, 100, 2048)   # ~250 MB of forward workspace
    assert B.workspace_size(too_big, 0) > 64 << 20
    st = lib.ckl_forward_noalloc(ctypes.byref(too_big), fake, fake, fake, fake, None, fake, fake, None, None)
    assert st == B.CKL_ERR_UNSUPPORTED
    assert b"64" in lib.ckl_last_error() or b"scratch" in lib.ckl_last_error()
    val = B.make_problem(100, 64, 1000, 8, 64, validate=True)
    st = lib.ckl_forward_noalloc(ctypes.byref(val), fake, fake, fake, fake, None, fake, fake, None, None)
    assert st == B.CKL_ERR_UNSUPPORTED


def test_noalloc_forward_under_graph_capture():
    # the callers this entry point is for: a forward captured into a HIP graph
    # (torch.cuda.graph) and replayed with new inputs copied into the captured
    # buffers, eager work and synchronisation between replays; every replay
    # equals an eager ckl_forward on the same inputs, bit for bit
    import dataclasses

    from tests.test_parity_gpu import _custom
    lib = B.load_library()
    xs = []
    for s in (7, 8, 9):   # packed documents of 64..511 rows, the first quarter of each masked
        rng = np.random.default_rng(s)
        mask = np.ones(3000, np.uint8)
        t = 0
        while t < 3000:
            n = int(rng.integers(64, 512))
            mask[t:t + n // 4] = 0
            t += n
        xs.append(dataclasses.replace(_custom(3000, 256, 30000, 100, "bf16", seed=s), mask=mask))
    x0 = xs[0]
    T, d, V, K = x0.T, x0.d, x0.V, x0.K
    prob = B.make_problem(T, d, V, K, 256, B.CKL_BF16, compact_mask=True)
    H, W, idx, tl, m = to_device(x0)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    lse = torch.zeros(T, dtype=torch.float32, device="cuda")
    rl = torch.zeros(T, dtype=torch.float32, device="cuda")

    def call(use_scratch, ws=None):
        st = torch.cuda.current_stream().cuda_stream
        if use_scratch:
            s = lib.ckl_forward_noalloc(ctypes.byref(prob), H.data_ptr(), W.data_ptr(), idx.data_ptr(),
                                        tl.data_ptr(), m.data_ptr(), loss.data_ptr(), lse.data_ptr(), rl.data_ptr(), st)
        else:
            s = lib.ckl_forward(ctypes.byref(prob), H.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(),
                                m.data_ptr(), loss.data_ptr(), lse.data_ptr(), rl.data_ptr(), ws.data_ptr(),
                                ws.numel(), st)
        B.check(s, lib)

    def load(x):
        h, w, i, t, mm = to_device(x)
        for dst, src in ((H, h), (W, w), (idx, i), (tl, t), (m, mm)):
            dst.copy_(src)

    ws = torch.full((B.workspace_size(prob, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    refs = []
    for x in xs:   # eager references (caller's workspace)
        load(x)
        call(False, ws)
        torch.cuda.synchronize()
        refs.append((loss.cpu().numpy().copy(), lse.cpu().numpy().copy(), rl.cpu().numpy().copy()))
    say("case no-alloc forward captured in a graph")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # the scratch address is looked up on the first call, before capture
        call(True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(True)
    for rep in range(2):
        for x, (l0, s0, r0) in zip(xs, refs):
            load(x)                      # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(loss.cpu().numpy(), l0), rep
            assert np.array_equal(lse.cpu().numpy(), s0), rep
            assert np.array_equal(rl.cpu().numpy(), r0), rep
