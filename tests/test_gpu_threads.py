"""The library's scratch (packed binary16 operands, split-K partial tiles and
arrival counters) under concurrent callers, growth and stream capture, through
the C ABI on the GPU.

Calls from several host threads on one stream (the default stream, where one
call's launches could land between another's) and on streams of their own must
each give the result of the same call made alone; a call whose scratch must
grow while earlier calls on the stream are still running must not disturb them
(the old buffer is freed stream-ordered); under capture a call that would have
to allocate fails cleanly and launches nothing.
"""
from __future__ import annotations

import ctypes
import threading

import numpy as np
import pytest

import oracle
from workloads import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import say, to_device  # noqa: E402

# (mode, M, N, K): f16r packed path (operands in scratch), f16r rounding on
# load with K split (partials + counters), f32 few rows (partials + counters),
# f32 split-K tiles (partials, second pass)
CASES = [("f16r", 1280, 384, 3072), ("f16r", 200, 1000, 3000), ("f32", 8, 4096, 4096),
         ("f32", 64, 2048, 4096), ("f16r", 1024, 1536, 640)]


def _prepare(seed0):
    out = []
    for i, (mode, M, N, K) in enumerate(CASES):
        A, B, C = make_inputs(M, N, K, "uniform", seed=seed0 + i)
        tA, tB = to_device(A), to_device(B)
        tC = torch.zeros((M, N), device="cuda", dtype=torch.float32)
        say(f"[threads] serial {mode} {M}x{N}x{K} {g.get_config(mode, M, N, K, beta=0.0)}")
        g.gemm(mode, tA, tB, tC, 1.25, 0.0)
        torch.cuda.synchronize()
        out.append((mode, A, B, C, tA, tB, tC.cpu().numpy()))
    return out


def _check(cases, outs):
    for (mode, A, B, C, _, _, ref), got in zip(cases, outs):
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (mode, A.shape, B.shape)
        st = oracle.check(mode, A, B, C, 1.25, 0.0, got)
        assert st["n_fail"] == 0, st


@pytest.mark.parametrize("own_streams", [False, True])
def test_threads_calling_at_once(own_streams):
    """Each case runs in a thread of its own, 40 calls in a row (beta = 0, so
    every call writes the same result); all threads on the default stream, or
    each on a stream of its own."""
    cases = _prepare(40)
    outs = [torch.full((c[1].shape[0], c[2].shape[1]), float("nan"), device="cuda")
            for c in cases]
    streams = [torch.cuda.Stream() if own_streams else torch.cuda.default_stream()
               for _ in cases]
    errors = []
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            mode, _, _, _, tA, tB, _ = cases[i]
            start.wait()
            with torch.cuda.stream(streams[i]):
                for _ in range(40):
                    g.gemm(mode, tA, tB, outs[i], 1.25, 0.0)
        except Exception as e:   # noqa: BLE001 -- reported below
            errors.append(e)

    say(f"[threads] {len(cases)} threads, own streams: {own_streams}")
    ts = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    _check(cases, [o.cpu().numpy() for o in outs])


def test_growth_while_earlier_calls_run():
    """On one stream, without synchronising: a small f16r call, a much larger
    one (its packed operands need a larger buffer: the old one is freed
    stream-ordered behind the first call), then a small one again; every
    result equals the call made alone."""
    shapes = [(256, 256, 256), (2048, 2048, 2048), (384, 128, 512)]
    s = torch.cuda.Stream()
    prepared, outs = [], []
    for i, (M, N, K) in enumerate(shapes):
        A, B, C = make_inputs(M, N, K, "normal", seed=70 + i)
        prepared.append(("f16r", A, B, C, to_device(A), to_device(B), None))
    torch.cuda.synchronize()
    say("[threads] growth on one stream")
    with torch.cuda.stream(s):
        for (_, A, B, _, tA, tB, _) in prepared:
            tC = torch.zeros((A.shape[0], B.shape[1]), device="cuda")
            g.gemm("f16r", tA, tB, tC, 1.25, 0.0)
            outs.append(tC)
    s.synchronize()
    for (mode, A, B, C, _, _, _), got in zip(prepared, outs):
        st = oracle.check(mode, A, B, C, 1.25, 0.0, got.cpu().numpy())
        assert st["n_fail"] == 0, st


def _new_hip_stream():
    """A stream created here (torch's own streams come from a pool that
    earlier calls may have used, so they may already hold scratch)."""
    hip = ctypes.CDLL("libamdhip64.so")
    ptr = ctypes.c_void_p()
    assert hip.hipStreamCreateWithFlags(ctypes.byref(ptr), ctypes.c_uint(1)) == 0   # non-blocking
    return hip, ptr, torch.cuda.ExternalStream(ptr.value)


def test_capture_without_scratch_fails_and_launches_nothing():
    """A new stream holds no scratch: capturing an f16r call on it (which
    needs its packed operands) must return GEMM355_ERR_CAPTURE (-106) and
    leave C untouched; the same call runs eagerly afterwards."""
    M, N, K = 1280, 384, 3072   # the packed path: its binary16 operands live in scratch
    assert g.get_plan("f16r", M, N, K, beta=0.5).startswith("form=packed")
    A, B, C = make_inputs(M, N, K, "uniform", seed=81)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    hip, ptr, s = _new_hip_stream()
    try:
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        say("[threads] capture on a new stream")
        with pytest.raises(g.Gemm355Error) as err:
            with torch.cuda.graph(graph, stream=s):
                g.gemm("f16r", tA, tB, tC, 1.0, 0.5)
        assert err.value.status == -106, err.value
        torch.cuda.synchronize()
        assert np.array_equal(tC.cpu().numpy(), C)
        with torch.cuda.stream(s):
            g.gemm("f16r", tA, tB, tC, 1.0, 0.5)
        s.synchronize()
        st = oracle.check("f16r", A, B, C, 1.0, 0.5, tC.cpu().numpy())
        assert st["n_fail"] == 0, st
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(ptr)
