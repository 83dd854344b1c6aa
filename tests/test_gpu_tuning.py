"""The library's own choice without tuning against the tuner's, at the two
scored shapes (the phobos docs, page "gemm, f32", section "Tuning": the best
tile depends on the card and the sizes, so the untuned choice should already
be close to what a search finds).  Both tiles are timed pinned, interleaved
over rounds (one sample = 10 back-to-back calls between two events), and the
untuned one must be within 2% of the tuned one by median; both results must
also be inside the oracle's bound on sampled elements."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, sample_indices, workload_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU-only hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

import gemm_tiled_amd as g  # noqa: E402
from tests.gpu_helpers import pinned, say, to_device  # noqa: E402


def _sample_time(w, cfg, tA, tB, tC, calls=10):
    s = torch.cuda.current_stream()
    with pinned(w.mode, cfg):
        for _ in range(3):
            g.gemm(w.mode, tA, tB, tC, w.alpha, w.beta)
        begin, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        begin.record(s)
        for _ in range(calls):
            g.gemm(w.mode, tA, tB, tC, w.alpha, w.beta)
        end.record(s)
        end.synchronize()
    return begin.elapsed_time(end) / calls


@pytest.mark.parametrize("name", ["f32_4096_a1_b0", "f32_4096_a1_b1", "f16r_8192_a0.75_b-0.25"])
def test_untuned_choice_within_2pct_of_tuned(name):
    w = WORKLOADS[name]
    A, B, C = workload_inputs(w)
    tA, tB, tC = to_device(A), to_device(B), to_device(C)
    g.cache_clear()
    try:
        heur = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)
        assert heur.endswith("source=heuristic"), heur
        heur = heur.split(" source=")[0]
        say(f"[tuning] {name}: untuned {heur}")
        g.tune(w.mode, tA, tB, tC, beta=w.beta)
        tuned = g.get_config(w.mode, w.M, w.N, w.K, beta=w.beta)
        assert tuned.endswith("source=tuned"), tuned
        tuned = tuned.split(" source=")[0]
        say(f"[tuning] {name}: tuned {tuned}")
        times = {heur: [], tuned: []}
        for _ in range(9):
            for cfg in times:
                times[cfg].append(_sample_time(w, cfg, tA, tB, tC))
        med = {c: float(np.median(t)) for c, t in times.items()}
        say(f"[tuning] {name}: untuned {med[heur]:.4f} ms, tuned {med[tuned]:.4f} ms")
        assert med[heur] <= 1.02 * med[tuned], med
        for cfg in times:   # both results correct
            C2 = to_device(C)
            with pinned(w.mode, cfg):
                g.gemm(w.mode, tA, tB, C2, w.alpha, w.beta)
            torch.cuda.synchronize()
            got = C2.cpu().numpy()
            r, c = sample_indices(w.M, w.N, 1024, seed=7)
            ref, W = oracle.entries(w.mode, A, B, C, w.alpha, w.beta, r, c)
            assert np.all(np.abs(got[r, c].astype(np.float64) - ref) <= oracle.TOL[w.mode] * W)
    finally:
        g.cache_clear()
