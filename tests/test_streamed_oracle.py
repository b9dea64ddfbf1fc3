"""The streamed (full-size) oracle agrees with the element-by-element oracle (CPU only).

The full-size GPU tests compare against StreamedOracle, which regroups the
oracle's own per-tensor functions into segments and windows; this checks that
the regrouping changes nothing: same overflow decisions, the same norm and the
same window states, bit for bit, including a step with an injected inf.
"""
import numpy as np
import pytest

from inputs import configs


@pytest.mark.parametrize("name", ["edges", "edges-fp16", "llama3-8B-small"])
def test_streamed_equals_full(name):
    from harness import OracleRun, StreamedOracle, sample_windows
    w = configs.make(name)
    full = OracleRun(w, threads=4)
    wins = sample_windows(w, per_tensor=300, random_count=8, random_len=777)
    so = StreamedOracle(w, wins, threads=4, log=lambda *a: None, seg=70_001)
    assert len(so.segments) > len(w.tensors)          # several segments per large tensor
    for s in range(1, min(w.steps, 4) + 1):
        full.step()
        so.step()
        assert so.found_inf == full.st.found_inf
        assert so.scaler.scale == full.st.scaler.scale
        assert so.clock.t == full.st.clock.t
        if full.st.found_inf:
            assert not np.isfinite(so.sumsq)
        else:
            assert np.float32(so.norm) == np.float32(full.st.norm)
            assert abs(so.sumsq - full.st.sumsq) <= 1e-14 * abs(full.st.sumsq)
        for (t, start, n), st in zip(so.windows, so.state):
            sl = slice(start, start + n)
            for key, arr in (("master", full.st.masters), ("m", full.st.m), ("v", full.st.v),
                             ("w16", full.st.w16)):
                assert np.array_equal(st[key], arr[t][sl]), (name, s, key, t, start)
