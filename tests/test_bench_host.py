"""Host-side logic of bench.py (no GPU): the capture plan of a timed window and
the keying of the profile figures to the kernels' sources."""

from __future__ import annotations

import json

import pytest

import bench


@pytest.mark.parametrize("steps", [1, 5, 16, 20, 255, 256, 257, 1000, 4096, 8192, 8195])
@pytest.mark.parametrize("replicas", [1, 3, 16])
def test_window_plan_covers_exactly_the_steps(steps, replicas):
    per, n_full, rem = bench.window_plan(steps, 256, replicas)
    assert per >= 1 and n_full >= 1 and 0 <= rem < per
    assert per * n_full + rem == steps
    if steps <= 256:
        assert (per, n_full, rem) == (steps, 1, 0)      # one graph, one launch per window
    else:
        assert per % replicas == 0                      # repeated graphs hold whole rotations
        assert per <= max(256, replicas)


def test_window_plan_replays_keep_the_rotation():
    """Step i of a window runs on replica i % R: each repeated graph starts at
    replica 0 and holds whole rotations, and the remainder graph starts at 0 too."""
    R = 16
    per, n_full, rem = bench.window_plan(1000, 256, R)
    order = [i % R for _ in range(n_full) for i in range(per)] + [i % R for i in range(rem)]
    assert order == [i % R for i in range(1000)]


def test_profile_figures_follow_the_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash(("k.hip",))
    prof = tmp_path / "p.json"
    prof.write_text(json.dumps({"kernel_source_hash": h, "kv_dtype": "i8", "hbm_bytes_per_launch": 123}))
    assert bench.profile_figures(str(prof), ("k.hip",), kv_dtype="i8")["hbm_bytes_per_launch"] == 123
    assert bench.profile_figures(str(prof), ("k.hip",), kv_dtype="fp8") is None       # another configuration
    assert bench.profile_figures(str(tmp_path / "none.json"), ("k.hip",)) is None     # no profile
    src.write_text("kernel v2\n")                                                       # the kernel changed
    assert bench.source_hash(("k.hip",)) != h
    assert bench.profile_figures(str(prof), ("k.hip",), kv_dtype="i8") is None
