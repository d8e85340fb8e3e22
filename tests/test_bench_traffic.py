"""bench.py's lookup of the decode kernel's measured HBM traffic (roofline.traffic).

A traffic profile counts only for a run of the same workload and the same launch settings
(partition, grid, packing, fused stages, read policy, late units, private tail) while the kernel
sources hash matches; anything else reports no figure. Host-only: the lookup reads text files.
"""
import os

import pytest

import bench

CFG = {"partition_size": 2048, "grid": "list", "pack_tokens": 0, "append": "fused",
       "copy_on_write": "none", "kv_policy": "stream", "late_units": "ticketed",
       "ticketed_tail_shared_items_moved": 12}


def _profile(tmp_path, name, cfg, sha, traffic):
    path = tmp_path / "profiles" / ("hbm_traffic_%s.txt" % name)
    path.parent.mkdir(exist_ok=True)
    path.write_text("# comment: with a colon\nworkload: %s\nlaunch_key: %s\n"
                    "kernel_source_sha256: %s\ntraffic_bytes_per_launch: %d\n"
                    % (name.split("__")[0], bench.traffic_launch_key(cfg), sha, traffic))


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    return tmp_path


def test_the_matching_launch_settings_pick_the_profile(fake_root):
    keep = dict(CFG, ticketed_tail_shared_items_moved=0)
    _profile(fake_root, "w1", CFG, "abc", 1000)
    _profile(fake_root, "w1__keep_tail", keep, "abc", 1100)
    assert bench.measured_traffic("w1", CFG) == 1000
    assert bench.measured_traffic("w1", keep) == 1100


def test_other_settings_workloads_or_sources_give_none(fake_root):
    _profile(fake_root, "w1", CFG, "abc", 1000)
    assert bench.measured_traffic("w1", dict(CFG, late_units="static")) is None
    assert bench.measured_traffic("w1", dict(CFG, partition_size=1024)) is None
    assert bench.measured_traffic("w2", CFG) is None
    _profile(fake_root, "w3", CFG, "old", 1000)                  # kernel sources changed since
    assert bench.measured_traffic("w3", CFG) is None


def test_committed_profiles_name_their_launch_settings():
    """Every committed traffic profile carries a launch key that bench.py can match."""
    pdir = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    names = [f for f in os.listdir(pdir) if f.startswith("hbm_traffic_")]
    assert names
    for f in names:
        text = open(os.path.join(pdir, f)).read()
        keys = [l.split(":", 1)[1].strip() for l in text.splitlines()
                if l.startswith("launch_key:")]
        assert len(keys) == 1, f
        assert keys[0].split(",")[0].startswith("partition_size=")
        assert len(keys[0].split(",")) == len(bench.TRAFFIC_LAUNCH_KEYS), f
