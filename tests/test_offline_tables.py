"""Persisted offline tables (placement, token->group table, affinity table):
the .npz round trip is exact, keys follow every configuration field, and
files of another configuration, corrupted keys or invalid tables are
rejected.  CPU only."""
import os

import numpy as np
import pytest

from token_routing_shuffle_amd import offline
from token_routing_shuffle_amd import workload as wl


def _lut(cfg):
    return (np.arange(cfg.V) * 7 % cfg.P).astype(np.int32)


@pytest.mark.parametrize("name", ["tiny", "dsv3_decode", "prism"])
def test_round_trip_is_exact(tmp_path, name):
    cfg = wl.CONFIGS[name]
    t = wl.make_tables(cfg, profile_tokens=1024)
    path = offline.save_tables(str(tmp_path), cfg, t, _lut(cfg), 1024)
    assert os.path.basename(path).startswith(name + "_")
    got = offline.load_tables(str(tmp_path), cfg, 1024)
    assert (got["slot_to_orig"] == t.slot_to_orig).all() and (got["perm"] == t.perm).all()
    assert (got["lut"] == _lut(cfg)).all()
    assert ("pref" in got) == (t.pref is not None)
    if t.pref is not None:
        assert (got["pref"] == t.pref).all()
    if t.ebias is not None:
        assert got["ebias"].tobytes() == t.ebias.tobytes()


def test_keys_follow_the_configuration(tmp_path):
    cfg = wl.CONFIGS["dsv2lite"]
    k = offline.config_key(cfg, 65536)
    assert k == offline.config_key(wl.CONFIGS["dsv2lite"], 65536)
    assert k != offline.config_key(cfg.replace(T=4095), 65536)
    assert k != offline.config_key(cfg.replace(aff_bias=2.0), 65536)
    assert k != offline.config_key(cfg, 4096)
    assert k != offline.config_key(cfg, 65536, placement="optimised")
    assert offline.load_tables(str(tmp_path), cfg, 65536) is None


def test_corrupted_files_are_rejected(tmp_path):
    cfg = wl.CONFIGS["tiny"]
    t = wl.make_tables(cfg, profile_tokens=256)
    path = offline.save_tables(str(tmp_path), cfg, t, _lut(cfg), 256)
    with np.load(path) as z:
        arrays = {k: z[k] for k in z.files}
    bad = dict(arrays, lut=np.full(cfg.V, cfg.P, np.int32))
    np.savez(path, **bad)
    with pytest.raises(ValueError):
        offline.load_tables(str(tmp_path), cfg, 256)
    bad = dict(arrays, key=np.frombuffer(b"0" * 24, np.uint8))
    np.savez(path, **bad)
    with pytest.raises(ValueError):
        offline.load_tables(str(tmp_path), cfg, 256)
