"""Calibration tables on disk (rope_aware_eviction_amd.calib_file): a saved
table loads back bit for bit, as the keyword arguments of tri_calibrate_load,
through numpy's pickle-free loader; malformed files are refused.  CPU only:
the library is not called."""
import inspect

import numpy as np
import pytest

import synth
import rope_aware_eviction_amd as tri
from rope_aware_eviction_amd import calib_file


def _table(L=3, n_kv=2, G=4, d=128, seed=5):
    rng = np.random.default_rng(seed)
    shape = (L, n_kv * G, d // 2)
    m = rng.uniform(0.5, 2.0, shape)
    r = rng.uniform(0.0, 1.0, shape)
    return dict(qc_re=rng.normal(size=shape), qc_im=rng.normal(size=shape), q_mean_norm=m,
                q_mrl=r, offsets=np.array(synth.pow2_offsets(16), dtype=np.int64),
                n_kv_heads=n_kv, head_dim=d)


@pytest.mark.parametrize("inv_freq", [None, "explicit"])
def test_round_trip_is_bit_exact(tmp_path, inv_freq):
    t = _table()
    inv = None if inv_freq is None else 1e6 ** (-np.arange(64) / 64.0)
    path = tmp_path / "calib.npz"
    tri.save_calibration(path, **t, rope_theta=1e6, inv_freq=inv)
    got = tri.load_calibration(path)
    # exactly the parameters of tri_calibrate_load, bar the device
    params = set(inspect.signature(tri.tri_calibrate_load).parameters) - {"device"}
    assert set(got) == params
    for k in ("qc_re", "qc_im", "q_mean_norm", "q_mrl"):
        assert got[k].dtype == np.float64 and np.array_equal(got[k], t[k]), k
    assert got["offsets"].dtype == np.int64 and np.array_equal(got["offsets"], t["offsets"])
    assert (got["n_layers"], got["n_kv_heads"], got["n_q_heads"], got["head_dim"]) == (3, 2, 8, 128)
    assert got["rope_theta"] == 1e6
    if inv is None:
        assert got["inv_freq"] is None
    else:
        assert np.array_equal(got["inv_freq"], inv)
    # plain arrays only: numpy's loader with pickles refused reads every field
    with np.load(path, allow_pickle=False) as z:
        assert all(z[k].dtype != object for k in z.files)


def _write(path, **over):
    t = _table()
    fields = dict(format=np.int64(1), n_kv_heads=np.int64(t["n_kv_heads"]),
                  head_dim=np.int64(t["head_dim"]), rope_theta=np.float64(1e4),
                  inv_freq=np.zeros(0), offsets=t["offsets"],
                  **{k: t[k] for k in ("qc_re", "qc_im", "q_mean_norm", "q_mrl")})
    fields.update(over)
    fields = {k: v for k, v in fields.items() if v is not None}
    np.savez(path, **fields)


@pytest.mark.parametrize("over", [
    dict(format=np.int64(2)),                          # unknown format
    dict(q_mrl=None),                                  # a table missing
    dict(qc_im=np.zeros((3, 8, 32))),                  # a table of another shape
    dict(n_kv_heads=np.int64(3)),                      # 8 query heads over 3 KV heads
    dict(head_dim=np.int64(64)),                       # bands do not match head_dim
    dict(offsets=np.zeros(0, dtype=np.int64)),         # no offsets
    dict(inv_freq=np.ones(10)),                        # wrong number of band frequencies
    dict(q_mean_norm=np.ones((3, 8, 64), dtype=np.float32)),   # not fp64
])
def test_malformed_files_are_refused(tmp_path, over):
    path = tmp_path / "bad.npz"
    _write(path, **over)
    with pytest.raises(ValueError):
        calib_file.load_calibration(path)


def test_save_refuses_inconsistent_tables(tmp_path):
    t = _table()
    t["q_mrl"] = t["q_mrl"][:, :4]
    with pytest.raises(ValueError):
        tri.save_calibration(tmp_path / "x.npz", **t)
