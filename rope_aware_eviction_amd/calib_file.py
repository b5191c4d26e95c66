"""Calibration tables on disk.

The calibration table is the only state the eviction pass keeps between
runs: the per-band query statistics are measured once, offline, and reused
for every prune step ("TriAttention" review, romaanj.github.io, section
"Method": offline calibration of the per-band centre, mean norm and mean
resultant length).  The file is a plain ``.npz`` of numeric arrays (no
pickled objects; it loads with ``numpy.load(allow_pickle=False)``):

    format        int64 scalar, 1
    n_kv_heads    int64 scalar
    head_dim      int64 scalar
    rope_theta    float64 scalar
    inv_freq      float64 [head_dim/2] explicit band frequencies, or [0] (theta^(-2f/d))
    offsets       int64 [n_offsets] future offsets
    qc_re, qc_im, q_mean_norm, q_mrl
                  float64 [n_layers][n_q_heads][head_dim/2]

``load_calibration`` returns the keyword arguments of ``tri_calibrate_load``,
so a context is ``tri_calibrate_load(**load_calibration(path), device=0)``.
The values themselves (finite, in range) are checked by the library when the
table is loaded onto a device.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

FORMAT = 1
_TABLES = ("qc_re", "qc_im", "q_mean_norm", "q_mrl")


def save_calibration(path, qc_re, qc_im, q_mean_norm, q_mrl, offsets, n_kv_heads: int,
                     head_dim: int, rope_theta: float = 10000.0, inv_freq=None) -> None:
    """Writes a calibration table (arrays [n_layers][n_q_heads][head_dim/2])."""
    tables = {n: np.ascontiguousarray(a, dtype=np.float64)
              for n, a in zip(_TABLES, (qc_re, qc_im, q_mean_norm, q_mrl))}
    inv = np.zeros(0) if inv_freq is None else np.ascontiguousarray(inv_freq, dtype=np.float64)
    fields = dict(format=np.int64(FORMAT), n_kv_heads=np.int64(n_kv_heads),
                  head_dim=np.int64(head_dim), rope_theta=np.float64(rope_theta), inv_freq=inv,
                  offsets=np.ascontiguousarray(offsets, dtype=np.int64), **tables)
    _check(fields)
    np.savez(path, **fields)


def load_calibration(path) -> dict:
    """Reads a table written by save_calibration; raises ValueError on a file
    that is not one."""
    with np.load(path, allow_pickle=False) as z:
        missing = {"format", "n_kv_heads", "head_dim", "rope_theta", "inv_freq", "offsets",
                   *_TABLES} - set(z.files)
        if missing:
            raise ValueError("not a calibration table: missing %s" % sorted(missing))
        fields = {k: z[k] for k in z.files}
    _check(fields)
    n_layers, n_q_heads, _ = fields["qc_re"].shape
    inv: Optional[np.ndarray] = fields["inv_freq"] if fields["inv_freq"].size else None
    return dict(n_layers=int(n_layers), n_kv_heads=int(fields["n_kv_heads"]),
                head_dim=int(fields["head_dim"]),
                **{n: fields[n].astype(np.float64, copy=False) for n in _TABLES},
                offsets=fields["offsets"].astype(np.int64, copy=False),
                rope_theta=float(fields["rope_theta"]), inv_freq=inv, n_q_heads=int(n_q_heads))


def _check(f: dict) -> None:
    if f["format"].shape != () or int(f["format"]) != FORMAT:
        raise ValueError("calibration table format %r, expected %d" % (f["format"], FORMAT))
    for k in ("n_kv_heads", "head_dim", "rope_theta"):
        if np.shape(f[k]) != ():
            raise ValueError("%s must be a scalar" % k)
    d, hkv = int(f["head_dim"]), int(f["n_kv_heads"])
    shape = f["qc_re"].shape
    if len(shape) != 3 or shape[2] != d // 2 or d < 2 or d % 2 or shape[0] < 1:
        raise ValueError("tables must be [n_layers][n_q_heads][head_dim/2], got %s" % (shape,))
    if hkv < 1 or shape[1] % hkv:
        raise ValueError("n_q_heads (%d) must be a multiple of n_kv_heads (%d)" % (shape[1], hkv))
    for n in _TABLES:
        if f[n].shape != shape or f[n].dtype != np.float64:
            raise ValueError("%s must be float64 of shape %s" % (n, shape))
    if f["offsets"].ndim != 1 or f["offsets"].size < 1 or f["offsets"].dtype != np.int64:
        raise ValueError("offsets must be a non-empty int64 vector")
    inv = f["inv_freq"]
    if inv.dtype != np.float64 or inv.ndim != 1 or inv.size not in (0, d // 2):
        raise ValueError("inv_freq must be float64 [head_dim/2] or empty")
