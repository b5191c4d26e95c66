"""fp64 CPU oracle of the TriAttention online KV-eviction pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product library never links,
loads or calls it, and it shares no code with the HIP path: the arithmetic
lives in ``tri_oracle.c`` (plain C99, fp64, literal steps) and this module only
marshals numpy arrays into it.

Sources: the "TriAttention" paper review on romaanj.github.io (section
"Method", figure 4 caption) and the "TriAttention ... Review" on
dimensionstp.github.io (sections 2-2 and 3-2).  The C file's header lists
the readings taken where the pages leave a step open.

Pinned by ``tests/test_oracle_pins.py`` against brute-force RoPE dot products,
the pages' polar per-band form, closed-form special cases, hand-worked
fixtures, library sorts, brute-force subset search and invariants;
``tests/test_oracle_mutants.py`` checks that planted mistakes fail those pins.
Every function has such pins.  Agreement with the authors' own
implementation cannot be checked (the pages print no worked score example);
the norm-term weight (1 - R_f) * E|q_f| is a reading of the pages' list of
calibrated quantities, stated in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tri_oracle.c")
LIBRARY = os.path.join(_HERE, "libtri_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, used
# when TRI_ORACLE_SANITIZE=1 (the process must preload the ASan runtime)
SAN_LIBRARY = os.path.join(_HERE, "libtri_oracle_san.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def compile_c(src: str, out: str, sanitize: bool = False) -> str:
    """gcc, plain C99, -O2, no fast-math; with sanitize, AddressSanitizer and
    UndefinedBehaviorSanitizer (host code only: the oracle has no GPU part)."""
    tmp = out + ".tmp%d" % os.getpid()
    flags = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra"]
    if sanitize:
        flags += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]
    subprocess.check_call(flags + ["-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def sanitized() -> bool:
    return os.environ.get("TRI_ORACLE_SANITIZE") == "1"


def build(force: bool = False) -> str:
    lib = SAN_LIBRARY if sanitized() else LIBRARY
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(SOURCE):
        compile_c(SOURCE, lib, sanitize=sanitized())
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a, t):
    return a.ctypes.data_as(t)


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        lib = ctypes.CDLL(path)
        lib.tri_oracle_omega.restype = ctypes.c_double
        lib.tri_oracle_omega.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.tri_oracle_unrotate.restype = None
        lib.tri_oracle_unrotate.argtypes = [ctypes.c_int, _dp, ctypes.c_int64, _dp, _dp, _dp]
        lib.tri_oracle_score_head.restype = None
        lib.tri_oracle_score_head.argtypes = [
            ctypes.c_int, ctypes.c_int, _dp, _i64p, ctypes.c_int64, _dp, _i64p,
            ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.tri_oracle_bound_head.restype = None
        lib.tri_oracle_bound_head.argtypes = [
            ctypes.c_int, ctypes.c_int, _dp, _dp, _i64p, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp]
        lib.tri_oracle_select_head.restype = ctypes.c_int
        lib.tri_oracle_select_head.argtypes = [
            ctypes.c_int, _dp, _i64p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.tri_oracle_gqa_head.restype = ctypes.c_int
        lib.tri_oracle_gqa_head.argtypes = [
            ctypes.c_int, ctypes.c_int, _dp, _i64p, ctypes.c_int64, _dp, _i64p,
            ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.tri_oracle_calib_stats.restype = ctypes.c_int
        lib.tri_oracle_calib_stats.argtypes = [ctypes.c_int, ctypes.c_long, _dp, _dp, _dp, _dp, _dp]
        lib.tri_oracle_distance_curve.restype = ctypes.c_int
        lib.tri_oracle_distance_curve.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _i64p,
                                                  ctypes.c_int, _dp]
        lib.tri_oracle_offset_set.restype = ctypes.c_int
        lib.tri_oracle_offset_set.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, _i64p,
                                              ctypes.c_int]
        lib.tri_oracle_select_shared.restype = ctypes.c_int
        lib.tri_oracle_select_shared.argtypes = [
            ctypes.c_int, _i32p, ctypes.c_int, _dp, _i64p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, _i32p, _i32p]
        lib.tri_oracle_gather_rows.restype = None
        lib.tri_oracle_gather_rows.argtypes = [
            ctypes.c_int, _i32p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        self.lib = lib
        self.path = path

    def omega(self, head_dim: int, rope_theta: float) -> np.ndarray:
        """Band frequencies w_f = theta^(-2f/d), f < d/2 (standard RoPE; reading)."""
        return np.array([self.lib.tri_oracle_omega(f, head_dim, float(rope_theta))
                         for f in range(head_dim // 2)], dtype=np.float64)

    def unrotate(self, K_row, p: int, om) -> np.ndarray:
        """Pre-RoPE complex bands of one stored key row at position ``p``."""
        K_row = _f64(K_row)
        om = _f64(om)
        d = K_row.shape[0]
        re = np.empty(d // 2)
        im = np.empty(d // 2)
        self.lib.tri_oracle_unrotate(d, _ptr(K_row, _dp), int(p), _ptr(om, _dp),
                                     _ptr(re, _dp), _ptr(im, _dp))
        return re + 1j * im

    def score_head(self, K, pos, p_now, om, offsets, qc_re, qc_im, q_mean_norm, q_mrl):
        """Returns (trig, norm, score), each fp64 [n], for one (layer, KV head).

        ``K`` is [n][d] stored post-RoPE key rows (any float dtype; upcast
        exactly to fp64), ``pos`` [n] their positions.
        """
        K = _f64(K)
        n, d = K.shape
        pos = _i64(pos)
        om = _f64(om)
        offsets = _i64(offsets)
        qc_re, qc_im, q_mean_norm, q_mrl = (_f64(x) for x in (qc_re, qc_im, q_mean_norm, q_mrl))
        assert pos.shape == (n,) and om.shape == (d // 2,)
        for x in (qc_re, qc_im, q_mean_norm, q_mrl):
            assert x.shape == (d // 2,)
        trig = np.empty(n)
        norm = np.empty(n)
        score = np.empty(n)
        self.lib.tri_oracle_score_head(
            d, n, _ptr(K, _dp), _ptr(pos, _i64p), int(p_now), _ptr(om, _dp),
            _ptr(offsets, _i64p), len(offsets), _ptr(qc_re, _dp), _ptr(qc_im, _dp),
            _ptr(q_mean_norm, _dp), _ptr(q_mrl, _dp),
            _ptr(trig, _dp), _ptr(norm, _dp), _ptr(score, _dp))
        return trig, norm, score

    def bound_head(self, K, om, offsets, qc_re, qc_im, q_mean_norm, q_mrl):
        """Per-key magnitude bound M_i (tolerance scale; |score_i| <= M_i)."""
        K = _f64(K)
        n, d = K.shape
        om = _f64(om)
        offsets = _i64(offsets)
        qc_re, qc_im, q_mean_norm, q_mrl = (_f64(x) for x in (qc_re, qc_im, q_mean_norm, q_mrl))
        out = np.empty(n)
        self.lib.tri_oracle_bound_head(
            d, n, _ptr(K, _dp), _ptr(om, _dp), _ptr(offsets, _i64p), len(offsets),
            _ptr(qc_re, _dp), _ptr(qc_im, _dp), _ptr(q_mean_norm, _dp), _ptr(q_mrl, _dp),
            _ptr(out, _dp))
        return out

    def gqa_head(self, K, pos, p_now, om, offsets, qc_re, qc_im, q_mean_norm, q_mrl):
        """GQA normalize-then-aggregate score of one KV head.

        The calibration arrays are [G][d/2], one row per query head of the
        group.  Returns (raw [G][n], z [G][n], score [n]), fp64: each query
        head's score row, its z-normalized row, and the max over the group.
        """
        K = _f64(K)
        n, d = K.shape
        pos = _i64(pos)
        om = _f64(om)
        offsets = _i64(offsets)
        qc_re, qc_im, q_mean_norm, q_mrl = (_f64(np.atleast_2d(x)) for x in (qc_re, qc_im, q_mean_norm, q_mrl))
        G = qc_re.shape[0]
        for x in (qc_re, qc_im, q_mean_norm, q_mrl):
            assert x.shape == (G, d // 2)
        raw = np.empty((G, n))
        z = np.empty((G, n))
        score = np.empty(n)
        r = self.lib.tri_oracle_gqa_head(
            d, n, _ptr(K, _dp), _ptr(pos, _i64p), int(p_now), _ptr(om, _dp),
            _ptr(offsets, _i64p), len(offsets), G, _ptr(qc_re, _dp), _ptr(qc_im, _dp),
            _ptr(q_mean_norm, _dp), _ptr(q_mrl, _dp), _ptr(raw, _dp), _ptr(z, _dp),
            _ptr(score, _dp))
        if r != 0:
            raise ValueError("bad arguments to the oracle's GQA score")
        return raw, z, score

    def distance_curve(self, om, qc_re, qc_im, kc_re, kc_im, deltas):
        """Distance-preference curve sum_f Re(qc_f conj(kc_f) e^{i w_f delta}) of one head."""
        om = _f64(om)
        qc_re, qc_im, kc_re, kc_im = (_f64(x) for x in (qc_re, qc_im, kc_re, kc_im))
        deltas = _i64(deltas)
        out = np.empty(len(deltas))
        r = self.lib.tri_oracle_distance_curve(2 * len(om), _ptr(om, _dp), _ptr(qc_re, _dp),
                                               _ptr(qc_im, _dp), _ptr(kc_re, _dp),
                                               _ptr(kc_im, _dp), _ptr(deltas, _i64p), len(deltas),
                                               _ptr(out, _dp))
        if r != 0:
            raise ValueError("bad arguments to the oracle's distance curve")
        return out

    def offset_set(self, kind: str, max_distance: int, count: int = 0) -> np.ndarray:
        """Future-offset set: 'geometric' (powers of two up to max_distance) or
        'linear' (count evenly spaced offsets ending at max_distance)."""
        k = {"geometric": 0, "linear": 1}[kind]
        n = self.lib.tri_oracle_offset_set(k, int(max_distance), int(count),
                                           _ptr(np.empty(1, dtype=np.int64), _i64p), 0)
        if n < 0:
            raise ValueError("bad offset-set arguments")
        out = np.empty(max(n, 1), dtype=np.int64)
        self.lib.tri_oracle_offset_set(k, int(max_distance), int(count), _ptr(out, _i64p), n)
        return out[:n].copy()

    def calib_stats(self, Q):
        """(qc_re, qc_im, q_mean_norm, q_mrl), each fp64 [d/2], of one query
        head from pre-RoPE query samples Q [n][d]."""
        Q = _f64(Q)
        n, d = Q.shape
        out = [np.empty(d // 2) for _ in range(4)]
        r = self.lib.tri_oracle_calib_stats(d, n, _ptr(Q, _dp), *(_ptr(o, _dp) for o in out))
        if r != 0:
            raise ValueError("bad arguments to the oracle's calibration statistics")
        return tuple(out)

    def select_head(self, score, pos, budget: int, window: int):
        """Kept slots (ascending) of one head, or None when the head does not fire."""
        score = _f64(score)
        pos = _i64(pos)
        n = score.shape[0]
        kept = np.empty(max(budget, 1), dtype=np.int32)
        r = self.lib.tri_oracle_select_head(n, _ptr(score, _dp), _ptr(pos, _i64p),
                                            int(budget), int(window), _ptr(kept, _i32p))
        if r < 0:
            raise ValueError("bad arguments to the oracle's select")
        if r == 0:
            return None
        return kept[:r].copy()

    def select_shared(self, scores, pos, lens, total: int, floor: int, window: int):
        """Head-specific budgets of one layer: ``scores``/``pos`` [H][stride],
        ``lens`` [H] keys in use per head.  Returns a list of H ascending kept
        slot arrays, or None when the layer does not fire."""
        scores = _f64(np.atleast_2d(scores))
        pos = _i64(np.atleast_2d(pos))
        H, stride = scores.shape
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        kept = np.empty(H * total, dtype=np.int32)
        count = np.empty(H, dtype=np.int32)
        r = self.lib.tri_oracle_select_shared(H, _ptr(lens, _i32p), stride, _ptr(scores, _dp),
                                              _ptr(pos, _i64p), int(total), int(floor),
                                              int(window), _ptr(kept, _i32p), _ptr(count, _i32p))
        if r < 0:
            raise ValueError("bad arguments to the oracle's shared select")
        if r == 0:
            return None
        return [kept[h * total:h * total + count[h]].copy() for h in range(H)]

    def gather_rows(self, kept, rows: np.ndarray) -> np.ndarray:
        """dst[r] = rows[kept[r]] (bytes copied exactly)."""
        kept = np.ascontiguousarray(kept, dtype=np.int32)
        rows = np.ascontiguousarray(rows)
        row_bytes = rows.strides[0] if rows.ndim > 1 else rows.itemsize
        out = np.empty((len(kept),) + rows.shape[1:], dtype=rows.dtype)
        self.lib.tri_oracle_gather_rows(len(kept), _ptr(kept, _i32p), int(row_bytes),
                                        rows.ctypes.data, out.ctypes.data)
        return out

    def prune_head(self, K, V, pos, p_now, om, offsets, qc_re, qc_im, q_mean_norm, q_mrl,
                   budget, window):
        """One head's full prune step: score, top-B, gather.  With [G][d/2]
        calibration arrays the score is the GQA normalize-then-aggregate one.

        Returns dict(score, kept, K, V, pos); kept/K/V/pos are None when the
        head does not fire.
        """
        if np.ndim(qc_re) == 2:         # [G][d/2]: a GQA group sharing this KV head
            _, _, score = self.gqa_head(K, pos, p_now, om, offsets, qc_re, qc_im, q_mean_norm, q_mrl)
        else:
            _, _, score = self.score_head(K, pos, p_now, om, offsets, qc_re, qc_im,
                                          q_mean_norm, q_mrl)
        kept = self.select_head(score, pos, budget, window)
        if kept is None:
            return dict(score=score, kept=None, K=None, V=None, pos=None)
        return dict(score=score, kept=kept, K=self.gather_rows(kept, K),
                    V=self.gather_rows(kept, V), pos=self.gather_rows(kept, np.asarray(pos)))

    def prune_layer_shared(self, heads, total: int, floor: int, window: int, threads: int = 1):
        """One layer's prune step with head-specific budgets: scores every
        head (``heads``: dicts of K, V, pos, p_now, om, offsets and the head's
        calibration arrays, [G][d/2] for a GQA group), selects with
        select_shared over the layer and gathers each head's kept rows.
        Returns a list of dicts (kept, K, V, pos) per head, or None when the
        layer does not fire."""
        def score(j):
            args = (j["K"], j["pos"], j["p_now"], j["om"], j["offsets"], j["qc_re"], j["qc_im"],
                    j["q_mean_norm"], j["q_mrl"])
            if np.ndim(j["qc_re"]) == 2:
                return self.gqa_head(*args)[2]
            return self.score_head(*args)[2]
        if threads > 1:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                sc = list(ex.map(score, heads))
        else:
            sc = [score(j) for j in heads]
        lens = [len(x) for x in sc]
        stride = max(lens) if lens else 0
        S = np.full((len(heads), max(stride, 1)), -np.inf)
        P = np.zeros((len(heads), max(stride, 1)), dtype=np.int64)
        for h, (x, j) in enumerate(zip(sc, heads)):
            S[h, :len(x)] = x
            P[h, :len(x)] = j["pos"]
        kept = self.select_shared(S, P, lens, total, floor, window)
        if kept is None:
            return None
        return [dict(kept=k, K=self.gather_rows(k, j["K"]), V=self.gather_rows(k, j["V"]),
                     pos=self.gather_rows(k, j["pos"])) for k, j in zip(kept, heads)]

    def prune_heads_parallel(self, jobs, threads: int):
        """Runs ``prune_head(**job)`` for every job on ``threads`` host threads
        (the C calls release the GIL).  Returns the results in job order."""
        if threads <= 1:
            return [self.prune_head(**j) for j in jobs]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(lambda j: self.prune_head(**j), jobs))


_default = None


def load() -> Oracle:
    """The oracle built from ``tri_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default
