"""Seeded synthetic KV caches and calibration tables for the eviction pass.

This module is the one place that makes inputs.  It serves the fp64 oracle,
the HIP path, the tests and the benchmark alike, and holds none of the
eviction method's arithmetic: it draws pre-RoPE keys around per-head centres,
stores them post-RoPE (the rotation a model applies before caching a key),
and draws the query-side calibration statistics.  It never scores, selects or
compacts anything.

Workloads (the five cache shapes the pass is specified on):

``toy``      1 layer x 2 KV heads, head_dim 64, theta 1e4, 512 keys at
             positions 0..511, budget 128, fp32, offsets 2^0..2^12.
``llama8b``  32 x 8, head_dim 128, theta 5e5, 8192 keys, budget 2048, bf16,
             noise sigma = 0.25*||c||/sqrt(d), 5% outlier keys with 3x norm.
``qwen3_32k`` 36 x 8, head_dim 128, theta 1e6, 32768 keys, budget 4096, bf16;
             per-head band-phase concentration R_h ~ U(0.6, 0.99).
``batched``  64 sequences of the llama8b shape with lengths ~ U{4096..32768},
             budget 2048, window 128.
``wide``     64 x 8, head_dim 128, theta 1e6, 131072 keys, budget 8192, bf16;
             20% of slots hold a copy of another slot's stored row with one
             element nudged by one bf16 ulp (adversarial near-ties).

GQA workloads (G query heads share each KV head; query head g > 0 of a group
has its own centre, concentration and a score scale e^U(-0.7, 0.7)):
``gqa_toy`` (toy shape, G = 2, fp32), ``gqa_small`` (2 x 4, d 128, 4096 keys,
G = 4, bf16), ``gqa_g7`` (1 x 4, d 128, G = 7, phase recipe), ``gqa_g8_d64``
(2 x 2, d 64, 8192 keys, G = 8) and ``qwen3_32k_gqa`` (the qwen3_32k shape with
G = 4: 32 query heads over 8 KV heads).

Recipe details and the readings behind them are written out in each
``_draw_*`` function.  Calibration statistics and key centres (the "model")
are drawn on the host in fp64 from numpy and do not depend on the device;
key noise is drawn with torch on the device the cache is made on, so a cache
made on the GPU differs from one made on the host with the same seed, and
tests that compare against the oracle copy the GPU-made inputs back to the
host before anything else touches them.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional, Sequence

import numpy as np
import torch


# --------------------------------------------------------------------------
# specs


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    n_layers: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    lengths: tuple          # one cache length per sequence
    budget: int
    window: int
    dtype: str              # "f32" or "bf16"
    offsets: tuple          # future offsets (the averaging set)
    recipe: str             # "toy", "concentrated", "phase", "neartie"
    outlier_frac: float = 0.0
    dup_frac: float = 0.0
    group: int = 1          # query heads per KV head (GQA); 1 = one query table per KV head

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def n_seq(self) -> int:
        return len(self.lengths)

    @property
    def heads(self) -> int:
        return self.n_layers * self.n_kv_heads

    @property
    def row_bytes(self) -> int:
        return self.head_dim * (4 if self.dtype == "f32" else 2)

    @property
    def keys(self) -> int:
        return self.heads * sum(self.lengths)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


def pow2_offsets(max_exp: int) -> tuple:
    """Geometric future offsets 1, 2, 4, ..., 2^max_exp."""
    return tuple(1 << e for e in range(max_exp + 1))


def _batched_lengths(seed: int, n: int = 64, lo: int = 4096, hi: int = 32768) -> tuple:
    rng = np.random.Generator(np.random.Philox(key=_key(seed, "batched-lengths")))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


def workload(name: str, seed: int = 0) -> Spec:
    """The named workload's spec (sizes as specified)."""
    if name == "toy":
        return Spec("toy", 1, 2, 64, 1e4, (512,), 128, 128, "f32", pow2_offsets(12), "toy")
    if name == "llama8b":
        return Spec("llama8b", 32, 8, 128, 5e5, (8192,), 2048, 128, "bf16",
                    pow2_offsets(16), "concentrated", outlier_frac=0.05)
    if name == "qwen3_32k":
        return Spec("qwen3_32k", 36, 8, 128, 1e6, (32768,), 4096, 128, "bf16",
                    pow2_offsets(16), "phase")
    if name == "batched":
        return Spec("batched", 32, 8, 128, 5e5, _batched_lengths(seed), 2048, 128, "bf16",
                    pow2_offsets(16), "concentrated", outlier_frac=0.05)
    if name == "wide":
        return Spec("wide", 64, 8, 128, 1e6, (131072,), 8192, 128, "bf16",
                    pow2_offsets(16), "neartie", dup_frac=0.20)
    # GQA: several query heads per KV head, each with its own calibration
    if name == "gqa_toy":
        return Spec("gqa_toy", 1, 2, 64, 1e4, (512,), 128, 128, "f32", pow2_offsets(12), "toy",
                    group=2)
    if name == "gqa_small":
        return Spec("gqa_small", 2, 4, 128, 5e5, (4096,), 1024, 128, "bf16", pow2_offsets(16),
                    "concentrated", outlier_frac=0.05, group=4)
    if name == "gqa_g7":
        return Spec("gqa_g7", 1, 4, 128, 1e6, (4096,), 1024, 128, "bf16", pow2_offsets(16),
                    "phase", group=7)
    if name == "gqa_g8_d64":
        return Spec("gqa_g8_d64", 2, 2, 64, 1.5e5, (8192,), 2048, 128, "bf16", pow2_offsets(16),
                    "concentrated", group=8)
    if name == "qwen3_32k_gqa":
        return Spec("qwen3_32k_gqa", 36, 8, 128, 1e6, (32768,), 4096, 128, "bf16",
                    pow2_offsets(16), "phase", group=4)
    raise KeyError(name)


WORKLOADS = ("toy", "llama8b", "qwen3_32k", "batched", "wide")
GQA_WORKLOADS = ("gqa_toy", "gqa_small", "gqa_g7", "gqa_g8_d64", "qwen3_32k_gqa")


# --------------------------------------------------------------------------
# seeding


def _key(seed: int, *parts) -> int:
    h = hashlib.sha256(repr((int(seed),) + tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little")


def _np_rng(seed: int, *parts) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=_key(seed, *parts)))


def _torch_gen(device, seed: int, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_key(seed, *parts) & ((1 << 63) - 1))
    return g


# --------------------------------------------------------------------------
# the "model": per-head key centres and query calibration statistics


@dataclasses.dataclass
class Calib:
    """Query-side calibration table, fp64, each [n_layers][n_q_heads][d/2]
    (query heads j*G .. j*G+G-1 share KV head j)."""
    qc_re: np.ndarray
    qc_im: np.ndarray
    q_mean_norm: np.ndarray
    q_mrl: np.ndarray
    rope_theta: float
    offsets: np.ndarray     # int64


def _unit_norm_scaled(rng: np.random.Generator, d: int, norm: float) -> np.ndarray:
    x = rng.standard_normal(d)
    return x * (norm / np.linalg.norm(x))


def _model(spec: Spec, seed: int):
    """Key centres c [L][H][d] and the calibration table, drawn in fp64.

    Key and query centres are N(0, I_d) scaled to norm 4 (the toy recipe,
    taken for every workload that does not say otherwise).  Band f of a
    vector x is x[f] + i*x[f+d/2].
    """
    L, H, d, G = spec.n_layers, spec.n_kv_heads, spec.head_dim, spec.group
    h = d // 2
    kc = np.empty((L, H, d))
    qc_re = np.empty((L, H * G, h))
    qc_im = np.empty((L, H * G, h))
    qm = np.empty((L, H * G, h))
    qr = np.empty((L, H * G, h))
    conc = np.empty((L, H))

    def query_table(rng, zq, R_h=None):
        if spec.recipe == "phase":
            # Query band phases with mean resultant length R_h: the
            # calibrated centre is |c_f| * R_h * e^{i arg c_f}, the mean
            # norm |c_f|, the band MRL R_h.
            qc = np.abs(zq) * R_h * np.exp(1j * np.angle(zq))
            return qc.real, qc.imag, np.abs(zq), np.full(h, R_h)
        # E[q_f] = centre band; E|q_f| = |E q_f| * (1 + U(0, 0.5));
        # R_f = |E q_f| / E|q_f| (consistent MRL).
        m = np.abs(zq) * (1.0 + rng.uniform(0.0, 0.5, size=h))
        return zq.real, zq.imag, m, np.abs(zq) / m

    for l in range(L):
        for j in range(H):
            rng = _np_rng(seed, spec.name, "model", l, j)
            kc[l, j] = _unit_norm_scaled(rng, d, 4.0)
            cq = _unit_norm_scaled(rng, d, 4.0)
            zq = cq[:h] + 1j * cq[h:]
            R_h = None
            if spec.recipe == "phase":
                R_h = rng.uniform(0.6, 0.99)
                conc[l, j] = R_h
            else:
                conc[l, j] = np.nan
            row = j * G
            qc_re[l, row], qc_im[l, row], qm[l, row], qr[l, row] = query_table(rng, zq, R_h)
            # GQA: the other query heads of the group have their own centres,
            # concentrations and score scales (scale e^U(-0.7, 0.7)), which is
            # what makes per-query-head normalization matter.
            for g in range(1, G):
                rq = _np_rng(seed, spec.name, "model-q", l, j, g)
                cq = _unit_norm_scaled(rq, d, 4.0) * math.exp(rq.uniform(-0.7, 0.7))
                zq = cq[:h] + 1j * cq[h:]
                R_g = rq.uniform(0.6, 0.99) if spec.recipe == "phase" else None
                qc_re[l, row + g], qc_im[l, row + g], qm[l, row + g], qr[l, row + g] = \
                    query_table(rq, zq, R_g)
    calib = Calib(qc_re, qc_im, qm, qr, float(spec.rope_theta),
                  np.asarray(spec.offsets, dtype=np.int64))
    return kc, conc, calib


# --------------------------------------------------------------------------
# caches


@dataclasses.dataclass
class Cache:
    spec: Spec
    k: List[torch.Tensor]        # per sequence [L][H][cap][d]
    v: List[torch.Tensor]        # same shape as k
    pos: List[torch.Tensor]      # per sequence int32 [L][H][cap]
    lens: List[int]
    p_now: List[int]
    calib: Calib
    seed: int

    @property
    def device(self):
        return self.k[0].device


def _torch_dtype(name: str):
    return torch.float32 if name == "f32" else torch.bfloat16


def _rope_tables(d: int, theta: float, positions: torch.Tensor, device):
    """cos/sin of theta^(-2f/d) * p, computed in fp64, returned as fp32."""
    h = d // 2
    f = torch.arange(h, dtype=torch.float64, device=device)
    inv = torch.pow(torch.tensor(float(theta), dtype=torch.float64, device=device), -2.0 * f / d)
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def _store_post_rope(k_pre: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotates pre-RoPE keys [..., n, d] to the stored form: band f turns by
    the angle of its position (real 2x2 rotation of (x[f], x[f+d/2]))."""
    h = k_pre.shape[-1] // 2
    a, b = k_pre[..., :h], k_pre[..., h:]
    return torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1)


def _draw_concentrated(gen, centre, n, sigma, outlier_frac, device):
    """k = c_h + sigma * N(0, I); a fraction of keys scaled by 3 (outliers)."""
    H, d = centre.shape
    k = torch.randn((H, n, d), generator=gen, device=device, dtype=torch.float32)
    k.mul_(sigma).add_(centre[:, None, :])
    if outlier_frac > 0:
        mask = torch.rand((H, n), generator=gen, device=device) < outlier_frac
        k = torch.where(mask[..., None], k * 3.0, k)
    return k


def _draw_phase(gen, centre, conc, n, device):
    """Band f = |c_f| * e^{0.25 N(0,1)} * e^{i(arg c_f + eps)}, eps ~ N(0, -2 ln R_h),
    so the band phases have mean resultant length R_h (wrapped normal) and the
    magnitudes jitter log-normally."""
    H, d = centre.shape
    h = d // 2
    zr, zi = centre[:, :h], centre[:, h:]
    mag = torch.sqrt(zr * zr + zi * zi)
    arg = torch.atan2(zi, zr)
    sig = torch.sqrt(-2.0 * torch.log(conc))
    jit = torch.randn((H, n, h), generator=gen, device=device, dtype=torch.float32)
    m = mag[:, None, :] * torch.exp(0.25 * jit)
    eps = torch.randn((H, n, h), generator=gen, device=device, dtype=torch.float32)
    ph = arg[:, None, :] + sig[:, None, None] * eps
    return torch.cat([m * torch.cos(ph), m * torch.sin(ph)], dim=-1)


def _nudge_bf16_ulp(x: torch.Tensor, sign: torch.Tensor) -> torch.Tensor:
    """Moves bf16 values one ulp in magnitude (+1 or -1 on the magnitude bits);
    zeros always move up, values next to infinity always move down."""
    bits = x.view(torch.int16).to(torch.int32) & 0xFFFF
    mag = bits & 0x7FFF
    s = torch.where(mag == 0, torch.ones_like(sign), sign)
    s = torch.where(mag + s >= 0x7F80, -torch.ones_like(s), s)
    out = (bits & 0x8000) | (mag + s)
    out = torch.where(out >= 0x8000, out - 0x10000, out)
    return out.to(torch.int16).view(torch.bfloat16)


def _near_ties(gen, K: torch.Tensor, frac: float) -> torch.Tensor:
    """Overwrites a fraction of slots per head with another slot's stored row,
    one random element nudged by one bf16 ulp.  K: [H][n][d] bf16."""
    H, n, d = K.shape
    n_dup = int(round(frac * n))
    if n_dup == 0:
        return K
    dev = K.device
    perm = torch.argsort(torch.rand((H, n), generator=gen, device=dev), dim=1)
    tgt = perm[:, :n_dup]                     # slots that receive a copy
    src_pool = perm[:, n_dup:]                # slots that keep their own row
    pick = torch.randint(0, n - n_dup, (H, n_dup), generator=gen, device=dev)
    src = torch.gather(src_pool, 1, pick)
    hh = torch.arange(H, device=dev)[:, None].expand(H, n_dup)
    rows = K[hh, src].clone()                 # [H][n_dup][d]
    col = torch.randint(0, d, (H, n_dup), generator=gen, device=dev)
    sign = torch.where(torch.rand((H, n_dup), generator=gen, device=dev) < 0.5, 1, -1).to(torch.int32)
    ii = torch.arange(n_dup, device=dev)[None, :].expand(H, n_dup)
    el = rows[hh, ii, col]
    rows[hh, ii, col] = _nudge_bf16_ulp(el, sign)
    K[hh, tgt] = rows
    return K


def query_samples(n_heads: int, head_dim: int, n_samples: int, seed: int = 0, dtype: str = "bf16",
                  device="cpu", r_range=(0.3, 0.99), constant_norm: bool = False):
    """Pre-RoPE query samples for the calibration statistics.

    Returns (q [n_samples][n_heads][head_dim] in ``dtype`` on ``device``,
    R_true [n_heads][d/2] fp64, centres [n_heads][d] fp64).  Band f of head h
    has phase arg(c_f) + N(0, sigma^2) with sigma^2 = -2 ln R_true[h, f], so
    that E[e^{i phase}] has modulus R_true (wrapped-normal law), and
    magnitude |c_f| (``constant_norm``) or |c_f| * e^{0.2 N(0, 1)}.  Centres
    are N(0, I_d) scaled to norm 4 as for the caches; R_true ~ U(r_range).
    Phases and magnitudes are drawn with torch on ``device`` in fp32.
    """
    h = head_dim // 2
    rng = _np_rng(seed, "query-samples", n_heads, head_dim)
    centres = np.stack([_unit_norm_scaled(rng, head_dim, 4.0) for _ in range(n_heads)])
    R_true = rng.uniform(r_range[0], r_range[1], size=(n_heads, h))
    zc = centres[:, :h] + 1j * centres[:, h:]
    sigma = torch.tensor(np.sqrt(-2.0 * np.log(R_true)), dtype=torch.float32, device=device)
    mu = torch.tensor(np.angle(zc), dtype=torch.float32, device=device)
    mag = torch.tensor(np.abs(zc), dtype=torch.float32, device=device)
    gen = _torch_gen(device, seed, "query-samples", n_heads, head_dim, n_samples)
    theta = mu + sigma * torch.randn((n_samples, n_heads, h), generator=gen, device=device)
    r = mag if constant_norm else mag * torch.exp(0.2 * torch.randn((n_samples, n_heads, h),
                                                                    generator=gen, device=device))
    q = torch.cat([r * torch.cos(theta), r * torch.sin(theta)], dim=-1)
    return q.to(_torch_dtype(dtype)).contiguous(), R_true, centres


def make_cache(spec: Spec, device="cpu", seed: int = 0,
               positions: Optional[Sequence[np.ndarray]] = None,
               p_now: Optional[Sequence[int]] = None,
               caps: Optional[Sequence[int]] = None) -> Cache:
    """Materialises the caches of ``spec`` on ``device``.

    positions: optional per-sequence ascending int positions (defaults to
    0..len-1, i.e. a cache that has never been pruned); p_now defaults to the
    newest position.  caps: optional per-sequence capacity >= length (rows past
    the length are filled with noise).
    """
    device = torch.device(device)
    kc, conc, calib = _model(spec, seed)
    L, H, d = spec.n_layers, spec.n_kv_heads, spec.head_dim
    dt = _torch_dtype(spec.dtype)
    ks, vs, ps, lens, nows = [], [], [], [], []
    for s, n in enumerate(spec.lengths):
        cap = int(caps[s]) if caps is not None else int(n)
        assert cap >= n
        if positions is not None:
            p = np.asarray(positions[s], dtype=np.int64)
            assert p.shape == (n,) and (n < 2 or np.all(np.diff(p) > 0))
        else:
            p = np.arange(n, dtype=np.int64)
        pn = int(p_now[s]) if p_now is not None else (int(p[-1]) if n else 0)
        pt = torch.from_numpy(p).to(device)
        cos, sin = _rope_tables(d, spec.rope_theta, pt, device)
        K = torch.empty((L, H, cap, d), dtype=dt, device=device)
        V = torch.empty((L, H, cap, d), dtype=dt, device=device)
        P = torch.empty((L, H, cap), dtype=torch.int32, device=device)
        for l in range(L):
            gen = _torch_gen(device, seed, spec.name, "keys", s, l)
            centre = torch.from_numpy(kc[l]).to(device=device, dtype=torch.float32)
            if spec.recipe == "toy":
                k_pre = _draw_concentrated(gen, centre, n, 0.3, 0.0, device)
            elif spec.recipe in ("concentrated", "neartie"):
                sigma = 0.25 * 4.0 / math.sqrt(d)
                k_pre = _draw_concentrated(gen, centre, n, sigma, spec.outlier_frac, device)
            elif spec.recipe == "phase":
                ch = torch.from_numpy(conc[l]).to(device=device, dtype=torch.float32)
                k_pre = _draw_phase(gen, centre, ch, n, device)
            else:
                raise KeyError(spec.recipe)
            Kl = _store_post_rope(k_pre, cos, sin).to(dt)
            del k_pre
            if spec.dup_frac > 0:
                assert dt == torch.bfloat16
                Kl = _near_ties(gen, Kl, spec.dup_frac)
            K[l, :, :n] = Kl
            del Kl
            if cap > n:
                K[l, :, n:] = torch.randn((H, cap - n, d), generator=gen, device=device).to(dt)
            V[l] = torch.randn((H, cap, d), generator=gen, device=device, dtype=torch.float32).to(dt)
            P[l, :, :n] = pt.to(torch.int32)[None, :]
            if cap > n:
                P[l, :, n:] = -1
        ks.append(K)
        vs.append(V)
        ps.append(P)
        lens.append(int(n))
        nows.append(pn)
    return Cache(spec, ks, vs, ps, lens, nows, calib, seed)


def pruned_positions(seed: int, n: int, start: int = 0, max_gap: int = 7) -> np.ndarray:
    """Strictly ascending positions with random gaps, as left by earlier prunes."""
    rng = _np_rng(seed, "pruned-positions", n, start)
    return start + np.cumsum(rng.integers(1, max_gap + 1, size=n)) - 1


def head_lengths(kind: str, n_layers: int, n_kv_heads: int, n: int, seed: int = 0) -> np.ndarray:
    """Per-head lengths int32 [n_layers][n_kv_heads], each in [0, n], of a
    ragged cache (the state head-specific budgets leave behind).

    kinds: ``full`` (every head n), ``ragged`` (U{n/2..n}), ``extreme``
    (each head one of 0, 1, U{1..64}, n, U{0..n}, equally likely).
    """
    rng = _np_rng(seed, "head-lengths", kind, n_layers, n_kv_heads, n)
    shape = (n_layers, n_kv_heads)
    if kind == "full":
        out = np.full(shape, n)
    elif kind == "ragged":
        out = rng.integers(n // 2, n + 1, size=shape)
    elif kind == "extreme":
        pick = rng.integers(0, 5, size=shape)
        choices = np.stack([np.zeros(shape, dtype=np.int64), np.ones(shape, dtype=np.int64),
                            rng.integers(1, 65, size=shape), np.full(shape, n),
                            rng.integers(0, n + 1, size=shape)])
        out = np.minimum(np.take_along_axis(choices, pick[None], 0)[0], n)
    else:
        raise KeyError(kind)
    return np.ascontiguousarray(out, dtype=np.int32)


# --------------------------------------------------------------------------
# inputs for the select-only and compact-only checks


def make_scores(kind: str, n_heads: int, n: int, seed: int = 0) -> np.ndarray:
    """fp32 score arrays [n_heads][n] with adversarial structure.

    kinds: ``normal`` (i.i.d. N(0,1)), ``ties`` (values from a 7-element set),
    ``allequal``, ``special`` (NaN, +/-inf, +/-0 and denormals mixed in),
    ``dups`` (normal with 30% exact duplicates of other slots),
    ``straddle`` (concentrated around 2.0), ``outlier`` (normal plus one
    +1e30 and one -1e30), ``narrow`` (all within a few ulps of 1.0),
    ``ulp`` (clusters of values one fp32 ulp apart), ``wide`` (positive
    values spread over the exponents from 2e-9 to 3e38, with +inf mixed in: the
    order-preserving keys span more than a quarter of the uint32 range, all in
    its top half), ``runs_high`` (normal, except 32 evenly spaced runs of 128
    consecutive slots, run c starting at slot c * (n - 128) / 31, which hold
    the largest values: high scores clustered in runs), ``cluster`` (40% of
    the keys within 1000 ulps of 3.0, the rest normal: the budget's threshold
    falls inside a dense cluster of distinct values).
    """
    rng = _np_rng(seed, "scores", kind, n_heads, n)
    if kind == "normal":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
    elif kind == "ties":
        s = rng.choice(np.array([-2, -1, 0, 0.5, 1, 3, 7], dtype=np.float32), size=(n_heads, n))
    elif kind == "allequal":
        s = np.full((n_heads, n), 1.25, dtype=np.float32)
    elif kind == "special":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
        specials = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -1e-40, 3.0e38],
                            dtype=np.float32)
        m = rng.random((n_heads, n)) < 0.2
        s[m] = rng.choice(specials, size=int(m.sum()))
    elif kind == "dups":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
        for h in range(n_heads):
            tgt = rng.random(n) < 0.3
            src = rng.integers(0, n, size=int(tgt.sum()))
            s[h, tgt] = s[h, src]
    elif kind == "straddle":
        # concentrated around 2.0: keys differ in the exponent bits
        s = (2.0 + 0.05 * rng.standard_normal((n_heads, n))).astype(np.float32)
    elif kind == "outlier":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
        s[:, int(rng.integers(0, n))] = 1e30
        s[:, int(rng.integers(0, n))] = -1e30
    elif kind == "narrow":
        # every score within a few ulps of 1.0
        base = np.full((n_heads, n), 1.0, dtype=np.float32)
        steps = rng.integers(0, 6, size=(n_heads, n)).astype(np.int32)
        s = (base.view(np.int32) + steps).view(np.float32)
    elif kind == "ulp":
        base = rng.standard_normal((n_heads, max(n // 16, 1))).astype(np.float32)
        idx = rng.integers(0, base.shape[1], size=(n_heads, n))
        s = np.take_along_axis(base, idx, axis=1)
        steps = rng.integers(-2, 3, size=(n_heads, n)).astype(np.int32)
        s = (s.view(np.int32) + steps).view(np.float32)
    elif kind == "wide":
        s = np.exp(rng.uniform(-20.0, 88.0, size=(n_heads, n))).astype(np.float32)
        s[rng.random((n_heads, n)) < 0.01] = np.inf
    elif kind == "runs_high":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
        for c in range(32):
            a = c * (n - 128) // 31
            s[:, a:a + 128] = (10.0 + rng.standard_normal((n_heads, 128))).astype(np.float32)
    elif kind == "cluster":
        s = rng.standard_normal((n_heads, n)).astype(np.float32)
        m = rng.random((n_heads, n)) < 0.4
        steps = rng.integers(0, 1000, size=int(m.sum())).astype(np.int32)
        s[m] = (np.full(int(m.sum()), 3.0, dtype=np.float32).view(np.int32) + steps).view(np.float32)
    else:
        raise KeyError(kind)
    return np.ascontiguousarray(s, dtype=np.float32)


def make_kept(kind: str, n_heads: int, n: int, budget: int, seed: int = 0) -> np.ndarray:
    """Ascending kept-slot lists [n_heads][budget] that stress in-place
    compaction: ``random``, ``all_but_first`` (drop slot 0), ``every8``,
    ``last`` (the last budget slots), ``prefix`` (identity), ``blocks``
    (alternating runs of kept and evicted rows)."""
    assert budget <= n
    rng = _np_rng(seed, "kept", kind, n_heads, n, budget)
    out = np.empty((n_heads, budget), dtype=np.int32)
    for h in range(n_heads):
        if kind == "random":
            out[h] = np.sort(rng.choice(n, size=budget, replace=False))
        elif kind == "all_but_first":
            out[h] = np.arange(1, budget + 1)
        elif kind == "every8":
            sel = np.arange(0, n, 8)[:budget]
            if len(sel) < budget:
                rest = np.setdiff1d(np.arange(n), sel)[:budget - len(sel)]
                sel = np.sort(np.concatenate([sel, rest]))
            out[h] = sel
        elif kind == "last":
            out[h] = np.arange(n - budget, n)
        elif kind == "prefix":
            out[h] = np.arange(budget)
        elif kind == "blocks":
            runs = []
            i, keep = 0, True
            while i < n:
                ln = int(rng.integers(1, 64))
                if keep:
                    runs.extend(range(i, min(n, i + ln)))
                i += ln
                keep = not keep
            sel = np.array(runs[:budget])
            if len(sel) < budget:
                rest = np.setdiff1d(np.arange(n), sel)[:budget - len(sel)]
                sel = np.sort(np.concatenate([sel, rest]))
            out[h] = sel
        else:
            raise KeyError(kind)
    return out
