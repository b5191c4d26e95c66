"""Python binding of libtri, the C-ABI library of the TriAttention online
KV-eviction pass for MI355X (gfx950).

Argument marshalling only: every step of the pass runs in the HIP kernels of
``libtri.so``; PyTorch supplies device memory and streams.  The function
names and semantics are those of ``include/tri.h``:

    ctx = tri_calibrate_load(n_layers, n_kv_heads, head_dim, qc_re, qc_im,
                             q_mean_norm, q_mrl, offsets, rope_theta=...)
    tri_score(ctx, seqs, scores)                         # fp32 per cached key
    tri_score(ctx, seqs, scores, workspace=ws)           # GQA contexts (n_q_heads > n_kv_heads)
    tri_select_topb(ctx, seqs, scores, budget, window, kept)
    tri_compact_kv(ctx, seqs, kept, budget, window)      # in place; updates seq.len

There is no CPU fallback: importing works without a GPU, but every call
needs the built library and a GPU, and raises otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libtri.so")

TRI_OK, TRI_E_INVAL, TRI_E_UNSUPPORTED, TRI_E_HIP, TRI_E_NOMEM, TRI_E_SCRATCH = 0, 1, 2, 3, 4, 5
TRI_F32, TRI_BF16 = 0, 1

EXPORTED = ("tri_calibrate_load", "tri_ctx_destroy", "tri_status_str", "tri_last_hip_error",
            "tri_scores_count", "tri_score", "tri_score_workspace_bytes", "tri_score_ws",
            "tri_select_topb", "tri_select_topb_ws", "tri_compact_kv", "tri_calibrate_stats",
            "tri_distance_curve",
            "tri_offset_set", "tri_select_shared_workspace_bytes", "tri_select_shared",
            "tri_compact_kv_counts", "tri_compact_kv_counts_workspace_bytes",
            "tri_compact_kv_counts_noalloc")


class TriError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        msg = "%s failed: %s (status %d)" % (what, _status_str(status), status)
        if status == TRI_E_HIP:
            msg += ", hipError %d" % hip_error
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


class _CalibDesc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("inv_freq", ctypes.POINTER(ctypes.c_double)),
        ("offsets", ctypes.POINTER(ctypes.c_int64)), ("n_offsets", ctypes.c_int32),
        ("qc_re", ctypes.POINTER(ctypes.c_double)), ("qc_im", ctypes.POINTER(ctypes.c_double)),
        ("q_mean_norm", ctypes.POINTER(ctypes.c_double)), ("q_mrl", ctypes.POINTER(ctypes.c_double)),
        ("n_q_heads", ctypes.c_int32),
    ]


class _Seq(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("cap", ctypes.c_int32), ("len", ctypes.c_int32), ("p_now", ctypes.c_int64),
                ("head_len", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libtri.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError("libtri.so is not built (%s); run __graft_entry__.build() or "
                              "python -m rope_aware_eviction_amd.build_lib" % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        vp = ctypes.c_void_p
        lib.tri_calibrate_load.restype = ctypes.c_int
        lib.tri_calibrate_load.argtypes = [ctypes.POINTER(_CalibDesc), ctypes.c_int, ctypes.POINTER(vp)]
        lib.tri_ctx_destroy.restype = None
        lib.tri_ctx_destroy.argtypes = [vp]
        lib.tri_status_str.restype = ctypes.c_char_p
        lib.tri_status_str.argtypes = [ctypes.c_int]
        lib.tri_last_hip_error.restype = ctypes.c_int
        lib.tri_last_hip_error.argtypes = []
        lib.tri_scores_count.restype = ctypes.c_int64
        lib.tri_scores_count.argtypes = [vp, ctypes.POINTER(_Seq), ctypes.c_int32]
        lib.tri_score.restype = ctypes.c_int
        lib.tri_score.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Seq), ctypes.c_int32, vp, vp]
        lib.tri_score_workspace_bytes.restype = ctypes.c_int64
        lib.tri_score_workspace_bytes.argtypes = [vp, ctypes.POINTER(_Seq), ctypes.c_int32]
        lib.tri_score_ws.restype = ctypes.c_int
        lib.tri_score_ws.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Seq), ctypes.c_int32, vp, vp,
                                     ctypes.c_int64, vp]
        lib.tri_calibrate_stats.restype = ctypes.c_int
        lib.tri_calibrate_stats.argtypes = [ctypes.c_int, vp, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, vp, vp, vp, vp, vp]
        lib.tri_distance_curve.restype = ctypes.c_int
        lib.tri_distance_curve.argtypes = [vp, vp, vp, vp, ctypes.c_int32, vp, vp]
        lib.tri_offset_set.restype = ctypes.c_int32
        lib.tri_offset_set.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]
        lib.tri_select_topb.restype = ctypes.c_int
        lib.tri_select_topb.argtypes = [vp, ctypes.POINTER(_Seq), ctypes.c_int32, vp,
                                        ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.tri_select_topb_ws.restype = ctypes.c_int
        lib.tri_select_topb_ws.argtypes = [vp, ctypes.POINTER(_Seq), ctypes.c_int32, vp, vp,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.tri_compact_kv.restype = ctypes.c_int
        lib.tri_compact_kv.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Seq), ctypes.c_int32, vp,
                                       ctypes.c_int32, ctypes.c_int32, vp]
        lib.tri_select_shared_workspace_bytes.restype = ctypes.c_int64
        lib.tri_select_shared_workspace_bytes.argtypes = [vp, ctypes.c_int32]
        lib.tri_select_shared.restype = ctypes.c_int
        lib.tri_select_shared.argtypes = [vp, ctypes.POINTER(_Seq), ctypes.c_int32, vp,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                          vp, ctypes.c_int64, vp]
        lib.tri_compact_kv_counts.restype = ctypes.c_int
        lib.tri_compact_kv_counts.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Seq),
                                              ctypes.c_int32, vp, ctypes.c_int32, vp, vp,
                                              ctypes.c_int64, vp]
        lib.tri_compact_kv_counts_noalloc.restype = ctypes.c_int
        lib.tri_compact_kv_counts_noalloc.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Seq),
                                                      ctypes.c_int32, vp, ctypes.c_int32, vp, vp]
        lib.tri_compact_kv_counts_workspace_bytes.restype = ctypes.c_int64
        lib.tri_compact_kv_counts_workspace_bytes.argtypes = [vp]
        _lib = lib
    return _lib


def _status_str(status: int) -> str:
    try:
        return library().tri_status_str(status).decode()
    except ImportError:
        return "status %d" % status


def _check(status: int, what: str):
    if status != TRI_OK:
        raise TriError(status, what, library().tri_last_hip_error())


class Context:
    """A loaded calibration table (owns the device tables of one tri_ctx)."""

    def __init__(self, handle: int, n_layers: int, n_kv_heads: int, head_dim: int, device: int,
                 group: int = 1):
        self.handle = handle
        self.n_layers = n_layers
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.device = device
        self.group = group          # query heads per KV head

    @property
    def n_heads(self) -> int:
        return self.n_layers * self.n_kv_heads

    def close(self):
        if self.handle:
            library().tri_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Seq:
    """One sequence's cache: K, V [n_layers][n_kv_heads][cap][head_dim] (float32
    or bfloat16), positions int32 [n_layers][n_kv_heads][cap], the length in
    use and the newest position.  ``len`` is updated by tri_compact_kv.
    ``head_len`` (optional int32 GPU tensor [n_layers][n_kv_heads]) gives
    every head its own length up to ``len`` (a ragged cache); the shared-budget
    compaction writes it."""

    def __init__(self, k: torch.Tensor, v: Optional[torch.Tensor], pos: Optional[torch.Tensor],
                 len: int, p_now: int, head_len: Optional[torch.Tensor] = None):
        self.k, self.v, self.pos = k, v, pos
        self.len = int(len)
        self.p_now = int(p_now)
        self.head_len = head_len

    @property
    def cap(self) -> int:
        return int(self.k.shape[2])


def _f64_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def tri_calibrate_load(n_layers: int, n_kv_heads: int, head_dim: int, qc_re, qc_im, q_mean_norm,
                       q_mrl, offsets, rope_theta: float = 10000.0, inv_freq=None,
                       device: Optional[int] = None, n_q_heads: Optional[int] = None) -> Context:
    """Loads a calibration table (host arrays [n_layers][n_q_heads][head_dim/2];
    n_q_heads defaults to n_kv_heads, a multiple of it is a GQA grouping)."""
    lib = library()
    if device is None:
        device = torch.cuda.current_device()
    n_q = n_kv_heads if n_q_heads is None else int(n_q_heads)
    arrs = [np.ascontiguousarray(x, dtype=np.float64) for x in (qc_re, qc_im, q_mean_norm, q_mrl)]
    shape = (n_layers, n_q, head_dim // 2)
    for a in arrs:
        if a.shape != shape:
            raise ValueError("calibration arrays must have shape %s, got %s" % (shape, a.shape))
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    inv = None if inv_freq is None else np.ascontiguousarray(inv_freq, dtype=np.float64)
    desc = _CalibDesc(
        n_layers, n_kv_heads, head_dim, float(rope_theta),
        _f64_ptr(inv) if inv is not None else None,
        off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(off),
        _f64_ptr(arrs[0]), _f64_ptr(arrs[1]), _f64_ptr(arrs[2]), _f64_ptr(arrs[3]), n_q)
    h = ctypes.c_void_p()
    _check(lib.tri_calibrate_load(ctypes.byref(desc), int(device), ctypes.byref(h)),
           "tri_calibrate_load")
    return Context(h.value, n_layers, n_kv_heads, head_dim, int(device), n_q // n_kv_heads)


def tri_calibrate_stats(q: torch.Tensor, stream=None):
    """Per-band calibration statistics (qc_re, qc_im, q_mean_norm, q_mrl), each
    an fp64 GPU tensor [n_heads][head_dim/2], from pre-RoPE query samples
    ``q`` [n_samples][n_heads][head_dim] (float32 or bfloat16, contiguous, on
    the GPU).  Enqueued on ``stream``; no synchronisation."""
    if not (q.is_cuda and q.is_contiguous() and q.dim() == 3):
        raise ValueError("q must be a contiguous 3-d GPU tensor [n_samples][n_heads][head_dim]")
    n, h, d = q.shape
    outs = [torch.empty((h, d // 2), dtype=torch.float64, device=q.device) for _ in range(4)]
    _check(library().tri_calibrate_stats(_dtype_code(q), q.data_ptr(), int(n), int(h), int(d),
                                         *(o.data_ptr() for o in outs), _stream_ptr(stream)),
           "tri_calibrate_stats")
    return tuple(outs)


def tri_distance_curve(ctx: Context, kc_re: torch.Tensor, kc_im: torch.Tensor,
                       deltas: torch.Tensor, stream=None) -> torch.Tensor:
    """Distance-preference curves [n_layers*n_q_heads][n_delta] (fp64 GPU tensor)
    from the context's query centres and key centres kc_re/kc_im (fp64 GPU
    [n_layers*n_kv_heads][head_dim/2]) at distances ``deltas`` (int64 GPU)."""
    h = ctx.n_heads
    for t in (kc_re, kc_im):
        if t.dtype != torch.float64 or not t.is_cuda or not t.is_contiguous() \
                or tuple(t.shape) != (h, ctx.head_dim // 2):
            raise ValueError("key centres must be contiguous fp64 GPU tensors [%d][%d]"
                             % (h, ctx.head_dim // 2))
    if deltas.dtype != torch.int64 or not deltas.is_cuda or not deltas.is_contiguous():
        raise ValueError("deltas must be a contiguous int64 GPU tensor")
    out = torch.empty((h * ctx.group, deltas.numel()), dtype=torch.float64, device=kc_re.device)
    _check(library().tri_distance_curve(ctx.handle, kc_re.data_ptr(), kc_im.data_ptr(),
                                        deltas.data_ptr(), int(deltas.numel()), out.data_ptr(),
                                        _stream_ptr(stream)), "tri_distance_curve")
    return out


def offset_set(kind: str, max_distance: int, count: int = 0) -> np.ndarray:
    """Future-offset set: 'geometric' (1, 2, 4, ... up to max_distance) or
    'linear' (count evenly spaced offsets ending at max_distance)."""
    k = {"geometric": 0, "linear": 1}[kind]
    n = library().tri_offset_set(k, int(max_distance), int(count), None, 0)
    if n < 0:
        raise ValueError("bad offset-set arguments")
    out = np.empty(n, dtype=np.int64)
    library().tri_offset_set(k, int(max_distance), int(count),
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n)
    return out


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TRI_F32
    if t.dtype == torch.bfloat16:
        return TRI_BF16
    raise TypeError("cache dtype must be float32 or bfloat16, got %s" % t.dtype)


def _seq_array(ctx: Context, seqs: Sequence[Seq], need_kv: bool):
    arr = (_Seq * max(1, len(seqs)))()
    dtype = None
    for i, s in enumerate(seqs):
        k = s.k
        if not (k.is_cuda and k.is_contiguous() and k.dim() == 4):
            raise ValueError("seq %d: k must be a contiguous 4-d GPU tensor" % i)
        if tuple(k.shape[:2]) != (ctx.n_layers, ctx.n_kv_heads) or k.shape[3] != ctx.head_dim:
            raise ValueError("seq %d: k shape %s does not match the context" % (i, tuple(k.shape)))
        code = _dtype_code(k)
        if dtype is not None and code != dtype:
            raise TypeError("all sequences must share one cache dtype")
        dtype = code
        if need_kv:
            if s.v is None or s.v.shape != k.shape or s.v.dtype != k.dtype or not s.v.is_contiguous():
                raise ValueError("seq %d: v must match k" % i)
            if s.pos is None or s.pos.dtype != torch.int32 or tuple(s.pos.shape) != tuple(k.shape[:3]) \
                    or not s.pos.is_contiguous():
                raise ValueError("seq %d: pos must be int32 [n_layers][n_kv_heads][cap]" % i)
        hl = getattr(s, "head_len", None)
        if hl is not None and not (hl.is_cuda and hl.dtype == torch.int32 and hl.is_contiguous()
                                   and tuple(hl.shape) == (ctx.n_layers, ctx.n_kv_heads)):
            raise ValueError("seq %d: head_len must be a contiguous int32 GPU tensor "
                             "[n_layers][n_kv_heads]" % i)
        arr[i] = _Seq(k.data_ptr(), s.v.data_ptr() if s.v is not None else None,
                      s.pos.data_ptr() if s.pos is not None else None,
                      int(k.shape[2]), int(s.len), int(s.p_now),
                      hl.data_ptr() if hl is not None else None)
    return arr, (TRI_BF16 if dtype is None else dtype)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def scores_count(ctx: Context, seqs: Sequence[Seq]) -> int:
    return sum(ctx.n_heads * s.len for s in seqs)


def score_workspace_bytes(ctx: Context, seqs: Sequence[Seq]) -> int:
    """Device workspace bytes tri_score needs (0 unless the context is GQA)."""
    arr, _ = _seq_array(ctx, seqs, need_kv=False)
    n = library().tri_score_workspace_bytes(ctx.handle, arr, len(seqs))
    if n < 0:
        raise ValueError("bad sequences for tri_score_workspace_bytes")
    return int(n)


def tri_score(ctx: Context, seqs: Sequence[Seq], scores: torch.Tensor, stream=None,
              workspace: Optional[torch.Tensor] = None):
    """Scores every cached key of every head; ``scores`` fp32 on the GPU with
    at least scores_count(ctx, seqs) elements, sequence-major [L][H][len].
    GQA contexts also need ``workspace``: a contiguous GPU tensor of at least
    score_workspace_bytes(ctx, seqs) bytes (tri_score_ws)."""
    arr, dtype = _seq_array(ctx, seqs, need_kv=False)
    if scores is None:
        # GQA contexts: raw per-query-head scores and their per-tile partial
        # sums only, into the workspace (for tri_select_topb_ws)
        if workspace is None:
            raise ValueError("scores=None needs the GQA workspace")
    elif scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous() \
            or scores.numel() < scores_count(ctx, seqs):
        raise ValueError("scores must be a contiguous fp32 GPU tensor of %d elements"
                         % scores_count(ctx, seqs))
    if workspace is None:
        _check(library().tri_score(ctx.handle, dtype, arr, len(seqs), scores.data_ptr(),
                                   _stream_ptr(stream)), "tri_score")
        return
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(library().tri_score_ws(ctx.handle, dtype, arr, len(seqs),
                                  None if scores is None else scores.data_ptr(),
                                  workspace.data_ptr(), nbytes, _stream_ptr(stream)),
           "tri_score_ws")


def tri_select_topb_ws(ctx: Context, seqs: Sequence[Seq], workspace: torch.Tensor, budget: int,
                       window: int, kept: torch.Tensor, stream=None,
                       scores: Optional[torch.Tensor] = None):
    """GQA contexts: top-``budget`` kept slots per head ranked by the GQA score
    formed on the fly from the raw scores and per-tile partial sums a
    tri_score(..., scores=None, workspace=workspace) call left in
    ``workspace``.  ``scores`` (fp32, the layout of tri_score) is needed only
    when a firing sequence has more than 32768 keys per head."""
    arr, _ = _seq_array(ctx, seqs, need_kv=False)
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * budget:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*budget")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_cuda
                               or not scores.is_contiguous()
                               or scores.numel() < scores_count(ctx, seqs)):
        raise ValueError("scores must be a contiguous fp32 GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(library().tri_select_topb_ws(ctx.handle, arr, len(seqs),
                                        None if scores is None else scores.data_ptr(),
                                        workspace.data_ptr(), nbytes, int(budget), int(window),
                                        kept.data_ptr(), _stream_ptr(stream)),
           "tri_select_topb_ws")


def tri_select_topb(ctx: Context, seqs: Sequence[Seq], scores: torch.Tensor, budget: int,
                    window: int, kept: torch.Tensor, stream=None):
    """Top-``budget`` kept slots per head (ascending) into ``kept`` int32
    [n_seq][n_layers][n_kv_heads][budget] for every sequence that fires."""
    arr, _ = _seq_array(ctx, seqs, need_kv=False)
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * budget:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*budget")
    if scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous() \
            or scores.numel() < scores_count(ctx, seqs):
        raise ValueError("scores must be a contiguous fp32 GPU tensor")
    _check(library().tri_select_topb(ctx.handle, arr, len(seqs), scores.data_ptr(), int(budget),
                                     int(window), kept.data_ptr(), _stream_ptr(stream)),
           "tri_select_topb")


def tri_compact_kv(ctx: Context, seqs: Sequence[Seq], kept: torch.Tensor, budget: int,
                   window: int, stream=None):
    """Compacts K, V and positions of every firing sequence in place and sets
    its ``len`` to ``budget``."""
    arr, dtype = _seq_array(ctx, seqs, need_kv=True)
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * budget:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*budget")
    _check(library().tri_compact_kv(ctx.handle, dtype, arr, len(seqs), kept.data_ptr(),
                                    int(budget), int(window), _stream_ptr(stream)),
           "tri_compact_kv")
    for i, s in enumerate(seqs):
        s.len = int(arr[i].len)


def prune_step_gqa(ctx: Context, seqs: List[Seq], budget: int, window: int, kept: torch.Tensor,
                   workspace: torch.Tensor, stream=None, scores: Optional[torch.Tensor] = None):
    """One GQA prune step without the normalized score array (score into the
    workspace, select from it, compact) on one stream, no host sync."""
    tri_score(ctx, seqs, None, stream, workspace)
    tri_select_topb_ws(ctx, seqs, workspace, budget, window, kept, stream, scores)
    tri_compact_kv(ctx, seqs, kept, budget, window, stream)


def fires(seq: Seq, budget: int, window: int) -> bool:
    """The pruning trigger: a head is pruned iff its length exceeds budget + window."""
    return seq.len > budget + window


def prune_step(ctx: Context, seqs: List[Seq], budget: int, window: int, scores: torch.Tensor,
               kept: torch.Tensor, stream=None, workspace: Optional[torch.Tensor] = None):
    """One prune step (score, select, compact) on one stream, no host sync."""
    tri_score(ctx, seqs, scores, stream, workspace)
    tri_select_topb(ctx, seqs, scores, budget, window, kept, stream)
    tri_compact_kv(ctx, seqs, kept, budget, window, stream)


def select_shared_workspace_bytes(ctx: Context, n_seq: int) -> int:
    """Device workspace bytes tri_select_shared needs for n_seq sequences."""
    n = library().tri_select_shared_workspace_bytes(ctx.handle, int(n_seq))
    if n < 0:
        raise ValueError("bad arguments for tri_select_shared_workspace_bytes")
    return int(n)


def tri_select_shared(ctx: Context, seqs: Sequence[Seq], scores: torch.Tensor, budget: int,
                      floor: int, window: int, kept: torch.Tensor, kept_count: torch.Tensor,
                      workspace: torch.Tensor, stream=None):
    """Head-specific budgets: the heads of a layer share budget * n_kv_heads
    slots, each keeping at least its ``floor`` best keys.  Writes kept slots
    into ``kept`` int32 [n_seq][n_layers][n_kv_heads][budget * n_kv_heads] and
    per-head counts (-1: the layer does not fire) into ``kept_count`` int32
    [n_seq][n_layers][n_kv_heads]."""
    arr, _ = _seq_array(ctx, seqs, need_kv=False)
    total = int(budget) * ctx.n_kv_heads
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * total:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*total")
    if kept_count.dtype != torch.int32 or not kept_count.is_cuda \
            or not kept_count.is_contiguous() or kept_count.numel() < len(seqs) * ctx.n_heads:
        raise ValueError("kept_count must be a contiguous int32 GPU tensor of n_seq*n_heads")
    if scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous() \
            or scores.numel() < scores_count(ctx, seqs):
        raise ValueError("scores must be a contiguous fp32 GPU tensor")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(library().tri_select_shared(ctx.handle, arr, len(seqs), scores.data_ptr(), int(budget),
                                       int(floor), int(window), kept.data_ptr(),
                                       kept_count.data_ptr(), workspace.data_ptr(), nbytes,
                                       _stream_ptr(stream)), "tri_select_shared")


def compact_counts_workspace_bytes(ctx: Context) -> int:
    """Device workspace bytes tri_compact_kv_counts needs."""
    n = library().tri_compact_kv_counts_workspace_bytes(ctx.handle)
    if n < 0:
        raise ValueError("bad context")
    return int(n)


def tri_compact_kv_counts(ctx: Context, seqs: Sequence[Seq], kept: torch.Tensor,
                          kept_stride: int, kept_count: torch.Tensor,
                          workspace: torch.Tensor, stream=None):
    """Compacts every head with a kept count >= 0 in place and writes the count
    into the sequence's ``head_len`` (which every sequence needs).
    ``workspace``: a contiguous GPU tensor of compact_counts_workspace_bytes."""
    arr, dtype = _seq_array(ctx, seqs, need_kv=True)
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * kept_stride:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*kept_stride")
    if kept_count.dtype != torch.int32 or not kept_count.is_cuda \
            or not kept_count.is_contiguous() or kept_count.numel() < len(seqs) * ctx.n_heads:
        raise ValueError("kept_count must be a contiguous int32 GPU tensor of n_seq*n_heads")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(library().tri_compact_kv_counts(ctx.handle, dtype, arr, len(seqs), kept.data_ptr(),
                                           int(kept_stride), kept_count.data_ptr(),
                                           workspace.data_ptr(), nbytes, _stream_ptr(stream)),
           "tri_compact_kv_counts")


def tri_compact_kv_counts_noalloc(ctx: Context, seqs: Sequence[Seq], kept: torch.Tensor,
                                  kept_stride: int, kept_count: torch.Tensor, stream=None):
    """tri_compact_kv_counts with the library's static scratch instead of a
    caller workspace (no device allocation; calls on one GPU must not overlap)."""
    arr, dtype = _seq_array(ctx, seqs, need_kv=True)
    if kept.dtype != torch.int32 or not kept.is_cuda or not kept.is_contiguous() \
            or kept.numel() < len(seqs) * ctx.n_heads * kept_stride:
        raise ValueError("kept must be a contiguous int32 GPU tensor of n_seq*n_heads*kept_stride")
    if kept_count.dtype != torch.int32 or not kept_count.is_cuda \
            or not kept_count.is_contiguous() or kept_count.numel() < len(seqs) * ctx.n_heads:
        raise ValueError("kept_count must be a contiguous int32 GPU tensor of n_seq*n_heads")
    _check(library().tri_compact_kv_counts_noalloc(ctx.handle, dtype, arr, len(seqs), kept.data_ptr(),
                                                   int(kept_stride), kept_count.data_ptr(),
                                                   _stream_ptr(stream)),
           "tri_compact_kv_counts_noalloc")


def prune_step_shared(ctx: Context, seqs: List[Seq], budget: int, floor: int, window: int,
                      scores: torch.Tensor, kept: torch.Tensor, kept_count: torch.Tensor,
                      select_workspace: torch.Tensor, compact_workspace: torch.Tensor,
                      stream=None, workspace: Optional[torch.Tensor] = None):
    """One prune step with head-specific budgets (score, shared select,
    compaction with per-head counts) on one stream, no host sync.  Every
    sequence needs ``head_len``."""
    tri_score(ctx, seqs, scores, stream, workspace)
    tri_select_shared(ctx, seqs, scores, budget, floor, window, kept, kept_count,
                      select_workspace, stream)
    tri_compact_kv_counts(ctx, seqs, kept, int(budget) * ctx.n_kv_heads, kept_count,
                          compact_workspace, stream)


from rope_aware_eviction_amd.calib_file import load_calibration, save_calibration  # noqa: E402,F401 (host-side file I/O)
