"""The C-ABI library without a GPU: it loads, exports every function that
include/tri.h declares, and rejects bad arguments on the host before any HIP
call.  No kernel is launched here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import rope_aware_eviction_amd as tri

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tri.LIBRARY):
        pytest.fail("libtri.so is not built; run __graft_entry__.build()")
    return tri.library()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("tri_calibrate_load", "tri_score", "tri_select_topb", "tri_compact_kv"):
        assert n in names
    assert set(names) == set(tri.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", tri.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tri_[a-z_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["nm", "-D", tri.LIBRARY], capture_output=True, text=True).stdout
    assert "tri_oracle" not in out
    ldd = subprocess.run(["ldd", tri.LIBRARY], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


def test_status_strings(lib):
    assert lib.tri_status_str(0) == b"ok"
    assert lib.tri_status_str(1) == b"invalid argument"
    assert lib.tri_status_str(2).startswith(b"unsupported")
    assert lib.tri_status_str(99) == b"unknown status"
    assert lib.tri_last_hip_error() == 0


def _desc(**over):
    h = 32
    arr = {k: np.ones((1, 2, h)) * v for k, v in
           (("qc_re", 0.5), ("qc_im", 0.25), ("q_mean_norm", 1.0), ("q_mrl", 0.5))}
    arr.update({k: v for k, v in over.items() if k in arr})
    off = np.array(over.get("offsets", [1, 2, 4]), dtype=np.int64)
    keep = [arr, off]
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    d = tri._CalibDesc(over.get("n_layers", 1), over.get("n_kv_heads", 2), over.get("head_dim", 64),
                       over.get("rope_theta", 1e4), None,
                       off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(off),
                       p(arr["qc_re"]), p(arr["qc_im"]), p(arr["q_mean_norm"]), p(arr["q_mrl"]),
                       over.get("n_q_heads", 0))
    return d, keep


@pytest.mark.parametrize("over,status", [
    ({"head_dim": 96}, tri.TRI_E_UNSUPPORTED),
    ({"head_dim": 256}, tri.TRI_E_UNSUPPORTED),
    ({"n_layers": 0}, tri.TRI_E_INVAL),
    ({"rope_theta": -1.0}, tri.TRI_E_INVAL),
    ({"rope_theta": float("nan")}, tri.TRI_E_INVAL),
    ({"offsets": []}, tri.TRI_E_INVAL),
    ({"offsets": [1, -2]}, tri.TRI_E_INVAL),
    ({"q_mrl": np.full((1, 2, 32), 1.5)}, tri.TRI_E_INVAL),
    ({"q_mean_norm": np.full((1, 2, 32), -1.0)}, tri.TRI_E_INVAL),
    ({"qc_re": np.full((1, 2, 32), np.inf)}, tri.TRI_E_INVAL),
    ({"n_q_heads": 3}, tri.TRI_E_INVAL),          # not a multiple of the 2 KV heads
    ({"n_q_heads": 1}, tri.TRI_E_INVAL),          # fewer query heads than KV heads
    ({"n_q_heads": -2}, tri.TRI_E_INVAL),
    ({"n_q_heads": 18}, tri.TRI_E_UNSUPPORTED),   # group of 9
])
def test_calibrate_rejects_bad_tables_before_any_hip_call(lib, over, status):
    d, keep = _desc(**over)
    h = ctypes.c_void_p(1234)
    r = lib.tri_calibrate_load(ctypes.byref(d), 0, ctypes.byref(h))
    assert r == status
    assert h.value is None


def test_calls_reject_null_context_and_bad_shapes(lib):
    seq = tri._Seq(None, None, None, 10, 5, 9)
    arr = (tri._Seq * 1)(seq)
    assert lib.tri_score(None, tri.TRI_BF16, arr, 1, None, None) == tri.TRI_E_INVAL
    assert lib.tri_select_topb(None, arr, 1, None, 4, 0, None, None) == tri.TRI_E_INVAL
    assert lib.tri_compact_kv(None, tri.TRI_BF16, arr, 1, None, 4, 0, None) == tri.TRI_E_INVAL
    assert lib.tri_scores_count(None, arr, 1) == -1
    assert lib.tri_score_ws(None, tri.TRI_BF16, arr, 1, None, None, 0, None) == tri.TRI_E_INVAL
    assert lib.tri_score_workspace_bytes(None, arr, 1) == -1
    assert lib.tri_select_shared_workspace_bytes(None, 1) == -1
    assert lib.tri_select_shared(None, arr, 1, None, 4, 1, 0, None, None, None, 0,
                                 None) == tri.TRI_E_INVAL
    assert lib.tri_compact_kv_counts(None, tri.TRI_BF16, arr, 1, None, 4, None, None, 0,
                                     None) == tri.TRI_E_INVAL
    assert lib.tri_compact_kv_counts_workspace_bytes(None) == -1
    lib.tri_ctx_destroy(None)     # allowed


def test_seq_struct_layout_matches_the_header(tmp_path):
    # the binding's ctypes mirror of tri_seq must agree with the C compiler's
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "tri.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu\\n", sizeof(tri_seq), '
                   'offsetof(tri_seq, len), offsetof(tri_seq, p_now), '
                   'offsetof(tri_seq, head_len), sizeof(tri_calib_desc)); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(tri._Seq), tri._Seq.len.offset, tri._Seq.p_now.offset,
            tri._Seq.head_len.offset, ctypes.sizeof(tri._CalibDesc)]
    assert got == want


def test_offset_sets_match_the_oracle(lib, oracle_lib):
    """The library's host helper and the oracle's, written separately from the
    same statement, agree on every set."""
    rng = __import__("numpy").random.default_rng(40)
    for m in [1, 2, 3, 100, 1000, 65536, 131071, 1 << 40]:
        np.testing.assert_array_equal(tri.offset_set("geometric", m), oracle_lib.offset_set("geometric", m))
    for _ in range(200):
        m = int(rng.integers(1, 1 << 20))
        c = int(rng.integers(1, 300))
        np.testing.assert_array_equal(tri.offset_set("linear", m, c), oracle_lib.offset_set("linear", m, c))
    assert lib.tri_offset_set(0, 0, 0, None, 0) == -1
    assert lib.tri_offset_set(1, 10, 0, None, 0) == -1
    assert lib.tri_offset_set(2, 10, 3, None, 0) == -1


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: with libtri.so absent, the first call raises."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "tri_missing", os.path.join(ROOT, "rope_aware_eviction_amd", "__init__.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    m.LIBRARY = str(tmp_path / "libtri.so")
    with pytest.raises(ImportError):
        m.library()
    with pytest.raises(ImportError):
        m.tri_calibrate_load(1, 2, 64, np.zeros((1, 2, 32)), np.zeros((1, 2, 32)),
                             np.ones((1, 2, 32)), np.ones((1, 2, 32)), [1], device=0)
