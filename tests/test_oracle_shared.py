"""Pins of the oracle's head-specific budgets (one shared budget per layer).

Source: romaanj.github.io TriAttention review, section "Future work"
(refined compression strategies including head-specific budgets).  Reading:
the layer's heads share total = budget x heads slots; every head first keeps
its `floor` best keys; the remaining slots go to the best remaining keys of
the layer under one threshold (ties to the lower head, then the lower
position).  Pins: hand examples (tests/golden/shared_budget_examples.json),
the special cases that reduce to the per-head top-B (floor = budget, one
head), and, on random inputs with many ties, the three properties that fix
the kept set uniquely: every head's floor best keys are kept, exactly
`total` keys are kept, and every kept unreserved key outranks every evicted
key in the layer order.  CPU only.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "shared_budget_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("i", range(7))
def test_shared_golden_examples(oracle_lib, i):
    ex = _golden()["examples"][i]
    sc = np.array(ex["scores"], dtype=np.float64)
    pos = np.tile(np.arange(sc.shape[1]), (sc.shape[0], 1))
    got = oracle_lib.select_shared(sc, pos, ex["lens"], ex["total"], ex["floor"], ex["window"])
    if ex["kept"] is None:
        assert got is None
    else:
        assert [list(g) for g in got] == ex["kept"]


def test_floor_equal_to_budget_is_the_per_head_top_b(oracle_lib):
    rng = np.random.default_rng(50)
    H, n, B = 5, 300, 40
    sc = rng.integers(0, 30, (H, n)).astype(np.float64) * rng.uniform(0.5, 3.0, (H, 1))
    pos = np.tile(np.arange(n) * 3 + 7, (H, 1)).astype(np.int64)
    got = oracle_lib.select_shared(sc, pos, [n] * H, H * B, B, 10)
    for h in range(H):
        np.testing.assert_array_equal(got[h], oracle_lib.select_head(sc[h], pos[h], B, 10))


def test_one_head_is_the_plain_top_b(oracle_lib):
    rng = np.random.default_rng(51)
    sc = rng.integers(0, 9, (1, 500)).astype(np.float64)
    pos = np.arange(500)[None, :]
    for floor in (0, 3, 77):
        got = oracle_lib.select_shared(sc, pos, [500], 77, floor, 5)
        np.testing.assert_array_equal(got[0], oracle_lib.select_head(sc[0], pos[0], 77, 5))


def _layer_key(s, h, p):
    # sort key: larger is better; NaN lowest
    return (-np.inf if np.isnan(s) else s, -h, -p)


@pytest.mark.parametrize("seed", range(10))
def test_shared_selection_properties(oracle_lib, seed):
    rng = np.random.default_rng(60 + seed)
    H = int(rng.integers(1, 6))
    stride = int(rng.integers(5, 40))
    lens = rng.integers(0, stride + 1, H)
    sc = rng.integers(0, 6, (H, stride)).astype(np.float64)
    sc[rng.random((H, stride)) < 0.1] = np.nan
    pos = np.tile(np.arange(stride), (H, 1)).astype(np.int64)
    all_keys = int(lens.sum())
    total = int(rng.integers(1, max(2, all_keys)))
    floor = int(rng.integers(0, total // H + 1))
    got = oracle_lib.select_shared(sc, pos, lens, total, floor, 0)
    if all_keys <= total:
        assert got is None
        return
    assert sum(len(g) for g in got) == total
    reserved = set()
    for h in range(H):
        own = sorted(range(lens[h]), key=lambda i: _layer_key(sc[h, i], 0, pos[h, i]), reverse=True)
        reserved |= {(h, i) for i in own[:floor]}
        assert np.all(np.diff(got[h]) > 0) and (len(got[h]) == 0 or got[h][-1] < lens[h])
    kept = {(h, int(i)) for h in range(H) for i in got[h]}
    assert reserved <= kept
    free_kept = kept - reserved
    evicted = {(h, i) for h in range(H) for i in range(lens[h])} - kept
    if free_kept and evicted:
        worst_kept = min(_layer_key(sc[h, i], h, pos[h, i]) for h, i in free_kept)
        best_evicted = max(_layer_key(sc[h, i], h, pos[h, i]) for h, i in evicted)
        assert worst_kept > best_evicted


def test_layer_prune_with_floor_equal_to_budget_is_the_uniform_prune(oracle_lib):
    """prune_layer_shared with floor = budget keeps, per head, exactly what the
    uniform per-head prune keeps (a different code path through the oracle:
    select_head instead of the shared ranking)."""
    import synth
    spec = synth.workload("toy").replace(n_kv_heads=3, lengths=(300,), budget=70, window=0)
    cache = synth.make_cache(spec, "cpu", seed=4)
    cal = cache.calib
    om = oracle_lib.omega(spec.head_dim, spec.rope_theta)
    heads = []
    for h in range(3):
        heads.append(dict(K=cache.k[0][0, h].numpy(), V=cache.v[0][0, h].numpy(),
                          pos=cache.pos[0][0, h].numpy(), p_now=cache.p_now[0], om=om,
                          offsets=cal.offsets, qc_re=cal.qc_re[0, h], qc_im=cal.qc_im[0, h],
                          q_mean_norm=cal.q_mean_norm[0, h], q_mrl=cal.q_mrl[0, h]))
    shared = oracle_lib.prune_layer_shared(heads, 70 * 3, 70, 0, threads=2)
    for h, j in enumerate(heads):
        uni = oracle_lib.prune_head(j["K"], j["V"], j["pos"], j["p_now"], om, cal.offsets, j["qc_re"],
                             j["qc_im"], j["q_mean_norm"], j["q_mrl"], 70, 0)
        np.testing.assert_array_equal(shared[h]["kept"], uni["kept"])
        np.testing.assert_array_equal(shared[h]["K"], uni["K"])
        np.testing.assert_array_equal(shared[h]["pos"], uni["pos"])
