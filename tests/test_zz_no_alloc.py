"""The allocation-free counted compaction, tri_compact_kv_counts_noalloc,
against the workspace call tri_compact_kv_counts through the C ABI: on
identical inputs both leave K, V, positions and head lengths bit-identical.
Two calls in a row, the second on a smaller input (the static scratch keeps
the first call's contents), and the size limit of the scratch."""
import numpy as np
import pytest
import torch

import synth
import rope_aware_eviction_amd as tri

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dummy_ctx(L, H, d):
    z = np.zeros((L, H, d // 2))
    o = np.ones((L, H, d // 2))
    return tri.tri_calibrate_load(L, H, d, z, z, o, o, [1], device=0)


def bits(t):
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])


def shared_lists(ctx, L, H, lens, B, F, W, seed):
    """Kept lists and counts of head-specific budgets for ragged caches of
    the given lengths (selected on the GPU from synthetic scores)."""
    total = B * H
    hls, seqs = [], []
    for s, n in enumerate(lens):
        hl = torch.from_numpy(synth.head_lengths("ragged", L, H, n, seed=seed + s)).cuda()
        hls.append(hl)
        seqs.append(tri.Seq(torch.empty((L, H, n, 128), dtype=torch.bfloat16, device="cuda"), None,
                            None, n, n - 1, hl))
    scores = torch.from_numpy(np.concatenate(
        [synth.make_scores("dups", L * H, n, seed=seed + s).reshape(-1) for s, n in enumerate(lens)])).cuda()
    kept = torch.full((len(lens) * L * H * total,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((len(lens) * L * H,), -9, dtype=torch.int32, device="cuda")
    ws = torch.empty(tri.select_shared_workspace_bytes(ctx, len(lens)), dtype=torch.uint8, device="cuda")
    tri.tri_select_shared(ctx, seqs, scores, B, F, W, kept, counts, ws)
    torch.cuda.synchronize()
    return kept, counts, [h.clone() for h in hls]


def compare_one_call(ctx, L, H, lens, B, F, W, seed):
    kept, counts, hls = shared_lists(ctx, L, H, lens, B, F, W, seed)
    total = B * H
    caches = []
    for s, n in enumerate(lens):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed * 100 + s)
        K = torch.randn((L, H, n, 128), generator=g, device="cuda").to(torch.bfloat16)
        V = torch.randn((L, H, n, 128), generator=g, device="cuda").to(torch.bfloat16)
        P = (torch.arange(n, dtype=torch.int32, device="cuda") * 3 + 1).repeat(L, H, 1)
        caches.append((K, V, P))
    # copy a: the workspace call; copy b: the allocation-free call
    a = [(K.clone(), V.clone(), P.clone(), hls[s].clone()) for s, (K, V, P) in enumerate(caches)]
    b = [(K.clone(), V.clone(), P.clone(), hls[s].clone()) for s, (K, V, P) in enumerate(caches)]
    seqs_a = [tri.Seq(K, V, P, n, n - 1, hl) for (K, V, P, hl), n in zip(a, lens)]
    seqs_b = [tri.Seq(K, V, P, n, n - 1, hl) for (K, V, P, hl), n in zip(b, lens)]
    cws = torch.empty(tri.compact_counts_workspace_bytes(ctx), dtype=torch.uint8, device="cuda")
    tri.tri_compact_kv_counts(ctx, seqs_a, kept, total, counts, cws)
    tri.tri_compact_kv_counts_noalloc(ctx, seqs_b, kept, total, counts)
    torch.cuda.synchronize()
    moved = 0
    for s in range(len(lens)):
        for x, y in zip(a[s], b[s]):
            assert torch.equal(bits(x) if x.dtype == torch.bfloat16 else x,
                               bits(y) if y.dtype == torch.bfloat16 else y)
        moved += int((counts.view(len(lens), L, H)[s] >= 0).sum())
        # the heads that fired took their counts
        c = counts.view(len(lens), L, H)[s]
        assert torch.equal(torch.where(c >= 0, c, hls[s]), a[s][3])
    return moved


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    ctx = dummy_ctx(4, 8, 128)
    m1 = compare_one_call(ctx, 4, 8, [6000, 4500, 300], B=500, F=60, W=16, seed=3)
    m2 = compare_one_call(ctx, 4, 8, [1200], B=100, F=10, W=8, seed=5)   # smaller input second
    assert m1 > 0 and m2 > 0
    print("allocation-free compaction matched the workspace call on %d + %d heads" % (m1, m2))


def test_noalloc_rejects_contexts_beyond_the_scratch():
    L = 65537                                  # one (layer, KV head) past the scratch's capacity
    ctx = dummy_ctx(L, 1, 64)
    n = 4
    K = torch.zeros((L, 1, n, 64), device="cuda")
    hl = torch.full((L, 1), n, dtype=torch.int32, device="cuda")
    seq = tri.Seq(K, K.clone(), torch.zeros((L, 1, n), dtype=torch.int32, device="cuda"), n, n - 1, hl)
    kept = torch.zeros(L * 2, dtype=torch.int32, device="cuda")
    counts = torch.full((L,), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(tri.TriError) as e:
        tri.tri_compact_kv_counts_noalloc(ctx, [seq], kept, 2, counts)
    assert e.value.status == tri.TRI_E_SCRATCH
    torch.cuda.synchronize()
