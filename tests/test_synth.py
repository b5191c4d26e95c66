"""The seeded input generator: shapes, determinism and the stated structure."""
import numpy as np
import torch

import synth


def _unrotate_np(K, pos, theta):
    d = K.shape[-1]
    h = d // 2
    om = np.array([theta ** (-2.0 * f / d) for f in range(h)])
    ang = pos[:, None].astype(np.float64) * om[None, :]
    z = (K[:, :h] + 1j * K[:, h:]) * np.exp(-1j * ang)
    return z


def test_workload_sizes():
    assert synth.workload("toy").keys == 1024
    assert synth.workload("llama8b").keys == 32 * 8 * 8192
    assert synth.workload("qwen3_32k").keys == 36 * 8 * 32768
    b = synth.workload("batched")
    assert b.n_seq == 64 and all(4096 <= n <= 32768 for n in b.lengths)
    assert synth.workload("wide").keys == 64 * 8 * 131072


def test_deterministic_and_seed_dependent():
    spec = synth.workload("toy")
    a = synth.make_cache(spec, "cpu", seed=0)
    b = synth.make_cache(spec, "cpu", seed=0)
    c = synth.make_cache(spec, "cpu", seed=1)
    assert torch.equal(a.k[0], b.k[0]) and torch.equal(a.v[0], b.v[0])
    assert not torch.equal(a.k[0], c.k[0])
    np.testing.assert_array_equal(a.calib.qc_re, b.calib.qc_re)


def test_toy_keys_concentrate_around_centre_of_norm_4():
    spec = synth.workload("toy")
    c = synth.make_cache(spec, "cpu", seed=0)
    K = c.k[0][0, 0].numpy().astype(np.float64)
    pos = c.pos[0][0, 0].numpy()
    z = _unrotate_np(K, pos, spec.rope_theta)
    pre = np.concatenate([z.real, z.imag], axis=1)
    centre = pre.mean(axis=0)
    assert abs(np.linalg.norm(centre) - 4.0) < 0.1
    assert abs(pre.std(axis=0).mean() - 0.3) < 0.03
    qc = c.calib.qc_re[0, 0] + 1j * c.calib.qc_im[0, 0]
    assert abs(np.linalg.norm(np.concatenate([qc.real, qc.imag])) - 4.0) < 1e-9
    R = c.calib.q_mrl[0, 0]
    assert np.all((R > 1 / 1.5 - 1e-12) & (R <= 1.0))


def test_phase_recipe_has_requested_concentration():
    spec = synth.workload("qwen3_32k").replace(n_layers=1, n_kv_heads=2, lengths=(4000,))
    c = synth.make_cache(spec, "cpu", seed=0)
    for h in range(2):
        R = c.calib.q_mrl[0, h, 0]
        assert 0.6 <= R <= 0.99
        K = c.k[0][0, h].float().numpy().astype(np.float64)
        z = _unrotate_np(K, c.pos[0][0, h].numpy(), spec.rope_theta)
        mrl = np.abs(np.mean(z / np.abs(z), axis=0))       # per band, over keys
        assert abs(np.median(mrl) - R) < 0.05


def test_near_ties_are_one_ulp_copies():
    """About 20% of rows differ from another row in exactly one element, whose
    magnitude bits differ by one (one bf16 ulp)."""
    spec = synth.workload("wide").replace(n_layers=1, n_kv_heads=1, lengths=(2000,))
    c = synth.make_cache(spec, "cpu", seed=0)
    K = c.k[0][0, 0].view(torch.int16).numpy().astype(np.int32) & 0xFFFF
    near = 0
    for i in range(K.shape[0]):
        eq = (K == K[i]).sum(axis=1)
        for j in np.nonzero(eq == K.shape[1] - 1)[0]:
            col = int(np.nonzero(K[j] != K[i])[0][0])
            if abs(int(K[j, col] & 0x7FFF) - int(K[i, col] & 0x7FFF)) == 1:
                near += 1
                break
    assert near >= 0.9 * 0.2 * 2000


def test_pruned_positions_strictly_ascending():
    p = synth.pruned_positions(0, 1000, start=50)
    assert p[0] >= 50 and np.all(np.diff(p) > 0)


def test_score_and_kept_generators():
    s = synth.make_scores("special", 3, 500, 0)
    assert s.dtype == np.float32 and np.isnan(s).any() and np.isinf(s).any()
    for kind in ("random", "all_but_first", "every8", "last", "prefix", "blocks"):
        k = synth.make_kept(kind, 2, 1000, 300, 0)
        assert k.shape == (2, 300)
        assert np.all(np.diff(k, axis=1) > 0) and k.min() >= 0 and k.max() < 1000
