"""CPU tests of the seeded input generator (no method arithmetic lives there)."""
import numpy as np
import pytest

from sparse_attention_token_absorb_amd import synth


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_bf16(x).view(np.uint32), ref.view(np.uint32))


def test_tiny_fp32_n512_shapes_and_determinism():
    a = synth.tiny_fp32_n512()
    b = synth.tiny_fp32_n512()
    assert a.dtype == "fp32" and a.B == 1 and a.Q == 1 and a.G == 4
    assert a.latent[0].shape == (512, 64)
    assert a.q[0].shape == (1, 4, 32) and a.W[0].shape == (32, 64) and a.w[0].shape == (1, 4)
    assert len(a.heavy[0]) == 8
    assert int(a.qpos[0]) == 511
    for l in range(4):
        assert np.array_equal(a.q[l], b.q[l]) and np.array_equal(a.W[l], b.W[l])
    assert np.array_equal(a.latent[0], b.latent[0])
    assert (a.w[0] >= 0).all() and (a.w[0] < 1).all()


def test_ragged_paged_layout():
    g = synth.make_decode("t", 3, B=5, lens=(100, 300), r=64, H=4, d=32, k=16, M=32)
    assert ((g.lens >= 100) & (g.lens <= 300)).all()
    used = g.block_table[g.block_table >= 0]
    assert sorted(used.tolist()) == list(range(g.num_pages))  # a permutation of all pages
    for b in range(g.B):
        npg = (int(g.lens[b]) + 63) // 64
        assert (g.block_table[b, :npg] >= 0).all() and (g.block_table[b, npg:] == -1).all()
    # bf16 values are exact
    x = g.latent[0]
    assert np.array_equal(synth.round_bf16(x), x)


def test_heavy_rows_planted():
    g = synth.make_decode("t", 7, B=1, lens=[2000], r=64, H=4, d=32, k=16, M=32, structure=False)
    h = g.heavy[0]
    assert len(h) == 20
    norms = np.linalg.norm(g.latent[0], axis=1)
    assert norms[h].mean() > 2.0 * np.delete(norms, h).mean()


def test_baseline_keys_are_the_decoded_latent():
    """The per-layer baseline caches each layer's decoder applied to the same
    latent rows, rounded once to bf16."""
    g = synth.make_decode("t", 8, B=2, lens=[70, 33], r=64, H=4, d=32, k=16, M=32, keys_a=True)
    for l in range(g.G):
        for b in range(g.B):
            k = g.keys_a[l][b]
            assert k.shape == (int(g.lens[b]), g.d)
            assert np.array_equal(synth.round_bf16(k), k)
            exact = g.latent[b].astype(np.float64) @ g.W[l].astype(np.float64).T
            assert np.all(np.abs(k - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)
