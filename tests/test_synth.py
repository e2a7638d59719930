"""The seeded input generator: determinism, rounding, token order and workload sizes (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], dtype=np.float32)])
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(mine),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_morton_order_is_a_permutation_and_compact():
    grid = (16, 45, 80)
    c = synth.morton_order(grid)
    assert c.shape == (16 * 45 * 80, 3)
    flat = (c[:, 0] * 45 + c[:, 1]) * 80 + c[:, 2]
    assert len(np.unique(flat)) == flat.size
    # a 64-token run of a Morton order is spatially compact: its bounding box is small
    ext = [np.ptp(c[s:s + 64], axis=0).prod() for s in range(0, c.shape[0], 64)]
    assert np.median(ext) <= 64


def test_cube_order_option_changes_only_the_token_order():
    # on power-of-two sides the two orders coincide; a side of 6 beside a longer one makes them differ
    assert np.array_equal(synth.cube_order((4, 8, 8), 64), synth.morton_order((4, 8, 8)))
    w = synth.workload(1).with_(grid=(4, 6, 16), heads=1)
    wc = w.with_(order="cubes")
    a, c = synth.generate(w), synth.generate(wc)
    np.testing.assert_array_equal(a.coords, synth.morton_order(w.grid))
    np.testing.assert_array_equal(c.coords, synth.cube_order(w.grid, w.group))
    assert not np.array_equal(a.coords, c.coords)
    assert sorted(map(tuple, a.coords.tolist())) == sorted(map(tuple, c.coords.tolist()))
    np.testing.assert_array_equal(c.q, synth.generate(wc).q)       # deterministic
    try:
        synth.generate(w.with_(order="raster"))
    except ValueError:
        pass
    else:
        raise AssertionError("unknown order accepted")


def test_generate_deterministic_and_shaped():
    w = synth.workload(1)
    a, b = synth.generate(w), synth.generate(w)
    for name in ("q", "k", "v"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
        assert getattr(a, name).shape == (1, 2, 1024, 64) and getattr(a, name).dtype == np.float32
    assert a.do is None
    assert a.w.shape == (2, 64, 16) and a.w.dtype == np.float32
    assert list(a.k_per_head) == [4, 4]
    w2 = synth.workload(2).with_(grid=(2, 8, 32), heads=3)
    x = synth.generate(w2)
    assert x.q.dtype == np.uint16 and x.q.shape == (1, 3, 512, 64)
    # threads do not change the values
    y = synth.generate(w2, threads=1)
    np.testing.assert_array_equal(x.k, y.k)


def test_workload_sizes():
    assert [synth.workload(i).seq_len for i in range(1, 6)] == [1024, 8192, 57600, 131072, 520000]
    assert synth.workload(2).uniform_k() == 13
    assert synth.workload(3).uniform_k() == 90
    assert synth.workload(4).uniform_k() == 102
    assert synth.workload(4).n_groups == 1024 and synth.workload(4).n_blocks == 2048
    assert synth.keep_to_k(0.1, 900) == 90 and synth.keep_to_k(1e-9, 10) == 1 and synth.keep_to_k(2.0, 10) == 10


def test_per_head_workload_structure():
    w = synth.workload(5).with_(grid=(4, 8, 16), n_centres=8)
    x = synth.generate(w)
    nb = w.n_blocks
    assert x.k_per_head.shape == (24,)
    assert (x.k_per_head >= 1).all() and (x.k_per_head <= nb).all()
    assert ((x.head_scale >= 1.5) & (x.head_scale <= 4.5)).all()
    assert ((x.head_keep >= 0.02) & (x.head_keep <= 0.30)).all()
    assert len(set(x.head_scale.tolist())) == 24


def test_clusters_shared_by_q_and_k():
    w = synth.workload(1)
    x = synth.generate(w)
    q = x.as_f64("q")[0, 0]
    k = x.as_f64("k")[0, 0]
    v = x.as_f64("v")[0, 0]
    same = x.cell_centre[:, None] == x.cell_centre[None, :]
    qk = q @ k.T
    assert qk[same].mean() > qk[~same].mean() + 20.0      # scale 3 clusters: ~9*64 shared energy
    assert abs((q @ v.T).mean()) < 1.0


def test_head_subset_is_exact():
    w = synth.workload(5).with_(grid=(2, 8, 16), n_centres=8)
    full = synth.generate(w)
    sub = synth.generate(w, heads=[3, 17])
    for name in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(getattr(sub, name)[:, 0], getattr(full, name)[:, 3])
        np.testing.assert_array_equal(getattr(sub, name)[:, 1], getattr(full, name)[:, 17])
    assert list(sub.k_per_head) == [full.k_per_head[3], full.k_per_head[17]]
    np.testing.assert_array_equal(sub.w[1], full.w[17])
