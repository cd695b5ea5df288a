"""Checks of the seeded input generators (not of the method)."""

import itertools

import numpy as np
import pytest
import torch

from sparse_gemv_memory_amd import synth, workloads


def _brute_topn(w_bits, n, m):
    rows, cols = w_bits.shape
    keep = np.zeros((rows, cols), dtype=np.uint8)
    for r in range(rows):
        for g in range(cols // m):
            idx = list(range(g * m, (g + 1) * m))
            mags = [int(w_bits[r, c]) & 0x7FFF for c in idx]
            order = sorted(range(m), key=lambda j: (-mags[j], j))
            for j in order[:n]:
                keep[r, idx[j]] = 1
    return keep


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_topn_mask_matches_brute_force(n, m):
    W = synth.weights(7, 64, seed=21)
    assert np.array_equal(synth.topn_mask(W, n, m), _brute_topn(W, n, m))


def test_topn_mask_ties_go_to_lower_column():
    f16 = lambda v: np.array(v, dtype=np.float16).view(np.uint16)
    # equal magnitudes with opposite signs, and +0 / -0
    W = np.stack([f16([0.5, -0.5, 0.5, -0.5]), f16([0.0, -0.0, 0.0, 0.0]),
                  f16([-1.0, 0.25, 1.0, 0.25]), f16([0.1, 0.2, 0.2, 0.2])])
    keep = synth.topn_mask(W, 2, 4)
    assert keep.tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [1, 0, 1, 0], [0, 1, 1, 0]]


def test_topn_mask_all_4tuples_of_small_magnitudes():
    # every ordering pattern of 4 magnitudes drawn from 3 levels (ties included)
    levels = [0x0000, 0x3C00, 0x4000]
    rows = [list(t) for t in itertools.product(levels, repeat=4)]
    W = np.array([rows[i] for i in range(len(rows))], dtype=np.uint16).reshape(-1, 4)
    W = np.concatenate([W, W | 0x8000], axis=0)
    assert np.array_equal(synth.topn_mask(W, 2, 4), _brute_topn(W, 2, 4))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125 + 2 ** -9, 3e38, -1e-40],
                                 dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generators_are_seeded_and_shaped():
    a = synth.weights(4, 64, seed=5)
    b = synth.weights(4, 64, seed=5)
    assert a.dtype == np.uint16 and a.shape == (4, 64) and np.array_equal(a, b)
    x = synth.activations(3, 4096, seed=5)
    xf = x.view(np.float16).astype(np.float32)
    # 4 outlier channels (0.1% of 4096, rounded), identical across the batch
    big = np.abs(xf) > 8
    assert big.any()
    assert synth.activations(1, 4096, seed=5, outliers=False).shape == (1, 4096)
    w = synth.weights(512, 512, seed=1).view(np.float16).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.001


def test_random_mask_is_valid():
    k = synth.random_mask(10, 64, 4, 8, seed=1)
    assert np.all(k.reshape(10, 8, 8).sum(axis=-1) == 4)


def test_workload_tables():
    c2 = workloads.config_matrices(2)
    assert [(m.rows, m.cols) for m, _ in c2] == [(r, c) for _, r, c in workloads.LLAMA8B_LAYER]
    assert workloads.config_matrices(1)[0][0].seed == 0
    assert len(workloads.config_matrices(5)) == 224
    # bytes per call of the 14336x4096 layer at batch 1, fp32 y (closed form)
    b = workloads.sparse_bytes(14336, 4096, 2, 4, 1, 4)
    assert b == 14336 * 4096 + 14336 * 4096 // 8 + 4096 * 2 + 14336 * 4
