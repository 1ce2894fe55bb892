"""Static-cube ordering used by the V-Smooth ordering ablation (host side)."""
import numpy as np

from bit_attention_video_smooth_amd.ablation import cube_permutation


def test_cube_permutation_blocks_are_cubes():
    T, Hg, W = 4, 16, 24
    perm = cube_permutation((T, Hg, W))
    assert np.array_equal(np.sort(perm), np.arange(T * Hg * W))
    t, rem = np.divmod(perm, Hg * W)
    h, w = np.divmod(rem, W)
    # a 2x8x8 cube is exactly one 128-token block
    for blk in range(len(perm) // 128):
        sl = slice(128 * blk, 128 * blk + 128)
        assert len({(a, b, c) for a, b, c in zip(t[sl] // 2, h[sl] // 8, w[sl] // 8)}) == 1
        assert np.all(np.diff(perm[sl]) > 0)  # sequence order inside a cube


def test_cube_permutation_ragged_grid():
    perm = cube_permutation((3, 5, 7))
    assert np.array_equal(np.sort(perm), np.arange(105))
