"""CPU checks of the parity helpers themselves: the selection check must reject a
selection of the wrong size even when every differing row is a near-tie, and the
attention sample must touch every tile. No GPU."""
import numpy as np
import pytest

from parity import attn_tile_rows, check_selection, tile_sample


def _ref(dev, sel, kth):
    return dict(sel_idx=np.asarray(sel, np.int64), dev=np.asarray(dev, np.float64),
                kth=np.asarray(kth, np.float64))


def test_check_selection_sizes_and_near_ties():
    # two requests of four rows; top-2 each; rows 2 and 3 are near-tied (gap 1e-6)
    dev = [5.0, 4.0, 3.0, 3.000003, 9.0, 8.0, 7.0, 1.0]
    req = np.array([0, 0, 0, 0, 1, 1, 1, 1])
    ref = _ref(dev, [0, 3, 4, 5], [3.000003, 8.0])
    check_selection(np.array([0, 3, 4, 5]), ref, req, "exact")
    assert check_selection(np.array([0, 2, 4, 5]), ref, req, "swap") == [2, 3]
    with pytest.raises(AssertionError, match="selects 3 rows"):
        check_selection(np.array([0, 2, 3, 4, 5]), ref, req, "one extra near-tie")
    with pytest.raises(AssertionError, match="selects 1 rows"):
        check_selection(np.array([0, 4, 5]), ref, req, "one missing")
    with pytest.raises(AssertionError, match="differs"):
        check_selection(np.array([0, 3, 4, 6]), ref, req, "far swap")


def test_tile_sample_hits_every_tile():
    off = [0, 130, 130, 200]  # requests of 130, 0 and 70 selected rows
    tr = attn_tile_rows("bf16", 40, 8)
    assert tr == 51 and attn_tile_rows("bf16", 32, 8) == 64 and attn_tile_rows("f32", 40, 8) == 32
    sp = tile_sample(off, tr, extra=0)
    tiles = {(0, 0), (0, 51), (0, 102), (2, 130), (2, 181)}
    for r, t in tiles:
        end = min(t + tr, off[r + 1])
        assert t in sp and end - 1 in sp
    assert sp.max() < off[-1] and len(sp) == 2 * len(tiles)


def test_attn_sigma_matches_monte_carlo():
    # the first-order deviation of the bf16 rounding model equals the spread of the
    # exact output under random relative errors of that model (uniform on [-u, u])
    from parity import BF16_U, attn_sigma
    rng = np.random.default_rng(4)
    nh, nkv, d, n = 2, 1, 16, 24
    q = rng.standard_normal((nh, d)) * 2.0
    K = rng.standard_normal((n, nkv, d)) * 1.5
    V = rng.standard_normal((n, nkv, d)) * 3.0
    keys = np.arange(n)

    def out(eq, ek, ep, ev, eo):
        o = np.zeros((nh, d))
        for h in range(nh):
            s = (K[:, 0] * (1 + ek[h])) @ (q[h] * (1 + eq[h])) / np.sqrt(d)
            p = np.exp(s - s.max())
            o[h] = ((p * (1 + ep[h])) @ (V[:, 0] * (1 + ev[h]))) / p.sum()
        return o * (1 + eo)

    zero = lambda: (np.zeros((nh, d)), np.zeros((nh, n, d)), np.zeros((nh, n)), np.zeros((nh, n, d)),
                    np.zeros((nh, d)))
    o0 = out(*zero())
    uni = lambda shape: rng.uniform(-BF16_U, BF16_U, shape)
    samples = np.stack([out(uni((nh, d)), uni((nh, n, d)), uni((nh, n)), uni((nh, n, d)), uni((nh, d))) - o0
                        for _ in range(3000)])
    sig = attn_sigma(q, K, V, o0, keys)
    ratio = samples.std(axis=0) / sig
    assert 0.85 < np.median(ratio) < 1.15 and ratio.min() > 0.7 and ratio.max() < 1.3, ratio
