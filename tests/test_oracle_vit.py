"""Pins for the oracle's ViT index tables (CPU only).

* rotary positions: against an independent numpy reshape/transpose of the
  (h, w) grids into merge blocks; against brute-force sorting of patch
  coordinates for column order; against the pixel path itself (a coded
  image whose rows carry their own patch coordinates); invariants;
* inv_freq: torch's float32 evaluation of theta ** (arange(0, dim, 2) / dim)
  and its reciprocal within one float32 ulp, and the float64 value on the
  float32 exponent within two;
* rope tables: torch's outer product of float32 positions and inv_freq,
  indexed by the positions, bitwise; cos/sin against numpy float64 on those
  angles (within 2 float64 ulps); sin^2 + cos^2 = 1;
* window index: identity for row-major; brute-force sort by
  (item, t, block col, block row); agrees with the row-level column
  permutation collapsed to units; a bijection;
* chunk seqlens: the repeat/cumsum closed form.
"""
import numpy as np
import pytest
import torch

import oracle

M = 2
GRIDS = [(1, 2, 2), (1, 4, 6), (1, 6, 4), (2, 4, 4), (3, 2, 8), (1, 12, 18), (5, 6, 10), (1, 2, 64)]


def _merge_order_grid(gt, gh, gw):
    """(h, w) per row in merge-block order from array reshapes alone."""
    hh, ww = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
    out = []
    for g in (hh, ww):
        b = g.reshape(gh // M, M, gw // M, M).transpose(0, 2, 1, 3).reshape(-1)
        out.append(np.tile(b, gt))
    return np.stack(out, axis=1).astype(np.int32)


@pytest.mark.parametrize("thw", GRIDS)
def test_positions_merge_order_match_reshape(thw):
    assert np.array_equal(oracle.rotary_positions(*thw), _merge_order_grid(*thw))


@pytest.mark.parametrize("thw", GRIDS)
def test_positions_column_order_brute_force(thw):
    gt, gh, gw = thw
    rows = []
    for t in range(gt):
        units = [(bc, br) for br in range(gh // M) for bc in range(gw // M)]
        for bc, br in sorted(units):
            for mh in range(M):
                for mw in range(M):
                    rows.append((br * M + mh, bc * M + mw))
    assert np.array_equal(oracle.rotary_positions(*thw, column=True), np.array(rows, np.int32))


@pytest.mark.parametrize("thw", GRIDS)
def test_positions_invariants(thw):
    gt, gh, gw = thw
    for column in (False, True):
        pos = oracle.rotary_positions(*thw, column=column).reshape(gt, gh * gw, 2)
        for t in range(gt):
            keys = pos[t, :, 0].astype(np.int64) * gw + pos[t, :, 1]
            assert np.array_equal(np.sort(keys), np.arange(gh * gw))  # every patch once per slice
        u = pos.reshape(-1, 4, 2)
        assert np.all(u[:, 0, 0] % 2 == 0) and np.all(u[:, 0, 1] % 2 == 0)
        assert np.all(u[:, 1] - u[:, 0] == [0, 1]) and np.all(u[:, 2] - u[:, 0] == [1, 0])
        assert np.all(u[:, 3] - u[:, 0] == [1, 1])


def test_positions_follow_the_pixel_rows():
    """An identity-sized image whose pixel (y, x) encodes y and x: each row's
    (py, px) = (0, 0) value decodes to (16 h, 16 w) of its rotary position,
    in both orders."""
    h, w = 96, 128
    y, x = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    img = np.stack([y, x, np.zeros_like(y)], axis=-1).astype(np.uint8)
    mean, std = [0.0, 0.0, 0.0], [1.0, 1.0, 1.0]
    rows = oracle.preprocess_image(img, h, w, mean, std)
    perm = oracle.column_permutation(1, h // 16, w // 16)
    for column, r in ((False, rows), (True, rows[perm])):
        pos = oracle.rotary_positions(1, h // 16, w // 16, column=column)
        first = r.reshape(-1, 3, 2, 16, 16)[:, :, 0, 0, 0]  # channel values at (py, px) = (0, 0)
        assert np.array_equal(first[:, 0], 16 * pos[:, 0])
        assert np.array_equal(first[:, 1], 16 * pos[:, 1])


@pytest.mark.parametrize("dim", [8, 16, 32, 40, 64, 80, 128])
def test_inv_freq_matches_torch_float32(dim):
    got = oracle.rope_inv_freq(dim)
    ref = (1.0 / (10000.0 ** (torch.arange(0, dim, 2, dtype=torch.float) / dim))).numpy()
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, (dim, ulps.max())
    # float64 value on the float32 exponent (2i / dim is inexact for dim = 40, 80):
    # two float32 roundings (power, reciprocal) stay within 2 ulps of it
    e = (np.arange(0, dim, 2, dtype=np.float32) / np.float32(dim)).astype(np.float64)
    exact = 10000.0 ** -e
    assert np.all(np.abs(got - exact) <= 2 * np.spacing(got).astype(np.float64))
    assert got[0] == 1.0


@pytest.mark.parametrize("thw,dim", [((1, 12, 18), 32), ((2, 4, 6), 64), ((1, 2, 512), 32), ((1, 600, 2), 16)])
def test_rope_tables_match_torch_outer_product(thw, dim):
    pos = oracle.rotary_positions(*thw)
    angle, c, s = oracle.rope_tables(pos, dim)
    inv = torch.from_numpy(oracle.rope_inv_freq(dim))
    seq = torch.arange(int(pos.max()) + 1, dtype=torch.float32)
    freqs = torch.outer(seq, inv)                         # forward(seqlen)
    ref = freqs[torch.from_numpy(pos).long()].flatten(1)  # [rows, 2 * dim/2]: h half, w half
    assert np.array_equal(angle, ref.numpy())
    a64 = angle.astype(np.float64)
    # numpy's SIMD float64 cos/sin and the C library's agree within 2 ulps
    for got, ref in ((c, np.cos(a64)), (s, np.sin(a64))):
        assert np.all(np.abs(got - ref) <= 2 * np.spacing(np.abs(ref)))
    assert np.abs(c * c + s * s - 1.0).max() < 1e-15
    assert np.all(c[pos[:, 0] == 0, : dim // 2] == 1.0)  # position 0: angle 0


def test_window_index_orders():
    rng = np.random.default_rng(41)
    for _ in range(40):
        n = int(rng.integers(1, 6))
        thw = [(int(rng.integers(1, 4)), 2 * int(rng.integers(1, 12)), 2 * int(rng.integers(1, 12)))
               for _ in range(n)]
        units = sum(t * (h // 2) * (w // 2) for t, h, w in thw)
        assert np.array_equal(oracle.window_index(thw, False), np.arange(units))
        col = oracle.window_index(thw, True)
        # brute force: global units keyed by (item, t, block col, block row)
        keyed, base = [], 0
        for i, (t, h, w) in enumerate(thw):
            bh, bw = h // 2, w // 2
            for tt in range(t):
                for br in range(bh):
                    for bc in range(bw):
                        keyed.append(((i, tt, bc, br), base + (tt * bh + br) * bw + bc))
            base += t * bh * bw
        assert np.array_equal(col, np.array([g for _, g in sorted(keyed)], np.int64))
        assert np.array_equal(np.sort(col), np.arange(units))
        # collapsed row-level column permutation, item by item
        off = 0
        for t, h, w in thw:
            u = t * (h // 2) * (w // 2)
            perm = oracle.column_permutation(t, h, w)
            assert np.array_equal(col[off:off + u] - off, perm[::4] // 4)
            off += u


def test_chunk_seqlens_closed_form():
    thw = np.array([(1, 4, 6), (3, 2, 8), (2, 10, 10), (1, 2, 2)])
    ref = np.concatenate([[0], np.cumsum(np.repeat(thw[:, 1] * thw[:, 2], thw[:, 0]))])
    assert np.array_equal(oracle.chunk_seqlens(thw), ref)
    assert np.array_equal(oracle.chunk_seqlens(np.zeros((0, 3))), [0])
