"""GPU parity for the ViT index tables: the HIP kernels (through the C ABI)
against the oracle.

Bar: positions, window index and its inverse bit-exact; cos/sin within
2^-22 absolute of the oracle's float64 cos/sin of the same float32 angle
(the angle is formed identically on both sides, float32(p * inv_freq[k]), so
what remains is the device sincosf error, a few float32 ulps of values in
[-1, 1]).  Outputs are prefilled with sentinels (NaN, -1) so an unwritten
element fails.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TRIG_TOL = 2.0 ** -22


def _say(*a):
    print("[gpu-vit]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _tables(V, desc, column, rope_dim=32, theta=10000.0):
    rows = int(desc["rows"].sum())
    n = max(rows, 1)
    ws = torch.empty(max(V.workspace_bytes(len(desc)), 16), dtype=torch.uint8, device="cuda")
    pos = torch.full((n, 2), -1, dtype=torch.int32, device="cuda")
    cos = torch.full((n, rope_dim), float("nan"), dtype=torch.float32, device="cuda")
    sin = torch.full((n, rope_dim), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((max(rows // 4, 1),), -1, dtype=torch.int64, device="cuda")
    inv = torch.full((max(rows // 4, 1),), -1, dtype=torch.int64, device="cuda")
    before = V.dispatch_count()
    V.rotary_tables(desc, ws, pos=pos, cos=cos, sin=sin, column=column, rope_dim=rope_dim,
                    theta=theta)
    V.window_index(desc, ws, index=idx, inverse=inv, column_major=column)
    torch.cuda.synchronize()
    if rows:
        assert V.dispatch_count() == before + 2
    return (pos[:rows].cpu().numpy(), cos[:rows].cpu().numpy(), sin[:rows].cpu().numpy(),
            idx[:rows // 4].cpu().numpy(), inv[:rows // 4].cpu().numpy())


def _check(desc, got, column, rope_dim=32, theta=10000.0, items=None):
    pos, cos, sin, idx, inv = got
    ok = desc["status"] == 0
    thw = np.stack([desc["grid_t"], desc["grid_h"], desc["grid_w"]], axis=1)
    for i in (range(len(desc)) if items is None else items):
        if not ok[i]:
            continue
        r0, r1 = int(desc["row_offset"][i]), int(desc["row_offset"][i] + desc["rows"][i])
        ref = oracle.rotary_positions(*[int(v) for v in thw[i]], column=column)
        assert np.array_equal(pos[r0:r1], ref), f"positions item {i}"
        _, c, s = oracle.rope_tables(ref, rope_dim, theta)
        for name, g, r in (("cos", cos[r0:r1], c), ("sin", sin[r0:r1], s)):
            err = np.abs(g.astype(np.float64) - r)
            assert np.isfinite(g).all() and err.max() <= TRIG_TOL, (name, i, float(err.max()))
    if items is None:
        ref_idx = oracle.window_index(thw[ok], column)
        assert np.array_equal(idx, ref_idx)
        assert np.array_equal(inv[idx], np.arange(idx.size))


MIXED = [(1, 200, 300, 3), (5, 64, 96, 3), (1, 1, 8193, 3), (3, 96, 128, 4), (1, 4000, 6000, 3),
         (7, 16, 192, 3), (1, 1, 1, 3), (2, 1080, 1920, 3), (1, 33, 1000, 3)]


@pytest.mark.parametrize("column", [False, True])
def test_mixed_batch_tables(V, column):
    _say("mixed batch, column =", column)
    desc, _, _, _ = V.plan_frames(MIXED, check=False)
    assert (desc["status"] != 0).sum() == 1  # 1x8193 is rejected and skipped
    _check(desc, _tables(V, desc, column), column)


@pytest.mark.parametrize("rope_dim,theta", [(8, 10000.0), (64, 10000.0), (40, 500.0), (256, 1e6)])
def test_rope_dims_and_bases(V, rope_dim, theta):
    _say("rope_dim", rope_dim, "theta", theta)
    desc, _, _, _ = V.plan_frames([(1, 700, 1000, 3), (4, 96, 96, 3)])
    _check(desc, _tables(V, desc, True, rope_dim, theta), True, rope_dim, theta)


def test_tables_match_the_pixel_rows(V):
    """A coded image whose pixel (y, x) holds (y, x): the GPU rows' (py, px) =
    (0, 0) value decodes to 16 x the GPU rotary position, in both orders."""
    _say("positions follow the rows")
    h, w = 192, 256
    y, x = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    img = np.stack([y, x, np.zeros_like(y)], axis=-1).astype(np.uint8)
    b = W._from_images("coded", [img], mean=(0.0, 0.0, 0.0), std=(1 / 255, 1 / 255, 1 / 255),
                       out_dtype="f32")
    plan = V.plan_batch(b.shapes)
    src = V.processor.upload_sources(b.packed, plan)
    out = V.preprocess(src, plan, mean=b.mean, std=b.std, merge_order=True, column_order=True)
    for column, rows in ((False, out["pixel_values"]), (True, out["pixel_values_col"])):
        t = V.vit_tables(plan, column=column)
        torch.cuda.synchronize()
        first = rows.view(-1, 3, 2, 16, 16)[:, :2, 0, 0, 0].round().to(torch.int32)
        assert torch.equal(first, 16 * t["rotary_pos"])


def test_back_to_back_and_empty(V):
    _say("back to back, then empty")
    d1, _, _, _ = V.plan_frames([(9, 300, 500, 3), (1, 64, 64, 4)])
    d2, _, _, _ = V.plan_frames([(1, 48, 48, 3)])
    _check(d1, _tables(V, d1, True), True)
    _check(d2, _tables(V, d2, False), False)
    d0, _, _, _ = V.plan_frames(np.zeros((0, 4), np.int32))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    pos = torch.empty((1, 2), dtype=torch.int32, device="cuda")
    V.rotary_tables(d0, ws, pos=pos)  # no-op


def test_throughput_batch_tables(V):
    """The 512 x 1024^2 batch's tables in column order: positions and the
    window index in full, cos/sin on sampled items."""
    _say("throughput batch tables")
    desc, _, _, _ = V.plan_geometry([(1024, 1024, 3)] * 512)
    got = _tables(V, desc, True)
    pos = got[0]
    ref = oracle.rotary_positions(1, 64, 64, column=True)
    assert np.array_equal(pos.reshape(512, 4096, 2), np.broadcast_to(ref, (512, 4096, 2)))
    _check(desc, got, True, items=[0, 1, 255, 511])
    thw = np.tile([1, 64, 64], (512, 1))
    assert np.array_equal(got[3], oracle.window_index(thw, True))
    assert np.array_equal(got[4][got[3]], np.arange(got[3].size))
