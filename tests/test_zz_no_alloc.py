"""The allocation-free entry point (mimo_preprocess_batch_noalloc) against
mimo_preprocess_batch, through the C ABI: the same kernel, so the rows must
be equal bit for bit, on two calls in a row (the second with a smaller
batch, which reuses the scratch the first one filled), plus the oracle's
bar on some images of each call."""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-noalloc]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _batch(n, seed):
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(1, 300)), int(rng.integers(1, 300)), int(rng.choice([3, 4])))
              for _ in range(n)]
    return W.uniform_images(shapes, seed=seed)


def _both(V, batch, out_dtype, column):
    plan = V.plan_batch(batch.shapes)
    src = V.processor.upload_sources(batch.packed, plan)
    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    m, s = V.stats255(batch.mean, batch.std)
    outs = []
    for noalloc in (False, True):
        rows = torch.full((plan.total_rows, 1536), float("nan"), dtype=tdtype, device="cuda")
        cols = torch.full_like(rows, float("nan")) if column else None
        before = V.dispatch_count()
        if noalloc:
            V._abi.preprocess_batch_noalloc(plan.desc, src, m, s, rows=rows, rows_col=cols)
        else:
            ws = torch.empty(V.workspace_bytes(len(plan)), dtype=torch.uint8, device="cuda")
            V.preprocess_batch(plan.desc, src, m, s, rows=rows, rows_col=cols, workspace=ws)
        torch.cuda.synchronize()
        assert V.dispatch_count() == before + 1
        outs.append((rows, cols))
    return plan, outs


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def _oracle_check(batch, plan, rows, out_dtype, images):
    m, s = oracle.stats255(batch.mean, batch.std)
    for i in images:
        d = plan.desc[i]
        ref = oracle.preprocess_image(batch.image(i), int(d["dst_h"]), int(d["dst_w"]), m, s)
        got = rows[int(d["row_offset"]):int(d["row_offset"] + d["rows"])].float().cpu().numpy()
        if out_dtype == "f32":
            assert np.abs(got.astype(np.float64) - ref).max() <= 1e-4, i
        else:
            want = oracle.to_bf16_bits(ref).astype(np.int64)
            have = (got.view(np.uint32) >> 16).astype(np.int64)
            signed = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b)
            assert np.abs(signed(have) - signed(want)).max() <= 1, i


def test_noalloc_equals_workspace_path_two_calls(V):
    # first call: 150 ragged RGB/RGBA images (tables of several 3 KB pieces),
    # both orders, float32; second call: 7 images, bf16, merge order
    for n, seed, out_dtype, column in ((150, 301, "f32", True), (7, 302, "bf16", False)):
        _say("batch", n, out_dtype, "column" if column else "merge")
        batch = _batch(n, seed)
        plan, ((r0, c0), (r1, c1)) = _both(V, batch, out_dtype, column)
        assert bool(torch.isfinite(r1).all())
        assert _same_bits(r0, r1), "merge order differs from the workspace path"
        if column:
            assert bool(torch.isfinite(c1).all())
            assert _same_bits(c0, c1), "column order differs from the workspace path"
        _oracle_check(batch, plan, r1, out_dtype, [0, n // 2, n - 1])


def test_noalloc_refuses_too_many_images(V):
    _say("capacity")
    n = V._abi.NOALLOC_MAX_IMAGES + 1
    desc, _, _, _ = V.plan_geometry([(32, 32, 3)] * n)
    src = torch.zeros(n * 32 * 32 * 3 + 16, dtype=torch.uint8, device="cuda")
    rows = torch.empty((desc["rows"].sum(), 1536), dtype=torch.float32, device="cuda")
    before = V.dispatch_count()
    with pytest.raises(V.MimoError) as e:
        V._abi.preprocess_batch_noalloc(desc, src, (0.0,) * 3, (1.0,) * 3, rows=rows)
    assert e.value.code == V.MIMO_E_CAPACITY and V.dispatch_count() == before
