"""GPU parity for the patch embedding (the rows' Conv3d consumer) against
the oracle's float64 dot products on the same bf16 inputs.

Bar, derived from the arithmetic.  bf16 x bf16 products are exact in
float32, so the only error of the float32-accumulated GEMM is the sum's
rounding: |err| <= K * 2^-24 * S with S = sum_k |x_k| |w_k| (the standard
bound for K terms), plus the final rounding of the output (unit roundoff
2^-24 |ref| for float32, 2^-8 |ref| for bf16, which keeps 8 significant
bits) and of the bias add.  The folded weight W' = bf16(W0 + W1) adds at
most 2^-8 * S (one bf16 rounding of each summed weight; for still images
the two halves of a row are equal, so sum |x| |W0 + W1| over the half is at
most S).
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-embed]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _bf16_rows(V, items, seed, video_budget=None):
    b = W.media_batch(items, seed=seed, video_budget=video_budget)
    plan = V.plan_media(b.items, video_budget=b.video_budget)
    src = V.processor.upload_sources(b.packed, plan)
    out = V.preprocess(src, plan, mean=b.mean, std=b.std, out_dtype="bf16")
    torch.cuda.synchronize()
    return plan, out["pixel_values"][:plan.total_rows]


def _weights(e, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    w = (torch.randn((e, 1536), generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(e, generator=g) * 0.1).float() if bias else None
    return w, b


def _reference(rows_bf16, w_bf16, bias):
    x = rows_bf16.float().cpu().numpy()
    w = w_bf16.float().cpu().numpy()
    b = None if bias is None else bias.cpu().numpy()
    ref = oracle.patch_embed(x, w, b)
    s = oracle.patch_embed(np.abs(x), np.abs(w))
    return ref, s


def _assert_within(got, ref, s, k, out_dtype, extra=0.0, what=""):
    g = got.float().cpu().numpy().astype(np.float64)
    out_rel = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -24
    tol = (k * 2.0 ** -24 + extra) * s + out_rel * np.abs(ref) + 2.0 ** -24 * np.abs(ref) + 1e-30
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), what
    bad = err > tol
    assert not bad.any(), (what, int(bad.sum()), float((err / tol).max()))


STILLS = [(1, 200, 300, 3), (1, 45, 77, 4), (1, 513, 257, 3), (1, 1, 64, 3)]
MIXED = STILLS + [(5, 64, 96, 3), (2, 120, 200, 4)]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("e", [256, 1280])
def test_full_k_ragged(V, out_dtype, e):
    _say("full K, E =", e, out_dtype)
    plan, rows = _bf16_rows(V, MIXED, seed=71)
    assert rows.shape[0] % 256 != 0  # a ragged last tile
    w, bias = _weights(e, seed=72)
    wd, bd = w.cuda(), bias.cuda()
    out = V.patch_embed(rows, wd, bd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, s = _reference(rows, w, bias)
    _assert_within(out, ref, s, 1536, out_dtype, what=f"E={e} {out_dtype}")


def test_fold_weights_bits(V):
    _say("fold weights")
    w, _ = _weights(1280, seed=73, bias=False)
    wf = V.fold_patch_weights(w.cuda())
    torch.cuda.synchronize()
    w4 = w.float().numpy().reshape(1280, 3, 2, 256)
    summed = (w4[:, :, 0] + w4[:, :, 1]).reshape(1280, 768)  # float32 sum of two bf16 values
    want = oracle.to_bf16_bits(np.ascontiguousarray(summed, dtype=np.float32))
    have = wf.cpu().view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(have, want)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_folded_stills_match_full_conv(V, out_dtype):
    _say("folded, stills", out_dtype)
    plan, rows = _bf16_rows(V, STILLS, seed=74)
    w, bias = _weights(1280, seed=75)
    wd, bd = w.cuda(), bias.cuda()
    wf = V.fold_patch_weights(wd)
    out = V.patch_embed(rows, wf, bd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, s = _reference(rows, w, bias)
    _assert_within(out, ref, s, 768, out_dtype, extra=2.0 ** -8, what=f"folded {out_dtype}")


def test_empty_and_argument_errors(V):
    _say("empty and errors")
    w, _ = _weights(256, seed=76, bias=False)
    wd = w.cuda()
    rows = torch.zeros((0, 1536), dtype=torch.bfloat16, device="cuda")
    out = V.patch_embed(rows, wd)
    assert out.shape == (0, 256)
    lib = V.load()
    r1 = torch.zeros((4, 1536), dtype=torch.bfloat16, device="cuda")
    o1 = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    assert lib.mimo_patch_embed(4, r1.data_ptr(), 100, wd.data_ptr(), 0, None, V.MIMO_F32,
                                o1.data_ptr(), None) == V.MIMO_E_INVALID  # E not a multiple of 256
    assert lib.mimo_patch_embed(4, r1.data_ptr() + 2, 256, wd.data_ptr(), 0, None, V.MIMO_F32,
                                o1.data_ptr(), None) == V.MIMO_E_INVALID  # misaligned rows
    assert lib.mimo_patch_embed(4, r1.data_ptr(), 256, wd.data_ptr(), 2, None, V.MIMO_F32,
                                o1.data_ptr(), None) == V.MIMO_E_INVALID


def test_throughput_batch_sampled(V):
    """512 x 1024^2 stills, bf16 rows, E = 1280, full and folded: sampled rows
    against the oracle."""
    _say("throughput batch")
    b = W.throughput_512_1024()
    plan = V.plan_batch(b.shapes)
    src = V.processor.upload_sources(b.packed, plan)
    rows = V.preprocess(src, plan, mean=b.mean, std=b.std, out_dtype="bf16")["pixel_values"]
    del src
    w, bias = _weights(1280, seed=77)
    wd, bd = w.cuda(), bias.cuda()
    rng = np.random.default_rng(78)
    pick = np.unique(np.concatenate([[0, rows.shape[0] - 1], rng.integers(0, rows.shape[0], 62)]))
    sel = rows[torch.from_numpy(pick).cuda()]
    ref, s = _reference(sel, w, bias)
    out = V.patch_embed(rows, wd, bd, out_dtype="bf16")
    torch.cuda.synchronize()
    _assert_within(out[torch.from_numpy(pick).cuda()], ref, s, 1536, "bf16", what="full")
    del out
    out = V.patch_embed(rows, V.fold_patch_weights(wd), bd, out_dtype="bf16")
    torch.cuda.synchronize()
    _assert_within(out[torch.from_numpy(pick).cuda()], ref, s, 768, "bf16", extra=2.0 ** -8,
                   what="folded")
