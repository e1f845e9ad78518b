"""GPU parity for the fused pixel path + patch embedding (mimo_pixel_embed,
mimo_prepare_pixel_embed) against the oracle.

The kernel computes sum_k xh_k * Wt[e][k] + bias'[e] over the 768 values of a
still patch in (py, px, c) order, where x are the resized 0-255 values,
xh = bf16(x) (exact for an image that is not resampled), Wt = bf16(s_c *
(W0 + W1)) with s_c = float32(1 / std255[c]), and bias' = bias - sum_k
mean255[c] * Wt[e][k].  That equals the Conv3d over the standardised rows up
to the roundings below.

Bars, derived from the arithmetic:

* Prepared weights: Wt bit for bit against a CPU restatement of its
  definition; bias' within 2^-23 |bias'| of its float64 value.
* (1) Tight: against the float64 value of the same formula on the oracle's
  own resized pixels (the resize is the oracle's float32 arithmetic, which
  the pixel kernel matches bit for bit).  bf16 x bf16 products are exact in
  float32, so the kernel's error is the float32 sum's, K 2^-24 S1 with
  S1 = sum |xh| |Wt|, the rounding of bias' (2^-24 |bias'|) and of the output.
* (2) Against the pages' definition: the oracle's standardised rows, rounded
  to bf16, through the full Conv3d (K = 1536) in float64.  On top of (1):
  the rounding of the oracle's rows and of Wt, each 2^-8 relative to a
  standardised value (bias' is formed from the rounded Wt, so Wt's rounding
  multiplies x - mean, not x), giving 2^-7 S_a with S_a = sum |a| |W|; for a
  resampled image the rounding of x to bf16, 2^-8 S1; float32 reciprocal and
  products, below 2^-20 of either sum.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-pixel-embed]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _weights(e, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    w = (torch.randn((e, 1536), generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(e, generator=g) * 0.1).float() if bias else None
    return w, b


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _prepared_reference(w, bias, m255, s255):
    """Wt (bf16 bits, [E, 768] in (py, px, c) order) and bias' (float64)."""
    e = w.shape[0]
    w4 = w.float().numpy().reshape(e, 3, 2, 256)
    summed = w4[:, :, 0] + w4[:, :, 1]                                   # float32
    inv = np.float32(1.0) / np.asarray(s255, dtype=np.float64)
    inv = inv.astype(np.float32)                                         # float32(1 / std255)
    scaled = (summed * inv[None, :, None]).astype(np.float32)           # float32 products
    scaled = np.ascontiguousarray(scaled.transpose(0, 2, 1)).reshape(e, 768)  # (pixel, c)
    bits = oracle.to_bf16_bits(scaled)
    wt = _bf16_to_f32(bits).astype(np.float64)
    mean_k = np.tile(np.asarray(m255, dtype=np.float64), 256)
    b = np.zeros(e) if bias is None else bias.double().numpy()
    return bits, b - wt @ mean_k


def _resized_patches(batch, plan, i):
    """The oracle's resized 0-255 values of image i, one row per patch in
    merge-block order, values in (py, px, c) order."""
    img = batch.image(i)
    rgb = oracle.flatten_rgba(img) if img.shape[2] == 4 else img
    planar = np.ascontiguousarray(rgb.transpose(2, 0, 1)).astype(np.float32)
    d = plan.desc[i]
    dh, dw = int(d["dst_h"]), int(d["dst_w"])
    x = oracle.resize_bilinear(planar, dh, dw)                 # [3, dh, dw]
    t = x.transpose(1, 2, 0).reshape(dh // 32, 2, 16, dw // 32, 2, 16, 3)
    t = t.transpose(0, 3, 1, 4, 2, 5, 6)                       # br, bc, mh, mw, py, px, c
    return np.ascontiguousarray(t).reshape(-1, 768)


def _run(V, batch, e, out_dtype, seed, bias=True, rows_pick=None):
    plan = V.plan_batch(batch.shapes)
    src = V.processor.upload_sources(batch.packed, plan)
    w, b = _weights(e, seed, bias)
    wp, bp = V.prepare_pixel_embed_weights(w.cuda(), None if b is None else b.cuda(), batch.mean, batch.std)
    before = V.dispatch_count()
    out = V.embed_pixels(src, plan, wp, bp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert V.dispatch_count() == before + 1
    m255, s255 = oracle.stats255(batch.mean, batch.std)
    bits, bias_ref = _prepared_reference(w, b, m255, s255)
    have = wp.cpu().view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(have, bits), "prepared weight differs from its definition"
    bdev = bp.cpu().double().numpy()
    assert np.all(np.abs(bdev - bias_ref) <= 2.0 ** -23 * np.abs(bias_ref) + 1e-12), "prepared bias"
    return plan, out, w, b, bits, bias_ref, m255, s255


def _check(V, batch, plan, out, w, b, bits, bias_ref, m255, s255, out_dtype, images=None, rows=None):
    wt = _bf16_to_f32(bits)
    got = out.float().cpu().numpy().astype(np.float64) if rows is None else None
    out_rel = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -24
    for i in (range(len(batch)) if images is None else images):
        d = plan.desc[i]
        r0, r1 = int(d["row_offset"]), int(d["row_offset"] + d["rows"])
        x = _resized_patches(batch, plan, i)
        xh = _bf16_to_f32(oracle.to_bf16_bits(x))
        resampled = (int(d["dst_h"]), int(d["dst_w"])) != batch.shapes[i][:2]
        sel = np.arange(r1 - r0) if rows is None else rows[i]
        g = got[r0 + sel] if rows is None else out[torch.from_numpy(r0 + sel).cuda()].float().cpu().numpy()
        xh = xh[sel]
        ref1 = oracle.patch_embed(xh, wt) + bias_ref[None, :]
        s1 = oracle.patch_embed(np.abs(xh), np.abs(wt))
        tol1 = 768 * 2.0 ** -24 * s1 + 2.0 ** -23 * np.abs(bias_ref)[None, :] + (out_rel + 2.0 ** -24) * np.abs(ref1)
        err1 = np.abs(g - ref1)
        assert np.isfinite(g).all(), i
        assert (err1 <= tol1).all(), ("same-formula bound", i, float((err1 / tol1).max()))
        rows_o = oracle.preprocess_image(batch.image(i), int(d["dst_h"]), int(d["dst_w"]), m255, s255)[sel]
        a = _bf16_to_f32(oracle.to_bf16_bits(rows_o))
        wf = w.float().numpy()
        ref2 = oracle.patch_embed(a, wf, None if b is None else b.numpy())
        sa = oracle.patch_embed(np.abs(a), np.abs(wf))
        tol2 = ((2.0 ** -7 + 2.0 ** -20) * sa + ((2.0 ** -8 if resampled else 0.0) + 768 * 2.0 ** -24 + 2.0 ** -20) * s1
                + 2.0 ** -23 * np.abs(bias_ref)[None, :] + (out_rel + 2.0 ** -24) * np.abs(ref2))
        err2 = np.abs(g - ref2)
        assert (err2 <= tol2).all(), ("Conv3d bound", i, float((err2 / tol2).max()))


IDENTITY = [(96, 96, 3), (64, 128, 3), (512, 512, 3), (32, 256, 3), (96, 160, 3), (128, 64, 3)]
GENERAL = [(200, 300, 3), (45, 77, 4), (513, 257, 3), (1, 64, 3), (64, 128, 4), (96, 96, 3)]


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("e", [256, 1280])
def test_identity_rgb_batch(V, e, out_dtype):
    _say("no-resample batch", e, out_dtype)
    batch = W.uniform_images(IDENTITY, seed=501)
    args = _run(V, batch, e, out_dtype, seed=502)
    plan = args[0]
    assert plan.total_rows % 256 != 0 and all(
        (int(d["dst_h"]), int(d["dst_w"])) == s[:2] for d, s in zip(plan.desc, batch.shapes))
    _check(V, batch, *args, out_dtype)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_general_batch_resized_and_rgba(V, out_dtype):
    _say("resampled / RGBA batch", out_dtype)
    batch = W.uniform_images([(h, w, 3) for (h, w, _) in GENERAL], seed=503)
    # RGBA items: uniform bytes including alpha (some fully transparent)
    rgba = W.uniform_images(GENERAL, seed=504)
    args = _run(V, rgba, 1280, out_dtype, seed=505, bias=False)
    _check(V, rgba, *args, out_dtype)
    del batch


def test_throughput_batch_sampled(V):
    """512 x 1024^2 stills, E = 1280, bf16: sampled rows of both ends and
    the middle of every image range against bound (1) and (2)."""
    _say("throughput batch")
    batch = W.throughput_512_1024()
    plan, out, w, b, bits, bias_ref, m255, s255 = _run(V, batch, 1280, "bf16", seed=506)
    rng = np.random.default_rng(507)
    images = [0, 1, 255, 511]
    picks = {i: np.unique(np.concatenate([[0, 4095], rng.integers(0, 4096, 14)])) for i in images}
    _check(V, batch, plan, out, w, b, bits, bias_ref, m255, s255, "bf16", images=images, rows=picks)


def test_clips_refused(V):
    _say("clips refused")
    b = W.media_batch([(1, 64, 64, 3), (3, 64, 64, 3)], seed=508)
    plan = V.plan_media(b.items)
    src = V.processor.upload_sources(b.packed, plan)
    w, bias = _weights(256, seed=509)
    wp, bp = V.prepare_pixel_embed_weights(w.cuda(), bias.cuda(), b.mean, b.std)
    with pytest.raises(V.MimoError) as e:
        V.embed_pixels(src, plan, wp, bp)
    assert e.value.code == V.MIMO_E_UNSUPPORTED
