"""Pins for the oracle's smart_resize geometry (CPU only).

What pins it, other than itself:
* the transformers Qwen2-VL smart_resize, which the processing page says
  gives identical geometry whenever the short side is at least the factor;
* the same library routine applied to the upscaled sides, for sub-factor
  images whose upscale is an integer (the upscale branch "scales the short
  side up to the factor first");
* hand-derived cases from the pages' statements (16x192, 8x500, ...);
* invariants: sides are multiples of the factor, the area bounds hold,
  transposition symmetry, identity on already-aligned sizes.
"""
import json
import os

import numpy as np
import pytest

import oracle

F = 32
MIN_PX = 8192
MAX_PX = 8388608
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _hf():
    mod = pytest.importorskip("transformers.models.qwen2_vl.image_processing_pil_qwen2_vl")
    return mod.smart_resize


def _hf_call(fn, h, w, factor=F, mn=MIN_PX, mx=MAX_PX):
    try:
        return fn(h, w, factor=factor, min_pixels=mn, max_pixels=mx)
    except ValueError:
        return "error"


def test_page_facts_match_defaults():
    facts = json.load(open(GOLDEN))
    assert oracle.PATCH == facts["patch_size"]["value"]
    assert oracle.TEMPORAL == facts["temporal_patch_size"]["value"]
    assert oracle.MERGE == facts["merge_size"]["value"]
    assert oracle.MIN_PIXELS == facts["min_pixels"]["value"]
    assert oracle.MAX_PIXELS == facts["max_pixels"]["value"]
    assert oracle.PATCH * oracle.MERGE == facts["factor"]["value"]
    # row length: 3 channels x temporal x patch x patch
    assert 3 * oracle.TEMPORAL * oracle.PATCH ** 2 == 1536


def test_full_factor_branch_matches_transformers_random():
    """Short side >= factor: identical to the Qwen2-VL routine, errors included."""
    fn = _hf()
    rng = np.random.default_rng(123)
    n = 40000
    # log-uniform sides from 32 to 40000, plus a band of extreme aspects
    hs = np.exp(rng.uniform(np.log(32), np.log(40000), n)).astype(np.int64)
    ws = np.exp(rng.uniform(np.log(32), np.log(40000), n)).astype(np.int64)
    hs[:2000] = rng.integers(32, 64, 2000)
    ws[:2000] = hs[:2000] * 200 + rng.integers(-40, 40, 2000)
    mismatches = []
    for h, w in zip(hs.tolist(), ws.tolist()):
        st, oh, ow = oracle.smart_resize_status(h, w)
        ref = _hf_call(fn, h, w)
        if ref == "error":
            ok = st == oracle.E_ASPECT
        else:
            ok = st == oracle.OK and (oh, ow) == tuple(ref)
        if not ok:
            mismatches.append((h, w, st, oh, ow, ref))
    assert not mismatches, mismatches[:10]


def test_full_factor_branch_ties_match_transformers():
    """Sides that are odd multiples of factor/2 are exact rounding ties."""
    fn = _hf()
    for k in range(1, 200, 3):
        for j in range(2, 120, 7):
            h = F * k + F // 2 if k > 0 else F
            w = F * j + F // 2
            if h < F or w < F:
                continue
            st, oh, ow = oracle.smart_resize_status(h, w)
            ref = _hf_call(fn, h, w)
            if ref == "error":
                assert st == oracle.E_ASPECT
            else:
                assert (oh, ow) == tuple(ref), (h, w)


def test_random_bounds_match_transformers_where_no_clamp():
    """Per-call min/max overrides.  Where the oracle rejects a degenerate
    shrink, the Qwen2-VL routine clamps that side to the factor instead."""
    fn = _hf()
    rng = np.random.default_rng(7)
    for _ in range(20000):
        h = int(rng.integers(32, 6000))
        w = int(rng.integers(32, 6000))
        mn = int(rng.integers(1, 50000))
        mx = int(rng.integers(mn, mn + 4_000_000))
        st, oh, ow = oracle.smart_resize_status(h, w, F, mn, mx)
        ref = _hf_call(fn, h, w, F, mn, mx)
        if ref == "error":
            assert st == oracle.E_ASPECT
        elif st == oracle.E_DEGENERATE:
            assert F in tuple(ref)
        else:
            assert st == oracle.OK and (oh, ow) == tuple(ref), (h, w, mn, mx)


def test_subfactor_equals_library_on_integer_upscale():
    """Upscale branch: the short side is scaled to the factor first, both
    sides by the same ratio; when that ratio gives integer sides the result
    is the library routine on the upscaled image (aspect kept <= 200)."""
    fn = _hf()
    checked = 0
    for s in range(1, F):
        for long_side in range(s, 201 * s, max(1, s // 3)):
            if (F * long_side) % s:
                continue
            up_long = F * long_side // s
            if up_long / F > 200:
                continue
            for h, w, uh, uw in ((s, long_side, F, up_long), (long_side, s, up_long, F)):
                if min(h, w) >= F:
                    continue
                got = oracle.smart_resize(h, w)
                ref = _hf_call(fn, uh, uw)
                assert ref != "error"
                assert got == tuple(ref), (h, w, got, ref)
                checked += 1
    assert checked > 1000


# Hand-derived cases.  Each comment derives the value from the pages' rules:
# round each side to the nearest multiple of 32 (ties to even, Python round),
# shrink if the area exceeds 8388608, grow if it is below 8192; a short side
# under 32 is first scaled to 32 with the long side scaled by the same ratio.
CASES = [
    # 200x300: round -> 192x288 (6.25 -> 6, 9.375 -> 9); area 55296 in bounds
    ((200, 300), (192, 288)),
    # 16x192: x2 -> 32x384, already multiples of 32, area 12288 in bounds.
    # The processing page says this case gets a different grid from HF.
    ((16, 192), (32, 384)),
    # 8x500: x4 -> 32x2000; 2000/32 = 62.5 is a tie, even -> 62 -> 1984
    ((8, 500), (32, 1984)),
    # 31x31: -> 32x32, area 1024 < 8192: beta = sqrt(8) = 2.83, ceil(2.83) = 3 -> 96
    ((31, 31), (96, 96)),
    # 1x64: x32 -> 32x2048, area 65536 in bounds
    ((1, 64), (32, 2048)),
    # 4000x6000: 125x187.5 -> 125x188 blocks = 24,064,000 px > max;
    # beta = sqrt(24e6/8388608) = 1.6914; 4000/beta/32 = 73.9 -> 73; 6000/beta/32 = 110.9 -> 110
    ((4000, 6000), (2336, 3520)),
    # multiples of 32 inside the bounds are unchanged
    ((1024, 1024), (1024, 1024)),
    ((480, 640), (480, 640)),
    # 1x8192: x32 -> 32x262144 = 8388608 exactly = max, accepted
    ((1, 8192), (32, 262144)),
]


@pytest.mark.parametrize("hw,expected", CASES)
def test_hand_derived_cases(hw, expected):
    assert oracle.smart_resize(*hw) == expected
    # transposition symmetry
    assert oracle.smart_resize(hw[1], hw[0]) == (expected[1], expected[0])


def test_page_subfactor_case_differs_from_hf():
    fn = _hf()
    facts = json.load(open(GOLDEN))
    h, w = facts["subfactor_case_differs_from_hf"]["value"]
    assert oracle.smart_resize(h, w) != tuple(fn(h, w, factor=F, min_pixels=MIN_PX,
                                                 max_pixels=MAX_PX))


def test_error_cases():
    # aspect 6401/32 > 200 on the full-factor branch
    assert oracle.smart_resize_status(32, 6401)[0] == oracle.E_ASPECT
    assert oracle.smart_resize_status(6401, 32)[0] == oracle.E_ASPECT
    # exactly 200 passes
    assert oracle.smart_resize_status(32, 6400)[0] == oracle.OK
    # sub-factor branch skips the aspect guard
    assert oracle.smart_resize_status(1, 4096)[0] == oracle.OK
    # 1x8193: upscaled area 32*262176 > max; shrink floors the short side to 0
    assert oracle.smart_resize_status(1, 8193)[0] == oracle.E_DEGENERATE
    for bad in ((0, 5), (5, 0), (-3, 10)):
        assert oracle.smart_resize_status(*bad)[0] == oracle.E_INVALID


def test_invariants_random_both_branches():
    rng = np.random.default_rng(11)
    for _ in range(20000):
        if rng.random() < 0.5:
            s = int(rng.integers(1, F))
            l = int(rng.integers(s, 8000))
        else:
            s = int(rng.integers(F, 3000))
            l = int(rng.integers(s, 200 * s + 1))
        h, w = (s, l) if rng.random() < 0.5 else (l, s)
        st, oh, ow = oracle.smart_resize_status(h, w)
        if st == oracle.E_DEGENERATE:
            # only reachable from the upscale branch with area above max
            assert min(h, w) < F and max(h, w) / min(h, w) > 8192
            continue
        assert st == oracle.OK
        assert oh % F == 0 and ow % F == 0 and oh >= F and ow >= F
        assert MIN_PX <= oh * ow <= MAX_PX
        assert oracle.smart_resize(w, h) == (ow, oh)


def test_counts_for_workloads():
    # one 300x200 image: 192x288 -> grid (1, 12, 18): 216 rows, 54 tokens
    assert oracle.image_grid(200, 300) == ((1, 12, 18), 216, 54)
    # 6000x4000 -> 3520x2336: grid (1, 146, 220): 32120 rows, 8030 tokens
    assert oracle.image_grid(4000, 6000) == ((1, 146, 220), 32120, 8030)
    # 1024x1024: grid (1, 64, 64): 4096 rows, 1024 tokens
    assert oracle.image_grid(1024, 1024) == ((1, 64, 64), 4096, 1024)
    # 16x192 -> 32x384: grid (1, 2, 24): 48 patches, 12 tokens
    assert oracle.image_grid(16, 192) == ((1, 2, 24), 48, 12)
