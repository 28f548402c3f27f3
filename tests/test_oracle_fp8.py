"""Pins of the fp8 KV-cache oracle (oracle/fp8.py) to facts outside it:
hand-derived codes (tests/golden/fp8_codes.json), torch's own float8
decoding and rounding casts, round trips and scale invariants."""

from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from oracle import (copy_blocks_fp8_ref, decode_fp8_ref, decode_ref, dequant_ref, fp8_values,
                    quantize_fp8_ref, reshape_and_cache_fp8_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_codes.json")
TORCH_DTYPE = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
MAX_FINITE = {"e4m3": 448.0, "e5m2": 57344.0}


def _num(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_code_values_match_hand_derivation(golden, fmt):
    vals = fp8_values(fmt)
    for code, want in golden["values"][fmt]:
        got = vals[int(code, 16)]
        w = _num(want)
        if np.isnan(w):
            assert np.isnan(got), code
        else:
            assert got == w and np.signbit(got) == np.signbit(w), (code, got, w)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_code_values_match_torch_float8_decoding(fmt):
    """All 256 codes against torch's float8 dtypes (a library decoding)."""
    lib = torch.arange(256, dtype=torch.uint8).view(TORCH_DTYPE[fmt]).to(torch.float64).numpy()
    mine = fp8_values(fmt)
    assert np.array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(mine[ok]))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_hand_cases(golden, fmt):
    for x, want in golden["quantize"][fmt]:
        got = int(quantize_fp8_ref(np.array([_num(x)], dtype=np.float32), 1.0, fmt)[0])
        assert got == int(want, 16), (x, hex(got), want)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_matches_torch_cast_in_range(fmt):
    """Inside the finite range torch's float -> float8 cast rounds to nearest,
    ties to even, exactly as the reading; compare on many values of every
    magnitude, including subnormals and exact ties."""
    rng = np.random.default_rng(3)
    mx = MAX_FINITE[fmt]
    x = np.concatenate([
        rng.standard_normal(20000) * 4,
        rng.uniform(-mx, mx, 5000),
        np.exp(rng.uniform(np.log(1e-9), np.log(mx), 20000)) * rng.choice([-1, 1], 20000),
        # midpoints between neighbouring codes: exact ties
        (fp8_values(fmt)[1:0x7B] + fp8_values(fmt)[2:0x7C]) / 2,
    ]).astype(np.float32)
    x = x[np.abs(x) <= mx]
    lib = torch.from_numpy(x).to(TORCH_DTYPE[fmt]).view(torch.uint8).numpy()
    mine = quantize_fp8_ref(x, 1.0, fmt)
    bad = np.nonzero(lib != mine)[0]
    assert bad.size == 0, [(float(x[i]), hex(lib[i]), hex(mine[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_code_round_trips(fmt):
    vals = fp8_values(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(vals[c])])
    back = quantize_fp8_ref(vals[codes].astype(np.float32), 1.0, fmt)
    assert np.array_equal(back, codes.astype(np.uint8))


# float32 operands whose exact quotient lies just below 1.1875 (the midpoint
# between e4m3 codes 0x39 = 1.125 and 0x3A = 1.25) while their float32
# quotient is exactly 1.1875 (found by search, checked with exact fractions)
TIE_X, TIE_S = 2.700284004211426, 2.273923397064209


def test_quantize_divides_in_float32_before_rounding():
    """y = fp32(x / s) is what gets rounded: here it is exactly the midpoint,
    so the tie goes to the even code 0x3A, although the exact quotient is
    below the midpoint (nearest code 0x39)."""
    from fractions import Fraction
    x, s = np.float32(TIE_X), np.float32(TIE_S)
    assert np.float32(x / s) == np.float32(1.1875)
    assert Fraction(float(x)) / Fraction(float(s)) < Fraction(19, 16)
    assert int(quantize_fp8_ref(np.array([x]), s, "e4m3")[0]) == 0x3A
    # per-element scales broadcast
    x = np.full((2, 3), 2.0, np.float32)
    s = np.array([[1.0], [2.0]], np.float32)
    got = quantize_fp8_ref(x, s, "e4m3")
    assert got[0].tolist() == [0x40] * 3 and got[1].tolist() == [0x38] * 3


def _fp8_cache(rng, nb, H, bs, D, fmt):
    codes_k = rng.integers(0, 256, size=(nb, H, bs, D), dtype=np.uint8)
    codes_v = rng.integers(0, 256, size=(nb, H, bs, D), dtype=np.uint8)
    vals = fp8_values(fmt)
    # no NaN/inf codes in referenced data
    for c in (codes_k, codes_v):
        bad = ~np.isfinite(vals[c])
        c[bad] = 0x30
    ks = rng.uniform(0.01, 0.2, size=(nb, H)).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, size=(nb, H)).astype(np.float32)
    return codes_k, codes_v, ks, vs


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_scale_invariants(fmt):
    """Multiplying every K scale by c equals multiplying the softmax scale by
    c; multiplying every V scale by c multiplies the output by c."""
    rng = np.random.default_rng(7)
    nb, H, bs, D = 10, 2, 16, 8
    kc, vc, ks, vs = _fp8_cache(rng, nb, H, bs, D, fmt)
    q = rng.standard_normal((3, H, D))
    tables = np.array([[3, 1, 7], [0, 9, -1], [5, -1, -1]], dtype=np.int32)
    lens = np.array([40, 20, 9], dtype=np.int32)
    base = decode_fp8_ref(q, kc, vc, ks, vs, tables, lens, 0.7, bs, fmt)
    k2 = decode_fp8_ref(q, kc, vc, ks * np.float32(4), vs, tables, lens, 0.7, bs, fmt)
    assert np.allclose(k2, decode_fp8_ref(q, kc, vc, ks, vs, tables, lens, 2.8, bs, fmt), rtol=1e-12, atol=1e-12)
    v2 = decode_fp8_ref(q, kc, vc, ks, vs * np.float32(0.5), tables, lens, 0.7, bs, fmt)
    assert np.allclose(v2, base * 0.5, rtol=1e-12, atol=1e-12)


def test_decode_equals_unquantized_decode_on_representable_values():
    """A cache whose values are exactly representable (small integers times a
    power-of-two scale) decodes to the unquantized attention of those values."""
    rng = np.random.default_rng(8)
    nb, H, bs, D = 6, 2, 16, 4
    kv = rng.integers(-6, 7, size=(2, nb, H, bs, D)).astype(np.float32)
    scale_k = np.full((nb, H), 0.25, np.float32)
    scale_v = np.full((nb, H), 2.0, np.float32)
    kc = quantize_fp8_ref(kv[0], scale_k[:, :, None, None], "e4m3")
    vc = quantize_fp8_ref(kv[1], scale_v[:, :, None, None], "e4m3")
    assert np.array_equal(dequant_ref(kc, scale_k, "e4m3"), kv[0])
    q = rng.standard_normal((2, H, D))
    tables = np.array([[4, 2, 0], [1, 5, -1]], dtype=np.int32)
    lens = np.array([41, 17], dtype=np.int32)
    got = decode_fp8_ref(q, kc, vc, scale_k, scale_v, tables, lens, 0.5, bs, "e4m3")
    want = decode_ref(q, kv[0], kv[1], tables, lens, 0.5, bs)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_reshape_and_cache_fp8_writes_quantized_codes_only_into_slots(fmt):
    rng = np.random.default_rng(9)
    nb, H, bs, D = 5, 3, 16, 8
    kc, vc, ks, vs = _fp8_cache(rng, nb, H, bs, D, fmt)
    k_new = torch.randn(4, H, D, dtype=torch.float16)
    v_new = torch.randn(4, H, D, dtype=torch.float16)
    slots = np.array([3 * bs + 5, -1, 0, 4 * bs + 15], dtype=np.int32)
    k2, v2 = reshape_and_cache_fp8_ref(kc, vc, ks, vs, k_new, v_new, slots, bs, fmt)
    touched = np.zeros((nb, bs), bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, r = divmod(int(slot), bs)
        touched[b, r] = True
        for h in range(H):
            # each code is the nearest representable value of x / scale
            y = (k_new[i, h].float().numpy() / ks[b, h]).astype(np.float32)
            got = fp8_values(fmt)[k2[b, h, r]]
            finite = fp8_values(fmt)[np.isfinite(fp8_values(fmt))]
            assert np.all(np.abs(got - y) <= np.abs(finite[None, :] - y[:, None]).min(axis=1))
            assert np.array_equal(v2[b, h, r], quantize_fp8_ref(v_new[i, h], vs[b, h], fmt))
    for b in range(nb):
        for r in range(bs):
            if not touched[b, r]:
                assert np.array_equal(k2[b, :, r], kc[b, :, r]) and np.array_equal(v2[b, :, r], vc[b, :, r])


def test_copy_blocks_fp8_copies_codes_and_scales():
    rng = np.random.default_rng(10)
    kc, vc, ks, vs = _fp8_cache(rng, 6, 2, 16, 8, "e4m3")
    mapping = np.array([[1, 4], [2, 5]], dtype=np.int32)
    k2, v2, ks2, vs2 = copy_blocks_fp8_ref(kc, vc, ks, vs, mapping)
    for src, dst in mapping:
        assert np.array_equal(k2[dst], kc[src]) and np.array_equal(v2[dst], vc[src])
        assert ks2[dst].tolist() == ks[src].tolist() and vs2[dst].tolist() == vs[src].tolist()
    for b in (0, 1, 2, 3):
        assert np.array_equal(k2[b], kc[b]) and ks2[b].tolist() == ks[b].tolist()
