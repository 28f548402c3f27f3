"""Plant plausible mistakes in copies of the fp8 oracle and check that its pins
catch every one (CPU only).

``_pins`` runs the checks of tests/test_oracle_fp8.py (hand-derived codes,
torch's float8 decoding and casts, round trips) against a (values,
quantize) pair passed in; the real oracle must pass and each mutant fail.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle.fp8 as of8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_codes.json")
TORCH_DTYPE = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _pins(values_fn, quant_fn) -> bool:
    g = json.load(open(GOLDEN))
    with np.errstate(all="ignore"):
        for fmt in ("e4m3", "e5m2"):
            vals = values_fn(fmt)
            for code, want in g["values"][fmt]:
                w = float(want)
                got = vals[int(code, 16)]
                if np.isnan(w) != np.isnan(got) or (not np.isnan(w) and (got != w or np.signbit(got) != np.signbit(w))):
                    return False
            lib = torch.arange(256, dtype=torch.uint8).view(TORCH_DTYPE[fmt]).to(torch.float64).numpy()
            if not np.array_equal(np.isnan(lib), np.isnan(vals)):
                return False
            ok = ~np.isnan(lib)
            if not np.array_equal(lib[ok], vals[ok]):
                return False
            for x, want in g["quantize"][fmt]:
                if int(quant_fn(np.array([float(x)], np.float32), 1.0, fmt)[0]) != int(want, 16):
                    return False
            rng = np.random.default_rng(3)
            mx = 448.0 if fmt == "e4m3" else 57344.0
            x = np.concatenate([rng.standard_normal(3000) * 4,
                                np.exp(rng.uniform(np.log(1e-9), np.log(mx), 3000))]).astype(np.float32)
            x = x[np.abs(x) <= mx]
            if not np.array_equal(torch.from_numpy(x).to(TORCH_DTYPE[fmt]).view(torch.uint8).numpy(),
                                  quant_fn(x, 1.0, fmt)):
                return False
            # division happens in float32: a quotient that rounds onto a tie
            if int(quant_fn(np.array([2.700284004211426], np.float32), np.float32(2.273923397064209),
                            "e4m3")[0]) != 0x3A:
                return False
    return True


def _values(bias_delta=0, sub_exp_delta=0, nan_all_top=False):
    def fn(fmt):
        E, M, bias, ieee = of8._FORMATS[fmt]
        bias += bias_delta
        vals = np.empty(256)
        top = (1 << E) - 1
        for c in range(256):
            s = -1.0 if c >> 7 else 1.0
            e = (c >> M) & top
            m = c & ((1 << M) - 1)
            if ieee and e == top:
                vals[c] = s * np.inf if m == 0 else np.nan
            elif not ieee and e == top and (nan_all_top or m == (1 << M) - 1):
                vals[c] = np.nan
            elif e == 0:
                vals[c] = s * m * 2.0 ** (1 - bias - M + sub_exp_delta)
            else:
                vals[c] = s * (1.0 + m / (1 << M)) * 2.0 ** (e - bias)
        return vals
    return fn


def _quant(values_fn=of8.fp8_values, ties="even", saturate=True, divide64=False, keep_sign=True,
           truncate=False):
    def fn(x, scale, fmt):
        xf = np.asarray(x, dtype=np.float32)
        sf = np.asarray(scale, dtype=np.float32)
        y = (xf.astype(np.float64) / sf) if divide64 else (xf / sf).astype(np.float32)
        flat = np.asarray(y, dtype=np.float64).reshape(-1)
        vals = values_fn(fmt)
        codes = np.array([c for c in range(128) if np.isfinite(vals[c])])
        mags = vals[codes]
        out = []
        for v in flat:
            if np.isnan(v):
                out.append(of8.NAN_CODE)
                continue
            a = abs(v)
            if truncate:
                idx = int(np.searchsorted(mags, a, side="right") - 1)
            else:
                d = np.abs(mags - a)
                tied = np.nonzero(d == d.min())[0]
                want = 0 if ties == "even" else 1
                pick = [i for i in tied if codes[i] % 2 == want]
                idx = pick[0] if pick else tied[0]
            c = int(codes[idx])
            if a > mags[-1]:
                c = int(codes[-1]) if saturate else of8.NAN_CODE
            if keep_sign and np.signbit(v) and not (not saturate and a > mags[-1]):
                c |= 0x80
            out.append(c)
        return np.array(out, dtype=np.uint8).reshape(np.shape(y))
    return fn


def test_the_oracle_passes_its_own_pins():
    assert _pins(of8.fp8_values, of8.quantize_fp8_ref)
    assert _pins(of8.fp8_values, _quant())  # the mutant builder without a slip


@pytest.mark.parametrize("name,values_fn,quant_fn", [
    ("exponent bias one too large", _values(bias_delta=1), None),
    ("subnormals a binade off", _values(sub_exp_delta=-1), None),
    ("whole top binade NaN in E4M3", _values(nan_all_top=True), None),
    ("ties to odd", None, _quant(ties="odd")),
    ("overflow to NaN instead of saturating", None, _quant(saturate=False)),
    ("division in float64", None, _quant(divide64=True)),
    ("sign dropped", None, _quant(keep_sign=False)),
    ("truncation instead of rounding", None, _quant(truncate=True)),
])
def test_each_mutant_is_caught(name, values_fn, quant_fn):
    v = values_fn or of8.fp8_values
    q = quant_fn or _quant(values_fn=v)
    assert not _pins(v, q), name
