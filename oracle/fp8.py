"""Float64 CPU oracle for an 8-bit floating-point KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

The pages name quantization only as future work (page "mlx-paged-attention:
Bringing vLLM-level High Throughput Inference to Apple Silicon", future
plans); they fix no format, no scale granularity and no rounding.  The
readings taken here:

* formats: the two 8-bit formats of the OCP 8-bit floating point
  specification (OFP8): E4M3 — 4 exponent bits, bias 7, 3 mantissa bits, no
  infinities, S.1111.111 is NaN, largest finite 448 — and E5M2 — 5 exponent
  bits, bias 15, 2 mantissa bits, IEEE-style infinities and NaNs, largest
  finite 57344.  Both have subnormals.
* scales: one float32 scale per (physical block, head) for K and one for V,
  supplied by the caller; a cached code c in block b, head h stands for
  scale[b, h] * value(c).
* quantization of a new token's element x (its float32 value): y is the
  float32 quotient x / scale (IEEE single-precision division, correctly
  rounded), then the code of the nearest finite value to |y| — ties to the
  code with an even mantissa — with the sign bit of y; |y| beyond the largest
  finite value saturates to it (so does an infinity); NaN maps to the code
  0x7F.
* decode over such a cache is the float64 attention of ``decode_ref`` applied
  to the dequantized pools: the method's mathematics is unchanged, only the
  stored values are.

Pin status (tests/test_oracle_fp8.py): ``fp8_values`` — pinned against
torch's float8_e4m3fn / float8_e5m2 decoding of all 256 codes and against
hand-derived codes (tests/golden/fp8_codes.json); ``quantize_fp8_ref`` —
pinned against torch's rounding casts for in-range values, hand-derived tie,
subnormal, saturation, zero and NaN cases, and the round trip of every code;
``decode_fp8_ref`` — pinned by scale invariants (scaling every K scale equals
scaling the softmax scale; scaling every V scale scales the output) and by
agreement with ``decode_ref`` on pools whose values are exactly
representable; ``reshape_and_cache_fp8_ref`` / ``copy_blocks_fp8_ref`` —
pinned like their unquantized counterparts plus code-level checks.
"""

from __future__ import annotations

import numpy as np
import torch

from .paged_attention import _as_int, decode_ref

# (exponent bits, mantissa bits, bias, IEEE-style specials?)
_FORMATS = {
    "e4m3": (4, 3, 7, False),
    "e5m2": (5, 2, 15, True),
}
NAN_CODE = 0x7F


def fp8_values(fmt: str) -> np.ndarray:
    """Value of each of the 256 codes of ``fmt`` ("e4m3" or "e5m2"), float64.

    Code bits: sign | exponent (E bits) | mantissa (M bits).  Exponent field 0
    holds zero and the subnormals m * 2^(1 - bias - M); otherwise the value is
    (1 + m / 2^M) * 2^(e - bias).  E4M3 spends only its all-ones pattern
    (exponent and mantissa all ones) on NaN; E5M2 reserves its top exponent for
    infinity (mantissa 0) and NaN (otherwise).
    """
    E, M, bias, ieee = _FORMATS[fmt]
    vals = np.empty(256, dtype=np.float64)
    top = (1 << E) - 1
    for c in range(256):
        s = -1.0 if c >> 7 else 1.0
        e = (c >> M) & top
        m = c & ((1 << M) - 1)
        if ieee and e == top:
            vals[c] = s * np.inf if m == 0 else np.nan
        elif not ieee and e == top and m == (1 << M) - 1:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** (1 - bias - M)
        else:
            vals[c] = s * (1.0 + m / (1 << M)) * 2.0 ** (e - bias)
    return vals


def _finite_magnitudes(fmt: str):
    """(codes, values) of the non-negative finite codes, in code order."""
    vals = fp8_values(fmt)
    codes = np.array([c for c in range(128) if np.isfinite(vals[c])], dtype=np.int64)
    return codes, vals[codes]


def quantize_fp8_ref(x, scale, fmt: str) -> np.ndarray:
    """Codes (uint8) of x / scale, elementwise; ``scale`` broadcasts against x.

    y = float32(x) / float32(scale) in float32; the magnitude code is the
    finite code nearest to |y| (brute force over all of them), ties broken
    towards the even code; the sign bit is y's; NaN gives NAN_CODE.
    """
    xf = x.detach().cpu().to(torch.float32).numpy() if isinstance(x, torch.Tensor) \
        else np.asarray(x, dtype=np.float32)
    sf = scale.detach().cpu().to(torch.float32).numpy() if isinstance(scale, torch.Tensor) \
        else np.asarray(scale, dtype=np.float32)
    y = (xf / sf).astype(np.float32)
    flat = y.reshape(-1).astype(np.float64)
    codes, mags = _finite_magnitudes(fmt)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 4096
    for i in range(0, flat.size, step):
        a = np.abs(flat[i:i + step])
        with np.errstate(invalid="ignore"):
            dist = np.abs(a[:, None] - mags[None, :])   # inf - finite = inf
        best = dist.min(axis=1, keepdims=True)
        tied = dist == best
        # among the nearest codes prefer an even one (even mantissa); when the
        # nearest is unique this picks it
        even = tied & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
        mag_code = codes[pick]
        # saturation: beyond the largest finite value (an infinity included)
        mag_code = np.where(a > mags[-1], codes[-1], mag_code)
        c = mag_code | np.where(np.signbit(flat[i:i + step]), 0x80, 0)
        c = np.where(np.isnan(flat[i:i + step]), NAN_CODE, c)
        out[i:i + step] = c.astype(np.uint8)
    return out.reshape(y.shape)


def dequant_ref(codes, scales, fmt: str) -> np.ndarray:
    """Float64 values of a code pool [num_blocks, H, bs, D] with scales [num_blocks, H]."""
    c = _as_int(codes)
    s = scales.detach().cpu().to(torch.float64).numpy() if isinstance(scales, torch.Tensor) \
        else np.asarray(scales, dtype=np.float64)
    return fp8_values(fmt)[c] * s[:, :, None, None]


def decode_fp8_ref(q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                   scale: float, block_size: int, fmt: str) -> np.ndarray:
    """Paged decode attention over an fp8 cache: ``decode_ref`` on the
    dequantized pools (the attention mathematics is that of PagedAttention原理
    §3.2 / closing remarks of §3.4; only the stored values change)."""
    return decode_ref(q, dequant_ref(k_codes, k_scales, fmt), dequant_ref(v_codes, v_scales, fmt),
                      block_tables, context_lens, scale, block_size)


def reshape_and_cache_fp8_ref(k_codes, v_codes, k_scales, v_scales, k_new, v_new,
                              slot_mapping, block_size: int, fmt: str):
    """Quantize each new token's K/V with its (block, head) scales and write
    the codes into its slot (slot n: row n % block_size of block
    n // block_size, PagedAttention原理 §3.3.2); negative slots write nothing.
    Returns new code pools (uint8 numpy); inputs are not modified."""
    k_out = np.array(_as_int(k_codes), dtype=np.uint8)
    v_out = np.array(_as_int(v_codes), dtype=np.uint8)
    ks = k_scales.detach().cpu().to(torch.float32).numpy() if isinstance(k_scales, torch.Tensor) \
        else np.asarray(k_scales, dtype=np.float32)
    vs = v_scales.detach().cpu().to(torch.float32).numpy() if isinstance(v_scales, torch.Tensor) \
        else np.asarray(v_scales, dtype=np.float32)
    for i, slot in enumerate(_as_int(slot_mapping)):
        if slot < 0:
            continue
        block, row = divmod(int(slot), block_size)
        k_out[block, :, row, :] = quantize_fp8_ref(k_new[i], ks[block][:, None], fmt)
        v_out[block, :, row, :] = quantize_fp8_ref(v_new[i], vs[block][:, None], fmt)
    return k_out, v_out


def copy_blocks_fp8_ref(k_codes, v_codes, k_scales, v_scales, block_mapping):
    """Copy-on-write for an fp8 cache: whole blocks of codes and their
    per-head scales, src -> dst (mlx-paged-attention, core feature 2;
    PagedAttentionMetal, section 块表管理).  Returns new arrays."""
    kc, vc = np.array(_as_int(k_codes), dtype=np.uint8), np.array(_as_int(v_codes), dtype=np.uint8)
    ks = np.array(k_scales.cpu().numpy() if isinstance(k_scales, torch.Tensor) else k_scales,
                  dtype=np.float32)
    vs = np.array(v_scales.cpu().numpy() if isinstance(v_scales, torch.Tensor) else v_scales,
                  dtype=np.float32)
    kc0, vc0, ks0, vs0 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    for src, dst in _as_int(block_mapping).reshape(-1, 2):
        kc[dst], vc[dst], ks[dst], vs[dst] = kc0[src], vc0[src], ks0[src], vs0[src]
    return kc, vc, ks, vs
