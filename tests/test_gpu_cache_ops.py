"""GPU parity of the cache operations: bit-exact against the oracle, whole pool
compared (bytes outside the written slots / copied blocks must not change)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_186_amd as pa
from oracle import copy_blocks_ref, reshape_and_cache_ref
from gpu_support import DEV, announce, bits

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


def _rand(shape, dtype, gen):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32])
def test_reshape_and_cache_bit_exact(dtype, D, bs):
    announce(f"reshape_and_cache dtype={dtype} D={D} bs={bs}")
    gen = torch.Generator().manual_seed(D * 7 + bs)
    N, H, T = 24, 3, 40
    k = _rand((N, H, bs, D), dtype, gen)
    v = _rand((N, H, bs, D), dtype, gen)
    kn = _rand((T, H, D), dtype, gen)
    vn = _rand((T, H, D), dtype, gen)
    rng = np.random.default_rng(D + bs)
    slots = rng.choice(N * bs, size=T, replace=False).astype(np.int32)
    slots[3] = -1                        # padding token: no write
    slots[11] = N * bs + 5               # past the pool: the kernel skips it
    expect_slots = slots.copy()
    expect_slots[11] = -1
    rk, rv = reshape_and_cache_ref(k, v, kn, vn, expect_slots, bs)
    gk, gv = k.to(DEV), v.to(DEV)
    pa.pa_reshape_and_cache(gk, gv, kn.to(DEV), vn.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(gk.cpu()), bits(rk))
    assert torch.equal(bits(gv.cpu()), bits(rv))


def test_reshape_and_cache_decode_step_shape():
    """64 new tokens, 32 heads x 128 dims, block 32, fp16 (one continuous-batching step)."""
    announce("reshape_and_cache step shape")
    gen = torch.Generator().manual_seed(3)
    N, H, D, bs, T = 3000, 32, 128, 32, 64
    k = _rand((N, H, bs, D), torch.float16, gen)
    v = _rand((N, H, bs, D), torch.float16, gen)
    kn = _rand((T, H, D), torch.float16, gen)
    vn = _rand((T, H, D), torch.float16, gen)
    slots = np.random.default_rng(4).choice(N * bs, size=T, replace=False).astype(np.int32)
    rk, rv = reshape_and_cache_ref(k, v, kn, vn, slots, bs)
    gk, gv = k.to(DEV), v.to(DEV)
    pa.pa_reshape_and_cache(gk, gv, kn.to(DEV), vn.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(gk.cpu()), bits(rk)) and torch.equal(bits(gv.cpu()), bits(rv))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("D,bs,H", [(64, 16, 4), (128, 32, 3), (128, 16, 32)])
def test_copy_blocks_bit_exact(dtype, D, bs, H):
    announce(f"copy_blocks dtype={dtype} D={D} bs={bs} H={H}")
    gen = torch.Generator().manual_seed(H + D)
    N = 40
    k = _rand((N, H, bs, D), dtype, gen)
    v = _rand((N, H, bs, D), dtype, gen)
    k[5] = float("nan")                  # NaN payloads must survive the copy bit for bit
    others = [int(b) for b in np.random.default_rng(H).permutation(N) if b not in (5, 7)]
    srcs = [5, 5, 7] + others[:6]          # a source may feed several destinations
    dsts = others[6:15]                    # distinct, and never a source
    mapping = np.array(list(zip(srcs, dsts)), dtype=np.int32)
    bad = np.array([[N + 1, 0], [1, -3]], dtype=np.int32)       # skipped by the kernel
    rk, rv = copy_blocks_ref(k, v, mapping)
    gk, gv = k.to(DEV), v.to(DEV)
    pa.pa_copy_blocks(gk, gv, torch.from_numpy(np.concatenate([mapping, bad])).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(gk.cpu()), bits(rk))
    assert torch.equal(bits(gv.cpu()), bits(rv))


def test_copy_blocks_copy_on_write_shape():
    """31 pairs of 32-head x 16-row x 128-dim bf16 blocks (the shared-prefix fork)."""
    announce("copy_blocks shared-prefix shape")
    gen = torch.Generator().manual_seed(9)
    N, H, bs, D = 200, 32, 16, 128
    k = _rand((N, H, bs, D), torch.bfloat16, gen)
    v = _rand((N, H, bs, D), torch.bfloat16, gen)
    mapping = np.array([[63, 100 + i] for i in range(31)], dtype=np.int32)
    rk, rv = copy_blocks_ref(k, v, mapping)
    gk, gv = k.to(DEV), v.to(DEV)
    pa.pa_copy_blocks(gk, gv, torch.from_numpy(mapping).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(gk.cpu()), bits(rk)) and torch.equal(bits(gv.cpu()), bits(rv))
