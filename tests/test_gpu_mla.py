"""GPU parity of decode over a multi-head latent cache (pa_decode_mla, the
matrix-core kernel with 576-element key rows whose first 512 elements are the
values) against the float64 oracle (mla_decode_ref), through the C ABI:
head counts that fill, half-fill and overflow 16-row tiles, ragged and empty
contexts, both block sizes, fp16 and bf16, the default split and explicit
partitions, NaN-poisoned unreferenced blocks and tail slots."""

import numpy as np
import pytest
import torch

import paged_kv_cache_186_amd as pa
from paged_kv_cache_186_amd import workloads as W
from oracle import mla_decode_ref
from gpu_support import DEV, announce, assert_close

pytestmark = pytest.mark.gpu

QK, V = pa.binding.MLA_QK_DIM, pa.binding.MLA_V_DIM


class LatentCase:
    def __init__(self, lens, H, bs, dtype, seed):
        rng = np.random.default_rng(seed)
        nb = sum(-(-L // bs) for L in lens) + len(lens) + 3
        m = W.BlockManager(nb, bs, free_order=rng.permutation(nb).tolist())
        for s, L in enumerate(lens):
            m.allocate(s)
            m.append_slots(s, L)
        self.lens = np.array(lens, dtype=np.int32)
        width = max(1, max(-(-L // bs) for L in lens))
        self.tables = m.block_tables(list(range(len(lens))), width)
        g = torch.Generator(device=DEV)
        g.manual_seed(seed)
        self.pool = W.normal((nb, bs, QK), dtype, DEV, g)
        self.q = W.normal((len(lens), H, QK), dtype, DEV, g)
        used = np.zeros(nb, bool)
        for s, L in enumerate(lens):
            used[self.tables[s, :-(-L // bs)]] = True
            if L % bs:   # tail slots of the last block
                self.pool[int(self.tables[s, L // bs]), L % bs:] = float("nan")
        self.pool[torch.from_numpy(np.nonzero(~used)[0]).to(DEV)] = float("nan")
        self.bs = bs
        self.scale = 1.0 / np.sqrt(192.0)   # DeepSeek's 128 + 64 query/key width

    def run(self, partition_size=0, tables=None):
        out = torch.empty((self.q.shape[0], self.q.shape[1], V), dtype=self.q.dtype, device=DEV)
        bt = torch.from_numpy(self.tables).to(DEV) if tables is None else tables
        pa.pa_decode_mla(out, self.q, self.pool, bt, torch.from_numpy(self.lens).to(DEV), self.scale, self.bs,
                         partition_size=partition_size)
        torch.cuda.synchronize()
        return out

    def oracle(self):
        return mla_decode_ref(self.q.cpu(), self.pool.cpu(), self.tables, self.lens, self.scale, self.bs, V)


@pytest.mark.parametrize("H", [16, 128, 8, 20])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_head_counts(H, dtype):
    announce(f"mla H={H} {dtype}")
    c = LatentCase([0, 1, 700, 33, 2100, 16], H, 16, dtype, 90 + H)
    ref = c.oracle()
    for part in (0, 256):
        out = c.run(part)
        assert_close(out, ref, dtype, f"H={H} partition={part}")
        assert not out[0].any()


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_block_size_32(dtype):
    announce(f"mla bs=32 {dtype}")
    c = LatentCase([5, 999, 64, 1], 16, 32, dtype, 95)
    assert_close(c.run(), c.oracle(), dtype, "bs=32")
    assert_close(c.run(64), c.oracle(), dtype, "bs=32 partition=64")


def test_long_context_one_sequence():
    announce("mla long 16384")
    c = LatentCase([16384], 16, 16, torch.bfloat16, 96)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "long")


def test_out_of_pool_table_id_poisons_only_its_sequence():
    announce("mla bad id")
    c = LatentCase([100, 200, 50], 16, 16, torch.float16, 97)
    bt = torch.from_numpy(c.tables).to(DEV)
    bt[1, 3] = -7
    out = c.run(tables=bt)
    assert torch.isnan(out[1]).all()
    ref = c.oracle()
    assert_close(out[[0, 2]], ref[[0, 2]], torch.float16, "other sequences")


def test_more_sequences_than_one_launch_holds():
    """2100 sequences: the library launches once per 2048 (the per-sequence
    offsets live in LDS); the second launch must pick up q, out and the
    tables at the right sequence."""
    announce("mla 2100 sequences")
    rng = np.random.default_rng(98)
    lens = rng.integers(0, 40, size=2100).tolist()
    c = LatentCase(lens, 16, 16, torch.bfloat16, 98)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "2100 sequences")


# ---- the workgroup-per-64-heads kernel (every head count under the default
#      split, up to 512 sequences; the cases above with partition 0 take it too)

@pytest.mark.parametrize("H", [64, 96, 128, 192])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_many_heads(H, dtype):
    """64 heads (one full group), 96 (a full and a half group), 128, 192;
    contexts of one partition and of several (merged by the second kernel),
    empty ones, NaN-poisoned unreferenced slots."""
    announce(f"mla many heads H={H} {dtype}")
    c = LatentCase([0, 1, 700, 33, 9000, 16, 4100], H, 16, dtype, 190 + H)
    out = c.run()
    assert_close(out, c.oracle(), dtype, f"many heads H={H}")
    assert not out[0].any()


@pytest.mark.parametrize("bs", [16, 32])
def test_many_heads_long_context_and_block_sizes(bs):
    announce(f"mla many heads long bs={bs}")
    c = LatentCase([20000, 3000], 128, bs, torch.bfloat16, 200 + bs)
    assert_close(c.run(), c.oracle(), torch.bfloat16, f"many heads bs={bs}")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_many_heads_negative_and_zero_scale(scale):
    announce(f"mla many heads scale {scale}")
    c = LatentCase([900, 5000], 64, 16, torch.float16, 210)
    c.scale = scale
    assert_close(c.run(), c.oracle(), torch.float16, f"scale {scale}")


def test_many_heads_out_of_pool_id():
    announce("mla many heads bad id")
    c = LatentCase([1000, 6000, 50], 128, 16, torch.bfloat16, 211)
    bt = torch.from_numpy(c.tables).to(DEV)
    bt[1, 100] = -3
    out = c.run(tables=bt)
    assert torch.isnan(out[1].float()).all()
    ref = c.oracle()
    assert_close(out[[0, 2]], ref[[0, 2]], torch.bfloat16, "other sequences")


def test_many_heads_more_sequences_than_the_kernel_takes():
    """600 sequences with 64 heads: past the many-heads kernel's 512, the call
    takes the split kernel; the result is the same attention."""
    announce("mla many heads 600 sequences")
    rng = np.random.default_rng(212)
    lens = rng.integers(0, 60, size=600).tolist()
    c = LatentCase(lens, 64, 16, torch.bfloat16, 212)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "600 sequences")


def test_many_heads_more_items_than_workgroups():
    """400 sequences with 64 heads: more rows than the GPU has workgroups, so
    the kernel takes its largest partition and its workgroups run several
    items each; the short contexts are whole items, the longer ones split."""
    announce("mla many heads 400 sequences")
    rng = np.random.default_rng(213)
    lens = rng.integers(0, 600, size=400)
    lens[[7, 100, 399]] = [5000, 9000, 4097]
    lens = lens.tolist()
    c = LatentCase(lens, 64, 16, torch.bfloat16, 213)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "400 sequences")


def test_many_heads_512_sequences():
    """512 sequences (the many-heads kernel's limit) with 64 heads: one item
    per row at the largest partition for the short ones, split rows for the
    few long ones."""
    announce("mla many heads 512 sequences")
    rng = np.random.default_rng(214)
    lens = rng.integers(1, 300, size=512)
    lens[[3, 511]] = [6000, 4500]
    c = LatentCase(lens.tolist(), 64, 32, torch.float16, 214)
    assert_close(c.run(), c.oracle(), torch.float16, "512 sequences")


# ---- up to 16 heads: one 16-row tile shared by the workgroup's four waves,
#      each scoring a quarter of the 576 elements (partial scores summed
#      through LDS) and accumulating its own 128 of the 512 values

@pytest.mark.parametrize("H", [1, 5, 16])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_few_heads_shared_tile(H, bs, dtype):
    """Contexts of one partition and of several (split rows merged by the
    second kernel), empty and one-token contexts, NaN-poisoned unreferenced
    blocks and tail slots; every value slice of every head compared."""
    announce(f"mla few heads H={H} bs={bs} {dtype}")
    c = LatentCase([0, 1, 700, 33, 9000, 16, 4100, 31], H, bs, dtype, 230 + H + bs)
    out = c.run()
    assert_close(out, c.oracle(), dtype, f"few heads H={H} bs={bs}")
    assert not out[0].any()


def test_few_heads_bench_shape():
    """The latent-cache workload's shape: 32 sequences of 1024..8192 tokens,
    16 heads, block 32, bf16; each row compared over all 512 values."""
    announce("mla few heads 32 x [1024, 8192]")
    rng = np.random.default_rng(240)
    lens = rng.integers(1024, 8192, size=32, endpoint=True).tolist()
    c = LatentCase(lens, 16, 32, torch.bfloat16, 240)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "32 sequences, 16 heads")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_few_heads_negative_and_zero_scale(scale):
    announce(f"mla few heads scale {scale}")
    c = LatentCase([900, 5000], 16, 16, torch.float16, 241)
    c.scale = scale
    assert_close(c.run(), c.oracle(), torch.float16, f"few heads scale {scale}")


def test_few_heads_out_of_pool_id():
    announce("mla few heads bad id")
    c = LatentCase([1000, 6000, 50], 16, 16, torch.bfloat16, 242)
    bt = torch.from_numpy(c.tables).to(DEV)
    bt[1, 100] = -3
    out = c.run(tables=bt)
    assert torch.isnan(out[1].float()).all()
    ref = c.oracle()
    assert_close(out[[0, 2]], ref[[0, 2]], torch.bfloat16, "other sequences")


def test_few_heads_repeatable():
    """The partial scores are summed in a fixed order: two calls agree bit for bit."""
    announce("mla few heads repeatable")
    c = LatentCase([3000, 700, 9000], 16, 16, torch.bfloat16, 243)
    a = c.run()
    b = c.run()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
