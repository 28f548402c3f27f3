"""GPU parity of pa_prefill on batches with few query rows per sequence —
speculative verification of a few drafted tokens, and one-token queries —
which the library runs on the grouped-query decode kernel (at most 64
sequences, at most 16 (or 32, for groups above 16) (query token, head) rows
per sequence and K/V head on average), against the float64 oracle
(prefill_ref), through the C ABI.

Covers: ragged drafted-token counts (0 to 6 per sequence), group sizes 1 to
32 (one tile partly filled, full, two tiles), both head dims and block sizes,
fp16 / bf16, long contexts split over many partitions (rows merged by the
second kernel, causal limits inside the last partition), more query tokens
than context (rows before position 0 come out zero), empty contexts, a table
id outside the pool (NaN exactly on the affected 16-row tiles), negative and
zero scales, the 64-sequence limit, and agreement with the partitioned
kernel (an explicit partition size takes that kernel)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_186_amd as pa
from paged_kv_cache_186_amd import workloads as W
from oracle import prefill_ref
from gpu_support import DEV, announce, assert_close, bits

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, lens, tq, H, Hkv, D, bs, dtype, seed):
        rng = np.random.default_rng(seed)
        nb = sum(-(-L // bs) for L in lens) + len(lens) + 4
        m = W.BlockManager(nb, bs, free_order=rng.permutation(nb).tolist())
        for s, L in enumerate(lens):
            m.allocate(s)
            m.append_slots(s, L)
        width = max(1, max(-(-L // bs) for L in lens))
        w = W.PagedWorkload("queries", dtype, H, D, bs, nb, 1.0 / np.sqrt(D), m, list(range(len(lens))),
                            width, seed, DEV)
        W.fill_values(w, poison=False)
        w.k_pool = w.k_pool[:, :Hkv].contiguous()
        w.v_pool = w.v_pool[:, :Hkv].contiguous()
        W.poison_unreferenced(w)
        g = torch.Generator(device=DEV)
        g.manual_seed(seed * 5 + 1)
        self.w, self.H, self.Hkv = w, H, Hkv
        self.lens, self.tq = list(lens), list(tq)
        self.qs = np.concatenate([[0], np.cumsum(self.tq)]).astype(np.int32)
        self.q = W.normal((int(self.qs[-1]), H, D), dtype, DEV, g)
        self.scale = w.scale
        G = H // Hkv
        rows = 32 if G > 16 else 16
        assert len(lens) <= 64 and int(self.qs[-1]) * G <= rows * len(lens), "not the few-rows path"

    def run(self, partition_size=0, tables=None):
        w = self.w
        out = torch.full_like(self.q, float("nan"))
        bt = w.block_tables().to(DEV) if tables is None else tables
        T = int(self.qs[-1])
        ws = pa.new_workspace(pa.pa_prefill_workspace_size(len(self.lens), T, self.H, self.Hkv, self.q.shape[2],
                                                           bt.shape[1], w.block_size, partition_size), DEV)
        pa.pa_prefill(out, self.q, w.k_pool, w.v_pool, bt, w.context_lens().to(DEV), torch.from_numpy(self.qs).to(DEV),
                      self.scale, w.block_size, partition_size=partition_size, workspace=ws)
        torch.cuda.synchronize()
        return out

    def oracle(self, tables=None):
        w = self.w
        return prefill_ref(self.q.cpu(), w.k_pool.cpu(), w.v_pool.cpu(),
                           w.block_tables_np() if tables is None else tables, np.array(self.lens), self.qs,
                           self.scale, w.block_size)


def _verify_batch(S, seed, G, max_tq=6, lo=1, hi=3000):
    """S seeded context lengths and drafted-token counts (0..max_tq, at most
    L), trimmed from the largest until the batch has at most 16 (32 for
    groups above 16) rows per sequence on average."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=S).tolist()
    tq = [min(int(x), L) for x, L in zip(rng.integers(0, max_tq + 1, size=S), lens)]
    while sum(tq) * G > (32 if G > 16 else 16) * S:
        tq[int(np.argmax(tq))] -= 1
    return lens, tq


@pytest.mark.parametrize("H,Hkv", [(32, 8), (32, 4), (12, 4), (16, 16), (32, 2), (32, 1), (48, 3)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_drafted_tokens_group_sizes(H, Hkv, dtype):
    """Groups of 4, 8, 3 (tiles partly filled, a token's rows split between
    two tiles), 1, 16 and 32 (two tiles of one token), ragged counts."""
    G = H // Hkv
    S = 24
    lens, tq = _verify_batch(S, 400 + H + Hkv, G, max_tq=min(6, (32 if G > 16 else 16) // G * 2))
    announce(f"prefill few rows H={H} Hkv={Hkv} {dtype}")
    c = Case(lens, tq, H, Hkv, 128, 16, dtype, 400 + H + Hkv)
    out = c.run()
    assert_close(out, c.oracle(), dtype, f"H={H} Hkv={Hkv}")
    assert torch.equal(bits(c.run()), bits(out)), "second call differs"


@pytest.mark.parametrize("D,bs", [(64, 16), (64, 32), (128, 32)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_head_dims_and_block_sizes(D, bs, dtype):
    announce(f"prefill few rows D={D} bs={bs} {dtype}")
    lens, tq = _verify_batch(40, 450 + D + bs, 4)
    c = Case(lens, tq, 32, 8, D, bs, dtype, 450 + D + bs)
    assert_close(c.run(), c.oracle(), dtype, f"D={D} bs={bs}")


def test_one_token_queries_and_64_sequences():
    """One query token per sequence (plain decode through pa_prefill) at the
    64-sequence limit."""
    announce("prefill few rows: 64 sequences, one token each")
    rng = np.random.default_rng(470)
    lens = rng.integers(1, 4000, size=64).tolist()
    c = Case(lens, [1] * 64, 32, 8, 128, 16, torch.float16, 470)
    assert_close(c.run(), c.oracle(), torch.float16, "one token")


@pytest.mark.parametrize("Hkv", [8, 1])
def test_long_contexts_split_over_partitions(Hkv):
    """Two long contexts and short ones: the long rows span many partitions
    (merged by the second kernel), the causal limits of the drafted tokens
    fall inside the last one."""
    announce(f"prefill few rows: long contexts, Hkv={Hkv}")
    lens = [40000, 3, 25000, 700]
    tq = [4, 2, 5, 1] if Hkv == 8 else [1, 1, 2, 0]  # 32 query heads per K/V head: fewer tokens
    c = Case(lens, tq, 32, Hkv, 128, 16, torch.bfloat16, 480 + Hkv)
    assert_close(c.run(), c.oracle(), torch.bfloat16, "long contexts")


def test_more_tokens_than_context_and_empty_contexts():
    """A sequence with 6 query tokens over a 3-token context (its first 3 rows
    would sit before position 0: zero; the others are the one-token prefill
    of their prefix), an empty context with 2 query tokens (zero), an idle
    sequence, and ordinary ones; also with a long context so that the rows
    with no keys go through the merge."""
    announce("prefill few rows: Tq > L, empty contexts")
    for lens, tq in (([3, 0, 500, 9, 1200], [6, 2, 0, 3, 4]), ([3, 0, 30000, 9], [6, 2, 3, 3])):
        c = Case(lens, tq, 32, 8, 128, 16, torch.float16, 490 + len(lens))
        out = c.run()
        assert not out[0:3].any() and not out[6:8].any()
        # every other row: query token i of sequence s is the one-token
        # prefill over the first L - Tq + i + 1 tokens
        w = c.w
        tables = w.block_tables_np()
        picks = [(s, i) for s in range(len(lens)) for i in range(tq[s]) if lens[s] - tq[s] + i + 1 > 0]
        rows = [int(c.qs[s]) + i for s, i in picks]
        ref = prefill_ref(c.q[rows].cpu(), w.k_pool.cpu(), w.v_pool.cpu(), np.stack([tables[s] for s, _ in picks]),
                          np.array([lens[s] - tq[s] + i + 1 for s, i in picks]),
                          np.arange(len(picks) + 1, dtype=np.int32), c.scale, w.block_size)
        assert_close(out[rows], ref, torch.float16, "Tq > L")


def test_out_of_pool_table_id():
    """An id outside the pool in sequence 2 at block 30 (keys 480..495): NaN
    on exactly the rows of the 16-row tiles of that sequence whose keys reach
    the block (every drafted token's row here); other sequences exact."""
    announce("prefill few rows: out-of-pool id")
    lens = [900, 1500, 2000, 300]
    tq = [4, 3, 4, 2]
    c = Case(lens, tq, 32, 8, 128, 16, torch.float16, 500)
    bt = c.w.block_tables().to(DEV)
    bt[2, 30] = c.w.num_blocks + 3
    out = c.run(tables=bt).float()
    q2 = slice(int(c.qs[2]), int(c.qs[3]))
    assert torch.isnan(out[q2]).all()
    keep = [s for s in range(4) if s != 2]
    ref = c.oracle()
    for s in keep:
        rows = slice(int(c.qs[s]), int(c.qs[s + 1]))
        assert_close(out[rows].to(torch.float16), ref[rows], torch.float16, f"sequence {s}")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_negative_and_zero_scale(scale):
    announce(f"prefill few rows: scale {scale}")
    lens, tq = _verify_batch(16, 510, 8)
    c = Case(lens, tq, 32, 4, 128, 32, torch.bfloat16, 510)
    c.scale = scale
    assert_close(c.run(), c.oracle(), torch.bfloat16, f"scale {scale}")


def test_agrees_with_the_partitioned_kernel():
    """The same batch through the partitioned prefill kernel (an explicit
    partition size): both within the oracle's tolerance."""
    announce("prefill few rows vs partitioned kernel")
    lens, tq = _verify_batch(48, 520, 4)
    c = Case(lens, tq, 32, 8, 128, 16, torch.bfloat16, 520)
    ref = c.oracle()
    a = c.run()
    b = c.run(partition_size=1024)
    assert_close(a, ref, torch.bfloat16, "few-rows path")
    assert_close(b, ref, torch.bfloat16, "partitioned")
