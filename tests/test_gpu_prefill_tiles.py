"""GPU parity of the row-block prefill kernel (pa_prefill with the default
split when the query rows of 128-row blocks alone fill the GPU: many query
tokens per sequence) against the float64 oracle, through the C ABI.

The shapes are the kernel's own: every case has at least one 128-row block
per CU, ragged query counts (partly filled last blocks) and contexts longer
than the query chunks.  Rows are compared on a sample — the first and last
rows of each sequence and of 128-row blocks, plus random ones — each row
recomputed by the oracle on its own (query token i of a sequence with L
tokens and Tq new ones is the one-row prefill over the first L - Tq + i + 1
tokens).  Also: both head dims and block sizes, fp16 / bf16, groups of 1, 4
and 8 query heads per K/V head, an idle sequence, more query tokens than
context (the rows before position 0 come out zero), a table id outside the
pool (NaN exactly on the 16-row tiles whose keys include that block),
negative and zero scales, and the whole output against the partitioned
kernel (an explicit partition size takes it)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_186_amd as pa
from paged_kv_cache_186_amd import workloads as W
from oracle import prefill_ref
from gpu_support import DEV, announce, assert_close, bits

pytestmark = pytest.mark.gpu


class TileCase:
    def __init__(self, lens, tq, H, Hkv, D, bs, dtype, seed):
        rng = np.random.default_rng(seed)
        nb = sum(-(-L // bs) for L in lens) + len(lens) + 4
        m = W.BlockManager(nb, bs, free_order=rng.permutation(nb).tolist())
        for s, L in enumerate(lens):
            m.allocate(s)
            m.append_slots(s, L)
        width = max(1, max(-(-L // bs) for L in lens))
        w = W.PagedWorkload("prefill_tiles", dtype, H, D, bs, nb, 1.0 / np.sqrt(D), m, list(range(len(lens))),
                            width, seed, DEV)
        W.fill_values(w, poison=False)
        w.k_pool = w.k_pool[:, :Hkv].contiguous()
        w.v_pool = w.v_pool[:, :Hkv].contiguous()
        W.poison_unreferenced(w)
        g = torch.Generator(device=DEV)
        g.manual_seed(seed * 7 + 3)
        self.w = w
        self.H, self.Hkv = H, Hkv
        self.lens = list(lens)
        self.tq = list(tq)
        self.qs = np.concatenate([[0], np.cumsum(self.tq)]).astype(np.int32)
        self.q = W.normal((int(self.qs[-1]), H, D), dtype, DEV, g)
        self.scale = w.scale

    def run(self, partition_size=0, tables=None):
        w = self.w
        out = torch.empty_like(self.q)
        bt = w.block_tables().to(DEV) if tables is None else tables
        ws = pa.new_workspace(pa.pa_prefill_workspace_size(len(self.lens), int(self.qs[-1]), self.H, self.Hkv,
                                                           self.q.shape[2], bt.shape[1], w.block_size,
                                                           partition_size), DEV)
        pa.pa_prefill(out, self.q, w.k_pool, w.v_pool, bt, w.context_lens().to(DEV), torch.from_numpy(self.qs).to(DEV),
                      self.scale, w.block_size, partition_size=partition_size, workspace=ws)
        torch.cuda.synchronize()
        return out

    def sample(self, rng, per_seq=6):
        """(sequence, query index) pairs: block edges and random rows."""
        G = self.H // self.Hkv
        picks = []
        for s, t in enumerate(self.tq):
            if t == 0:
                continue
            cand = {0, t - 1, min(t - 1, 128 // G), min(t - 1, 128 // G - 1), max(0, t - 1 - 128 // G)}
            cand |= set(int(x) for x in rng.integers(0, t, size=per_seq))
            picks += [(s, i) for i in sorted(cand)]
        return picks

    def oracle_rows(self, picks):
        """Each sampled row as a one-row prefill over its visible prefix."""
        w = self.w
        tables = w.block_tables_np()
        rows = [int(self.qs[s]) + i for s, i in picks]
        lens = [self.lens[s] - self.tq[s] + i + 1 for s, i in picks]
        ref = prefill_ref(self.q[rows].cpu(), w.k_pool.cpu(), w.v_pool.cpu(), np.stack([tables[s] for s, _ in picks]),
                          np.array(lens), np.arange(len(picks) + 1, dtype=np.int32), self.scale, w.block_size)
        return rows, ref


# ragged query chunks over longer contexts: 3163 query tokens
LENS = [2100, 900, 1500, 3000, 700, 640]
TQ = [700, 333, 900, 1000, 130, 100]


@pytest.mark.parametrize("D,bs", [(128, 16), (128, 32), (64, 16), (64, 32)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_head_dims_block_sizes_dtypes(D, bs, dtype):
    announce(f"prefill tiles D={D} bs={bs} {dtype}")
    c = TileCase(LENS, TQ, 32, 8, D, bs, dtype, 300 + D + bs)
    out = c.run()
    rows, ref = c.oracle_rows(c.sample(np.random.default_rng(D + bs)))
    err = assert_close(out[rows], ref, dtype, f"D={D} bs={bs}")
    print(f"prefill tiles D={D} bs={bs} {dtype}: max abs err {err:.2e} over {len(rows)} rows")
    assert torch.equal(bits(c.run()), bits(out)), "second call differs"


@pytest.mark.parametrize("H,Hkv", [(16, 16), (32, 4), (64, 8)])
def test_group_sizes(H, Hkv):
    """Groups of 1, 8 and 8 query heads per K/V head (rows token-major: a
    128-row block holds 128 / G query tokens)."""
    announce(f"prefill tiles H={H} Hkv={Hkv}")
    lens = [2600, 1800, 2300]
    tq = [1500, 700, 1200]
    c = TileCase(lens, tq, H, Hkv, 128, 16, torch.float16, 320 + H + Hkv)
    out = c.run()
    rows, ref = c.oracle_rows(c.sample(np.random.default_rng(H)))
    assert_close(out[rows], ref, torch.float16, f"H={H} Hkv={Hkv}")


def test_whole_output_matches_the_partitioned_kernel():
    """Every row: the row-block kernel (default split) against the
    partitioned kernel (an explicit partition of the whole context), both
    within the tolerance of the oracle; here within twice it of each other."""
    announce("prefill tiles vs partitioned kernel")
    c = TileCase(LENS, TQ, 32, 8, 128, 16, torch.bfloat16, 330)
    a = c.run()
    b = c.run(partition_size=-(-max(LENS) // 16) * 16)
    diff = (a.float() - b.float()).abs().max().item()
    assert diff <= 2 * 2e-2, diff
    rows, ref = c.oracle_rows(c.sample(np.random.default_rng(5), per_seq=3))
    assert_close(a[rows], ref, torch.bfloat16, "tiles")
    assert_close(b[rows], ref, torch.bfloat16, "partitioned")


def test_idle_sequence_and_more_queries_than_context():
    """An idle sequence (no query tokens) and one with 300 query tokens over
    a 200-token context: its first 100 rows see no key (they would sit before
    position 0) and come out zero, the others are the prefill of their
    prefix."""
    announce("prefill tiles idle and Tq > L")
    lens = [2000, 500, 200, 3000]
    tq = [1200, 0, 300, 1700]
    c = TileCase(lens, tq, 32, 8, 128, 16, torch.float16, 340)
    out = c.run()
    q0 = int(c.qs[2])
    assert not out[q0:q0 + 100].any()
    picks = [p for p in c.sample(np.random.default_rng(9)) if not (p[0] == 2 and p[1] < 100)]
    picks += [(2, 100), (2, 101), (2, 299)]
    rows, ref = c.oracle_rows(picks)
    assert_close(out[rows], ref, torch.float16, "idle / Tq > L")


def test_out_of_pool_table_id():
    """A table id outside the pool in sequence 1 at block 40 (keys 640..655):
    NaN on exactly the rows of the 16-row tiles (one K/V head, token-major)
    whose keys reach that block; every other row is exact."""
    announce("prefill tiles out-of-pool id")
    lens = [2000, 1400, 2500]
    tq = [1100, 900, 1300]
    H, Hkv = 32, 8
    G = H // Hkv
    c = TileCase(lens, tq, H, Hkv, 128, 16, torch.float16, 350)
    bt = c.w.block_tables().to(DEV)
    bt[1, 40] = c.w.num_blocks + 7
    out = c.run(tables=bt).float()
    first = lens[1] - tq[1]                      # position of query token 0
    q0 = int(c.qs[1])
    for r0 in range(0, tq[1] * G, 16):          # the 16-row tiles of sequence 1
        last = min(tq[1] * G, r0 + 16) - 1
        sees = first + last // G >= 40 * 16      # the tile's last row reaches the block
        for r in range(r0, last + 1):
            t, h = q0 + r // G, r % G
            vals = out[t, [kv * G + h for kv in range(Hkv)]]
            assert torch.isnan(vals).all() == sees, (r0, r)
    ok = [p for p in c.sample(np.random.default_rng(3)) if p[0] != 1]
    rows, ref = c.oracle_rows(ok)
    assert_close(out[rows], ref, torch.float16, "other sequences")


@pytest.mark.parametrize("scale", [-0.06, 0.0])
def test_negative_and_zero_scale(scale):
    announce(f"prefill tiles scale {scale}")
    c = TileCase([1800, 2400], [1000, 1400], 32, 8, 128, 32, torch.bfloat16, 360)
    c.scale = scale
    out = c.run()
    rows, ref = c.oracle_rows(c.sample(np.random.default_rng(11)))
    assert_close(out[rows], ref, torch.bfloat16, f"scale {scale}")


def test_many_sequences_and_more_than_one_launch():
    """2100 sequences of 40 query tokens over 40..300-token contexts: the
    workgroups' item offsets over all of a launch's sequences (8 per thread)
    and a second launch for the sequences past 2048."""
    announce("prefill tiles 2100 sequences")
    rng = np.random.default_rng(370)
    S = 2100
    tq = [40] * S
    lens = rng.integers(40, 301, size=S).tolist()
    c = TileCase(lens, tq, 32, 8, 128, 16, torch.float16, 370)
    out = c.run()
    picks = [(s, i) for s in (0, 1, 1000, 2047, 2048, 2049, S - 1) for i in (0, 17, 39)]
    picks += [(int(s), int(i)) for s, i in zip(rng.integers(0, S, size=24), rng.integers(0, 40, size=24))]
    rows, ref = c.oracle_rows(picks)
    assert_close(out[rows], ref, torch.float16, "2100 sequences")
