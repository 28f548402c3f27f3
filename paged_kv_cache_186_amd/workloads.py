"""Seeded synthetic inputs for paged decode: shapes, lengths, block layouts, values.

This module only draws random numbers and lays out blocks (through
``BlockManager``); it holds none of the attention, cache-write or copy
arithmetic.  Tests, the benchmark and the smoke check use it to feed the same
inputs to the HIP library and to the CPU oracle.

Workloads (shapes follow the pages: 32 heads x 128 dims over a 1024-block pool
in the usage example of "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理
引擎"; block sizes 16 or 32 from "3. PagedAttention原理" §3.3.1; 128K-token
contexts from the same two pages):

* ``tiny``                 4 sequences, lengths {1, 7, 16, 33}, 4 heads, D=64,
                           block 16, fp32, 16-block pool; tables are a seeded
                           permutation of pool ids dealt out in order.
* ``layer_shape``          8 sequences, lengths uniform in [1, 2048], 32 heads,
                           D=128, block 16, fp16, 1024-block pool; blocks popped
                           from a shuffled free list.
* ``continuous_batching``  64 sequences, lengths round(lognormal(ln 512, 1))
                           clipped to [32, 4096], 32 heads, D=128, block 32, fp16;
                           each step appends one token per sequence.
* ``shared_prefix``        32 sequences sharing a 1024-token prefix (64 blocks of
                           16, refcount 32) plus private suffixes uniform in
                           [0, 512]; bf16; the last shared block is made private
                           (copy-on-write) before each sequence's first suffix write.
* ``long_context``         batch 1 or 4 at 131072 tokens each, 32 heads, D=128,
                           block 16, fp16; 8192 randomly scattered blocks each.

Multi-token and latent-cache workloads (``QUERY_OPS``, built by
``query_workload``; lengths and blocks from a numpy generator, values from a
seeded ``torch.Generator``):

* ``prefill``   4 sequences of 4096 tokens whose last 1024 are new (a prompt
                chunk), 32 query / 8 K/V heads, D=128, block 16, fp16.
* ``verify``    64 sequences with the ``continuous_batching`` length mix and 4
                drafted tokens each, 32 query / 8 K/V heads, D=128, block 32,
                fp16.
* ``verify1``   the same batch with one query token per sequence.
* ``mla``       32 sequences, lengths uniform in [1024, 8192], 16 heads over a
                576-element latent row (values are its first 512), block 32,
                bf16.

q, K and V are N(0, 1) drawn in float32 from a seeded ``torch.Generator`` on
the target device and rounded to the storage dtype.  Pool blocks that no table
references (and rows past a sequence's length) are filled the same way unless
``poison`` asks for NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from .block_manager import BlockManager

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class PagedWorkload:
    name: str
    dtype: torch.dtype
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    manager: BlockManager
    seq_ids: List[int]
    table_width: int
    seed: int
    device: torch.device
    q: Optional[torch.Tensor] = None
    k_pool: Optional[torch.Tensor] = None
    v_pool: Optional[torch.Tensor] = None
    cow_pairs: List[Tuple[int, int]] = field(default_factory=list)
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_ids)

    def context_lens_np(self) -> np.ndarray:
        return self.manager.context_lens(self.seq_ids)

    def block_tables_np(self) -> np.ndarray:
        return self.manager.block_tables(self.seq_ids, self.table_width)

    def context_lens(self) -> torch.Tensor:
        return torch.from_numpy(self.context_lens_np()).to(self.device)

    def block_tables(self) -> torch.Tensor:
        return torch.from_numpy(self.block_tables_np()).to(self.device)

    def kv_bytes(self) -> int:
        """K+V bytes the decode must read for the current lengths."""
        e = torch.tensor([], dtype=self.dtype).element_size()
        return int(self.context_lens_np().astype(np.int64).sum()) * self.num_heads * self.head_dim * 2 * e


def _generator(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, dtype, device, gen, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """N(0,1) in float32 rounded to ``dtype``, generated in chunks along dim 0."""
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel() == 0:
        return out
    flat = out.view(shape[0], -1)
    per_row = flat.shape[1]
    rows = max(1, chunk_elems // max(1, per_row))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        flat[r0:r1] = torch.randn((r1 - r0, per_row), generator=gen, device=device,
                                  dtype=torch.float32).to(dtype)
    return out


def fill_values(w: PagedWorkload, poison: bool = False, value_seed_offset: int = 0) -> PagedWorkload:
    """Draw q, k_pool, v_pool on ``w.device`` (seeded)."""
    g = _generator(w.device, w.seed * 1000003 + 17 + value_seed_offset)
    S, H, D = w.num_seqs, w.num_heads, w.head_dim
    w.q = normal((S, H, D), w.dtype, w.device, g)
    shape = (w.num_blocks, H, w.block_size, D)
    w.k_pool = normal(shape, w.dtype, w.device, g)
    w.v_pool = normal(shape, w.dtype, w.device, g)
    if poison:
        poison_unreferenced(w)
    return w


def poison_unreferenced(w: PagedWorkload, value: float = float("nan")) -> None:
    """Fill unreferenced blocks and rows past each sequence's length."""
    bs = w.block_size
    used = np.zeros(w.num_blocks, dtype=bool)
    tables = w.block_tables_np()
    lens = w.context_lens_np()
    for s in range(w.num_seqs):
        nb = -(-int(lens[s]) // bs)
        used[tables[s, :nb]] = True
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(w.device)
    if unused.numel():
        w.k_pool[unused] = value
        w.v_pool[unused] = value
    for s in range(w.num_seqs):
        L = int(lens[s])
        nb = -(-L // bs)
        if nb and L % bs:
            last = int(tables[s, nb - 1])
            w.k_pool[last, :, L % bs:, :] = value
            w.v_pool[last, :, L % bs:, :] = value


FP8_DTYPES = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def fp8_pools(w: PagedWorkload, fmt: str, chunk_blocks: int = 2048):
    """An 8-bit copy of the workload's K/V pools for the *_fp8 calls.

    Input generation only: each (block, head) gets the scale
    max|x| / (largest finite value of ``fmt``) over its rows (NaN ignored; an
    all-zero or all-NaN tile gets scale 1), and each element is cast to the
    float8 dtype after division by it (torch's cast; the values stay in range).
    NaN-poisoned rows stay NaN codes.  Returns (k_codes, v_codes, k_scales,
    v_scales) on the workload's device; the 16-bit pools are left as they are.
    """
    out = []
    for pool in (w.k_pool, w.v_pool):
        codes = torch.empty(pool.shape, dtype=FP8_DTYPES[fmt], device=pool.device)
        scales = torch.empty(pool.shape[:2], dtype=torch.float32, device=pool.device)
        for b0 in range(0, pool.shape[0], chunk_blocks):
            x = pool[b0:b0 + chunk_blocks].float()
            amax = torch.nan_to_num(x.abs(), nan=0.0).amax(dim=(2, 3))
            sc = torch.where(amax > 0, amax / FP8_MAX[fmt], torch.ones_like(amax))
            scales[b0:b0 + chunk_blocks] = sc
            codes[b0:b0 + chunk_blocks] = (x / sc[:, :, None, None]).to(FP8_DTYPES[fmt])
            del x
        out += [codes, scales]
    return out[0], out[2], out[1], out[3]


def _manager_from_shuffled_free_list(num_blocks, block_size, rng) -> BlockManager:
    return BlockManager(num_blocks, block_size, free_order=rng.permutation(num_blocks).tolist())


def tiny(seed: int = 0, device="cpu", values: bool = True, poison: bool = True) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    lens = [1, 7, 16, 33]
    bs, nb = 16, 16
    perm = rng.permutation(nb).tolist()
    # blocks are taken from the end of the free list, so reverse the
    # permutation to hand out perm[0], perm[1], ... in order
    m = BlockManager(nb, bs, free_order=perm[::-1])
    for s, L in enumerate(lens):
        m.allocate(s)
        m.append_slots(s, L)
    w = PagedWorkload("tiny", torch.float32, 4, 64, bs, nb, 1.0 / math.sqrt(64), m,
                      list(range(4)), 3, seed, torch.device(device))
    return fill_values(w, poison) if values else w


def layer_shape(seed: int = 0, device="cpu", values: bool = True, poison: bool = False) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    S, H, D, bs, nb = 8, 32, 128, 16, 1024
    lens = rng.integers(1, 2048, size=S, endpoint=True)
    # cap so the total fits the pool (never binds: 8 * 128 blocks == 1024)
    while sum(-(-int(L) // bs) for L in lens) > nb:
        lens[np.argmax(lens)] -= bs
    m = _manager_from_shuffled_free_list(nb, bs, rng)
    for s, L in enumerate(lens):
        m.allocate(s)
        m.append_slots(s, int(L))
    w = PagedWorkload("layer_shape", torch.float16, H, D, bs, nb, 1.0 / math.sqrt(D), m,
                      list(range(S)), 2048 // bs, seed, torch.device(device))
    return fill_values(w, poison) if values else w


def continuous_batching(seed: int = 0, device="cpu", values: bool = True, poison: bool = False,
                        n_steps: int = 48, num_seqs: int = 64) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    S, H, D, bs = num_seqs, 32, 128, 32
    lens = np.clip(np.rint(rng.lognormal(mean=math.log(512.0), sigma=1.0, size=S)), 32, 4096).astype(np.int64)
    nb = int(sum(-(-(int(L) + n_steps) // bs) for L in lens)) + 64
    m = _manager_from_shuffled_free_list(nb, bs, rng)
    for s, L in enumerate(lens):
        m.allocate(s)
        m.append_slots(s, int(L))
    width = -(-(4096 + n_steps) // bs)
    w = PagedWorkload("continuous_batching", torch.float16, H, D, bs, nb, 1.0 / math.sqrt(D), m,
                      list(range(S)), width, seed, torch.device(device))
    w.extra["n_steps"] = n_steps
    return fill_values(w, poison) if values else w


def new_token_values(w: PagedWorkload, step: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Seeded (q, k_new, v_new) for one decode step, each [S, H, D]."""
    g = _generator(w.device, w.seed * 7919 + 1000 + step)
    shape = (w.num_seqs, w.num_heads, w.head_dim)
    return (normal(shape, w.dtype, w.device, g), normal(shape, w.dtype, w.device, g),
            normal(shape, w.dtype, w.device, g))


def shared_prefix(seed: int = 0, device="cpu", values: bool = True, poison: bool = False,
                  num_seqs: int = 32, prefix_tokens: int = 1024, max_suffix: int = 512) -> PagedWorkload:
    """Shared prefix with copy-on-write of the last shared block.

    The prefix is written once for sequence 0 and forked to the others
    (refcount ``num_seqs``).  Then, in sequence order, before a sequence's
    first suffix token the last shared block is made private if it is still
    shared; the resulting (src, dst) pairs are in ``w.cow_pairs`` and must be
    copied (``pa_copy_blocks``) before the suffix is written.  Suffix slots are
    in ``w.extra["suffix_slots"]`` (one list per sequence).
    """
    rng = np.random.default_rng(seed)
    S, H, D, bs = num_seqs, 32, 128, 16
    suffix = rng.integers(0, max_suffix, size=S, endpoint=True)
    n_prefix_blocks = -(-prefix_tokens // bs)
    nb = n_prefix_blocks + int(sum(-(-int(n) // bs) for n in suffix)) + S + 16
    m = _manager_from_shuffled_free_list(nb, bs, rng)
    m.allocate(0)
    prefix_slots, _ = m.append_slots(0, prefix_tokens)
    for s in range(1, S):
        m.fork(0, s)
    cow_pairs: List[Tuple[int, int]] = []
    suffix_slots: List[List[int]] = []
    for s in range(S):
        if suffix[s] > 0:
            pair = m.make_private(s, n_prefix_blocks - 1)
            if pair is not None:
                cow_pairs.append(pair)
        slots, cows = m.append_slots(s, int(suffix[s]))
        assert not cows  # the prefix fills whole blocks: suffix writes land in new blocks
        suffix_slots.append(slots)
    width = -(-(prefix_tokens + max_suffix) // bs)
    w = PagedWorkload("shared_prefix", torch.bfloat16, H, D, bs, nb, 1.0 / math.sqrt(D), m,
                      list(range(S)), width, seed, torch.device(device))
    w.cow_pairs = cow_pairs
    w.extra["prefix_slots"] = prefix_slots
    w.extra["suffix_slots"] = suffix_slots
    w.extra["suffix_lens"] = suffix.astype(np.int64)
    return fill_values(w, poison) if values else w


def long_context(seed: int = 0, batch: int = 1, device="cpu", values: bool = True,
                 context: int = 131072) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    H, D, bs = 32, 128, 16
    per_seq = -(-context // bs)
    nb = batch * per_seq
    perm = rng.permutation(nb).tolist()
    m = BlockManager(nb, bs, free_order=perm[::-1])
    for s in range(batch):
        m.allocate(s)
        # allocate() takes the first block; the remaining ones come from the
        # same shuffled order, one new block every ``bs`` tokens
        m.append_slots(s, context)
    w = PagedWorkload(f"long_context_b{batch}", torch.float16, H, D, bs, nb, 1.0 / math.sqrt(D), m,
                      list(range(batch)), per_seq, seed, torch.device(device))
    return fill_values(w, False) if values else w


BUILDERS = {
    "tiny": tiny,
    "layer_shape": layer_shape,
    "continuous_batching": continuous_batching,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
}


# multi-token query workloads (pa_prefill) and the latent cache (pa_decode_mla)
QUERY_OPS = {
    # a prompt chunk per sequence: 4 sequences whose last 1024 of 4096 tokens
    # are new (chunked prefill), 32 query / 8 K/V heads, D=128, BS=16, fp16
    "prefill": dict(S=4, lens="4096", tq=1024, H=32, Hkv=8, D=128, bs=16, dtype=torch.float16),
    # speculative verification: 64 sequences with lengths as in continuous
    # batching (log-normal, median 512, clipped to [32, 4096]), 4 drafted
    # tokens each, 32 query / 8 K/V heads, D=128, BS=32, fp16
    "verify": dict(S=64, lens="lognormal", tq=4, H=32, Hkv=8, D=128, bs=32, dtype=torch.float16),
    # the same batch with one query token each: grouped-query decode through
    # the matrix-core kernel (compare pa_decode_gqa on continuous batching)
    "verify1": dict(S=64, lens="lognormal", tq=1, H=32, Hkv=8, D=128, bs=32, dtype=torch.float16),
    # MLA decode: 32 sequences, lengths uniform in [1024, 8192], 16 heads (a
    # 128-head model split over 8 GPUs by heads), 576-element latent rows,
    # BS=32, bf16
    "mla": dict(S=32, lens="uniform", tq=1, H=16, Hkv=1, D=576, bs=32, dtype=torch.bfloat16),
}


@dataclass
class QueryWorkload:
    """Inputs of one pa_prefill / pa_decode_mla call (see QUERY_OPS)."""
    op: str
    S: int
    H: int
    Hkv: int
    D: int
    Dv: int
    bs: int
    dtype: torch.dtype
    tq: int
    mla: bool
    lens: np.ndarray        # int64 [S]
    tables_np: np.ndarray   # int32 [S, width]
    qs_np: np.ndarray       # int32 [S + 1]
    T: int
    width: int
    scale: float
    pools: tuple            # (k_pool, v_pool) or (latent pool,)
    q: torch.Tensor


def query_workload(op: str, seed: int = 0, device="cpu", heads: int = 0) -> QueryWorkload:
    """Seeded inputs of a QUERY_OPS workload: lengths, blocks popped from a
    shuffled free list, N(0,1) pools and queries in the workload's dtype."""
    cfg = dict(QUERY_OPS[op])
    if heads:
        cfg["H"] = heads
    S, H, Hkv, D, bs, dtype, tq = cfg["S"], cfg["H"], cfg["Hkv"], cfg["D"], cfg["bs"], cfg["dtype"], cfg["tq"]
    mla = op == "mla"
    dev = torch.device(device)
    rng = np.random.default_rng(seed)
    if cfg["lens"] == "4096":
        lens = np.full(S, 4096, dtype=np.int64)
    elif cfg["lens"] == "lognormal":
        lens = np.clip(np.rint(rng.lognormal(math.log(512.0), 1.0, S)), 32, 4096).astype(np.int64)
    else:
        lens = rng.integers(1024, 8192, size=S, endpoint=True)
    nb = int(sum(-(-int(L) // bs) for L in lens)) + 8
    m = BlockManager(nb, bs, free_order=rng.permutation(nb).tolist())
    for s, L in enumerate(lens):
        m.allocate(s)
        m.append_slots(s, int(L))
    width = int(max(-(-int(L) // bs) for L in lens))
    tables_np = m.block_tables(list(range(S)), width)
    qs_np = np.concatenate([[0], np.cumsum(np.full(S, tq, dtype=np.int64))]).astype(np.int32)
    T = int(qs_np[-1])
    g = _generator(dev, seed * 1000003 + 29)
    pools = (normal((nb, bs, D), dtype, dev, g),) if mla else \
        (normal((nb, Hkv, bs, D), dtype, dev, g), normal((nb, Hkv, bs, D), dtype, dev, g))
    q = normal((T, H, D), dtype, dev, g)
    return QueryWorkload(op, S, H, Hkv, D, 512 if mla else D, bs, dtype, tq, mla, lens, tables_np, qs_np, T, width,
                         1.0 / math.sqrt(192.0 if mla else D), pools, q)
