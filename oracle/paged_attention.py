"""Float64 CPU oracle for paged decode attention and its cache operations.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Conventions shared with the library's documented ABI (a layout contract, not
code): ``q`` and outputs are ``[S, H, D]``; each of ``k_pool`` / ``v_pool`` is
``[num_blocks, H, block_size, D]``; ``block_tables`` is ``[S, W]`` int32 whose
first ``ceil(L_s / block_size)`` entries are physical block ids;
``context_lens`` is ``[S]``.  Pools may be numpy arrays or torch CPU tensors of
any float storage dtype (float32, float16, bfloat16); values are upcast to
float64 exactly before any arithmetic.

Readings taken where the pages are silent:

* softmax scale is an explicit argument (the pages give none);
* an empty context (L = 0) yields a zero output row;
* table entries at or past ``ceil(L / block_size)`` and rows at or past L in the
  last block are never read, whatever they hold;
* split-context decode merges per-partition softmax partials with the
  log-sum-exp identity (the pages only name "Flash-Dec" as a roadmap item).

Pin status (tests/test_oracle.py):

* ``gather_sequence_kv`` — pinned: hand-derived fixture (tests/golden), block
  permutation invariance, contiguous round trip built by an independent
  block-wise scatter.
* ``decode_ref`` — pinned: torch ``scaled_dot_product_attention`` in float64,
  closed forms (one token, identical keys, zero scale, two-token logistic,
  dominant score), hand-derived fixture, sharing and poison invariants.
* ``split_decode_ref`` / ``lse_merge_ref`` — pinned: equal to ``decode_ref`` to
  1e-12 for every partition size; merge of one partial is the identity.
* ``reshape_and_cache_ref`` — pinned: tokens appended through allocator slots
  are read back in logical order by the gather; untouched bytes unchanged.
* ``copy_blocks_ref`` — pinned: destination bytes equal source bytes, all
  other blocks unchanged, and copy-on-write leaves decode output bit-identical.
* ``decode_gqa_ref`` — pinned: torch ``scaled_dot_product_attention`` with
  ``enable_gqa`` in float64 on contiguous caches; equal to ``decode_ref`` on
  pools whose K/V heads are repeated G times (numpy ``repeat``) and when
  there is one query head per K/V head.
* ``swap_blocks_ref`` — pinned: a swap out and back in restores the cache
  bit for bit and decode over it is unchanged; untouched blocks unchanged.
"""

from __future__ import annotations

import math

import numpy as np
import torch


def _as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch CPU tensor to float64 numpy."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _as_int(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


def _rows(pool, phys: np.ndarray, head: int, rows: np.ndarray) -> np.ndarray:
    """pool[phys[i], head, rows[i], :] for every i, upcast to float64."""
    if isinstance(pool, torch.Tensor):
        picked = pool[torch.from_numpy(phys), head, torch.from_numpy(rows)]
        return _as_f64(picked)
    return np.asarray(pool[phys, head, rows], dtype=np.float64)


def gather_sequence_kv(k_pool, v_pool, table_row, context_len: int, head: int,
                       block_size: int):
    """Rebuild one (sequence, head)'s contiguous K and V from the block table.

    Token t of the sequence lives in logical block t // block_size, at row
    t % block_size of that block; the table maps the logical block to its
    physical block in the pool (PagedAttention原理 §3.2; PagedAttentionMetal
    section 块表管理).  Only the first ``context_len`` tokens are read.

    Returns (K, V) as float64 arrays of shape [context_len, D].
    """
    L = int(context_len)
    table = _as_int(table_row)
    t = np.arange(L, dtype=np.int64)
    logical_block = t // block_size
    row_in_block = t % block_size
    phys = table[logical_block]
    return (_rows(k_pool, phys, head, row_in_block),
            _rows(v_pool, phys, head, row_in_block))


def decode_ref(q, k_pool, v_pool, block_tables, context_lens, scale: float,
               block_size: int) -> np.ndarray:
    """Single-query softmax attention per (sequence, head) over a paged cache.

    For every sequence s and head h with L = context_lens[s] > 0:
        K, V = the contiguous cache rebuilt from the block table,
        z_t  = scale * <q[s, h], K_t>              for t < L,
        w_t  = exp(z_t - max_t z_t),
        out  = sum_t w_t V_t / sum_t w_t.
    Subtracting the maximum changes nothing mathematically; it only keeps
    exp finite.  Paging does not alter this arithmetic (PagedAttention原理,
    closing remarks of §3.4); the pages' kernels differ only in how K/V are
    fetched (PagedAttention MLX, architecture list; PagedAttentionMetal,
    section 注意力计算优化).  L = 0 gives a zero row (reading, see module
    docstring).  Returns float64 [S, H, D].
    """
    qf = _as_f64(q)
    S, H, D = qf.shape
    tables = _as_int(block_tables)
    lens = _as_int(context_lens)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(H):
            K, V = gather_sequence_kv(k_pool, v_pool, tables[s], L, h, block_size)
            z = scale * (K @ qf[s, h])
            w = np.exp(z - z.max())
            out[s, h] = (w @ V) / w.sum()
    return out


def lse_merge_ref(partials):
    """Merge per-partition softmax partials into one attention output.

    Each partial is (m_i, l_i, o_i): the partition's maximum score, the sum of
    exp(z - m_i) over its tokens, and its own normalised output.  With
    M = max_i m_i and a_i = l_i * exp(m_i - M), the full result is
    sum_i a_i o_i / sum_i a_i — the log-sum-exp rescaling used by split-context
    ("Flash-Dec"-style) decoding (PagedAttention MLX, roadmap milestone 4).
    Partials with l_i = 0 (no tokens) carry no weight.
    """
    live = [(m, l, o) for (m, l, o) in partials if l > 0.0]
    if not live:
        return None
    M = max(m for (m, _, _) in live)
    num = sum(l * math.exp(m - M) * o for (m, l, o) in live)
    den = sum(l * math.exp(m - M) for (m, l, _) in live)
    return num / den


def split_decode_ref(q, k_pool, v_pool, block_tables, context_lens,
                     scale: float, block_size: int, partition_size: int):
    """Decode with each context cut into partitions of ``partition_size`` tokens.

    Partition i covers tokens [i*P, min((i+1)*P, L)).  Each partition computes
    its own (m_i, l_i, o_i) exactly as ``decode_ref`` would on that token
    range, and ``lse_merge_ref`` combines them.  Returns (out, partials) where
    partials[s][h] is the list of (m_i, l_i, o_i).
    """
    if partition_size <= 0 or partition_size % block_size != 0:
        raise ValueError("partition_size must be a positive multiple of block_size")
    qf = _as_f64(q)
    S, H, D = qf.shape
    tables = _as_int(block_tables)
    lens = _as_int(context_lens)
    out = np.zeros((S, H, D), dtype=np.float64)
    all_partials = []
    for s in range(S):
        L = int(lens[s])
        per_head = []
        for h in range(H):
            parts = []
            if L > 0:
                K, V = gather_sequence_kv(k_pool, v_pool, tables[s], L, h, block_size)
                for start in range(0, L, partition_size):
                    stop = min(start + partition_size, L)
                    z = scale * (K[start:stop] @ qf[s, h])
                    m = float(z.max())
                    w = np.exp(z - m)
                    l = float(w.sum())
                    parts.append((m, l, (w @ V[start:stop]) / l))
                out[s, h] = lse_merge_ref(parts)
            per_head.append(parts)
        all_partials.append(per_head)
    return out, all_partials


def reshape_and_cache_ref(k_pool, v_pool, k_new, v_new, slot_mapping,
                          block_size: int):
    """Write each new token's K/V into its cache slot; returns new pools.

    Slot n names row n % block_size of physical block n // block_size (the
    token position inside the block the allocator handed out: PagedAttention原理
    §3.3.2 and the append step of its §3.3.4 example).  A negative slot means
    "no write".  All heads of the token are written.  Byte copy: the stored
    dtype is kept, nothing is converted.  Inputs are not modified.
    """
    k_out = k_pool.clone() if isinstance(k_pool, torch.Tensor) else np.array(k_pool, copy=True)
    v_out = v_pool.clone() if isinstance(v_pool, torch.Tensor) else np.array(v_pool, copy=True)
    slots = _as_int(slot_mapping)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        block, row = divmod(int(slot), block_size)
        k_out[block, :, row, :] = k_new[i]
        v_out[block, :, row, :] = v_new[i]
    return k_out, v_out


def copy_blocks_ref(k_pool, v_pool, block_mapping):
    """Copy whole physical blocks (all heads, all rows) src -> dst in both pools.

    This is the copy half of copy-on-write for shared, reference-counted blocks
    (mlx-paged-attention, core feature 2; PagedAttentionMetal, section 块表管理;
    PagedAttention原理 §3.3.3).  Each destination receives the source block as it
    was before the call.  Returns new pools; inputs are not modified.
    """
    k_out = k_pool.clone() if isinstance(k_pool, torch.Tensor) else np.array(k_pool, copy=True)
    v_out = v_pool.clone() if isinstance(v_pool, torch.Tensor) else np.array(v_pool, copy=True)
    pairs = _as_int(block_mapping).reshape(-1, 2)
    for src, dst in pairs:
        k_out[int(dst)] = k_pool[int(src)]
        v_out[int(dst)] = v_pool[int(src)]
    return k_out, v_out


def swap_blocks_ref(dst_k, dst_v, src_k, src_v, block_mapping):
    """Copy whole blocks between two pools: dst[d] = src[s] for each {s, d}
    pair, in both the K and the V pool.  This is the data movement of swapping
    an inactive sequence's cache out to host memory and back in (page
    "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎", dynamic
    scheduling in the feature list and the physical KV pool of the
    architecture list, which can swap out to CPU memory).  Byte copy; returns
    new destination pools, inputs unchanged."""
    k_out = dst_k.clone() if isinstance(dst_k, torch.Tensor) else np.array(dst_k, copy=True)
    v_out = dst_v.clone() if isinstance(dst_v, torch.Tensor) else np.array(dst_v, copy=True)
    for src, dst in _as_int(block_mapping).reshape(-1, 2):
        k_out[int(dst)] = src_k[int(src)]
        v_out[int(dst)] = src_v[int(src)]
    return k_out, v_out


def decode_gqa_ref(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                   block_size: int) -> np.ndarray:
    """``decode_ref`` with fewer K/V heads than query heads (grouped-query
    attention): the pools hold Hkv heads, q holds H = G * Hkv, and query head h
    attends over K/V head h // G (contiguous groups).  The pages only have one
    head count (usage example of "PagedAttention MLX：为Apple Silicon打造的高吞吐量
    LLM推理引擎"); the grouping is this library's generalization, and the
    attention of each query head is exactly ``decode_ref``'s.  float64 [S, H, D]."""
    qf = _as_f64(q)
    S, H, D = qf.shape
    Hkv = k_pool.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    G = H // Hkv
    tables = _as_int(block_tables)
    lens = _as_int(context_lens)
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(H):
            K, V = gather_sequence_kv(k_pool, v_pool, tables[s], L, h // G, block_size)
            z = scale * (K @ qf[s, h])
            w = np.exp(z - z.max())
            out[s, h] = (w @ V) / w.sum()
    return out
