"""Float64 CPU oracle for attention of several new tokens per sequence over the
paged cache, and for decode over a multi-head latent (MLA) cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Multi-token queries.  The page "mlx-paged-attention: Bringing vLLM-level High
Throughput Inference to Apple Silicon" names speculative decoding as a feature
vLLM has and the project lacks (comparison with vLLM) and as future work
(future plans); verifying k drafted tokens — like prefilling a prompt in
chunks — means attending with several new query tokens of a sequence at once
over its paged cache.  The pages give no semantics; the readings taken here:

* the new tokens are already in the cache: sequence s has context length L_s
  including them, and its Tq_s query tokens are its LAST Tq_s tokens, token i
  (0 <= i < Tq_s) sitting at position p_i = L_s - Tq_s + i;
* causal: query token i attends over the keys at positions 0 .. p_i (itself
  included), and over nothing else;
* queries are packed: ``q`` is [T, H, D] and sequence s owns rows
  query_start[s] .. query_start[s+1] - 1 (query_start[0] = 0,
  query_start[S] = T, non-decreasing, Tq_s <= L_s);
* heads: query head h reads K/V head h // (H / Hkv), as for grouped-query
  decode; each (token, head) row is the ordinary softmax attention of
  ``decode_ref`` over its visible keys (PagedAttention原理 §3.2 and the closing
  remarks of §3.4: paging leaves the mathematics of attention unchanged).

MLA latent cache.  "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎",
roadmap milestone 3, names multi-head latent attention (the DeepSeek-V3
architecture) and nothing more.  Reading, from the published form of MLA
decode with the up-projections absorbed into the query and the output
(DeepSeek-V2 technical report, section on MLA): the cache keeps ONE row per
token, the compressed latent vector followed by the shared rotary key part
(Dqk = d_latent + d_rope elements, e.g. 512 + 64); every query head h brings
a query of Dqk elements; the score of token t is scale * <q_h, row_t> over
all Dqk elements and the value of token t is the first Dv = d_latent
elements of the same row.  The output per head is the Dv-element weighted
latent (the model applies its value up-projection afterwards, outside this
library).  Pool layout [num_blocks, block_size, Dqk].

Pin status (tests/test_oracle_multi_query.py):

* ``prefill_ref`` — pinned: torch ``scaled_dot_product_attention`` with its
  own causal mask (``is_causal``) in float64 when the whole context is new
  (Tq = L, where the reading's alignment and torch's coincide), also with
  ``enable_gqa``; one query token per sequence equals ``decode_gqa_ref``
  bit for bit; every row equals a decode at context length p_i + 1
  (speculative verification); a chunk's rows equal the same rows of the
  whole-context prefill (the prefix property of causal attention); mutants
  (mask off by one, top-left alignment, no mask, reversed positions, wrong
  sequence's rows, wrong head grouping) are caught.
* ``mla_decode_ref`` — pinned: torch ``scaled_dot_product_attention`` in
  float64 with a value width different from the key width, on contiguous
  rows built by an independent scatter; closed forms (one token → its first
  Dv elements; zero scale → mean of the latents); mutants (value taken from
  the tail of the row, score over the latent part only, wrong block) caught.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import _as_f64, _as_int, gather_sequence_kv


def _query_bounds(query_start, S: int, T: int) -> np.ndarray:
    qs = _as_int(query_start).astype(np.int64)
    if qs.shape != (S + 1,) or qs[0] != 0 or qs[S] != T or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must be [S+1], non-decreasing, from 0 to the number of query rows")
    return qs


def prefill_ref(q, k_pool, v_pool, block_tables, context_lens, query_start, scale: float,
                block_size: int) -> np.ndarray:
    """Causal attention of each sequence's last Tq_s tokens over its paged
    cache (readings in the module docstring).  q: [T, H, D]; pools
    [num_blocks, Hkv, block_size, D]; returns float64 [T, H, D]."""
    qf = _as_f64(q)
    T, H, D = qf.shape
    Hkv = k_pool.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of K/V heads")
    G = H // Hkv
    tables = _as_int(block_tables)
    lens = _as_int(context_lens)
    S = len(lens)
    qs = _query_bounds(query_start, S, T)
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        Tq = int(qs[s + 1] - qs[s])
        if Tq > L:
            raise ValueError("a sequence cannot have more query tokens than context")
        if Tq == 0:
            continue
        for h in range(H):
            K, V = gather_sequence_kv(k_pool, v_pool, tables[s], L, h // G, block_size)
            for i in range(Tq):
                p = L - Tq + i                      # position of query token i
                z = scale * (K[:p + 1] @ qf[qs[s] + i, h])
                w = np.exp(z - z.max())
                out[qs[s] + i, h] = (w @ V[:p + 1]) / w.sum()
    return out


def mla_decode_ref(q, kv_pool, block_tables, context_lens, scale: float, block_size: int,
                   v_dim: int) -> np.ndarray:
    """Decode over a latent cache: q [S, H, Dqk]; kv_pool [num_blocks,
    block_size, Dqk] (one row per token: latent then rotary part); the value
    of a token is the first v_dim elements of its row.  Returns float64
    [S, H, v_dim]; an empty context gives zeros."""
    qf = _as_f64(q)
    S, H, Dqk = qf.shape
    if kv_pool.shape[2] != Dqk or not 0 < v_dim <= Dqk:
        raise ValueError("latent rows must have the query's width and v_dim must fit in it")
    pool = kv_pool[:, None]                         # one latent "head": [N, 1, bs, Dqk]
    tables = _as_int(block_tables)
    lens = _as_int(context_lens)
    out = np.zeros((S, H, v_dim), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        C, _ = gather_sequence_kv(pool, pool, tables[s], L, 0, block_size)
        for h in range(H):
            z = scale * (C @ qf[s, h])
            w = np.exp(z - z.max())
            out[s, h] = (w @ C[:, :v_dim]) / w.sum()
    return out
