/*
 * libpagedattn — paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument that names
 * tensor data is DEVICE memory owned by the caller; the library allocates
 * nothing and holds no handle (the only thing carried from one call to the
 * next is the all-zero state of the arrival counters in the caller's decode
 * workspace, see pa_decode_workspace_size; pa_decode_noalloc keeps its own
 * in a static device array instead).  All work is
 * enqueued asynchronously on the given stream (a hipStream_t passed as void*;
 * NULL means the default stream).
 *
 * The method (sources cited by page title and section):
 *   - the KV cache is cut into fixed-size blocks of 16 or 32 tokens that live
 *     anywhere in a physical pool; a per-sequence block table maps logical
 *     block j to its physical block (vLLM tutorial page "3. PagedAttention原理",
 *     §3.2 and §3.3.1; page "PagedAttentionMetal：基于Metal 3的Apple Silicon原生
 *     LLM推理加速方案", sections 分页KV缓存机制 and 块表管理);
 *   - decode attention fetches K/V through the table and otherwise computes
 *     ordinary softmax attention; sequences of different lengths share one
 *     batch without padding (PagedAttentionMetal, section 注意力计算优化;
 *     "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎", architecture
 *     list; PagedAttention原理, closing remarks of §3.4);
 *   - a new token is written into the next row of its sequence's last block
 *     (PagedAttention原理 §3.3.2);
 *   - shared blocks are copied before a private write: copy-on-write
 *     ("mlx-paged-attention: Bringing vLLM-level High Throughput Inference to
 *     Apple Silicon", core feature 2; PagedAttention原理 §3.3.3).
 *
 * Layouts (row-major, dense, part of the ABI):
 *   q, out            [num_seqs][num_heads][head_dim]
 *   k_pool, v_pool    [num_blocks][num_heads][block_size][head_dim]  (two arrays)
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]
 *   context_lens      int32 [num_seqs]
 *   slot_mapping      int32 [num_tokens]; slot = physical_block*block_size + row
 *   block_mapping     int32 [num_pairs][2] = {src, dst}
 * One element dtype covers q, k_pool, v_pool, out, k_new and v_new (the *_fp8
 * calls below: an 8-bit pool with per-block scales).  Keys and values have as
 * many heads as queries.  head_dim is 64 or 128; block_size is
 * 16 or 32.  Every tensor pointer must be 16-byte aligned.
 *
 * Errors: arguments are validated on the host before anything is launched; a
 * failed check returns a status and enqueues nothing.  A launch failure returns
 * PA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  Entries the host cannot check (table ids, slots, copy pairs)
 * are bounds-checked in the kernels: see each call.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_F16 = 1,
  PA_DTYPE_BF16 = 2,
  /* 8-bit KV-cache element formats (the *_fp8 calls only), OCP 8-bit floats:
   * E4M3 = sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
   * S.1111.111 = NaN, largest finite 448; E5M2 = sign, 5 exponent bits
   * (bias 15), 2 mantissa bits, IEEE infinities and NaNs, largest finite
   * 57344.  Both have subnormals. */
  PA_DTYPE_FP8_E4M3 = 3,
  PA_DTYPE_FP8_E5M2 = 4
} pa_dtype_t;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, misaligned pointer, bad size, bad scale */
  PA_ERR_UNSUPPORTED = 2, /* head_dim, block_size or dtype outside what is built */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 4,         /* the HIP runtime refused the launch */
  PA_ERR_TOO_LARGE = 5    /* pa_decode_noalloc: the call exceeds its static scratch */
} pa_status_t;

/* Version of this ABI; bumped on any incompatible change. */
int32_t pa_abi_version(void);

/* Human-readable name of a status (static storage; never NULL). */
const char* pa_status_string(pa_status_t status);

/*
 * Bytes of device workspace pa_decode needs for these sizes and this
 * partition_size (the same rule as pa_decode; with an explicit partition_size
 * it is 0 when every sequence fits in one partition).  Returns 0 for sizes
 * pa_decode would reject.
 *
 * Workspace contract: the workspace begins with one 32-bit arrival counter per
 * (sequence, head), 4*num_seqs*num_heads bytes rounded up to 256.  Those bytes
 * must be zero when pa_decode starts; every pa_decode call leaves them zero
 * when it completes.  So zero-fill a workspace once after allocating it, and
 * again if it was used for anything else or with a different
 * num_seqs*num_heads.  The rest of the workspace is scratch.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t partition_size);

/*
 * Decode attention over a paged KV cache: for every sequence s and head h,
 *   out[s][h][:] = sum_t softmax_t(scale * <q[s][h], K_t>) * V_t,  t < L_s,
 * where K_t, V_t are row t % block_size of physical block
 * block_tables[s][t / block_size] (head h) and L_s = context_lens[s].
 * Sources: PagedAttentionMetal, section 注意力计算优化; PagedAttention原理 §3.2
 * and the closing remarks of §3.4.
 *
 * Long contexts are split and the pieces' softmax partials (max, sum,
 * weighted values) are merged with the log-sum-exp identity — the
 * split-context decode the "PagedAttention MLX" page names as its "Flash-Dec"
 * roadmap milestone — inside the one kernel launch: the last piece of a
 * (sequence, head) to finish merges them.  How contexts are split:
 *   - partition_size 0 with num_seqs <= 2048 (the default): every wave of a
 *     fixed grid takes an equal share of all (sequence, head, block) work, so
 *     the load is balanced whatever the mix of lengths; a (sequence, head)
 *     lying inside one share is finished without any partial;
 *   - partition_size > 0 (a multiple of block_size), or num_seqs > 2048: one
 *     workgroup per partition of partition_size tokens (0 then picks 512,
 *     halved while the grid would be too small to fill the GPU, never below 8
 *     blocks).
 * Within rounding the result does not depend on how contexts are split.
 *
 * Arithmetic: inputs are converted to fp32, dot products, softmax and the
 * weighted sum accumulate in fp32, and out is rounded to nearest-even once.
 *
 * Semantics of edge cases:
 *   - L_s == 0 writes a zero row; L_s is clamped to [0, max_blocks_per_seq*block_size];
 *   - table entries at or past ceil(L_s/block_size) and rows at or past L_s in
 *     the last block are never read (may hold anything, NaN included);
 *   - a referenced table entry outside [0, num_blocks) is not dereferenced:
 *     that (sequence, head) row of out becomes NaN.
 * Preconditions: out aliases no input; the workspace follows the contract of
 * pa_decode_workspace_size() and is not shared by calls that may overlap in
 * time.  num_seqs == 0 returns PA_OK and launches nothing.
 * Limits: num_seqs <= 65535, num_heads <= 65535, partitions per sequence <= 65535.
 */
pa_status_t pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      float scale, int32_t block_size,
                      int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                      int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t partition_size, pa_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus workspace and
 * workspace_bytes), semantics, kernels and results as pa_decode with the same
 * sizes and partition_size.  The arrival counters and partials live in a
 * static device array of the library, PA_NOALLOC_SCRATCH_BYTES (32 MiB) per
 * GPU, which each GPU the library runs this call on holds until the process
 * ends; the call itself allocates nothing (no hipMalloc, no allocating
 * library routine).  Its first 4*PA_NOALLOC_MAX_ROWS bytes hold the counters
 * of every call (cleared by a fill kernel on `stream` before the first call
 * on a device; every call leaves them zero), the partials follow.
 * Limits: num_seqs*num_heads <= PA_NOALLOC_MAX_ROWS and a partial area that
 * fits the rest of the array — e.g. 4 x 131072 tokens x 32 heads at
 * head_dim 128 fits with the default split (~0.6 MB of partials) and with
 * partitions of 512 tokens (~17 MB); otherwise PA_ERR_TOO_LARGE and nothing
 * is launched.  Every call on one GPU shares that GPU's array: calls that
 * may overlap in time on one GPU (other streams, other host threads) race
 * and give wrong results; serialise them.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
#define PA_NOALLOC_MAX_ROWS 262144
pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, int32_t block_size,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t partition_size, pa_dtype_t dtype, void* stream);

/*
 * Write each new token's K and V (all heads) into its cache slot:
 *   k_pool[slot / block_size][h][slot % block_size][:] = k_new[i][h][:]
 * and likewise for v, for i < num_tokens with slot = slot_mapping[i].
 * Bit-exact byte copy.  Source: PagedAttention原理 §3.3.2 (append into the last
 * block, or row 0 of a fresh one).
 * k_new, v_new: [num_tokens][num_heads][head_dim].  A negative slot, or one
 * >= num_blocks*block_size, writes nothing.  Slots must be distinct (two
 * writes to one slot race).  num_tokens == 0 returns PA_OK.
 */
pa_status_t pa_reshape_and_cache(void* k_pool, void* v_pool,
                                 const void* k_new, const void* v_new,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype_t dtype, void* stream);

/*
 * Copy whole physical blocks (every head and row) in both pools:
 *   k_pool[dst] = k_pool[src], v_pool[dst] = v_pool[src]
 * for each {src, dst} pair of block_mapping.  Bit-exact.  This is the copy step
 * of copy-on-write for shared, reference-counted blocks (mlx-paged-attention,
 * core feature 2; PagedAttentionMetal, section 块表管理; PagedAttention原理
 * §3.3.3).  Pairs with an id outside [0, num_blocks) are skipped.
 * Preconditions: destinations are distinct and no destination is also a
 * source (otherwise the result depends on scheduling).  num_pairs == 0
 * returns PA_OK.
 */
pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping,
                           int32_t num_pairs, int32_t num_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, pa_dtype_t dtype,
                           void* stream);

/*
 * ---- Grouped-query attention -----------------------------------------------
 * pa_decode with fewer K/V heads than query heads (grouped-query attention;
 * multi-query attention is num_kv_heads == 1): query head h attends over K/V
 * head h / (num_heads / num_kv_heads), the usual contiguous grouping.  The
 * pages only have num_heads (usage example of "PagedAttention MLX：为Apple
 * Silicon打造的高吞吐量LLM推理引擎"); this generalization is the library's.
 * Pools are [num_blocks][num_kv_heads][block_size][head_dim] (scales, for an
 * 8-bit cache, [num_blocks][num_kv_heads]); q and out are
 * [num_seqs][num_heads][head_dim].  kv_dtype is q_dtype (F32, F16, BF16) or,
 * for F16 / BF16 queries, an 8-bit format (then k_scales / v_scales are
 * required, else ignored).  num_heads must be a multiple of num_kv_heads.
 * With the default split (partition_size 0, num_seqs <= 2048) and 16-bit
 * queries, one K/V tile load serves 4 or 2 query heads of a group (the
 * largest dividing the group size; a larger group is served 4 heads at a
 * time); otherwise every query head reads its K/V head's tiles itself.  Workspace: pa_decode_gqa_workspace_size() for the
 * same arguments; same contract as pa_decode_workspace_size().
 */
size_t pa_decode_gqa_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size,
                                    pa_dtype_t q_dtype, pa_dtype_t kv_dtype);

pa_status_t pa_decode_gqa(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, const int32_t* context_lens,
                          float scale, int32_t block_size,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t partition_size, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- Several query tokens per sequence (chunked prefill, speculative
 * verification) ----------------------------------------------------------------
 * Causal attention of each sequence's LAST Tq_s tokens over its paged cache
 * ("mlx-paged-attention: Bringing vLLM-level High Throughput Inference to
 * Apple Silicon": speculative decoding, named in the comparison with vLLM and
 * in the future plans; the pages give no semantics, this is the library's
 * reading).  The new tokens' K/V must already be in the cache
 * (pa_reshape_and_cache), so context_lens[s] = L_s counts them; query token
 * i < Tq_s of sequence s sits at position p = L_s - Tq_s + i and attends over
 * the keys at positions 0..p.  Query head h reads K/V head h / (num_heads /
 * num_kv_heads).
 *   q, out:       [num_query_tokens][num_heads][head_dim], packed by sequence:
 *                 sequence s owns rows query_start[s] .. query_start[s+1]-1
 *   query_start:  int32 [num_seqs + 1] device array, query_start[0] = 0,
 *                 non-decreasing, query_start[num_seqs] = num_query_tokens,
 *                 Tq_s <= L_s
 *   pools:        [num_blocks][num_kv_heads][block_size][head_dim]
 *   dtype:        PA_DTYPE_F16 or PA_DTYPE_BF16 (q, pools and out; the
 *                 products run on the matrix cores with fp32 accumulation and
 *                 the probabilities rounded to dtype before the V product);
 *                 anything else is PA_ERR_UNSUPPORTED.  head_dim 64 or 128,
 *                 block_size 16 or 32.
 *   partition_size: 0 lets the library split long contexts only when the
 *                 query rows alone would not fill the GPU; otherwise keys per
 *                 partition, a positive multiple of 16.  With 0, at most 64
 *                 sequences and few rows — num_query_tokens * (num_heads /
 *                 num_kv_heads) <= 16 * num_seqs (32 * num_seqs for groups
 *                 of more than 16 heads), as when verifying a few drafted
 *                 tokens — the call runs on the grouped-query decode kernel
 *                 (a workgroup's four waves share each item's keys) and a
 *                 second kernel merges the split rows; its workspace holds
 *                 the partials and 32 bytes per query token, no counters.
 *   workspace:    pa_prefill_workspace_size() bytes for the same sizes, 0
 *                 when nothing is split (then workspace may be NULL).  It
 *                 begins with arrival counters that must be zero when a call
 *                 starts; every call leaves its own counters zero.  How many
 *                 counters there are depends on every size argument
 *                 (num_seqs, num_query_tokens, num_heads, num_kv_heads,
 *                 head_dim, max_blocks_per_seq, block_size, partition_size),
 *                 and the partials of a call follow its counters, so a call
 *                 with fewer counters writes partials where a call with more
 *                 keeps counters: zero the whole workspace again before a
 *                 call whose sizes differ from those of the previous call
 *                 that used it.  Its layout differs from pa_decode*'s: do not
 *                 hand one workspace to both kinds without zeroing it.
 * Device-side contents never cause an access outside the arrays: lengths are
 * clamped to [0, max_blocks_per_seq * block_size], query bounds to
 * [0, num_query_tokens], and a table id outside the pool makes NaN every
 * output row of each 16-row tile (query rows of one K/V head, token-major)
 * whose keys include that block.  A row that sees no key at all comes out
 * zero, as an empty context does in pa_decode (with Tq_s > L_s, which breaks
 * the contract, the rows that would sit before position 0).
 */
size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t partition_size);

pa_status_t pa_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, float scale, int32_t block_size,
                       int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- Decode over a multi-head latent (MLA) cache ------------------------------
 * "PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎", roadmap
 * milestone 3, names multi-head latent attention (DeepSeek-V3).  Reading (the
 * published absorbed form of MLA decode): the cache keeps one 576-element
 * row per token — the 512-element compressed latent followed by the 64-element
 * shared rotary key; every query head brings a 576-element query (its
 * no-position part already multiplied by the key up-projection); the score of
 * token t is scale * <q_h, row_t> and its value the row's first 512 elements.
 *   q:        [num_seqs][num_heads][576]
 *   kv_pool:  [num_blocks][block_size][576]
 *   out:      [num_seqs][num_heads][512] (the weighted latent; the value
 *             up-projection is the model's)
 *   dtype:    PA_DTYPE_F16 or PA_DTYPE_BF16; block_size 16 or 32.
 * Everything else (tables, lengths, partition_size, workspace from
 * pa_decode_mla_workspace_size(), error behaviour) as for pa_prefill with one
 * query token per sequence; in particular zero the workspace again before a
 * call whose sizes (num_seqs, num_heads, max_blocks_per_seq, block_size,
 * partition_size) differ from those of the previous call that used it.
 */
size_t pa_decode_mla_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size);

pa_status_t pa_decode_mla(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, int32_t block_size,
                          int32_t num_seqs, int32_t num_heads, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Copy whole blocks from one pool pair to another (K and V):
 *   dst_k[d] = src_k[s], dst_v[d] = src_v[s]     for each {s, d} of block_mapping
 * — swapping an inactive sequence's blocks out to host memory and back in
 * ("PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎": dynamic
 * scheduling with preemption and swapping, and the physical KV pool that can
 * swap out to CPU memory).  Either pool pair may live in pinned host memory
 * that is mapped into the GPU's address space (hipHostMalloc; torch's
 * pin_memory) and the other in device memory; block_mapping (int32 [n][2])
 * and the scales may be in either too.  Host pointers are passed as they are:
 * the library asks HIP for the GPU address of pinned host memory and returns
 * PA_ERR_INVALID_ARG, launching nothing, for any pointer HIP does not know as
 * device or pinned host memory (pageable host memory included).  One kernel
 * moves all pairs, with many 16 KiB chunks in flight over the host link.
 * Bit-exact.  Pool layout as above, src with src_num_blocks blocks and dst
 * with dst_num_blocks; pairs naming an id outside its pool are skipped.
 * dtype may be F32, F16, BF16, or an 8-bit format — then each block's K and
 * V scales move too (the four scale pointers, [blocks][num_heads] fp32, must
 * be non-null; they are ignored for the other dtypes).  Destinations must be
 * distinct; with the same pools on both sides no destination may be a
 * source.  num_pairs == 0 returns PA_OK.
 */
pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                           float* dst_k_scales, float* dst_v_scales,
                           const float* src_k_scales, const float* src_v_scales,
                           const int32_t* block_mapping, int32_t num_pairs,
                           int32_t num_heads, int32_t head_dim, int32_t block_size,
                           int32_t src_num_blocks, int32_t dst_num_blocks,
                           pa_dtype_t dtype, void* stream);

/*
 * ---- 8-bit KV cache --------------------------------------------------------
 * The pages name quantization only as future work (page "mlx-paged-attention:
 * Bringing vLLM-level High Throughput Inference to Apple Silicon", future
 * plans); the scheme below is this library's reading.  The pools hold one
 * byte per element in kv_dtype (PA_DTYPE_FP8_E4M3 or PA_DTYPE_FP8_E5M2); each
 * (physical block, head) has one fp32 scale for K and one for V:
 *   k_scales, v_scales  float [num_blocks][num_heads], caller-owned device
 *   memory, 4-byte aligned; a cached code c of block b, head h stands for
 *   scale[b][h] * value(c).  Scales are chosen by the caller (for instance
 *   when it takes a fresh block) and must be finite and positive for every
 *   block in use; these calls never change them (pa_copy_blocks_fp8 copies
 *   them along with the blocks).
 * q, out, k_new, v_new keep a 16-bit or 32-bit dtype; the pool layout is the
 * one above with 1-byte elements.
 */

/*
 * pa_decode over an 8-bit cache: as pa_decode, with each K element read as
 * k_scales[b][h] * value(code) and each V element as v_scales[b][h] *
 * value(code).  q_dtype (PA_DTYPE_F16 or PA_DTYPE_BF16) is the dtype of q and
 * out; arithmetic is fp32 as in pa_decode (scores sk*<q, k_code>, V weights
 * p*sv).  Workspace: pa_decode_workspace_size() with the same sizes and
 * partition_size, same contract.  Tensor pointers 16-byte aligned, except
 * block_tables, context_lens and the scales (4 bytes).  Returns
 * PA_ERR_UNSUPPORTED for other dtype pairs.
 */
pa_status_t pa_decode_fp8(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, const int32_t* context_lens,
                          float scale, int32_t block_size,
                          int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                          int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t partition_size, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_reshape_and_cache into an 8-bit cache: for i < num_tokens with
 * slot = slot_mapping[i], b = slot / block_size, r = slot % block_size and
 * every head h and element d,
 *   k_pool[b][h][r][d] = Q(k_new[i][h][d] / k_scales[b][h])   (likewise v)
 * where the division is fp32 (correctly rounded) and Q rounds to the nearest
 * kv_dtype value, ties to the even code, saturating beyond the largest finite
 * value (infinities included) and mapping NaN to the code 0x7F; the sign of
 * the quotient is kept (-0 gives 0x80).  new_dtype (F32, F16 or BF16) is the
 * dtype of k_new / v_new.  Slots as in pa_reshape_and_cache (negative or past
 * the pool: no write).
 */
pa_status_t pa_reshape_and_cache_fp8(void* k_pool, void* v_pool,
                                     const float* k_scales, const float* v_scales,
                                     const void* k_new, const void* v_new,
                                     const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, pa_dtype_t new_dtype,
                                     pa_dtype_t kv_dtype, void* stream);

/*
 * pa_copy_blocks for an 8-bit cache: copies the blocks' codes and their
 * per-head K and V scales (k_scales[dst][:] = k_scales[src][:], likewise v).
 * Same pair rules and preconditions as pa_copy_blocks.
 */
pa_status_t pa_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                               const int32_t* block_mapping, int32_t num_pairs,
                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype_t kv_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
