// Internal interface between the C ABI (pa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

#ifndef PA_DEFAULT_PARTITION_TOKENS
#define PA_DEFAULT_PARTITION_TOKENS 512
#endif
#ifndef PA_TARGET_WORKGROUPS
#define PA_TARGET_WORKGROUPS 2048
#endif
#ifndef PA_MIN_PARTITION_BLOCKS
#define PA_MIN_PARTITION_BLOCKS 8
#endif
#ifndef PA_BALANCED_WAVES
#define PA_BALANCED_WAVES 4
#endif
#ifndef PA_BALANCED_WORKGROUPS
#define PA_BALANCED_WORKGROUPS 256
#endif
#ifndef PA_BALANCED_MIN_TILES
#define PA_BALANCED_MIN_TILES 2
#endif

constexpr int kDefaultPartitionTokens = PA_DEFAULT_PARTITION_TOKENS;
constexpr int kMaxGridYZ = 65535;
constexpr int kCopyChunkBytes = 16384;  // bytes one copy_blocks workgroup moves

// Two work decompositions of one decode call:
//  * kBalanced (partition_size 0, at most kBalancedMaxSeqs sequences): a fixed
//    grid whose waves each take an equal contiguous share of all (sequence,
//    head, block) tiles; only rows that straddle a share boundary produce
//    partials.
//  * kPartitioned (partition_size > 0, or more sequences): one workgroup per
//    (head, partition, sequence); every multi-partition row produces one
//    partial per partition.
//  * kMfma (grouped-query heads, a group of 3 to 32 heads, 16-bit q and
//    cache, partition_size 0, at most kBalancedMaxSeqs sequences): items of
//    (sequence, K/V head, partition) on the matrix cores, the group's heads
//    as the rows of a 16-row tile; split rows merged by a second kernel.
enum class DecodeMode { kBalanced, kPartitioned, kMfma };

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  int block_size;
  int num_seqs;
  int num_heads;         // query heads
  int num_kv_heads;      // K/V heads (divides num_heads)
  int group_width;       // kBalanced: query heads per K/V tile load (1, 2 or 4)
  int head_dim;
  int num_blocks;
  int max_blocks_per_seq;
  int dtype;             // pa_dtype_t of q and out
  int kv_dtype;          // pa_dtype_t of the pools (dtype, or an 8-bit format)
  const float* k_scales;  // [num_blocks][H] (8-bit pools only)
  const float* v_scales;
  DecodeMode mode;
  int partition_blocks;  // kPartitioned: blocks per partition
  int max_partitions;    // kPartitioned: ceil(max_blocks_per_seq / partition_blocks)
  int workgroups;        // kBalanced: grid size
  uint32_t* counters;    // [S][H] arrival tickets (null when no row can be split)
  float* ws_ml;          // [slots][2]  (max, sum) of each partial
  float* ws_acc;         // [slots][D]  unnormalised weighted V sum of each partial
  int* ws_off;           // kMfma: [S + 2] item offsets and the partition size, for the merge
  int max_items;         // kMfma: items the workspace holds (slots = max_items * group)
  int mfma_slots;        // kMfma: workgroups resident on the whole GPU at once
  int mfma_fuse;         // kMfma: split rows merged in the kernel (no merge kernel)
  // several query tokens per sequence (pa_prefill through the grouped-query
  // kernel): query_start [S + 1], num_tokens, and the per-token merge
  // descriptors [num_tokens][8]; null / 0 for decode
  const int32_t* query_start;
  int num_tokens;
  int* ws_tok;
};

// Workspace of pa_decode: the ticket counters come first (they must be zero
// when a call starts; every call leaves the ones it used at zero), then the
// partial slots.
struct WorkspaceLayout {
  size_t counter_offset, ml_offset, acc_offset, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WorkspaceLayout workspace_layout(size_t rows, size_t slots, int head_dim) {
  WorkspaceLayout w{0, 0, 0, 0};
  if (slots == 0) return w;
  w.counter_offset = 0;
  w.ml_offset = align_up(rows * sizeof(uint32_t), 256);
  w.acc_offset = align_up(w.ml_offset + slots * 2 * sizeof(float), 256);
  w.total = align_up(w.acc_offset + slots * head_dim * sizeof(float), 256);
  return w;
}

// Partition size when the caller passes 0 but the balanced split does not
// apply: start at kDefaultPartitionTokens and halve while the grid would hold
// fewer than kTargetWorkgroups workgroups (an upper bound: sequences shorter
// than the table width use fewer), but keep at least kMinPartitionBlocks.
constexpr long long kTargetWorkgroups = PA_TARGET_WORKGROUPS;
constexpr int kMinPartitionBlocks = PA_MIN_PARTITION_BLOCKS;

inline int default_partition_blocks(int num_seqs, int num_heads, int max_blocks, int block_size) {
  int pb = kDefaultPartitionTokens / block_size;
  const long long rows = static_cast<long long>(num_seqs) * num_heads;
  while (pb > kMinPartitionBlocks && rows * ((max_blocks + pb - 1) / pb) < kTargetWorkgroups) pb /= 2;
  return pb;
}

// Balanced split: at most kBalancedWorkgroups workgroups of kBalancedWaves
// waves — one workgroup per CU of a 256-CU MI355X.  Measured: several
// workgroups per CU finish at very different times (the older workgroup on a
// CU is served first), so an equal static split only balances when each CU
// runs one; it also keeps just enough bytes in flight.  Fewer workgroups are
// used when the upper bound on tiles
// (num_seqs * num_heads * max_blocks) would leave waves with under
// kBalancedMinTiles tiles each.  The per-sequence prefix sums live in LDS,
// hence the sequence limit.
constexpr int kBalancedMaxSeqs = 2048;
// Cost model of the balanced split: a unit costs kBalancedCostUnit, and each
// row segment a wave walks costs kBalancedCostRow more for the kernels with
// one head per load over a 16-bit or fp32 cache, kBalancedCostRowWide for
// those whose row change folds more state (grouped heads, or 16 elements per
// lane over an 8-bit cache).  Measured: a row change takes about two thirds
// of a 4 KiB unit's time (fp16, D = 128; layer-shape and
// continuous-batching workloads: with the same number of units, a wave that
// walked six rows took ~2 us longer than one that walked one); for the
// others a charge of 10 was fastest (8-bit layer shape 18.6 / 17.3 / 17.0 /
// 16.8 / 16.5 / 16.5 / 16.5 us with charges 0 / 2 / 4 / 6 / 8 / 10 / 12;
// grouped layer shape with 8 K/V heads 20.2 / 19.4 / 19.2 / 19.4 us with
// 6 / 8 / 10 / 12), while the 16-bit kernel is best at 2 (153.7 us against
// 154.5 / 154.8 / 154.0 with 0 / 4 / 6).
constexpr int kBalancedCostUnit = 3;
constexpr int kBalancedCostRow = 2;
constexpr int kBalancedCostRowWide = 10;
// Cost positions stay within int per head and within 2^43 over all rows.  Per
// block the cost is at most (unit + row charge) x units per block: up to 8
// units (fp32, D = 128, BS = 32) at 3 + 2, or up to 2 units (16 or 32 rows)
// at 3 + 10 — the kernel asserts the units per block.
inline bool balanced_cost_fits(long long num_seqs, long long rows, long long max_blocks) {
  constexpr long long c8 = (kBalancedCostUnit + kBalancedCostRow) * 8LL;
  constexpr long long c16 = (kBalancedCostUnit + kBalancedCostRowWide) * 2LL;
  constexpr long long c = c8 > c16 ? c8 : c16;
  return num_seqs * max_blocks * c < (1LL << 31) && rows * max_blocks * c < (1LL << 43);
}
constexpr int kBalancedWaves = PA_BALANCED_WAVES;
constexpr int kBalancedWorkgroups = PA_BALANCED_WORKGROUPS;
constexpr int kBalancedMinTiles = PA_BALANCED_MIN_TILES;

inline int balanced_workgroups(int num_seqs, int num_heads, int max_blocks) {
  const long long tiles = static_cast<long long>(num_seqs) * num_heads * max_blocks;
  const long long per_wg = static_cast<long long>(kBalancedWaves) * kBalancedMinTiles;
  const long long g = (tiles + per_wg - 1) / per_wg;
  return static_cast<int>(g < 1 ? 1 : (g > kBalancedWorkgroups ? kBalancedWorkgroups : g));
}

hipError_t launch_decode_partitioned(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_balanced(const DecodeArgs& a, hipStream_t stream);
// group_width 2, 4
hipError_t launch_decode_balanced_gqa2(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_balanced_gqa4(const DecodeArgs& a, hipStream_t stream);
// grouped-query heads on the matrix cores (kMfma)
constexpr int kMfmaMinGroup = 3;
constexpr int kMfmaMaxGroup = 32;
constexpr int kMfmaMinPartTokens = 128;   // the smallest partition the kernel picks
#ifndef PA_GQ_MAX_PART
#define PA_GQ_MAX_PART 2048
#endif
// Grid bound: the grid is one workgroup per item as far as this allows (the
// hardware starts each on whichever CU frees first; past the bound the
// workgroups take the remaining items by stride).  Continuous batching with
// 8 K/V heads (~1040 items): 47.5 us with 1024, 46.9 with 2048 or 4096.
#ifndef PA_GQ_MAX_WG
#define PA_GQ_MAX_WG 2048
#endif
constexpr int kMfmaMaxPartTokens = PA_GQ_MAX_PART;  // the largest
constexpr int kMfmaMaxWorkgroups = PA_GQ_MAX_WG;
// Workgroups of the kernel resident on one CU: two with one 16-row tile
// (groups of up to 16 heads), one with two (register file).
inline int mfma_wg_per_cu(int group) { return group > 16 ? 1 : 2; }
// Small batches whose contexts are at most this many tokens (the table
// width; at most 64 partitions a row) and whose (sequence, K/V head) rows
// number at most one per kMfmaFuseRowsPerSlot resident workgroups: split
// rows are merged inside the kernel by the item that arrives last, and the
// second kernel (whose launch costs a few microseconds whatever it does) is
// not launched.  Longer contexts can have hundreds of partials per row, more
// than one workgroup folds quickly; larger batches run several items per
// workgroup, each then waiting for its stores and its ticket (layer shape
// with 8 K/V heads 12.6 -> 12.1 us, but continuous batching with 8 / 4
// 46.6 / 32.0 -> 48.9 / 32.5 us when fused); and groups of at most 4 heads:
// one workgroup folds G heads' partials serially, so larger groups lengthen
// the last item more than the second kernel costs (layer shape with 4 / 1
// K/V heads, groups of 8 / 32: 10.1 / 12.6 -> 10.6 / 18.4 us when fused).
constexpr int kMfmaFuseMaxTokens = 64 * kMfmaMinPartTokens;
constexpr int kMfmaFuseRowsPerSlot = 8;
constexpr int kMfmaFuseMaxGroup = 4;
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// the same kernel over several query tokens per sequence (pa_prefill with at
// most kMfmaQueriesMaxSeqs sequences and few rows each): rows (query token, head of the
// group), token-major, in chunks of 16 or 32; causal per row
hipError_t launch_decode_mfma_queries(const DecodeArgs& a, hipStream_t stream);
constexpr int kMfmaQueriesMaxSeqs = 64;  // one lane of a wave per sequence

// Attention of several query rows per (sequence, K/V head) on the matrix
// cores: multi-token queries (pa_prefill) and decode over an MLA latent cache
// (pa_decode_mla, latent == true: 576-element key rows whose first 512
// elements are the values, one K/V head, v_pool == k_pool).  Items are
// (sequence, K/V head, tile of 16 query rows, context partition); each
// workgroup rebuilds the per-sequence item offsets in LDS, hence the sequence
// limit per launch (the host launches once per group of kPfMaxSeqs).
constexpr int kPfMaxSeqs = 2048;
constexpr int kPfMaxWorkgroups = 1024;
constexpr int kMlaQkDim = 576;  // latent 512 + rotary 64 (DeepSeek-V2/V3)
constexpr int kMlaVDim = 512;

struct PrefillArgs {
  void* out;                    // [T][H][DV]
  const void* q;                // [T][H][DQK]
  const void* k_pool;           // [num_blocks][Hkv][BS][DQK]
  const void* v_pool;           // [num_blocks][Hkv][BS][DV] (latent: == k_pool)
  const int32_t* block_tables;  // [S][W]
  const int32_t* context_lens;  // [S]
  const int32_t* query_start;   // [S+1]; null: one query row per sequence
  float scale;
  int block_size, num_seqs, num_query_rows, num_heads, num_kv_heads, head_dim, num_blocks,
      max_blocks_per_seq;
  int dtype;        // PA_DTYPE_F16 or PA_DTYPE_BF16
  bool latent;
  int part_tokens;  // keys per context partition (multiple of 16)
  int row_tiles;    // 16-row tiles per wave (1 or 2; latent: 1)
  int max_items;    // workspace capacity in items; the kernel never goes past it
  int workgroups;
  uint32_t* counters;  // [max_items] (null when no row can be split)
  float* ws_ml;        // [max_items][16 * row_tiles][2]
  float* ws_acc;       // [max_items][16 * row_tiles][DV]
  int* ws_off;         // mla_heads: [S + 2] item offsets and the partition size, for the merge
  int slots;           // mla_heads: CUs of the device
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// many query rows per sequence and the default split (one partition): one
// workgroup per block of 128 rows of a (sequence, K/V head), the keys and
// values of each step staged in LDS by direct loads (pa_prefill_tiles.hip)
constexpr int kPfTileRows = 128;
hipError_t launch_prefill_tiles(const PrefillArgs& a, hipStream_t stream);
// the latent cache: one workgroup per (sequence, 16 heads, partition), the
// 576 elements of a row split across its four waves
hipError_t launch_mla_split(const PrefillArgs& a, hipStream_t stream);
// the latent cache under the default split (up to kMlaHeadsMaxSeqs
// sequences): items (sequence, partition of 256..4096 tokens, up to 64
// heads), one workgroup per CU, each wave 16 heads over the whole row, the
// rows staged in LDS once per workgroup; split rows merged by a second kernel
constexpr int kMlaHeadsGroup = 64;      // heads per workgroup
constexpr int kMlaHeadsMinPart = 256;   // partition sizes (tokens, multiples of 32)
constexpr int kMlaHeadsMaxPart = 4096;
constexpr int kMlaHeadsMaxSeqs = 512;   // per-sequence offsets in LDS beside the rows and queries
hipError_t launch_mla_heads(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_reshape_and_cache(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                    const int32_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int num_blocks, hipStream_t stream);

// Whole-block copies src[s] -> dst[d] (K and V pools); the pools may be the
// same (copy-on-write) or different (swap to / from host memory).  Scales:
// [blocks][num_heads] per-block scales copied along (8-bit pools), or null.
struct CopyArgs {
  void* dst_k;
  void* dst_v;
  const void* src_k;
  const void* src_v;
  float* dst_ks;
  float* dst_vs;
  const float* src_ks;
  const float* src_vs;
  const int32_t* block_mapping;
  int num_pairs;
  size_t block_bytes;
  int src_blocks, dst_blocks, num_heads;
};
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

struct ReshapeFp8Args {
  void* k_pool;
  void* v_pool;
  const float* k_scales;
  const float* v_scales;
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int num_tokens, num_heads, head_dim, block_size, num_blocks;
  int in_dtype;  // pa_dtype_t of k_new / v_new
  int kv_dtype;  // PA_DTYPE_FP8_E4M3 or PA_DTYPE_FP8_E5M2
};
hipError_t launch_reshape_and_cache_fp8(const ReshapeFp8Args& a, hipStream_t stream);

}  // namespace pa
