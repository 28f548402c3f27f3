// Internal interface between the C ABI (pa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kDefaultPartitionTokens = 512;
constexpr int kMaxGridYZ = 65535;
constexpr int kCopyChunkBytes = 16384;  // bytes one copy_blocks workgroup moves

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
  int num_heads;
  int head_dim;
  int num_blocks;
  int max_blocks_per_seq;
  int partition_blocks;  // blocks per partition
  int max_partitions;    // ceil(max_blocks_per_seq / partition_blocks)
  int dtype;             // pa_dtype_t
  uint32_t* counters;    // [S][H] arrival tickets — null when max_partitions == 1
  float* ws_ml;          // [S][H][max_partitions][2]  (max, sum)
  float* ws_acc;         // [S][H][max_partitions][D]  unnormalised weighted V sums
};

// Workspace of pa_decode: the ticket counters come first (they must be zero
// when a call starts; every call leaves the ones it used at zero), then the
// per-partition softmax partials.
struct WorkspaceLayout {
  size_t counter_offset, ml_offset, acc_offset, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WorkspaceLayout workspace_layout(int num_seqs, int num_heads, int head_dim, int max_partitions) {
  WorkspaceLayout w{0, 0, 0, 0};
  if (max_partitions <= 1) return w;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads;
  w.counter_offset = 0;
  w.ml_offset = align_up(rows * sizeof(uint32_t), 256);
  w.acc_offset = align_up(w.ml_offset + rows * max_partitions * 2 * sizeof(float), 256);
  w.total = align_up(w.acc_offset + rows * max_partitions * head_dim * sizeof(float), 256);
  return w;
}

// Partition size when the caller passes 0: start at kDefaultPartitionTokens and
// halve while the grid would hold fewer than kTargetWorkgroups workgroups (an
// upper bound: sequences shorter than the table width use fewer), but keep at
// least kMinPartitionBlocks blocks so every wave pipelines two tile groups.
constexpr long long kTargetWorkgroups = 2048;
constexpr int kMinPartitionBlocks = 8;

inline int default_partition_blocks(int num_seqs, int num_heads, int max_blocks, int block_size) {
  int pb = kDefaultPartitionTokens / block_size;
  const long long rows = static_cast<long long>(num_seqs) * num_heads;
  while (pb > kMinPartitionBlocks && rows * ((max_blocks + pb - 1) / pb) < kTargetWorkgroups) pb /= 2;
  return pb;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_reshape_and_cache(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                    const int32_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping, int num_pairs,
                              size_t block_bytes, int num_blocks, hipStream_t stream);

}  // namespace pa
