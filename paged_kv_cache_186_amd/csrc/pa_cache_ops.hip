// Cache maintenance kernels: slot writes and whole-block copies (gfx950).
//
// Both are byte copies (bit-exact for every dtype) moved as 16-byte lane
// vectors, so each wave instruction moves 1 KiB.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kCopyVecs = 4;                                 // vectors per thread per chunk
constexpr int kCopyChunk = kThreads * kCopyVecs * kVecBytes;  // 16 KiB per workgroup
static_assert(kCopyChunk == kCopyChunkBytes, "host sizing and kernel agree");

// One workgroup per new token: write its K and V rows (all heads) into row
// slot % BS of physical block slot / BS.  Source: vLLM tutorial page
// "3. PagedAttention原理" §3.3.2 (a new token fills the next free row of the
// sequence's last block, or row 0 of a freshly taken block).  Slots that are
// negative or past the pool are skipped.
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ slot_mapping, int num_heads,
    int row_bytes, int block_size, long long num_slots) {
  const int t = blockIdx.x;
  const int slot = slot_mapping[t];
  if (slot < 0 || static_cast<long long>(slot) >= num_slots) return;
  const int blk = slot / block_size;
  const int r = slot % block_size;
  const int vecs_per_row = row_bytes / kVecBytes;
  const int total = num_heads * vecs_per_row;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int hh = i / vecs_per_row;
    const int c = i % vecs_per_row;
    const size_t src = (static_cast<size_t>(t) * num_heads + hh) * row_bytes + c * kVecBytes;
    const size_t dst =
        ((static_cast<size_t>(blk) * num_heads + hh) * block_size + r) * row_bytes + c * kVecBytes;
    const u32x4 kv = load16(k_new + src);
    const u32x4 vv = load16(v_new + src);
    store16(k_pool + dst, kv);
    store16(v_pool + dst, vv);
  }
}

// Copy-on-write copy: pool[dst] = pool[src] for every {src, dst} pair, for both
// pools (blockIdx.y selects K or V).  Grid x enumerates (pair, 16 KiB chunk).
// Source: page "mlx-paged-attention: Bringing vLLM-level High Throughput
// Inference to Apple Silicon", core feature 2.  Pairs naming an id outside the
// pool are skipped.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const int32_t* __restrict__ block_mapping,
    size_t block_bytes, int chunks_per_block, int num_blocks) {
  const int pair = blockIdx.x / chunks_per_block;
  const int chunk = blockIdx.x % chunks_per_block;
  char* pool = blockIdx.y ? v_pool : k_pool;
  const int src = block_mapping[2 * pair + 0];
  const int dst = block_mapping[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(num_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(num_blocks))
    return;
  const char* from = pool + static_cast<size_t>(src) * block_bytes;
  char* to = pool + static_cast<size_t>(dst) * block_bytes;
  const size_t base = static_cast<size_t>(chunk) * kCopyChunk + threadIdx.x * kVecBytes;
  u32x4 v[kCopyVecs];
#pragma unroll
  for (int u = 0; u < kCopyVecs; ++u) {
    const size_t off = base + static_cast<size_t>(u) * kThreads * kVecBytes;
    if (off < block_bytes) v[u] = load16(from + off);
  }
#pragma unroll
  for (int u = 0; u < kCopyVecs; ++u) {
    const size_t off = base + static_cast<size_t>(u) * kThreads * kVecBytes;
    if (off < block_bytes) store16(to + off, v[u]);
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                    const int32_t* slot_mapping, int num_tokens, int num_heads,
                                    int row_bytes, int block_size, int num_blocks,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kThreads), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), slot_mapping,
                     num_heads, row_bytes, block_size,
                     static_cast<long long>(num_blocks) * block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping, int num_pairs,
                              size_t block_bytes, int num_blocks, hipStream_t stream) {
  const int chunks = static_cast<int>((block_bytes + kCopyChunk - 1) / kCopyChunk);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs * chunks, 2), dim3(kThreads), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), block_mapping,
                     block_bytes, chunks, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
