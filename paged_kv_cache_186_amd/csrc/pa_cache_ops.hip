// Cache maintenance kernels: slot writes and whole-block copies (gfx950).
//
// Both are byte copies (bit-exact for every dtype) moved as 16-byte lane
// vectors, so each wave instruction moves 1 KiB.

#include "pa_device.h"
#include "pa_internal.h"
#include "pagedattn.h"

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

// The same slot write for an 8-bit cache: every element of the new token's
// K/V row (storage IT) becomes the code of x / scale[blk][head] (an fp32
// division, correctly rounded), rounded to the nearest value with ties to
// even and saturated to the largest finite value (QFn).  One thread makes 16
// codes — one 16-byte store — from 16 input elements.  The quantization is
// this library's reading: the pages name quantization only as future work
// (page "mlx-paged-attention: Bringing vLLM-level High Throughput Inference
// to Apple Silicon", future plans).
template <typename IT, uint32_t (*QFn)(float)>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, const typename IT::storage* __restrict__ k_new,
    const typename IT::storage* __restrict__ v_new, const int32_t* __restrict__ slot_mapping,
    int num_heads, int head_dim, int block_size, long long num_slots) {
  constexpr int kCodes = 16;                        // codes per thread step
  constexpr int kInVecs = kCodes / IT::kElems;      // 16-byte input vectors per step
  const int t = blockIdx.x;
  const int slot = slot_mapping[t];
  if (slot < 0 || static_cast<long long>(slot) >= num_slots) return;
  const int blk = slot / block_size;
  const int r = slot % block_size;
  const int vecs_per_row = head_dim / kCodes;
  const int total = num_heads * vecs_per_row;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int hh = i / vecs_per_row;
    const int c = i % vecs_per_row;
    const size_t src = (static_cast<size_t>(t) * num_heads + hh) * head_dim + c * kCodes;
    const size_t dst = ((static_cast<size_t>(blk) * num_heads + hh) * block_size + r) * head_dim + c * kCodes;
    const float sk = k_scales[static_cast<size_t>(blk) * num_heads + hh];
    const float sv = v_scales[static_cast<size_t>(blk) * num_heads + hh];
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const typename IT::storage* in = (kv ? v_new : k_new) + src;
      const float sc = kv ? sv : sk;
      float x[kCodes];
#pragma unroll
      for (int u = 0; u < kInVecs; ++u) IT::unpack(load16(in + u * IT::kElems), x + u * IT::kElems);
      u32x4 w;
      uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) word |= QFn(x[4 * q + b] / sc) << (8 * b);
        wp[q] = word;
      }
      store16((kv ? v_pool : k_pool) + dst, w);
    }
  }
}

// Whole-block copy from a source pool pair to a destination pool pair:
// dst[d] = src[s] for every {s, d} pair, in the K and V pools (blockIdx.y
// selects which), and for an 8-bit cache the block's per-head scales too.
// Grid x enumerates (pair, 16 KiB chunk).  Source and destination are the
// same pools for copy-on-write (page "mlx-paged-attention: Bringing vLLM-level
// High Throughput Inference to Apple Silicon", core feature 2) and different
// pools — one of them in GPU-mapped pinned host memory — for swapping a
// sequence's cache out and back in (page "PagedAttention MLX：为Apple
// Silicon打造的高吞吐量LLM推理引擎", dynamic scheduling and the physical KV
// pool's swap-out).  Every chunk is read into registers before any of it is
// written, and many chunks are in flight at once, which is what a host link
// needs to run at speed.  Pairs naming an id outside either pool are skipped.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* dst_k, char* dst_v, const char* src_k, const char* src_v, float* dst_ks, float* dst_vs,
    const float* src_ks, const float* src_vs, const int32_t* __restrict__ block_mapping,
    size_t block_bytes, int chunks_per_block, int src_blocks, int dst_blocks, int num_heads) {
  const int pair = blockIdx.x / chunks_per_block;
  const int chunk = blockIdx.x % chunks_per_block;
  const int src = block_mapping[2 * pair + 0];
  const int dst = block_mapping[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(src_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(dst_blocks))
    return;
  const float* sscale = blockIdx.y ? src_vs : src_ks;
  float* dscale = blockIdx.y ? dst_vs : dst_ks;
  if (sscale != nullptr && chunk == 0)
    for (int i = threadIdx.x; i < num_heads; i += kThreads)
      dscale[static_cast<size_t>(dst) * num_heads + i] = sscale[static_cast<size_t>(src) * num_heads + i];
  const char* from = (blockIdx.y ? src_v : src_k) + static_cast<size_t>(src) * block_bytes;
  char* to = (blockIdx.y ? dst_v : dst_k) + static_cast<size_t>(dst) * block_bytes;
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

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  const int chunks = static_cast<int>((a.block_bytes + kCopyChunk - 1) / kCopyChunk);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs * chunks, 2), dim3(kThreads), 0, stream,
                     static_cast<char*>(a.dst_k), static_cast<char*>(a.dst_v),
                     static_cast<const char*>(a.src_k), static_cast<const char*>(a.src_v), a.dst_ks,
                     a.dst_vs, a.src_ks, a.src_vs, a.block_mapping, a.block_bytes, chunks,
                     a.src_blocks, a.dst_blocks, a.num_heads);
  return hipGetLastError();
}

namespace {
template <typename IT>
hipError_t run_reshape_fp8(const ReshapeFp8Args& a, hipStream_t stream) {
  using S = typename IT::storage;
  const long long slots = static_cast<long long>(a.num_blocks) * a.block_size;
  if (a.kv_dtype == PA_DTYPE_FP8_E4M3)
    hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<IT, quantize_e4m3>), dim3(a.num_tokens),
                       dim3(kThreads), 0, stream, static_cast<uint8_t*>(a.k_pool),
                       static_cast<uint8_t*>(a.v_pool), a.k_scales, a.v_scales,
                       static_cast<const S*>(a.k_new), static_cast<const S*>(a.v_new), a.slot_mapping,
                       a.num_heads, a.head_dim, a.block_size, slots);
  else
    hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<IT, quantize_e5m2>), dim3(a.num_tokens),
                       dim3(kThreads), 0, stream, static_cast<uint8_t*>(a.k_pool),
                       static_cast<uint8_t*>(a.v_pool), a.k_scales, a.v_scales,
                       static_cast<const S*>(a.k_new), static_cast<const S*>(a.v_new), a.slot_mapping,
                       a.num_heads, a.head_dim, a.block_size, slots);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_reshape_and_cache_fp8(const ReshapeFp8Args& a, hipStream_t stream) {
  switch (a.in_dtype) {
    case PA_DTYPE_F32:
      return run_reshape_fp8<F32>(a, stream);
    case PA_DTYPE_F16:
      return run_reshape_fp8<F16>(a, stream);
    default:
      return run_reshape_fp8<BF16>(a, stream);
  }
}

}  // namespace pa
