// C ABI of libpagedattn: argument validation, sizing and dispatch.
//
// Every check here runs on the host before anything is enqueued; a failed
// check returns a status and launches nothing.  No allocation; the only state
// is the per-device address of pa_decode_noalloc's static scratch array.

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa_internal.h"
#include "pagedattn.h"

namespace {

constexpr int32_t kAbiVersion = 3;

// Bytes of one element of a 16/32-bit dtype (0 for anything else).
int elem_bytes(pa_dtype_t dtype) {
  switch (dtype) {
    case PA_DTYPE_F32:
      return 4;
    case PA_DTYPE_F16:
    case PA_DTYPE_BF16:
      return 2;
    default:
      return 0;
  }
}

bool is_fp8(pa_dtype_t dtype) { return dtype == PA_DTYPE_FP8_E4M3 || dtype == PA_DTYPE_FP8_E5M2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_shape(int head_dim, int block_size) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

// Blocks per partition, or 0 when partition_size is not a positive multiple of
// block_size.  0 lets the library choose from the shape.
int partition_blocks(int partition_size, int num_seqs, int num_heads, int max_blocks,
                     int block_size) {
  if (partition_size == 0)
    return pa::default_partition_blocks(num_seqs, num_heads, max_blocks, block_size);
  if (partition_size < 0 || partition_size % block_size != 0) return 0;
  return partition_size / block_size;
}

struct DecodePlan {
  pa_status_t status;
  pa::DecodeMode mode;
  int part_blocks;
  int max_parts;
  int workgroups;
  int group_width;
  size_t rows;   // arrival counters: one per (sequence, query head)
  size_t slots;  // partial slots (each of head_dim fp32 sums and a (max, sum) pair)
  int max_items;     // kMfma: items the workspace holds
  int mfma_slots;    // kMfma: workgroups resident at once
  int mfma_fuse;     // kMfma: split rows merged in the kernel
  size_t off_offset; // kMfma: byte offset of the item offsets in the workspace
  pa::WorkspaceLayout ws;
};

// Compute units of the current device (256 on an MI355X), asked once per
// device; 256 if HIP cannot tell (the sizes then stay valid, only the
// partition choice of the grouped-query kernel is less tuned).
int cu_count() {
  static std::mutex mu;
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

// Query heads that one K/V tile load serves in the balanced kernel: 4 or 2,
// the largest dividing the group size, for 16-bit queries; 1 otherwise.  A
// group of 8 or more is served by several work rows of 4 heads each, which
// read the same tiles (the second and later from L2).  Measured against a
// kernel serving 8 heads per load: layer shape with 4 / 1 K/V heads 41.7 /
// 40.8 us -> 23.0 / 23.0 us, continuous batching 63.3 / 62.1 -> 49.9 / 49.2
// us, 128K context 197 / 193 -> 98.6 / 98.0 us (8 heads' state per lane
// left too few registers: 2.3 us per 16-row unit and a long merge tail).
int group_width(int num_heads, int num_kv_heads, pa_dtype_t dtype, pa_dtype_t kv_dtype) {
  (void)kv_dtype;
  const int g = num_heads / num_kv_heads;
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return 1;
  for (int w : {4, 2})
    if (g % w == 0) return w;
  return 1;
}

// partition_size 0 selects the balanced split whenever it applies (at most
// kBalancedMaxSeqs sequences); otherwise, or with an explicit partition size,
// the partitioned kernel runs.  Balanced work rows are (sequence, group of
// group_width query heads); each partial slot holds group_width partials.
DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t partition_size, pa_dtype_t dtype, pa_dtype_t kv_dtype) {
  DecodePlan p{PA_OK, pa::DecodeMode::kPartitioned, 0, 0, 0, 1, 0, 0, 0, 0, 0, 0, {0, 0, 0, 0}};
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  if (!supported_shape(head_dim, block_size)) {
    p.status = PA_ERR_UNSUPPORTED;
    return p;
  }
  if (num_seqs > pa::kMaxGridYZ || num_heads > pa::kMaxGridYZ ||
      max_blocks_per_seq > INT_MAX / block_size) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads;
  const int group = num_heads / num_kv_heads;
  if (partition_size == 0 && num_seqs <= pa::kBalancedMaxSeqs && group >= pa::kMfmaMinGroup &&
      group <= pa::kMfmaMaxGroup && (dtype == PA_DTYPE_F16 || dtype == PA_DTYPE_BF16) && kv_dtype == dtype) {
    // the group's heads as the rows of matrix-core tiles; items (sequence,
    // K/V head, partition), the partition (>= 128 tokens) chosen on the device
    p.mode = pa::DecodeMode::kMfma;
    const long long ctx = static_cast<long long>(max_blocks_per_seq) * block_size;
    const long long parts = (ctx + pa::kMfmaMinPartTokens - 1) / pa::kMfmaMinPartTokens;
    const long long items = static_cast<long long>(num_seqs) * num_kv_heads * parts;
    if (items > INT_MAX / pa::kMfmaMaxGroup) {
      p.status = PA_ERR_INVALID_ARG;
      return p;
    }
    p.max_items = static_cast<int>(items);
    // grid: the items of the partition the kernel would pick if every
    // sequence filled the table (more items: workgroups take several)
    p.mfma_slots = cu_count() * pa::mfma_wg_per_cu(group);
    const long long per_slot = static_cast<long long>(num_seqs) * num_kv_heads * ctx / p.mfma_slots;
    int pt = pa::kMfmaMaxPartTokens;
    while (pt > pa::kMfmaMinPartTokens && pt > per_slot) pt /= 2;
    const long long grid = static_cast<long long>(num_seqs) * num_kv_heads * ((ctx + pt - 1) / pt);
    p.workgroups = static_cast<int>(grid < 1 ? 1 : (grid > pa::kMfmaMaxWorkgroups ? pa::kMfmaMaxWorkgroups : grid));
    p.rows = rows;
    if (ctx > pa::kMfmaMinPartTokens) {  // a row can span several partitions
      p.mfma_fuse = (ctx <= pa::kMfmaFuseMaxTokens && group <= pa::kMfmaFuseMaxGroup &&
                     static_cast<long long>(num_seqs) * num_kv_heads * pa::kMfmaFuseRowsPerSlot <= p.mfma_slots)
                        ? 1
                        : 0;
      p.slots = static_cast<size_t>(items) * group;
      p.ws = pa::workspace_layout(rows, p.slots, head_dim);
      p.off_offset = p.ws.total;
      p.ws.total = pa::align_up(p.ws.total + (static_cast<size_t>(num_seqs) + 2) * sizeof(int), 256);
    }
    return p;
  }
  if (partition_size == 0 && num_seqs <= pa::kBalancedMaxSeqs &&
      pa::balanced_cost_fits(num_seqs, static_cast<long long>(rows), max_blocks_per_seq)) {
    p.mode = pa::DecodeMode::kBalanced;
    p.group_width = group_width(num_heads, num_kv_heads, dtype, kv_dtype);
    const int row_heads = num_heads / p.group_width;
    const size_t wrows = static_cast<size_t>(num_seqs) * row_heads;
    p.workgroups = pa::balanced_workgroups(num_seqs, row_heads, max_blocks_per_seq);
    const size_t slots = static_cast<size_t>(p.workgroups) * pa::kBalancedWaves + wrows;
    // the counter region is sized for one counter per (sequence, query head)
    // whatever the grouping (only the first wrows are used here), so that
    // every call with the same num_seqs * num_heads lays the workspace out
    // with its partials after the same counter region: calls of different
    // kinds can share one workspace without a partial landing on a counter
    p.rows = rows;
    p.slots = slots * p.group_width;
    p.ws = pa::workspace_layout(rows, p.slots, head_dim);
    return p;
  }
  p.part_blocks =
      partition_blocks(partition_size, num_seqs, num_heads, max_blocks_per_seq, block_size);
  if (p.part_blocks == 0) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  p.max_parts = (max_blocks_per_seq + p.part_blocks - 1) / p.part_blocks;
  if (p.max_parts > pa::kMaxGridYZ) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  const size_t slots = p.max_parts > 1 ? rows * p.max_parts : 0;
  p.rows = rows;
  p.slots = slots;
  p.ws = pa::workspace_layout(rows, slots, head_dim);
  return p;
}

// ---- static scratch of pa_decode_noalloc -----------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the partials and arrival counters live in this file-scope device
// array instead of a caller workspace.  Each GPU holds its own copy of it for
// the life of the process.  Its first kStaticCounterBytes hold the counters
// of every call at a fixed place, so the partials of one call never land on
// another call's counters; every call leaves its counters zero.
constexpr size_t kStaticScratchBytes = size_t(PA_NOALLOC_SCRATCH_BYTES);
constexpr size_t kStaticMaxRows = size_t(PA_NOALLOC_MAX_ROWS);
constexpr size_t kStaticCounterBytes = kStaticMaxRows * sizeof(uint32_t);
static_assert(kStaticCounterBytes % 256 == 0, "counter region keeps the partials 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` on each GPU, once set up

__global__ void zero_words_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Counter region fixed at the start, partials after it; total 0 when the
// call does not fit.
pa::WorkspaceLayout static_scratch_layout(size_t rows, size_t slots, int head_dim) {
  pa::WorkspaceLayout w{0, 0, 0, 0};
  if (rows > kStaticMaxRows) return w;
  const size_t ml = kStaticCounterBytes;
  const size_t acc = pa::align_up(ml + slots * 2 * sizeof(float), 256);
  const size_t total = pa::align_up(acc + slots * static_cast<size_t>(head_dim) * sizeof(float), 256);
  if (total > kStaticScratchBytes) return w;
  w.counter_offset = 0;
  w.ml_offset = ml;
  w.acc_offset = acc;
  w.total = total;
  return w;
}

// The current device's address of `scratch`.  On the first call on a device
// the address is looked up with hipGetSymbolAddress and the counter region is
// cleared by a fill kernel on `stream` (ordered before the decode that
// follows on the same stream).
pa_status_t static_scratch_ready(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream,
                       static_cast<uint4*>(ptr), kStaticCounterBytes / sizeof(uint4));
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// Shared by pa_decode (kv_dtype == dtype, no scales) and pa_decode_fp8; the
// caller has checked the dtype pair.
pa_status_t decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                        const float* k_scales, const float* v_scales,
                        const int32_t* block_tables, const int32_t* context_lens, float scale,
                        int32_t block_size, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                        pa_dtype_t kv_dtype, void* workspace, size_t workspace_bytes,
                        void* stream, bool static_scratch = false) {
  const DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                                      max_blocks_per_seq, block_size, partition_size, dtype,
                                      kv_dtype);
  if (plan.status != PA_OK) return plan.status;
  pa::WorkspaceLayout layout = plan.ws;
  if (static_scratch && plan.ws.total > 0) {
    layout = static_scratch_layout(plan.rows, plan.slots, head_dim);
    if (layout.total == 0) return PA_ERR_TOO_LARGE;
  }
  if (num_blocks <= 0 || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (is_fp8(kv_dtype) && (!k_scales || !v_scales || !aligned(k_scales, 4) || !aligned(v_scales, 4)))
    return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  if (static_scratch && plan.ws.total > 0) {
    void* scratch_ptr = nullptr;
    const pa_status_t st = static_scratch_ready(static_cast<hipStream_t>(stream), &scratch_ptr);
    if (st != PA_OK) return st;
    workspace = scratch_ptr;
    workspace_bytes = kStaticScratchBytes;
  }
  if (layout.total > 0) {
    if (!workspace || workspace_bytes < layout.total) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
  }

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale = scale;
  a.block_size = block_size;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group_width = plan.group_width;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.dtype = dtype;
  a.kv_dtype = kv_dtype;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.mode = plan.mode;
  a.partition_blocks = plan.part_blocks;
  a.max_partitions = plan.max_parts;
  a.workgroups = plan.workgroups;
  a.max_items = plan.max_items;
  a.mfma_slots = plan.mfma_slots;
  a.mfma_fuse = plan.mfma_fuse;
  if (layout.total > 0) {
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<uint32_t*>(ws + layout.counter_offset);
    a.ws_ml = reinterpret_cast<float*>(ws + layout.ml_offset);
    a.ws_acc = reinterpret_cast<float*>(ws + layout.acc_offset);
    if (plan.mode == pa::DecodeMode::kMfma) a.ws_off = reinterpret_cast<int*>(ws + plan.off_offset);
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = plan.mode == pa::DecodeMode::kBalanced ? pa::launch_decode_balanced(a, hs)
                       : plan.mode == pa::DecodeMode::kMfma   ? pa::launch_decode_mfma(a, hs)
                                                              : pa::launch_decode_partitioned(a, hs);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---- multi-token queries and the latent cache (matrix-core kernel) ----------

struct PrefillPlan {
  pa_status_t status;
  int part_tokens;
  long long max_items;  // over all launches of the call (the workspace holds this many)
  int workgroups;
  pa::WorkspaceLayout ws;
};

constexpr long long kPfTargetItems = 2048;  // ~2 waves per SIMD of a 256-CU GPU
// Default partition when contexts are split (measured on 64 sequences of
// log-normal lengths, 4 query tokens, 8 K/V heads: 256 keys 86 us, 512 keys
// 90 us, 1024 keys 70 us, 2048 keys 101 us; the latent kernel on 32
// sequences of 1024..8192 tokens, 16 heads: 512 keys 150 us, 768 keys 96 us,
// 1024 keys 102 us, 2048 keys 156 us)
constexpr int kPfPartTokens = 1024;
constexpr int kPfPartTokensLatent = 768;
constexpr int kPfMaxDefaultParts = 64;     // ... but no row merges more partials than this

// 16-row tiles per wave: two when the sequences have at least 32 query rows
// per K/V head on average (each K/V load then feeds twice the matrix work),
// else one.  The latent cache always takes one (register budget).
int prefill_row_tiles(int32_t num_seqs, int32_t num_query_rows, int32_t num_heads, int32_t num_kv_heads,
                      bool latent) {
  if (latent || num_seqs <= 0) return 1;
  const long long rows = static_cast<long long>(num_query_rows) * (num_heads / num_kv_heads);
  return rows >= 32LL * num_seqs ? 2 : 1;
}

// Items are (sequence, K/V head, group of row_tiles 16-row tiles, value
// slice, partition).  Their number is bounded from host-known sizes: the
// tile groups of a call are at most ceil(T*G/(16*row_tiles)) + S (a
// sequence's partial group adds at most one), partitions at most
// ceil(W*BS / part_tokens).  partition_size 0 splits the context only when
// the unsplit items would not fill the GPU, into partitions of 1024 keys (768
// for the latent cache; fewer, larger ones beyond 64 partitions).
PrefillPlan plan_prefill(int32_t num_seqs, int32_t num_query_rows, int32_t num_heads,
                         int32_t num_kv_heads, int32_t max_blocks_per_seq, int32_t block_size,
                         int32_t partition_size, int32_t v_per_item, int32_t slices, int32_t row_tiles,
                         bool wg_items = false) {
  PrefillPlan p{PA_OK, 0, 0, 0, {0, 0, 0, 0}};
  if (num_seqs < 0 || num_query_rows < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || max_blocks_per_seq <= 0 ||
      max_blocks_per_seq > INT_MAX / block_size / 2) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  const long long ctx = static_cast<long long>(max_blocks_per_seq) * block_size;
  const long long group = num_heads / num_kv_heads;
  const long long group_rows = 16LL * row_tiles;
  const long long tiles = (static_cast<long long>(num_query_rows) * group + group_rows - 1) / group_rows + num_seqs;
  const long long base = tiles * num_kv_heads * slices;
  // an item of the latent kernel is a whole workgroup: a quarter as many fill the GPU
  const long long target = wg_items ? kPfTargetItems / 4 : kPfTargetItems;
  if (partition_size == 0) {
    if (base >= target) {
      p.part_tokens = static_cast<int>((ctx + 31) / 32 * 32);  // one partition
    } else {
      const long long spread = (ctx + kPfMaxDefaultParts - 1) / kPfMaxDefaultParts;
      const long long dflt = wg_items ? kPfPartTokensLatent : kPfPartTokens;
      const long long per = spread > dflt ? spread : dflt;
      p.part_tokens = static_cast<int>((per + 31) / 32 * 32);
    }
  } else {
    if (partition_size < 0 || partition_size % 16 != 0) {
      p.status = PA_ERR_INVALID_ARG;
      return p;
    }
    p.part_tokens = partition_size;
  }
  const long long max_parts = (ctx + p.part_tokens - 1) / p.part_tokens;
  p.max_items = base * max_parts;
  if (p.max_items > INT_MAX / 16) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  // a multiple of 8 workgroups: the kernel gives each XCD an equal share
  const long long wg = ((wg_items ? p.max_items : (p.max_items + 3) / 4) + 7) / 8 * 8;
  p.workgroups = static_cast<int>(wg < 8 ? 8 : (wg > pa::kPfMaxWorkgroups ? pa::kPfMaxWorkgroups : wg));
  if (max_parts > 1)
    p.ws = pa::workspace_layout(static_cast<size_t>(p.max_items),
                                static_cast<size_t>(p.max_items) * group_rows, v_per_item);
  return p;
}

// pa_decode_mla under the default split: items (sequence, partition, group
// of up to 64 heads), the partition (256..4096 tokens) chosen on the device;
// the workspace holds every item's 64 partials and the item offsets the
// merge kernel reads.  At most kMlaHeadsMaxSeqs sequences (more, or an
// explicit partition size, take the split kernel).  Measured against the
// split kernel on 32 sequences of 1K-8K tokens: 65-67 us for 1 to 16 heads
// (95-96 us), 72 us for 32 (150 us).
bool use_mla_heads(int32_t num_seqs, int32_t num_heads, int32_t partition_size) {
  return partition_size == 0 && num_heads > 0 && num_seqs <= pa::kMlaHeadsMaxSeqs;
}

struct MlaHeadsPlan {
  pa_status_t status;
  int max_items;
  int workgroups;
  size_t off_offset;
  pa::WorkspaceLayout ws;
};

MlaHeadsPlan plan_mla_heads(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq, int32_t block_size,
                            bool sizes_only) {
  MlaHeadsPlan p{PA_OK, 0, 0, 0, {0, 0, 0, 0}};
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > INT_MAX / block_size / 2 ||
      num_seqs > pa::kMlaHeadsMaxSeqs) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  const long long ctx = static_cast<long long>(max_blocks_per_seq) * block_size;
  const long long groups = (num_heads + pa::kMlaHeadsGroup - 1) / pa::kMlaHeadsGroup;
  // the kernel picks its partition P on the device: below the largest size
  // only when that leaves at most one item per resident workgroup (one per
  // CU), so the items number at most max(slots, rows * ceil(ctx / largest))
  // and never more than at the smallest size
  const long long rows = static_cast<long long>(num_seqs) * groups;
  const long long slots = cu_count();
  const long long at_min = rows * ((ctx + pa::kMlaHeadsMinPart - 1) / pa::kMlaHeadsMinPart);
  const long long at_max = rows * ((ctx + pa::kMlaHeadsMaxPart - 1) / pa::kMlaHeadsMaxPart);
  const long long items = std::min(at_min, std::max(slots, at_max));
  if (items > INT_MAX / pa::kMlaHeadsGroup) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  p.max_items = static_cast<int>(items);
  if (!sizes_only) {
    const long long grid = std::min(items, slots);
    p.workgroups = static_cast<int>(grid < 1 ? 1 : grid);
  }
  if (ctx > pa::kMlaHeadsMinPart) {  // a row can span several partitions
    // per item and head the partial's (max, sum) in fp32 and its 512
    // normalised values in the output type (2 bytes); then the S + 2 item
    // offsets and partition size the merge reads
    const size_t slots_n = static_cast<size_t>(items) * pa::kMlaHeadsGroup;
    p.ws.ml_offset = 0;
    p.ws.acc_offset = pa::align_up(slots_n * 2 * sizeof(float), 256);
    p.off_offset = pa::align_up(p.ws.acc_offset + slots_n * pa::kMlaVDim * 2, 256);
    p.ws.total = pa::align_up(p.off_offset + (static_cast<size_t>(num_seqs) + 2) * sizeof(int), 256);
  }
  return p;
}

pa_status_t mla_heads_impl(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                           const int32_t* context_lens, float scale, int32_t block_size, int32_t num_seqs,
                           int32_t num_heads, int32_t num_blocks, int32_t max_blocks_per_seq, pa_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (num_seqs > pa::kMlaHeadsMaxSeqs) return PA_ERR_INVALID_ARG;
  const MlaHeadsPlan plan = plan_mla_heads(num_seqs, num_heads, max_blocks_per_seq, block_size, false);
  if (plan.status != PA_OK) return plan.status;
  if (num_blocks <= 0 || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !kv_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  if (plan.ws.total > 0) {
    if (!workspace || workspace_bytes < plan.ws.total) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
  }
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = kv_pool;
  a.v_pool = kv_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale = scale;
  a.block_size = block_size;
  a.num_seqs = num_seqs;
  a.num_query_rows = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = 1;
  a.head_dim = pa::kMlaQkDim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.dtype = dtype;
  a.latent = true;
  a.max_items = plan.max_items;
  a.workgroups = plan.workgroups;
  a.slots = cu_count();
  if (plan.ws.total > 0) {
    char* ws = static_cast<char*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(ws + plan.ws.ml_offset);
    a.ws_acc = reinterpret_cast<float*>(ws + plan.ws.acc_offset);  // the 2-byte partials
    a.ws_off = reinterpret_cast<int*>(ws + plan.off_offset);
  }
  return pa::launch_mla_heads(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Shared by pa_prefill and pa_decode_mla; the caller has checked dtype and
// the head dimension.  Launches once per group of kPfMaxSeqs sequences (the
// query bounds are absolute row numbers, so q and out are passed whole).
// pa_prefill through the grouped-query decode kernel (launch_decode_mfma_queries):
// at most kMfmaQueriesMaxSeqs sequences (its wave-local prologue), the default split, and
// few rows per sequence — T * G <= 16 * NT * S, i.e. on average at most one
// chunk of 16 * NT (query token, head) rows per (sequence, K/V head), as in
// speculative verification of a few drafted tokens.  Its four waves share
// each item's keys, where prefill_kernel gives an item to one wave.
// Measured on 64 sequences of continuous-batching lengths, 32 query / 8 K/V
// heads (prefill_kernel -> this path): 4 drafted tokens 68.8 -> 58.8 us, one
// token 68.0 -> 51.7 us; with a partition chosen for half or a quarter of the
// resident workgroups 62.6 / 116.7 and 59.4 / 113.7 us.
struct QueriesPlan {
  bool applies;
  pa_status_t status;
  int max_items;
  int workgroups;
  int slots;
  size_t tok_offset;  // the per-token merge descriptors ([T][8] int32)
  pa::WorkspaceLayout ws;
};

QueriesPlan plan_queries(int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                         int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                         int32_t head_dim) {
  QueriesPlan p{false, PA_OK, 0, 0, 0, 0, {0, 0, 0, 0}};
  if (partition_size != 0 || num_seqs < 1 || num_seqs > pa::kMfmaQueriesMaxSeqs || num_tokens < 1 || num_heads <= 0 ||
      num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || max_blocks_per_seq <= 0 ||
      max_blocks_per_seq > INT_MAX / block_size / 2)
    return p;
  const long long group = num_heads / num_kv_heads;
  if (group > pa::kMfmaMaxGroup) return p;
  const long long rows_per_item = group > 16 ? 32 : 16;
  if (static_cast<long long>(num_tokens) * group > rows_per_item * num_seqs) return p;
  p.applies = true;
  // items: sum over sequences of Hkv * chunks * ceil(L / P), the partition P
  // (128..2048) chosen on the device as the largest not above
  // Hkv * sum(chunks * L) / slots.  Bound: that sum is at most
  // Hkv * sum(chunks) * (L / P + 1), and Hkv * sum(chunks * L) / P is below
  // 2 * slots unless P is the largest size, where it is at most
  // Hkv * sum(chunks) * cap / 2048; sum(chunks) <= ceil(T * G / rows) + S.
  p.slots = cu_count() * pa::mfma_wg_per_cu(static_cast<int>(group));
  const long long cap = static_cast<long long>(max_blocks_per_seq) * block_size;
  const long long chunks = (static_cast<long long>(num_tokens) * group + rows_per_item - 1) / rows_per_item + num_seqs;
  const long long at_max = num_kv_heads * chunks * ((cap + pa::kMfmaMaxPartTokens - 1) / pa::kMfmaMaxPartTokens);
  const long long items = std::max(2LL * p.slots, at_max) + num_kv_heads * chunks;
  if (items * rows_per_item > INT_MAX / 2) {
    p.status = PA_ERR_INVALID_ARG;
    return p;
  }
  p.max_items = static_cast<int>(items);
  // one workgroup per item as far as the bound allows, as in decode: the
  // hardware starts each on whichever CU frees first, where a grid of one
  // workgroup per slot taking items by stride left the CUs that drew long
  // items behind (verify with one token per sequence: main kernel 48.3 us
  // against 43.5 us for the same rows through pa_decode_gqa)
  p.workgroups = static_cast<int>(std::min<long long>(items, pa::kMfmaMaxWorkgroups));
  if (cap > pa::kMfmaMinPartTokens) {  // a row can span several partitions
    p.ws = pa::workspace_layout(0, static_cast<size_t>(items) * rows_per_item, head_dim);
    p.tok_offset = p.ws.total;
    p.ws.total = pa::align_up(p.ws.total + static_cast<size_t>(num_tokens) * 8 * sizeof(int32_t), 256);
  }
  return p;
}

pa_status_t prefill_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start, float scale, int32_t block_size,
                         int32_t num_seqs, int32_t num_query_rows, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                         bool latent, void* workspace, size_t workspace_bytes, void* stream) {
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  const int v_per_item = latent ? pa::kMlaVDim : head_dim;
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  const int row_tiles = prefill_row_tiles(num_seqs, num_query_rows, num_heads, num_kv_heads, latent);
  const PrefillPlan plan = plan_prefill(num_seqs, num_query_rows, num_heads, num_kv_heads,
                                        max_blocks_per_seq, block_size, partition_size,
                                        v_per_item, 1, row_tiles, latent);
  if (plan.status != PA_OK) return plan.status;
  const QueriesPlan qp = latent ? QueriesPlan{false, PA_OK, 0, 0, 0, 0, {0, 0, 0, 0}}
                                : plan_queries(num_seqs, num_query_rows, num_heads, num_kv_heads,
                                               max_blocks_per_seq, block_size, partition_size, head_dim);
  if (qp.status != PA_OK) return qp.status;
  if (num_blocks <= 0 || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_query_rows == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (!latent && !query_start) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_INVALID_ARG;
  const size_t need = qp.applies ? qp.ws.total : plan.ws.total;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PA_ERR_INVALID_ARG;
  }
  if (qp.applies) {  // few rows per sequence: the grouped-query decode kernel
    pa::DecodeArgs d{};
    d.out = out;
    d.q = q;
    d.k_pool = k_pool;
    d.v_pool = v_pool;
    d.block_tables = block_tables;
    d.context_lens = context_lens;
    d.scale = scale;
    d.block_size = block_size;
    d.num_seqs = num_seqs;
    d.num_heads = num_heads;
    d.num_kv_heads = num_kv_heads;
    d.group_width = 1;
    d.head_dim = head_dim;
    d.num_blocks = num_blocks;
    d.max_blocks_per_seq = max_blocks_per_seq;
    d.dtype = dtype;
    d.kv_dtype = dtype;
    d.mode = pa::DecodeMode::kMfma;
    d.workgroups = qp.workgroups;
    d.max_items = qp.max_items;
    d.mfma_slots = qp.slots;
    d.query_start = query_start;
    d.num_tokens = num_query_rows;
    if (qp.ws.total > 0) {
      char* ws = static_cast<char*>(workspace);
      d.ws_ml = reinterpret_cast<float*>(ws + qp.ws.ml_offset);
      d.ws_acc = reinterpret_cast<float*>(ws + qp.ws.acc_offset);
      d.ws_tok = reinterpret_cast<int*>(ws + qp.tok_offset);
    }
    return pa::launch_decode_mfma_queries(d, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.scale = scale;
  a.block_size = block_size;
  a.num_query_rows = num_query_rows;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.dtype = dtype;
  a.latent = latent;
  a.part_tokens = plan.part_tokens;
  a.row_tiles = row_tiles;
  a.max_items = static_cast<int>(plan.max_items);
  a.workgroups = plan.workgroups;
  if (plan.ws.total > 0) {
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<uint32_t*>(ws + plan.ws.counter_offset);
    a.ws_ml = reinterpret_cast<float*>(ws + plan.ws.ml_offset);
    a.ws_acc = reinterpret_cast<float*>(ws + plan.ws.acc_offset);
  }
  // the row-block kernel when every row stays in one partition, the caller
  // left the split to the library and the 128-row blocks fill the GPU
  const long long group = num_heads / num_kv_heads;
  const long long full_blocks = num_kv_heads * (static_cast<long long>(num_query_rows) * group / pa::kPfTileRows);
  const bool tiles = !latent && partition_size == 0 &&
                     plan.part_tokens >= static_cast<long long>(max_blocks_per_seq) * block_size &&
                     full_blocks >= cu_count() &&
                     static_cast<long long>(num_query_rows) * group >= 64LL * num_seqs;
  for (int32_t s0 = 0; s0 < num_seqs; s0 += pa::kPfMaxSeqs) {
    a.num_seqs = num_seqs - s0 < pa::kPfMaxSeqs ? num_seqs - s0 : pa::kPfMaxSeqs;
    a.block_tables = block_tables + static_cast<size_t>(s0) * max_blocks_per_seq;
    a.context_lens = context_lens + s0;
    a.query_start = query_start ? query_start + s0 : nullptr;
    if (!query_start) {  // one row per sequence: rows s0 .. s0 + n - 1
      a.q = static_cast<const char*>(q) + static_cast<size_t>(s0) * num_heads * head_dim * 2;
      a.out = static_cast<char*>(out) +
              static_cast<size_t>(s0) * num_heads * (latent ? pa::kMlaVDim : head_dim) * 2;
      a.num_query_rows = a.num_seqs;
    }
    if (tiles) {  // one workgroup per item: at most this many 128-row blocks
      const long long items =
          num_kv_heads * ((static_cast<long long>(num_query_rows) * group + pa::kPfTileRows - 1) / pa::kPfTileRows +
                          a.num_seqs);
      a.max_items = static_cast<int>(std::min(items, static_cast<long long>(INT_MAX)));
      a.workgroups = a.max_items;
    }
    const hipError_t e = latent  ? pa::launch_mla_split(a, static_cast<hipStream_t>(stream))
                         : tiles ? pa::launch_prefill_tiles(a, static_cast<hipStream_t>(stream))
                                 : pa::launch_prefill(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// The address under which the GPU reaches *p: device memory as is; pinned
// host memory through the device pointer its mapping has (HIP reports it).
// Anything else — pageable host memory, an unknown address — is refused
// here, on the host, instead of faulting in a kernel.
template <typename P>
bool device_view(P*& p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the caller
    return false;
  }
  if (at.type == hipMemoryTypeHost) {
    if (at.devicePointer == nullptr) return false;
    p = static_cast<P*>(at.devicePointer);
  } else if (at.type != hipMemoryTypeDevice) {
    return false;
  }
  return true;
}

// Shared by pa_copy_blocks, pa_copy_blocks_fp8 and pa_swap_blocks; e =
// element bytes.  The caller has checked dtype and shape.  With host_ok the
// pools, the scales and the mapping may be pinned host memory.
pa_status_t copy_impl(const pa::CopyArgs& c, int32_t num_pairs, int32_t head_dim,
                      int32_t block_size, int e, void* stream, bool host_ok = false) {
  if (num_pairs < 0 || c.num_heads <= 0 || c.src_blocks <= 0 || c.dst_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!c.dst_k || !c.dst_v || !c.src_k || !c.src_v || !c.block_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(c.dst_k, 16) || !aligned(c.dst_v, 16) || !aligned(c.src_k, 16) ||
      !aligned(c.src_v, 16) || !aligned(c.block_mapping, 4))
    return PA_ERR_INVALID_ARG;
  pa::CopyArgs a = c;
  a.num_pairs = num_pairs;
  a.block_bytes = static_cast<size_t>(c.num_heads) * block_size * head_dim * e;
  const size_t chunks = (a.block_bytes + pa::kCopyChunkBytes - 1) / pa::kCopyChunkBytes;
  if (chunks * static_cast<size_t>(num_pairs) > static_cast<size_t>(INT_MAX))
    return PA_ERR_INVALID_ARG;
  if (host_ok) {
    if (!device_view(a.dst_k) || !device_view(a.dst_v) || !device_view(a.src_k) ||
        !device_view(a.src_v) || !device_view(a.block_mapping))
      return PA_ERR_INVALID_ARG;
    if (a.src_ks && (!device_view(a.dst_ks) || !device_view(a.dst_vs) || !device_view(a.src_ks) ||
                     !device_view(a.src_vs)))
      return PA_ERR_INVALID_ARG;
  }
  const hipError_t err = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

bool scales_ok(const float* a, const float* b) { return a && b && aligned(a, 4) && aligned(b, 4); }

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(pa_status_t status) {
  switch (status) {
    case PA_OK:
      return "PA_OK";
    case PA_ERR_INVALID_ARG:
      return "PA_ERR_INVALID_ARG: null or misaligned pointer, or a size out of range";
    case PA_ERR_UNSUPPORTED:
      return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128, block_size 16 or 32, dtype f32/f16/bf16";
    case PA_ERR_WORKSPACE:
      return "PA_ERR_WORKSPACE: workspace missing or smaller than pa_decode_workspace_size()";
    case PA_ERR_HIP:
      return "PA_ERR_HIP: the HIP runtime rejected a kernel launch";
    case PA_ERR_TOO_LARGE:
      return "PA_ERR_TOO_LARGE: pa_decode_noalloc needs more than its static scratch holds "
             "(PA_NOALLOC_MAX_ROWS (sequence, head) rows, PA_NOALLOC_SCRATCH_BYTES bytes)";
    default:
      return "unknown pa_status_t";
  }
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int32_t block_size,
                                int32_t partition_size) {
  const DecodePlan p = plan_decode(num_seqs, num_heads, num_heads, head_dim, max_blocks_per_seq,
                                   block_size, partition_size, PA_DTYPE_F32, PA_DTYPE_F32);
  return p.status == PA_OK ? p.ws.total : 0;
}

size_t pa_decode_gqa_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size,
                                    pa_dtype_t q_dtype, pa_dtype_t kv_dtype) {
  if (elem_bytes(q_dtype) == 0) return 0;
  const DecodePlan p = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                                   max_blocks_per_seq, block_size, partition_size, q_dtype,
                                   kv_dtype);
  return p.status == PA_OK ? p.ws.total : 0;
}

pa_status_t pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t partition_size,
                      pa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, k_pool, v_pool, nullptr, nullptr, block_tables, context_lens, scale,
                     block_size, num_seqs, num_heads, num_heads, head_dim, num_blocks,
                     max_blocks_per_seq, partition_size, dtype, dtype, workspace, workspace_bytes,
                     stream);
}

pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, int32_t block_size, int32_t num_seqs,
                              int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t partition_size,
                              pa_dtype_t dtype, void* stream) {
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, k_pool, v_pool, nullptr, nullptr, block_tables, context_lens, scale,
                     block_size, num_seqs, num_heads, num_heads, head_dim, num_blocks,
                     max_blocks_per_seq, partition_size, dtype, dtype, nullptr, 0, stream,
                     /*static_scratch=*/true);
}

pa_status_t pa_decode_fp8(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          int32_t block_size, int32_t num_seqs, int32_t num_heads,
                          int32_t head_dim, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t partition_size, pa_dtype_t q_dtype, pa_dtype_t kv_dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if ((q_dtype != PA_DTYPE_F16 && q_dtype != PA_DTYPE_BF16) || !is_fp8(kv_dtype))
    return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens,
                     scale, block_size, num_seqs, num_heads, num_heads, head_dim, num_blocks,
                     max_blocks_per_seq, partition_size, q_dtype, kv_dtype, workspace,
                     workspace_bytes, stream);
}

pa_status_t pa_decode_gqa(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scales, const float* v_scales,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          int32_t block_size, int32_t num_seqs, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t q_dtype,
                          pa_dtype_t kv_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (elem_bytes(q_dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (kv_dtype != q_dtype && !(is_fp8(kv_dtype) && q_dtype != PA_DTYPE_F32))
    return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, k_pool, v_pool, is_fp8(kv_dtype) ? k_scales : nullptr,
                     is_fp8(kv_dtype) ? v_scales : nullptr, block_tables, context_lens, scale,
                     block_size, num_seqs, num_heads, num_kv_heads, head_dim, num_blocks,
                     max_blocks_per_seq, partition_size, q_dtype, kv_dtype, workspace,
                     workspace_bytes, stream);
}

pa_status_t pa_reshape_and_cache(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                 const int32_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype_t dtype, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0 || !supported_shape(head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (num_heads > INT_MAX / (head_dim * e)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(slot_mapping, 4))
    return PA_ERR_INVALID_ARG;
  const hipError_t err =
      pa::launch_reshape_and_cache(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                                   num_heads, head_dim * e, block_size, num_blocks,
                                   static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping,
                           int32_t num_pairs, int32_t num_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, pa_dtype_t dtype,
                           void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0 || !supported_shape(head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  const pa::CopyArgs c{k_pool,  v_pool,  k_pool,        v_pool,   nullptr,    nullptr,  nullptr,
                       nullptr, block_mapping, 0, 0, num_blocks, num_blocks, num_heads};
  return copy_impl(c, num_pairs, head_dim, block_size, e, stream);
}

pa_status_t pa_reshape_and_cache_fp8(void* k_pool, void* v_pool, const float* k_scales,
                                     const float* v_scales, const void* k_new, const void* v_new,
                                     const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, pa_dtype_t new_dtype,
                                     pa_dtype_t kv_dtype, void* stream) {
  const int e = elem_bytes(new_dtype);
  if (e == 0 || !is_fp8(kv_dtype) || !supported_shape(head_dim, block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (num_heads > INT_MAX / (head_dim * e)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scales || !v_scales || !k_new || !v_new || !slot_mapping)
    return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(slot_mapping, 4))
    return PA_ERR_INVALID_ARG;
  pa::ReshapeFp8Args a{k_pool,    v_pool,     k_scales,   v_scales,   k_new,
                       v_new,     slot_mapping, num_tokens, num_heads, head_dim,
                       block_size, num_blocks, new_dtype,  kv_dtype};
  const hipError_t err = pa::launch_reshape_and_cache_fp8(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                               const int32_t* block_mapping, int32_t num_pairs, int32_t num_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               pa_dtype_t kv_dtype, void* stream) {
  if (!is_fp8(kv_dtype) || !supported_shape(head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  if (num_pairs > 0 && !scales_ok(k_scales, v_scales)) return PA_ERR_INVALID_ARG;
  const pa::CopyArgs c{k_pool,   v_pool,   k_pool,        v_pool, k_scales,   v_scales,  k_scales,
                       v_scales, block_mapping, 0, 0, num_blocks, num_blocks, num_heads};
  return copy_impl(c, num_pairs, head_dim, block_size, 1, stream);
}

pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                           float* dst_k_scales, float* dst_v_scales, const float* src_k_scales,
                           const float* src_v_scales, const int32_t* block_mapping,
                           int32_t num_pairs, int32_t num_heads, int32_t head_dim,
                           int32_t block_size, int32_t src_num_blocks, int32_t dst_num_blocks,
                           pa_dtype_t dtype, void* stream) {
  const int e = is_fp8(dtype) ? 1 : elem_bytes(dtype);
  if (e == 0 || !supported_shape(head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  if (is_fp8(dtype) && num_pairs > 0 &&
      (!scales_ok(dst_k_scales, dst_v_scales) || !scales_ok(src_k_scales, src_v_scales)))
    return PA_ERR_INVALID_ARG;
  const bool fp8 = is_fp8(dtype);
  const pa::CopyArgs c{dst_k,
                       dst_v,
                       src_k,
                       src_v,
                       fp8 ? dst_k_scales : nullptr,
                       fp8 ? dst_v_scales : nullptr,
                       fp8 ? src_k_scales : nullptr,
                       fp8 ? src_v_scales : nullptr,
                       block_mapping,
                       0,
                       0,
                       src_num_blocks,
                       dst_num_blocks,
                       num_heads};
  return copy_impl(c, num_pairs, head_dim, block_size, e, stream, /*host_ok=*/true);
}

size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t partition_size) {
  if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32)) return 0;
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return 0;
  const QueriesPlan qp = plan_queries(num_seqs, num_query_tokens, num_heads, num_kv_heads, max_blocks_per_seq,
                                      block_size, partition_size, head_dim);
  if (qp.applies) return qp.status == PA_OK ? qp.ws.total : 0;
  const PrefillPlan p = plan_prefill(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                     max_blocks_per_seq, block_size, partition_size, head_dim, 1,
                                     prefill_row_tiles(num_seqs, num_query_tokens, num_heads, num_kv_heads,
                                                       false));
  return p.status == PA_OK ? p.ws.total : 0;
}

pa_status_t pa_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, float scale, int32_t block_size,
                       int32_t num_seqs, int32_t num_query_tokens, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  return prefill_impl(out, q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                      block_size, num_seqs, num_query_tokens, num_heads, num_kv_heads, head_dim,
                      num_blocks, max_blocks_per_seq, partition_size, dtype, false, workspace,
                      workspace_bytes, stream);
}

size_t pa_decode_mla_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t partition_size) {
  if (block_size != 16 && block_size != 32) return 0;
  if (use_mla_heads(num_seqs, num_heads, partition_size)) {
    const MlaHeadsPlan p = plan_mla_heads(num_seqs, num_heads, max_blocks_per_seq, block_size, true);
    return p.status == PA_OK ? p.ws.total : 0;
  }
  const PrefillPlan p = plan_prefill(num_seqs, num_seqs, num_heads, 1, max_blocks_per_seq, block_size,
                                     partition_size, pa::kMlaVDim, 1, 1, true);
  return p.status == PA_OK ? p.ws.total : 0;
}

pa_status_t pa_decode_mla(void* out, const void* q, const void* kv_pool, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, int32_t block_size,
                          int32_t num_seqs, int32_t num_heads, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t partition_size, pa_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (use_mla_heads(num_seqs, num_heads, partition_size))
    return mla_heads_impl(out, q, kv_pool, block_tables, context_lens, scale, block_size, num_seqs, num_heads,
                          num_blocks, max_blocks_per_seq, dtype, workspace, workspace_bytes, stream);
  return prefill_impl(out, q, kv_pool, kv_pool, block_tables, context_lens, nullptr, scale,
                      block_size, num_seqs, num_seqs, num_heads, 1, pa::kMlaQkDim, num_blocks,
                      max_blocks_per_seq, partition_size, dtype, true, workspace, workspace_bytes,
                      stream);
}

}  // extern "C"
