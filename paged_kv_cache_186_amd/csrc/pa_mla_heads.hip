// Decode over the MLA latent cache with many query heads (gfx950 MFMA).
//
// What is computed: multi-head latent attention decode in its absorbed form
// ("PagedAttention MLX：为Apple Silicon打造的高吞吐量LLM推理引擎", roadmap
// milestone 3, names MLA; the form is the published one: one 576-element
// cache row per token — 512-element latent then 64-element rotary key — every
// query head scores scale * <q_h, row_t> over all 576 elements and takes the
// row's first 512 elements as its value), through the block table (vLLM
// tutorial page "3. PagedAttention原理", §3.2), long contexts split into
// partitions merged with the log-sum-exp identity ("Flash-Dec", milestone 4).
//
// Why this shape: every head of a sequence reads the same latent rows, so the
// rows should come from HBM once per sequence and feed as many heads as
// possible.  Here a workgroup serves up to 64 heads (a wave whose 16 heads
// all lie past the last one only loads rows): each of
// its four waves owns 16 heads (the rows of its MFMA tiles) over the whole
// 576-element row, and each 32-key step's rows (36 KiB) are loaded from HBM
// once per workgroup into LDS (row stride padded by 16 bytes so that the 16
// rows an operand load touches fall on different banks), from where every
// wave reads its operands; the workgroup's 64 query rows sit in LDS too (in
// registers, beside the 128 accumulator registers of a wave's 16 x 512
// outputs, they would not fit).  The next step's rows are in flight in
// registers while a step is computed; one barrier per step.  A step's 32 keys
// lie in one table block (two of 16 tokens): their ids are read from LDS once
// per step, not once per load (the per-load reads had put nine dependent LDS
// round trips before the step's loads: 128 heads 138 -> 130 us).
//
// Up to 16 heads (SPLIT) there is one 16-row tile, and with one wave owning
// it the other three only loaded rows: the step's arithmetic, on one wave
// per CU, set the time.  There the four waves share the tile instead: wave w
// scores the 32-element latent slices 4w .. 4w + 3 (and, for w < 2, rotary
// slice 16 + w), the four partial score tiles are summed through LDS in wave
// order (every wave then holds the same scores, softmax state and row sums),
// and wave w accumulates values 128 w .. 128 w + 127 (16 heads, 32 sequences
// of 1024..8192 tokens: 65 -> 54.5 us; 51 us with the masking of an item's
// last step under a uniform branch and the row loads addressed from the
// step's uniform block base).  Per step and wave that is 5 (4) score slices
// x 2 key blocks and 8 P.V tiles instead of 18 x 2 and 32.
//
// Per step and wave (16 heads, 32 keys; without SPLIT):
//   S^T = K Q^T     18 v_mfma_f32_16x16x32 per 16-key block over the 576
//                   elements (A = 16 keys x 32 elements, B = the wave's 16
//                   query rows, both from LDS);
//   softmax         the lane's 8 scores, the row's maximum across its four
//                   lanes, rescaling deferred until it grows by more than 2^8;
//   O^T += V^T P^T  one product per 16-value tile of the 512 latent values
//                   (A = V transposed, from LDS by two transposing reads),
//                   plus one with every value 1 for the row sums.
// Items are (sequence, partition of P tokens, group of 64 heads), in that
// order, one workgroup per CU.  P, a multiple of 32 from 256 to 4096, is
// chosen on the device from the lengths: the smallest of eight sizes between
// the two bounds below that gives every workgroup at most one item, so that
// the longest item, which sets the kernel's time, is as short as the lengths
// allow.  Consecutive items run on one XCD, so the head groups of a
// partition, which read the same rows, share that XCD's L2.  A row of one
// partition is written at once, the partials of split rows are merged by
// lse_merge_kernel.

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"
#include "pagedattn.h"

namespace pa {
namespace {

typedef __attribute__((address_space(3))) s4_t lds_s4_t;

// Waves per workgroup, one per SIMD.  (Up to 16 heads share one tile; eight
// waves then, two per SIMD, were slower: every wave reads every other
// wave's partial scores, 128 KiB of LDS per step against 32 KiB with four.)
constexpr int kMhWaves = 4;
constexpr int kMhHeads = kMlaHeadsGroup;             // heads per workgroup (16 per wave)
constexpr int kMhRowB = kMlaQkDim * 2;               // bytes of one latent row
constexpr int kMhLdsRow = kMhRowB + 16;              // padded LDS row stride
constexpr int kMhStepKeys = 32;
constexpr int kMhChunks = kMhRowB / 16;              // 16-byte chunks per row (72)
constexpr int kMhStepChunks = kMhStepKeys * kMhChunks;  // 16-byte chunks of one step's rows (2304)
constexpr int kMhQK = kMlaQkDim / 32;                // S^T products per 16 keys (18)
constexpr int kMhDt = kMlaVDim / 16;                 // 16-value tiles (32): rows of the P.V A operand
constexpr int kMhMaxBlocks = kMlaHeadsMaxPart / 16;  // table entries of the longest item

// A lane's share of one head's 512 outputs: 4 consecutive values of each
// 16-value tile (values 16 dt + 4 g4 + i in acc[dt][i]), scaled by inv,
// rounded and stored 8 bytes a tile; row points at the lane's first value.
template <typename T, int N>
__device__ __forceinline__ void store_row(typename T::storage* row, const f4_t (&acc)[N], float inv) {
#pragma unroll
  for (int dt = 0; dt < N; ++dt)
    *reinterpret_cast<u32x2*>(row + 16 * dt) = u32x2{Mfma<T>::pack2(acc[dt][0] * inv, acc[dt][1] * inv),
                                                     Mfma<T>::pack2(acc[dt][2] * inv, acc[dt][3] * inv)};
}

template <typename T, int BS, bool SPLIT>
__global__ __launch_bounds__(kMhWaves* kWave, 1) void mla_heads_kernel(
    typename T::storage* __restrict__ out, const typename T::storage* __restrict__ q,
    const char* __restrict__ kv_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int* __restrict__ ws_off, float* __restrict__ ws_ml,
    typename T::storage* __restrict__ ws_part, float qk_scale, uint32_t q_sign_bits, int num_seqs,
    int num_heads, int num_blocks, int max_blocks, int max_items, int slots) {
  using S16 = typename T::storage;
  using M = Mfma<T>;
  using PV = PvOps<T, 2>;
  using pw_t = typename PV::word_t;
  constexpr int NW = kMhWaves;
  constexpr int kThreads = NW * kWave;
  constexpr int kMhLoads = (kMhStepChunks + kThreads - 1) / kThreads;  // per thread per step (9)
  constexpr int kPer = (kMlaHeadsMaxSeqs + kThreads - 1) / kThreads;
  constexpr int kCand = 8;  // partition sizes tried
  __shared__ int s_off[kMlaHeadsMaxSeqs + 1];
  __shared__ int s_len[kMlaHeadsMaxSeqs];
  __shared__ int s_wsum[kCand][NW];
  __shared__ int s_wtok[NW];
  __shared__ int s_wpre[NW];
  __shared__ int s_tbl[kMhMaxBlocks];
  // the workgroup's query rows (64; SPLIT: 16) and two steps of latent rows
  // (padded rows)
  constexpr int kQRows = SPLIT ? 16 : kMhHeads;
  __shared__ __attribute__((aligned(16))) char s_q[kQRows * kMhLdsRow];
  __shared__ __attribute__((aligned(16))) char s_rows[2][kMhStepKeys * kMhLdsRow];
  // SPLIT: each wave's partial scores (its share of the 576 elements), lane l's
  // four scores of key block kb at s_x[wave][kb][l]
  __shared__ f4_t s_x[SPLIT ? NW : 1][2][SPLIT ? kWave : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int NG = (num_heads + kMhHeads - 1) / kMhHeads;  // head groups per sequence
  const int cap = max_blocks * BS;

  // 1. lengths (thread t holds sequences kPer t ..) and their total
  for (int s = tid; s < S; s += kThreads) s_len[s] = min(max(context_lens[s], 0), cap);
  __syncthreads();
  int lens[kPer];
  int mine_tok = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    lens[i] = s < S ? s_len[s] : 0;
    mine_tok += lens[i];
  }
  const int incl_tok = wave_prefix_sum(mine_tok);
  if (lane == kWave - 1) s_wtok[wave] = incl_tok;
  __syncthreads();
  long long tokens = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tokens += s_wtok[w];

  // 2. the partition P, a multiple of the 32-key step: items (sequence,
  //    partition, head group) number NG * sum ceil(L / P); the smallest P
  //    with at most one item per resident workgroup is wanted.  NG * tokens
  //    / slots bounds it from below, NG * tokens / (slots - NG * S) from
  //    above (each sequence adds less than one partition); kCand sizes
  //    spaced geometrically between the two are counted, the smallest that
  //    fits is taken (else the largest), clamped to [min, max] partition.
  const long long work = static_cast<long long>(NG) * tokens;
  const int free_slots = slots - NG * S;
  auto round_part = [](long long x) {
    x = (x + kMhStepKeys - 1) / kMhStepKeys * kMhStepKeys;
    return static_cast<int>(min(max(x, static_cast<long long>(kMlaHeadsMinPart)),
                                static_cast<long long>(kMlaHeadsMaxPart)));
  };
  const int p_lo = round_part((work + slots - 1) / max(slots, 1));
  const int p_hi = free_slots > 0 ? max(p_lo, round_part((work + free_slots - 1) / free_slots)) : kMlaHeadsMaxPart;
  const float lg = log2f(static_cast<float>(p_hi) / static_cast<float>(p_lo));
  int cand[kCand];
  double rcand[kCand];
  int cnt[kCand];
#pragma unroll
  for (int c = 0; c < kCand; ++c) {
    const float x = static_cast<float>(p_lo) * exp2f(lg * c / (kCand - 1));
    cand[c] = (c == kCand - 1) ? p_hi : min(round_part(static_cast<long long>(x)), p_hi);
    rcand[c] = 1.0 / cand[c];
    cnt[c] = 0;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
#pragma unroll
    for (int c = 0; c < kCand; ++c) cnt[c] += ceil_div_nonneg(lens[i], cand[c], rcand[c]);
#pragma unroll
  for (int c = 0; c < kCand; ++c) {
    const int incl = wave_prefix_sum(cnt[c]);
    if (lane == kWave - 1) s_wsum[c][wave] = incl;
  }
  __syncthreads();
  int P = cand[kCand - 1];
#pragma unroll
  for (int c = kCand - 1; c >= 0; --c) {
    long long tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_wsum[c][w];
    if (static_cast<long long>(NG) * tot <= slots) P = cand[c];
  }
  P = __builtin_amdgcn_readfirstlane(P);

  // 3. item offsets of the sequences for that P
  const double rP = 1.0 / P;
  int parts_of[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    parts_of[i] = ceil_div_nonneg(lens[i], P, rP);
    mine += NG * parts_of[i];
  }
  const int incl = wave_prefix_sum(mine);
  if (lane == kWave - 1) s_wpre[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  int total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    run += (w < wave) ? s_wpre[w] : 0;
    total += s_wpre[w];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    if (s < S) s_off[s] = run;
    run += NG * parts_of[i];
  }
  total = min(__builtin_amdgcn_readfirstlane(total), max_items);
  if (tid == 0) s_off[S] = total;
  __syncthreads();
  if (blockIdx.x == 0 && ws_off != nullptr) {  // for the merge
    for (int s = tid; s <= S; s += kThreads) ws_off[s] = s_off[s];
    if (tid == 0) ws_off[S + 1] = P;
  }

  // 4. empty contexts give zero rows
  for (int s = blockIdx.x; s < S; s += gridDim.x)
    if (s_len[s] == 0)
      for (int i = tid; i < num_heads * kMlaVDim; i += kThreads)
        out[static_cast<size_t>(s) * num_heads * kMlaVDim + i] = T::pack(0.f);

  const u32x4 q_sign = {q_sign_bits, q_sign_bits, q_sign_bits, q_sign_bits};
  const int col = lane % 16;
  const int g4 = lane / 16;

  // items in order (sequence, partition, head group); workgroup b runs on
  // XCD b % 8, and its logical index makes consecutive items share an XCD:
  // the head groups of one partition read the same rows through one L2
  for (int item = xcd_local_index(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    int lo = 0;
    int hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= item)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int L = __builtin_amdgcn_readfirstlane(s_len[s]);
    const int parts = (L + P - 1) / P;
    const int local = item - __builtin_amdgcn_readfirstlane(s_off[s]);
    const int part = local / NG;
    const int hg = local - part * NG;
    const int k_begin = part * P;
    const int k_end = min(k_begin + P, L);
    const int n_steps = (k_end - k_begin + kMhStepKeys - 1) / kMhStepKeys;
    const int blk0 = k_begin / BS;
    const int nblk = (k_end - k_begin + BS - 1) / BS;

    // the item's block-table entries in LDS (the step loads gather per lane)
    const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
    for (int b = tid; b < nblk; b += kThreads) s_tbl[b] = tbl[blk0 + b];

    // this wave's 16 heads; the workgroup's 64 query rows go to LDS (the B
    // operands of S^T are read from there every step: in registers they and
    // the O^T accumulators would not fit the register file)
    // (SPLIT: every wave serves heads 0..15, each over its own 128 values)
    const int h = SPLIT ? col : hg * kMhHeads + wave * 16 + col;
    const bool row_ok = h < num_heads;
    const bool wave_rows = SPLIT || hg * kMhHeads + wave * 16 < num_heads;  // the wave has a head (uniform)
    {
      const S16* qg = q + (static_cast<size_t>(s) * num_heads + hg * kMhHeads) * kMlaQkDim;
      constexpr int kQChunks = kQRows * kMhChunks;
      constexpr int kQLoads = (kQChunks + kThreads - 1) / kThreads;  // 18 per thread (SPLIT: 5)
      constexpr int kQBatch = SPLIT ? kQLoads : kMhLoads;             // issued together
      static_assert(kQLoads % kQBatch == 0, "whole batches");
#pragma unroll
      for (int i0 = 0; i0 < kQLoads; i0 += kQBatch) {
        u32x4 r[kQBatch];
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int x = min(tid + (i0 + i) * kThreads, kQChunks - 1);
          const int row = x / kMhChunks;
          const int chunk = x - row * kMhChunks;
          const bool ok = hg * kMhHeads + row < num_heads;
          // every lane loads (a row past the last head reads the group's
          // first row, which exists), so that the loads are issued together
          // instead of one conditional round trip after another; a negative
          // scale flips q's signs instead
          const u32x4 v =
              load16(reinterpret_cast<const char*>(qg + static_cast<size_t>(ok ? row : 0) * kMlaQkDim) + chunk * 16);
          r[i] = ok ? (v ^ q_sign) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int x = tid + (i0 + i) * kThreads;
          const int row = x / kMhChunks;
          const int chunk = x - row * kMhChunks;
          if (x < kQChunks) *reinterpret_cast<u32x4*>(&s_q[row * kMhLdsRow + chunk * 16]) = r[i];
        }
      }
    }
    // the wave's 16-value tiles: all 32, or (SPLIT) tiles 8 wave .. 8 wave + 7
    constexpr int kDtW = SPLIT ? kMhDt / NW : kMhDt;
    const int dt0 = SPLIT ? kDtW * wave : 0;
    float m = -INFINITY;
    f4_t lacc = {0.f, 0.f, 0.f, 0.f};
    f4_t acc[kDtW];
#pragma unroll
    for (int dt = 0; dt < kDtW; ++dt) acc[dt] = f4_t{0.f, 0.f, 0.f, 0.f};
    int bad = 0;
    __syncthreads();  // s_tbl and s_q written; the previous item's LDS rows no longer read

    // cooperative load of one step's 32 rows: thread chunk x = tid + kThreads i
    // covers row x / 72, 16-byte chunk x % 72; keys past the item's end read
    // the step's first row instead (their table entry may not exist; they
    // are masked).  The step's keys lie in one block (two for 16-token
    // blocks), whose ids are read once, uniformly, and selected per key.
    auto load_step = [&](u32x4 (&r)[kMhLoads], int step) __attribute__((always_inline)) {
      const int c0 = k_begin + step * kMhStepKeys;
      const int b0 = c0 / BS - blk0;
      int ph[2];
      ph[0] = __builtin_amdgcn_readfirstlane(s_tbl[b0]);
      ph[1] = (BS < kMhStepKeys && c0 + BS < k_end) ? __builtin_amdgcn_readfirstlane(s_tbl[b0 + 1]) : ph[0];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (static_cast<unsigned>(ph[j]) >= static_cast<unsigned>(num_blocks)) {
          bad = 1;  // never dereference an id outside the pool
          ph[j] = 0;
        }
      // uniform block bases, a 32-bit offset per load (c0 is a multiple of
      // both block sizes, so key o of the step is row o % BS of block o / BS)
      const char* const base0 = kv_pool + static_cast<size_t>(ph[0]) * (BS * kMhRowB);
      const char* const base1 = kv_pool + static_cast<size_t>(ph[1]) * (BS * kMhRowB);
      const bool tail = c0 + kMhStepKeys > k_end;
#pragma unroll
      for (int i = 0; i < kMhLoads; ++i) {
        const int x = min(tid + i * kThreads, kMhStepChunks - 1);
        const int key = x / kMhChunks;
        const int chunk = x - key * kMhChunks;
        const int o = (!tail || c0 + key < k_end) ? key : 0;  // the key's offset from c0
        const uint32_t off = static_cast<uint32_t>((o % BS) * kMhRowB + chunk * 16);
        const char* const base = (BS >= kMhStepKeys || o < BS) ? base0 : base1;
        r[i] = load16(base + off);
      }
    };
    auto store_step = [&](const u32x4 (&r)[kMhLoads], int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kMhLoads; ++i) {
        const int x = tid + i * kThreads;
        const int key = x / kMhChunks;
        const int chunk = x - key * kMhChunks;
        if (kMhStepChunks % kThreads == 0 || x < kMhStepChunks)
          *reinterpret_cast<u32x4*>(&s_rows[buf][key * kMhLdsRow + chunk * 16]) = r[i];
      }
    };

    auto compute_step = [&](int buf, int step) __attribute__((always_inline)) {
      const int c0 = k_begin + step * kMhStepKeys;
      const char* rows = s_rows[buf];
      // S^T: the 36 operand loads of the two blocks in chunks of kQc, each
      // chunk's loads issued before the previous chunk's products (the
      // scheduling barriers keep the compiler from hoisting every load at
      // once, which would not fit the register file)
      // S^T over the 576 elements, kQc 32-element slices at a time: the K
      // operands of both blocks and the wave's query operands from LDS, the
      // next chunk's loads issued before this chunk's products (scheduling
      // barriers keep the compiler from hoisting every load at once)
      f4_t sc[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
      if constexpr (SPLIT) {
        // this wave's share of the 576 elements: latent slices kL w ..
        // kL w + kL - 1 and, for waves 0 and 1, rotary slice 16 + w; the NW
        // partial score tiles are summed through LDS in wave order, so that
        // every wave holds the same scores (and the same softmax state)
        constexpr int kL = 16 / NW;  // latent 32-element slices per wave
        const char* qrow = s_q + col * kMhLdsRow + 16 * g4;
        const char* krow = rows + col * kMhLdsRow + 16 * g4;
        u32x4 kd[kL + 1][2], qd[kL + 1];
#pragma unroll
        for (int j = 0; j <= kL; ++j) {
          const int off = 64 * (j < kL ? kL * wave + j : 16 + (wave & 1));
          qd[j] = *reinterpret_cast<const u32x4*>(qrow + off);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) kd[j][kb] = *reinterpret_cast<const u32x4*>(krow + 16 * kb * kMhLdsRow + off);
        }
#pragma unroll
        for (int j = 0; j < kL; ++j)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) sc[kb] = M::qk(kd[j][kb], qd[j], sc[kb]);
        if (wave < 2)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) sc[kb] = M::qk(kd[kL][kb], qd[kL], sc[kb]);
        s_x[wave][0][lane] = sc[0];
        s_x[wave][1][lane] = sc[1];
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sc[kb] = s_x[0][kb][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) sc[kb] += s_x[w][kb][lane];
        }
      } else {
      constexpr int kQc = 2;
      constexpr int kChunksQ = kMhQK / kQc;
      u32x4 kbuf[2][2][kQc], qbuf[2][kQc];
      const char* qrow = s_q + (wave * 16 + col) * kMhLdsRow + 16 * g4;
      auto load_qc = [&](int ch, u32x4 (&kd)[2][kQc], u32x4 (&qd)[kQc]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kQc; ++j) {
          const int off = 64 * (ch * kQc + j);
          qd[j] = *reinterpret_cast<const u32x4*>(qrow + off);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            kd[kb][j] = *reinterpret_cast<const u32x4*>(rows + (16 * kb + col) * kMhLdsRow + 16 * g4 + off);
        }
      };
      load_qc(0, kbuf[0], qbuf[0]);
#pragma unroll
      for (int ch = 0; ch < kChunksQ; ++ch) {
        if (ch + 1 < kChunksQ) load_qc(ch + 1, kbuf[(ch + 1) & 1], qbuf[(ch + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kQc; ++j)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) sc[kb] = M::qk(kbuf[ch & 1][kb][j], qbuf[ch & 1][j], sc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      // only an item's last step can hold keys past its end: the masking is
      // a uniform branch, skipped by every other step
      const bool masked = c0 + kMhStepKeys > k_end;
      float z[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[kb][i] = sc[kb][i];
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c0 + 16 * kb + 4 * g4 + i >= k_end) z[kb][i] = -INFINITY;
      }
      float cm = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                       fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
      cm = fold_max<16>(cm);
      const float cms = (cm == -INFINITY) ? -INFINITY : cm * qk_scale;
      const float mn = fmaxf(m, cms);
      if (__builtin_amdgcn_ballot_w64(mn > m + kRescaleLog2) != 0) {
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
        lacc *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDtW; ++dt) acc[dt] *= alpha;
        m = mn;
      }
      const float nm = -m;
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kb][i] = fast_exp2(fmaf(z[kb][i], qk_scale, nm));
      if (masked) {  // masked scores (-inf) weigh 0 (with a zero scale -inf * 0 would be a NaN)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (z[kb][i] == -INFINITY) p[kb][i] = 0.f;
      }
      const pw_t pw = {M::pack2(p[0][0], p[0][1]), M::pack2(p[0][2], p[0][3]), M::pack2(p[1][0], p[1][1]),
                       M::pack2(p[1][2], p[1][3])};
      // V^T operand per 16-value tile dt by two transposing reads
      // (ds_read_b64_tr_b16): in each group of 16 lanes, lane 4 j + a reads
      // values 16 dt + 4 a .. of key j of the group's four (4 g4 + j of each
      // block), and the read hands lane l value 16 dt + l % 16 of all four —
      // the keys its P operand holds.  One tile ahead.
      const char* vrow = rows + (4 * g4 + col / 4) * kMhLdsRow + 8 * (col % 4);
      auto load_vt = [&](int dt, u32x4& dst) __attribute__((always_inline)) {
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(vrow + 32 * dt)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t*)(vrow + 16 * kMhLdsRow + 32 * dt)));
        dst = u32x4{lo.x, lo.y, hi.x, hi.y};
      };
      u32x4 vbuf[2];
      load_vt(dt0, vbuf[0]);
#pragma unroll
      for (int dt = 0; dt < kDtW; ++dt) {
        if (dt + 1 < kDtW) load_vt(dt0 + dt + 1, vbuf[(dt + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        acc[dt] = PV::mma(vbuf[dt & 1], pw, acc[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const pw_t ones = {M::kOnes, M::kOnes, M::kOnes, M::kOnes};
      lacc = PV::mma(ones, pw, lacc);
    };

    // steps: LDS double-buffered, the next step's rows in flight in registers
    // while a step is computed, one barrier per step
    u32x4 ra[kMhLoads];
    load_step(ra, 0);
    store_step(ra, 0);
    __syncthreads();
    if (n_steps > 1) load_step(ra, 1);
    for (int st = 0; st < n_steps; ++st) {
      if (wave_rows) compute_step(st & 1, st);  // a wave past the last head only loads
      if (st + 1 < n_steps) store_step(ra, (st + 1) & 1);
      __syncthreads();
      if (st + 2 < n_steps) load_step(ra, st + 2);
    }

    // 5. this wave's 16 rows; lane l holds row col's values 16 dt + 4 g4 + i
    //    in acc[dt][i]
    // (the output and workspace addresses are formed only here: opaque
    // copies of the base pointers keep the compiler from computing them
    // before the steps and holding them in registers across the loop)
    S16* out_b = out;
    S16* part_b = ws_part;
    float* ml_b = ws_ml;
    asm volatile("" : "+s"(out_b), "+s"(part_b), "+s"(ml_b));
    const int any_bad = __syncthreads_or(bad);
    float lrow = lacc[0];  // the row sum (every element of the ones product holds it)
    if (any_bad) lrow = __builtin_nanf("");
    S16* orow = out_b + (static_cast<size_t>(s) * num_heads + h) * kMlaVDim + 16 * dt0 + 4 * g4;
    if (parts == 1) {
      if (row_ok) store_row<T>(orow, acc, 1.f / lrow);
      continue;
    }
    // a split row: the item's partial, normalised and rounded to the output
    // type, and its (max, sum) in fp32, for mla_merge_kernel
    const size_t slot = static_cast<size_t>(item) * kMhHeads + (SPLIT ? 0 : wave * 16) + col;
    store_row<T>(part_b + slot * kMlaVDim + 16 * dt0 + 4 * g4, acc, 1.f / lrow);
    if (g4 == 0 && (!SPLIT || wave == 0)) *reinterpret_cast<f32x2*>(ml_b + slot * 2) = f32x2{m, lrow};
  }
}

// The rows split over several partitions: one wave per (sequence, head),
// lane l owning elements 8 l .. 8 l + 7.  A partial holds o_p = acc_p / l_p
// (output type) and (m_p, l_p); the row is sum_p w_p o_p / sum_p w_p with
// w_p = l_p 2^(m_p - M), M the running maximum, folded in partition order
// with kU partials' loads in flight.  Item (sequence s, partition p, head
// group g) is off[s] + p * NG + g, off[] and P as the first kernel wrote them.
template <typename T>
__global__ __launch_bounds__(kWave) void mla_merge_kernel(typename T::storage* __restrict__ out,
                                                          const int* __restrict__ ws_off,
                                                          const float* __restrict__ ws_ml,
                                                          const typename T::storage* __restrict__ ws_part,
                                                          const int32_t* __restrict__ context_lens, int num_seqs,
                                                          int num_heads, int cap) {
  constexpr int kU = 8;
  const int s = blockIdx.x / num_heads;
  const int h = blockIdx.x % num_heads;
  const int NG = (num_heads + kMhHeads - 1) / kMhHeads;
  const int L = min(max(context_lens[s], 0), cap);
  const int P = ws_off[num_seqs + 1];
  const int parts = (L + P - 1) / P;
  if (parts <= 1) return;
  const size_t item0 = static_cast<size_t>(ws_off[s]) + h / kMhHeads;
  const int g = h % kMhHeads;
  const int lane = threadIdx.x;
  float mx = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < parts; p0 += kU) {
    f32x2 ml[kU];
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t slot = (item0 + static_cast<size_t>(min(p0 + u, parts - 1)) * NG) * kMhHeads + g;
      ml[u] = *reinterpret_cast<const f32x2*>(ws_ml + slot * 2);
      v[u] = load16(ws_part + slot * kMlaVDim + 8 * lane);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u < parts) bm = fmaxf(bm, ml[u][0]);
    const float mn = fmaxf(mx, bm);
    if (mn == -INFINITY) continue;
    const float a = (mx == -INFINITY) ? 0.f : fast_exp2(mx - mn);
    den *= a;
#pragma unroll
    for (int k = 0; k < 8; ++k) num[k] *= a;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float mu = ml[u][0];
      const float w = (p0 + u < parts && mu != -INFINITY) ? fast_exp2(mu - mn) * ml[u][1] : 0.f;
      float o[8];
      T::unpack(v[u], o);
      den += w;
#pragma unroll
      for (int k = 0; k < 8; ++k) num[k] = fmaf(w, o[k], num[k]);
    }
    mx = mn;
  }
  const float inv = 1.f / den;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = Mfma<T>::pack2(num[2 * k] * inv, num[2 * k + 1] * inv);
  store16(out + (static_cast<size_t>(s) * num_heads + h) * kMlaVDim + 8 * lane, u32x4{w[0], w[1], w[2], w[3]});
}

template <typename T, int BS, bool SPLIT>
hipError_t run_mla_heads(const PrefillArgs& a, hipStream_t stream) {
  using S16 = typename T::storage;
  hipLaunchKernelGGL((mla_heads_kernel<T, BS, SPLIT>), dim3(a.workgroups), dim3(kMhWaves * kWave), 0, stream,
                     static_cast<S16*>(a.out), static_cast<const S16*>(a.q), static_cast<const char*>(a.k_pool),
                     a.block_tables, a.context_lens, a.ws_off, a.ws_ml, reinterpret_cast<S16*>(a.ws_acc),
                     fabsf(a.scale) * kLog2e, a.scale < 0.f ? 0x80008000u : 0u, a.num_seqs, a.num_heads,
                     a.num_blocks, a.max_blocks_per_seq, a.max_items, a.slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ws_ml == nullptr) return e;
  hipLaunchKernelGGL((mla_merge_kernel<T>), dim3(a.num_seqs * a.num_heads), dim3(kWave), 0, stream,
                     static_cast<S16*>(a.out), a.ws_off, a.ws_ml, reinterpret_cast<const S16*>(a.ws_acc),
                     a.context_lens, a.num_seqs, a.num_heads, a.max_blocks_per_seq * a.block_size);
  return hipGetLastError();
}

template <typename T, bool SPLIT>
hipError_t run_mla_heads_bs(const PrefillArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_mla_heads<T, 16, SPLIT>(a, stream) : run_mla_heads<T, 32, SPLIT>(a, stream);
}

// up to 16 heads: one 16-row tile, shared by the four waves (SPLIT)
template <typename T>
hipError_t run_mla_heads_t(const PrefillArgs& a, hipStream_t stream) {
  return a.num_heads <= 16 ? run_mla_heads_bs<T, true>(a, stream) : run_mla_heads_bs<T, false>(a, stream);
}

}  // namespace

hipError_t launch_mla_heads(const PrefillArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_mla_heads_t<BF16>(a, stream) : run_mla_heads_t<F16>(a, stream);
}

}  // namespace pa
