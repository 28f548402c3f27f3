// Grouped-query decode on the matrix cores (gfx950 MFMA).
//
// What is computed: pa_decode with fewer K/V heads than query heads — every
// query head h of sequence s attends over the K/V rows of K/V head h / G
// found through the block table (vLLM tutorial page "3. PagedAttention原理",
// §3.2 and the closing remarks of §3.4; page "PagedAttentionMetal：基于Metal 3
// 的Apple Silicon原生LLM推理加速方案", section 注意力计算优化), contexts split
// into partitions whose softmax partials are merged with the log-sum-exp
// identity (the "Flash-Dec" milestone of "PagedAttention MLX：为Apple Silicon
// 打造的高吞吐量LLM推理引擎").
//
// Why the matrix cores: the G query heads of a group read the same keys and
// values, so per K/V byte there are G dot products and G weighted sums.  On
// the vector unit that arithmetic, not the bytes, bounds a group of 4 or
// more; as a 16-row MFMA tile (rows = the group's heads) it costs a few
// products per 16 keys, and the kernel is left with the bytes.
//
// Work decomposition (our design).  Items are (sequence, K/V head, partition
// of P tokens); P, a power of two from 128 to 2048 tokens, is chosen on the
// device from the lengths — the largest not above the K/V tokens per
// resident workgroup, so that a long context gives each workgroup one long
// item and a ragged batch many short ones — and every workgroup rebuilds the
// per-sequence item offsets in LDS.  The four waves of
// a workgroup share an item: wave w takes its 32-key steps w, w + 4, ...
// (adjacent waves read adjacent 8 KiB of K and V at once), each with its own
// online softmax over NT tiles of 16 query rows; at the end of the item the
// four states are merged through LDS.  An item that is its row's only
// partition writes the output; otherwise it writes per head its (max, sum)
// in fp32 and its normalised output in the 16-bit type (the weighted V sum
// over the sum) to the workspace.  Small batches with groups of at most 4
// heads and contexts of at most 8192 tokens merge them in this kernel: the
// item of a (sequence, K/V head) that arrives last (a ticket from the row's
// arrival counter) folds the row's partials.  Otherwise a second, small
// kernel merges each split row's partials — a 131072-token context on one
// K/V head has hundreds of partials, far more than one workgroup could
// merge at the end of the first kernel.
//
// One 32-key step of one wave (two 16-key blocks), per tile of 16 query rows:
//   S^T = K Q^T    v_mfma_f32_16x16x32_{f16,bf16}, D/32 products per block:
//                  A = 16 keys x 32 elements (lane l: key l%16, elements
//                  8*(l/16)..+7), B = the same elements of the 16 query rows;
//                  lane l gets keys 4*(l/16)+i of the block for row l%16;
//   softmax        the lane's 8 scores, the row's maximum across its four
//                  lanes; rescaling deferred until a row's maximum grows by
//                  more than 2^8;
//   O^T += V^T P^T v_mfma_f32_16x16x32 over the step's 32 keys (the operand
//                  layout of the query kernels), D/16 products, plus one with
//                  every value 1 for the row sums of the rounded weights.

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr int kGqWaves = 4;
// The merge's shape.  Few (sequence, head) rows (long contexts: many
// partials per row): lse_merge_kernel, a workgroup of 128 lanes per
// 32-element slice of a row.  Many rows (batches: few partials each):
// lse_merge_wave_kernel, one wave per row, four rows per workgroup.
// Measured (main kernel + merge, µs): 128K with 4 K/V heads 48.3 / 49.0 /
// 49.1 with slices of 32 / 64 / 32 elements over 128 / 128 / 256 lanes, with
// 1 K/V head 23.0 / 24.2 / 22.9; layer shape with 8 K/V heads 15.1 / 14.1 /
// 16.3 and 12.75 one wave per row; continuous batching with 8 K/V heads
// 53.6 / 51.5 / 56.7 and 47.6, with 4 K/V heads 34.3 (64 / 128) and 32.5.
constexpr int kMergeRowsFew = 256;  // fewer rows than this: a workgroup per slice
static_assert(kMfmaQueriesMaxSeqs == kWave, "the query kernel keeps one sequence per lane");

// MQ: several query tokens per sequence (query_start, num_tokens): a
// sequence's rows are its (query token, head of the group) pairs,
// token-major, in chunks of 16 * NT rows; items (sequence, K/V head, chunk,
// partition); row r of a chunk sees the keys up to its token's position
// (causal); split rows are merged by lse_merge_wave_kernel through the
// per-token descriptors in ws_tok.  Only with at most kMfmaQueriesMaxSeqs
// (= kWave) sequences (the wave-local prologue).
template <typename T, int D, int BS, int NT, bool MQ>
__global__ __launch_bounds__(kGqWaves* kWave, NT == 1 ? 2 : 1) void decode_mfma_kernel(
    typename T::storage* __restrict__ out, const typename T::storage* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int* __restrict__ ws_off, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, float qk_scale, uint32_t q_sign_bits, int num_seqs, int num_heads,
    int num_kv_heads, int group, int num_blocks, int max_blocks, int max_items, int slots,
    const int32_t* __restrict__ query_start, int num_tokens, int* __restrict__ ws_tok,
    uint32_t* __restrict__ counters) {
  static_assert(D % 64 == 0 && BS % 16 == 0, "MFMA slices");
  using S16 = typename T::storage;
  using M = Mfma<T>;
  using PV = PvOps<T, 2>;
  using pw_t = typename PV::word_t;
  constexpr int kTblRegs = (kMfmaMaxPartTokens / BS + kWave - 1) / kWave;  // table entries per lane
  constexpr int kQK = D / 32;  // S^T products per 16 keys
  constexpr int kDq = D / 64;  // 64-element value slices
  constexpr int kThreads = kGqWaves * kWave;
  constexpr int kPer = (kBalancedMaxSeqs + kThreads - 1) / kThreads;
  // partition candidates kMfmaMaxPartTokens, half that, ... kMfmaMinPartTokens
  constexpr int kMinShift = __builtin_ctz(kMfmaMinPartTokens);
  constexpr int kMaxShift = __builtin_ctz(kMfmaMaxPartTokens);
  constexpr int kParts = kMaxShift - kMinShift + 1;
  constexpr int kRows = 16 * NT;  // rows of an item (MQ: a chunk of the sequence's rows)
  __shared__ int s_off[kBalancedMaxSeqs + 1];
  __shared__ int s_len[kBalancedMaxSeqs];
  // MQ: first query token, query tokens and chunks of each sequence (each wave its own copy)
  __shared__ int s_qst[MQ ? kGqWaves * (kWave + 1) : 1];
  __shared__ int s_tq[MQ ? kGqWaves * (kWave + 1) : 1];
  __shared__ int s_nch[MQ ? kGqWaves * (kWave + 1) : 1];
  __shared__ int s_wsum[kParts][kGqWaves];
  __shared__ int s_wtok[kGqWaves];
  __shared__ float s_m[kGqWaves][NT][16];
  __shared__ float s_l[kGqWaves][NT][16];
  __shared__ int s_bad[kGqWaves];
  __shared__ uint32_t s_ticket;
  __shared__ f4_t s_o[kGqWaves][NT][16][D / 4];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int HKV = num_kv_heads;
  const int G = group;
  const int cap = max_blocks * BS;

  // 1. lengths, then the items per sequence for each candidate partition
  //    (HKV * ceil(L / P)), their exclusive prefix sums for the chosen one.
  //    The partition: the largest power of two (kMfmaMinPartTokens ..
  //    kMfmaMaxPartTokens) not above the K/V tokens per resident workgroup,
  //    HKV * sum(L) / slots — long contexts get one long item per workgroup,
  //    ragged batches many short ones.  Up to kWave sequences every wave
  //    builds its own copy (lane s owns sequence s; wave w's copy at offset
  //    w * (kWave + 1) of each array, no workgroup barrier); past that the
  //    workgroup shares one.
  static_assert(kGqWaves * (kWave + 1) <= kBalancedMaxSeqs, "every wave's copy of the offsets fits");
  if (MQ && S > kWave) return;  // the host never launches this
  const bool wave_local = S <= kWave;
  const int sb = wave_local ? wave * (kWave + 1) : 0;
  int* const off_l = s_off + sb;
  int* const len_l = s_len + sb;
  int* const qst_l = s_qst + (MQ ? sb : 0);
  int* const tq_l = s_tq + (MQ ? sb : 0);
  int* const nch_l = s_nch + (MQ ? sb : 0);
  int pshift = kMinShift;
  int total = 0;
  int my_qst = 0, my_tq = 0;  // MQ: lane s's first query token and query tokens
  if (wave_local) {
    const int L = lane < S ? min(max(context_lens[lane], 0), cap) : 0;
    int nch = 1;  // chunks of the sequence's rows (one row group without MQ)
    if constexpr (MQ) {
      if (lane < S) {
        const int a0 = min(max(query_start[lane], 0), num_tokens);
        const int a1 = min(max(query_start[lane + 1], 0), num_tokens);
        my_qst = a0;
        my_tq = max(a1 - a0, 0);
      }
      nch = (my_tq * G + kRows - 1) / kRows;
    }
    // the work: sum over sequences of chunks * L, exactly, from 21-bit pieces
    // (chunks * L < 2^52, at most 64 terms per piece sum)
    const unsigned long long x = static_cast<unsigned long long>(nch) * static_cast<unsigned long long>(L);
    long long tokens = 0;
#pragma unroll
    for (int piece = 0; piece < (MQ ? 3 : 2); ++piece) {
      const int v = static_cast<int>((x >> (21 * piece)) & 0x1FFFFF);
      tokens += static_cast<long long>(__builtin_amdgcn_readlane(wave_prefix_sum(v), kWave - 1)) << (21 * piece);
    }
    const long long per_slot = static_cast<long long>(HKV) * tokens / max(slots, 1);
#pragma unroll
    for (int c = kParts - 1; c >= 0; --c)
      if ((1LL << (kMaxShift - c)) <= per_slot) pshift = kMaxShift - c;
    const int n = HKV * nch * ((L + (1 << pshift) - 1) >> pshift);
    const int incl = wave_prefix_sum(n);
    if (lane < S) {
      len_l[lane] = L;
      off_l[lane] = incl - n;
      if constexpr (MQ) {
        qst_l[lane] = my_qst;
        tq_l[lane] = my_tq;
        nch_l[lane] = nch;
      }
    }
    total = min(__builtin_amdgcn_readlane(incl, kWave - 1), max_items);
    if (lane == 0) off_l[S] = total;
    // the wave's own LDS writes before its reads below (no other wave reads them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  } else {
    for (int s = tid; s < S; s += kThreads) s_len[s] = min(max(context_lens[s], 0), cap);
    __syncthreads();
    int mine[kParts];
#pragma unroll
    for (int c = 0; c < kParts; ++c) mine[c] = 0;
    int mine_tok = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int s = tid * kPer + i;
      const int L = s < S ? s_len[s] : 0;
      mine_tok += L;
#pragma unroll
      for (int c = 0; c < kParts; ++c) mine[c] += HKV * ((L + (1 << (kMaxShift - c)) - 1) >> (kMaxShift - c));
    }
    int incl[kParts];
#pragma unroll
    for (int c = 0; c < kParts; ++c) {
      incl[c] = wave_prefix_sum(mine[c]);
      if (lane == kWave - 1) s_wsum[c][wave] = incl[c];
    }
    const int incl_tok = wave_prefix_sum(mine_tok);
    if (lane == kWave - 1) s_wtok[wave] = incl_tok;
    __syncthreads();
    long long tokens = 0;
#pragma unroll
    for (int w = 0; w < kGqWaves; ++w) tokens += s_wtok[w];
    const long long per_slot = static_cast<long long>(HKV) * tokens / max(slots, 1);
    int ci = kParts - 1;
    int run = 0;
#pragma unroll
    for (int c = kParts - 1; c >= 0; --c) {
      int tot = 0, bef = 0;
#pragma unroll
      for (int w = 0; w < kGqWaves; ++w) {
        tot += s_wsum[c][w];
        bef += (w < wave) ? s_wsum[c][w] : 0;
      }
      if (c == kParts - 1 || (1LL << (kMaxShift - c)) <= per_slot) {
        ci = c;
        total = tot;
        run = bef + incl[c] - mine[c];
      }
    }
    ci = __builtin_amdgcn_readfirstlane(ci);
    pshift = kMaxShift - ci;  // P = 2^pshift tokens
    const int P = 1 << pshift;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int s = tid * kPer + i;
      if (s < S) s_off[s] = run;
      run += s < S ? HKV * ((s_len[s] + P - 1) >> pshift) : 0;
    }
    total = min(__builtin_amdgcn_readfirstlane(total), max_items);
    if (tid == 0) s_off[S] = total;
    __syncthreads();
  }
  pshift = __builtin_amdgcn_readfirstlane(pshift);
  const int P = 1 << pshift;
  if constexpr (!MQ) {
    // the merge kernel reads the same offsets and partition size
    if (blockIdx.x == 0 && wave == 0 && ws_off != nullptr) {
      for (int s = lane; s <= S; s += kWave) ws_off[s] = off_l[s];
      if (lane == 0) ws_off[S + 1] = P;
    }
  } else if (wave == 0 && ws_tok != nullptr) {
    // the merge kernel's descriptor of every query token (its sequence, its
    // index there, the sequence's query tokens, item offset, partitions and
    // chunks, the partition size; or not covered), the tokens spread over
    // the workgroups: lane l finds its token's sequence — the last whose
    // first token is at most its own (the lanes' first tokens are
    // non-decreasing) — by binary lifting over the lanes, six steps in every
    // lane: a lane that reads another's value by a cross-lane read must not
    // have left the loop before it (an inactive source lane reads as zero)
    for (int t0 = blockIdx.x * kWave; t0 < num_tokens; t0 += gridDim.x * kWave) {
      const int t = t0 + lane;
      int lo = 0;
#pragma unroll
      for (int step = kWave / 2; step > 0; step >>= 1) {
        const int cand = lo + step;
        const int v = __shfl(my_qst, min(cand, S - 1));  // every lane, every step
        lo = (cand < S && v <= t) ? cand : lo;
      }
      const int a0 = __shfl(my_qst, lo);
      const int n0 = __shfl(my_tq, lo);
      if (t < num_tokens) {
        const bool in = t >= a0 && t - a0 < n0;
        const int Ls = len_l[lo];
        const int4 d0 = {lo, t - a0, n0, off_l[lo]};
        const int4 d1 = {(Ls + P - 1) >> pshift, nch_l[lo], P, in ? 1 : 0};
        *reinterpret_cast<int4*>(ws_tok + 8 * static_cast<size_t>(t)) = d0;
        *reinterpret_cast<int4*>(ws_tok + 8 * static_cast<size_t>(t) + 4) = d1;
      }
    }
  }

  // 2. empty contexts give zero rows (spread over the workgroups)
  for (int s = blockIdx.x; s < S; s += gridDim.x)
    if (len_l[s] == 0) {
      if constexpr (MQ) {
        const size_t r0 = static_cast<size_t>(qst_l[s]) * num_heads * D;
        for (int i = tid; i < tq_l[s] * num_heads * D; i += kThreads) out[r0 + i] = T::pack(0.f);
      } else {
        for (int i = tid; i < num_heads * D; i += kThreads)
          out[static_cast<size_t>(s) * num_heads * D + i] = T::pack(0.f);
      }
    }

  const u32x4 q_sign = {q_sign_bits, q_sign_bits, q_sign_bits, q_sign_bits};
  const int col = lane % 16;  // query row of a tile / key of a 16-key block
  const int g4 = lane / 16;   // lane group: 8-element slice of S^T's K dim, key quad of P

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // 3. which (sequence, K/V head, partition)
    int lo = 0;
    int hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off_l[mid] <= item)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int L = __builtin_amdgcn_readfirstlane(len_l[s]);
    const int parts = (L + P - 1) >> pshift;
    const int local = item - __builtin_amdgcn_readfirstlane(off_l[s]);
    const int pc = local / parts;  // (K/V head, chunk) pair
    const int part = local - pc * parts;
    // MQ: the sequence's query tokens, its first, this item's chunk
    const int tq = MQ ? __builtin_amdgcn_readfirstlane(tq_l[s]) : 1;
    const int qs0 = MQ ? __builtin_amdgcn_readfirstlane(qst_l[s]) : s;
    const int nch = MQ ? __builtin_amdgcn_readfirstlane(nch_l[s]) : 1;
    const int kvh = MQ ? pc / nch : pc;
    const int chunk = MQ ? pc - kvh * nch : 0;
    const int nrows = MQ ? tq * G : G;  // rows of this (sequence, K/V head)
    const int row0 = chunk * kRows;     // first row of the item
    // keys the chunk's rows see: up to the position of its last row's token
    // (query token i sits at L - tq + i); its first row's bound below which
    // no key needs a mask
    const int last_row = min(nrows, row0 + kRows) - 1;
    const int L_c = MQ ? min(L, L - tq + last_row / G + 1) : L;
    const int lim_min = MQ ? L - tq + row0 / G + 1 : L;
    const int k_begin = part * P;
    const int k_end = max(min(k_begin + P, L_c), k_begin);  // MQ: an item past L_c has no keys
    const int k_unmasked = min(k_end, lim_min);

    // query rows of tile t: rows row0 + 16t + col (B operand of S^T), row r
    // being token r / G and head kvh*G + r % G (without MQ: token 0, head
    // kvh*G + r); klim[t]: the keys this lane's row of tile t sees
    u32x4 qv[NT][kQK];
    int klim[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = row0 + 16 * t + col;
      const bool ok = r < nrows;
      const int tok = MQ ? (ok ? r / G : 0) : 0;
      const int hg = MQ ? (ok ? r - tok * G : 0) : (ok ? r : 0);
      klim[t] = MQ ? min(k_end, L - tq + tok + 1) : k_end;
      const S16* qrow = q + (static_cast<size_t>(qs0 + tok) * num_heads + kvh * G + hg) * D + 8 * g4;
#pragma unroll
      for (int j = 0; j < kQK; ++j) {
        const u32x4 v = load16(qrow + 32 * j) ^ q_sign;  // a negative scale flips q's signs instead
        qv[t][j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }

    float m[NT];
    f4_t lacc[NT];
    f4_t acc[NT][kDq][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m[t] = -INFINITY;
      lacc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][dq][e] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
    int bad = 0;

    struct Stage {
      u32x4 k[2][kQK];
      u32x2 v[2][kDq][4];
      int c;
      int bad;
    };
    // the item's block-table entries, one per lane (entry blk0 + lane + 64r),
    // loaded once: each step then takes its block ids by v_readlane instead
    // of a scalar memory round trip before its K/V loads can be issued
    const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
    const int blk0 = k_begin / BS;
    const int nblk = max((k_end - k_begin + BS - 1) / BS, 1);  // an empty item reads its first entry
    int tblv[kTblRegs];
#pragma unroll
    for (int r = 0; r < kTblRegs; ++r) tblv[r] = tbl[blk0 + min(lane + kWave * r, nblk - 1)];
    auto load_step = [&](Stage& st, int c) __attribute__((always_inline)) {
      st.c = c;
      st.bad = 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // a 16-key block wholly past the item's keys reads the step's first
        // block again (its table entry may not exist); its keys are masked
        const int key0 = (c + 16 * kb < k_end) ? c + 16 * kb : c;
        const int b = key0 / BS - blk0;  // < nblk
        int tv = tblv[0];
#pragma unroll
        for (int r = 1; r < kTblRegs; ++r) tv = (b >> 6) == r ? tblv[r] : tv;
        int phys = __builtin_amdgcn_readlane(tv, b & (kWave - 1));
        if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
          st.bad = 1;  // never dereference an id outside the pool
          phys = 0;
        }
        const size_t row0 = (static_cast<size_t>(phys) * HKV + kvh) * BS + (key0 % BS);
        const char* kp = k_pool + row0 * (D * sizeof(S16)) + static_cast<uint32_t>((col * D + 8 * g4) * sizeof(S16));
#pragma unroll
        for (int j = 0; j < kQK; ++j) st.k[kb][j] = load16_stream(kp + 32 * j * sizeof(S16));
        const char* vp = v_pool + row0 * (D * sizeof(S16)) + static_cast<uint32_t>((4 * g4 * D + 4 * col) * sizeof(S16));
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.v[kb][dq][e] = load8_stream(vp + (e * D + 64 * dq) * sizeof(S16));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    auto attend_step = [&](Stage& st) __attribute__((always_inline)) {
      bad |= st.bad;
      if (st.c + 32 > L) {  // value rows past the context may hold anything: zero
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (st.c + 16 * kb + 4 * g4 + e >= L)
#pragma unroll
              for (int dq = 0; dq < kDq; ++dq) st.v[kb][dq][e] = u32x2{0u, 0u};
      }
      const bool masked = st.c + 32 > k_unmasked;
      f4_t scs[NT][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          f4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < kQK; ++j) sc = M::qk(st.k[kb][j], qv[t][j], sc);
          scs[t][kb] = sc;
        }
      pw_t pw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float z[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[kb][i] = scs[t][kb][i];
          if (masked) {
            const int key = st.c + 16 * kb + 4 * g4;
#pragma unroll
            for (int i = 0; i < 4; ++i) z[kb][i] = (key + i < klim[t]) ? z[kb][i] : -INFINITY;
          }
        }
        float cm = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                         fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
        cm = fold_max<16>(cm);  // the row's four lanes: l, l ^ 16, l ^ 32, l ^ 48
        const float cms = (cm == -INFINITY) ? -INFINITY : cm * qk_scale;  // qk_scale >= 0
        const float mn = fmaxf(m[t], cms);
        if (__builtin_amdgcn_ballot_w64(mn > m[t] + kRescaleLog2) != 0) {
          const float alpha = (m[t] == -INFINITY) ? 0.f : fast_exp2(m[t] - mn);
          lacc[t] *= alpha;
#pragma unroll
          for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][dq][e] *= alpha;
          m[t] = mn;
        }
        // p = 2^(scale*log2e*z - m); masked scores (-inf) are set to 0
        // explicitly (a zero scale would make -inf * scale a NaN)
        const float nm = -m[t];
        float p[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[kb][i] = fast_exp2(fmaf(z[kb][i], qk_scale, nm));
        if (masked) {  // a uniform branch: only steps at a limit hold masked keys
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (z[kb][i] == -INFINITY) p[kb][i] = 0.f;
        }
        pw[t] = pw_t{M::pack2(p[0][0], p[0][1]), M::pack2(p[0][2], p[0][3]), M::pack2(p[1][0], p[1][1]),
                     M::pack2(p[1][2], p[1][3])};
      }
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const pw_t a = {col_pair(st.v[0][dq][0], st.v[0][dq][1], e), col_pair(st.v[0][dq][2], st.v[0][dq][3], e),
                          col_pair(st.v[1][dq][0], st.v[1][dq][1], e), col_pair(st.v[1][dq][2], st.v[1][dq][3], e)};
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][dq][e] = PV::mma(a, pw[t], acc[t][dq][e]);
        }
      const pw_t ones = {M::kOnes, M::kOnes, M::kOnes, M::kOnes};
#pragma unroll
      for (int t = 0; t < NT; ++t) lacc[t] = PV::mma(ones, pw[t], lacc[t]);
    };

    // 4. this wave's steps of the item: keys k_begin + 32*(wave + 4i), two in flight
    const int first = k_begin + 32 * wave;
    const int n_steps = k_end > first ? (k_end - first + 32 * kGqWaves - 1) / (32 * kGqWaves) : 0;
    if (n_steps > 0) {
      Stage a, b;
      load_step(a, first);
      int c = 0;
      for (; c + 2 < n_steps; c += 2) {
        load_step(b, first + (c + 1) * 32 * kGqWaves);
        attend_step(a);
        load_step(a, first + (c + 2) * 32 * kGqWaves);
        attend_step(b);
      }
      if (c + 1 < n_steps) {
        load_step(b, first + (c + 1) * 32 * kGqWaves);
        attend_step(a);
        attend_step(b);
      } else {
        attend_step(a);
      }
    }

    // 5. the four waves' states merged through LDS; lane l holds, for row col
    //    of tile t, value elements 64*dq + 16*g4 + 4*i + e
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (g4 == 0) {
        s_m[wave][t][col] = m[t];
        s_l[wave][t][col] = lacc[t][0];
      }
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_o[wave][t][col][16 * dq + 4 * g4 + i] =
              f4_t{acc[t][dq][0][i], acc[t][dq][1][i], acc[t][dq][2][i], acc[t][dq][3][i]};
    }
    if (lane == 0) s_bad[wave] = bad;
    __syncthreads();
    const bool any_bad = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
    constexpr int kQuads = NT * 16 * (D / 4);  // 4-element pieces of the item's output
    for (int x = tid; x < kQuads; x += kThreads) {
      const int c4 = x % (D / 4);
      const int r = (x / (D / 4)) % 16;
      const int t = x / (16 * (D / 4));
      const int row = 16 * t + r;  // row of the item (without MQ: head of the group)
      if (row0 + row >= nrows) continue;
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kGqWaves; ++w) Mx = fmaxf(Mx, s_m[w][t][r]);
      float l = 0.f;
      f4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kGqWaves; ++w) {
        const float mw = s_m[w][t][r];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - Mx);
        l += f * s_l[w][t][r];
        o += f * s_o[w][t][r][c4];
      }
      if (any_bad) l = __builtin_nanf("");
      // the row's query token (a sequence's rows are token-major) and head
      const int tok = MQ ? (row0 + row) / G : 0;
      const size_t h = static_cast<size_t>(kvh) * G + (MQ ? row0 + row - tok * G : row);
      if (parts == 1) {
        // MQ: a row whose token sits before position 0 sees no key: zero
        const float inv = (MQ && l == 0.f) ? 0.f : 1.f / l;
        const uint32_t w0 = M::pack2(o[0] * inv, o[1] * inv);
        const uint32_t w1 = M::pack2(o[2] * inv, o[3] * inv);
        *reinterpret_cast<u32x2*>(out + (static_cast<size_t>(qs0 + tok) * num_heads + h) * D + 4 * c4) =
            u32x2{w0, w1};
      } else {
        // a split row's partial: o / l rounded to the 16-bit type (half the
        // bytes of fp32 sums, written here and read by the merge) and its
        // (max, sum) in fp32; an empty partial (l = 0) is zero
        const size_t slot = static_cast<size_t>(item) * (MQ ? kRows : G) + row;
        const float inv = (l == 0.f) ? 0.f : 1.f / l;
        const u32x2 w = {M::pack2(o[0] * inv, o[1] * inv), M::pack2(o[2] * inv, o[3] * inv)};
        S16* const po = reinterpret_cast<S16*>(ws_acc) + slot * D + 4 * c4;
        if (!MQ && counters != nullptr) {  // merged in this kernel: stores other XCDs will read
          // (the 64-bit value built from the two words, not passed as floats)
          const uint64_t wv = static_cast<uint64_t>(w.x) | (static_cast<uint64_t>(w.y) << 32);
          __hip_atomic_store(reinterpret_cast<uint64_t*>(po), wv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (c4 == 0) store_coherent_u64(ws_ml + slot * 2, Mx, l);
        } else {
          *reinterpret_cast<u32x2*>(po) = w;
          if (c4 == 0) *reinterpret_cast<f32x2*>(ws_ml + slot * 2) = f32x2{Mx, l};
        }
      }
    }
    if constexpr (!MQ) {
      if (counters != nullptr && parts > 1) {
        // the split rows of (sequence, K/V head) merged by the item that
        // arrives last: every thread's partial stores performed, then one
        // ticket per item; the last ticket's workgroup folds the `parts`
        // partials of each of the G heads in partition order (o_p weighs
        // l_p 2^(m_p - M)) and clears the counter for the next call.  No
        // workgroup waits for another.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        uint32_t* const ctr = counters + static_cast<size_t>(s) * HKV + kvh;
        if (tid == 0) s_ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_ticket == static_cast<uint32_t>(parts - 1)) {
          constexpr int kU = 8;  // partials in flight per thread
          const size_t item0 = static_cast<size_t>(item - part);
          for (int x = tid; x < G * (D / 4); x += kThreads) {
            const int g = x / (D / 4);
            const int c4 = x - g * (D / 4);
            float Mx = -INFINITY, den = 0.f;
            f4_t num = {0.f, 0.f, 0.f, 0.f};
            for (int p0 = 0; p0 < parts; p0 += kU) {
              uint64_t mlv[kU], ov[kU];
#pragma unroll
              for (int u = 0; u < kU; ++u) {
                const size_t slot = (item0 + min(p0 + u, parts - 1)) * G + g;
                mlv[u] = load_coherent_u64(ws_ml + slot * 2);
                ov[u] = load_coherent_u64(reinterpret_cast<const float*>(reinterpret_cast<const S16*>(ws_acc) + slot * D + 4 * c4));
              }
              float bm = -INFINITY;
#pragma unroll
              for (int u = 0; u < kU; ++u)
                if (p0 + u < parts) bm = fmaxf(bm, lo_float(mlv[u]));
              const float mn = fmaxf(Mx, bm);
              if (mn == -INFINITY) continue;  // only empty partials so far
              const float a = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - mn);
              den *= a;
              num *= a;
#pragma unroll
              for (int u = 0; u < kU; ++u) {
                const float mu = lo_float(mlv[u]);
                const float wl = ((p0 + u < parts && mu != -INFINITY) ? fast_exp2(mu - mn) : 0.f) * hi_float(mlv[u]);
                float f[4];
                T::unpack_word(static_cast<uint32_t>(ov[u]), f);
                T::unpack_word(static_cast<uint32_t>(ov[u] >> 32), f + 2);
                den += wl;
                num += wl * f4_t{f[0], f[1], f[2], f[3]};
              }
              Mx = mn;
            }
            const float inv = 1.f / den;
            *reinterpret_cast<u32x2*>(out + (static_cast<size_t>(s) * num_heads + static_cast<size_t>(kvh) * G + g) * D +
                                      4 * c4) = u32x2{M::pack2(num[0] * inv, num[1] * inv), M::pack2(num[2] * inv, num[3] * inv)};
          }
          if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();  // the LDS state is rewritten by the next item
  }
}

// Log-sum-exp merge of the split rows of several query tokens per sequence
// (launch_decode_mfma_queries): one wave per (query token, head) row, four
// rows per workgroup.  The token's descriptor in ws_tok (what the first
// kernel wrote: its sequence, its index i there, the sequence's query
// tokens, item offset, partitions, chunks, partition size, whether a
// sequence covers it) places row r = i * group + h % group of K/V head
// h / group in chunk r / RPI of the sequence's items, at slot
// item * RPI + r % RPI of each.  A partial is o_p = acc_p / l_p in the
// 16-bit type with (m_p, l_p) in fp32, weighing l_p 2^(m_p - M).  Lane l
// holds elements 4 * (l % kC) .. + 3 of
// the partials l / kC, l / kC + kG, ..., kU of them in flight per round,
// folded into a running (max, sum, sums) with the online rescaling; the kG
// lane groups are then folded by cross-lane reads.  Slots past max_items are
// never read; a row that saw no key (every partial empty) comes out zero.
//
// TOKENS false: the rows of pa_decode_gqa, (sequence, head), addressed as in
// lse_merge_kernel through ws_off and context_lens (slot (off[s] + (h /
// group) * parts + p) * group + h % group): for many rows with few
// partials each, where one wave per row beats a workgroup per slice.
template <typename T, int D, int RPI, bool TOKENS>
__global__ __launch_bounds__(256) void lse_merge_wave_kernel(
    typename T::storage* __restrict__ out, const int* __restrict__ ws_tok, const int* __restrict__ ws_off,
    const int32_t* __restrict__ context_lens, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    int num_rows, int num_seqs, int num_heads, int group, int cap, int max_items) {
  constexpr int kC = D / 4;        // lanes over one partial's D elements
  constexpr int kG = kWave / kC;   // partials side by side
  constexpr int kU = 8;
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + static_cast<int>(threadIdx.x / kWave);
  if (row >= num_rows) return;
  const int t = row / num_heads;  // query token (TOKENS) or sequence
  const int h = row - t * num_heads;
  int parts, g, stride;
  size_t item0;
  if constexpr (TOKENS) {
    const int4 d0 = *reinterpret_cast<const int4*>(ws_tok + 8 * static_cast<size_t>(t));
    const int4 d1 = *reinterpret_cast<const int4*>(ws_tok + 8 * static_cast<size_t>(t) + 4);
    parts = d1.x;
    if (d1.w == 0 || parts <= 1) return;  // not covered, or written by the first kernel
    const int r = d0.y * group + h % group;
    item0 = static_cast<size_t>(d0.w) + (static_cast<size_t>(h / group) * d1.y + r / RPI) * parts;
    g = r % RPI;
    stride = RPI;
  } else {
    const int L = min(max(context_lens[t], 0), cap);
    const int P = ws_off[num_seqs + 1];
    parts = (L + P - 1) / P;
    if (parts <= 1) return;  // written by the first kernel
    item0 = static_cast<size_t>(ws_off[t]) + static_cast<size_t>(h / group) * parts;
    g = h % group;
    stride = group;
  }
  if (item0 + parts > static_cast<size_t>(max_items)) return;
  const int c = lane % kC;
  const int gl = lane / kC;
  float Mx = -INFINITY, den = 0.f;
  f4_t num = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < parts; p0 += kG * kU) {
    f32x2 ml[kU];
    f4_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t slot = (item0 + min(p0 + u * kG + gl, parts - 1)) * stride + g;
      ml[u] = *reinterpret_cast<const f32x2*>(ws_ml + slot * 2);
      const u32x2 w = *reinterpret_cast<const u32x2*>(
          reinterpret_cast<const typename T::storage*>(ws_acc) + slot * D + 4 * c);
      float f[4];
      T::unpack_word(w.x, f);
      T::unpack_word(w.y, f + 2);
      v[u] = f4_t{f[0], f[1], f[2], f[3]};
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u * kG + gl < parts) bm = fmaxf(bm, ml[u][0]);
    const float mn = fmaxf(Mx, bm);
    if (mn == -INFINITY) continue;  // only empty partials so far
    const float a = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - mn);
    den *= a;
    num *= a;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float mu = ml[u][0];
      // partial p holds o_p = acc_p / l_p: it weighs l_p 2^(m_p - M)
      const float wl = ((p0 + u * kG + gl < parts && mu != -INFINITY) ? fast_exp2(mu - mn) : 0.f) * ml[u][1];
      den += wl;
      num += wl * v[u];
    }
    Mx = mn;
  }
  const float M = fold_max<kC>(Mx);
  const float f = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - M);
  den = fold_sum<kC>(den * f);
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = fold_sum<kC>(num[e] * f);
  if (gl == 0) {
    const float inv = den == 0.f ? 0.f : 1.f / den;
    const uint32_t w0 = Mfma<T>::pack2(o[0] * inv, o[1] * inv);
    const uint32_t w1 = Mfma<T>::pack2(o[2] * inv, o[3] * inv);
    *reinterpret_cast<u32x2*>(out + (static_cast<size_t>(t) * num_heads + h) * D + 4 * c) = u32x2{w0, w1};
  }
}

template <typename T, int D, int BS, int NT, bool MQ>
hipError_t run_mfma(const DecodeArgs& a, hipStream_t stream) {
  using S16 = typename T::storage;
  hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, NT, MQ>), dim3(a.workgroups), dim3(kGqWaves * kWave), 0, stream,
                     static_cast<S16*>(a.out), static_cast<const S16*>(a.q), static_cast<const char*>(a.k_pool),
                     static_cast<const char*>(a.v_pool), a.block_tables, a.context_lens, a.ws_off, a.ws_ml,
                     a.ws_acc, fabsf(a.scale) * kLog2e, a.scale < 0.f ? 0x80008000u : 0u, a.num_seqs,
                     a.num_heads, a.num_kv_heads, a.num_heads / a.num_kv_heads, a.num_blocks,
                     a.max_blocks_per_seq, a.max_items, a.mfma_slots, a.query_start, a.num_tokens, a.ws_tok,
                     (!MQ && a.mfma_fuse) ? a.counters : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ws_ml == nullptr || (!MQ && a.mfma_fuse)) return e;
  const int group = a.num_heads / a.num_kv_heads;
  if constexpr (MQ) {  // (query token, head) rows, four per workgroup
    const int rows = a.num_tokens * a.num_heads;
    hipLaunchKernelGGL((lse_merge_wave_kernel<T, D, 16 * NT, true>), dim3((rows + 3) / 4), dim3(4 * kWave), 0,
                       stream, static_cast<S16*>(a.out), a.ws_tok, nullptr, nullptr, a.ws_ml, a.ws_acc, rows,
                       a.num_seqs, a.num_heads, group, 0, a.max_items);
    return hipGetLastError();
  }
  const int rows = a.num_seqs * a.num_heads;
  const int cap = a.max_blocks_per_seq * a.block_size;
  if (rows >= kMergeRowsFew) {  // many rows: one wave per row
    hipLaunchKernelGGL((lse_merge_wave_kernel<T, D, 16, false>), dim3((rows + 3) / 4), dim3(4 * kWave), 0, stream,
                       static_cast<S16*>(a.out), nullptr, a.ws_off, a.context_lens, a.ws_ml, a.ws_acc, rows,
                       a.num_seqs, a.num_heads, group, cap, a.max_items);
    return hipGetLastError();
  }
  // few rows (long contexts: many partials per row): a workgroup per 32-element slice
  hipLaunchKernelGGL((lse_merge_kernel<T, D, 32, 128>), dim3(rows * (D / 32)), dim3(128), 0, stream,
                     static_cast<S16*>(a.out), a.ws_off, a.ws_ml, a.ws_acc, a.context_lens, a.num_seqs,
                     a.num_heads, group, cap);
  return hipGetLastError();
}

template <typename T, int D, int BS, bool MQ>
hipError_t run_mfma_nt(const DecodeArgs& a, hipStream_t stream) {
  return (a.num_heads / a.num_kv_heads) > 16 ? run_mfma<T, D, BS, 2, MQ>(a, stream)
                                             : run_mfma<T, D, BS, 1, MQ>(a, stream);
}

template <typename T, int D, bool MQ>
hipError_t run_mfma_bs(const DecodeArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_mfma_nt<T, D, 16, MQ>(a, stream) : run_mfma_nt<T, D, 32, MQ>(a, stream);
}

template <typename T, bool MQ>
hipError_t run_mfma_d(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? run_mfma_bs<T, 64, MQ>(a, stream) : run_mfma_bs<T, 128, MQ>(a, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_mfma_d<BF16, false>(a, stream) : run_mfma_d<F16, false>(a, stream);
}

hipError_t launch_decode_mfma_queries(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_mfma_d<BF16, true>(a, stream) : run_mfma_d<F16, true>(a, stream);
}

}  // namespace pa
