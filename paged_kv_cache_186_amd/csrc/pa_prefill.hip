// Attention of several query rows at once over the paged KV cache, on the
// matrix cores (gfx950 MFMA).
//
// What is computed: for every sequence s, its last Tq_s tokens attend
// causally over its cache — query token i at position p = L_s - Tq_s + i sees
// the keys at positions 0..p — and query head h reads K/V head h / G (page
// "mlx-paged-attention: Bringing vLLM-level High Throughput Inference to Apple
// Silicon", comparison with vLLM and future plans: speculative decoding,
// i.e. verifying several drafted tokens in one pass; the attention itself is
// the ordinary softmax attention read through the block table, vLLM tutorial
// page "3. PagedAttention原理", §3.2 and the closing remarks of §3.4).  The
// same kernel, with one latent K/V "head" whose value is a prefix of the key
// row, is decode over a multi-head latent (MLA) cache ("PagedAttention MLX：
// 为Apple Silicon打造的高吞吐量LLM推理引擎", roadmap milestone 3).
//
// Work decomposition (our design).  The rows of one (sequence, K/V head) are
// its (query token, head of the group) pairs, token-major: M_s = Tq_s * G
// rows.  A wave owns a tile of 16 rows; the context may be cut into
// partitions of part_tokens tokens.  Items (sequence, K/V head, row tile,
// partition) are numbered with the partition fastest and taken by the waves
// of the grid in turn; each workgroup rebuilds the per-sequence item offsets
// in LDS from context_lens and query_start.
//
// One 32-key chunk (two 16-key blocks) of one item, per wave:
//   S^T = K Q^T   per block, with v_mfma_f32_16x16x32_{f16,bf16}: A = 16 keys
//                 x 32 head elements (lane l: key l%16, elements 8*(l/16)..+7
//                 of the slice — four lanes read 64 contiguous bytes of a key
//                 row), B = the same elements of the 16 query rows; the
//                 result gives lane l the scores of keys 4*(l/16)+i, i < 4,
//                 of each block for query row l%16;
//   softmax       per query row: the lane's eight scores, then across the
//                 four lanes of the row (two cross-lane maxima);
//   O^T += V^T P^T with v_mfma_f32_16x16x32_{f16,bf16} over the chunk's 32
//                 keys: B = the probabilities exactly as the scores came out
//                 (lane l: keys 4*(l/16)+i of both blocks for row l%16,
//                 rounded to the 16-bit type), A = V transposed — lane l
//                 reads 8 bytes (4 elements) of each of its 8 keys, 16 lanes
//                 cover a 128-byte line, and byte permutes regroup the
//                 elements by column; the column labels of the 4 products of
//                 a 64-element slice are chosen so that lane l ends with 16
//                 consecutive output elements of row l%16.  The row sums are
//                 one more such product with every value 1.
// Two chunks are in flight (loads of the next chunk are issued before the
// current one is consumed).  Masked keys (after a row's position, or past the
// context in the last block) get probability 0 by selection, and V rows past
// the context are zeroed, so poisoned cache slots never reach a result.
// A row split over several partitions stores (max, sum, weighted V sum) per
// partition; the wave that draws the last ticket merges them with the
// log-sum-exp identity and resets the counter.

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kXcds = 8;     // MI355X: 8 XCDs of 32 CUs
constexpr int kPfRows = 16;  // query rows per tile (MFMA N of S^T)

// T: storage of q, pools and out (F16 or BF16).  DQK: elements of a query /
// key row; DV: elements of a value row; DVS: value elements one item
// produces (DV, or a slice of it: the 512-element latent values are split in
// two items of 256 that share the scores, so that one wave's registers hold
// the query, two chunks in flight and the accumulators); KV_STRIDE: elements
// between consecutive value rows of the V pool (DV for a separate V pool; DQK
// when values are the first DV elements of the key rows, v_pool == k_pool).
// KB: 16-key blocks per chunk (2: the P.V products run at the full 16x16x32
// rate).  NT: 16-row tiles per wave; every K/V operand a wave loads serves
// all NT tiles (more matrix work per byte when a sequence has many rows).
template <typename T, int DQK, int DV, int DVS, int KV_STRIDE, int BS, int KB, int NT>
__global__ __launch_bounds__(kPfWaves* kWave, (DQK > 128 || NT > 1 ? 1 : 2)) void prefill_kernel(
    typename T::storage* __restrict__ out, const typename T::storage* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ query_start, uint32_t* __restrict__ counters, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, float qk_scale, int num_seqs, int num_rows, int num_heads, int num_kv_heads,
    int group, int num_blocks, int max_blocks, int part_tokens, int max_items, uint32_t q_sign_bits) {
  static_assert(DQK % 32 == 0 && DVS % 64 == 0 && DV % DVS == 0, "MFMA slices");
  static_assert(BS % 16 == 0, "a 16-key block never crosses a cache block");
  using S16 = typename T::storage;
  using M = Mfma<T>;
  using PV = PvOps<T, KB>;
  using pw_t = typename PV::word_t;
  constexpr int kQK = DQK / 32;   // S^T products per 16 keys
  constexpr int kDq = DVS / 64;   // 64-element value slices of an item
  constexpr int kSlices = DV / DVS;
  constexpr int kChunk = 16 * KB;
  constexpr int kGroupRows = kPfRows * NT;
  // partials loaded at once while merging: 1 + 8*kDq loads each per lane, at
  // most 60 in all (a wave has at most 63 loads in flight; past that a batch
  // costs two memory round trips), at most 4 (register budget)
  constexpr int kMergeBatch = 60 / (1 + 8 * kDq) < 4 ? 60 / (1 + 8 * kDq) : 4;
  static_assert(kMergeBatch >= 1, "one partial per batch at least");
  constexpr int kThreads = kPfWaves * kWave;
  constexpr int kPer = (kPfMaxSeqs + kThreads - 1) / kThreads;
  __shared__ int s_off[kPfMaxSeqs + 1];  // items of all sequences before s
  __shared__ int s_len[kPfMaxSeqs];
  __shared__ int s_q0[kPfMaxSeqs + 1];   // first query row of s (s_q0[S] = rows)
  __shared__ int s_wsum[kPfWaves];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int HKV = num_kv_heads;
  const int cap = max_blocks * BS;

  // 1. lengths, query bounds and the exclusive prefix sum of items
  for (int s = tid; s < S; s += kThreads) s_len[s] = min(max(context_lens[s], 0), cap);
  // query bounds clamped to the q / out rows, so that no value in
  // query_start can send an access outside them
  for (int s = tid; s <= S; s += kThreads) s_q0[s] = min(max(query_start ? query_start[s] : s, 0), num_rows);
  __syncthreads();
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    int c = 0;
    if (s < S) {
      const int rows = max(s_q0[s + 1] - s_q0[s], 0) * group;
      const int tiles = rows > 0 ? (rows + kGroupRows - 1) / kGroupRows : 0;
      const int parts = max(1, (s_len[s] + part_tokens - 1) / part_tokens);
      c = HKV * tiles * kSlices * parts;
    }
    cnt[i] = c;
    mine += c;
  }
  const int incl = wave_prefix_sum(mine);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kPfWaves; ++w) {
    const int v = s_wsum[w];
    before += (w < wave) ? v : 0;
    total += v;
  }
  int run = before + incl - mine;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    if (s < S) s_off[s] = run;
    run += cnt[i];
  }
  if (tid == 0) s_off[S] = total;
  __syncthreads();
  // the host sized the workspace for max_items; query bounds that break the
  // contract (overlapping ranges) could ask for more: those items are dropped
  total = min(__builtin_amdgcn_readfirstlane(total), max_items);

  const u32x4 q_sign = {q_sign_bits, q_sign_bits, q_sign_bits, q_sign_bits};
  const int col = lane % 16;  // query row of a tile / key of a 16-key block (A rows)
  const int g4 = lane / 16;   // lane group: 8-element slice of S^T's K dim, key quad of P
  const int NH = num_heads;

  // XCD-aware item order: workgroups are dispatched to the 8 XCDs round
  // robin (workgroup i on XCD i % 8), and each XCD has its own L2.  The items
  // are cut into 8 contiguous ranges, one per XCD, so that the row tiles and
  // partitions of one (sequence, K/V head) — which read the same keys and
  // values — run on one XCD and share its L2 (the grid is a multiple of 8).
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int x_end = min(total, (xcd + 1) * per_xcd);
  const int x_step = (gridDim.x / kXcds) * kPfWaves;
  for (int item = xcd * per_xcd + (blockIdx.x / kXcds) * kPfWaves + wave; item < x_end; item += x_step) {
    // 2. which (sequence, K/V head, tile group, value slice, partition)
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
    const int q0 = __builtin_amdgcn_readfirstlane(s_q0[s]);
    const int Tq = max(__builtin_amdgcn_readfirstlane(s_q0[s + 1]) - q0, 0);
    const int Mrows = Tq * group;
    const int tiles = (Mrows + kGroupRows - 1) / kGroupRows;
    const int parts = max(1, (L + part_tokens - 1) / part_tokens);
    // value slices fastest (the slices of one partition read the same key
    // rows: adjacent waves, mostly of one workgroup, so the second read
    // hits the cache), then partitions
    const int local = item - __builtin_amdgcn_readfirstlane(s_off[s]);
    const int slice = local % kSlices;
    const int rest = local / kSlices;
    const int part = rest % parts;
    const int rest2 = rest / parts;
    const int tg = rest2 % tiles;
    const int hk = rest2 / tiles;
    const int v_off = slice * DVS;  // first value element of the item

    // this lane's query row in each tile
    bool row_ok[NT];
    int ti[NT], h[NT], pos[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = (tg * NT + t) * kPfRows + col;
      row_ok[t] = r < Mrows;
      ti[t] = row_ok[t] ? r / group : 0;
      h[t] = hk * group + (row_ok[t] ? r % group : 0);
      pos[t] = row_ok[t] ? L - Tq + ti[t] : -1;  // keys 0..pos are visible
    }
    // wave-uniform key range of the item
    const int r_last = min(Mrows, (tg + 1) * kGroupRows) - 1;
    const int pos_max = L - Tq + r_last / group;
    const int pos_min = L - Tq + (tg * kGroupRows) / group;
    const int k_begin = part * part_tokens;
    const int k_end = min(min(k_begin + part_tokens, L), pos_max + 1);

    // query slices (B operand of S^T): lane holds elements 32j + 8*g4 .. +7
    u32x4 qv[NT][kQK];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const S16* qrow = q + (static_cast<size_t>(q0 + ti[t]) * NH + h[t]) * DQK + 8 * g4;
#pragma unroll
      for (int j = 0; j < kQK; ++j) {
        const u32x4 v = load16(qrow + 32 * j) ^ q_sign;  // a negative scale flips q's signs instead
        qv[t][j] = row_ok[t] ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }

    float m[NT];      // running max of row `col` of tile t (same in its 4 lanes)
    f4_t lacc[NT];    // running row sums: the P.V product with every value 1
                      // (each of the 4 elements holds row col's sum)
    f4_t acc[NT][kDq][4];  // O^T products: [tile][slice][column label e]
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
      u32x4 k[KB][kQK];
      u32x2 v[KB][kDq][4];
      int c;  // first key of the chunk
      int bad;
    };
    const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
    auto load_chunk = [&](Stage& st, int c) __attribute__((always_inline)) {
      st.c = c;
      st.bad = 0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // a 16-key block wholly past the item's keys (tail chunk) reads the
        // chunk's first block again instead — its table entry may not exist,
        // and a block the item does not need must not poison it: its keys
        // are masked (and values past the context zeroed) like any other
        const int key0 = (c + 16 * kb < k_end) ? c + 16 * kb : c;
        int phys = tbl[key0 / BS];
        if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
          st.bad = 1;  // never dereference an id outside the pool
          phys = 0;
        }
        // wave-uniform 64-bit row base + a 32-bit lane offset + constant
        // offsets per load: scalar-base addressing, no 64-bit lane arithmetic
        const size_t row0 = (static_cast<size_t>(phys) * HKV + hk) * BS + (key0 % BS);
        const char* kb_ptr = k_pool + row0 * (DQK * sizeof(S16)) +
                             static_cast<uint32_t>((col * DQK + 8 * g4) * sizeof(S16));
#pragma unroll
        for (int j = 0; j < kQK; ++j) st.k[kb][j] = load16(kb_ptr + 32 * j * sizeof(S16));
        const char* vb_ptr = v_pool + row0 * (KV_STRIDE * sizeof(S16)) +
                             static_cast<uint32_t>((4 * g4 * KV_STRIDE + v_off + 4 * col) * sizeof(S16));
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.v[kb][dq][e] =
                *reinterpret_cast<const u32x2*>(vb_ptr + (e * KV_STRIDE + 64 * dq) * sizeof(S16));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    auto attend_chunk = [&](Stage& st) __attribute__((always_inline)) {
      bad |= st.bad;
      if (st.c + kChunk > L) {  // value rows past the context may hold anything: zero
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (st.c + 16 * kb + 4 * g4 + e >= L)
#pragma unroll
              for (int dq = 0; dq < kDq; ++dq) st.v[kb][dq][e] = u32x2{0u, 0u};
      }
      const bool masked = (st.c + kChunk - 1 > pos_min) || (st.c + kChunk > k_end);
      // raw scores <q, k> of every tile first (the softmax scale is folded
      // into the exponent): the matrix unit then works on the later tiles'
      // products while the vector unit runs the first tile's softmax
      f4_t scs[NT][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
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
        float z[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[kb][i] = scs[t][kb][i];
          if (masked) {
            const int key0 = st.c + 16 * kb + 4 * g4;  // key of z[kb][0]
#pragma unroll
            for (int i = 0; i < 4; ++i) z[kb][i] = (key0 + i <= pos[t] && key0 + i < k_end) ? z[kb][i] : -INFINITY;
          }
        }
        float cm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) cm = fmaxf(cm, fmaxf(fmaxf(z[kb][0], z[kb][1]), fmaxf(z[kb][2], z[kb][3])));
        cm = fold_max<16>(cm);  // the row's four lanes: l, l ^ 16, l ^ 32, l ^ 48
        const float cms = (cm == -INFINITY) ? -INFINITY : cm * qk_scale;  // qk_scale > 0
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
        // explicitly, in the steps that have any (a zero scale would make
        // -inf * scale a NaN)
        const float nm = -m[t];
        float p[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[kb][i] = fast_exp2(fmaf(z[kb][i], qk_scale, nm));
        if (masked) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[kb][i] = (z[kb][i] == -INFINITY) ? 0.f : p[kb][i];
        }
        if constexpr (KB == 1) {
          pw[t] = pw_t{M::pack2(p[0][0], p[0][1]), M::pack2(p[0][2], p[0][3])};
        } else {
          pw[t] = pw_t{M::pack2(p[0][0], p[0][1]), M::pack2(p[0][2], p[0][3]), M::pack2(p[1][0], p[1][1]),
                       M::pack2(p[1][2], p[1][3])};
        }
      }
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // column e of this slice for the lane's keys (rows 4*g4 .. +3 of each block)
          pw_t a;
          if constexpr (KB == 1) {
            a = pw_t{col_pair(st.v[0][dq][0], st.v[0][dq][1], e), col_pair(st.v[0][dq][2], st.v[0][dq][3], e)};
          } else {
            a = pw_t{col_pair(st.v[0][dq][0], st.v[0][dq][1], e), col_pair(st.v[0][dq][2], st.v[0][dq][3], e),
                     col_pair(st.v[1][dq][0], st.v[1][dq][1], e), col_pair(st.v[1][dq][2], st.v[1][dq][3], e)};
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][dq][e] = PV::mma(a, pw[t], acc[t][dq][e]);
        }
      // row sums of the rounded probabilities the products used
      pw_t ones;
#pragma unroll
      for (int w = 0; w < static_cast<int>(sizeof(pw_t) / 4); ++w) ones[w] = M::kOnes;
#pragma unroll
      for (int t = 0; t < NT; ++t) lacc[t] = PV::mma(ones, pw[t], lacc[t]);
    };

    // 3. the chunks of the item, two in flight
    const int n_chunks = k_end > k_begin ? (k_end - k_begin + kChunk - 1) / kChunk : 0;
    if (n_chunks > 0) {
      Stage a, b;
      load_chunk(a, k_begin);
      int c = 0;
      for (; c + 2 < n_chunks; c += 2) {
        load_chunk(b, k_begin + (c + 1) * kChunk);
        attend_chunk(a);
        load_chunk(a, k_begin + (c + 2) * kChunk);
        attend_chunk(b);
      }
      if (c + 1 < n_chunks) {
        load_chunk(b, k_begin + (c + 1) * kChunk);
        attend_chunk(a);
        attend_chunk(b);
      } else {
        attend_chunk(a);
      }
    }

    // lane holds, for row `col` of tile t, output elements 64*dq + 16*g4 + 4*i + e
    auto write_row = [&](int t, const float (&o)[kDq][16]) __attribute__((always_inline)) {
      S16* orow = out + (static_cast<size_t>(q0 + ti[t]) * NH + h[t]) * DV + v_off + 16 * g4;
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq) {
        uint32_t w[8];
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) w[k2] = M::pack2(o[dq][2 * k2], o[dq][2 * k2 + 1]);
        store16(orow + 64 * dq, u32x4{w[0], w[1], w[2], w[3]});
        store16(orow + 64 * dq + 8, u32x4{w[4], w[5], w[6], w[7]});
      }
    };

    float lrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) lrow[t] = bad ? __builtin_nanf("") : lacc[t][0];

    if (parts == 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (!row_ok[t]) continue;
        float o[kDq][16];
        const float inv = (lrow[t] == 0.f) ? 0.f : 1.f / lrow[t];  // no visible key (empty context): zeros
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dq][4 * i + e] = acc[t][dq][e][i] * inv;
        write_row(t, o);
      }
      continue;
    }

    // 4. a partial of a split row group: slot `item`, NT x 16 rows of
    //    (max, sum) and DVS sums
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t row = (static_cast<size_t>(item) * NT + t) * kPfRows + col;
      float* av = ws_acc + row * DVS + 16 * g4;
      if (g4 == 0) store_coherent_u64(ws_ml + row * 2, m[t], lrow[t]);
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          store_coherent_u64(av + 64 * dq + 4 * i, acc[t][dq][0][i], acc[t][dq][1][i]);
          store_coherent_u64(av + 64 * dq + 4 * i + 2, acc[t][dq][2][i], acc[t][dq][3][i]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partial stores before the ticket
    const int item0 = item - part * kSlices;  // the partition-0 item of this tile group and slice
    uint32_t ticket = 0;
    if (lane == 0)
      ticket = __hip_atomic_fetch_add(&counters[item0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket != static_cast<uint32_t>(parts - 1)) continue;

    // 5. last arrival: merge the partials of each tile (slots item0 + p*kSlices, p < parts)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float Mx = -INFINITY;
      float den = 0.f;
      float num[kDq][16];
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) num[dq][k2] = 0.f;
      for (int p0 = 0; p0 < parts; p0 += kMergeBatch) {
        uint64_t pml[kMergeBatch];
        uint64_t pv[kMergeBatch][kDq][8];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const size_t slot = static_cast<size_t>(item0) + static_cast<size_t>(min(p0 + u, parts - 1)) * kSlices;
          const size_t row = (slot * NT + t) * kPfRows + col;
          pml[u] = load_coherent_u64(ws_ml + row * 2);
#pragma unroll
          for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
            for (int k2 = 0; k2 < 8; ++k2)
              pv[u][dq][k2] = load_coherent_u64(ws_acc + row * DVS + 64 * dq + 16 * g4 + 2 * k2);
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          if (p0 + u >= parts) break;
          const float mu = lo_float(pml[u]);
          if (mu == -INFINITY) continue;  // an empty partition
          const float mn = fmaxf(Mx, mu);
          const float a = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - mn);
          const float b = fast_exp2(mu - mn);
          den = den * a + hi_float(pml[u]) * b;
#pragma unroll
          for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
            for (int k2 = 0; k2 < 8; ++k2) {
              num[dq][2 * k2] = num[dq][2 * k2] * a + lo_float(pv[u][dq][k2]) * b;
              num[dq][2 * k2 + 1] = num[dq][2 * k2 + 1] * a + hi_float(pv[u][dq][k2]) * b;
            }
          Mx = mn;
        }
      }
      if (row_ok[t]) {
        float o[kDq][16];
        const float inv = (den == 0.f) ? 0.f : 1.f / den;
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int k2 = 0; k2 < 16; ++k2) o[dq][k2] = num[dq][k2] * inv;
        write_row(t, o);
      }
    }
    if (lane == 0)  // ready for the next call
      __hip_atomic_store(&counters[item0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int DQK, int DV, int DVS, int KV_STRIDE, int BS, int KB, int NT>
hipError_t run_prefill(const PrefillArgs& a, hipStream_t stream) {
  using S16 = typename T::storage;
  hipLaunchKernelGGL((prefill_kernel<T, DQK, DV, DVS, KV_STRIDE, BS, KB, NT>), dim3(a.workgroups),
                     dim3(kPfWaves * kWave), 0, stream, static_cast<S16*>(a.out), static_cast<const S16*>(a.q),
                     static_cast<const char*>(a.k_pool), static_cast<const char*>(a.v_pool), a.block_tables,
                     a.context_lens, a.query_start, a.counters, a.ws_ml, a.ws_acc, fabsf(a.scale) * kLog2e,
                     a.num_seqs, a.num_query_rows, a.num_heads, a.num_kv_heads, a.num_heads / a.num_kv_heads,
                     a.num_blocks, a.max_blocks_per_seq, a.part_tokens, a.max_items,
                     a.scale < 0.f ? 0x80008000u : 0u);
  return hipGetLastError();
}

template <typename T, int DQK, int DV, int DVS, int KV_STRIDE, int KB, int NT>
hipError_t run_prefill_bs(const PrefillArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_prefill<T, DQK, DV, DVS, KV_STRIDE, 16, KB, NT>(a, stream)
                            : run_prefill<T, DQK, DV, DVS, KV_STRIDE, 32, KB, NT>(a, stream);
}

template <typename T, int D>
hipError_t run_prefill_nt(const PrefillArgs& a, hipStream_t stream) {
  return a.row_tiles == 2 ? run_prefill_bs<T, D, D, D, D, 2, 2>(a, stream)
                          : run_prefill_bs<T, D, D, D, D, 2, 1>(a, stream);
}

template <typename T>
hipError_t run_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  if (a.latent) return hipErrorInvalidValue;  // the latent cache has its own kernel (mla_split_kernel)
  return a.head_dim == 64 ? run_prefill_nt<T, 64>(a, stream) : run_prefill_nt<T, 128>(a, stream);
}

// ---------------------------------------------------------------------------
// Decode over the latent (MLA) cache with the head dimension split across the
// four waves of a workgroup.  A latent row is 576 elements: wave w owns latent
// elements [128w, 128w + 128) — its share of the scores and its 128-element
// slice of the values — and waves 0 and 1 also one 32-element half of the
// 64-element rotary part.  Per 32-key step each wave loads only its slice of
// the key rows (so the workgroup reads every latent row once), computes the
// partial scores S^T over its elements with the 16x16x32 products, and the
// four partials are summed through LDS (double-buffered: one barrier per
// step); every wave then runs the same softmax on the full scores and
// accumulates O^T += V^T P^T for its own value slice (whose rows it loads in
// the transposed-operand layout; the lines are the ones it just read for its
// scores).  A work item is (sequence, context partition, 16 heads).
constexpr int kMlaWaves = 4;
constexpr int kMlaOwn = kMlaVDim / kMlaWaves;  // latent elements per wave (128)

template <typename T, int BS>
__global__ __launch_bounds__(kMlaWaves* kWave, 2) void mla_split_kernel(
    typename T::storage* __restrict__ out, const typename T::storage* __restrict__ q,
    const char* __restrict__ kv_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, uint32_t* __restrict__ counters, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, float qk_scale, int num_seqs, int num_heads, int num_blocks, int max_blocks,
    int part_tokens, int max_items, uint32_t q_sign_bits) {
  using S16 = typename T::storage;
  using M = Mfma<T>;
  using PV = PvOps<T, 2>;
  using pw_t = typename PV::word_t;
  constexpr int kThreads = kMlaWaves * kWave;
  constexpr int kPer = (kPfMaxSeqs + kThreads - 1) / kThreads;
  constexpr int kJ = 5;       // 32-element score slices a wave may own (4 latent + 1 rotary)
  constexpr int kDq = kMlaOwn / 64;
  constexpr int kRowB = kMlaQkDim * 2;
  __shared__ int s_off[kPfMaxSeqs + 1];
  __shared__ int s_len[kPfMaxSeqs];
  __shared__ int s_wsum[kMlaWaves];
  __shared__ uint32_t s_ticket;
  __shared__ f4_t s_sc[2][kMlaWaves][2][kWave];  // partial scores of the last two steps

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int cap = max_blocks * BS;
  const int tiles = (num_heads + kPfRows - 1) / kPfRows;

  // 1. lengths and the prefix sum of items (tiles x partitions) per sequence
  for (int s = tid; s < S; s += kThreads) s_len[s] = min(max(context_lens[s], 0), cap);
  __syncthreads();
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    cnt[i] = s < S ? tiles * max(1, (s_len[s] + part_tokens - 1) / part_tokens) : 0;
    mine += cnt[i];
  }
  const int incl = wave_prefix_sum(mine);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kMlaWaves; ++w) {
    const int v = s_wsum[w];
    before += (w < wave) ? v : 0;
    total += v;
  }
  int run = before + incl - mine;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    if (s < S) s_off[s] = run;
    run += cnt[i];
  }
  if (tid == 0) s_off[S] = total;
  __syncthreads();
  total = min(__builtin_amdgcn_readfirstlane(total), max_items);

  const u32x4 q_sign = {q_sign_bits, q_sign_bits, q_sign_bits, q_sign_bits};
  const int col = lane % 16;
  const int g4 = lane / 16;
  const int nj = wave < 2 ? 5 : 4;  // waves 0 and 1 also take a rotary half
  // element offset of score slice j of this wave
  auto dim_of = [&](int j) __attribute__((always_inline)) {
    return j < 4 ? kMlaOwn * wave + 32 * j : kMlaVDim + 32 * wave;
  };
  const int own0 = kMlaOwn * wave;  // first value element of this wave

  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int x_end = min(total, (xcd + 1) * per_xcd);
  const int x_step = gridDim.x / kXcds;
  int parity = 0;
  for (int item = xcd * per_xcd + blockIdx.x / kXcds; item < x_end; item += x_step) {
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
    const int parts = max(1, (L + part_tokens - 1) / part_tokens);
    // head tiles fastest: the tiles of one partition read the same latent
    // rows, in adjacent workgroups of one XCD, so all but the first read hit L2
    const int local = item - __builtin_amdgcn_readfirstlane(s_off[s]);
    const int tile = local % tiles;
    const int part = local / tiles;
    const int h = tile * kPfRows + col;
    const bool row_ok = h < num_heads;
    const int k_begin = part * part_tokens;
    const int k_end = min(k_begin + part_tokens, L);

    u32x4 qv[kJ];
    {
      const S16* qrow = q + (static_cast<size_t>(s) * num_heads + (row_ok ? h : 0)) * kMlaQkDim + 8 * g4;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const u32x4 v = (j < nj) ? (load16(qrow + dim_of(j)) ^ q_sign) : u32x4{0u, 0u, 0u, 0u};
        qv[j] = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
    float m = -INFINITY, lsum = 0.f;
    f4_t acc[kDq][4];
#pragma unroll
    for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[dq][e] = f4_t{0.f, 0.f, 0.f, 0.f};
    int bad = 0;

    struct Stage {
      u32x4 k[2][kJ];
      u32x2 v[2][kDq][4];
      int c, bad;
    };
    const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
    auto load_step = [&](Stage& st, int c) __attribute__((always_inline)) {
      st.c = c;
      st.bad = 0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key0 = (c + 16 * kb < k_end) ? c + 16 * kb : c;
        int phys = tbl[key0 / BS];
        if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
          st.bad = 1;
          phys = 0;
        }
        const char* rows = kv_pool + (static_cast<size_t>(phys) * BS + key0 % BS) * kRowB;
#pragma unroll
        for (int j = 0; j < kJ; ++j)
          st.k[kb][j] = (j < nj) ? load16(rows + col * kRowB + (dim_of(j) + 8 * g4) * 2) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.v[kb][dq][e] =
                *reinterpret_cast<const u32x2*>(rows + (4 * g4 + e) * kRowB + (own0 + 64 * dq + 4 * col) * 2);
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
      // partial scores over this wave's elements, summed across the waves
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kJ; ++j)
          if (j < nj) sc = M::qk(st.k[kb][j], qv[j], sc);
        s_sc[parity][wave][kb][lane] = sc;
      }
      __syncthreads();
      float z[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f4_t t = s_sc[parity][0][kb][lane];
#pragma unroll
        for (int w = 1; w < kMlaWaves; ++w) t += s_sc[parity][w][kb][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[kb][i] = t[i];
      }
      parity ^= 1;
      const bool masked = st.c + 32 > k_end;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            z[kb][i] = (st.c + 16 * kb + 4 * g4 + i < k_end) ? z[kb][i] : -INFINITY;
      }
      float cm = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                       fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
      cm = fold_max<16>(cm);  // the row's four lanes: l, l ^ 16, l ^ 32, l ^ 48
      const float cms = (cm == -INFINITY) ? -INFINITY : cm * qk_scale;
      const float mn = fmaxf(m, cms);
      if (__builtin_amdgcn_ballot_w64(mn > m + kRescaleLog2) != 0) {
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[dq][e] *= alpha;
        m = mn;
      }
      const float nm = -m;
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = fast_exp2(fmaf(z[kb][i], qk_scale, nm));
          p[kb][i] = (masked && z[kb][i] == -INFINITY) ? 0.f : x;
          lsum += p[kb][i];
        }
      const pw_t pw = {M::pack2(p[0][0], p[0][1]), M::pack2(p[0][2], p[0][3]), M::pack2(p[1][0], p[1][1]),
                       M::pack2(p[1][2], p[1][3])};
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const pw_t a = {col_pair(st.v[0][dq][0], st.v[0][dq][1], e), col_pair(st.v[0][dq][2], st.v[0][dq][3], e),
                          col_pair(st.v[1][dq][0], st.v[1][dq][1], e), col_pair(st.v[1][dq][2], st.v[1][dq][3], e)};
          acc[dq][e] = PV::mma(a, pw, acc[dq][e]);
        }
    };

    const int n_steps = k_end > k_begin ? (k_end - k_begin + 31) / 32 : 0;
    if (n_steps > 0) {
      Stage a, b;
      load_step(a, k_begin);
      int c = 0;
      for (; c + 2 < n_steps; c += 2) {
        load_step(b, k_begin + (c + 1) * 32);
        attend_step(a);
        load_step(a, k_begin + (c + 2) * 32);
        attend_step(b);
      }
      if (c + 1 < n_steps) {
        load_step(b, k_begin + (c + 1) * 32);
        attend_step(a);
        attend_step(b);
      } else {
        attend_step(a);
      }
    }
    float lrow = fold_sum<16>(lsum);
    if (bad) lrow = __builtin_nanf("");

    auto write_row = [&](const float (&o)[kDq][16]) __attribute__((always_inline)) {
      S16* orow = out + (static_cast<size_t>(s) * num_heads + h) * kMlaVDim + own0 + 16 * g4;
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq) {
        uint32_t w[8];
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) w[k2] = M::pack2(o[dq][2 * k2], o[dq][2 * k2 + 1]);
        store16(orow + 64 * dq, u32x4{w[0], w[1], w[2], w[3]});
        store16(orow + 64 * dq + 8, u32x4{w[4], w[5], w[6], w[7]});
      }
    };
    if (parts == 1) {
      if (row_ok) {
        float o[kDq][16];
        const float inv = (lrow == 0.f) ? 0.f : 1.f / lrow;
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[dq][4 * i + e] = acc[dq][e][i] * inv;
        write_row(o);
      }
      continue;
    }
    // partial of a split item: slot `item`, 16 rows x (max, sum) and 512 sums
    {
      const size_t row = static_cast<size_t>(item) * kPfRows + col;
      if (wave == 0 && g4 == 0) store_coherent_u64(ws_ml + row * 2, m, lrow);
      float* av = ws_acc + row * kMlaVDim + own0 + 16 * g4;
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          store_coherent_u64(av + 64 * dq + 4 * i, acc[dq][0][i], acc[dq][1][i]);
          store_coherent_u64(av + 64 * dq + 4 * i + 2, acc[dq][2][i], acc[dq][3][i]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int item0 = item - part * tiles;  // this tile's partition-0 item; its partitions are tiles apart
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(&counters[item0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != static_cast<uint32_t>(parts - 1)) continue;
    // last arrival: each wave merges its value slice of the 16 rows
    float Mx = -INFINITY, den = 0.f;
    float num[kDq][16];
#pragma unroll
    for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
      for (int k2 = 0; k2 < 16; ++k2) num[dq][k2] = 0.f;
    constexpr int kB = 60 / (1 + 8 * kDq);  // partials per batch: at most 60 loads per lane in flight
    for (int p0 = 0; p0 < parts; p0 += kB) {
      uint64_t pml[kB];
      uint64_t pvv[kB][kDq][8];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const size_t row = (static_cast<size_t>(item0) + static_cast<size_t>(min(p0 + u, parts - 1)) * tiles) *
                               kPfRows + col;
        pml[u] = load_coherent_u64(ws_ml + row * 2);
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2)
            pvv[u][dq][k2] = load_coherent_u64(ws_acc + row * kMlaVDim + own0 + 64 * dq + 16 * g4 + 2 * k2);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (p0 + u >= parts) break;
        const float mu = lo_float(pml[u]);
        if (mu == -INFINITY) continue;
        const float mn = fmaxf(Mx, mu);
        const float a = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - mn);
        const float b = fast_exp2(mu - mn);
        den = den * a + hi_float(pml[u]) * b;
#pragma unroll
        for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2) {
            num[dq][2 * k2] = num[dq][2 * k2] * a + lo_float(pvv[u][dq][k2]) * b;
            num[dq][2 * k2 + 1] = num[dq][2 * k2 + 1] * a + hi_float(pvv[u][dq][k2]) * b;
          }
        Mx = mn;
      }
    }
    if (row_ok) {
      float o[kDq][16];
      const float inv = (den == 0.f) ? 0.f : 1.f / den;
#pragma unroll
      for (int dq = 0; dq < kDq; ++dq)
#pragma unroll
        for (int k2 = 0; k2 < 16; ++k2) o[dq][k2] = num[dq][k2] * inv;
      write_row(o);
    }
    if (tid == 0) __hip_atomic_store(&counters[item0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int BS>
hipError_t run_mla(const PrefillArgs& a, hipStream_t stream) {
  using S16 = typename T::storage;
  hipLaunchKernelGGL((mla_split_kernel<T, BS>), dim3(a.workgroups), dim3(kMlaWaves * kWave), 0, stream,
                     static_cast<S16*>(a.out), static_cast<const S16*>(a.q), static_cast<const char*>(a.k_pool),
                     a.block_tables, a.context_lens, a.counters, a.ws_ml, a.ws_acc, fabsf(a.scale) * kLog2e,
                     a.num_seqs, a.num_heads, a.num_blocks, a.max_blocks_per_seq, a.part_tokens, a.max_items,
                     a.scale < 0.f ? 0x80008000u : 0u);
  return hipGetLastError();
}

template <typename T>
hipError_t run_mla_t(const PrefillArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_mla<T, 16>(a, stream) : run_mla<T, 32>(a, stream);
}

}  // namespace

hipError_t launch_mla_split(const PrefillArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_mla_t<BF16>(a, stream) : run_mla_t<F16>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_prefill_t<BF16>(a, stream) : run_prefill_t<F16>(a, stream);
}

}  // namespace pa
