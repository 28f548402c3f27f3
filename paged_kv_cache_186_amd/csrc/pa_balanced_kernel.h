// Balanced-split decode kernel template (gfx950), included by
// pa_decode_balanced.hip (one query head per K/V head) and
// pa_decode_balanced_gqa{2,4}.hip (grouped-query heads, 2 or 4 per K/V load).
//
// Same computation as the partitioned kernel (pa_decode.hip): single-query
// softmax attention per (sequence, head) over K/V rows found through the block
// table — page "PagedAttentionMetal：基于Metal 3的Apple Silicon原生LLM推理加速方案",
// section 注意力计算优化; vLLM tutorial page "3. PagedAttention原理", §3.2 and
// the closing remarks of §3.4 — with the log-sum-exp merge of split rows (the
// "Flash-Dec" milestone named on the "PagedAttention MLX：为Apple Silicon打造的
// 高吞吐量LLM推理引擎" page).  Only the distribution of work differs.
//
// Work decomposition (our design): all (sequence, head, block) units are laid
// out in one sequence — sequence-major, then head, then logical block — and
// W = min(waves of a fixed grid, T) waves take shares of equal cost: a unit
// costs kBalancedCostUnit and each row (sequence, head) kBalancedCostRow more,
// the measured time of a row change, so a wave whose share crosses many short
// rows gets fewer units.  Each share is a contiguous run of units (possibly
// none, for a share that falls between two rows' units).  Every wave moves
// about the same bytes whatever the mix of context lengths, every workgroup
// starts at once, and consecutive shares — which land on different XCDs —
// read every head.  Each workgroup rebuilds the per-sequence unit and cost
// offsets in LDS from context_lens (exclusive prefix sums), so the host needs
// no knowledge of the lengths.
//
// A wave walks its share with the same two-stage load pipeline and per-lane-
// group online softmax as the partitioned kernel.  When the row (sequence,
// head) changes it folds its lane groups into one (max, sum, weighted V sum):
//  * a row lying entirely inside the share is final: written to out at once;
//  * only the first and the last row of a share can straddle a boundary; for
//    those the wave stores a partial in slot (k + row) — distinct for every
//    (wave, row) pair, because a later wave never touches an earlier row — and
//    after its loop takes a ticket from the row's counter.  The wave that draws
//    the last ticket merges the row's partials (slots kf+row .. kl+row for the
//    first and last waves kf, kl covering it) and resets the counter.
// Partials and tickets use L2-bypassing agent-scope accesses: the shares of one
// row run on different XCDs, whose L2 caches are not coherent with each other.

#pragma once

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr int kWaveMergeBatch = 8;  // partials in flight per lane group while merging
// Batches of up to this many sequences build their prefix sums per wave (one
// lane per sequence) instead of per workgroup.
#ifndef PA_WAVE_LOCAL_SEQS
#define PA_WAVE_LOCAL_SEQS 64
#endif
constexpr int kWaveLocalSeqs = PA_WAVE_LOCAL_SEQS;
static_assert(kWaveLocalSeqs <= kWave, "one lane per sequence");

// Cost of one row of `units` units in the balanced split, with a row charge
// RC (kBalancedCostUnit, kBalancedCostRow / kBalancedCostRowWide:
// pa_internal.h).
constexpr int kCostUnit = kBalancedCostUnit;
template <int RC>
__device__ __forceinline__ int row_cost(int units) {
  return units > 0 ? RC + kCostUnit * units : 0;
}

// One pipeline stage: one tile's K/V, its row's query slice, and its place.
// A unit is R consecutive rows of one (block, head) tile, at most
// kUnitLoads wave loads per tensor, so two pipeline stages stay well inside
// the register budget of 4 waves per SIMD (16 waves per CU keep far more
// bytes in flight than the memory system needs).  A 16-row fp16 block is two
// units of 8 rows by default.
#ifndef PA_UNIT_LOADS
#define PA_UNIT_LOADS 2
#endif
constexpr int kUnitLoads = PA_UNIT_LOADS;
// Grouped-query waves spend GW times the arithmetic on each byte, so between
// two loads they compute for much longer; a unit twice as large keeps as many
// bytes in flight per wave relative to that work.
#ifndef PA_UNIT_LOADS_GROUPED
#define PA_UNIT_LOADS_GROUPED 4
#endif
constexpr int kUnitLoadsGrouped = PA_UNIT_LOADS_GROUPED;
// Grouped kernels use at most T / grouped_min_units<GW>() waves: their units
// are few and arithmetic-heavy on small batches, and splitting a row over
// many waves made the split rows' tickets (many waves' atomics on one row
// counter) and merges (GW heads' partials from each wave) the bulk of the
// time.  Measured on the layer shape (8 sequences, 32 query heads): with 16
// K/V heads (GW 2) 20.5 us with every wave, 17.9 us with at least 8 units per
// wave; with 8, 4 or 1 K/V heads (GW 4) at least 2 / 3 / 4 / 6 / 8 / 10 units:
// 25.7 / 23.9 / 22.1 / 21.2 / 22.9 / 25.1 us (8 K/V heads); large batches
// keep every wave busy either way.
template <int GW>
constexpr long long grouped_min_units() {
  return GW >= 4 ? 6 : 8;
}

template <typename T, int D, int BS, int GW>
struct Unit {
  static constexpr int kLoads = GW > 1 ? kUnitLoadsGrouped : kUnitLoads;
  static constexpr int kRowsPerLoad = kWave / (D / T::kElems);
  static constexpr int kRows =
      (kLoads * kRowsPerLoad < BS) ? kLoads * kRowsPerLoad : BS;  // R
  static constexpr int kPerBlock = BS / kRows;
  static_assert(BS % kRows == 0, "units tile a block");
};

template <typename QT, typename KT, int D, int BS, int GW>
struct BStage {
  u32x4 k[Tile<KT, D, Unit<KT, D, BS, GW>::kRows>::kLoads];
  u32x4 v[Tile<KT, D, Unit<KT, D, BS, GW>::kRows>::kLoads];
  u32x4 q[GW][QSlice<QT, KT>::kVecs];  // the query slices of the row's GW heads
  float sk, sv;         // K and V scales of the unit's (block, head) (8-bit KV only)
  int s, h, u, L, bad;  // u: unit index within the row
  int newrow;           // the unit opens a row segment of this wave (q is loaded)
};

// floor(a / b) for 0 <= a <= 2^53 and b >= 1, given rb = 1.0 / b in fp64.  A
// 64-bit integer division expands to a long software sequence on this GPU
// (it sat in every row change of the walk below); here the fp64 quotient
// a * rb (a is exact in fp64, rb and the product are correctly rounded) lies
// within 2^-51 * (a / b) < 1 of a / b, so its truncation is off by at most
// one, and one integer step makes it exact.
__device__ __forceinline__ long long floor_div(long long a, long long b, double rb) {
  long long c = static_cast<long long>(static_cast<double>(a) * rb);
  if (c * b > a)
    --c;
  else if ((c + 1) * b <= a)
    ++c;
  return c;
}

// The wave whose share holds position x: the largest k with
// floor(k*T/W) <= x (rT = 1.0 / T).
__device__ __forceinline__ long long wave_of_tile(long long x, long long T, long long W, double rT) {
  return floor_div((x + 1) * W - 1, T, rT);
}

// Log-sum-exp merge of one row's partials by a single wave (64 lanes), for
// the GW heads of the row at once.  A slot holds the partials of GW heads side
// by side: head g of partial i sits at ml + 2*(i*GW + g) and acc + D*(i*GW + g).
// Every load is independent of every other, so a batch of B partials per lane
// group and head — their (max, sum) pairs and 16-byte slices of their vectors —
// is issued at once: a row split over up to kG*B waves merges in one memory
// round trip, whatever GW.  Each batch is folded into a running (max, sum,
// vector) per head with the online rescaling, so any number of partials works.
// out_row: the output of the row's first head (head g at out_row + g*D).
template <typename T, int D, int GW>
__device__ __forceinline__ void merge_row_wave(typename T::storage* __restrict__ out_row,
                                               const float* __restrict__ ml,
                                               const float* __restrict__ acc, int nparts, int lane) {
  constexpr int kChunks = D / 4;       // 16-byte slices of a partial row
  constexpr int kG = kWave / kChunks;  // partials read side by side
  // B partials per lane group and batch: 3 loads each per head, GW*B*3 <= 48
  // per lane, within the 63 loads a wave can have in flight, so that a batch
  // is one memory round trip
  constexpr int B = GW <= 2 ? kWaveMergeBatch : (2 * kWaveMergeBatch) / GW;
  const int c = lane % kChunks;
  const int gl = lane / kChunks;
  float M[GW];       // running max per head (identical in every lane)
  float den[GW];     // running sum of this lane group's partials, scaled to M
  float num[GW][4];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    M[h] = -INFINITY;
    den[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[h][e] = 0.f;
  }
  for (int i0 = 0; i0 < nparts; i0 += kG * B) {
    uint64_t pr[GW][B], lo[GW][B], hi[GW][B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const size_t i = min(i0 + u * kG + gl, nparts - 1);  // clamped: always issue the loads
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        pr[h][u] = load_coherent_u64(ml + 2 * (i * GW + h));
        lo[h][u] = load_coherent_u64(acc + (i * GW + h) * D + 4 * c);
        hi[h][u] = load_coherent_u64(acc + (i * GW + h) * D + 4 * c + 2);
      }
    }
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (i0 + u * kG + gl < nparts) bm = fmaxf(bm, lo_float(pr[h][u]));
      bm = fold_max<kChunks>(bm);
      const float Mn = fmaxf(M[h], bm);
      const float rs = (M[h] == -INFINITY) ? 0.f : fast_exp2(M[h] - Mn);
      den[h] *= rs;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[h][e] *= rs;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const float wi = (i0 + u * kG + gl < nparts) ? fast_exp2(lo_float(pr[h][u]) - Mn) : 0.f;
        den[h] = fmaf(wi, hi_float(pr[h][u]), den[h]);
        num[h][0] = fmaf(wi, lo_float(lo[h][u]), num[h][0]);
        num[h][1] = fmaf(wi, hi_float(lo[h][u]), num[h][1]);
        num[h][2] = fmaf(wi, lo_float(hi[h][u]), num[h][2]);
        num[h][3] = fmaf(wi, hi_float(hi[h][u]), num[h][3]);
      }
      M[h] = Mn;
    }
  }
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    den[h] = fold_sum<kChunks>(den[h]);
#pragma unroll
    for (int e = 0; e < 4; ++e) num[h][e] = fold_sum<kChunks>(num[h][e]);
    if (gl == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) out_row[h * D + 4 * c + e] = T::pack(num[h][e] / den[h]);
  }
}

// QT: query / output storage; KT: K/V cache storage (QT itself, or an 8-bit
// type whose (block, head) scales come from k_scales / v_scales).  GW: query
// heads served by each K/V tile load (grouped-query attention: the GW heads
// of a work row share one K/V head; 1 for plain multi-head attention).  A work
// "row" is (sequence, group of GW query heads); query head h reads K/V head
// h / group, group = num_heads / num_kv_heads.
// Launch bounds: the plain 16-bit kernels fit 4 waves per SIMD (<= 128
// VGPRs); the 8-bit ones 2 (<= 256); the grouped ones, which hold several
// heads' state per lane, may use the whole register file of one wave per
// SIMD (the launch shape has one wave per SIMD in every case).
template <typename QT, typename KT, int D, int BS, int NW, int GW>
__global__ __launch_bounds__(NW* kWave, GW > 1 ? 1 : (KT::kScaled ? 2 : 16 / NW)) void decode_balanced_kernel(
    typename QT::storage* __restrict__ out, uint32_t* __restrict__ counters,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, const typename QT::storage* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    float q_scale, int num_seqs, int num_heads, int num_kv_heads, int group, int num_blocks,
    int max_blocks) {
  using U = Unit<KT, D, BS, GW>;
  constexpr int R = U::kRows;
  constexpr int kUnitsPerBlock = U::kPerBlock;
  using C = Tile<KT, D, R>;
  using St = BStage<QT, KT, D, BS, GW>;
  using QS = QSlice<QT, KT>;
  constexpr int E = KT::kElems;
  constexpr int kThreads = NW * kWave;
  constexpr int kPer = (kBalancedMaxSeqs + kThreads - 1) / kThreads;  // sequences per thread
  // the row charge of the cost model: the wide one where a row change folds
  // more state (grouped heads, or 16 elements per lane over an 8-bit cache);
  // the host's range bound assumes at most 2 units per block for it, 8 else
  constexpr int kCostRow = (GW > 1 || KT::kScaled) ? kBalancedCostRowWide : kBalancedCostRow;
  static_assert(U::kPerBlock <= (kCostRow == kBalancedCostRow ? 8 : 2),
                "units per block within the host's cost bound");
  static_assert(NW * (kWave + 1) <= kBalancedMaxSeqs, "every wave's copy of the prefix sums fits");
  __shared__ int s_off[kBalancedMaxSeqs + 1];   // units of all sequences before s (per head)
  __shared__ int s_coff[kBalancedMaxSeqs + 1];  // cost of all sequences before s (per head)
  __shared__ int s_len[kBalancedMaxSeqs];
  __shared__ int s_wsum[NW];
  __shared__ int s_wcost[NW];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int NH = num_heads;      // query heads
  const int H = num_heads / GW;  // work rows per sequence
  const int HKV = num_kv_heads;
  const int cap = max_blocks * BS;

  // 1. clamped lengths and the exclusive prefix sums of units and of cost per
  //    sequence (one row's cost: kCostRow + kCostUnit per unit, nothing for an
  //    empty row).  Up to kWaveLocalSeqs sequences every wave builds its own
  //    copy (lane s owns sequence s; wave w's copy at offset w * (kWave + 1) of
  //    each array): no workgroup barrier between the lengths load and the
  //    first K/V loads.  Past that thread t owns sequences [t*kPer,
  //    (t+1)*kPer) and the workgroup shares one copy.
  // (not for fp16 queries with four heads per load over an 8-bit cache:
  // those instances use the whole register file, and the second prologue
  // pushed 12 bytes per lane of the unit loop's values to scratch memory —
  // continuous batching with 8 K/V heads over E4M3 46.4 -> 48.2 us; the bf16
  // instances keep 24 bytes there either way and gain 0.8 us)
  constexpr bool kWaveLocalOk = !(GW >= 4 && KT::kScaled && __is_same(QT, F16));
  const bool wave_local = kWaveLocalOk && S <= kWaveLocalSeqs;
  const int sb = wave_local ? wave * (kWave + 1) : 0;
  int* const off_l = s_off + sb;
  int* const coff_l = s_coff + sb;
  int* const len_l = s_len + sb;
  int total = 0;
  int total_c = 0;
  if (wave_local) {
    const int L = lane < S ? min(max(context_lens[lane], 0), cap) : 0;
    const int nb = (L + R - 1) / R;  // units of sequence `lane` (per head)
    const int c = row_cost<kCostRow>(nb);
    const int incl = wave_prefix_sum(nb);
    const int incl_c = wave_prefix_sum(c);
    if (lane < S) {
      len_l[lane] = L;
      off_l[lane] = incl - nb;
      coff_l[lane] = incl_c - c;
    }
    total = __builtin_amdgcn_readlane(incl, kWave - 1);
    total_c = __builtin_amdgcn_readlane(incl_c, kWave - 1);
    if (lane == 0) {
      off_l[S] = total;
      coff_l[S] = total_c;
    }
    // the wave's own LDS writes before its reads below (no other wave reads them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  } else {
    for (int s = tid; s < S; s += kThreads) s_len[s] = min(max(context_lens[s], 0), cap);  // coalesced
    __syncthreads();
    int nbl[kPer];
    int mine = 0;
    int mine_c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int s = tid * kPer + i;
      nbl[i] = s < S ? (s_len[s] + R - 1) / R : 0;  // units of sequence s (per head)
      mine += nbl[i];
      mine_c += row_cost<kCostRow>(nbl[i]);
    }
    const int incl = wave_prefix_sum(mine);
    const int incl_c = wave_prefix_sum(mine_c);
    if (lane == kWave - 1) {
      s_wsum[wave] = incl;
      s_wcost[wave] = incl_c;
    }
    __syncthreads();
    int before = 0;
    int before_c = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = s_wsum[w];
      const int vc = s_wcost[w];
      before += (w < wave) ? v : 0;
      before_c += (w < wave) ? vc : 0;
      total += v;
      total_c += vc;
    }
    int run = before + incl - mine;
    int run_c = before_c + incl_c - mine_c;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int s = tid * kPer + i;
      if (s < S) {
        s_off[s] = run;
        s_coff[s] = run_c;
      }
      run += nbl[i];
      run_c += row_cost<kCostRow>(nbl[i]);
    }
    if (tid == 0) {
      s_off[S] = total;
      s_coff[S] = total_c;
    }
    __syncthreads();
  }
  total = __builtin_amdgcn_readfirstlane(total);
  total_c = __builtin_amdgcn_readfirstlane(total_c);

  // 2. empty contexts give zero rows (spread over the workgroups)
  for (int s = blockIdx.x; s < S; s += gridDim.x)
    if (len_l[s] == 0)
      for (int i = tid; i < NH * D; i += kThreads) out[static_cast<size_t>(s) * NH * D + i] = QT::pack(0.f);

  // 3. this wave's share (no workgroup barrier after this point).  Work is
  // laid out as rows (sequence-major, then head), each a row cost kCostRow
  // followed by its units at kCostUnit each; unit x starts at cost position
  // C(x).  Wave k owns the units whose cost start lies in
  // [floor(k*C_all/Wn), floor((k+1)*C_all/Wn)): a contiguous run of units,
  // and equal cost per wave charges each row segment for the time a row
  // change takes.  Wn = min(waves in the grid, T): a share is then at least
  // kCostUnit long, so every wave between the owners of a row's first and
  // last units owns some of that row, and stores exactly one partial of it.
  const long long T_all = static_cast<long long>(H) * total;
  const long long C_all = static_cast<long long>(H) * total_c;
  const long long Wn = min(static_cast<long long>(gridDim.x) * NW,
                           GW > 1 ? max(1LL, T_all / grouped_min_units<GW>()) : T_all);
  const long long k = static_cast<long long>(blockIdx.x) * NW + wave;
  if (k >= Wn) return;
  // C_all < 2^43 (the host bounds it) and Wn <= 2^10, so every dividend
  // below stays within floor_div's 2^53
  const double rC = 1.0 / static_cast<double>(C_all);
  const double rW = 1.0 / static_cast<double>(Wn);
  // cost start of the first unit of row (s, h)
  auto row_start = [&](int s, int h) __attribute__((always_inline)) {
    const int nb = __builtin_amdgcn_readfirstlane(off_l[s + 1] - off_l[s]);
    return static_cast<long long>(H) * __builtin_amdgcn_readfirstlane(coff_l[s]) +
           static_cast<long long>(h) * row_cost<kCostRow>(nb) + kCostRow;
  };
  // the first unit whose cost start is >= c: its sequence, head and index in
  // the row, and its place in the unit order (T_all and s = S past the end)
  auto first_unit_at = [&](long long c, int& s, int& h, int& j) __attribute__((always_inline)) {
    if (c >= C_all) {
      s = S;
      h = j = 0;
      return T_all;
    }
    // the largest s with H*coff[s] <= c (its cost range holds c, so it has
    // units): the lanes test 64 candidates at once, evenly spaced over all
    // sequences, then the 64 (or fewer) that follow the last one that passed
    int base = 0;
    int span = S;
    if (S > kWave) {
      const int stride = (S + kWave - 1) / kWave;
      const int cand = lane * stride;
      const uint64_t pass = __builtin_amdgcn_ballot_w64(cand < S && static_cast<long long>(H) * coff_l[cand] <= c);
      base = (63 - __builtin_clzll(pass)) * stride;  // lane 0 always passes (coff[0] = 0)
      span = min(stride, S - base);
    }
    const uint64_t pass =
        __builtin_amdgcn_ballot_w64(lane < span && static_cast<long long>(H) * coff_l[base + min(lane, span - 1)] <= c);
    s = base + (63 - __builtin_clzll(pass));
    const int nb = __builtin_amdgcn_readfirstlane(off_l[s + 1] - off_l[s]);
    const int rc = row_cost<kCostRow>(nb);
    const long long local = c - static_cast<long long>(H) * __builtin_amdgcn_readfirstlane(coff_l[s]);
    h = static_cast<int>(floor_div(local, rc, 1.0 / static_cast<double>(rc)));
    const int o = static_cast<int>(local - static_cast<long long>(h) * rc);  // in [0, rc)
    j = o <= kCostRow ? 0 : (o - kCostRow + kCostUnit - 1) / kCostUnit;   // in [0, nb]
    if (j == nb) {  // past the row's last unit start: the next row's first unit
      j = 0;
      if (++h == H) {
        h = 0;
        do {
          ++s;
        } while (s < S && __builtin_amdgcn_readfirstlane(off_l[s + 1] - off_l[s]) == 0);
        if (s == S) return T_all;
      }
    }
    const int nbs = __builtin_amdgcn_readfirstlane(off_l[s + 1] - off_l[s]);
    return static_cast<long long>(H) * __builtin_amdgcn_readfirstlane(off_l[s]) +
           static_cast<long long>(h) * nbs + j;
  };
  int w_s, w_h, w_j;
  const long long c1 = floor_div((k + 1) * C_all, Wn, rW);
  const long long t0 = first_unit_at(floor_div(k * C_all, Wn, rW), w_s, w_h, w_j);
  // a share that falls between two rows' units holds none: nothing to do
  if (w_s == S || row_start(w_s, w_h) + static_cast<long long>(kCostUnit) * w_j >= c1) return;
  // the share's end is found after its first loads are issued (below)
  long long t1 = 0;
  int w_nb = __builtin_amdgcn_readfirstlane(off_l[w_s + 1] - off_l[w_s]);
  // the K/V head of the row's query heads, updated only when the row changes
  // (no division when each work row is one whole group, as in plain MHA)
  auto kv_head = [&](int h) __attribute__((always_inline)) { return group == GW ? h : (h * GW) / group; };
  int w_kvh = kv_head(w_h);
  auto advance = [&]() __attribute__((always_inline)) {
    if (++w_j < w_nb) return;
    w_j = 0;
    if (++w_h < H) {
      w_kvh = kv_head(w_h);
      return;
    }
    w_h = 0;
    w_kvh = 0;
    do {
      ++w_s;
    } while (w_s < S && __builtin_amdgcn_readfirstlane(off_l[w_s + 1] - off_l[w_s]) == 0);
    if (w_s < S) w_nb = __builtin_amdgcn_readfirstlane(off_l[w_s + 1] - off_l[w_s]);
  };

  const int grp = lane / C::kLanesPerRow;
  const int col = lane % C::kLanesPerRow;

  bool first_stage = true;
  auto load_stage = [&](St& st) __attribute__((always_inline)) {
    // a row segment of this wave opens with its first stage or a row's first unit
    st.newrow = first_stage || w_j == 0;
    first_stage = false;
    // the query is needed only when a segment opens; grouped kernels load it
    // only then (first, so that the loads of the previous stage can be waited
    // for exactly whether or not these were issued)
    auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const char* qrow =
            reinterpret_cast<const char*>(q + (static_cast<size_t>(w_s) * NH + w_h * GW + g) * D);
#pragma unroll
        for (int i = 0; i < QS::kVecs; ++i) st.q[g][i] = load16(qrow + col * QS::kBytes + i * kVecBytes);
      }
    };
    if constexpr (GW > 1) {
      if (st.newrow) load_q();
    }
    const int blk = w_j / kUnitsPerBlock;
    const int sub = w_j % kUnitsPerBlock;
    int phys = block_tables[static_cast<size_t>(w_s) * max_blocks + blk];
    st.bad = 0;
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
      st.bad = 1;  // never dereference an id outside the pool
      phys = 0;
    }
    const int kvh = w_kvh;  // the K/V head of this row's query heads
    const size_t tile = ((static_cast<size_t>(phys) * HKV + kvh) * BS + sub * R) * C::kRowBytes;
    const char* kb = k_pool + tile + lane * kVecBytes;
    const char* vb = v_pool + tile + lane * kVecBytes;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) st.k[i] = load16_stream(kb + i * C::kLoadBytes);
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) st.v[i] = load16_stream(vb + i * C::kLoadBytes);
    if constexpr (GW == 1) load_q();
    if constexpr (KT::kScaled) {
      st.sk = load_uniform_f32(k_scales + static_cast<size_t>(phys) * HKV + kvh);
      st.sv = load_uniform_f32(v_scales + static_cast<size_t>(phys) * HKV + kvh);
    } else {
      st.sk = st.sv = 1.f;
    }
    st.s = w_s;
    st.h = w_h;
    st.u = w_j;
    st.L = __builtin_amdgcn_readfirstlane(len_l[w_s]);
    advance();
    // keep the scheduler from sinking these loads below the compute that
    // follows: they must be in flight while the previous stage is consumed
    __builtin_amdgcn_sched_barrier(0);
  };

  // state of the current row segment
  int cur_s = -1;
  int cur_h = 0;
  int seg_bad = 0;
  float m[GW];
  float l[GW];
  float acc[GW][E];
  float qf[GW][E];
  uint32_t qw[GW][E / 2];  // grouped heads over a 16-bit cache: the query's own words
  static_assert(!(GW > 1 && KT::kDot2) || (__is_same(QT, KT) && E == 8),
                "packed dot products need the query in the cache's 16-bit format");
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = qf[g][e] = 0.f;
  }
  // rows whose partial is stored and whose ticket is still to be taken (<= 2)
  int pend = 0;
  size_t pend_row[2] = {0, 0};
  int pend_s[2] = {0, 0};
  int pend_h[2] = {0, 0};
  int pend_n[2] = {0, 0};
  size_t pend_slot0[2] = {0, 0};

  auto flush = [&]() __attribute__((always_inline)) {
    const int nb = __builtin_amdgcn_readfirstlane(off_l[cur_s + 1] - off_l[cur_s]);
    const int off_s = __builtin_amdgcn_readfirstlane(off_l[cur_s]);
    const long long first = static_cast<long long>(H) * off_s + static_cast<long long>(cur_h) * nb;
    // the whole row lies in this share: final, no partial to merge
    const bool whole = first >= t0 && first + nb <= t1;
    const size_t row = static_cast<size_t>(cur_s) * H + cur_h;
    const size_t slot = static_cast<size_t>(k) + row;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      // fold the lane groups of the wave into one state
      float M = m[g];
      M = fold_max<C::kLanesPerRow>(M);
      const float sc = (m[g] == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
      float lt = l[g] * sc;
      float a[E];
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = acc[g][e] * sc;
      lt = fold_sum<C::kLanesPerRow>(lt);
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = fold_sum<C::kLanesPerRow>(a[e]);
      if (whole) {
        if (grp == 0) {
          float o[E];
          const float inv = 1.f / lt;
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = seg_bad ? __builtin_nanf("") : a[e] * inv;
          QS::store(out + (static_cast<size_t>(cur_s) * NH + cur_h * GW + g) * D, col, o);
        }
      } else {  // partial of head g in slot `slot`
        const size_t sg = slot * GW + g;
        if (grp == 0)
#pragma unroll
          for (int e = 0; e < E; e += 2) store_coherent_u64(ws_acc + sg * D + col * E + e, a[e], a[e + 1]);
        if (lane == 0) store_coherent_u64(ws_ml + sg * 2, M, seg_bad ? __builtin_nanf("") : lt);
      }
    }
    if (!whole) {  // the waves kf..kl cover the row: the owners of its first and last units
      const long long cf = row_start(cur_s, cur_h);
      const long long kf = wave_of_tile(cf, C_all, Wn, rC);
      const long long kl = wave_of_tile(cf + static_cast<long long>(kCostUnit) * (nb - 1), C_all, Wn, rC);
      if (pend == 0) {
        pend_row[0] = row;
        pend_s[0] = cur_s;
        pend_h[0] = cur_h;
        pend_n[0] = static_cast<int>(kl - kf + 1);
        pend_slot0[0] = static_cast<size_t>(kf) + row;
      } else {
        pend_row[1] = row;
        pend_s[1] = cur_s;
        pend_h[1] = cur_h;
        pend_n[1] = static_cast<int>(kl - kf + 1);
        pend_slot0[1] = static_cast<size_t>(kf) + row;
      }
      ++pend;
    }
  };

  auto attend_stage = [&](const St& st) __attribute__((always_inline)) {
    if (st.newrow) {  // a new row segment begins
      if (cur_s >= 0) flush();
      cur_s = st.s;
      cur_h = st.h;
      seg_bad = 0;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < QS::kVecs; ++i) QT::unpack(st.q[g][i], qf[g] + i * QT::kElems);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          acc[g][e] = 0.f;
          qf[g][e] *= q_scale;
        }
        if constexpr (GW > 1 && KT::kDot2) {
          qw[g][0] = st.q[g][0].x;
          qw[g][1] = st.q[g][0].y;
          qw[g][2] = st.q[g][0].z;
          qw[g][3] = st.q[g][0].w;
        }
      }
    }
    seg_bad |= st.bad;
    const int tok0 = st.u * R + grp;  // unit u holds tokens [u*R, (u+1)*R)
    if constexpr (GW == 1) {
      if ((st.u + 1) * R <= st.L)
        attend_tile<KT, D, R, false>(st.k, st.v, qf[0], m[0], l[0], acc[0], tok0, st.L, st.sk, st.sv);
      else
        attend_tile<KT, D, R, true>(st.k, st.v, qf[0], m[0], l[0], acc[0], tok0, st.L, st.sk, st.sv);
    } else {
      if ((st.u + 1) * R <= st.L)
        attend_tile_heads<KT, D, R, GW, false>(st.k, st.v, qf, qw, q_scale, m, l, acc, tok0, st.L, st.sk,
                                               st.sv);
      else
        attend_tile_heads<KT, D, R, GW, true>(st.k, st.v, qf, qw, q_scale, m, l, acc, tok0, st.L, st.sk,
                                              st.sv);
    }
  };

  // two-stage pipeline over the share (steady state without conditional
  // loads, then a one- or two-stage epilogue), then the last segment
  St a, b;
  load_stage(a);
  {
    int e_s, e_h, e_j;
    t1 = first_unit_at(c1, e_s, e_h, e_j);
  }
  const int nt = static_cast<int>(t1 - t0);  // >= 1
  int st = 0;
  for (; st + 2 < nt; st += 2) {
    load_stage(b);
    attend_stage(a);
    load_stage(a);
    attend_stage(b);
  }
  if (st + 1 < nt) {
    load_stage(b);
    attend_stage(a);
    attend_stage(b);
  } else {
    attend_stage(a);
  }
  flush();

  if (pend == 0) return;
  // tickets: this wave's partial stores must be performed first
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lane p (< pend) takes pending row p's ticket: both in one round trip
  uint32_t ticket = 0;
  const size_t my_row = lane == 1 ? pend_row[1] : pend_row[0];
  if (lane < pend)
    ticket = __hip_atomic_fetch_add(&counters[my_row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tk[2] = {static_cast<uint32_t>(__builtin_amdgcn_readlane(ticket, 0)),
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(ticket, 1))};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p >= pend) break;
    if (tk[p] == static_cast<uint32_t>(pend_n[p] - 1)) {
      const size_t rs = pend_s[p];  // sequence and head group of the row
      const size_t rh = pend_h[p];
      merge_row_wave<QT, D, GW>(out + (rs * NH + rh * GW) * D, ws_ml + pend_slot0[p] * GW * 2,
                                ws_acc + pend_slot0[p] * GW * D, pend_n[p], lane);
      if (lane == 0)  // ready for the next call
        __hip_atomic_store(&counters[pend_row[p]], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename QT, typename KT, int D, int BS, int GW>
hipError_t run_balanced(const DecodeArgs& a, hipStream_t stream) {
  using S = typename QT::storage;
  hipLaunchKernelGGL((decode_balanced_kernel<QT, KT, D, BS, kBalancedWaves, GW>), dim3(a.workgroups),
                     dim3(kBalancedWaves * kWave), 0, stream, static_cast<S*>(a.out), a.counters,
                     a.ws_ml, a.ws_acc, static_cast<const S*>(a.q),
                     static_cast<const char*>(a.k_pool), static_cast<const char*>(a.v_pool),
                     a.k_scales, a.v_scales, a.block_tables, a.context_lens, a.scale * kLog2e,
                     a.num_seqs, a.num_heads, a.num_kv_heads, a.num_heads / a.num_kv_heads,
                     a.num_blocks, a.max_blocks_per_seq);
  return hipGetLastError();
}

template <typename QT, typename KT, int D, int GW>
hipError_t run_balanced_bs(const DecodeArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_balanced<QT, KT, D, 16, GW>(a, stream)
                            : run_balanced<QT, KT, D, 32, GW>(a, stream);
}

template <typename QT, typename KT, int GW>
hipError_t run_balanced_d(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? run_balanced_bs<QT, KT, 64, GW>(a, stream)
                          : run_balanced_bs<QT, KT, 128, GW>(a, stream);
}

template <typename QT, int GW>
hipError_t run_balanced_kv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.kv_dtype) {
    case PA_DTYPE_FP8_E4M3:
      return run_balanced_d<QT, FP8E4M3, GW>(a, stream);
    case PA_DTYPE_FP8_E5M2:
      return run_balanced_d<QT, FP8E5M2, GW>(a, stream);
    default:
      return run_balanced_d<QT, QT, GW>(a, stream);
  }
}

}  // namespace
}  // namespace pa
