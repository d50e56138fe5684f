// Prefill view: the global context summary initialised over the whole prefix
// (LongSpark paper page, Fig. 3 caption) and the recent KV window filled
// from its last W rows (Fig. 2 (b)).
//
// For each (sequence c, KV head h) with newest position t = L0-1 and slot j:
//   a_jp = u_j.k_p/sqrt(d) + (t-p) ln lambda_j       (0 when p = t)
//   m = max_p a_jp, l = sum_p e^(a_jp-m), n = sum_p e^(a_jp-m) [k_p ; v_p]
// i.e. attention of S slot queries over the prefix rows with values [k|v]
// and a linear distance bias of slope -ln lambda_j per slot.
//
// Phase 1 (init_*_partial): the rows of each (c, h) are cut into `nsplit`
// contiguous ranges; one workgroup streams its range once (token-major
// [C, rows, Hkv, d] input, 256-byte row segments) and writes an (m, l, n)
// partial.  The bf16 d=128 kernel runs both contractions on MFMA
// (v_mfma_f32_32x32x16_bf16): S^T = K U^T per tile, then the online
// softmax in registers, then n^T += [K|V]^T P^T with P rounded to bf16 (l
// sums the same rounded weights, so n/l stays an exact weighted mean of the
// inputs).  Tiles run newest first, so each slot's maximum (the distance
// bias favours new rows) is met early and the lazy rescale rarely fires.
// Its splits are counted back from the newest row (InitPlan): the newest
// ~12K rows pool every slot, older rows only the slower-decaying half, once
// the faster half's weights there are shown negligible (see the kernel).
// The f32 kernel is a plain LDS-tiled loop for small shapes.
// Phase 2 (init_finalize): merges the partials (associative max-rescale;
// an empty partial has weight 0), writes the state and the slots, fills the
// ring, sets seq_len and err_flag.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// partial block of (split, unit): m[S] | l[S] | n[S][2d]
__device__ __host__ inline int64_t part_off(int split, int units, int unit, int S, int D) {
  return (int64_t(split) * units + unit) * int64_t(S) * (2 * D + 2);
}

// ---------------------------------------------------------------------------
// MFMA partial kernel, bf16, d = 128, S = 32 * NG slots, 2 * NG waves (two
// per SIMD at S = 128), both products on v_mfma_f32_32x32x16_bf16.
//  * NQ = 2, near splits (the newest rows): every slot.  Wave w owns slot
//    group w % NG (32 slots) and row half w / NG of every 64-row tile.
//  * NQ = 4, far splits (older rows): the slots are ranked by ln lambda and
//    only the slower-decaying half (NG / 2 groups) is pooled.  Wave w owns
//    pooled group w % (NG / 2) and row quarter w / (NG / 2) of every 128-row
//    tile, so a tile costs each wave what a near tile does and the split's
//    rows go by at twice the rate.  The faster half is then bounded: a slot's
//    maximum m_j is at least its score on the newest row t, and |u.k| <=
//    |u| |k| (Cauchy-Schwarz), so every row p of the split has
//      a_jp - m_j <= |u_j| (max_p |k_p| + |k_t|) / sqrt(d) - (t - p) |ln lambda_j|.
//    When that is below -48 for every slot of the faster half (rows at least
//    ~10K back for unit-scale keys and lambda <= 1 - 2^-7), the split records
//    those slots as empty (m = -inf, l = 0): the weights left out are below
//    e^-48 of the slot's largest, far under fp32 resolution even summed over
//    2^31 rows.  Otherwise it sets the split's flag, and a second launch
//    (kRest) pools the faster half of the flagged splits.
// Operands (both cases, rows counted inside the wave's 32-row group):
//   S^T[row][slot] = K U^T over the wave's 32 rows: A = 32 rows x 16 dims
//     from the row-major K tile, B = U^T (8 k-steps, read from LDS).
//     A-row m = 8j + 4h + r (j < 4, h < 2, r < 4) reads row 16(j/2) + 8h +
//     4(j%2) + r of the group, so that the output lane (slot, half h) holds
//     rows 8h..8h+7 and 16+8h..16+8h+7 in order: exactly the 8-row
//     k-slices of the P^T operand of the second product.
//   n^T[dim][slot] += [K|V]^T P^T per 16-row k-step: A = 32 dims x 16 rows,
//     read from the same row-major K and V tiles with ds_read_b64_tr_b16
//     (two 4-row transposed reads per operand), B = P^T packed from the
//     scores.
// The tiles hold K and V rows as they arrive (256 bytes per row, no
// transposition while staging); 16-byte chunk c of row r sits at chunk
// c ^ tile_swz(r), which keeps the score reads (16 rows, one chunk) and the
// transposed reads (4 rows x 4 chunks per 16 lanes) on distinct banks.
// Tiles go from global memory straight into LDS (global_load_lds_dwordx4:
// lane i of an instruction fills the i-th 16 bytes of a 1 KB LDS block, so
// each lane fetches the chunk that the swizzle places there), and the next
// tile streams in while one is computed, with one barrier per tile between
// reads and refills.  (That barrier's fence waits for all of a wave's loads,
// so the near kernel's third buffer holds no second tile in flight; it is
// the merge space of a slot group.)  The row groups of a slot group keep
// separate (m, l, n) and merge through LDS at the end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <int NG, int NQ, bool kRest = false>
__global__ __launch_bounds__(128 * NG, 1) void init_mfma32_partial(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, int64_t rows_stride,
    int L0, InitPlan plan, int split0, int nspl, const uint16_t* __restrict__ u,
    const float* __restrict__ log_lambda, int Hkv, float* __restrict__ part,
    int32_t* __restrict__ rest_flag) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  constexpr bool kFar = NQ == 4;
  static_assert(NQ == 2 || (NQ == 4 && NG % 2 == 0), "near: every slot group; far: half of them");
  static_assert(kFar || !kRest, "only far splits leave a rest");
  constexpr int D = 128, S = 32 * NG, NT = 128 * NG, NA = 2 * NG / NQ, TR = 32 * NQ;
  constexpr int KLS = D + 8;   // slot-query row stride (bf16 elements)
  constexpr int RS = D;        // K / V tile row stride: 256 bytes, swizzled chunks
  constexpr int KI = TR * RS / 512 / (NT / 64);  // 1 KB blocks of a K (or V) tile per wave
  static_assert(KI >= 1 && KI * (NT / 64) * 512 == TR * RS, "tile blocks must cover the waves");
  // merge records: 64 lanes x (m_true, m_run, l, 128 n).  Near: four LDS
  // arrays of at least one record each, tile buffers 0, 1, 2 ([K rows | V
  // rows] each) and the slot queries, and slot group g merges through array
  // g.  Far: two tile buffers of at least two records each, and the row
  // quarters of pooled group g merge through buffer g.  Separate arrays let
  // the compiler see that the tiles streaming into one buffer do not alias
  // the reads of another.
  constexpr int kRecFloats = 64 * 131;
  constexpr int kMergeElems = (kFar ? 2 : 1) * kRecFloats * 2;
  constexpr int kBufElems = 2 * TR * RS > kMergeElems ? 2 * TR * RS : kMergeElems;
  constexpr int kUElems = kFar ? NA * 32 * KLS : (S * KLS > kMergeElems ? S * KLS : kMergeElems);
  static_assert(NG <= 4, "one merge array per slot group");
  __shared__ __attribute__((aligned(16))) uint16_t buf0[kBufElems];
  __shared__ __attribute__((aligned(16))) uint16_t buf1[kBufElems];
  __shared__ __attribute__((aligned(16))) uint16_t buf2[kFar ? 8 : kBufElems];
  __shared__ __attribute__((aligned(16))) uint16_t UL[kUElems];  // [pooled slots][KLS]: their queries
  __shared__ int32_t s_order[kFar ? S : 1];  // far: the slot of each rank by ln lambda
  __shared__ float s_red[kFar ? 2 * (NT / 64) : 1];  // far: per-wave key bounds
  // s_waitcnt immediates: every load of this wave done / all but the newest
  // tile's 2 KI loads done (vmcnt in bits 3:0, expcnt and lgkmcnt not waited)
  static_assert(kFar || 2 * KI < 16, "one tile's loads fit the low vmcnt field");
  constexpr int kWaitAll = 0x0F70, kWaitButOne = 0x0F70 | ((2 * KI) & 15);
  // element offset of 16-byte chunk c of tile row r
  auto chunk_at = [](int r, int c) { return r * RS + ((c ^ tile_swz(r)) << 3); };

  const int split = split0 + int(blockIdx.x) % nspl;
  const int unit = int(blockIdx.x) / nspl;  // c * Hkv + h
  const int h = unit % Hkv;
  const int c = unit / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sgl = wave % NA, q = wave / NA;  // pooled slot group, row group
  const int m32 = lane & 31, hh = lane >> 5;
  // the split's rows, counted back from the newest
  int r_begin, r_end;
  init_split_rows(plan, L0, split, &r_begin, &r_end);
  const int t_newest = L0 - 1;
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float k2 = 0.08838834764831845f * kLog2e;  // log2(e) / sqrt(128)
  float* pb = part + part_off(split, int(gridDim.x) / nspl, unit, S, D);
  // far: one flag per (split, unit), set when the faster half is still to pool
  int32_t* flag = nullptr;
  if constexpr (kFar) flag = rest_flag + int64_t(split - plan.n_near) * (int(gridDim.x) / nspl) + unit;
  if constexpr (kRest)
    if (*flag == 0) return;

  if constexpr (kFar) {
    // rank the slots by ln lambda, ascending, ties by index (the integer
    // image of the bits orders every float, NaN included)
    auto key = [&](int i) {
      const int b = __float_as_int(log_lambda[i]);
      return b >= 0 ? b : b ^ 0x7fffffff;
    };
    for (int j = tid; j < S; j += NT) {
      const int kj = key(j);
      int r = 0;
      for (int i = 0; i < S; ++i) {
        const int ki = key(i);
        r += (ki < kj) || (ki == kj && i < j);
      }
      s_order[r] = j;
    }
  }

  // the tile row read by this lane as A-row m32 of its row group
  const int prow = q * 32 + 16 * (m32 >> 4) + 8 * ((m32 >> 2) & 1) + 4 * ((m32 >> 3) & 1) + (m32 & 3);
  // LDS element offsets, the same for every tile:
  //  score operand k-step ks: chunk 2 ks + hh of row prow of the K tile;
  //  P.V operands: in 16-lane group g = lane / 16 reader lane r reads
  //  dimensions 32 (db % 4) + 16 (g % 2) + 4 (r % 4) .. +3 of row
  //  tr_row + 16 t + 4 u (u = 0, 1: the two 4-row halves of the operand).
  //  With tile_swz, chunk 4 (db % 4) + c0 of such a row lands at
  //  ((db % 4) ^ (row % 4)) << 2 | (c0 ^ ((row / 4) % 4)), and row % 4 and
  //  (row / 4) % 4 do not depend on t, so an operand's offset is
  //  pv_base[u] + pv_blk[db % 4] + 16 t RS (+ the V tile's offset).
  int sc_off[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) sc_off[ks] = chunk_at(prow, 2 * ks + hh);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int tr_row = q * 32 + 8 * (g4 >> 1) + (r16 >> 2);
  const int c0 = 2 * (g4 & 1) + ((r16 & 3) >> 1);
  int pv_base[2], pv_blk[4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    pv_base[u] = (tr_row + 4 * u) * RS + ((c0 ^ (((tr_row >> 2) + u) & 3)) << 3) + 4 * (r16 & 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) pv_blk[k] = (k ^ (tr_row & 3)) << 5;

  // tile t0 -> LDS buffer b: wave w's block j holds K (or V) rows
  // 4(KI w + j) .. +3; lane i of it lands at 16-byte position p = 64 (KI w + j)
  // + i of the tile, i.e. row p / 16, chunk slot p % 16, which holds chunk
  // (p % 16) ^ tile_swz(row).  Rows past the tail repeat the last real row
  // (their scores are masked and their weights are 0).
  auto issue_tile = [&](int t0, uint16_t* buf) __attribute__((always_inline)) {
    const int nrows = min(TR, r_end - t0);
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int blk = KI * wave + j, p = 64 * blk + lane;
      const int row = p >> 4, ch = (p & 15) ^ tile_swz(p >> 4);
      const int64_t off = ((int64_t(c) * rows_stride + t0 + min(row, nrows - 1)) * Hkv + h) * D + ch * 8;
      uint16_t* kl = buf + blk * 512;
      __builtin_amdgcn_global_load_lds(kp + off, (__attribute__((address_space(3))) void*)kl, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + off, (__attribute__((address_space(3))) void*)(kl + TR * RS), 16, 0, 0);
    }
  };

  // Tiles run from the newest to the oldest: the distance bias makes newer
  // rows score higher, so each slot's maximum is met in the first tiles and
  // the lazy rescale below almost never fires (oldest first, it would fire
  // every few tiles as the bias grows by |ln lambda| per row).
  const int ntiles = (r_end - r_begin + TR - 1) / TR;
  auto tile_t0 = [&](int idx) { return r_begin + (ntiles - 1 - idx) * TR; };
  float kn_max = 0.f;  // far: the largest squared norm of this lane's half of its rows' keys

  {
    // far: the slower half (ranks S/2 .. S-1), or in kRest the faster half
    const int gbase = kFar && !kRest ? NG - NA : 0;
    if (kFar) __syncthreads();  // the ranking is done
    const int slot = kFar ? s_order[32 * (gbase + sgl) + m32] : sgl * 32 + m32;
    const int urow = sgl * 32 + m32;  // the slot's row in UL
    const float lnl2 = log_lambda[slot] * kLog2e;  // -inf stays -inf (lambda = 0)
    // the slot queries of the pooled groups, read per tile as the B operand
    // (lane (slot m32, hh) takes u[slot][16ks + 8hh .. +7]) from LDS:
    // registers go to the accumulators
    for (int p = tid; p < NA * 32 * 16; p += NT) {
      const int row = p >> 4;
      const int sj = kFar ? s_order[32 * gbase + row] : row;
      *reinterpret_cast<u16x8*>(&UL[row * KLS + (p & 15) * 8]) =
          *reinterpret_cast<const u16x8*>(u + (int64_t(h) * S + sj) * D + (p & 15) * 8);
    }

    float m_run = -INFINITY, l_run = 0.f;  // reference max (may lag) and weight sum
    float m_true = -INFINITY;               // exact running max
    f32x16 acc[8];  // n^T block db: lane (slot m32, hh) holds dims 32db + 8j + 4hh + r at [4j + r]
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x16{};

    // one tile computed from buffer cur while the next ones stream in; nxt
    // (the buffer of tile idx - 1) receives tile idx + 2 (near) or idx + 1 (far)
    auto tile_step = [&](int idx, const uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
      const int t0 = tile_t0(idx);
      const int nrows = min(TR, r_end - t0);
      const uint16_t* KL = cur;
      const uint16_t* VL = cur + TR * RS;
      if constexpr (kFar) {
        __builtin_amdgcn_s_waitcnt(kWaitAll);  // this wave's blocks of tile idx are in LDS
        __syncthreads();  // ... and every wave's; the reads of tile idx - 1 are done
        if (idx + 1 < ntiles) issue_tile(tile_t0(idx + 1), nxt);  // streams in during this tile
      } else {
        // this wave's blocks of tile idx are in LDS (tile idx + 1 may still stream)
        if (idx + 1 < ntiles)
          __builtin_amdgcn_s_waitcnt(kWaitButOne);
        else
          __builtin_amdgcn_s_waitcnt(kWaitAll);
        __syncthreads();  // ... and every wave's; the reads of tile idx - 1 are done
        if (idx + 2 < ntiles) issue_tile(tile_t0(idx + 2), nxt);  // streams in during this tile
      }

      // S^T for the wave's 32 rows (far: and the squared norm of the lane's
      // half of its row's key, from the same operand)
      f32x16 s = f32x16{};
      float kn = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u16x8 araw = *reinterpret_cast<const u16x8*>(&KL[sc_off[ks]]);
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u16x8*>(&UL[urow * KLS + ks * 16 + hh * 8]));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(araw), b, s, 0, 0, 0);
        if constexpr (kFar) {
          const uint4 w4 = __builtin_bit_cast(uint4, araw);
          const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 x2 = __builtin_bit_cast(bf16x2, wv[i]);
            kn = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, kn, false);
          }
        }
      }
      if constexpr (kFar) kn_max = fmaxf(kn_max, kn);

      // online softmax per slot over the row group (base 2).  Element 4j + r
      // is tile row 32 q + 16(j/2) + 8hh + 4(j%2) + r, at distance
      // t_newest - t0 - row >= 1 except in the tile holding the newest row or
      // the ragged tail, which take the exact per-row path.
      float tmax = -INFINITY;
      if (t0 + TR <= t_newest && nrows == TR) {
        const float dk = float(t_newest - t0 - 32 * q - 8 * hh);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = i >> 2, r = i & 3;
          const float bias = (dk - float(16 * (j >> 1) + 4 * (j & 1) + r)) * lnl2;
          const float a = fmaf(s[i], k2, bias);
          s[i] = a;
          tmax = fmaxf(tmax, a);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = i >> 2, r = i & 3;
          const int row = 32 * q + 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + r;
          const int dist = t_newest - (t0 + row);
          const float bias = dist == 0 ? 0.f : float(dist) * lnl2;
          float a = fmaf(s[i], k2, bias);
          if (row >= nrows) a = -INFINITY;
          s[i] = a;
          tmax = fmaxf(tmax, a);
        }
      }
      // the slot's max over the two lane halves (the other rows)
      {
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      // lazy rescale: the reference max moves only when some slot's max grows
      // by more than 8 e-folds (weights stay <= e^8), so the 128-register
      // accumulator rescale is skipped in the steady state
      m_true = fmaxf(m_true, tmax);
      if (__any(tmax > m_run + 8.f * kLog2e)) {
        const float m_new = fmaxf(m_run, tmax);
        const float scale = m_run == -INFINITY ? 0.f : exp2_f(m_run - m_new);
        m_run = m_new;
        l_run *= scale;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[db] *= scale;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      // weights rounded to bf16 in pairs; l sums the same rounded weights;
      // elements 8t..8t+7 are the P^T operand of k-step t
      const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
      bf16x8 pk[2];
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t pw[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x2 e2 = {exp2_f(s[8 * t + 2 * qq] - m_use), exp2_f(s[8 * t + 2 * qq + 1] - m_use)};
          const bf16x2 b2 = __builtin_convertvector(e2, bf16x2);
          pw[qq] = __builtin_bit_cast(uint32_t, b2);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(b2, ones, lsum, false);
        }
        pk[t] = as_bf16x8(__builtin_bit_cast(u16x8, uint4{pw[0], pw[1], pw[2], pw[3]}));
      }
      l_run += lsum;

      // n^T[dim][slot] += [K|V]^T[dim][row] P^T[row][slot], 16 rows per k-step.
      // A operand of dimension block db: lane l takes dimension 32db + l % 32
      // and rows 8(l/32) .. +7 of the k-step as two transposed 4-row reads
      // (offsets above): lane 4a + b of a 16-lane group receives element b of
      // the reads of lanes a, a+4, a+8, a+12, which cover 4 consecutive rows.
      typedef short i16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const uint16_t* tile = (db < 4 ? KL : VL) + 16 * t * RS + pv_blk[db & 3];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + pv_base[0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + pv_base[1]));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[t], acc[db], 0, 0, 0);
        }
    };
    if constexpr (kFar) {
      if (ntiles > 0) issue_tile(tile_t0(0), buf0);
      for (int idx = 0; idx < ntiles; idx += 2) {  // tile i in buffer i mod 2
        tile_step(idx, buf0, buf1);
        if (idx + 1 < ntiles) tile_step(idx + 1, buf1, buf0);
      }
    } else {
      if (ntiles > 0) issue_tile(tile_t0(0), buf0);
      if (ntiles > 1) issue_tile(tile_t0(1), buf1);
      for (int idx = 0; idx < ntiles; idx += 3) {  // tile i in buffer i mod 3
        tile_step(idx, buf0, buf2);
        if (idx + 1 < ntiles) tile_step(idx + 1, buf1, buf0);
        if (idx + 2 < ntiles) tile_step(idx + 2, buf2, buf1);
      }
    }

    float lt = l_run;  // the slot's weight sum over both lane halves
    {
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
      lt = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
    }
    __syncthreads();  // the last tile's LDS reads are done
    float* nrow = pb + 2 * S + int64_t(slot) * 2 * D;
    if constexpr (!kFar) {
      // merge the two row halves of each slot group: half 1 leaves (m_true,
      // m_run, l, n) in LDS, half 0 takes the exact max of both and rescales
      float* mg = reinterpret_cast<float*>(sgl == 0 ? buf0 : sgl == 1 ? buf1 : sgl == 2 ? buf2 : UL);
      if (q == 1) {
        float* dst = mg + lane * 131;
        dst[0] = m_true;
        dst[1] = m_run;
        dst[2] = lt;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) dst[3 + db * 16 + i] = acc[db][i];
      }
      __syncthreads();
      if (q == 1) return;
      const float* src = mg + lane * 131;
      const float mt = fmaxf(m_true, src[0]);  // the state's m: the exact max of all rows
      const float w0 = m_run == -INFINITY ? 0.f : exp2_f(m_run - mt);
      const float w1 = src[1] == -INFINITY ? 0.f : exp2_f(src[1] - mt);
      lt = fmaf(lt, w0, src[2] * w1);

      // write the partial: lane (slot, hh) holds n[slot][32db + 8j + 4hh + r];
      // each block is combined and stored in turn
      if (hh == 0) {
        pb[slot] = mt * kLn2;  // natural units, as the state keeps m
        pb[S + slot] = lt;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = fmaf(acc[db][4 * j + r], w0, src[3 + db * 16 + 4 * j + r] * w1);
          *reinterpret_cast<f32x4*>(nrow + db * 32 + 8 * j + 4 * hh) = o;
        }
    } else {
      // merge the four row quarters of each pooled group in two rounds
      // through records 0 and 1 of buffer sgl: quarters 2, 3 into 0, 1, then
      // quarter 1 into 0
      float* rec = reinterpret_cast<float*>(sgl == 0 ? buf0 : buf1) + lane * 131;
      auto put = [&](float* dst) __attribute__((always_inline)) {
        dst[0] = m_true;
        dst[1] = m_run;
        dst[2] = lt;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) dst[3 + db * 16 + i] = acc[db][i];
      };
      auto take = [&](const float* src) __attribute__((always_inline)) {
        const float mt = fmaxf(m_true, src[0]);
        const float w0 = m_run == -INFINITY ? 0.f : exp2_f(m_run - mt);
        const float w1 = src[1] == -INFINITY ? 0.f : exp2_f(src[1] - mt);
        lt = fmaf(lt, w0, src[2] * w1);
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] = fmaf(acc[db][i], w0, src[3 + db * 16 + i] * w1);
        m_true = mt;
        m_run = mt;
      };
      if (q >= 2) put(rec + (q - 2) * kRecFloats);
      __syncthreads();
      if (q < 2) take(rec + q * kRecFloats);
      __syncthreads();
      if (q == 1) put(rec);
      __syncthreads();
      if (q == 0) {
        take(rec);
        if (hh == 0) {
          pb[slot] = m_true * kLn2;
          pb[S + slot] = lt;
        }
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = acc[db][4 * j + r];
            *reinterpret_cast<f32x4*>(nrow + db * 32 + 8 * j + 4 * hh) = o;
          }
      }
      if constexpr (kRest) return;

      // the bound on the faster half (above): the largest key norm of the
      // split, bounded by the sum of the largest squared norms of the two
      // interleaved dimension halves (lane halves hh), and the newest row's
      float kb = kn_max;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) kb = fmaxf(kb, __shfl_xor(kb, o, 64));
      if (m32 == 0) s_red[2 * wave + hh] = kb;
      __syncthreads();
      if (wave == 0) {
        float k0 = 0.f, k1 = 0.f;
        for (int w = 0; w < NT / 64; ++w) {
          k0 = fmaxf(k0, s_red[2 * w]);
          k1 = fmaxf(k1, s_red[2 * w + 1]);
        }
        const uint32_t kt = *reinterpret_cast<const uint32_t*>(
            kp + ((int64_t(c) * rows_stride + t_newest) * Hkv + h) * D + 2 * lane);
        const bf16x2 kt2 = __builtin_bit_cast(bf16x2, kt);
        const float ktn = wave_sum(__builtin_amdgcn_fdot2_f32_bf16(kt2, kt2, 0.f, false));
        bool ok = true;
        if (lane < 32 * NA) {  // the faster half: ranks 0 .. 32 NA - 1
          const int j = s_order[lane];
          float un = 0.f;
          for (int e = 0; e < D; e += 8) {
            const uint4 x = *reinterpret_cast<const uint4*>(u + (int64_t(h) * S + j) * D + e);
            const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16x2 x2 = __builtin_bit_cast(bf16x2, xv[i]);
              un = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, un, false);
            }
          }
          // 1 + 2^-10 covers the rounding of the norms; NaN fails
          const float bound =
              sqrtf(un) * (sqrtf(k0 + k1) + sqrtf(ktn)) * (0.08838834764831845f * (1.f + 0x1p-10f)) + 48.f;
          const float decay = float(L0 - r_end) * -log_lambda[j];
          ok = decay >= bound;
        }
        const bool all_ok = __ballot(!ok) == 0;
        if (lane == 0) *flag = all_ok ? 0 : 1;
        if (all_ok && lane < 32 * NA) {
          const int j = s_order[lane];
          pb[j] = -INFINITY;  // an empty partial: the merge gives it weight 0
          pb[S + j] = 0.f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// generic partial kernel (f32 storage, small shapes): LDS tiles of 16 rows
// ---------------------------------------------------------------------------
template <typename Ty, int D>
__global__ __launch_bounds__(kThreads) void init_generic_partial(
    const typename Ty::T* __restrict__ kp, const typename Ty::T* __restrict__ vp,
    int64_t rows_stride, int L0, int rows_per_split, int nsplit,
    const typename Ty::T* __restrict__ u, const float* __restrict__ log_lambda, int Hkv, int S,
    float* __restrict__ part) {
  constexpr int TR = 16, RS = 2 * D + 1;
  extern __shared__ float smem[];
  float* kv = smem;               // [TR][RS]
  float* sc = kv + TR * RS;       // [S][TR]
  float* s_scale = sc + S * TR;   // [S]
  float* s_m = s_scale + S;       // [S]
  float* s_l = s_m + S;           // [S]

  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;
  const int h = unit % Hkv, c = unit / Hkv;
  const int tid = threadIdx.x;
  const int r_begin = split * rows_per_split;
  const int r_end = min(L0, r_begin + rows_per_split);
  const int t_newest = L0 - 1;
  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
  float* pb = part + part_off(split, gridDim.x / nsplit, unit, S, D);
  float* pn = pb + 2 * S;

  for (int j = tid; j < S; j += kThreads) { s_m[j] = -INFINITY; s_l[j] = 0.f; }
  for (int p = tid; p < S * 2 * D; p += kThreads) pn[p] = 0.f;

  for (int t0 = r_begin; t0 < r_end; t0 += TR) {
    const int nrows = min(TR, r_end - t0);
    __syncthreads();
    for (int idx = tid; idx < TR * 2 * D; idx += kThreads) {
      const int r = idx / (2 * D), e = idx % (2 * D);
      float x = 0.f;
      if (r < nrows) {
        const int64_t off = ((int64_t(c) * rows_stride + t0 + r) * Hkv + h) * D + (e % D);
        x = Ty::load(e < D ? kp : vp, off);
      }
      kv[r * RS + e] = x;
    }
    __syncthreads();
    for (int p = tid; p < S * TR; p += kThreads) {
      const int j = p / TR, r = p % TR;
      float a = -INFINITY;
      if (r < nrows) {
        const typename Ty::T* uj = u + (int64_t(h) * S + j) * D;
        float dot = 0.f;
        for (int e = 0; e < D; ++e) dot = fmaf(Ty::load(uj, e), kv[r * RS + e], dot);
        const int dist = t_newest - (t0 + r);
        const float lnl = log_lambda[j];
        a = dot * inv_sqrt_d + (dist == 0 ? 0.f : float(dist) * lnl);
      }
      sc[j * TR + r] = a;
    }
    __syncthreads();
    for (int j = tid; j < S; j += kThreads) {
      float tmax = -INFINITY;
      for (int r = 0; r < TR; ++r) tmax = fmaxf(tmax, sc[j * TR + r]);
      const float m_old = s_m[j];
      const float m_new = fmaxf(m_old, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float scale = m_old == -INFINITY ? 0.f : exp_f(m_old - m_use);
      float lsum = 0.f;
      for (int r = 0; r < TR; ++r) {
        const float pw = exp_f(sc[j * TR + r] - m_use);
        sc[j * TR + r] = pw;
        lsum += pw;
      }
      s_l[j] = fmaf(s_l[j], scale, lsum);
      s_m[j] = m_new;
      s_scale[j] = scale;
    }
    __syncthreads();
    for (int p = tid; p < S * 2 * D; p += kThreads) {
      const int j = p / (2 * D), e = p % (2 * D);
      float a = pn[p] * s_scale[j];
      for (int r = 0; r < nrows; ++r) a = fmaf(sc[j * TR + r], kv[r * RS + e], a);
      pn[p] = a;
    }
  }
  __syncthreads();
  for (int j = tid; j < S; j += kThreads) {
    pb[j] = s_m[j];
    pb[S + j] = s_l[j];
  }
}

// ---------------------------------------------------------------------------
// merge the partials, write state + slots, fill the ring
// ---------------------------------------------------------------------------
template <typename Ty, int D>
__global__ __launch_bounds__(kThreads) void init_finalize(
    const float* __restrict__ part, int nsplit, int units, int L0,
    const typename Ty::T* __restrict__ kp, const typename Ty::T* __restrict__ vp,
    int64_t rows_stride, int Hkv, int S, int W, int NT, float* __restrict__ sum_m,
    float* __restrict__ sum_l, float* __restrict__ sum_n, typename Ty::T* __restrict__ slot_k,
    typename Ty::T* __restrict__ slot_v, typename Ty::T* __restrict__ ring_k,
    typename Ty::T* __restrict__ ring_v, int32_t* __restrict__ ring_pos,
    int32_t* __restrict__ seq_len, int32_t* __restrict__ err_flag) {
  constexpr int SPB = 16;
  extern __shared__ float wsm[];  // [nsplit][SPB] merge weights
  __shared__ float s_inv_l[SPB];
  const int tile = blockIdx.x % NT;
  const int unit = blockIdx.x / NT;
  const int h = unit % Hkv, c = unit / Hkv;
  const int tid = threadIdx.x;
  const int j0 = tile * SPB;
  const int nj = min(SPB, S - j0);

  if (tid < nj) {
    const int j = j0 + tid;
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part[part_off(s, units, unit, S, D) + j]);
    float l = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* pb = part + part_off(s, units, unit, S, D);
      const float ms = pb[j];
      const float wgt = ms == -INFINITY ? 0.f : exp_f(ms - mx);
      wsm[s * SPB + tid] = wgt;
      l = fmaf(pb[S + j], wgt, l);
    }
    const int64_t si = int64_t(unit) * S + j;
    sum_m[si] = mx;
    sum_l[si] = l;
    s_inv_l[tid] = 1.0f / l;
  }
  __syncthreads();
  // 4 consecutive entries of one slot per thread, one 16-byte piece of the
  // stored numerators (both layouts keep entries 4q .. 4q+3 of a slot
  // together).  Tiled numerators: neighbouring threads take neighbouring
  // slots of one piece position, so the pieces they store are contiguous;
  // otherwise neighbouring threads take a slot's neighbouring pieces.
  const bool ntiled = n_tiled(Ty::kBytes, D, S);
  auto entries4 = [&](int jj, int e) {
    const int j = j0 + jj;
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float* pn = part + part_off(s, units, unit, S, D) + 2 * S + int64_t(j) * 2 * D + e;
      const float w = wsm[s * SPB + jj];  // (partials are only 4-byte aligned for odd S)
      if (w != 0.f) a += f32x4{pn[0], pn[1], pn[2], pn[3]} * w;  // an empty partial holds no n
    }
    *reinterpret_cast<f32x4*>(sum_n + n_index(ntiled, unit, S, D, j, e)) = a;
    const float il = s_inv_l[jj];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (e < D)
        Ty::store(slot_k, key_index(unit, S, D, j, e + r), a[r] * il);
      else  // values in key tiles of 32 (one tile of S keys when S % 32 != 0)
        Ty::store(slot_v,
                  S % 32 == 0 ? ((int64_t(unit) * (S >> 5) + (j >> 5)) * D + (e + r - D)) * 32 + (j & 31)
                              : (int64_t(unit) * D + (e + r - D)) * S + j,
                  a[r] * il);
    }
  };
  for (int p = tid; p < nj * (2 * D / 4); p += kThreads) {
    if (ntiled)  // p = ((t*4 + g)*2 + b)*nj + slot: entry 32t + 8g + 4b
      entries4(p % nj, (p / nj) * 4);
    else
      entries4(p / (2 * D / 4), (p % (2 * D / 4)) * 4);
  }

  // ring window: window slot ws holds the newest prefix position p with
  // p mod W == ws, if p >= max(0, L0 - W) (else it is empty: zeros, -1).
  // This workgroup fills the 32-slot key tiles kt = tile, tile + NT, ...:
  // every key and value piece of a tile is loaded first (several 16-byte
  // loads in flight per thread), each key piece goes straight to its place
  // in the key layout (key_index), values pass through LDS and leave as
  // 16-byte pieces of the tile [d][32].
  auto newest_of = [&](int ws) -> int {  // -1: empty slot
    const int back = ((L0 - 1 - ws) % W + W) % W;
    return max(L0 - 1 - back, -1);
  };
  if (W % 32 == 0) {
    using T = typename Ty::T;
    constexpr int E16 = 16 / Ty::kBytes, P16 = D / E16;  // 16-byte pieces per row
    constexpr int NP = 32 * P16;                         // pieces per tile (in and out)
    constexpr int NPT = (NP + kThreads - 1) / kThreads;  // pieces per thread per tile
    constexpr int VS = D + E16;                          // LDS row stride (elements)
    T* vls = reinterpret_cast<T*>(wsm + nsplit * SPB);   // [32][VS]
    for (int kt = tile; kt < W / 32; kt += NT) {
      uint4 kr[NPT], vr[NPT];
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const int pc = min(tid + q * kThreads, NP - 1), i = pc / P16, e = pc % P16;
        const int p = newest_of(kt * 32 + i);
        const int64_t src = ((int64_t(c) * rows_stride + max(p, 0)) * Hkv + h) * D;
        kr[q] = p >= 0 ? reinterpret_cast<const uint4*>(kp + src)[e] : uint4{0, 0, 0, 0};
        vr[q] = p >= 0 ? reinterpret_cast<const uint4*>(vp + src)[e] : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const int pc = tid + q * kThreads, i = pc / P16, e = pc % P16;
        if (pc >= NP) break;
        *reinterpret_cast<uint4*>(ring_k + key_index(unit, W, D, kt * 32 + i, e * E16)) = kr[q];
        reinterpret_cast<uint4*>(vls + i * VS)[e] = vr[q];
      }
      if (h == 0 && tid < 32) ring_pos[int64_t(c) * W + kt * 32 + tid] = newest_of(kt * 32 + tid);
      __syncthreads();
      // output piece (dim, kq): keys kq*E16 .. +E16-1 of one dimension
      T* tile_v = ring_v + (int64_t(unit) * (W / 32) + kt) * D * 32;
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const int pc = tid + q * kThreads, dim = pc / (32 / E16), kq = pc % (32 / E16);
        if (pc >= NP) break;
        T x[E16];
#pragma unroll
        for (int e = 0; e < E16; ++e) x[e] = vls[(kq * E16 + e) * VS + dim];
        reinterpret_cast<uint4*>(tile_v + dim * 32)[kq] = *reinterpret_cast<const uint4*>(x);
      }
      __syncthreads();
    }
  } else {  // W % 32 != 0 (small f32 windows): values in one tile [d][W]
    for (int wsl = tile; wsl < W; wsl += NT) {
      const int p = newest_of(wsl);
      const int64_t src = ((int64_t(c) * rows_stride + max(p, 0)) * Hkv + h) * D;
      for (int e = tid; e < D; e += kThreads) {
        ring_k[key_index(unit, W, D, wsl, e)] = p >= 0 ? kp[src + e] : typename Ty::T(0);
        ring_v[(int64_t(unit) * D + e) * W + wsl] = p >= 0 ? vp[src + e] : typename Ty::T(0);
      }
      if (h == 0 && tid == 0) ring_pos[int64_t(c) * W + wsl] = p;
    }
  }
  if (h == 0 && tile == 0 && tid == 0) seq_len[c] = L0;
  if (blockIdx.x == 0 && tid == 0) *err_flag = 0;
}

template <typename Ty, int D>
ls_status finalize(const ls_dims& d, const ls_state& st, const float* part, int nsplit,
                   const void* kp, const void* vp, int L0, int64_t rows_stride,
                   hipStream_t stream) {
  using T = typename Ty::T;
  // S/16 tiles of slots per unit; at least one workgroup per unit fills the
  // window, seq_len and err_flag when there is no summary (S = 0)
  const int NT = std::max(1, int(cdiv(d.S, 16)));
  const int units = d.C * d.Hkv;
  // merge weights [nsplit][16], then the value staging tile [32][d + 16 bytes]
  const size_t shmem = sizeof(float) * size_t(nsplit) * 16 + 32 * (D * sizeof(T) + 16);
  hipLaunchKernelGGL((init_finalize<Ty, D>), dim3(units * NT), dim3(kThreads), shmem, stream,
                     part, nsplit, units, L0, static_cast<const T*>(kp),
                     static_cast<const T*>(vp), rows_stride, d.Hkv, d.S, d.W, NT, st.sum_m,
                     st.sum_l, st.sum_n, static_cast<T*>(st.slot_k), static_cast<T*>(st.slot_v),
                     static_cast<T*>(st.ring_k), static_cast<T*>(st.ring_v), st.ring_pos,
                     st.seq_len, st.err_flag);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

template <int D>
ls_status run_f32(const ls_dims& d, const ls_state& st, const void* kp, const void* vp, int L0,
                  int64_t rows_stride, float* part, int rows, int nsplit, hipStream_t stream) {
  const size_t shmem = sizeof(float) * (16 * (2 * D + 1) + size_t(d.S) * 16 + 3 * size_t(d.S));
  if (d.S == 0) return finalize<F32, D>(d, st, part, nsplit, kp, vp, L0, rows_stride, stream);
  hipLaunchKernelGGL((init_generic_partial<F32, D>), dim3(d.C * d.Hkv * nsplit), dim3(kThreads),
                     shmem, stream, static_cast<const float*>(kp), static_cast<const float*>(vp),
                     rows_stride, L0, rows, nsplit, static_cast<const float*>(st.u),
                     st.log_lambda, d.Hkv, d.S, part);
  if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
  return finalize<F32, D>(d, st, part, nsplit, kp, vp, L0, rows_stride, stream);
}

}  // namespace

ls_status launch_init(const ls_dims& d, const ls_state& st, const void* kp, const void* vp,
                      int32_t L0, int64_t rows_stride, hipStream_t stream) {
  const WsLayout lay = ws_layout(d, L0);
  float* part = reinterpret_cast<float*>(static_cast<char*>(st.workspace) + lay.init_part);
  if (d.dtype == LS_BF16) {
    const InitPlan plan = init_plan(d, L0);
    if (plan.nsplit() > lay.isplit) return LS_ERR_SHAPE;  // the workspace bound must cover the plan
    const int units = d.C * d.Hkv;
    const uint16_t* k16 = static_cast<const uint16_t*>(kp);
    const uint16_t* v16 = static_cast<const uint16_t*>(vp);
    const uint16_t* u16 = static_cast<const uint16_t*>(st.u);
    // near splits 0 .. n_near - 1, then far splits n_near .. nsplit - 1: the
    // slower half of the slots, then the faster half where its bound failed
    int32_t* rest = reinterpret_cast<int32_t*>(static_cast<char*>(st.workspace) + lay.init_flag);
    auto run = [&](auto near, auto far, auto rest_k, int threads) {
      hipLaunchKernelGGL(near, dim3(units * plan.n_near), dim3(threads), 0, stream, k16, v16, rows_stride, L0,
                         plan, 0, plan.n_near, u16, st.log_lambda, d.Hkv, part, rest);
      if (plan.n_far > 0) {
        hipLaunchKernelGGL(far, dim3(units * plan.n_far), dim3(threads), 0, stream, k16, v16, rows_stride,
                           L0, plan, plan.n_near, plan.n_far, u16, st.log_lambda, d.Hkv, part, rest);
        hipLaunchKernelGGL(rest_k, dim3(units * plan.n_far), dim3(threads), 0, stream, k16, v16,
                           rows_stride, L0, plan, plan.n_near, plan.n_far, u16, st.log_lambda, d.Hkv,
                           part, rest);
      }
    };
    if (d.S == 128)
      run(init_mfma32_partial<4, 2>, init_mfma32_partial<4, 4>, init_mfma32_partial<4, 4, true>, 512);
    else if (d.S == 64)
      run(init_mfma32_partial<2, 2>, init_mfma32_partial<2, 4>, init_mfma32_partial<2, 4, true>, 256);
    // S = 0: no summary to pool; the finalize fills the window only
    if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    return finalize<BF16, 128>(d, st, part, plan.nsplit(), kp, vp, L0, rows_stride, stream);
  }
  const int rows = init_rows_per_split(d, L0);
  const int nsplit = int(cdiv(L0, rows));
  switch (d.d) {
    case 16: return run_f32<16>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 32: return run_f32<32>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 64: return run_f32<64>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 128: return run_f32<128>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
  }
  return LS_ERR_SHAPE;
}

}  // namespace ls
