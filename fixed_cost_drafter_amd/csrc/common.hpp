// Shared device helpers and the workspace layout of liblongspark.
//
// Element access for the two storage types (IEEE float32 and bfloat16 bit
// patterns), the MFMA operand vector types of gfx950, wave-level reductions
// for 64-lane wavefronts, and where each kernel keeps its scratch inside the
// caller's workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

#include "../../include/longspark.h"

namespace ls {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  __device__ static inline float load(const T* p, int64_t i) { return p[i]; }
  __device__ static inline void store(T* p, int64_t i, float x) { p[i] = x; }
};

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round to nearest, ties to even (inputs are finite)
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static inline float load(const T* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static inline void store(T* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// MFMA operand / accumulator vectors
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// wave (64 lanes) reductions
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline uint64_t shfl_xor_u64(uint64_t x, int o) {
  uint32_t lo = __shfl_xor(uint32_t(x), o, 64);
  uint32_t hi = __shfl_xor(uint32_t(x >> 32), o, 64);
  return (uint64_t(hi) << 32) | lo;
}

// e^(x) for the online softmax; e^(-inf) = 0
__device__ inline float exp_f(float x) { return __expf(x); }

// ---------------------------------------------------------------------------
// value layout of the window and of the slots: key tiles of 32,
// [unit][rows/32][d][32], so the 32 keys of a tile are contiguous for each
// dimension and a whole tile is one contiguous block; when rows is not a
// multiple of 32 the tile is the whole row range ([unit][d][rows]).
// ---------------------------------------------------------------------------
__host__ __device__ inline int value_tile(int rows) { return rows % 32 == 0 ? 32 : rows; }
__host__ __device__ inline int64_t value_index(int64_t unit, int rows, int d, int key, int dim) {
  const int tw = value_tile(rows);
  return ((unit * (rows / tw) + key / tw) * d + dim) * tw + key % tw;
}

// ---------------------------------------------------------------------------
// key layout of the window and of the slots.  With d = 128 and rows a
// multiple of 32, each tile of 32 keys is stored in the order in which the
// drafter's MFMA reads its A operand (S^T = K Q^T with 16x16x32 products),
// so that every 64-lane operand load is 1 KB contiguous:
//   key k = 8a + 4b + r (a < 4, b < 2, r < 4), dimension e = 32s + 8g + i
//   -> element ((((b*4 + s)*4 + g)*16 + 4a + r)*8 + i of the tile.
// The 8 dimensions 8g' .. 8g'+7 of one key stay contiguous (16 bytes in
// bf16).  Other shapes keep keys row-major, [unit][rows][d].
// ---------------------------------------------------------------------------
__host__ __device__ inline bool key_tiled(int rows, int d) { return d == 128 && rows % 32 == 0; }
__host__ __device__ inline int64_t key_index(int64_t unit, int rows, int d, int key, int dim) {
  if (!key_tiled(rows, d)) return (unit * rows + key) * d + dim;
  const int k = key & 31;
  const int piece = ((((k >> 2) & 1) * 4 + (dim >> 5)) * 4 + ((dim >> 3) & 3)) * 16 + 4 * (k >> 3) + (k & 3);
  return (unit * rows + (key & ~31)) * d + piece * 8 + (dim & 7);
}

// ---------------------------------------------------------------------------
// layout of the fp32 summary numerators n ([unit][S][2d] entries: keys |
// values).  bf16 states at d = 128 (S a multiple of 32) keep each 32-slot
// tile in the order of the summary update's MFMA accumulators, so that each
// 64-lane 16-byte load or store of the state is 1 KB contiguous: entry
// e = 32 t + 8 g + 4 b + r (t < 8, g < 4, b < 2, r < 4) of slot 32 T + s goes
// to float ((t*4 + g)*64 + 32b + s)*4 + r of tile T.  Other states keep
// [unit][S][2d].
// ---------------------------------------------------------------------------
__host__ __device__ inline bool n_tiled(int dtype_bytes, int d, int S) {
  return dtype_bytes == 2 && d == 128 && S % 32 == 0;
}
__host__ __device__ inline int64_t n_index(bool tiled, int64_t unit, int S, int d, int slot, int e) {
  if (!tiled) return (unit * S + slot) * 2 * d + e;
  const int lane = (slot & 31) + 32 * ((e >> 2) & 1);
  return (unit * S + (slot & ~31)) * 2 * d + ((((e >> 5) * 4 + ((e >> 3) & 3)) * 64 + lane) << 2) + (e & 3);
}

// ---------------------------------------------------------------------------
// workspace layout (bytes), shared by the host code and the kernels
// ---------------------------------------------------------------------------
#ifndef LS_VERIFY_CHUNK
#define LS_VERIFY_CHUNK 8192
#endif
constexpr int kVerifyChunk = LS_VERIFY_CHUNK;  // logits per verify workgroup
// Largest drafted block: B + 1 verified rows fit one 64-lane ballot, the
// block's keys fill at most two 32-key chunks of the draft attention, and the
// append's staging of B + 1 fp32 rows of [k | v] (d = 128) stays under 64 KB
// of LDS.
constexpr int kMaxBlock = 47;
#ifndef LS_INIT_TARGET_BLOCKS
#define LS_INIT_TARGET_BLOCKS 512
#endif
constexpr int kInitTargetBlocks = LS_INIT_TARGET_BLOCKS; // aim of the init grid size
constexpr int kInitRowTile = 64;       // rows per init tile (MFMA path)
// bf16 init, d = 128, S in {64, 128}: rows at least this far from the newest
// go to "far" workgroups that pool them into the slower-decaying half of the
// slots only (the other half's weights there are checked to be negligible),
// in about kInitFarBlocks workgroups (one per CU: a second, partial round
// costs more than longer workgroups), once the prefix holds at least twice
// the near rows.  Measured on MI355X at C = 16, Hkv = 8 against near splits
// only: the init 4% faster at a 32K prefix, 20% at 64K, 27% at 128K.
#ifndef LS_INIT_NEAR_ROWS
#define LS_INIT_NEAR_ROWS 12288
#endif
#ifndef LS_INIT_FAR_BLOCKS
#define LS_INIT_FAR_BLOCKS 256
#endif
#ifndef LS_INIT_NEAR_BLOCKS
#define LS_INIT_NEAR_BLOCKS 256
#endif
#ifndef LS_INIT_FAR_MIN
#define LS_INIT_FAR_MIN (2 * LS_INIT_NEAR_ROWS)
#endif
constexpr int64_t kInitNearRows = LS_INIT_NEAR_ROWS;
constexpr int64_t kInitFarBlocks = LS_INIT_FAR_BLOCKS;
constexpr int64_t kInitNearBlocks = LS_INIT_NEAR_BLOCKS;  // near workgroups when there are far ones
constexpr int64_t kInitFarMin = LS_INIT_FAR_MIN;          // shortest prefix with far splits

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// arrival counters per sequence: one per (KV head, 32-slot tile)
inline int arrivals_per_seq(const ls_dims& d) { return d.Hkv * int(cdiv(d.S < 1 ? 1 : d.S, 32)); }

struct WsLayout {
  int64_t draft_part;                         // float [C*Hkv*halves * Mpad*(d+2)]
  int64_t verify_part;                        // uint64 keys [C*(B+1)*vsplit]
  int64_t init_part;                          // float [isplit*C*Hkv*S*(2d+2)]
  int64_t init_flag;                          // int32 [isplit*C*Hkv]: far splits whose faster slots are left
  int64_t attn_part;                          // float [C*Hkv*asplit * Mq*(d+2)]
  int64_t samp_stats;                         // float2 (max, sum) [C*(2B+1)*vsplit]
  int64_t samp_seq;                           // per-sequence decision record [C*8] (4-byte words)
  int64_t samp_sums;                          // float [C*vsplit] chunk sums of the drawn row
  int64_t len_snap;                           // int32 [C] lengths before an update
  int64_t arrivals;                           // int32 [C*Hkv*tiles] waves of a (unit, slot tile) past their state reads
  int64_t total;
  int vsplit, isplit, init_rows, asplit;
};

// target verification attention: (B+1)*G query rows per KV head, padded to
// row groups of 16, over up to max_rows context rows cut into `splits`
// ranges of whole 64-row tiles (about kInitTargetBlocks workgroups in all)
inline int attn_query_rows(const ls_dims& d) {
  return int(cdiv(int64_t(d.B + 1) * (d.Hq / d.Hkv), 16) * 16);
}
inline int attn_splits(const ls_dims& d, int64_t max_rows) {
  const int64_t want = cdiv(kInitTargetBlocks, int64_t(d.C) * d.Hkv);
  const int64_t by_rows = cdiv(max_rows < 1 ? 1 : max_rows, kInitRowTile);
  return int(want < by_rows ? want : by_rows);
}
inline int attn_rows_per_split(const ls_dims& d, int64_t max_rows) {
  return int(cdiv(cdiv(max_rows < 1 ? 1 : max_rows, attn_splits(d, max_rows)), kInitRowTile) *
             kInitRowTile);
}

inline int verify_splits(const ls_dims& d) { return int(cdiv(d.V, kVerifyChunk)); }

inline int init_rows_per_split(const ls_dims& d, int32_t L0) {
  // split each (sequence, head) prefix so the grid has ~kInitTargetBlocks blocks
  int64_t units = int64_t(d.C) * d.Hkv;
  int64_t want = cdiv(kInitTargetBlocks, units);
  int64_t rows = cdiv(L0, want);
  rows = cdiv(rows, kInitRowTile) * kInitRowTile;
  if (rows < kInitRowTile) rows = kInitRowTile;
  return int(rows);
}

// How the bf16 init cuts each (sequence, KV head) prefix, counted back from
// the newest row: split s < n_near covers rows [L0 - (s+1) near_rows,
// L0 - s near_rows) (clipped at 0) for every slot; far split f covers the
// next far_rows rows each, older still, for the slower half of the slots.
struct InitPlan {
  int near_rows, n_near, far_rows, n_far;
  int nsplit() const { return n_near + n_far; }
};
inline bool init_has_far(const ls_dims& d) {
  return d.dtype == LS_BF16 && d.d == 128 && (d.S == 64 || d.S == 128);
}
inline InitPlan init_plan(const ls_dims& d, int32_t L0) {
  const int64_t units = int64_t(d.C) * d.Hkv;
  const int64_t want = cdiv(kInitTargetBlocks, units);
  const int64_t L = L0 < 1 ? 1 : L0;
  auto round_up = [](int64_t x, int64_t m) { return cdiv(x, m) * m; };
  if (init_has_far(d) && L >= kInitFarMin) {
    // the near rows in about kInitNearBlocks workgroups
    const int64_t R = round_up(cdiv(kInitNearRows, cdiv(kInitNearBlocks, units)), kInitRowTile);
    const int64_t n_near = cdiv(kInitNearRows, R);
    const int64_t far = L - n_near * R;
    if (far > 0) {
      // n_far <= cdiv(kInitFarBlocks, units); a far split pools half the
      // slots, so it takes at least twice a near split's rows
      const int64_t FR = std::max(round_up(cdiv(far, cdiv(kInitFarBlocks, units)), 2 * kInitRowTile),
                                  round_up(2 * R, 2 * kInitRowTile));
      return InitPlan{int(R), int(n_near), int(FR), int(cdiv(far, FR))};
    }
  }
  const int64_t R = std::max(round_up(cdiv(L, want), kInitRowTile), int64_t(kInitRowTile));
  return InitPlan{int(R), int(cdiv(L, R)), 0, 0};
}
// rows [*r_begin, *r_end) of split `split` (0 = the newest rows) of a plan
__host__ __device__ inline void init_split_rows(const InitPlan& p, int L0, int split, int* r_begin,
                                                int* r_end) {
  int e, n;
  if (split < p.n_near) {
    e = L0 - split * p.near_rows;
    n = p.near_rows;
  } else {
    e = L0 - p.n_near * p.near_rows - (split - p.n_near) * p.far_rows;
    n = p.far_rows;
  }
  *r_end = e;
  *r_begin = e - n > 0 ? e - n : 0;
}
// an upper bound of init_plan(d, L0).nsplit() over 1 <= L0 <= max_L0
inline int init_split_bound(const ls_dims& d, int32_t max_L0) {
  const int64_t units = int64_t(d.C) * d.Hkv;
  const int64_t L = max_L0 < 1 ? 1 : max_L0;
  const int64_t want = cdiv(kInitTargetBlocks, units), by_rows = cdiv(L, kInitRowTile);
  int64_t n = want < by_rows ? want : by_rows;
  if (init_has_far(d) && L >= kInitFarMin) {
    const int64_t far_plan = cdiv(kInitNearBlocks, units) + cdiv(kInitFarBlocks, units);
    n = n > far_plan ? n : far_plan;
  }
  return int(n);
}

// bf16 draft attention: one workgroup per (KV head, 32 query rows, key
// range).  The key range is the whole key list unless the (KV head, rows)
// pairs alone leave the chip idle; then the keys are cut into up to 4
// ranges whose (m, l, O) partials a second launch merges.
inline int draft_row_splits(const ls_dims& d) { return int(cdiv(int64_t(d.B) * (d.Hq / d.Hkv), 32)); }
inline int draft_halves(const ls_dims& d) {
  if (d.dtype != LS_BF16) return 1;
  const int64_t chunks = (int64_t(d.W) + d.S) / 32 + cdiv(d.B, 32);
  const int64_t blocks = int64_t(d.C) * d.Hkv * draft_row_splits(d);
  int k = 1;
  while (k < 4 && blocks * k * 2 <= 256 && chunks >= 8 * k * 2) k *= 2;
  return k;
}

inline WsLayout ws_layout(const ls_dims& d, int32_t max_L0) {
  WsLayout w{};
  int64_t off = 0;
  {
    const int64_t Mpad = 64;  // draft partials hold 4 row groups of 16
    w.draft_part = off;
    const int halves = draft_halves(d);
    if (halves > 1) off = align256(off + 4 * int64_t(d.C) * d.Hkv * halves * Mpad * (d.d + 2));
  }
  w.vsplit = verify_splits(d);
  w.verify_part = off; off = align256(off + 8 * int64_t(d.C) * (d.B + 1) * w.vsplit);
  // the split count of a call with L0 <= max_L0 never exceeds this bound
  const int64_t L = max_L0 < 1 ? 1 : max_L0;
  w.init_rows = init_rows_per_split(d, int32_t(L));
  w.isplit = init_split_bound(d, int32_t(L));
  w.init_part = off;
  off = align256(off + 4 * int64_t(w.isplit) * d.C * d.Hkv * d.S * (2 * d.d + 2));
  w.init_flag = off;
  off = align256(off + 4 * int64_t(w.isplit) * d.C * d.Hkv);
  // verification attention over up to max_L0 + B + 1 rows
  w.asplit = attn_splits(d, L + d.B + 1);
  w.attn_part = off;
  off = align256(off + 4 * int64_t(w.asplit) * d.C * d.Hkv * attn_query_rows(d) * (d.d + 2));
  // sampled verification: softmax statistics of the C*(2B+1) rows, a record
  // per sequence, and the chunk sums of the row its token is drawn from
  w.samp_stats = off; off = align256(off + 8 * int64_t(d.C) * (2 * d.B + 1) * w.vsplit);
  w.samp_seq = off; off = align256(off + 32 * int64_t(d.C));
  w.samp_sums = off; off = align256(off + 4 * int64_t(d.C) * w.vsplit);
  w.len_snap = off; off = align256(off + 4 * int64_t(d.C));
  w.arrivals = off; off = align256(off + 4 * int64_t(d.C) * arrivals_per_seq(d));
  w.total = off;
  return w;
}

}  // namespace ls
