// Per-round update of the drafter's fixed-size context (LongSpark paper page,
// Fig. 2 (b): recent KV window + global context summary; Fig. 3: the summary
// is updated with only the newly retained rows N, |N| <= B+1).
//
// For sequence c with L retained rows and tau = tau[c] new rows (read on the
// device, so verification and update chain without a host round trip):
//   ring slot (L+i) mod W <- row i, ring_pos <- L+i        (i < tau)
//   per slot j: relative to the new newest row t' = L+tau-1 every old
//   a_jp grows by tau*ln(lambda_j), so m' = m + tau*ln(lambda_j) and l, n
//   keep their values; the new rows a_ji = u_j.k_i/sqrt(d) + (tau-1-i) ln
//   lambda_j are merged by the online-softmax rule; slot = n / l.
//   seq_len[c] += tau.
//
// bf16 (d = 128, S = 0, 64 or 128): append_units below, one workgroup per
// (sequence, KV head, 32-slot tile); the summary merge on MFMA; the window
// copy shared out among a unit's workgroups.  The length L before the update
// comes from a snapshot taken by the launch before (the verification's key
// pass in ls_verify_append, a one-line kernel in ls_append_accepted), so no
// workgroup reads the seq_len that one of them advances: no device-scope
// fence, no second kernel after the update.
//
// f32: C window workgroups (one per sequence: the only reader and writer of
// seq_len in the launch, after a barrier), then the summary workgroups,
// append_kernel: one workgroup per (sequence, KV head, 32 slots), LPS
// lanes per slot (32; at most d).  Lane g of a slot owns 2d/LPS consecutive
// entries of the slot's [k | v] numerator n (the first half of the lanes the
// key half, the rest the value half) and keeps them in registers from the
// first load to the last store, so the fp32 state crosses HBM once each way.
// All B+1 verified rows of the (sequence, KV head) are staged once in LDS as
// fp32, whatever tau is, so no load waits for tau.  The tau new rows are
// merged two at a time: the key lanes form partial dot products with the
// slot query, a DPP butterfly over the slot's lanes completes the scores,
// and one rescale per batch folds them into (m, l, n).  The slots n / l
// leave as pooled keys (each lane's entries at their place in the key
// layout) and pooled values; the values of the workgroup's 32 slots are one
// key tile ([d][32]) of the value layout the drafter reads, assembled in LDS
// and stored contiguously.
#include <algorithm>

#include "accept.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "merge_ops.hpp"

namespace ls {
namespace {

#ifndef LS_APPEND_LPS
#define LS_APPEND_LPS 32
#endif
#ifndef LS_APPEND_BATCH
#define LS_APPEND_BATCH 2
#endif
constexpr int kSlotsPerBlock = 32;     // one value key tile
constexpr int kBatch = LS_APPEND_BATCH;  // new rows merged per rescale

// lanes per slot: the 2d entries of a slot's [k | v] numerator over LPS lanes,
// EPL = 2d / LPS entries each (2 at least, so every access is 8 bytes or more)
template <int D>
constexpr int lanes_per_slot() { return D >= LS_APPEND_LPS ? LS_APPEND_LPS : D; }
// one lane group per slot of the tile
template <int D>
constexpr int block_threads() { return kSlotsPerBlock * lanes_per_slot<D>(); }

// EPL consecutive elements starting at p (EPL * element size is a multiple
// of 8 bytes and p is aligned to it) -> fp32
template <typename Ty, int EPL>
__device__ __forceinline__ void load_elems(const typename Ty::T* p, float (&out)[EPL]) {
  if constexpr (Ty::kBytes == 2) {
    static_assert(EPL % 8 == 0, "bf16 lanes hold whole 16-byte pieces");
#pragma unroll
    for (int q = 0; q < EPL / 8; ++q) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[q];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[q * 8 + 2 * e] = __uint_as_float(ws[e] << 16);
        out[q * 8 + 2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
      }
    }
  } else if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < EPL / 4; ++q) {
      const float4 w = reinterpret_cast<const float4*>(p)[q];
      out[4 * q] = w.x; out[4 * q + 1] = w.y; out[4 * q + 2] = w.z; out[4 * q + 3] = w.w;
    }
  } else {
    static_assert(EPL == 2, "f32 lanes hold 2, 4, 8 or 16 elements");
    const float2 w = *reinterpret_cast<const float2*>(p);
    out[0] = w.x; out[1] = w.y;
  }
}

template <typename Ty, int EPL>
__device__ __forceinline__ void store_elems(typename Ty::T* p, const float (&v)[EPL], float s) {
  if constexpr (Ty::kBytes == 2) {
#pragma unroll
    for (int q = 0; q < EPL / 8; ++q) {
      uint32_t ws[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ws[e] = uint32_t(f32_to_bf16(v[q * 8 + 2 * e] * s)) |
                (uint32_t(f32_to_bf16(v[q * 8 + 2 * e + 1] * s)) << 16);
      reinterpret_cast<uint4*>(p)[q] = uint4{ws[0], ws[1], ws[2], ws[3]};
    }
  } else if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < EPL / 4; ++q)
      reinterpret_cast<float4*>(p)[q] =
          float4{v[4 * q] * s, v[4 * q + 1] * s, v[4 * q + 2] * s, v[4 * q + 3] * s};
  } else {
    *reinterpret_cast<float2*>(p) = float2{v[0] * s, v[1] * s};
  }
}

// EPL consecutive elements of one row as loaded (bf16 stays packed until use)
template <typename Ty, int EPL>
struct Frag {
  float v[EPL];
  __device__ __forceinline__ void load(const typename Ty::T* p) { load_elems<Ty, EPL>(p, v); }
  __device__ __forceinline__ float operator[](int e) const { return v[e]; }
  __device__ __forceinline__ float dot(const Frag& o, float acc) const {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf(v[e], o.v[e], acc);
    return acc;
  }
};
template <int EPL>
struct Frag<BF16, EPL> {
  uint32_t w[EPL / 2];
  __device__ __forceinline__ void load(const uint16_t* p) {
#pragma unroll
    for (int q = 0; q < EPL / 8; ++q) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[q];
      w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
    }
  }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
  }
  // packed bf16 pairs straight into the fp32 dot product (v_dot2_f32_bf16),
  // so the rows need not stay unpacked in registers
  __device__ __forceinline__ float dot(const Frag& o, float acc) const {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int q = 0; q < EPL / 2; ++q)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[q]),
                                            __builtin_bit_cast(bf16x2, o.w[q]), acc, false);
    return acc;
  }
};

// fp32 state entries: EPL consecutive floats, aligned to 8 * EPL bytes at most 16
template <int EPL>
__device__ __forceinline__ void load_state(const float* p, float (&out)[EPL]) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < EPL / 4; ++q) {
      const float4 w = reinterpret_cast<const float4*>(p)[q];
      out[4 * q] = w.x; out[4 * q + 1] = w.y; out[4 * q + 2] = w.z; out[4 * q + 3] = w.w;
    }
  } else {
    const float2 w = *reinterpret_cast<const float2*>(p);
    out[0] = w.x; out[1] = w.y;
  }
}

template <int EPL>
__device__ __forceinline__ void store_state(float* p, const float (&v)[EPL]) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < EPL / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  } else {
    *reinterpret_cast<float2*>(p) = float2{v[0], v[1]};
  }
}

// x + (x taken from another lane of the same 16-lane DPP row)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the LPS (16 or 32) lanes of a slot group, left in every lane of it:
// within a 16-lane row by DPP (quad swaps, then rotations by 4 and 8), across
// the two rows of a 32-lane group by one lane shuffle
template <int LPS>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPS == 16 || LPS == 32, "slot groups are one or two DPP rows");
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x124>(x);  // row_ror:4
  x = dpp_add<0x128>(x);  // row_ror:8
  if constexpr (LPS == 32) x += __shfl_xor(x, 16);
  return x;
}

// The window part of one sequence: rows 0..tau-1 of the verified block go to
// window slots (L + i) mod W of every KV head, their positions to ring_pos,
// and seq_len advances by tau.  One workgroup per sequence does all of it, so
// it is the only reader of seq_len in the launch and may update it in place.
// Thread t takes row i = t mod (B+1) and the (head, 16-byte piece) pairs
// t / (B+1), + G, + 2G, ... (G = threads / (B+1)): it copies the key piece to
// its place in the key layout and scatters the value piece's elements into
// the value layout, where lanes of neighbouring rows land in neighbouring
// window slots of one dimension's tile row.  Every row of the block is
// loaded, so the loads wait neither for tau nor for seq_len; only rows
// i < tau are stored.  kWindowUnroll pieces' loads are in flight before their
// stores.  Tn: tau, already clamped into [1, B+1] (its value is needed only
// by the stores).
template <typename Ty, int D, int kThreads, int kWindowUnroll>
__device__ __forceinline__ void append_window(
    const typename Ty::T* __restrict__ k_new, const typename Ty::T* __restrict__ v_new, int Tn,
    typename Ty::T* __restrict__ ring_k, typename Ty::T* __restrict__ ring_v,
    int32_t* __restrict__ ring_pos, int32_t* __restrict__ seq_len, int c, int Hkv, int W, int B) {
  using T = typename Ty::T;
  constexpr int E16 = 16 / Ty::kBytes;      // elements per 16-byte piece
  constexpr int V16 = D / E16;              // 16-byte pieces per key row
  static_assert(kThreads > 48, "every row of the block gets a thread");
  const int tid = threadIdx.x;
  const int B1 = B + 1;
  if (W == 0) {  // no window view: only the count advances (one thread reads and writes it)
    if (tid == 0) seq_len[c] += Tn;
    return;
  }
  const int L = seq_len[c];
  const int G = kThreads / B1, i = tid % B1, g = tid / B1;
  const int pairs = Hkv * V16;
  const int64_t src0 = (int64_t(c) * B1 + i) * Hkv * D;
  const int64_t hstride = int64_t(W) * D;
  const int kstep = key_tiled(W, D) ? 16 * 8 : E16;  // tiled keys: 16 pieces apart
  const int tw = value_tile(W);
  // pass hp0: pairs hp0, hp0 + G, ... (kWindowUnroll of them) of this row
  auto load_pass = [&](int hp0, uint4 (&kv)[kWindowUnroll], uint4 (&vv)[kWindowUnroll]) {
#pragma unroll
    for (int u = 0; u < kWindowUnroll; ++u) {
      const int hp = min(hp0 + u * G, pairs - 1);  // past the end: repeat the last pair
      const int64_t src = src0 + (hp / V16) * D + (hp % V16) * E16;
      kv[u] = *reinterpret_cast<const uint4*>(k_new + src);
      vv[u] = *reinterpret_cast<const uint4*>(v_new + src);
    }
  };
  auto store_pass = [&](int hp0, const uint4 (&kv)[kWindowUnroll], const uint4 (&vv)[kWindowUnroll],
                        int64_t kb0, int64_t vb0) {
#pragma unroll
    for (int u = 0; u < kWindowUnroll; ++u) {
      const int hp = hp0 + u * G;
      if (hp < pairs) {
        const int e = hp % V16;
        const int64_t ho = (hp / V16) * hstride;
        *reinterpret_cast<uint4*>(ring_k + kb0 + ho + e * kstep) = kv[u];
        T* vd = ring_v + vb0 + ho + int64_t(e * E16) * tw;
        const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
        for (int q = 0; q < E16; ++q) {
          if constexpr (Ty::kBytes == 2)
            vd[q * tw] = T(w[q >> 1] >> (16 * (q & 1)));
          else
            vd[q * tw] = __uint_as_float(w[q]);
        }
      }
    }
  };
  if (g < G) {
    // offsets of this thread's row: head hl and piece e add hl W d and e
    // kstep (keys) or (e E16 + q) tw (value element q)
    const int slot = (L + i) % W;
    const int64_t kb0 = key_index(int64_t(c) * Hkv, W, D, slot, 0);
    const int64_t vb0 = value_index(int64_t(c) * Hkv, W, D, slot, 0);
    for (int hp0 = g; hp0 < pairs; hp0 += G * kWindowUnroll) {
      uint4 kv[kWindowUnroll], vv[kWindowUnroll];
      load_pass(hp0, kv, vv);
      if (i < Tn) store_pass(hp0, kv, vv, kb0, vb0);
    }
  }
  if (tid < Tn) ring_pos[int64_t(c) * W + (L + tid) % W] = L + tid;
  // every thread has read the old length (and used it for its stores) before
  // it is replaced
  __syncthreads();
  if (tid == 0) seq_len[c] = L + Tn;
}

// tau of sequence c read from device memory, clamped into [1, B+1]; a value
// outside sets bit 0 of *err_flag (when flag is set: the window workgroup)
__device__ __forceinline__ int read_tau(const int32_t* __restrict__ tau_in, int c, int B,
                                        int32_t* __restrict__ err_flag, bool flag) {
  const int B1 = B + 1;
  int Tn = tau_in[c];
  if (Tn < 1 || Tn > B1) {
    if (flag && threadIdx.x == 0) atomicOr(err_flag, 1);
    Tn = Tn < 1 ? 1 : B1;
  }
  return Tn;
}

template <typename Ty, int D>
__global__ __launch_bounds__(block_threads<D>()) void append_kernel(
    const typename Ty::T* __restrict__ k_new, const typename Ty::T* __restrict__ v_new,
    const int32_t* __restrict__ tau_in, typename Ty::T* __restrict__ ring_k,
    typename Ty::T* __restrict__ ring_v, int32_t* __restrict__ ring_pos,
    int32_t* __restrict__ seq_len, float* __restrict__ sum_m, float* __restrict__ sum_l,
    float* __restrict__ sum_n, typename Ty::T* __restrict__ slot_k,
    typename Ty::T* __restrict__ slot_v, const typename Ty::T* __restrict__ u,
    const float* __restrict__ log_lambda, int32_t* __restrict__ err_flag, int C, int Hkv, int W,
    int S, int B) {
  using T = typename Ty::T;
  extern __shared__ float4 smem4[];
  T* lds = reinterpret_cast<T*>(smem4);
  if (int(blockIdx.x) < C) {
    const int c = int(blockIdx.x);
    append_window<Ty, D, block_threads<D>(), 4>(k_new, v_new, read_tau(tau_in, c, B, err_flag, true),
                                                 ring_k, ring_v, ring_pos, seq_len, c, Hkv, W, B);
    return;
  }
  constexpr int LPS = lanes_per_slot<D>();
  constexpr int EPL = 2 * D / LPS;       // n entries per lane
  constexpr int HALF = LPS / 2;          // lanes of the key half
  const int tid = threadIdx.x;
  const int g = tid % LPS;               // entry group: g < HALF key half, else value half
  const int js = tid / LPS;              // slot within the tile
  const int ntile = (S + kSlotsPerBlock - 1) / kSlotsPerBlock;
  const int bid = int(blockIdx.x) - C;
  const int tile = bid % ntile;
  constexpr int kThreads = block_threads<D>();
  const int unit = bid / ntile;          // c * Hkv + h
  const int c = unit / Hkv, h = unit % Hkv;
  const int j = tile * kSlotsPerBlock + js;
  const bool active = j < S;
  const int jc = active ? j : S - 1;     // idle lanes (S % 32 != 0) load in bounds
  const int64_t sidx = int64_t(unit) * S + jc;
  const bool key_lane = g < HALF;
  const int col = (key_lane ? g : g - HALF) * EPL;  // first dimension of this lane's entries

  // Issue the state and slot-query loads, then stage all B+1 verified rows
  // of this (c, h) ([k | v] per row) in LDS with 16-byte pieces.  Rows past
  // tau exist in the buffer, so nothing here waits for tau, and the merge
  // below reads rows from LDS whatever the number of batches.
  const int B1 = B + 1;
  // [B+1][2d] fp32 after the value tile (16-byte aligned: the tile is d*32 elements)
  float* rows = reinterpret_cast<float*>(lds + D * kSlotsPerBlock);
  float n[EPL], uq[EPL];
  load_state<EPL>(sum_n + sidx * 2 * D + g * EPL, n);
  const float m_old = sum_m[sidx], l_old = sum_l[sidx], lnl = log_lambda[jc];
  load_elems<Ty, EPL>(u + (int64_t(h) * S + jc) * D + col, uq);
  {
    // rows are widened to fp32 once here, so the merge reads them ready to use
    constexpr int E16 = 16 / Ty::kBytes, V16 = D / E16;
    for (int p = tid; p < B1 * 2 * V16; p += kThreads) {
      const int e = p % V16, half = (p / V16) & 1, i = p / (2 * V16);
      float x[E16];
      load_elems<Ty, E16>((half ? v_new : k_new) + ((int64_t(c) * B1 + i) * Hkv + h) * D + e * E16, x);
      float4* dst = reinterpret_cast<float4*>(rows + i * 2 * D + half * D + e * E16);
#pragma unroll
      for (int q = 0; q < E16 / 4; ++q) dst[q] = float4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
    }
  }
  int Tn = tau_in[c];
  Tn = Tn < 1 ? 1 : (Tn > B1 ? B1 : Tn);
  __syncthreads();

  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
  // every old score grows by tau*ln(lambda); lambda = 0 drops the old state
  float m_run = (lnl == -INFINITY) ? -INFINITY : fmaf(float(Tn), lnl, m_old);
  float l_run = l_old;
  for (int i0 = 0; i0 < Tn; i0 += kBatch) {
    float r[kBatch][EPL], a[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) load_state<EPL>(rows + min(i0 + q, Tn - 1) * 2 * D + g * EPL, r[q]);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      // every lane forms the product (no branch); only the key half counts
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(uq[e], r[q][e], part);
      const float dot = group_sum<LPS>(key_lane ? part : 0.f);
      const int i = i0 + q, dist = Tn - 1 - i;
      const float bias = dist == 0 ? 0.f : float(dist) * lnl;
      a[q] = i < Tn ? dot * inv_sqrt_d + bias : -INFINITY;
    }
    float mb = m_run;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) mb = fmaxf(mb, a[q]);
    const float sc = (m_run == -INFINITY) ? 0.f : exp_f(m_run - mb);
    float wq[kBatch], lsum = 0.f;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      wq[q] = (a[q] == -INFINITY) ? 0.f : exp_f(a[q] - mb);
      lsum += wq[q];
    }
    l_run = fmaf(l_run, sc, lsum);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = n[e] * sc;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) x = fmaf(wq[q], r[q][e], x);
      n[e] = x;
    }
    m_run = mb;
  }

  const float il = 1.0f / l_run;
  if (active) {
    store_state<EPL>(sum_n + sidx * 2 * D + g * EPL, n);
    if (g == 0) {
      sum_m[sidx] = m_run;
      sum_l[sidx] = l_run;
    }
    // a lane's EPL key entries stay inside one group of 8 dimensions, which
    // the key layout keeps contiguous
    static_assert(D != 128 || EPL <= 8, "one key group of 8 dimensions per lane");
    if (key_lane) store_elems<Ty, EPL>(slot_k + key_index(unit, S, D, jc, col), n, il);
  }
  // pooled values -> the tile [d][32] in LDS -> slot_v
  if (!key_lane) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float x = n[e] * il;
      T t;
      if constexpr (Ty::kBytes == 2) t = f32_to_bf16(x); else t = x;
      lds[(col + e) * kSlotsPerBlock + js] = t;
    }
  }
  __syncthreads();
  if (value_tile(S) == kSlotsPerBlock) {
    // the tile is contiguous in slot_v: D * 32 elements as 16-byte pieces
    constexpr int P16 = D * kSlotsPerBlock * Ty::kBytes / 16;
    uint4* dst = reinterpret_cast<uint4*>(slot_v + value_index(unit, S, D, tile * kSlotsPerBlock, 0));
    const uint4* srcv = reinterpret_cast<const uint4*>(lds);
    for (int p = tid; p < P16; p += kThreads) dst[p] = srcv[p];
  } else {
    for (int p = tid; p < D * kSlotsPerBlock; p += kThreads) {
      const int dim = p / kSlotsPerBlock, jt = p % kSlotsPerBlock;
      const int jj = tile * kSlotsPerBlock + jt;
      if (jj < S) slot_v[value_index(unit, S, D, jj, dim)] = lds[p];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, d = 128, S a multiple of 32: the summary merge on MFMA.
//
// Workgroup = one unit (sequence, KV head) and a group of kTPW tiles of 32
// slots, 4 waves per tile; the S / (32 kTPW) workgroups of a unit are
// consecutive on one XCD.  For the 32 slots j of a tile and the tau new rows i
// of the unit, with a_ji = u_j.k_i/sqrt(d) + (tau-1-i) ln(lambda_j):
//   S^T = K U^T        rows x slots, 32x32x16 MFMA, each wave for itself;
//   per slot (one lane column): m' = max(m + tau ln(lambda), max_i a_ji),
//   s = e^(m + tau ln(lambda) - m'), w_ji = e^(a_ji - m'), l' = l s + sum_i w_ji;
//   N^T = s N^T + R^T W^T    entries x slots, R = [k | v] of the new rows;
//   wave q of a tile owns the entries 64q..64q+63 (two 32x32 accumulators).
// The weights enter the MFMA as bf16 hi + lo (w - hi), so the products keep
// about 16 bits of the fp32 weight; l sums the fp32 weights.  The state n is
// read once into the accumulators and written once; its tiled layout makes
// each 16-byte load or store of a wave 1 KB contiguous.  The workgroup
// stages all B+1 verified rows of its unit whatever tau is (keys row-major
// for S^T, [entry][row] for R^T, rows past B+1 zero) and its slot queries,
// so no load waits for tau; K-steps past tau are skipped and the weights of
// rows past tau are 0.  The pooled slots leave through LDS as one key tile
// (operand order) and one value tile ([d][32]) per tile, in 16-byte stores.
//
// The window: the unit's workgroups share out the copy of its tau new rows
// from the staged rows to ring slots (L + i) mod W: keys as 16-byte pieces
// at their tiled place, values with lanes over rows (neighbouring lanes,
// neighbouring slots of one tile row).  L is the sequence's length before
// the call, read from a snapshot that the launch before this one took
// (len_snap), so no workgroup here reads seq_len; the lead workgroup of the
// sequence (KV head 0, first tile group) writes ring_pos and seq_len = L + tau.
// ---------------------------------------------------------------------------
// kVerify: tau is not an input but the accepted prefix of the greedy
// verification whose partial argmax keys are vkeys (nkeys per row): every
// workgroup derives it for its sequence, and the lead workgroup also writes
// target_tok and tau_out.
struct VerifyKeys {
  const uint64_t* keys;
  int nkeys;
  const int32_t* draft;
  int32_t* target_tok;
  int32_t* tau_out;
};

// the length snapshot that the separate update takes before its main launch
__global__ __launch_bounds__(256) void len_snapshot(const int32_t* __restrict__ seq_len,
                                                    int32_t* __restrict__ snap, int C) {
  const int c = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (c < C) snap[c] = seq_len[c];
}

// kRB: 32-row score blocks (B + 1 <= 32 kRB); kTPW: tiles of 32 slots per
// workgroup (S / (32 kTPW) workgroups per unit; one when S = 0)
template <int kRB, int kTPW, bool kVerify>
__global__ __launch_bounds__(256 * kTPW) void append_units(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ tau_in, VerifyKeys vk, const int32_t* __restrict__ len_snap,
    uint16_t* __restrict__ ring_k, uint16_t* __restrict__ ring_v, int32_t* __restrict__ ring_pos,
    int32_t* __restrict__ seq_len, float* __restrict__ sum_m, float* __restrict__ sum_l,
    float* __restrict__ sum_n, uint16_t* __restrict__ slot_k, uint16_t* __restrict__ slot_v,
    const uint16_t* __restrict__ u, const float* __restrict__ log_lambda,
    int32_t* __restrict__ err_flag, int C, int Hkv, int W, int S, int B) {
  constexpr int D = 128, E = 2 * D;
  constexpr int kThreads = 256 * kTPW;
  constexpr int RP = 32 * kRB;              // staged rows
  constexpr int KLS = D + 8;                // key / query row stride (bf16)
  constexpr int RTS = RP + 8;               // [entry][row] stride (bf16), 16-byte multiple
  constexpr int kStage = RP * KLS + E * RTS + 32 * kTPW * KLS;
  constexpr int kOut = kTPW * 2 * 32 * D;   // pooled key and value tiles
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStage > kOut ? kStage : kOut];
  uint16_t* KL = lds;                       // [RP][KLS]   verified keys
  uint16_t* RT = KL + RP * KLS;             // [E][RTS]    verified [k | v], transposed
  uint16_t* UL = RT + E * RTS;              // [32 kTPW][KLS] slot queries
  __shared__ int32_t g_tok[64];             // kVerify: the rows' argmax tokens
  const int tid = threadIdx.x, lane = tid & 63;
  // blocks of one unit are consecutive in the order each XCD receives them
  // (block b runs on XCD b mod 8): the unit's staged rows come from one L2
  const int groups = S > 0 ? S / (32 * kTPW) : 1;
  const int nblk = int(gridDim.x);
  int bid = int(blockIdx.x);
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int unit = bid / groups, grp = bid % groups;
  const int c = unit / Hkv, h = unit % Hkv;
  const bool lead = h == 0 && grp == 0;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tl = wave >> 2, q4 = wave & 3;  // tile of the group, entry quarter
  const int tile = grp * kTPW + tl;
  const int ln = lane & 31, hi = lane >> 5;
  const int B1 = B + 1;
  const bool summ = S > 0;
  const int j = tile * 32 + ln;             // this lane's slot
  const int64_t sidx = int64_t(unit) * S + j;
  // the wave's part of the tile's state (tiled numerator layout):
  // acc[t][4k + r] = n[j][32 (2 q4 + t) + 8k + 4 hi + r]
  float* nt = sum_n + (int64_t(unit) * S + tile * 32) * E + q4 * 2 * 4 * 64 * 4 + lane * 4;
  f32x16 acc[2];
  float m_old = 0.f, l_old = 0.f, lnl = 0.f;
  if (summ) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(nt + (t * 4 + k) * 64 * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][4 * k + r] = v[r];
      }
    m_old = sum_m[sidx];
    l_old = sum_l[sidx];
    lnl = log_lambda[j];
  }
  const int L = len_snap[c];

  // staging loads: item (16-byte piece of [k | v], row), rows fastest, so the
  // [entry][row] writes of a wave fall on consecutive banks; then the group's
  // slot queries, 16 pieces per slot
  constexpr int kItems = RP * (E / 8) / kThreads;
  static_assert(kItems >= 1 && kItems * kThreads == RP * (E / 8), "whole passes");
  constexpr int kUItems = 32 * kTPW * (D / 8) / kThreads;
  static_assert(kUItems * kThreads == 32 * kTPW * (D / 8), "whole passes");
  u16x8 x[kItems], xu[kUItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int p = q * kThreads + tid, row = p % RP, pc = p / RP;
    const int half = pc >> 4, e = pc & 15;
    const int rc = min(row, B1 - 1);  // rows past B+1 load a real row and are zeroed
    x[q] = *reinterpret_cast<const u16x8*>((half ? v_new : k_new) + ((int64_t(c) * B1 + rc) * Hkv + h) * D + 8 * e);
  }
  if (summ) {
#pragma unroll
    for (int q = 0; q < kUItems; ++q) {
      const int p = q * kThreads + tid, sl = p >> 4, pc = p & 15;
      xu[q] = *reinterpret_cast<const u16x8*>(u + (int64_t(h) * S + grp * 32 * kTPW + sl) * D + 8 * pc);
    }
  }
  int Tn = 1;
  int32_t dj = 0;
  if constexpr (kVerify) {
    dj = lane < B ? vk.draft[int64_t(c) * B + lane] : 0;
    accept_rows<kThreads>(vk.keys, vk.nkeys, c, B, g_tok, lead ? vk.target_tok : nullptr);
  } else {
    Tn = read_tau(tau_in, c, B, err_flag, lead);
  }
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int p = q * kThreads + tid, row = p % RP, pc = p / RP;
    const int half = pc >> 4, e = pc & 15;
    const u16x8 v = row < B1 ? x[q] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (!half) *reinterpret_cast<u16x8*>(&KL[row * KLS + 8 * e]) = v;
#pragma unroll
    for (int r = 0; r < 8; ++r) RT[(half * D + 8 * e + r) * RTS + row] = v[r];
  }
  if (summ) {
#pragma unroll
    for (int q = 0; q < kUItems; ++q) {
      const int p = q * kThreads + tid, sl = p >> 4, pc = p & 15;
      *reinterpret_cast<u16x8*>(&UL[sl * KLS + 8 * pc]) = xu[q];
    }
  }
  __syncthreads();
  if constexpr (kVerify) {
    Tn = accept_tau(g_tok, dj, B);  // every wave, from the LDS tokens
    if (lead && tid == 0) vk.tau_out[c] = Tn;
  }

  // the window: this workgroup's share of the unit's copies (Tn 16-byte key
  // pieces, then 128 Tn value elements, lanes over rows), from the staged rows
  if (W > 0) {
    const int nk = Tn * (D / 8), n_all = nk + D * Tn;
    const int per = (n_all + groups - 1) / groups;
    const int p0 = grp * per, p1 = min(n_all, p0 + per);
    for (int p = p0 + tid; p < p1; p += kThreads) {
      if (p < nk) {
        const int i = p >> 4, e = p & 15;
        const int slot = (L + i) % W;
        *reinterpret_cast<u16x8*>(ring_k + key_index(unit, W, D, slot, 8 * e)) =
            *reinterpret_cast<const u16x8*>(&KL[i * KLS + 8 * e]);
      } else {
        const int q = p - nk, dim = q / Tn, i = q - dim * Tn;
        ring_v[value_index(unit, W, D, (L + i) % W, dim)] = RT[(D + dim) * RTS + i];
      }
    }
    if (lead && tid < Tn) ring_pos[int64_t(c) * W + (L + tid) % W] = L + tid;
  }
  if (lead && tid == 0) seq_len[c] = L + Tn;
  if (!summ) return;

  // the merge of the wave's two accumulator tiles (merge_ops.hpp)
  float m_new;
  const float l_new = merge_wave<kRB, 2>(KL, RT, UL + 32 * tl * KLS, acc, m_old, l_old, lnl, Tn, q4,
                                         lane, m_new);
  // non-temporal stores: the state is next read a round later, and the
  // round's other streams leave nothing of it in L2 by then
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      __builtin_nontemporal_store(f32x4{acc[t][4 * k], acc[t][4 * k + 1], acc[t][4 * k + 2], acc[t][4 * k + 3]},
                                  reinterpret_cast<f32x4*>(nt + (t * 4 + k) * 64 * 4));
  if (q4 == 0 && hi == 0) {
    sum_m[sidx] = m_new;
    sum_l[sidx] = l_new;
  }

  // pooled slots n / l -> the tile's key tile (operand order) and value tile
  // [d][32] in LDS, then 16-byte stores of the group's tiles
  __syncthreads();  // every wave is done with the staged rows
  pooled_to_lds<2>(acc, 1.0f / l_new, q4, lane, lds + tl * 2 * 32 * D, lds + tl * 2 * 32 * D + 32 * D);
  __syncthreads();
  constexpr int P16 = 32 * D * 2 / 16;  // 16-byte pieces per key (or value) tile
  const uint4* src = reinterpret_cast<const uint4*>(lds);
#pragma unroll
  for (int q = 0; q < 2 * P16 * kTPW / kThreads; ++q) {
    const int p = q * kThreads + tid, t2 = p / (2 * P16), r = p % (2 * P16);
    const int t_glob = grp * kTPW + t2;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 val = *reinterpret_cast<const u32x4*>(src + p);
    u32x4* dst = r < P16 ? reinterpret_cast<u32x4*>(slot_k + key_index(unit, S, D, t_glob * 32, 0)) + r
                         : reinterpret_cast<u32x4*>(slot_v + value_index(unit, S, D, t_glob * 32, 0)) + (r - P16);
    __builtin_nontemporal_store(val, dst);
  }
}

#ifndef LS_APPEND_TPW
#define LS_APPEND_TPW 2
#endif
constexpr int kTilesPerGroup = LS_APPEND_TPW;  // tiles of 32 slots per update workgroup

template <int kRB, int kTPW, bool kVerify>
void launch_units(const ls_dims& d, const ls_state& st, const void* k_new, const void* v_new,
                  const int32_t* tau, const VerifyKeys& vk, const int32_t* len_snap,
                  hipStream_t stream) {
  const int groups = d.S > 0 ? d.S / (32 * kTPW) : 1;
  hipLaunchKernelGGL((append_units<kRB, kTPW, kVerify>), dim3(unsigned(d.C * d.Hkv * groups)),
                     dim3(256 * kTPW), 0, stream, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), tau, vk, len_snap,
                     static_cast<uint16_t*>(st.ring_k), static_cast<uint16_t*>(st.ring_v),
                     st.ring_pos, st.seq_len, st.sum_m, st.sum_l, st.sum_n,
                     static_cast<uint16_t*>(st.slot_k), static_cast<uint16_t*>(st.slot_v),
                     static_cast<const uint16_t*>(st.u), st.log_lambda, st.err_flag, d.C, d.Hkv, d.W,
                     d.S, d.B);
}

// bf16: the shape's instantiation (S in {0, 64, 128}: whole tile groups)
template <bool kVerify>
void launch_units_for(const ls_dims& d, const ls_state& st, const void* k_new, const void* v_new,
                      const int32_t* tau, const VerifyKeys& vk, const int32_t* len_snap,
                      hipStream_t stream) {
  static_assert(64 % (32 * kTilesPerGroup) == 0, "tile groups divide S = 64 and S = 128");
  if (d.B + 1 <= 32)
    launch_units<1, kTilesPerGroup, kVerify>(d, st, k_new, v_new, tau, vk, len_snap, stream);
  else
    launch_units<2, kTilesPerGroup, kVerify>(d, st, k_new, v_new, tau, vk, len_snap, stream);
}

template <typename Ty, int D>
ls_status run(const ls_dims& d, const ls_state& st, const void* k_new, const void* v_new,
              const int32_t* tau, hipStream_t stream) {
  using T = typename Ty::T;
  const int ntile = int(cdiv(d.S, kSlotsPerBlock));
  // LDS of a summary workgroup: the value tile [d][32] and the B+1 staged
  // rows [B+1][2d] (fp32); the window workgroups use none
  const size_t shmem = size_t(D) * kSlotsPerBlock * sizeof(T) + size_t(d.B + 1) * 2 * D * sizeof(float);
  hipLaunchKernelGGL((append_kernel<Ty, D>), dim3(d.C + d.C * d.Hkv * ntile), dim3(block_threads<D>()), shmem,
                     stream, static_cast<const T*>(k_new), static_cast<const T*>(v_new), tau,
                     static_cast<T*>(st.ring_k), static_cast<T*>(st.ring_v), st.ring_pos,
                     st.seq_len, st.sum_m, st.sum_l, st.sum_n, static_cast<T*>(st.slot_k),
                     static_cast<T*>(st.slot_v), static_cast<const T*>(st.u), st.log_lambda,
                     st.err_flag, d.C, d.Hkv, d.W, d.S, d.B);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

ls_status launch_append(const ls_dims& d, const ls_state& st, const void* k_new,
                        const void* v_new, const int32_t* tau, hipStream_t stream) {
  if (d.dtype == LS_BF16) {  // d = 128, S in {0, 64, 128}
    // the lengths before the update, then the update (which advances seq_len)
    int32_t* snap = reinterpret_cast<int32_t*>(static_cast<char*>(st.workspace) + ws_layout(d, 1).len_snap);
    hipLaunchKernelGGL(len_snapshot, dim3(unsigned(cdiv(d.C, 256))), dim3(256), 0, stream, st.seq_len,
                       snap, d.C);
    if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    launch_units_for<false>(d, st, k_new, v_new, tau, VerifyKeys{}, snap, stream);
    return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
  }
  switch (d.d) {
    case 16: return run<F32, 16>(d, st, k_new, v_new, tau, stream);
    case 32: return run<F32, 32>(d, st, k_new, v_new, tau, stream);
    case 64: return run<F32, 64>(d, st, k_new, v_new, tau, stream);
    case 128: return run<F32, 128>(d, st, k_new, v_new, tau, stream);
  }
  return LS_ERR_SHAPE;
}

ls_status launch_append_from_keys(const ls_dims& d, const ls_state& st, const int32_t* draft,
                                  int32_t* target_tok, int32_t* tau, const void* k_new,
                                  const void* v_new, hipStream_t stream) {
  char* ws = static_cast<char*>(st.workspace);
  if (d.dtype != LS_BF16) {  // f32: finish the verification, then the update
    const ls_status s1 = launch_verify_finalize(d, draft, target_tok, tau, ws, stream);
    return s1 != LS_OK ? s1 : launch_append(d, st, k_new, v_new, tau, stream);
  }
  // the update derives tau from the keys; L from the key pass's snapshot
  const WsLayout lay = ws_layout(d, 1);
  const VerifyKeys vk{reinterpret_cast<const uint64_t*>(ws + lay.verify_part), lay.vsplit, draft,
                      target_tok, tau};
  launch_units_for<true>(d, st, k_new, v_new, nullptr, vk,
                         reinterpret_cast<const int32_t*>(ws + lay.len_snap), stream);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

ls_status launch_verify_append(const ls_dims& d, const ls_state& st, const void* logits,
                               const int32_t* draft, int32_t* target_tok, int32_t* tau,
                               const void* k_new, const void* v_new, hipStream_t stream) {
  char* ws = static_cast<char*>(st.workspace);
  if (d.dtype != LS_BF16) {  // f32: the two entry points' launches
    const ls_status s1 = launch_verify(d, logits, draft, target_tok, tau, ws, stream);
    return s1 != LS_OK ? s1 : launch_append(d, st, k_new, v_new, tau, stream);
  }
  // the verification's partial keys; the same launch takes the length snapshot
  const ls_status s1 = launch_verify_keys(d, logits, ws, st.seq_len,
                                          reinterpret_cast<int32_t*>(ws + ws_layout(d, 1).len_snap), stream);
  return s1 != LS_OK ? s1 : launch_append_from_keys(d, st, draft, target_tok, tau, k_new, v_new, stream);
}

}  // namespace ls
