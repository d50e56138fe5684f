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
// Grid: C window workgroups (one per sequence: the only reader and writer of
// seq_len in the launch, so the update needs no second kernel and no
// device-scope fence), then one workgroup per (sequence, KV head, 32 slots).
//
// Summary workgroups: 32 slots, LPS lanes per slot (32; at most d for f32).
// Lane g of a slot owns 2d/LPS consecutive entries of the slot's [k | v]
// numerator n (the first half of the lanes the key half, the rest the value
// half) and keeps them in registers from the first load to the last store,
// so the fp32 state crosses HBM once each way.  All B+1 verified rows of the
// (sequence, KV head) are staged once in LDS as fp32, whatever tau is, so no
// load waits for tau.  The tau new rows are merged two at a time: the key
// lanes form partial dot products with the slot query, a DPP butterfly over
// the slot's lanes completes the scores, and one rescale per batch folds them
// into (m, l, n).  The slots n / l leave as pooled keys (each lane's 8
// dimensions as one 16-byte piece at its place in the key layout) and
// pooled values; the values of the workgroup's 32
// slots are one key tile ([d][32]) of the value layout the drafter reads,
// assembled in LDS and stored contiguously.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

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
// Work item p = (head, 16-byte piece, row), rows fastest: a thread copies the
// key piece to its place in the key layout and scatters the value piece's
// elements into the value layout, where neighbouring lanes (neighbouring rows)
// land in neighbouring window slots of one dimension's tile row.  Every load
// of a thread's items is in flight before its first store, and nothing waits
// on another thread, so the latency is tau's load, one load and the stores,
// whatever tau is.
constexpr int kWindowUnroll = 4;  // items per thread per pass
template <typename Ty, int D>
__device__ __forceinline__ void append_window(
    const typename Ty::T* __restrict__ k_new, const typename Ty::T* __restrict__ v_new,
    const int32_t* __restrict__ tau_in, typename Ty::T* __restrict__ ring_k,
    typename Ty::T* __restrict__ ring_v, int32_t* __restrict__ ring_pos,
    int32_t* __restrict__ seq_len, int32_t* __restrict__ err_flag, int c, int Hkv, int W, int B) {
  using T = typename Ty::T;
  constexpr int kThreads = block_threads<D>();
  constexpr int E16 = 16 / Ty::kBytes;      // elements per 16-byte piece
  constexpr int V16 = D / E16;              // 16-byte pieces per key row
  const int tid = threadIdx.x;
  const int B1 = B + 1;
  int Tn = tau_in[c];
  if (Tn < 1 || Tn > B1) {
    if (tid == 0) atomicOr(err_flag, 1);
    Tn = Tn < 1 ? 1 : B1;
  }
  const int L = seq_len[c];
  if (W == 0) {  // no window view: only the count advances
    if (tid == 0) seq_len[c] = L + Tn;
    return;
  }
  const int slot0 = L % W;                  // window slot of row 0; row i -> slot0 + i (mod W)
  const bool tiled = value_tile(W) == 32;   // values in 32-key tiles (else one tile of W keys)
  const int items = Hkv * V16 * Tn;
  for (int p0 = 0; p0 < items; p0 += kThreads * kWindowUnroll) {
    uint4 kv[kWindowUnroll], vv[kWindowUnroll];
#pragma unroll
    for (int u = 0; u < kWindowUnroll; ++u) {
      const int p = min(p0 + u * kThreads + tid, items - 1);  // past the end: repeat the last item
      const int i = p % Tn, hp = p / Tn, e = hp % V16, hl = hp / V16;
      const int64_t src = ((int64_t(c) * B1 + i) * Hkv + hl) * D + e * E16;
      kv[u] = *reinterpret_cast<const uint4*>(k_new + src);
      vv[u] = *reinterpret_cast<const uint4*>(v_new + src);
    }
#pragma unroll
    for (int u = 0; u < kWindowUnroll; ++u) {
      const int p = p0 + u * kThreads + tid;
      if (p < items) {
        const int i = p % Tn, hp = p / Tn, e = hp % V16, hl = hp / V16;
        const int slot = slot0 + i >= W ? slot0 + i - W : slot0 + i;
        const int64_t unit = int64_t(c) * Hkv + hl;
        *reinterpret_cast<uint4*>(ring_k + key_index(unit, W, D, slot, e * E16)) = kv[u];
        const T* ve = reinterpret_cast<const T*>(&vv[u]);
#pragma unroll
        for (int q = 0; q < E16; ++q) {
          const int dim = e * E16 + q;
          const int64_t idx = tiled ? ((unit * (W >> 5) + (slot >> 5)) * D + dim) * 32 + (slot & 31)
                                    : (unit * D + dim) * W + slot;
          ring_v[idx] = ve[q];
        }
      }
    }
  }
  for (int i = tid; i < Tn; i += kThreads) {
    const int slot = slot0 + i >= W ? slot0 + i - W : slot0 + i;
    ring_pos[int64_t(c) * W + slot] = L + i;
  }
  if (tid == 0) seq_len[c] = L + Tn;
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
    append_window<Ty, D>(k_new, v_new, tau_in, ring_k, ring_v, ring_pos, seq_len, err_flag,
                         int(blockIdx.x), Hkv, W, B);
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
  if (d.dtype == LS_BF16) return run<BF16, 128>(d, st, k_new, v_new, tau, stream);
  switch (d.d) {
    case 16: return run<F32, 16>(d, st, k_new, v_new, tau, stream);
    case 32: return run<F32, 32>(d, st, k_new, v_new, tau, stream);
    case 64: return run<F32, 64>(d, st, k_new, v_new, tau, stream);
    case 128: return run<F32, 128>(d, st, k_new, v_new, tau, stream);
  }
  return LS_ERR_SHAPE;
}

}  // namespace ls
