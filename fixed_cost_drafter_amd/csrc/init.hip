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
// (v_mfma_f32_16x16x32_bf16): S^T = K U^T per 64-row tile, then the online
// softmax in registers, then n^T += [K|V]^T P^T with P rounded to bf16 (l
// sums the same rounded weights, so n/l stays an exact weighted mean of the
// inputs).  The f32 kernel is a plain LDS-tiled loop for small shapes.
// Phase 2 (init_finalize): merges the partials (associative max-rescale),
// writes the state and the slots, fills the ring, sets seq_len and err_flag.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }
#ifndef LS_INIT_PREFETCH
#define LS_INIT_PREFETCH 2
#endif

// partial block of (split, unit): m[S] | l[S] | n[S][2d]
__device__ __host__ inline int64_t part_off(int split, int units, int unit, int S, int D) {
  return (int64_t(split) * units + unit) * int64_t(S) * (2 * D + 2);
}

// ---------------------------------------------------------------------------
// MFMA partial kernel: bf16, d = 128, S = 16 * NW; wave w owns slots 16w..16w+15
// and every wave reads the whole LDS tile of TR rows
// ---------------------------------------------------------------------------
template <int NW, int TR>
__global__ __launch_bounds__(64 * NW, 1) void init_mfma_partial(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, int64_t rows_stride,
    int L0, int rows_per_split, int nsplit, const uint16_t* __restrict__ u,
    const float* __restrict__ log_lambda, int Hkv, float* __restrict__ part) {
  constexpr int D = 128, S = 16 * NW, NT = 64 * NW;
  constexpr int KLS = D + 8;   // row-major K tile stride (bf16 elements)
  constexpr int VTS = TR + 4;  // transposed [dim][row] stride (bf16 elements)
  constexpr int MB = TR / 16;  // 16-row blocks per tile
  constexpr int KS2 = TR / 32; // 32-row k-steps of the PV product
  constexpr int PAIRS = TR / (8 * NW);  // row pairs staged per thread
  static_assert(PAIRS >= 1 && TR % (8 * NW) == 0, "tile rows must cover the threads");
  // prefix tiles loading in registers per thread (deeper when a thread's
  // share of a tile is one row pair, so the registers still fit two waves)
  constexpr int kInitPrefetch = PAIRS == 1 ? LS_INIT_PREFETCH : 1;
  __shared__ __attribute__((aligned(16))) uint16_t KL[TR * KLS];
  __shared__ __attribute__((aligned(16))) uint16_t KVT[2 * D * VTS];

  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;  // c * Hkv + h
  const int h = unit % Hkv;
  const int c = unit / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int r_begin = split * rows_per_split;
  const int r_end = min(L0, r_begin + rows_per_split);
  const int t_newest = L0 - 1;
  // scores in base 2 (one v_exp_f32 per weight): a2 = a * log2(e)
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float k2 = 0.08838834764831845f * kLog2e;  // log2(e) / sqrt(128)

  // slot queries as the B operand of S^T = K U^T: lane (slot ln, kg) holds
  // u[slot][ks*32 + kg*8 .. +7]
  const int slot = wave * 16 + ln;
  const float lnl2 = log_lambda[slot] * kLog2e;  // -inf stays -inf (lambda = 0)
  bf16x8 ub[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    ub[ks] = as_bf16x8(
        *reinterpret_cast<const u16x8*>(u + (int64_t(h) * S + slot) * D + ks * 32 + kg * 8));

  float m_run = -INFINITY, l_run = 0.f;  // reference max (may lag) and weight sum
  float m_true = -INFINITY;               // exact running max
  f32x4 acc[16];  // n^T: lane (slot ln, kg) holds dims mb*16 + kg*4 + r
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // global -> register staging: thread (dg = tid%16, rp = tid/16) loads row
  // pairs rp + k*(NT/16); 16 lanes cover one 256-byte row segment
  const int dg = tid & 15, rp = tid >> 4;
  // kInitPrefetch tiles are loading into registers while one is computed
  u16x8 kr[kInitPrefetch][2 * PAIRS], vr[kInitPrefetch][2 * PAIRS];
  auto load_tile = [&](int t0, u16x8 (&kd)[2 * PAIRS], u16x8 (&vd)[2 * PAIRS])
                       __attribute__((always_inline)) {
    const int nrows = min(TR, r_end - t0);
#pragma unroll
    for (int i = 0; i < 2 * PAIRS; ++i) {
      const int row = 2 * (rp + (i >> 1) * (NT / 16)) + (i & 1);
      if (row < nrows) {
        const int64_t off = ((int64_t(c) * rows_stride + t0 + row) * Hkv + h) * D + dg * 8;
        kd[i] = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(kp + off));
        vd[i] = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(vp + off));
      } else {
        kd[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        vd[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };

#pragma unroll
  for (int u = 0; u < kInitPrefetch; ++u)
    if (r_begin + u * TR < r_end) load_tile(r_begin + u * TR, kr[u], vr[u]);
  for (int tb = r_begin; tb < r_end; tb += kInitPrefetch * TR) {
#pragma unroll
  for (int u = 0; u < kInitPrefetch; ++u) {  // tile t0 uses registers kr[u], vr[u]
    const int t0 = tb + u * TR;
    if (t0 >= r_end) break;
    const int nrows = min(TR, r_end - t0);
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int pp = 0; pp < PAIRS; ++pp) {
      const int row0 = 2 * (rp + pp * (NT / 16));  // even row of the pair
      *reinterpret_cast<u16x8*>(&KL[row0 * KLS + dg * 8]) = kr[u][2 * pp];
      *reinterpret_cast<u16x8*>(&KL[(row0 + 1) * KLS + dg * 8]) = kr[u][2 * pp + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // (row0, row0 + 1) of one dimension as one dword: v_perm of the two rows
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint4 k0 = __builtin_bit_cast(uint4, kr[u][2 * pp]), k1 = __builtin_bit_cast(uint4, kr[u][2 * pp + 1]);
        const uint4 v0 = __builtin_bit_cast(uint4, vr[u][2 * pp]), v1 = __builtin_bit_cast(uint4, vr[u][2 * pp + 1]);
        const uint32_t k0w[4] = {k0.x, k0.y, k0.z, k0.w}, k1w[4] = {k1.x, k1.y, k1.z, k1.w};
        const uint32_t v0w[4] = {v0.x, v0.y, v0.z, v0.w}, v1w[4] = {v1.x, v1.y, v1.z, v1.w};
        const uint32_t kk = __builtin_amdgcn_perm(k1w[e >> 1], k0w[e >> 1], sel);
        const uint32_t vv = __builtin_amdgcn_perm(v1w[e >> 1], v0w[e >> 1], sel);
        *reinterpret_cast<uint32_t*>(&KVT[(dg * 8 + e) * VTS + row0]) = kk;
        *reinterpret_cast<uint32_t*>(&KVT[(D + dg * 8 + e) * VTS + row0]) = vv;
      }
    }
    __syncthreads();
    if (t0 + kInitPrefetch * TR < r_end)  // refill: that tile loads during the next computes
      load_tile(t0 + kInitPrefetch * TR, kr[u], vr[u]);

    // S^T[row][slot]: lane (slot ln, kg) holds rows mb*16 + kg*4 + r
    f32x4 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u16x8*>(&KL[(mb * 16 + ln) * KLS + ks * 32 + kg * 8]));
        s[mb] = mfma16x16x32(a, ub[ks], s[mb]);
      }
    }

    // online softmax per slot over this tile (base 2).  Row r of the tile
    // sits at distance t_newest - t0 - r >= 1 from the newest row except in
    // the tile holding the newest row or the ragged tail, which take the
    // exact per-row path (distance 0 has no bias; rows past the end are out).
    float tmax = -INFINITY;
    if (t0 + TR <= t_newest && nrows == TR) {
      const float dk = float(t_newest - t0 - kg * 4);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float bias = (dk - float(mb * 16 + r)) * lnl2;
          const float a = fmaf(s[mb][r], k2, bias);
          s[mb][r] = a;
          tmax = fmaxf(tmax, a);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mb * 16 + kg * 4 + r;
          const int dist = t_newest - (t0 + row);
          const float bias = dist == 0 ? 0.f : float(dist) * lnl2;
          float a = fmaf(s[mb][r], k2, bias);
          if (row >= nrows) a = -INFINITY;
          s[mb][r] = a;
          tmax = fmaxf(tmax, a);
        }
    }
    // the slot's max over the 4 lane groups (rows): swapping a register with
    // itself across row pairs / halves leaves the partner's value in one result
    {
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    // lazy rescale: the reference max moves only when some slot's max grows
    // by more than 8 e-folds (weights stay <= e^8), so the 64-register
    // accumulator rescale is skipped in the steady state
    m_true = fmaxf(m_true, tmax);
    if (__any(tmax > m_run + 8.f * kLog2e)) {
      const float m_new = fmaxf(m_run, tmax);
      const float scale = m_run == -INFINITY ? 0.f : exp2_f(m_run - m_new);
      m_run = m_new;
      l_run *= scale;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) acc[mb] *= scale;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // weights rounded to bf16 in pairs; l sums the same rounded weights
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
    uint32_t pw[MB * 2];
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const f32x2 e2 = {exp2_f(s[mb][r] - m_use), exp2_f(s[mb][r + 1] - m_use)};
        const bf16x2 b2 = __builtin_convertvector(e2, bf16x2);
        pw[mb * 2 + r / 2] = __builtin_bit_cast(uint32_t, b2);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(b2, ones, lsum, false);
      }
    l_run += lsum;
    u16x8 pv[KS2];
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks)  // rows of 16-row blocks 2ks and 2ks+1
      pv[ks] = __builtin_bit_cast(u16x8, uint4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});

    // n^T[dim][slot] += [K|V]^T[dim][row] P^T[row][slot]; the k order of the
    // A operand (rows 32ks+4kg..+3, 32ks+16+4kg..+3) matches pv's element order
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) {
      const bf16x8 pk = as_bf16x8(pv[ks]);
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        const uint16_t* base = &KVT[(mb * 16 + ln) * VTS + ks * 32 + kg * 4];
        const u16x4 lo = *reinterpret_cast<const u16x4*>(base);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(base + 16);
        const bf16x8 a = as_bf16x8(u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        acc[mb] = mfma16x16x32(a, pk, acc[mb]);
      }
    }
  }
  }

  // the state's m is the exact max: move the reference there once
  if (m_true > m_run) {
    const float scale = exp2_f(m_run - m_true);
    m_run = m_true;
    l_run *= scale;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) acc[mb] *= scale;
  }

  // write the partial: lane (slot ln, kg) holds n[slot][mb*16 + kg*4 + r]
  float* pb = part + part_off(split, gridDim.x / nsplit, unit, S, D);
  float lt = l_run;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (kg == 0) {
    pb[slot] = m_run * kLn2;  // natural units, as the state keeps m
    pb[S + slot] = lt;
  }
  float* nrow = pb + 2 * S + int64_t(slot) * 2 * D;
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) *reinterpret_cast<f32x4*>(nrow + mb * 16 + kg * 4) = acc[mb];
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
  for (int p = tid; p < nj * 2 * D; p += kThreads) {
    const int jj = p / (2 * D), e = p % (2 * D);
    float a = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* pn = part + part_off(s, units, unit, S, D) + 2 * S;
      a = fmaf(pn[int64_t(j0 + jj) * 2 * D + e], wsm[s * SPB + jj], a);
    }
    const int64_t ni = (int64_t(unit) * S + j0 + jj) * 2 * D + e;
    sum_n[ni] = a;
    const int j = j0 + jj;
    if (e < D)
      Ty::store(slot_k, key_index(unit, S, D, j, e), a * s_inv_l[jj]);
    else  // values in key tiles of 32 (one tile of S keys when S % 32 != 0)
      Ty::store(slot_v,
                S % 32 == 0 ? ((int64_t(unit) * (S >> 5) + (j >> 5)) * D + (e - D)) * 32 + (j & 31)
                            : (int64_t(unit) * D + (e - D)) * S + j,
                a * s_inv_l[jj]);
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
  const int rows = init_rows_per_split(d, L0);
  const int nsplit = int(cdiv(L0, rows));
  float* part = reinterpret_cast<float*>(static_cast<char*>(st.workspace) + lay.init_part);
  if (d.dtype == LS_BF16) {
    const dim3 grid(d.C * d.Hkv * nsplit);
    const uint16_t* k16 = static_cast<const uint16_t*>(kp);
    const uint16_t* v16 = static_cast<const uint16_t*>(vp);
    const uint16_t* u16 = static_cast<const uint16_t*>(st.u);
    if (d.S == 128)
      hipLaunchKernelGGL((init_mfma_partial<8, 64>), grid, dim3(512), 0, stream, k16, v16,
                         rows_stride, L0, rows, nsplit, u16, st.log_lambda, d.Hkv, part);
    else if (d.S == 64)
      hipLaunchKernelGGL((init_mfma_partial<4, 64>), grid, dim3(256), 0, stream, k16, v16,
                         rows_stride, L0, rows, nsplit, u16, st.log_lambda, d.Hkv, part);
    // S = 0: no summary to pool; the finalize fills the window only
    if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    return finalize<BF16, 128>(d, st, part, nsplit, kp, vp, L0, rows_stride, stream);
  }
  switch (d.d) {
    case 16: return run_f32<16>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 32: return run_f32<32>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 64: return run_f32<64>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
    case 128: return run_f32<128>(d, st, kp, vp, L0, rows_stride, part, rows, nsplit, stream);
  }
  return LS_ERR_SHAPE;
}

}  // namespace ls
