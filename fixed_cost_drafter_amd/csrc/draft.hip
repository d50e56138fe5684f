// Drafter block attention over the three fixed-size views (LongSpark paper
// page, Fig. 2 (c): the drafter proposes the next block from the views at a
// cost independent of the prefix length; Fig. 6: one block proposal).
//
// For sequence c, KV head h and query row (b, hq) with hq / (Hq/Hkv) == h:
//   out = softmax(q k^T / sqrt(d)) v over the keys
//         [ring rows with ring_pos >= 0 | S summary slots | B block rows]
// bidirectional (no mask inside the block).  The B*G query rows of one KV
// head (G = Hq/Hkv) share its keys, so they form one query tile.
//
// bf16, d = 128 (draft_mfma).  One workgroup per (KV head unit, 32 query
// rows), so a Qwen3-8B-shaped layer at C = 16 (128 units x 64 rows) fills the
// 256 CUs.  Its 4 waves are 4 key parts, each for all 32 rows (2 row groups
// of 16, one wave per SIMD with the full register file).  The keys are cut
// in 32-key chunks that never straddle two views (W and S are multiples of
// 32; the block gets its own chunks); each wave streams its part's chunks
// with every MFMA operand loaded straight from memory into registers in
// operand layout, two chunks in flight, with no LDS staging and no barrier
// in the loop:
//   S^T = K Q^T : A = key rows (row-major [key][d]: 16 contiguous bytes per
//                 lane), B = the wave's 16 query rows (registers);
//   O^T += V^T P^T : A = values, which the state keeps in key tiles of 32
//                 ([rows/32][d][32]) so a lane's keys of one dimension are
//                 16 contiguous bytes and a chunk is one 8 KB block; B = the
//                 softmax weights from the S^T output layout, rounded to bf16.
// Each loaded operand serves both row groups of the wave.  The block's
// values arrive token-major from the caller and are transposed through LDS
// once per workgroup.  The online softmax lives in registers (per query row,
// per lane); the key parts merge (m, l, O) in LDS at the end.
// f32 (draft_generic): one workgroup per query row, plain loop (small shapes).
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
#ifndef LS_DRAFT_INFLIGHT
#define LS_DRAFT_INFLIGHT 2
#endif
constexpr int kInFlight = LS_DRAFT_INFLIGHT;  // chunks loading into registers per thread
// Scores are kept in base-2 units (log2(e) folded into the 1/sqrt(d) scale),
// so every softmax weight is one v_exp_f32 (2^x).
constexpr float kScale2 = 0.08838834764831845f * 1.4426950408889634f;  // log2(e)/sqrt(128)
constexpr float kRescale = 8.f * 1.4426950408889634f;  // the running max may lag by e^8
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // v_cvt, nearest-even
}

// Keys are permuted inside a 32-key chunk so that the S^T output puts keys
// 8kg..8kg+7 in lane group kg: A-row m of score block mb holds key
// 8*(m/4) + 4*mb + m%4.  Then the P^T operand, the V^T operand (one 16-byte
// read per dimension block) and the positions all see the lane's 8 keys in
// natural order.
__device__ __forceinline__ int chunk_key(int m, int mb) { return 8 * (m >> 2) + 4 * mb + (m & 3); }

// LDS image of one staged 32-key chunk: keys row-major (padded rows), values
// [d][32] (padded), and a score bias per key (0, or -inf for an empty window
// slot or a block row past B).
constexpr int kKS = 128 + 8;   // key row stride (bf16)
constexpr int kVS = 32 + 8;    // value row stride (bf16)
constexpr int kStageElems = 32 * kKS + 128 * kVS + 64;  // bf16 elements (+ 32 int positions)

struct Stage {  // pointers into one stage buffer
  uint16_t* k;
  uint16_t* v;
  float* bias;
  __device__ explicit Stage(uint16_t* base)
      : k(base), v(base + 32 * kKS), bias(reinterpret_cast<float*>(base + 32 * kKS + 128 * kVS)) {}
};

// One thread's share of a chunk: PPT pieces of 16 bytes of keys and PPT of
// values out of the chunk's 512 + 512 (TPP = 512 / PPT staging threads per
// key part), plus one key's score bias for t < 32.
template <int PPT>
struct Piece {
  u16x8 d[2 * PPT];
  float bias;
};

// Source of chunk ch of one unit: [window W/32 | slots S/32 | block].
struct Views {
  const uint16_t *rk, *rv, *sk, *sv, *kb, *vb;
  const int32_t* rp;
  int W, S, B, Hkv, c, h, nring, ngl;
};

// loads for staging chunk ch (thread t of the part's 512 / PPT staging threads)
template <int PPT>
__device__ __forceinline__ void load_piece(Piece<PPT>& x, const Views& s, int ch, int t) {
  constexpr int D = 128, TPP = 512 / PPT;
  if (ch < s.ngl) {  // window or slots: K rows [key][d], V tile [d][32], contiguous
    const bool ring = ch < s.nring;
    const int key0 = (ring ? ch : ch - s.nring) * 32;
    const uint16_t* kt = (ring ? s.rk : s.sk) + int64_t(key0) * D;
    const uint16_t* vt = (ring ? s.rv : s.sv) + int64_t(ring ? ch : ch - s.nring) * D * 32;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      x.d[j] = *reinterpret_cast<const u16x8*>(kt + (t + TPP * j) * 8);
      x.d[PPT + j] = *reinterpret_cast<const u16x8*>(vt + (t + TPP * j) * 8);
    }
    const int p = ring ? s.rp[key0 + (t & 31)] : 0;  // slots are always occupied
    x.bias = p < 0 ? -INFINITY : 0.f;
  } else {  // block: K and V rows are the caller's token-major [b][Hkv][d]
    const int key0 = (ch - s.ngl) * 32;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int piece = t + TPP * j, row = piece >> 4, col = (piece & 15) * 8;
      const int64_t off = ((int64_t(s.c) * s.B + min(key0 + row, s.B - 1)) * s.Hkv + s.h) * D + col;
      x.d[j] = *reinterpret_cast<const u16x8*>(s.kb + off);
      x.d[PPT + j] = *reinterpret_cast<const u16x8*>(s.vb + off);
    }
    x.bias = key0 + (t & 31) < s.B ? 0.f : -INFINITY;
  }
}

template <int PPT>
__device__ __forceinline__ void store_piece(const Piece<PPT>& x, Stage st, bool block_chunk, int t) {
  constexpr int TPP = 512 / PPT;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int piece = t + TPP * j, row = piece >> 4, col = (piece & 15) * 8;
    *reinterpret_cast<u16x8*>(st.k + row * kKS + col) = x.d[j];
    if (!block_chunk) {  // value tile piece: dim = piece / 4, keys (piece % 4) * 8 ..
      *reinterpret_cast<u16x8*>(st.v + (piece >> 2) * kVS + (piece & 3) * 8) = x.d[PPT + j];
    } else {  // token-major value row -> [d][32]
#pragma unroll
      for (int e = 0; e < 8; ++e) st.v[(col + e) * kVS + row] = x.d[PPT + j][e];
    }
  }
  if (t < 32) st.bias[t] = x.bias;
}

// Online softmax state of one row group of 16 query rows.
struct Softmax {
  float m, l;
  f32x4 o[8];
};

// one staged chunk for the wave's row group: scores (base 2, biased), lazy
// online softmax update, P.V
__device__ __forceinline__ void compute_chunk(Softmax& st, Stage sg, const bf16x8 (&qb)[4], int ln,
                                              int kg) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x4 s[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint16_t* krow = sg.k + chunk_key(ln, mb) * kKS + kg * 8;
    s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      s[mb] = mfma16x16x32(as_bf16x8(*reinterpret_cast<const u16x8*>(krow + ks * 32)), qb[ks], s[mb]);
  }
  // s[mb][r] is key 8kg + 4mb + r of the chunk: score = s * log2(e)/sqrt(d) + bias
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(sg.bias + 8 * kg);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(sg.bias + 8 * kg + 4);
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[0][r] = fmaf(s[0][r], kScale2, b0[r]);
    s[1][r] = fmaf(s[1][r], kScale2, b1[r]);
    tmax = fmaxf(tmax, fmaxf(s[0][r], s[1][r]));
  }
  // the row's max over the 4 lane groups (lanes ln, ln+16, ln+32, ln+48):
  // swapping a register with itself across row pairs / halves leaves the
  // partner's value in one of the two results
  {
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
  }
  // lazy rescale: the reference max moves only when some row's max grows by
  // more than kRescale, so weights stay <= e^8 and the O / l rescale is
  // skipped in the steady state
  if (__any(tmax > st.m + kRescale)) {
    const float m_new = fmaxf(st.m, tmax);
    const float scale = st.m == -INFINITY ? 0.f : exp2_f(st.m - m_new);
    st.m = m_new;
    st.l *= scale;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.o[mb] *= scale;
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
  // weights rounded to bf16 in pairs; l sums the same rounded weights
  uint32_t pw[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const f32x2 e2 = {exp2_f(s[mb][r] - m_use), exp2_f(s[mb][r + 1] - m_use)};
      pw[mb * 2 + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(e2, bf16x2));
    }
  const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), ones, lsum, false);
  st.l += lsum;
  const u16x8 pv = __builtin_bit_cast(u16x8, uint4{pw[0], pw[1], pw[2], pw[3]});
  const bf16x8 pk = as_bf16x8(pv);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(sg.v + (mb * 16 + ln) * kVS + kg * 8);
    st.o[mb] = mfma16x16x32(as_bf16x8(v), pk, st.o[mb]);
  }
}

// Workgroup = (KV head unit, split); 64*RG*KPW threads = RG row groups of 16
// query rows x KPW key parts.  A split is either one of `ksplit` key ranges
// (all rows; the ranges' (m, l, O) go to the workspace for draft_combine, a
// kernel boundary, no fence) or, with ksplit = 1, one range of 16*RG query
// rows over all keys (the output is written here).  The splits of a unit are
// blockIdx = unit + k * units, on one XCD when units is a multiple of 8, so
// the keys they share are fetched from HBM once.  Each key part stages its
// chunks into its own double-buffered LDS stages (kInFlight chunks loading
// in registers) and its RG row-group waves read them; the parts merge in LDS.
template <int RG, int KPW>
__global__ __launch_bounds__(64 * RG * KPW, 1) void draft_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ ring_k,
    const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ring_pos,
    const uint16_t* __restrict__ slot_k, const uint16_t* __restrict__ slot_v,
    uint16_t* __restrict__ out, float* __restrict__ part_out, int Hq, int Hkv, int W, int S,
    int B, int units, int ksplit) {
  constexpr int D = 128, TPP = 64 * RG, PPT = 512 / TPP;
  __shared__ __attribute__((aligned(16))) uint16_t lds[KPW * 2 * kStageElems];

  const int split = blockIdx.x / units;
  const int unit = blockIdx.x % units;
  const int kidx = split % ksplit, ridx = split / ksplit;
  const int c = unit / Hkv, h = unit % Hkv;
  const int G = Hq / Hkv, M = B * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int g = wave % RG, kq = wave / RG;   // row group, key part
  const int t = tid % TPP;                   // staging thread within the part

  // query operand: lane (row ln of group g, kg) holds q[row][ks*32+kg*8..+7]
  const int row = ridx * 16 * RG + g * 16 + ln;
  const bool row_ok = row < M;
  bf16x8 qb[4];
  {
    const int bq = row_ok ? row / G : 0, hq = h * G + (row_ok ? row % G : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (row_ok)
        v = *reinterpret_cast<const u16x8*>(q + ((int64_t(c) * B + bq) * Hq + hq) * D + ks * 32 + kg * 8);
      qb[ks] = as_bf16x8(v);
    }
  }

  const int nring = W / 32, ngl = nring + S / 32, nch = ngl + (B + 31) / 32;
  const Views views{ring_k + int64_t(unit) * W * D, ring_v + int64_t(unit) * D * W,
                    slot_k + int64_t(unit) * S * D, slot_v + int64_t(unit) * D * S, kb, vb,
                    ring_pos + int64_t(c) * W, W, S, B, Hkv, c, h, nring, ngl};
  const int nparts = ksplit * KPW, pidx = kidx * KPW + kq;
  const int per = (nch + nparts - 1) / nparts;
  const int ch0 = pidx * per, ch1 = min(nch, ch0 + per);
  const int steps = per;  // same count in every part (empty chunks are skipped)
  uint16_t* mine = lds + kq * 2 * kStageElems;
  const bool active = ridx * 16 * RG + g * 16 < M;

  Softmax st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // kInFlight chunks are loading into registers while one is computed; the
  // LDS holds two stages (written at step k, read at step k, rewritten at
  // step k + 2 after the barrier of step k + 1)
  Piece<PPT> pc[kInFlight];
#pragma unroll
  for (int u = 0; u < kInFlight; ++u)
    if (ch0 + u < ch1) load_piece(pc[u], views, ch0 + u, t);
  for (int i = 0; i < steps; i += kInFlight) {
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {  // step i + u uses registers pc[u]
      const int stp = i + u, ch = ch0 + stp;
      Stage sg(mine + (stp & 1) * kStageElems);
      if (stp < steps) {
        if (ch < ch1) store_piece(pc[u], sg, ch >= ngl, t);
        __syncthreads();  // stage ready; the stage written two steps ago was read before
        if (ch + kInFlight < ch1) load_piece(pc[u], views, ch + kInFlight, t);
        if (active && ch < ch1) compute_chunk(st, sg, qb, ln, kg);
      }
    }
  }

  // merge the KPW key parts in LDS (reusing the stages), then write
  float lt = st.l;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [KPW-1][RG][64 lanes][34]
  static_assert((KPW - 1) * RG * 64 * 34 * 4 <= KPW * 2 * kStageElems * 2, "merge buffer fits the stages");
  if (kq > 0) {
    float* dst = red + (((kq - 1) * RG + g) * 64 + lane) * 34;
    dst[0] = st.m;
    dst[1] = lt;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[2 + mb * 4 + r] = st.o[mb][r];
  }
  __syncthreads();
  if (kq != 0) return;
  float mx = st.m;
#pragma unroll
  for (int k = 1; k < KPW; ++k) mx = fmaxf(mx, red[(((k - 1) * RG + g) * 64 + lane) * 34]);
  const float w0 = st.m == -INFINITY ? 0.f : exp2_f(st.m - mx);
  float l = lt * w0;
  f32x4 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = st.o[mb] * w0;
#pragma unroll
  for (int k = 1; k < KPW; ++k) {
    const float* src = red + (((k - 1) * RG + g) * 64 + lane) * 34;
    const float wk = src[0] == -INFINITY ? 0.f : exp2_f(src[0] - mx);
    l = fmaf(src[1], wk, l);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[mb][r] = fmaf(src[2 + mb * 4 + r], wk, o[mb][r]);
  }
  if (ksplit == 1) {  // the whole key range: write the output
    if (!row_ok) return;
    const float il = 1.0f / l;
    uint16_t* orow = out + ((int64_t(c) * B + row / G) * Hq + h * G + row % G) * D;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *reinterpret_cast<u16x4*>(orow + mb * 16 + kg * 4) =
          u16x4{bf16_bits(o[mb][0] * il), bf16_bits(o[mb][1] * il), bf16_bits(o[mb][2] * il),
                bf16_bits(o[mb][3] * il)};
  } else {  // partial of this key range: m[64] | l[64] | O[64][D] (m in base 2)
    constexpr int Mpad = 64;
    float* pbuf = part_out + (int64_t(unit) * ksplit + kidx) * int64_t(Mpad) * (D + 2);
    if (kg == 0) {
      pbuf[row] = mx;
      pbuf[Mpad + row] = l;
    }
    float* po = pbuf + 2 * Mpad + int64_t(row) * D;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(po + mb * 16 + kg * 4) = o[mb];
  }
}

// merge the key halves: one thread per (unit, query row, 4 dimensions)
__global__ __launch_bounds__(kThreads) void draft_combine(
    const float* __restrict__ part, uint16_t* __restrict__ out, int Hq, int Hkv, int B,
    int halves, int Mpad, int units) {
  constexpr int D = 128;
  const int G = Hq / Hkv, M = B * G;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int e4 = int(idx % (D / 4)) * 4;
  const int row = int((idx / (D / 4)) % Mpad);
  const int unit = int(idx / (int64_t(D / 4) * Mpad));
  if (unit >= units || row >= M) return;
  const int c = unit / Hkv, h = unit % Hkv;
  const int64_t pstride = int64_t(Mpad) * (D + 2);
  const float* ub = part + int64_t(unit) * halves * pstride;
  float ms[4], ls[4];
  f32x4 os[4];
  float mx = -INFINITY;
  for (int s2 = 0; s2 < halves; ++s2) {
    const float* sp = ub + s2 * pstride;
    ms[s2] = sp[row];
    ls[s2] = sp[Mpad + row];
    os[s2] = *reinterpret_cast<const f32x4*>(sp + 2 * Mpad + int64_t(row) * D + e4);
    mx = fmaxf(mx, ms[s2]);
  }
  float l = 0.f;
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < halves; ++s2) {
    const float wgt = ms[s2] == -INFINITY ? 0.f : exp2_f(ms[s2] - mx);
    l = fmaf(ls[s2], wgt, l);
    a += os[s2] * wgt;
  }
  const float il = 1.0f / l;
  uint16_t* orow = out + ((int64_t(c) * B + row / G) * Hq + h * G + row % G) * D + e4;
  *reinterpret_cast<u16x4*>(orow) = u16x4{bf16_bits(a[0] * il), bf16_bits(a[1] * il),
                                          bf16_bits(a[2] * il), bf16_bits(a[3] * il)};
}

// generic path: one workgroup per (sequence, block row, query head)
template <typename Ty, int D>
__global__ __launch_bounds__(kThreads) void draft_generic(
    const typename Ty::T* __restrict__ q, const typename Ty::T* __restrict__ kb,
    const typename Ty::T* __restrict__ vb, const typename Ty::T* __restrict__ ring_k,
    const typename Ty::T* __restrict__ ring_v, const int32_t* __restrict__ ring_pos,
    const typename Ty::T* __restrict__ slot_k, const typename Ty::T* __restrict__ slot_v,
    typename Ty::T* __restrict__ out, int Hq, int Hkv, int W, int S, int B) {
  __shared__ float qs[D];
  __shared__ float sc[kThreads];
  __shared__ float red[kThreads / 64];
  const int hq = blockIdx.x % Hq;
  const int b = (blockIdx.x / Hq) % B;
  const int c = blockIdx.x / (Hq * B);
  const int G = Hq / Hkv, h = hq / G;
  const int unit = c * Hkv + h;
  const int tid = threadIdx.x;
  const int N = W + S + B;
  const float sm_scale = 1.0f / sqrtf(float(D));
  const int64_t qo = ((int64_t(c) * B + b) * Hq + hq) * D;
  for (int e = tid; e < D; e += kThreads) qs[e] = Ty::load(q, qo + e);

  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  __syncthreads();
  for (int k0 = 0; k0 < N; k0 += kThreads) {
    const int key = k0 + tid;
    float a = -INFINITY;
    if (key < N && (key >= W || ring_pos[int64_t(c) * W + key] >= 0)) {
      float dot = 0.f;
      if (key < W) {
        for (int e = 0; e < D; ++e)
          dot = fmaf(qs[e], Ty::load(ring_k, (int64_t(unit) * W + key) * D + e), dot);
      } else if (key < W + S) {
        for (int e = 0; e < D; ++e)
          dot = fmaf(qs[e], Ty::load(slot_k, (int64_t(unit) * S + key - W) * D + e), dot);
      } else {
        for (int e = 0; e < D; ++e)
          dot = fmaf(qs[e], Ty::load(kb, ((int64_t(c) * B + key - W - S) * Hkv + h) * D + e), dot);
      }
      a = dot * sm_scale;
    }
    float mx = wave_max(a);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float scale = m_run == -INFINITY ? 0.f : exp_f(m_run - m_use);
    const float p = exp_f(a - m_use);
    sc[tid] = p;
    float ps = wave_sum(p);
    if ((tid & 63) == 0) red[tid >> 6] = ps;
    __syncthreads();
    ps = red[0] + red[1] + red[2] + red[3];
    l_run = l_run * scale + ps;
    m_run = m_new;
    if (tid < D) {
      o *= scale;
      const int nk = min(kThreads, N - k0);
      for (int k = 0; k < nk; ++k) {
        const float pk = sc[k];
        if (pk == 0.f) continue;
        const int kk = k0 + k;
        float v;  // values of the window and of the slots are key-tiled
        if (kk < W)
          v = Ty::load(ring_v, value_index(unit, W, D, kk, tid));
        else if (kk < W + S)
          v = Ty::load(slot_v, value_index(unit, S, D, kk - W, tid));
        else
          v = Ty::load(vb, ((int64_t(c) * B + kk - W - S) * Hkv + h) * D + tid);
        o = fmaf(pk, v, o);
      }
    }
    __syncthreads();
  }
  if (tid < D) Ty::store(out, qo + tid, o / l_run);
}

template <int D>
ls_status run_generic(const ls_dims& d, const ls_state& st, const void* q, const void* kb,
                      const void* vb, void* out, hipStream_t stream) {
  hipLaunchKernelGGL((draft_generic<F32, D>), dim3(d.C * d.B * d.Hq), dim3(kThreads), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(kb),
                     static_cast<const float*>(vb), static_cast<const float*>(st.ring_k),
                     static_cast<const float*>(st.ring_v), st.ring_pos,
                     static_cast<const float*>(st.slot_k), static_cast<const float*>(st.slot_v),
                     static_cast<float*>(out), d.Hq, d.Hkv, d.W, d.S, d.B);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

ls_status launch_draft(const ls_dims& d, const ls_state& st, const void* q, const void* kb,
                       const void* vb, void* out, hipStream_t stream) {
  if (d.dtype == LS_BF16) {
    const int units = d.C * d.Hkv;
    const int M = d.B * (d.Hq / d.Hkv);
    const int ksplit = draft_halves(d);  // 1 under the row split
    float* part = reinterpret_cast<float*>(static_cast<char*>(st.workspace) + ws_layout(d, 1).draft_part);
    const uint16_t *q16 = static_cast<const uint16_t*>(q), *kb16 = static_cast<const uint16_t*>(kb),
                   *vb16 = static_cast<const uint16_t*>(vb);
    const uint16_t *rk = static_cast<const uint16_t*>(st.ring_k), *rv = static_cast<const uint16_t*>(st.ring_v),
                   *sk = static_cast<const uint16_t*>(st.slot_k), *sv = static_cast<const uint16_t*>(st.slot_v);
    uint16_t* o16 = static_cast<uint16_t*>(out);
    if (draft_row_split(d)) {
      // query rows in two halves of 32 (2 row groups x 4 key parts), all keys each
      const int rsplit = int(cdiv(M, 32));
      hipLaunchKernelGGL((draft_mfma<2, 4>), dim3(units * rsplit), dim3(512), 0, stream, q16, kb16, vb16,
                         rk, rv, st.ring_pos, sk, sv, o16, part, d.Hq, d.Hkv, d.W, d.S, d.B, units, 1);
      return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
    }
    hipLaunchKernelGGL((draft_mfma<4, 2>), dim3(units * ksplit), dim3(512), 0, stream, q16, kb16, vb16,
                       rk, rv, st.ring_pos, sk, sv, o16, part, d.Hq, d.Hkv, d.W, d.S, d.B, units, ksplit);
    if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    if (ksplit > 1) {
      const int Mpad = 64;
      const int64_t threads = int64_t(units) * Mpad * (128 / 4);
      hipLaunchKernelGGL(draft_combine, dim3(unsigned(cdiv(threads, kThreads))), dim3(kThreads), 0,
                         stream, part, o16, d.Hq, d.Hkv, d.B, ksplit, Mpad, units);
    }
    return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
  }
  switch (d.d) {
    case 16: return run_generic<16>(d, st, q, kb, vb, out, stream);
    case 32: return run_generic<32>(d, st, q, kb, vb, out, stream);
    case 64: return run_generic<64>(d, st, q, kb, vb, out, stream);
    case 128: return run_generic<128>(d, st, q, kb, vb, out, stream);
  }
  return LS_ERR_SHAPE;
}

}  // namespace ls
