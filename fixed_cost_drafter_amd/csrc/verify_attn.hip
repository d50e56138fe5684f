// Target-side verification attention of one layer (LongSpark paper page,
// Fig. 2 (a): the target verifies the proposed block, attending over its
// whole context).  This is the per-round cost that grows with the prefix --
// the cost the drafter's fixed-size views avoid.
//
// For sequence c with L = L[c] context rows, the B+1 verified positions sit
// at rows L..L+B of the token-major cache [C, rows, Hkv, d]; query i (row
// L+i) of head hq attends causally to rows 0..L+i of KV head hq/(Hq/Hkv),
// softmax scale 1/sqrt(d):
//   out[c, i, hq] = softmax_{p <= L+i}(q . k_p / sqrt(d)) v_p.
//
// bf16, d = 128 (attn_mfma_partial + attn_combine): the (B+1)*G query rows of
// a KV head are one tile (one wave per 16 rows); the L+B+1 keys are cut into
// `nsplit` ranges of whole 64-row tiles, one workgroup each (flash-decoding).
// A workgroup stages each 64-row tile in LDS (keys row-major for
// S^T = K Q^T, values transposed for O^T += V^T P^T, both on
// v_mfma_f32_16x16x32_bf16), keeps the online softmax per query row in its
// lane (base 2, lazy rescale), masks the keys past a query's own row only in
// the tiles that reach row L, and writes a partial (m, l, O).  A second
// launch merges the ranges (a kernel boundary, no device-scope fence).
// f32 (attn_generic): one workgroup per (sequence, verified row, query head).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// L[c] is read on the device; a value outside [0, max_rows - B - 1] is
// clamped and flagged
__device__ __forceinline__ int context_rows(const int32_t* Lctx, int c, int B, int max_rows,
                                            int32_t* err_flag, bool report) {
  int L = Lctx[c];
  const int hi = max_rows - B - 1;
  if (L < 0 || L > hi) {
    if (report && err_flag != nullptr) atomicOr(err_flag, 1);
    L = L < 0 ? 0 : hi;
  }
  return L;
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_mfma_partial(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int64_t rows_stride,
    const int32_t* __restrict__ Lctx, int max_rows, const uint16_t* __restrict__ q, int Hq,
    int Hkv, int B, int rows_per_split, int nsplit, float* __restrict__ part,
    int32_t* __restrict__ err_flag) {
  constexpr int D = 128, TR = 64, NT = 64 * NW, Mq = 16 * NW;
  // K and V tiles: 64 rows of 256 bytes as they arrive, 16-byte chunk c of
  // row r at chunk c ^ (r % 16).  That puts the score operand reads (16 rows,
  // one chunk per lane group) and the transposed P.V reads (16 rows x 32
  // bytes) on the fewest bank cycles.  Tiles go from global memory straight
  // into LDS (global_load_lds_dwordx4: lane i of an instruction fills the
  // i-th 16 bytes of a 1 KB block, so each lane fetches the chunk the swizzle
  // puts there), double buffered in separate arrays so that the compiler can
  // tell the tile in flight from the one being read.
  constexpr int MB = TR / 16;  // 16-row key blocks per tile
  constexpr int KS2 = TR / 32; // 32-row k-steps of the PV product
  constexpr int NBLK = TR * D * 2 / 1024;  // 1 KB blocks per K (or V) tile
  __shared__ __attribute__((aligned(16))) uint16_t K0[TR * D];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TR * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TR * D];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TR * D];
  auto chunk_at = [](int r, int ch) { return r * D + ((ch ^ (r & 15)) << 3); };

  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;  // c * Hkv + h
  const int h = unit % Hkv, c = unit / Hkv;
  const int G = Hq / Hkv, M = (B + 1) * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int L = context_rows(Lctx, c, B, max_rows, err_flag, h == 0 && split == 0 && tid == 0);
  const int nkeys = L + B + 1;
  const int r_begin = split * rows_per_split;
  const int r_end = min(nkeys, r_begin + rows_per_split);
  const float k2 = 0.08838834764831845f * kLog2e;  // log2(e) / sqrt(128)

  // query operand of S^T = K Q^T: lane (row ln of wave w's group, kg) holds
  // q[row][ks*32 + kg*8 .. +7]; row = i*G + g is verified position i, head h*G+g
  const int qrow = wave * 16 + ln;
  const bool q_ok = qrow < M;
  const int qi = q_ok ? qrow / G : 0;
  const int lim = q_ok ? L + qi : -1;  // last key row this query sees
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (q_ok)
      v = *reinterpret_cast<const u16x8*>(
          q + ((int64_t(c) * (B + 1) + qi) * Hq + h * G + qrow % G) * D + ks * 32 + kg * 8);
    qb[ks] = as_bf16x8(v);
  }

  float m_run = -INFINITY, l_run = 0.f;  // reference max (base 2, may lag) and weight sum
  f32x4 acc[8];  // O^T: lane (row ln, kg) holds dims mb*16 + kg*4 + r
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile rows t0 .. t0+63 -> (Kb, Vb): wave w fills blocks w, w + NW, ...;
  // rows past the range repeat its last row (masked, weight 0)
  auto issue_tile = [&](int t0, uint16_t* Kb, uint16_t* Vb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < (NBLK + NW - 1) / NW; ++j) {
      const int blk = wave + NW * j;
      if (blk < NBLK) {  // uniform in the wave
        const int p = 64 * blk + lane, row = p >> 4, ch = (p & 15) ^ (row & 15);
        const int64_t off = ((int64_t(c) * rows_stride + min(t0 + row, r_end - 1)) * Hkv + h) * D + ch * 8;
        __builtin_amdgcn_global_load_lds(kc + off, (__attribute__((address_space(3))) void*)(Kb + blk * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vc + off, (__attribute__((address_space(3))) void*)(Vb + blk * 512), 16, 0, 0);
      }
    }
  };

  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto tile_step = [&](int t0, const uint16_t* KL, const uint16_t* VL, uint16_t* Kn, uint16_t* Vn)
                       __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's blocks of the tile are in LDS
    __syncthreads();  // ... and every wave's; the other buffers' reads (previous tile) are done
    if (t0 + TR < r_end) issue_tile(t0 + TR, Kn, Vn);  // streams in during this tile

    // S^T[key][query]: lane (query ln, kg) holds keys mb*16 + kg*4 + r
    f32x4 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[mb] = mfma16x16x32(
            as_bf16x8(*reinterpret_cast<const u16x8*>(&KL[chunk_at(mb * 16 + ln, ks * 4 + kg)])),
            qb[ks], s[mb]);
    }
    // base-2 scores; keys past the query's own row (or past the range) only
    // occur in tiles that reach row L or the range's end
    float tmax = -INFINITY;
    const bool masked = t0 + TR > L || t0 + TR > r_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = s[mb][r] * k2;
        if (masked) {
          const int kp = t0 + mb * 16 + kg * 4 + r;
          if (kp > lim || kp >= r_end) a = -INFINITY;
        }
        s[mb][r] = a;
        tmax = fmaxf(tmax, a);
      }
    {  // the query's max over its 4 lane groups
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    if (__any(tmax > m_run + 8.f * kLog2e)) {  // lazy rescale: weights stay <= e^8
      const float m_new = fmaxf(m_run, tmax);
      const float scale = m_run == -INFINITY ? 0.f : exp2_f(m_run - m_new);
      m_run = m_new;
      l_run *= scale;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb] *= scale;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
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
    // O^T[dim][query] += V^T[dim][key] P^T[key][query]; the k order of the A
    // operand (keys 32ks+4kg..+3, 32ks+16+4kg..+3) matches the weights'
    // order.  ds_read_b64_tr_b16 gives lane 4a + b of a 16-lane group element
    // b of the 8-byte reads of lanes a, a+4, a+8, a+12: reader lane ln of
    // group kg reads row 32ks + 4kg + ln / 4 (+16 for the second half) at
    // dimensions 16mb + 4(ln % 4) .. +3, so lane ln receives those 4 keys of
    // dimension 16mb + ln.
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) {
      const bf16x8 pk = as_bf16x8(__builtin_bit_cast(
          u16x8, uint4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]}));
      const int vrow = 32 * ks + 4 * kg + (ln >> 2);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int ch = 2 * mb + ((ln & 3) >> 1), sub = 4 * (ln & 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(VL + chunk_at(vrow, ch) + sub));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(VL + chunk_at(vrow + 16, ch) + sub));
        acc[mb] = mfma16x16x32(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                               pk, acc[mb]);
      }
    }
  };
  if (r_begin < r_end) issue_tile(r_begin, K0, V0);
  for (int t0 = r_begin; t0 < r_end; t0 += 2 * TR) {  // even tiles in buffers 0, odd in 1
    tile_step(t0, K0, V0, K1, V1);
    if (t0 + TR < r_end) tile_step(t0 + TR, K1, V1, K0, V0);
  }

  // partial of this range: m[Mq] | l[Mq] | O[Mq][D]  (m in base 2)
  float* pb = part + (int64_t(unit) * nsplit + split) * int64_t(Mq) * (D + 2);
  float lt = l_run;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (kg == 0) {
    pb[qrow] = m_run;
    pb[Mq + qrow] = lt;
  }
  float* orow = pb + 2 * Mq + int64_t(qrow) * D;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(orow + mb * 16 + kg * 4) = acc[mb];
}

// merge the ranges: one thread per (unit, query row, 4 dimensions)
__global__ __launch_bounds__(kThreads) void attn_combine(const float* __restrict__ part,
                                                         uint16_t* __restrict__ out, int Hq, int Hkv,
                                                         int B, int nsplit, int Mq, int units) {
  constexpr int D = 128;
  const int G = Hq / Hkv, M = (B + 1) * G;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int e4 = int(idx % (D / 4)) * 4;
  const int row = int((idx / (D / 4)) % Mq);
  const int unit = int(idx / (int64_t(D / 4) * Mq));
  if (unit >= units || row >= M) return;
  const int c = unit / Hkv, h = unit % Hkv;
  const int64_t pstride = int64_t(Mq) * (D + 2);
  const float* ub = part + int64_t(unit) * nsplit * pstride;
  float mx = -INFINITY;
  for (int s2 = 0; s2 < nsplit; ++s2) mx = fmaxf(mx, ub[s2 * pstride + row]);
  float l = 0.f;
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < nsplit; ++s2) {
    const float* sp = ub + s2 * pstride;
    const float ms = sp[row];
    const float wgt = ms == -INFINITY ? 0.f : exp2_f(ms - mx);
    l = fmaf(sp[Mq + row], wgt, l);
    a += *reinterpret_cast<const f32x4*>(sp + 2 * Mq + int64_t(row) * D + e4) * wgt;
  }
  const float il = 1.0f / l;
  const int i = row / G, hq = h * G + row % G;
  uint16_t* orow = out + ((int64_t(c) * (B + 1) + i) * Hq + hq) * D + e4;
#pragma unroll
  for (int r = 0; r < 4; ++r) orow[r] = f32_to_bf16(a[r] * il);
}

// generic path (f32, small shapes): one workgroup per (c, verified row i, hq)
template <int D>
__global__ __launch_bounds__(kThreads) void attn_generic(
    const float* __restrict__ kc, const float* __restrict__ vc, int64_t rows_stride,
    const int32_t* __restrict__ Lctx, int max_rows, const float* __restrict__ q,
    float* __restrict__ out, int Hq, int Hkv, int B, int32_t* __restrict__ err_flag) {
  __shared__ float qs[D];
  __shared__ float sc[kThreads];
  __shared__ float red[kThreads / 64];
  const int hq = blockIdx.x % Hq;
  const int i = (blockIdx.x / Hq) % (B + 1);
  const int c = blockIdx.x / (Hq * (B + 1));
  const int h = hq / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int L = context_rows(Lctx, c, B, max_rows, err_flag, i == 0 && hq == 0 && tid == 0);
  const int n = L + i + 1;  // causal: rows 0..L+i
  const float sm_scale = 1.0f / sqrtf(float(D));
  const int64_t qo = ((int64_t(c) * (B + 1) + i) * Hq + hq) * D;
  for (int e = tid; e < D; e += kThreads) qs[e] = q[qo + e];
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  __syncthreads();
  for (int k0 = 0; k0 < n; k0 += kThreads) {
    const int key = k0 + tid;
    float a = -INFINITY;
    if (key < n) {
      const float* kr = kc + ((int64_t(c) * rows_stride + key) * Hkv + h) * D;
      float dot = 0.f;
      for (int e = 0; e < D; ++e) dot = fmaf(qs[e], kr[e], dot);
      a = dot * sm_scale;
    }
    float mx = wave_max(a);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, mx);
    const float scale = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
    const float p = __expf(a - m_new);
    sc[tid] = p;
    float ps = wave_sum(p);
    if ((tid & 63) == 0) red[tid >> 6] = ps;
    __syncthreads();
    ps = red[0] + red[1] + red[2] + red[3];
    l_run = l_run * scale + ps;
    m_run = m_new;
    if (tid < D) {
      o *= scale;
      const int nk = min(kThreads, n - k0);
      for (int k = 0; k < nk; ++k)
        o = fmaf(sc[k], vc[((int64_t(c) * rows_stride + k0 + k) * Hkv + h) * D + tid], o);
    }
    __syncthreads();
  }
  if (tid < D) out[qo + tid] = o / l_run;
}

template <int NW>
ls_status launch_mfma(const ls_dims& d, const void* kc, const void* vc, int64_t rows_stride,
                      const int32_t* L, int32_t max_rows, const void* q, void* out, char* ws,
                      int32_t* err_flag, hipStream_t stream) {
  const int units = d.C * d.Hkv;
  const int nsplit = attn_splits(d, max_rows);
  const int rows = attn_rows_per_split(d, max_rows);
  const WsLayout lay = ws_layout(d, std::max<int32_t>(1, max_rows - d.B - 1));
  float* part = reinterpret_cast<float*>(ws + lay.attn_part);
  hipLaunchKernelGGL((attn_mfma_partial<NW>), dim3(units * nsplit), dim3(64 * NW), 0, stream,
                     static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), rows_stride,
                     L, max_rows, static_cast<const uint16_t*>(q), d.Hq, d.Hkv, d.B, rows, nsplit,
                     part, err_flag);
  if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
  const int Mq = 16 * NW;
  const int64_t threads = int64_t(units) * Mq * (128 / 4);
  hipLaunchKernelGGL(attn_combine, dim3(unsigned(cdiv(threads, kThreads))), dim3(kThreads), 0, stream,
                     part, static_cast<uint16_t*>(out), d.Hq, d.Hkv, d.B, nsplit, Mq, units);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

template <int D>
ls_status launch_generic(const ls_dims& d, const void* kc, const void* vc, int64_t rows_stride,
                         const int32_t* L, int32_t max_rows, const void* q, void* out,
                         int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL((attn_generic<D>), dim3(d.C * (d.B + 1) * d.Hq), dim3(kThreads), 0, stream,
                     static_cast<const float*>(kc), static_cast<const float*>(vc), rows_stride, L,
                     max_rows, static_cast<const float*>(q), static_cast<float*>(out), d.Hq, d.Hkv,
                     d.B, err_flag);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

ls_status launch_verify_attention(const ls_dims& d, const void* k_cache, const void* v_cache,
                                  int64_t rows_stride, const int32_t* L, int32_t max_rows,
                                  const void* q, void* out, char* ws, int32_t* err_flag,
                                  hipStream_t stream) {
  if (d.dtype == LS_BF16) {
    switch (attn_query_rows(d) / 16) {  // one wave per 16 query rows
      case 1: return launch_mfma<1>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 2: return launch_mfma<2>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 3: return launch_mfma<3>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 4: return launch_mfma<4>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 5: return launch_mfma<5>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 6: return launch_mfma<6>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 7: return launch_mfma<7>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
      case 8: return launch_mfma<8>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, ws, err_flag, stream);
    }
    return LS_ERR_SHAPE;
  }
  switch (d.d) {
    case 16: return launch_generic<16>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, err_flag, stream);
    case 32: return launch_generic<32>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, err_flag, stream);
    case 64: return launch_generic<64>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, err_flag, stream);
    case 128: return launch_generic<128>(d, k_cache, v_cache, rows_stride, L, max_rows, q, out, err_flag, stream);
  }
  return LS_ERR_SHAPE;
}

}  // namespace ls
