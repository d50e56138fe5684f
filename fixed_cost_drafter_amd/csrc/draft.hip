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
// bf16, d = 128: one workgroup per (KV head unit, key split).  4 waves own 16
// query rows each; key tiles of 64 are staged in LDS (row-major K for the
// S^T = K Q^T MFMA, transposed V for the O^T += V^T P^T MFMA); the online
// softmax lives in registers (per query row, per lane).  Splits write
// (m, l, O) partials and the last split of a unit to finish merges them.
// Workgroup index = split * units + unit, so with units % 8 == 0 all splits
// of one unit land on the same XCD and share its L2.
// f32: one workgroup per query row, plain LDS loop (small shapes).
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads, 2) void draft_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ ring_k,
    const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ring_pos,
    const uint16_t* __restrict__ slot_k, const uint16_t* __restrict__ slot_v,
    uint16_t* __restrict__ out, float* __restrict__ part, uint32_t* __restrict__ counter,
    int Hq, int Hkv, int W, int S, int B, int nsplit, int keys_per_split) {
  constexpr int D = 128, TK = 64;
  constexpr int KLS = D + 8, VTS = TK + 4;
  __shared__ __attribute__((aligned(16))) uint16_t KL[TK * KLS];
  __shared__ __attribute__((aligned(16))) uint16_t VT[D * VTS];
  __shared__ int kvalid[TK];
  __shared__ int is_last;

  const int units = gridDim.x / nsplit;
  const int split = blockIdx.x / units;
  const int unit = blockIdx.x % units;
  const int c = unit / Hkv, h = unit % Hkv;
  const int G = Hq / Hkv, M = B * G;
  const int N = W + S + B;
  const int k_begin = split * keys_per_split;
  const int k_end = min(N, k_begin + keys_per_split);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const float sm_scale = 0.08838834764831845f;  // 1/sqrt(128)

  // query operand: lane (row ln of this wave, kg) holds q[row][ks*32+kg*8..+7]
  const int row = wave * 16 + ln;
  const bool row_ok = row < M;
  const int b = row_ok ? row / G : 0;
  const int hq = h * G + (row_ok ? row % G : 0);
  const bool wave_active = wave * 16 < M;
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (row_ok)
      v = *reinterpret_cast<const u16x8*>(q + ((int64_t(c) * B + b) * Hq + hq) * D + ks * 32 +
                                          kg * 8);
    qb[ks] = as_bf16x8(v);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int dg = tid & 15, rp = tid >> 4;
  u16x8 kr[4], vr[4];
  int kv_ok[4];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t0 + (i >> 1) * 32 + 2 * rp + (i & 1);
      const uint16_t* ks = nullptr;
      const uint16_t* vs = nullptr;
      bool ok = false;
      if (key < k_end) {
        if (key < W) {
          ok = ring_pos[int64_t(c) * W + key] >= 0;
          const int64_t off = (int64_t(unit) * W + key) * D;
          ks = ring_k + off;
          vs = ring_v + off;
        } else if (key < W + S) {
          ok = true;
          const int64_t off = (int64_t(unit) * S + (key - W)) * D;
          ks = slot_k + off;
          vs = slot_v + off;
        } else {
          ok = true;
          const int64_t off = ((int64_t(c) * B + (key - W - S)) * Hkv + h) * D;
          ks = kb + off;
          vs = vb + off;
        }
      }
      kv_ok[i] = ok;
      if (ok) {
        kr[i] = *reinterpret_cast<const u16x8*>(ks + dg * 8);
        vr[i] = *reinterpret_cast<const u16x8*>(vs + dg * 8);
      } else {
        kr[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        vr[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };

  if (k_begin < k_end) load_tile(k_begin);
  for (int t0 = k_begin; t0 < k_end; t0 += TK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (i >> 1) * 32 + 2 * rp + (i & 1);
      *reinterpret_cast<u16x8*>(&KL[r * KLS + dg * 8]) = kr[i];
      if (dg == 0) kvalid[r] = kv_ok[i];
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r0 = half * 32 + 2 * rp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t vv = uint32_t(vr[2 * half][e]) | (uint32_t(vr[2 * half + 1][e]) << 16);
        *reinterpret_cast<uint32_t*>(&VT[(dg * 8 + e) * VTS + r0]) = vv;
      }
    }
    __syncthreads();
    if (t0 + TK < k_end) load_tile(t0 + TK);
    if (!wave_active) continue;

    // S^T[key][row]: lane (row ln, kg) holds keys mb*16 + kg*4 + r
    f32x4 s[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const u16x8*>(&KL[(mb * 16 + ln) * KLS + ks * 32 + kg * 8]));
        s[mb] = mfma16x16x32(a, qb[ks], s[mb]);
      }

    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = mb * 16 + kg * 4 + r;
        float a = s[mb][r] * sm_scale;
        if (!kvalid[key]) a = -INFINITY;
        s[mb][r] = a;
        tmax = fmaxf(tmax, a);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float scale = m_run == -INFINITY ? 0.f : exp_f(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
    u16x8 pv[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint16_t pb = f32_to_bf16(exp_f(s[mb][r] - m_use));
        lsum += bf16_to_f32(pb);
        pv[mb >> 1][(mb & 1) * 4 + r] = pb;
      }
    l_run = fmaf(l_run, scale, lsum);
    const bf16x8 pk0 = as_bf16x8(pv[0]), pk1 = as_bf16x8(pv[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= scale;

    // O^T[dim][row] += V^T[dim][key] P^T[key][row]
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint16_t* base = &VT[(mb * 16 + ln) * VTS + ks * 32 + kg * 4];
        const u16x4 lo = *reinterpret_cast<const u16x4*>(base);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(base + 16);
        const bf16x8 a = as_bf16x8(u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        o[mb] = mfma16x16x32(a, ks == 0 ? pk0 : pk1, o[mb]);
      }
  }

  float lt = l_run;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);

  if (nsplit == 1) {
    if (row_ok) {
      const float il = 1.0f / lt;
      uint16_t* orow = out + ((int64_t(c) * B + b) * Hq + hq) * D;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) orow[mb * 16 + kg * 4 + r] = f32_to_bf16(o[mb][r] * il);
    }
    return;
  }

  // partial of this split: pm[Mpad] | pl[Mpad] | po[Mpad][D]
  const int Mpad = (M + 15) & ~15;
  const int64_t pstride = int64_t(Mpad) * (D + 2);
  float* pb = part + (int64_t(unit) * nsplit + split) * pstride;
  if (wave_active) {
    if (kg == 0) {
      pb[row] = m_run;
      pb[Mpad + row] = lt;
    }
    float* po = pb + 2 * Mpad + int64_t(row) * D;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(po + mb * 16 + kg * 4) = o[mb];
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t ticket = atomicAdd(&counter[unit], 1u);
    is_last = ticket == uint32_t(nsplit - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // merge the splits of this unit
  const float* ub = part + int64_t(unit) * nsplit * pstride;
  for (int p = tid; p < M * (D / 4); p += kThreads) {
    const int r = p / (D / 4), e4 = (p % (D / 4)) * 4;
    float mx = -INFINITY;
    for (int s2 = 0; s2 < nsplit; ++s2) mx = fmaxf(mx, __builtin_nontemporal_load(ub + s2 * pstride + r));
    float l = 0.f;
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < nsplit; ++s2) {
      const float* sp = ub + s2 * pstride;
      const float ms = __builtin_nontemporal_load(sp + r);
      const float wgt = ms == -INFINITY ? 0.f : exp_f(ms - mx);
      l = fmaf(__builtin_nontemporal_load(sp + Mpad + r), wgt, l);
      const f32x4 ov = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(sp + 2 * Mpad + int64_t(r) * D + e4));
      a += ov * wgt;
    }
    const float il = 1.0f / l;
    const int bb = r / G, hh = h * G + r % G;
    uint16_t* orow = out + ((int64_t(c) * B + bb) * Hq + hh) * D + e4;
    u16x4 ob = u16x4{f32_to_bf16(a[0] * il), f32_to_bf16(a[1] * il), f32_to_bf16(a[2] * il),
                     f32_to_bf16(a[3] * il)};
    *reinterpret_cast<u16x4*>(orow) = ob;
  }
  if (tid == 0) counter[unit] = 0u;
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

  auto key_ptr = [&](int key, bool vals, bool& ok) -> const typename Ty::T* {
    ok = true;
    if (key < W) {
      ok = ring_pos[int64_t(c) * W + key] >= 0;
      return (vals ? ring_v : ring_k) + (int64_t(unit) * W + key) * D;
    }
    if (key < W + S) return (vals ? slot_v : slot_k) + (int64_t(unit) * S + key - W) * D;
    return (vals ? vb : kb) + ((int64_t(c) * B + key - W - S) * Hkv + h) * D;
  };

  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  __syncthreads();
  for (int k0 = 0; k0 < N; k0 += kThreads) {
    const int key = k0 + tid;
    float a = -INFINITY;
    if (key < N) {
      bool ok;
      const typename Ty::T* kp = key_ptr(key, false, ok);
      if (ok) {
        float dot = 0.f;
        for (int e = 0; e < D; ++e) dot = fmaf(qs[e], Ty::load(kp, e), dot);
        a = dot * sm_scale;
      }
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
        if (pk != 0.f) {
          bool ok;
          const typename Ty::T* vp = key_ptr(k0 + k, true, ok);
          o = fmaf(pk, Ty::load(vp, tid), o);
        }
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
    const WsLayout lay = ws_layout(d, 1);
    const int N = d.W + d.S + d.B;
    const int kps = int(cdiv(cdiv(N, lay.dsplit), 64) * 64);
    const int nsplit = int(cdiv(N, kps));  // <= lay.dsplit
    const int units = d.C * d.Hkv;
    char* ws = static_cast<char*>(st.workspace);
    hipLaunchKernelGGL(draft_mfma, dim3(units * nsplit), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kb),
                       static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(st.ring_k),
                       static_cast<const uint16_t*>(st.ring_v), st.ring_pos,
                       static_cast<const uint16_t*>(st.slot_k),
                       static_cast<const uint16_t*>(st.slot_v), static_cast<uint16_t*>(out),
                       reinterpret_cast<float*>(ws + lay.draft_part),
                       reinterpret_cast<uint32_t*>(ws + lay.cnt_draft), d.Hq, d.Hkv, d.W, d.S,
                       d.B, nsplit, kps);
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
