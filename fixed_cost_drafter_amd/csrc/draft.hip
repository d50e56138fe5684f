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
// bf16, d = 128: one workgroup per (KV head unit, 32 query rows), so a
// Qwen3-8B-shaped layer at C = 16 (128 units x 64 rows) fills 256 CUs.  Its
// waves split the key range in parts that stream through LDS in parallel and
// merge (m, l, O) in LDS at the end: no partials leave the workgroup, no
// second launch.  The online softmax lives in registers (per query row).
// f32: one workgroup per query row, plain LDS loop (small shapes).
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;

// launch shape of the bf16 kernel: query row groups of 16 per workgroup, key
// parts per workgroup, keys per part per step (overridable for tuning builds)
#ifndef LS_DRAFT_RG
#define LS_DRAFT_RG 2
#endif
#ifndef LS_DRAFT_KQ
#define LS_DRAFT_KQ 4
#endif
#ifndef LS_DRAFT_TK
#define LS_DRAFT_TK 32
#endif

// Where the keys of one (sequence, KV head) live: [ring | slots | block].
struct KeySources {
  const uint16_t *ring_k, *ring_v;
  const int32_t* ring_pos;
  const uint16_t *slot_k, *slot_v, *kb, *vb;
  int W, S, B, Hkv, c, h, unit;
};

// Branch-free staging loads of NL keys (pairs 2rp, 2rp+1 every STEP keys from
// t0): each key's source row is chosen with integer selects and all loads
// issue back to back.  A key past `end` reads row 0 of the unit's window
// (valid memory).  Validity is NOT decided here: `kpos` keeps the raw ring
// position (or a marker) and `key_state` says how to read it, so nothing
// waits on these loads until the tile is staged into LDS one step later.
// An empty ring row holds zeros (written by init) and is masked there.
template <int NL, int STEP>
__device__ __forceinline__ void load_keys(u16x8 (&kr)[NL], u16x8 (&vr)[NL], int (&kpos)[NL],
                                          int (&key_state)[NL], const KeySources s, int t0,
                                          int end, int rp, int dg) {
  constexpr int D = 128;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int key_raw = t0 + (i >> 1) * STEP + 2 * rp + (i & 1);
    const bool live = key_raw < end;
    const int key = live ? key_raw : 0;
    const bool in_ring = key < s.W, in_slots = !in_ring && key < s.W + s.S;
    const int row = in_ring ? s.unit * s.W + key
                  : in_slots ? s.unit * s.S + (key - s.W)
                             : (s.c * s.B + (key - s.W - s.S)) * s.Hkv + s.h;
    const int64_t off = int64_t(row) * D + dg * 8;
    const uint16_t* kbase = in_ring ? s.ring_k : (in_slots ? s.slot_k : s.kb);
    const uint16_t* vbase = in_ring ? s.ring_v : (in_slots ? s.slot_v : s.vb);
    kr[i] = *reinterpret_cast<const u16x8*>(kbase + off);
    vr[i] = *reinterpret_cast<const u16x8*>(vbase + off);
    kpos[i] = s.ring_pos[s.c * s.W + (in_ring ? key : 0)];
    key_state[i] = !live ? 0 : (in_ring ? 1 : 2);  // 0 dead, 1 ring (check pos), 2 always valid
  }
}

// bf16, d = 128.  Workgroup = (KV head unit, half of the query tile: 32 rows
// = 2 row groups of 16).  Its 8 waves are 2 row groups x KQ key parts; part
// q streams keys [q*Np, (q+1)*Np) in tiles of TK through its own LDS tile
// (row-major K, transposed V), then the parts' (m, l, O) merge in LDS.
// 128 threads stage one part's tile: 16 lanes cover one 256-byte key row.
template <int RG, int KQ, int TK>
__global__ __launch_bounds__(64 * RG * KQ, 1) void draft_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ ring_k,
    const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ring_pos,
    const uint16_t* __restrict__ slot_k, const uint16_t* __restrict__ slot_v,
    uint16_t* __restrict__ out, int Hq, int Hkv, int W, int S, int B, int units) {
  constexpr int D = 128;
  constexpr int KLS = D + 8, VTS = TK + 4;
  constexpr int MB = TK / 16, KS = TK / 32;
  constexpr int PT = 64 * RG;               // threads staging one part's tile
  constexpr int PAIRS = TK / (8 * RG);      // key pairs staged per thread
  static_assert(PAIRS >= 1 && TK % (8 * RG) == 0, "tile must cover the staging threads");
  constexpr int PART_ELEMS = TK * KLS + D * VTS;  // bf16 elements of one part's tile
  static_assert(TK % 32 == 0, "tile must hold whole 32-key MFMA k-steps");
  __shared__ __attribute__((aligned(16))) uint16_t tiles[KQ * PART_ELEMS];
  __shared__ int kvalid[KQ][TK];

  const int rh = blockIdx.x / units;  // which (16*RG)-row slice of the query tile
  const int unit = blockIdx.x % units;
  const int c = unit / Hkv, h = unit % Hkv;
  const int G = Hq / Hkv, M = B * G;
  const int N = W + S + B;
  const int Np = ((N + KQ - 1) / KQ + TK - 1) / TK * TK;  // keys per part, whole tiles
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int rg = wave % RG, part = wave / RG;
  const float sm_scale = 0.08838834764831845f;  // 1/sqrt(128)

  // query operand: lane (row ln of this wave's group, kg) holds q[row][ks*32+kg*8..+7]
  const int row = (rh * RG + rg) * 16 + ln;
  const bool row_ok = row < M;
  const int b = row_ok ? row / G : 0;
  const int hq = h * G + (row_ok ? row % G : 0);
  const bool group_active = (rh * RG + rg) * 16 < M;
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

  // staging: thread (lpart, dg, rp) loads keys 2rp, 2rp+1 (+ 8*RG*k) of part lpart
  const int lpart = tid / PT;
  const int dg = tid & 15, rp = (tid % PT) >> 4;
  const int p_begin = lpart * Np;
  const int p_end = min(N, p_begin + Np);
  u16x8 kr[2 * PAIRS] = {}, vr[2 * PAIRS] = {};
  int kpos[2 * PAIRS] = {}, kstate[2 * PAIRS] = {};
  const KeySources src{ring_k, ring_v, ring_pos, slot_k, slot_v, kb, vb, W, S, B, Hkv, c, h, unit};

  uint16_t* myKL = tiles + lpart * PART_ELEMS;   // staged by this thread
  uint16_t* myVT = myKL + TK * KLS;
  const uint16_t* KL = tiles + part * PART_ELEMS;  // read by this wave
  const uint16_t* VT = KL + TK * KLS;
  const int steps = Np / TK;
  const int w_begin = part * Np;

  load_keys<2 * PAIRS, 8 * RG>(kr, vr, kpos, kstate, src, p_begin, p_end, rp, dg);
  for (int st = 0; st < steps; ++st) {
    __syncthreads();  // the previous tiles' LDS reads are done
#pragma unroll
    for (int i = 0; i < 2 * PAIRS; ++i) {
      const int r = (i >> 1) * (8 * RG) + 2 * rp + (i & 1);
      *reinterpret_cast<u16x8*>(&myKL[r * KLS + dg * 8]) = kr[i];
      if (dg == 0) kvalid[lpart][r] = kstate[i] == 2 || (kstate[i] == 1 && kpos[i] >= 0);
    }
#pragma unroll
    for (int pp = 0; pp < PAIRS; ++pp) {
      const int r0 = pp * (8 * RG) + 2 * rp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t vv = uint32_t(vr[2 * pp][e]) | (uint32_t(vr[2 * pp + 1][e]) << 16);
        *reinterpret_cast<uint32_t*>(&myVT[(dg * 8 + e) * VTS + r0]) = vv;
      }
    }
    __syncthreads();
    if (st + 1 < steps)  // next tile in flight during compute
      load_keys<2 * PAIRS, 8 * RG>(kr, vr, kpos, kstate, src, p_begin + (st + 1) * TK, p_end,
                                   rp, dg);
    if (!group_active || w_begin + st * TK >= N) continue;

    // S^T[key][row]: lane (row ln, kg) holds keys mb*16 + kg*4 + r
    f32x4 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const u16x8*>(&KL[(mb * 16 + ln) * KLS + ks * 32 + kg * 8]));
        s[mb] = mfma16x16x32(a, qb[ks], s[mb]);
      }

    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = s[mb][r] * sm_scale;
        if (!kvalid[part][mb * 16 + kg * 4 + r]) a = -INFINITY;
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
    u16x8 pv[KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint16_t pb = f32_to_bf16(exp_f(s[mb][r] - m_use));
        lsum += bf16_to_f32(pb);
        pv[mb >> 1][(mb & 1) * 4 + r] = pb;
      }
    l_run = fmaf(l_run, scale, lsum);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= scale;

    // O^T[dim][row] += V^T[dim][key] P^T[key][row]; the A operand's k order
    // (keys 32ks+4kg..+3, 32ks+16+4kg..+3) matches pv's element order
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 pk = as_bf16x8(pv[ks]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const uint16_t* base = &VT[(mb * 16 + ln) * VTS + ks * 32 + kg * 4];
        const u16x4 lo = *reinterpret_cast<const u16x4*>(base);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(base + 16);
        const bf16x8 a = as_bf16x8(u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        o[mb] = mfma16x16x32(a, pk, o[mb]);
      }
    }
  }

  float lt = l_run;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);

  // merge the key parts in LDS (reusing the tile buffers): parts 1..KQ-1
  // publish (m, l, O) in the same lane layout, part 0 combines and writes
  __syncthreads();
  float* red = reinterpret_cast<float*>(tiles);  // [KQ-1][RG groups][64 lanes][34]
  static_assert((KQ - 1) * RG * 64 * 34 * 4 <= KQ * PART_ELEMS * 2, "merge area fits the tiles");
  if (part > 0 && group_active) {
    float* dst = red + (((part - 1) * RG + rg) * 64 + lane) * 34;
    dst[0] = m_run;
    dst[1] = lt;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[2 + mb * 4 + r] = o[mb][r];
  }
  __syncthreads();
  if (part == 0 && row_ok) {
    float mx = m_run;
#pragma unroll
    for (int p2 = 1; p2 < KQ; ++p2) mx = fmaxf(mx, red[(((p2 - 1) * RG + rg) * 64 + lane) * 34]);
    const float w0 = m_run == -INFINITY ? 0.f : exp_f(m_run - mx);
    float l = lt * w0;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= w0;
#pragma unroll
    for (int p2 = 1; p2 < KQ; ++p2) {
      const float* src = red + (((p2 - 1) * RG + rg) * 64 + lane) * 34;
      const float wq = src[0] == -INFINITY ? 0.f : exp_f(src[0] - mx);
      l = fmaf(src[1], wq, l);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[mb][r] = fmaf(src[2 + mb * 4 + r], wq, o[mb][r]);
    }
    const float il = 1.0f / l;
    uint16_t* orow = out + ((int64_t(c) * B + b) * Hq + hq) * D;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *reinterpret_cast<u16x4*>(orow + mb * 16 + kg * 4) =
          u16x4{f32_to_bf16(o[mb][0] * il), f32_to_bf16(o[mb][1] * il),
                f32_to_bf16(o[mb][2] * il), f32_to_bf16(o[mb][3] * il)};
  }
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
    constexpr int RG = LS_DRAFT_RG, KQ = LS_DRAFT_KQ, TK = LS_DRAFT_TK;
    const int units = d.C * d.Hkv;
    const int M = d.B * (d.Hq / d.Hkv);
    const int slices = int(cdiv(M, 16 * RG));
    hipLaunchKernelGGL((draft_mfma<RG, KQ, TK>), dim3(units * slices), dim3(64 * RG * KQ), 0,
                       stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kb),
                       static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(st.ring_k),
                       static_cast<const uint16_t*>(st.ring_v), st.ring_pos,
                       static_cast<const uint16_t*>(st.slot_k),
                       static_cast<const uint16_t*>(st.slot_v), static_cast<uint16_t*>(out), d.Hq,
                       d.Hkv, d.W, d.S, d.B, units);
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
