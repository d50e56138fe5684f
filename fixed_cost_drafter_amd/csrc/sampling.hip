// Sampled verification of a drafted block (LongSpark paper page, Table 1:
// accepted lengths with sampling at temperature 1; Table 3 is the greedy
// case).  The pages do not print the rule; this is the textbook
// speculative-sampling rule:
//   p_j = softmax(target row j / T), q_j = softmax(drafter row j / T);
//   draft j is accepted when u_accept[j] * q_j(d_j) < p_j(d_j);
//   at the first rejection j the emitted token is drawn from max(0, p_j - q_j)
//   (from p_j when that residual is zero everywhere), after B acceptances
//   from p_B; the draw is the inverse CDF over the
//   vocabulary in index order: the smallest k whose running sum exceeds
//   u_sample times the total.
//
// Three launches, kernel boundaries between them (no device-scope fences):
//  (1) samp_stats: (row, 8192-logit chunk) workgroups stream both logit
//      tensors once and reduce each chunk to base-2 softmax statistics
//      (max of x log2(e) / T, sum of 2^(y - max));
//  (2) samp_decide_sums: (chunk, sequence) workgroups; each merges its
//      sequence's 2B+1 rows' statistics (a wave per row, a lane per chunk),
//      gathers p_j(d_j), q_j(d_j) and runs the acceptance rule, then sums
//      the weights of the row to draw from over its chunk;
//  (3) samp_draw: one workgroup per sequence locates the chunk, then (a
//      workgroup scan over per-thread sums of 32 entries held in registers)
//      the thread, then the entry where the running sum crosses u_sample
//      times the total.
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) += (m2, s2) for base-2 softmax statistics (s = sum of 2^(y - m))
__device__ __forceinline__ void merge_stat(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;
  s = s * exp2_f(m - mx) + s2 * exp2_f(m2 - mx);
  m = mx;
}

__device__ __forceinline__ void wave_merge_stat(float& m, float& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    merge_stat(m, s, m2, s2);
  }
}

template <typename Ty>
struct Vec16;  // 16 bytes of logits
template <>
struct Vec16<F32> {
  static constexpr int N = 4;
  using V = float __attribute__((ext_vector_type(4)));
  __device__ static inline float get(const V& v, int i) { return v[i]; }
};
template <>
struct Vec16<BF16> {
  static constexpr int N = 8;
  using V = u16x8;
  __device__ static inline float get(const V& v, int i) { return bf16_to_f32(v[i]); }
};

// per-sequence record of the decision (written by the chunk-0 workgroup)
struct Record {
  int32_t row;   // j: the verified row the emitted token is drawn from
  int32_t bonus; // 1: drawn from p_B (all drafts accepted), 0: from max(0, p_j - q_j)
  float mt, izt; // target row j: max and 1 / sum (base 2)
  float md, izd; // drafter row j (residual draw only)
  float pad[2];
};
static_assert(sizeof(Record) == 32, "one 32-byte record per sequence");

template <typename Ty>
__global__ __launch_bounds__(kThreads) void samp_stats(
    const typename Ty::T* __restrict__ tl, const typename Ty::T* __restrict__ dl,
    float2* __restrict__ stats, int C, int B, int V, int nsplit, float k2, int vec_ok) {
  using VT = Vec16<Ty>;
  const int split = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int nt = C * (B + 1);
  const typename Ty::T* x = r < nt ? tl + int64_t(r) * V : dl + int64_t(r - nt) * V;
  const int begin = split * kVerifyChunk, end = min(V, begin + kVerifyChunk);
  float m = -INFINITY, s = 0.f;
  if (vec_ok) {
    const typename VT::V* xv = reinterpret_cast<const typename VT::V*>(x + begin);
    const int nvec = (end - begin) / VT::N;
    constexpr int U = (kVerifyChunk / VT::N + kThreads - 1) / kThreads;
    typename VT::V buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = u * kThreads + tid;
      if (v < nvec) buf[u] = __builtin_nontemporal_load(xv + v);
    }
    float bm = -INFINITY;  // batch max, then one rescale
    if constexpr (Ty::kBytes == 2) {
      // bf16: the max over packed 16-bit order keys (two logits per
      // instruction), converted back to a value once
      typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
      typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
      u16x2 best = {0, 0};  // 0: below every key of a real value
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u * kThreads + tid < nvec) {
          const uint4 w4 = __builtin_bit_cast(uint4, buf[u]);
          const uint32_t ws4[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const i16x2 h = __builtin_bit_cast(i16x2, ws4[q]);
            const u16x2 flip = __builtin_bit_cast(u16x2, i16x2(h >> 15)) | u16x2{0x8000, 0x8000};
            best = __builtin_elementwise_max(best, __builtin_bit_cast(u16x2, ws4[q]) ^ flip);
          }
        }
      const uint32_t key = max(uint32_t(best[0]), uint32_t(best[1]));
      if (key != 0u) {
        const uint32_t hb = key >= 0x8000u ? (key ^ 0x8000u) : (~key & 0xFFFFu);
        bm = bf16_to_f32(uint16_t(hb)) * k2;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u * kThreads + tid < nvec)
#pragma unroll
          for (int e = 0; e < VT::N; ++e) bm = fmaxf(bm, VT::get(buf[u], e) * k2);
    }
    float bs = 0.f;
    const float nbm = bm == -INFINITY ? 0.f : -bm;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u * kThreads + tid < nvec)
#pragma unroll
        for (int e = 0; e < VT::N; ++e) bs += exp2_f(fmaf(VT::get(buf[u], e), k2, nbm));
    merge_stat(m, s, bm, bs);
    for (int i = begin + nvec * VT::N + tid; i < end; i += kThreads)
      merge_stat(m, s, Ty::load(x, i) * k2, 1.f);
  } else {
    for (int i = begin + tid; i < end; i += kThreads) merge_stat(m, s, Ty::load(x, i) * k2, 1.f);
  }
  wave_merge_stat(m, s);
  __shared__ float wm[kThreads / 64], ws[kThreads / 64];
  if ((tid & 63) == 0) { wm[tid >> 6] = m; ws[tid >> 6] = s; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w) merge_stat(m, s, wm[w], ws[w]);
    stats[int64_t(r) * nsplit + split] = make_float2(m, s);
  }
}

// weight of vocabulary entry k in the draw of a record's row.  p and q are
// each rounded before the difference: a fused multiply-subtract would leave
// the rounding error of one product where p == q, and an identically zero
// residual must stay zero (the draw then falls back to p_j).
template <typename Ty>
__device__ __forceinline__ float draw_weight(const typename Ty::T* rt, const typename Ty::T* rd,
                                             const Record& r, float k2, int k) {
#pragma clang fp contract(off)
  const float p = exp2_f(Ty::load(rt, k) * k2 - r.mt) * r.izt;
  if (r.bonus) return p;
  const float q = exp2_f(Ty::load(rd, k) * k2 - r.md) * r.izd;
  return fmaxf(p - q, 0.f);
}

// weights of the N logits of one 16-byte vector of the drawn row (vt: target
// logits, vd: drafter logits, unused for a bonus draw)
template <typename Ty>
__device__ __forceinline__ void draw_weights16(const typename Vec16<Ty>::V& vt, const typename Vec16<Ty>::V& vd,
                                               const Record& r, float k2, float* w) {
#pragma clang fp contract(off)
  using VT = Vec16<Ty>;
#pragma unroll
  for (int e = 0; e < VT::N; ++e) {
    const float p = exp2_f(VT::get(vt, e) * k2 - r.mt) * r.izt;
    w[e] = r.bonus ? p : fmaxf(p - exp2_f(VT::get(vd, e) * k2 - r.md) * r.izd, 0.f);
  }
}

// (chunk, sequence) workgroups.  Every workgroup of sequence c first takes
// the acceptance decision of c itself (the same loads and arithmetic in
// each, so the same result): wave w merges the chunk statistics of target
// rows w, w + 4, ... and of the drafter rows of the same index (a lane per
// chunk, all loads issued before the first merge), with p_j(d_j) and
// q_j(d_j) gathered by lane i for row w + 4i; thread 0 runs the rule.  The
// chunk-0 workgroup writes tau, the accepted drafts and the record that the
// draw reads.  Then each workgroup sums the drawn row's weights over its
// chunk, all 16-byte loads of a thread in flight at once.
template <typename Ty>
__global__ __launch_bounds__(kThreads) void samp_decide_sums(
    const typename Ty::T* __restrict__ tl, const typename Ty::T* __restrict__ dl,
    const int32_t* __restrict__ draft, const float* __restrict__ u_accept,
    const float2* __restrict__ stats, Record* __restrict__ rec, int32_t* __restrict__ tokens,
    int32_t* __restrict__ tau, float* __restrict__ sums, int C, int B, int V, int nsplit,
    float k2, int vec_ok) {
  using VT = Vec16<Ty>;
  constexpr int kW = kThreads / 64;
  constexpr int kRows = (kMaxBlock + 1 + kW - 1) / kW;  // rows per wave
  static_assert(kRows <= 64, "a lane per row for the gathers");
  __shared__ float pt[64], qd[64], mt[64], izt[64], md[64], izd[64], ua[64];
  __shared__ Record s_rec;
  __shared__ int s_js;
  const int split = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63,
            wave = tid >> 6;
  const int nt = C * (B + 1);

  // the decision's loads: chunk statistics (lane = chunk) and, in lane i,
  // the drafted token's logits of row wave + kW i
  float2 ts[kRows], ds[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int j = wave + kW * i;
    ts[i] = make_float2(-INFINITY, 0.f);
    ds[i] = make_float2(-INFINITY, 0.f);
    if (j <= B && lane < nsplit) ts[i] = stats[(int64_t(c) * (B + 1) + j) * nsplit + lane];
    if (j < B && lane < nsplit) ds[i] = stats[(int64_t(nt) + int64_t(c) * B + j) * nsplit + lane];
  }
  // the acceptance draws, one per lane, for thread 0's rule below (one
  // round trip instead of a dependent load per drafted position)
  if (tid < B) ua[tid] = u_accept[int64_t(c) * B + tid];
  float xt = 0.f, xd = 0.f;
  {
    const int j = wave + kW * lane;
    if (lane < kRows && j < B) {
      const int d = min(max(draft[int64_t(c) * B + j], 0), V - 1);
      xt = Ty::load(tl, (int64_t(c) * (B + 1) + j) * V + d);
      xd = Ty::load(dl, (int64_t(c) * B + j) * V + d);
    }
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int j = wave + kW * i;
    if (j > B) break;  // uniform in the wave
    float m = -INFINITY, sm = 0.f, m2 = -INFINITY, s2 = 0.f;
    merge_stat(m, sm, ts[i].x, ts[i].y);
    merge_stat(m2, s2, ds[i].x, ds[i].y);
    for (int k = lane + 64; k < nsplit; k += 64) {  // more than 64 chunks: V > 512K
      merge_stat(m, sm, stats[(int64_t(c) * (B + 1) + j) * nsplit + k].x,
                 stats[(int64_t(c) * (B + 1) + j) * nsplit + k].y);
      if (j < B)
        merge_stat(m2, s2, stats[(int64_t(nt) + int64_t(c) * B + j) * nsplit + k].x,
                   stats[(int64_t(nt) + int64_t(c) * B + j) * nsplit + k].y);
    }
    wave_merge_stat(m, sm);
    if (j < B) wave_merge_stat(m2, s2);
    const float yt = __shfl(xt, i), yd = __shfl(xd, i);
    if (lane == 0) {
      mt[j] = m;
      izt[j] = 1.0f / sm;
      if (j < B) {
        md[j] = m2;
        izd[j] = 1.0f / s2;
        pt[j] = exp2_f(yt * k2 - m) * izt[j];
        qd[j] = exp2_f(yd * k2 - m2) * izd[j];
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int j = 0;
    while (j < B && ua[j] * qd[j] < pt[j]) ++j;
    s_js = j;
    Record r;
    r.row = j;
    r.bonus = j == B;
    r.mt = mt[j];
    r.izt = izt[j];
    r.md = j < B ? md[j] : 0.f;
    r.izd = j < B ? izd[j] : 0.f;
    r.pad[0] = r.pad[1] = 0.f;
    s_rec = r;
    if (split == 0) {
      tau[c] = j + 1;
      rec[c] = r;
    }
  }
  __syncthreads();
  const Record r = s_rec;
  if (split == 0) {
    const int js = s_js;
    for (int i = tid; i <= B; i += kThreads)  // accepted drafts, then -1 (token js is drawn later)
      if (i != js) tokens[int64_t(c) * (B + 1) + i] = i < js ? draft[int64_t(c) * B + i] : -1;
  }

  // chunk sum of the drawn row's weights
  constexpr int U = kVerifyChunk / VT::N / kThreads;  // vectors per thread
  const typename Ty::T* rt = tl + (int64_t(c) * (B + 1) + r.row) * V;
  const typename Ty::T* rd = dl + (int64_t(c) * B + min(r.row, B - 1)) * V;
  const int begin = split * kVerifyChunk, end = min(V, begin + kVerifyChunk);
  float a = 0.f;
  if (vec_ok) {
    const typename VT::V* vt = reinterpret_cast<const typename VT::V*>(rt + begin);
    const typename VT::V* vd = reinterpret_cast<const typename VT::V*>(rd + begin);
    const int nvec = (end - begin) / VT::N;  // whole: V is a multiple of N here
    typename VT::V bt[U], bd[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = min(u * kThreads + tid, nvec - 1);
      bt[u] = vt[v];
      bd[u] = r.bonus ? bt[u] : vd[v];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u * kThreads + tid < nvec) {
        float w[VT::N];
        draw_weights16<Ty>(bt[u], bd[u], r, k2, w);
#pragma unroll
        for (int e = 0; e < VT::N; ++e) a += w[e];
      }
  } else {
    for (int k = begin + tid; k < end; k += kThreads) a += draw_weight<Ty>(rt, rd, r, k2, k);
  }
  a = wave_sum(a);
  __shared__ float wsum[kW];
  if (lane == 0) wsum[wave] = a;
  __syncthreads();
  if (tid == 0) sums[int64_t(c) * nsplit + split] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// The draw: one workgroup per sequence.  Thread 0 finds the chunk where the
// running sum of the chunk sums crosses u_sample * total.  Each thread then
// forms the weights of its SEG consecutive entries of that chunk in
// registers; a workgroup scan of the thread totals finds the thread whose
// entries hold the crossing, and that thread walks its registers.  When
// rounding leaves the threshold past the end, the last entry with weight
// is drawn (last non-empty chunk, thread, entry).  A rejection whose residual
// max(0, p_j - q_j) is zero everywhere (p_j == q_j: the drafted token had
// p = q = 0) draws from p_j instead; its chunk sums come from the target
// row's chunk statistics.
// at most 2^20 logits per row (checked by the ABI): the chunks of a row
constexpr int kMaxChunks = ((1 << 20) + kVerifyChunk - 1) / kVerifyChunk;

template <typename Ty>
__global__ __launch_bounds__(kThreads) void samp_draw(
    const typename Ty::T* __restrict__ tl, const typename Ty::T* __restrict__ dl,
    const Record* __restrict__ rec, const float* __restrict__ sums,
    const float2* __restrict__ stats, const float* __restrict__ u_sample,
    int32_t* __restrict__ tokens, int B, int V, int nsplit, float k2, int vec_ok) {
  using VT = Vec16<Ty>;
  constexpr int SEG = kVerifyChunk / kThreads;  // entries per thread
  constexpr int NV = SEG / VT::N;               // 16-byte vectors per thread
  static_assert(SEG % VT::N == 0, "whole vectors per thread");
  __shared__ int s_split, s_bonus;
  __shared__ float s_base, s_thr;
  __shared__ float s_sm[kMaxChunks];
  __shared__ float2 s_st[kMaxChunks];
  __shared__ float wtot[kThreads / 64];
  __shared__ int s_first[kThreads / 64], s_last[kThreads / 64];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Record r = rec[c];
  const typename Ty::T* rt = tl + (int64_t(c) * (B + 1) + r.row) * V;
  const typename Ty::T* rd = dl + (int64_t(c) * B + min(r.row, B - 1)) * V;
  // the chunk sums and the drawn row's chunk statistics, loaded in parallel
  // for thread 0's scan (which adds them in chunk order, as before)
  for (int k = tid; k < nsplit; k += kThreads) {
    s_sm[k] = sums[int64_t(c) * nsplit + k];
    s_st[k] = stats[(int64_t(c) * (B + 1) + r.row) * nsplit + k];
  }
  __syncthreads();
  if (tid == 0) {
    const float* sm = s_sm;
    const float2* st = s_st;
    float total = 0.f;
    for (int k = 0; k < nsplit; ++k) total += sm[k];
    // an empty residual: draw from p_j, whose chunk k holds
    // s_k 2^(m_k - mt) / Z of the probability mass
    const bool from_p = !r.bonus && !(total > 0.f);
    auto chunk = [&](int k) {
      return from_p ? (st[k].x == -INFINITY ? 0.f : st[k].y * exp2_f(st[k].x - r.mt) * r.izt) : sm[k];
    };
    if (from_p) {
      total = 0.f;
      for (int k = 0; k < nsplit; ++k) total += chunk(k);
    }
    const float thr = u_sample[c] * total;
    float run = 0.f;
    int sp = -1, last = 0;
    for (int k = 0; k < nsplit; ++k) {
      const float a = chunk(k);
      if (a > 0.f) last = k;
      if (sp < 0 && run + a > thr) sp = k;
      if (sp < 0) run += a;
    }
    if (sp < 0) {  // rounding left the threshold at the very end: the last non-empty chunk
      sp = last;
      run = 0.f;
      for (int k = 0; k < last; ++k) run += chunk(k);
    }
    s_split = sp;
    s_base = run;
    s_thr = thr;
    s_bonus = from_p ? 1 : r.bonus;
  }
  __syncthreads();
  r.bonus = s_bonus;
  const int begin = s_split * kVerifyChunk, end = min(V, begin + kVerifyChunk);
  const int k0 = begin + tid * SEG;
  float w[SEG];
  if (vec_ok && k0 + SEG <= end) {
    typename VT::V bt[NV], bd[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      bt[i] = *reinterpret_cast<const typename VT::V*>(rt + k0 + i * VT::N);
      bd[i] = r.bonus ? bt[i] : *reinterpret_cast<const typename VT::V*>(rd + k0 + i * VT::N);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) draw_weights16<Ty>(bt[i], bd[i], r, k2, w + i * VT::N);
  } else {
#pragma unroll
    for (int e = 0; e < SEG; ++e) w[e] = k0 + e < end ? draw_weight<Ty>(rt, rd, r, k2, k0 + e) : 0.f;
  }
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < SEG; ++e) a += w[e];
  // inclusive scan of the thread totals over the workgroup
  float incl = a;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  float before = s_base;
  for (int w2 = 0; w2 < wave; ++w2) before += wtot[w2];
  incl += before;                       // running sum up to this thread's last entry
  const float excl = incl - a;          // ... up to its first entry
  const float thr = s_thr;
  const uint64_t cross = __ballot(incl > thr && a > 0.f);
  const uint64_t some = __ballot(a > 0.f);
  if (lane == 0) {
    s_first[wave] = cross ? wave * 64 + __builtin_ctzll(cross) : kThreads;
    s_last[wave] = some ? wave * 64 + 63 - __builtin_clzll(some) : -1;
  }
  __syncthreads();
  int first = kThreads, lastt = -1;
#pragma unroll
  for (int w2 = 0; w2 < kThreads / 64; ++w2) {
    first = min(first, s_first[w2]);
    lastt = max(lastt, s_last[w2]);
  }
  const int pick = first < kThreads ? first : (lastt >= 0 ? lastt : 0);
  if (tid == pick) {
    float run = excl;
    int tok = -1, lst = -1;
#pragma unroll
    for (int e = 0; e < SEG; ++e) {
      if (w[e] > 0.f) lst = e;
      run += w[e];
      if (tok < 0 && run > thr) tok = e;
    }
    const int e = tok >= 0 ? tok : (lst >= 0 ? lst : 0);
    tokens[int64_t(c) * (B + 1) + r.row] = k0 + e;
  }
}

template <typename Ty>
ls_status run(const ls_dims& d, const void* tl, const void* dl, const int32_t* draft, float T,
              const float* u_accept, const float* u_sample, int32_t* tokens, int32_t* tau,
              char* ws, hipStream_t stream) {
  using E = typename Ty::T;
  const WsLayout lay = ws_layout(d, 1);
  const int nsplit = lay.vsplit;
  const float k2 = kLog2e / T;
  auto* stats = reinterpret_cast<float2*>(ws + lay.samp_stats);
  auto* rec = reinterpret_cast<Record*>(ws + lay.samp_seq);
  auto* sums = reinterpret_cast<float*>(ws + lay.samp_sums);
  const E* t = static_cast<const E*>(tl);
  const E* dd = static_cast<const E*>(dl);
  const int vec_ok = ((int64_t(d.V) * Ty::kBytes) % 16 == 0) && ((uintptr_t(tl) & 15) == 0) &&
                     ((uintptr_t(dl) & 15) == 0);
  hipLaunchKernelGGL(samp_stats<Ty>, dim3(nsplit, d.C * (2 * d.B + 1)), dim3(kThreads), 0, stream,
                     t, dd, stats, d.C, d.B, d.V, nsplit, k2, vec_ok);
  if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
  hipLaunchKernelGGL(samp_decide_sums<Ty>, dim3(nsplit, d.C), dim3(kThreads), 0, stream, t, dd, draft,
                     u_accept, stats, rec, tokens, tau, sums, d.C, d.B, d.V, nsplit, k2, vec_ok);
  if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
  hipLaunchKernelGGL(samp_draw<Ty>, dim3(d.C), dim3(kThreads), 0, stream, t, dd, rec, sums, stats,
                     u_sample, tokens, d.B, d.V, nsplit, k2, vec_ok);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

ls_status launch_sampling(const ls_dims& d, const void* target_logits, const void* draft_logits,
                          const int32_t* draft, float temperature, const float* u_accept,
                          const float* u_sample, int32_t* tokens, int32_t* tau, char* ws,
                          hipStream_t stream) {
  if (d.dtype == LS_BF16)
    return run<BF16>(d, target_logits, draft_logits, draft, temperature, u_accept, u_sample,
                     tokens, tau, ws, stream);
  return run<F32>(d, target_logits, draft_logits, draft, temperature, u_accept, u_sample, tokens,
                  tau, ws, stream);
}

}  // namespace ls
