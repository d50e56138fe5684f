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
//   seq_len[c] += tau (by the last workgroup of the sequence).
//
// Grid: one workgroup per (sequence, KV head, tile of 16 slots).  Each
// workgroup stages the tau rows (and its 16 slot queries) in LDS, computes
// the 16 x tau scores, and streams its slots' fp32 state once (coalesced
// float4), so the per-round traffic is the state read + write + slot write,
// independent of the prefix length.
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
constexpr int kSlotsPerBlock = 16;

template <typename Ty, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(
    const typename Ty::T* __restrict__ k_new, const typename Ty::T* __restrict__ v_new,
    const int32_t* __restrict__ tau_in, typename Ty::T* __restrict__ ring_k,
    typename Ty::T* __restrict__ ring_v, int32_t* __restrict__ ring_pos,
    int32_t* __restrict__ seq_len, float* __restrict__ sum_m, float* __restrict__ sum_l,
    float* __restrict__ sum_n, typename Ty::T* __restrict__ slot_k,
    typename Ty::T* __restrict__ slot_v, const typename Ty::T* __restrict__ u,
    const float* __restrict__ log_lambda, int32_t* __restrict__ err_flag,
    uint32_t* __restrict__ counter, int Hkv, int W, int S, int B, int NT) {
  constexpr int RS = 2 * D + 1;  // LDS row stride (floats): +1 avoids bank conflicts
  constexpr int US = D + 1;
  extern __shared__ float smem[];
  float* rows = smem;                              // [B+1][RS]  k | v
  float* ush = rows + (B + 1) * RS;                // [16][US]   slot queries
  float* w = ush + kSlotsPerBlock * US;            // [16][B+1]  scores -> weights
  __shared__ float s_scale[kSlotsPerBlock], s_inv_l[kSlotsPerBlock];

  const int tile = blockIdx.x % NT;
  const int ch = blockIdx.x / NT;
  const int h = ch % Hkv;
  const int c = ch / Hkv;
  const int tid = threadIdx.x;
  const int B1 = B + 1;

  int T = tau_in[c];
  if (T < 1 || T > B1) {
    if (tid == 0 && h == 0 && tile == 0) atomicOr(err_flag, 1);
    T = T < 1 ? 1 : B1;
  }
  const int L = seq_len[c];
  const int j0 = tile * kSlotsPerBlock;
  const int nj = min(kSlotsPerBlock, S - j0);

  // stage the new rows and this tile's slot queries
  for (int idx = tid; idx < T * 2 * D; idx += kThreads) {
    const int i = idx / (2 * D), e = idx % (2 * D);
    const int64_t src = ((int64_t(c) * B1 + i) * Hkv + h) * D + (e % D);
    rows[i * RS + e] = Ty::load(e < D ? k_new : v_new, src);
  }
  for (int idx = tid; idx < nj * D; idx += kThreads) {
    const int jj = idx / D, e = idx % D;
    ush[jj * US + e] = Ty::load(u, (int64_t(h) * S + j0 + jj) * D + e);
  }
  // ring window: this tile copies rows i = tile, tile + NT, ...
  for (int i = tile; i < T; i += NT) {
    const int slot = int((int64_t(L) + i) % W);
    const int64_t dst = ((int64_t(c) * Hkv + h) * W + slot) * D;
    const int64_t src = ((int64_t(c) * B1 + i) * Hkv + h) * D;
    for (int e = tid; e < D; e += kThreads) {
      ring_k[dst + e] = k_new[src + e];
      ring_v[dst + e] = v_new[src + e];
    }
    if (h == 0 && tid == 0) ring_pos[int64_t(c) * W + slot] = L + i;
  }
  __syncthreads();

  // scores a_ji = u_j . k_i / sqrt(d) + (tau-1-i) ln lambda_j
  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
  for (int p = tid; p < nj * T; p += kThreads) {
    const int jj = p / T, i = p % T;
    float acc = 0.f;
#pragma unroll 16
    for (int e = 0; e < D; ++e) acc = fmaf(ush[jj * US + e], rows[i * RS + e], acc);
    const float lnl = log_lambda[j0 + jj];
    const int dist = T - 1 - i;
    const float bias = dist == 0 ? 0.f : float(dist) * lnl;
    w[jj * B1 + i] = acc * inv_sqrt_d + bias;
  }
  __syncthreads();

  // per-slot merge of (m, l) with the new rows
  if (tid < nj) {
    const int j = j0 + tid;
    const int64_t sidx = (int64_t(c) * Hkv + h) * S + j;
    const float lnl = log_lambda[j];
    const float m_old = sum_m[sidx];
    const float m_shift = (lnl == -INFINITY) ? -INFINITY : fmaf(float(T), lnl, m_old);
    float mx = m_shift;
    for (int i = 0; i < T; ++i) mx = fmaxf(mx, w[tid * B1 + i]);
    const float scale = (m_shift == -INFINITY) ? 0.f : exp_f(m_shift - mx);
    float lsum = 0.f;
    for (int i = 0; i < T; ++i) {
      const float pw = exp_f(w[tid * B1 + i] - mx);
      w[tid * B1 + i] = pw;
      lsum += pw;
    }
    const float l_new = fmaf(sum_l[sidx], scale, lsum);
    sum_m[sidx] = mx;
    sum_l[sidx] = l_new;
    s_scale[tid] = scale;
    s_inv_l[tid] = 1.0f / l_new;
  }
  __syncthreads();

  // numerator n = n * scale + sum_i w_i [k_i ; v_i]; slots = n / l
  constexpr int Q = 2 * D / 4;  // float4 per slot
  for (int p = tid; p < nj * Q; p += kThreads) {
    const int jj = p / Q, e4 = (p % Q) * 4;
    float4* np = reinterpret_cast<float4*>(sum_n + ((int64_t(c) * Hkv + h) * S + j0 + jj) * 2 * D + e4);
    float4 acc = *np;
    const float sc = s_scale[jj];
    acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
    for (int i = 0; i < T; ++i) {
      const float wi = w[jj * B1 + i];
      const float* r = rows + i * RS + e4;
      acc.x = fmaf(wi, r[0], acc.x);
      acc.y = fmaf(wi, r[1], acc.y);
      acc.z = fmaf(wi, r[2], acc.z);
      acc.w = fmaf(wi, r[3], acc.w);
    }
    *np = acc;
    const float il = s_inv_l[jj];
    const int64_t so = ((int64_t(c) * Hkv + h) * S + j0 + jj) * D + (e4 % D);
    typename Ty::T* dst = e4 < D ? slot_k : slot_v;
    Ty::store(dst, so + 0, acc.x * il);
    Ty::store(dst, so + 1, acc.y * il);
    Ty::store(dst, so + 2, acc.z * il);
    Ty::store(dst, so + 3, acc.w * il);
  }

  // the last workgroup of sequence c advances seq_len (all have read L)
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t ticket = atomicAdd(&counter[c], 1u);
    if (ticket == uint32_t(Hkv * NT - 1)) {
      seq_len[c] = L + T;
      counter[c] = 0u;
    }
  }
}

template <typename Ty, int D>
ls_status run(const ls_dims& d, const ls_state& st, const void* k_new, const void* v_new,
              const int32_t* tau, hipStream_t stream) {
  using T = typename Ty::T;
  const int NT = int(cdiv(d.S, kSlotsPerBlock));
  const WsLayout lay = ws_layout(d, 1);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(st.workspace) + lay.cnt_append);
  const size_t shmem = sizeof(float) * (size_t(d.B + 1) * (2 * D + 1) +
                                        size_t(kSlotsPerBlock) * (D + 1) +
                                        size_t(kSlotsPerBlock) * (d.B + 1));
  hipLaunchKernelGGL((append_kernel<Ty, D>), dim3(d.C * d.Hkv * NT), dim3(kThreads), shmem, stream,
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), tau,
                     static_cast<T*>(st.ring_k), static_cast<T*>(st.ring_v), st.ring_pos,
                     st.seq_len, st.sum_m, st.sum_l, st.sum_n, static_cast<T*>(st.slot_k),
                     static_cast<T*>(st.slot_v), static_cast<const T*>(st.u), st.log_lambda,
                     st.err_flag, cnt, d.Hkv, d.W, d.S, d.B, NT);
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
