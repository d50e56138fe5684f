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
//   seq_len[c] += tau (a second, tiny launch: every workgroup of the first
//   launch reads the old L, and the kernel boundary orders those reads
//   before the update without a device-scope fence).
//
// Grid: one workgroup per (sequence, KV head, tile of 16 slots).  Each
// workgroup stages the tau rows (and its 16 slot queries) in LDS, computes
// the 16 x tau scores, and streams its slots' fp32 state once (coalesced
// float4), so the per-round traffic is the state read + write + slot write,
// independent of the prefix length.  The tiles share the ring copy of the
// tau rows.  Values of the window and of the slots are written in key tiles
// of 32 ([rows/32][d][32]), the layout the drafter's P.V product reads.
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
    const int32_t* __restrict__ seq_len, float* __restrict__ sum_m, float* __restrict__ sum_l,
    float* __restrict__ sum_n, typename Ty::T* __restrict__ slot_k,
    typename Ty::T* __restrict__ slot_v, const typename Ty::T* __restrict__ u,
    const float* __restrict__ log_lambda, int32_t* __restrict__ err_flag, int Hkv, int W,
    int S, int B, int NT) {
  constexpr int RS = 2 * D + 4;  // LDS row stride (floats): 16-byte rows, banks offset by 4
  constexpr int US = D + 4;
  constexpr int Q = 2 * D / 4;   // float4 per slot of n
  constexpr int NQ = (kSlotsPerBlock * Q + kThreads - 1) / kThreads;  // float4 of n per thread
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  float* rows = smem;                              // [B+1][RS]  k | v
  float* ush = rows + (B + 1) * RS;                // [16][US]   slot queries
  float* w = ush + kSlotsPerBlock * US;            // [16][B+1]  scores -> weights
  constexpr int SVS = kSlotsPerBlock + 1;          // slot-value staging stride
  float* svals = w + kSlotsPerBlock * (B + 1);     // [d][SVS]   slot values
  __shared__ float s_scale[kSlotsPerBlock], s_inv_l[kSlotsPerBlock];

  const int tid = threadIdx.x;
  const int B1 = B + 1;
  const int tile = blockIdx.x % NT;
  const int ch = blockIdx.x / NT;
  const int h = ch % Hkv;
  const int c = ch / Hkv;
  const int j0 = tile * kSlotsPerBlock;
  const int nj = min(kSlotsPerBlock, S - j0);
  const int64_t slot0 = (int64_t(c) * Hkv + h) * S + j0;  // first slot of this tile

  // issue the state loads first: they do not depend on tau, and their
  // latency then overlaps the staging below
  float4 nreg[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int p = tid + k * kThreads, jj = p / Q;
    nreg[k] = jj < nj ? reinterpret_cast<const float4*>(sum_n + slot0 * 2 * D)[p]
                      : float4{0.f, 0.f, 0.f, 0.f};
  }
  float m_old = 0.f, l_old = 0.f, lnl_t = 0.f;
  if (tid < nj) {
    m_old = sum_m[slot0 + tid];
    l_old = sum_l[slot0 + tid];
    lnl_t = log_lambda[j0 + tid];
  }

  int T = tau_in[c];
  if (T < 1 || T > B1) {
    if (tid == 0 && h == 0 && tile == 0) atomicOr(err_flag, 1);
    T = T < 1 ? 1 : B1;
  }
  const int L = seq_len[c];

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
  // ring window, shared by the NT tiles of (c, h): tile t copies the key
  // pieces p = t, t + NT, ... (16 bytes of one new row each) and the values
  // of dimensions t, t + NT, ...; lanes run over the tau rows, so their
  // 2-byte stores land on consecutive slots of the key-tiled value layout
  {
    constexpr int V16 = D * Ty::kBytes / 16;  // 16-byte pieces per key row
    const int64_t unit = int64_t(c) * Hkv + h;
    for (int p = tile + NT * tid; p < T * V16; p += NT * kThreads) {
      const int i = p / V16, e = p % V16;
      const int slot = int((int64_t(L) + i) % W);
      reinterpret_cast<uint4*>(ring_k + (unit * W + slot) * D)[e] =
          reinterpret_cast<const uint4*>(k_new + ((int64_t(c) * B1 + i) * Hkv + h) * D)[e];
    }
    const int ndim = (D - tile + NT - 1) / NT;  // dimensions tile, tile+NT, ...
    for (int p = tid; p < ndim * T; p += kThreads) {
      const int dim = tile + NT * (p / T), i = p % T;
      const int slot = int((int64_t(L) + i) % W);
      ring_v[value_index(unit, W, D, slot, dim)] = v_new[((int64_t(c) * B1 + i) * Hkv + h) * D + dim];
    }
    if (h == 0 && tile == 0)
      for (int i = tid; i < T; i += kThreads) ring_pos[int64_t(c) * W + int((int64_t(L) + i) % W)] = L + i;
  }
  __syncthreads();

  // scores a_ji = u_j . k_i / sqrt(d) + (tau-1-i) ln lambda_j
  const float inv_sqrt_d = 1.0f / sqrtf(float(D));
  for (int p = tid; p < nj * T; p += kThreads) {
    const int jj = p / T, i = p % T;
    const float4* ur = reinterpret_cast<const float4*>(ush + jj * US);
    const float4* kr = reinterpret_cast<const float4*>(rows + i * RS);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 4; ++e) {
      const float4 x = ur[e], y = kr[e];
      a0 = fmaf(x.x, y.x, a0);
      a1 = fmaf(x.y, y.y, a1);
      a0 = fmaf(x.z, y.z, a0);
      a1 = fmaf(x.w, y.w, a1);
    }
    const float lnl = log_lambda[j0 + jj];
    const int dist = T - 1 - i;
    const float bias = dist == 0 ? 0.f : float(dist) * lnl;
    w[jj * B1 + i] = (a0 + a1) * inv_sqrt_d + bias;
  }
  __syncthreads();

  // per-slot merge of (m, l) with the new rows
  if (tid < nj) {
    const float m_shift = (lnl_t == -INFINITY) ? -INFINITY : fmaf(float(T), lnl_t, m_old);
    float mx = m_shift;
    for (int i = 0; i < T; ++i) mx = fmaxf(mx, w[tid * B1 + i]);
    const float scale = (m_shift == -INFINITY) ? 0.f : exp_f(m_shift - mx);
    float lsum = 0.f;
    for (int i = 0; i < T; ++i) {
      const float pw = exp_f(w[tid * B1 + i] - mx);
      w[tid * B1 + i] = pw;
      lsum += pw;
    }
    const float l_new = fmaf(l_old, scale, lsum);
    sum_m[slot0 + tid] = mx;
    sum_l[slot0 + tid] = l_new;
    s_scale[tid] = scale;
    s_inv_l[tid] = 1.0f / l_new;
  }
  __syncthreads();

  // numerator n = n * scale + sum_i w_i [k_i ; v_i]; slots = n / l
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int p = tid + k * kThreads, jj = p / Q, e4 = (p % Q) * 4;
    if (jj >= nj) continue;
    float4 acc = nreg[k];
    const float sc = s_scale[jj];
    acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
    for (int i = 0; i < T; ++i) {
      const float wi = w[jj * B1 + i];
      const float4 r = *reinterpret_cast<const float4*>(rows + i * RS + e4);
      acc.x = fmaf(wi, r.x, acc.x);
      acc.y = fmaf(wi, r.y, acc.y);
      acc.z = fmaf(wi, r.z, acc.z);
      acc.w = fmaf(wi, r.w, acc.w);
    }
    reinterpret_cast<float4*>(sum_n + slot0 * 2 * D)[p] = acc;
    const float il = s_inv_l[jj];
    if (e4 < D) {  // pooled key, [S][d]
      const int64_t so = (slot0 + jj) * D + e4;
      Ty::store(slot_k, so + 0, acc.x * il);
      Ty::store(slot_k, so + 1, acc.y * il);
      Ty::store(slot_k, so + 2, acc.z * il);
      Ty::store(slot_k, so + 3, acc.w * il);
    } else {  // pooled value: staged [dim][slot] in LDS, written below
      float* sv = svals + (e4 - D) * SVS + jj;
      sv[0 * SVS] = acc.x * il;
      sv[1 * SVS] = acc.y * il;
      sv[2 * SVS] = acc.z * il;
      sv[3 * SVS] = acc.w * il;
    }
  }
  // slot values to the key-tiled layout: per dimension the tile's nj slots
  // are consecutive, so each thread stores a run of slots of one dimension
  __syncthreads();
  {
    const int64_t unit = int64_t(c) * Hkv + h;
    for (int p = tid; p < D * nj; p += kThreads) {
      const int dim = p / nj, jj = p % nj;
      Ty::store(slot_v, value_index(unit, S, D, j0 + jj, dim), svals[dim * SVS + jj]);
    }
  }
}

// seq_len[c] += clamp(tau[c], 1, B+1), after every append workgroup read it
__global__ void append_commit(const int32_t* __restrict__ tau_in, int32_t* __restrict__ seq_len,
                              int C, int B) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  int T = tau_in[c];
  T = T < 1 ? 1 : (T > B + 1 ? B + 1 : T);
  seq_len[c] += T;
}

template <typename Ty, int D>
ls_status run(const ls_dims& d, const ls_state& st, const void* k_new, const void* v_new,
              const int32_t* tau, hipStream_t stream) {
  using T = typename Ty::T;
  const int NT = int(cdiv(d.S, kSlotsPerBlock));
  const size_t shmem = sizeof(float) * (size_t(d.B + 1) * (2 * D + 4) +
                                        size_t(kSlotsPerBlock) * (D + 4) +
                                        size_t(kSlotsPerBlock) * (d.B + 1) +
                                        size_t(D) * (kSlotsPerBlock + 1));
  hipLaunchKernelGGL((append_kernel<Ty, D>), dim3(d.C * d.Hkv * NT), dim3(kThreads), shmem, stream,
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), tau,
                     static_cast<T*>(st.ring_k), static_cast<T*>(st.ring_v), st.ring_pos,
                     st.seq_len, st.sum_m, st.sum_l, st.sum_n, static_cast<T*>(st.slot_k),
                     static_cast<T*>(st.slot_v), static_cast<const T*>(st.u), st.log_lambda,
                     st.err_flag, d.Hkv, d.W, d.S, d.B, NT);
  if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
  hipLaunchKernelGGL(append_commit, dim3(unsigned(cdiv(d.C, 256))), dim3(256), 0, stream, tau,
                     st.seq_len, d.C, d.B);
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
