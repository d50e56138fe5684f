// Greedy verification of a drafted block (LongSpark paper page, Fig. 2 (a);
// Table 3: greedy decoding, T = 0; Table 1: accepted length tau).
//
// g_i = argmax_v logits[c, i, v] with the lowest index on ties; M = longest
// prefix with draft[c, i] == g_i; tau = M + 1.
//
// Two launches.  (1) Each workgroup scans one chunk of one logits row with
// 16-byte non-temporal loads and reduces (value, index) to a 64-bit key whose
// unsigned order is "larger value first, then lower index": the high word is
// the value's bits mapped to an order-preserving unsigned integer (+0 and -0
// merged), the low word is ~index.  (2) One workgroup per sequence reduces
// its (B+1) x splits keys, counts the accepted prefix and writes target_tok
// and tau.  The kernel boundary orders (1) before (2): no device-scope fence
// is needed, which on a multi-XCD GPU would write back and invalidate L2.
// The logits are streamed once (HBM-bound: 2 bytes per bf16 logit).
//
// The drafter's own proposal at T = 0 (Fig. 1 caption: drafting time counts
// the proposal and sampling of the drafted tokens) is the same reduction over
// its C*B rows of logits, finished by one thread per row (argmax_finalize).
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;

__device__ inline uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 compares equal to +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t make_key(float x, uint32_t idx) {
  return (uint64_t(ordered_bits(x)) << 32) | uint64_t(~idx);
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

#ifndef LS_VERIFY_PACKED
#define LS_VERIFY_PACKED 1
#endif
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// two bf16 (one 32-bit word) -> two 16-bit keys whose unsigned order is the
// values' order: positive h -> h | 0x8000, negative h -> ~h.  -0 lands just
// below +0 (0x7FFF vs 0x8000); the index search merges the two.
__device__ __forceinline__ u16x2 order16x2(uint32_t x) {
  const i16x2 h = __builtin_bit_cast(i16x2, x);
  const u16x2 flip = __builtin_bit_cast(u16x2, i16x2(h >> 15)) | u16x2{0x8000, 0x8000};
  return __builtin_bit_cast(u16x2, x) ^ flip;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), o, 64)));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, uint32_t(__shfl_xor(int(v), o, 64)));
  return v;
}

// bf16 rows with 16-byte aligned chunks: the chunk's 8192 logits are one
// 16-byte load per thread per 2048 logits (all in flight at once).  The
// values are compared as packed 16-bit integer keys (two logits per
// instruction), the workgroup agrees on the maximum key, and only the
// threads that hold it search their registers for its lowest index.
__device__ __forceinline__ uint64_t chunk_argmax_bf16(const uint16_t* __restrict__ x, int begin, int end,
                                                      int tid) {
  constexpr int U = kVerifyChunk / 8 / kThreads;
  static_assert(U * 8 * kThreads == kVerifyChunk, "one load per thread per 2048 logits");
  __shared__ uint32_t red[kThreads / 64];
  const u32x4v* xv = reinterpret_cast<const u32x4v*>(x + begin);
  const int nvec = (end - begin) / 8;
  u32x4v buf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int v = u * kThreads + tid;
    buf[u] = v < nvec ? __builtin_nontemporal_load(xv + v) : u32x4v{0, 0, 0, 0};
  }
  u16x2 best = {0, 0};  // 0: below every key of a real value
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u * kThreads + tid < nvec) {
#pragma unroll
      for (int w = 0; w < 4; ++w) best = __builtin_elementwise_max(best, order16x2(buf[u][w]));
    }
  const uint32_t tmax = max(uint32_t(best[0]), uint32_t(best[1]));
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t M = wave_max_u32(tmax);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = max(M, red[w]);
  __syncthreads();
  // +0 and -0 are the same value: a maximum of either sign matches both
  const bool zero = M == 0x8000u || M == 0x7FFFu;
  const uint32_t lo = zero ? 0x7FFFu : M, hi = zero ? 0x8000u : M;
  uint32_t idx = 0xFFFFFFFFu;
  if (tmax >= lo && tmax <= hi && M != 0u) {
    // this thread's logits in index order: vector u*kThreads + tid, then word, then half
#pragma unroll
    for (int u = U - 1; u >= 0; --u)
      if (u * kThreads + tid < nvec) {
#pragma unroll
        for (int w = 3; w >= 0; --w) {
          const u16x2 k = order16x2(buf[u][w]);
          const int i0 = begin + (u * kThreads + tid) * 8 + 2 * w;
          if (k[1] >= lo && k[1] <= hi) idx = uint32_t(i0 + 1);
          if (k[0] >= lo && k[0] <= hi) idx = uint32_t(i0);
        }
      }
  }
  idx = wave_min_u32(idx);
  if (lane == 0) red[wave] = idx;
  __syncthreads();
  idx = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) idx = min(idx, red[w]);
  if (idx == 0xFFFFFFFFu) return 0ull;
  const uint32_t h = M >= 0x8000u ? (M ^ 0x8000u) : (~M & 0xFFFFu);  // the bf16 bits back
  return make_key(bf16_to_f32(uint16_t(h)), idx);
}

template <typename Ty>
__global__ __launch_bounds__(kThreads) void verify_partial(
    const typename Ty::T* __restrict__ logits, uint64_t* __restrict__ part, int V, int nsplit,
    int chunk, int vec_ok) {
  using VT = Vec16<Ty>;
  const int split = blockIdx.x;
  const int row = blockIdx.y;  // c * (B+1) + i
  const int tid = threadIdx.x;
  const typename Ty::T* x = logits + int64_t(row) * V;
  const int begin = split * chunk;
  const int end = min(V, begin + chunk);

  if constexpr (Ty::kBytes == 2 && LS_VERIFY_PACKED) {
    if (vec_ok) {
      const uint64_t k = chunk_argmax_bf16(x, begin, end, tid);
      if (tid == 0) part[int64_t(row) * nsplit + split] = k;
      return;
    }
  }
  float best = -INFINITY;
  uint32_t best_i = 0xFFFFFFFFu;
  if (vec_ok) {
    // 16-byte loads; each thread walks its vectors in increasing index order,
    // so a strict '>' keeps the lowest index among equal values.
    const typename VT::V* xv = reinterpret_cast<const typename VT::V*>(x + begin);
    const int nvec = (end - begin) / VT::N;
    constexpr int U = (kVerifyChunk / VT::N + kThreads - 1) / kThreads;  // loads in flight
    for (int base = 0; base < nvec; base += kThreads * U) {
      typename VT::V buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int v = base + u * kThreads + tid;
        if (v < nvec) buf[u] = __builtin_nontemporal_load(xv + v);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int v = base + u * kThreads + tid;
        if (v < nvec) {
#pragma unroll
          for (int e = 0; e < VT::N; ++e) {
            float f = VT::get(buf[u], e);
            if (f > best || best_i == 0xFFFFFFFFu) {  // the first element counts even at -inf
              best = f;
              best_i = uint32_t(begin + v * VT::N + e);
            }
          }
        }
      }
    }
    // tail that does not fill a vector (only in the last chunk)
    for (int i = begin + nvec * VT::N + tid; i < end; i += kThreads) {
      float f = Ty::load(x, i);
      if (f > best || best_i == 0xFFFFFFFFu) { best = f; best_i = uint32_t(i); }
    }
  } else {
    for (int i = begin + tid; i < end; i += kThreads) {
      float f = Ty::load(x, i);
      if (f > best || best_i == 0xFFFFFFFFu) { best = f; best_i = uint32_t(i); }
    }
  }

  uint64_t key = (best_i == 0xFFFFFFFFu) ? 0ull : make_key(best, best_i);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t other = shfl_xor_u64(key, o);
    key = other > key ? other : key;
  }
  __shared__ uint64_t wkeys[kThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) wkeys[wave] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = wkeys[0];
    for (int w = 1; w < kThreads / 64; ++w) k = wkeys[w] > k ? wkeys[w] : k;
    part[int64_t(row) * nsplit + split] = k;
  }
}

// one workgroup per sequence: keys -> g_i -> accepted prefix -> tau
__global__ __launch_bounds__(kThreads) void verify_finalize(
    const uint64_t* __restrict__ part, const int32_t* __restrict__ draft,
    int32_t* __restrict__ target_tok, int32_t* __restrict__ tau, int B, int nsplit) {
  extern __shared__ uint64_t keys[];  // [(B+1) * nsplit]
  __shared__ int32_t g[64];
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = (B + 1) * nsplit;
  const uint64_t* p = part + int64_t(c) * n;
  for (int i = tid; i < n; i += kThreads) keys[i] = p[i];
  __syncthreads();
  for (int i = tid; i <= B; i += kThreads) {
    uint64_t k = 0;
    for (int s = 0; s < nsplit; ++s) k = keys[i * nsplit + s] > k ? keys[i * nsplit + s] : k;
    const int32_t gi = int32_t(~uint32_t(k));
    g[i] = gi;
    target_tok[int64_t(c) * (B + 1) + i] = gi;
  }
  __syncthreads();
  if (tid == 0) {
    int M = 0;
    while (M < B && draft[int64_t(c) * B + M] == g[M]) ++M;
    tau[c] = M + 1;
  }
}

// one thread per row: the row's split keys -> its argmax token
__global__ __launch_bounds__(kThreads) void argmax_finalize(const uint64_t* __restrict__ part,
                                                            int32_t* __restrict__ tok, int rows,
                                                            int nsplit) {
  const int row = blockIdx.x * kThreads + threadIdx.x;
  if (row >= rows) return;
  const uint64_t* p = part + int64_t(row) * nsplit;
  uint64_t k = 0;
  for (int s = 0; s < nsplit; ++s) k = p[s] > k ? p[s] : k;
  tok[row] = int32_t(~uint32_t(k));
}

template <typename Ty>
ls_status launch_partials(const ls_dims& d, const void* logits, int rows, uint64_t* part,
                          int nsplit, hipStream_t stream) {
  const int esz = Ty::kBytes;
  // 16-byte loads need every row start (and chunk start) 16-byte aligned
  const int vec_ok = ((int64_t(d.V) * esz) % 16 == 0) && ((uintptr_t(logits) & 15) == 0);
  hipLaunchKernelGGL(verify_partial<Ty>, dim3(nsplit, rows), dim3(kThreads), 0, stream,
                     static_cast<const typename Ty::T*>(logits), part, d.V, nsplit, kVerifyChunk,
                     vec_ok);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

ls_status launch_argmax(const ls_dims& d, const void* logits, int32_t* draft_tok, char* ws,
                        hipStream_t stream) {
  const WsLayout lay = ws_layout(d, 1);
  const int nsplit = lay.vsplit;
  const int rows = d.C * d.B;  // the verify key area holds C*(B+1) rows
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + lay.verify_part);
  const ls_status st = d.dtype == LS_BF16 ? launch_partials<BF16>(d, logits, rows, part, nsplit, stream)
                                          : launch_partials<F32>(d, logits, rows, part, nsplit, stream);
  if (st != LS_OK) return st;
  hipLaunchKernelGGL(argmax_finalize, dim3(unsigned(cdiv(rows, kThreads))), dim3(kThreads), 0, stream,
                     part, draft_tok, rows, nsplit);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

ls_status launch_verify(const ls_dims& d, const void* logits, const int32_t* draft,
                        int32_t* target_tok, int32_t* tau, char* ws, hipStream_t stream) {
  const WsLayout lay = ws_layout(d, 1);
  const int nsplit = lay.vsplit;
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + lay.verify_part);
  const int rows = d.C * (d.B + 1);
  const ls_status st = d.dtype == LS_BF16 ? launch_partials<BF16>(d, logits, rows, part, nsplit, stream)
                                          : launch_partials<F32>(d, logits, rows, part, nsplit, stream);
  if (st != LS_OK) return st;
  const size_t shmem = sizeof(uint64_t) * size_t(d.B + 1) * nsplit;
  hipLaunchKernelGGL(verify_finalize, dim3(d.C), dim3(kThreads), shmem, stream, part, draft,
                     target_tok, tau, d.B, nsplit);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace ls
