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
// its (B+1) x splits keys, 16 lanes per row, counts the accepted prefix with
// one ballot and writes target_tok and tau.  The kernel boundary orders (1)
// before (2): no device-scope fence is needed, which on a multi-XCD GPU would
// write back and invalidate L2.  The logits are streamed once (HBM-bound:
// 2 bytes per bf16 logit).
//
// The drafter's own proposal at T = 0 (Fig. 1 caption: drafting time counts
// the proposal and sampling of the drafted tokens) is the same reduction over
// its C*B rows of logits, finished by 16 lanes per row (argmax_finalize).
#include "accept.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

// 8 waves per (row, chunk) workgroup, two 16-byte loads per thread: measured
// faster than 4 waves with four loads each (13.8 against 14.2 us for the
// 82.7 MB key pass of 272 rows of 151,936 logits) and than 16 waves with one
constexpr int kThreads = 512;

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

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// two bf16 (one 32-bit word) -> two 16-bit keys whose unsigned order is the
// values' order, with -0 and +0 equal: positive h -> h ^ 0x8000, negative
// h -> -h (mod 2^16).  Every key of a real value is at least 1.
__device__ __forceinline__ uint32_t key16x2(uint32_t x) {
  const u16x2 s = __builtin_bit_cast(u16x2, i16x2(__builtin_bit_cast(i16x2, x) >> 15));  // 0xFFFF: negative
  return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(u16x2, x) ^ (s | u16x2{0x8000, 0x8000})) - s);
}
// the bf16 bits of a 16-bit key
__device__ __forceinline__ uint16_t key16_bits(uint32_t k) {
  return uint16_t(k >= 0x8000u ? k ^ 0x8000u : 0x10000u - k);
}

// wave max in registers (every lane gets it): quad swaps and rotations by 4
// and 8 inside each 16-lane row (DPP), then the rows swap in pairs and the
// wave's halves swap (v_permlane16_swap / v_permlane32_swap)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(x), int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x124>(v));  // row_ror:4
  v = max(v, dpp_u32<0x128>(v));  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(uint32_t(a[0]), uint32_t(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(uint32_t(b[0]), uint32_t(b[1]));
}

// bf16 rows with 16-byte aligned chunks: the chunk's 8192 logits are one
// 16-byte load per thread per 8 * kThreads logits (all in flight at once; the tail
// chunk's missing vectors repeat its last one and are masked afterwards).
// Each logit becomes one 32-bit key, value key in the high half and
// 0xFFFF - (index in the chunk) in the low half, so a single max finds the
// largest value and its lowest index.  Fast path: while the maximum is
// positive, the raw bits ordered as signed 16-bit integers already order the
// values that matter (the positive ones; every negative one and -0 rank below
// them), so a key is one shift-or of the raw word.  A wave whose maximum is
// not positive redoes its keys with key16x2, which orders every value and
// merges -0 with +0.  One barrier merges the workgroup's waves.
__device__ __forceinline__ uint64_t chunk_argmax_bf16(const uint16_t* __restrict__ x, int begin, int end,
                                                      int tid) {
  constexpr int U = kVerifyChunk / 8 / kThreads;
  static_assert(U * 8 * kThreads == kVerifyChunk, "whole 16-byte loads per thread");
  static_assert(kVerifyChunk <= 8192, "indices in the chunk fit the low key half with room to spare");
  __shared__ uint32_t red[kThreads / 64];
  const u32x4v* xv = reinterpret_cast<const u32x4v*>(x + begin);
  const int nvec = (end - begin) / 8;
  u32x4v buf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) buf[u] = __builtin_nontemporal_load(xv + min(u * kThreads + tid, nvec - 1));
  // low key halves of the thread's elements in vector u = c0[e] - 8 * kThreads * u
  // (c0 >= 0xFFFF - 8 * kThreads + 1 > 8 * kThreads * (U - 1): no borrow)
  uint32_t c0[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c0[e] = 0xFFFFu - 8u * tid - e;

  int32_t fast = INT32_MIN;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int32_t acc = INT32_MIN;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t ww = buf[u][w];
      acc = max(acc, max(int32_t((ww << 16) | c0[2 * w]), int32_t((ww & 0xFFFF0000u) | c0[2 * w + 1])));
    }
    fast = max(fast, u * kThreads + tid < nvec ? acc - 8 * kThreads * u : INT32_MIN);
  }
  // signed -> unsigned order: the value key becomes h ^ 0x8000, as key16x2 has it
  uint32_t W = __builtin_amdgcn_readfirstlane(wave_max_u32(uint32_t(fast) ^ 0x80000000u));
  if ((W >> 16) <= 0x8000u) {  // the wave's maximum is <= +0: exact keys for every value
    uint32_t slow = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t acc = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t k = key16x2(buf[u][w]);
        acc = max(acc, max((k << 16) | c0[2 * w], (k & 0xFFFF0000u) | c0[2 * w + 1]));
      }
      slow = max(slow, u * kThreads + tid < nvec ? acc - 8u * kThreads * u : 0u);
    }
    W = __builtin_amdgcn_readfirstlane(wave_max_u32(slow));
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) red[wave] = W;
  __syncthreads();
  uint32_t K = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) K = max(K, red[w]);
  // every chunk holds at least one logit, so K >= 1 << 16
  const uint32_t idx = uint32_t(begin) + (0xFFFFu - (K & 0xFFFFu));
  return make_key(bf16_to_f32(key16_bits(K >> 16)), idx);
}

// len_snap (may be null): the first chunk of each sequence's first row also
// copies seq_len[c] to len_snap[c] (rows_per_seq rows per sequence), the
// length before the update that the next launch makes, and clears the
// sequence's n_arr arrival counters when `arrivals` is not null
template <typename Ty>
__global__ __launch_bounds__(kThreads) void verify_partial(
    const typename Ty::T* __restrict__ logits, uint64_t* __restrict__ part, int V, int nsplit,
    int chunk, int vec_ok, const int32_t* __restrict__ seq_len, int32_t* __restrict__ len_snap,
    int rows_per_seq, int32_t* __restrict__ arrivals, int n_arr) {
  using VT = Vec16<Ty>;
  const int split = blockIdx.x;
  const int row = blockIdx.y;  // c * (B+1) + i
  const int tid = threadIdx.x;
  if (len_snap != nullptr && split == 0 && row % rows_per_seq == 0) {
    const int c = row / rows_per_seq;
    if (tid == 0) len_snap[c] = seq_len[c];
    if (arrivals != nullptr)
      for (int i = tid; i < n_arr; i += kThreads) arrivals[int64_t(c) * n_arr + i] = 0;
  }
  const typename Ty::T* x = logits + int64_t(row) * V;
  const int begin = split * chunk;
  const int end = min(V, begin + chunk);

  if constexpr (Ty::kBytes == 2) {
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

// one workgroup per sequence: keys -> g_i -> accepted prefix -> tau.  Rows
// are spread kLanesPerRow lanes each over the workgroup (B + 1 <= 64 rows in
// one pass); the draft tokens are requested first, so their latency hides
// behind the key loads; the accepted prefix is one ballot of mismatches.
constexpr int kFinalizeThreads = 64 * kLanesPerRow;
__global__ __launch_bounds__(kFinalizeThreads) void verify_finalize(
    const uint64_t* __restrict__ part, const int32_t* __restrict__ draft,
    int32_t* __restrict__ target_tok, int32_t* __restrict__ tau, int B, int nkeys) {
  __shared__ int32_t g[64];
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t dj = tid < B ? draft[int64_t(c) * B + tid] : 0;
  accept_rows<kFinalizeThreads>(part, nkeys, c, B, g, target_tok);
  __syncthreads();
  if (tid < 64) {
    const int t = accept_tau(g, dj, B);
    if (tid == 0) tau[c] = t;
  }
}

// kLanesPerRow lanes per row: the row's partial keys -> its argmax token
__global__ __launch_bounds__(kThreads) void argmax_finalize(const uint64_t* __restrict__ part,
                                                            int32_t* __restrict__ tok, int rows,
                                                            int nkeys) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int row = int(t / kLanesPerRow), sub = int(t % kLanesPerRow);
  if (row >= rows) return;  // whole 16-lane groups leave together (kThreads % 16 == 0)
  const uint64_t k = row_key(part + int64_t(row) * nkeys, nkeys, sub);
  if (sub == 0) tok[row] = int32_t(~uint32_t(k));
}

template <typename Ty>
ls_status launch_partials(const ls_dims& d, const void* logits, int rows, uint64_t* part,
                          int nsplit, hipStream_t stream, const int32_t* seq_len = nullptr,
                          int32_t* len_snap = nullptr, int32_t* arrivals = nullptr) {
  const int esz = Ty::kBytes;
  // 16-byte loads need every row start (and chunk start) 16-byte aligned
  const int vec_ok = ((int64_t(d.V) * esz) % 16 == 0) && ((uintptr_t(logits) & 15) == 0);
  hipLaunchKernelGGL(verify_partial<Ty>, dim3(nsplit, rows), dim3(kThreads), 0, stream,
                     static_cast<const typename Ty::T*>(logits), part, d.V, nsplit, kVerifyChunk,
                     vec_ok, seq_len, len_snap, d.B + 1, arrivals, arrivals_per_seq(d));
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
  hipLaunchKernelGGL(argmax_finalize, dim3(unsigned(cdiv(int64_t(rows) * kLanesPerRow, kThreads))),
                     dim3(kThreads), 0, stream,
                     part, draft_tok, rows, nsplit);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

ls_status launch_verify_keys(const ls_dims& d, const void* logits, char* ws,
                             const int32_t* seq_len, int32_t* len_snap, hipStream_t stream,
                             int32_t* arrivals) {
  const WsLayout lay = ws_layout(d, 1);
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + lay.verify_part);
  const int rows = d.C * (d.B + 1);
  return d.dtype == LS_BF16
             ? launch_partials<BF16>(d, logits, rows, part, lay.vsplit, stream, seq_len, len_snap, arrivals)
             : launch_partials<F32>(d, logits, rows, part, lay.vsplit, stream, seq_len, len_snap, arrivals);
}

ls_status launch_verify(const ls_dims& d, const void* logits, const int32_t* draft,
                        int32_t* target_tok, int32_t* tau, char* ws, hipStream_t stream) {
  return launch_verify_into(d, logits, draft, target_tok, tau,
                            reinterpret_cast<uint64_t*>(ws + ws_layout(d, 1).verify_part), stream);
}

ls_status launch_verify_finalize(const ls_dims& d, const int32_t* draft, int32_t* target_tok,
                                 int32_t* tau, const char* ws, hipStream_t stream) {
  hipLaunchKernelGGL(verify_finalize, dim3(d.C), dim3(kFinalizeThreads), 0, stream,
                     reinterpret_cast<const uint64_t*>(ws + ws_layout(d, 1).verify_part), draft,
                     target_tok, tau, d.B, verify_splits(d));
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

ls_status launch_verify_into(const ls_dims& d, const void* logits, const int32_t* draft,
                             int32_t* target_tok, int32_t* tau, uint64_t* part,
                             hipStream_t stream) {
  const int nsplit = verify_splits(d);
  const int rows = d.C * (d.B + 1);
  const ls_status st = d.dtype == LS_BF16 ? launch_partials<BF16>(d, logits, rows, part, nsplit, stream)
                                          : launch_partials<F32>(d, logits, rows, part, nsplit, stream);
  if (st != LS_OK) return st;
  static_assert(kMaxBlock + 1 <= 64, "one ballot covers the drafts, one pass covers the rows");
  hipLaunchKernelGGL(verify_finalize, dim3(d.C), dim3(kFinalizeThreads), 0, stream, part, draft,
                     target_tok, tau, d.B, nsplit);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace ls
