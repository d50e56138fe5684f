// Operands, online softmax and MFMA steps of the drafter's block attention
// (LongSpark paper page, Fig. 2 (c)), shared by the draft kernel and by the
// round kernel that fuses the per-round update with the draft.
//
// The attention runs S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA,
// keys and values as the A operand, over 32-key chunks; each wave keeps an
// online softmax per query row (base 2, lazy rescale) in its lanes.
#pragma once

#include "common.hpp"

namespace ls {
namespace {

#ifndef LS_DRAFT_KPW
#define LS_DRAFT_KPW 8
#endif
constexpr int kKPW = LS_DRAFT_KPW;             // key parts (waves) per workgroup
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
// 8*(m/4) + 4*mb + m%4.  Then the P^T operand and the V^T operand (one
// 16-byte load per dimension block) see the lane's 8 keys in natural order.
// The stored key tiles (key_index) follow the same permutation.
__device__ __forceinline__ int chunk_key(int m, int mb) { return 8 * (m >> 2) + 4 * mb + (m & 3); }

// LDS image of one staged block chunk: its 32 value rows as they arrive
// (row-major, rows padded to 288 bytes so that the 16 rows one transposed
// read touches fall on 8 distinct 8-bank groups, twice)
constexpr int kBVS = 128 + 16;  // value row stride (bf16)
constexpr int kBlkElems = 32 * kBVS;

// Half of one 32-key chunk's MFMA operands for one wave: the 8 key loads
// (A operands of S^T = K Q^T, [mb*4 + ks]) or the 8 value loads (A operands
// of O^T += V^T P^T, [dimension block of 16]).
struct Half {
  u16x8 r[8];
  int pos;  // key halves: ring_pos of key (lane & 31); 0 for the slots
};

// The positions read for a slot chunk: slots are always occupied.
__device__ const int32_t kSlotPos[32] = {};

// kt: the chunk's key tile (operand order); pp: the chunk's 32 positions
// (its ring_pos, or kSlotPos for the slots).  The position loads first, so
// the occupancy mask never waits for the operands behind it.
// No branch around any load: the compiler can then count the loads in
// flight exactly and wait only for the ones a step needs.
__device__ __forceinline__ void load_keys(Half& x, const uint16_t* kt, const int32_t* pp, bool ring,
                                          int lane) {
  const int p = pp[lane & 31];
#pragma unroll
  for (int i = 0; i < 8; ++i) x.r[i] = *reinterpret_cast<const u16x8*>(kt + (i * 64 + lane) * 8);
  x.pos = ring ? p : 0;
}
// vt: the chunk's value tile [d][32]
__device__ __forceinline__ void load_values(Half& x, const uint16_t* vt, int lane) {
  const int ln = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    x.r[db] = *reinterpret_cast<const u16x8*>(vt + (db * 16 + ln) * 32 + kg * 8);
}

// Online softmax state of one row group of 16 query rows.
struct Softmax {
  float m, l;
  f32x4 o[8];
};

// raw scores of one row group for the chunk (s[mb][r] is key 8kg + 4mb + r)
// -> lazy online softmax update in base 2; returns the bf16 weights as the
// P^T operand.  valid8 bit e: key 8kg + e is present (all set for full
// chunks, where masking is skipped).
__device__ __forceinline__ bf16x8 softmax_chunk(Softmax& st, f32x4 (&s)[2], uint32_t valid8, bool full) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if (!full) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((valid8 >> (4 * mb + r)) & 1u)) s[mb][r] = -INFINITY;
  }
  float tmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  // the row's max over the 4 lane groups (lanes ln, ln+16, ln+32, ln+48):
  // swapping a register with itself across row pairs / halves leaves the
  // partner's value in one of the two results
  {
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
  }
  tmax *= kScale2;  // the scale is positive: max of the scaled scores
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
  // weights 2^(s*scale - m) rounded to bf16 in pairs; l sums the same
  // rounded weights
  uint32_t pw[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      const f32x2 e2 = {exp2_f(fmaf(s[mb][r], kScale2, -m_use)), exp2_f(fmaf(s[mb][r + 1], kScale2, -m_use))};
      pw[mb * 2 + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(e2, bf16x2));
    }
  const bf16x2 ones = {__bf16(1.0f), __bf16(1.0f)};
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), ones, lsum, false);
  st.l += lsum;
  return as_bf16x8(__builtin_bit_cast(u16x8, uint4{pw[0], pw[1], pw[2], pw[3]}));
}

// S^T = K Q^T for both row groups (raw dot products)
__device__ __forceinline__ void chunk_scores(f32x4 (&s)[2][2], const Half& k, const bf16x8 (&qb)[2][4]) {
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) s[rg][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
        s[rg][mb] = mfma16x16x32(as_bf16x8(k.r[mb * 4 + ks]), qb[rg][ks], s[rg][mb]);
}

// O^T += V^T P^T for both row groups
__device__ __forceinline__ void chunk_pv(Softmax (&st)[2], const Half& v, const bf16x8 (&pk)[2]) {
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) st[rg].o[db] = mfma16x16x32(as_bf16x8(v.r[db]), pk[rg], st[rg].o[db]);
}

}  // namespace
}  // namespace ls
