// One wave's share of the summary merge on MFMA (LongSpark paper page,
// Fig. 3: the summary is updated with only the newly retained rows), shared
// by the update kernel and by the round kernel that fuses the update with
// the draft.
//
// For the 32 slots j of a tile and the tau new rows i of a (sequence, KV
// head) unit, with a_ji = u_j.k_i/sqrt(d) + (tau-1-i) ln(lambda_j):
//   S^T = K U^T        rows x slots, 32x32x16 MFMA;
//   per slot (one lane column): m' = max(m + tau ln(lambda), max_i a_ji),
//   s = e^(m + tau ln(lambda) - m'), w_ji = e^(a_ji - m'), l' = l s + sum_i w_ji;
//   N^T = s N^T + R^T W^T    entries x slots, R = [k | v] of the new rows;
// the wave owns kAT consecutive 32-entry accumulator tiles (entries
// 32 kAT q .. 32 kAT (q + 1) - 1).  The weights enter the MFMA as bf16 hi + lo
// (w - hi), so the products keep about 16 bits of the fp32 weight; l sums the
// fp32 weights.  The rows and the slot queries are staged in LDS by the
// caller: keys row-major for S^T, [entry][row] for R^T, rows past B+1 zero.
#pragma once

#include "common.hpp"

namespace ls {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// A-row m of a 32-row score block holds verified row tile_row(m) (bits 2 and
// 3 of m swapped): the S^T output then gives lanes 0-31 rows 0-7 and 16-23 of
// the block, lanes 32-63 rows 8-15 and 24-31, which are the 8 consecutive
// rows each lane feeds the N^T product as its B operand.
__device__ __forceinline__ int tile_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

constexpr int kMergeD = 128;                 // head dimension of the MFMA merge
constexpr int kMergeKLS = kMergeD + 8;       // key / query row stride in LDS (bf16)

// kRB: 32-row score blocks of the staged rows (RP = 32 kRB rows, [entry][row]
// stride RP + 8).  KL: the staged keys [RP][kMergeKLS]; RT: [2d][RP + 8];
// UT: the tile's 32 slot queries [32][kMergeKLS].  acc: the wave's kAT
// accumulator tiles, loaded from the state by the caller (acc[t][4k + r] =
// n[slot][32 (kAT q + t) + 8k + 4hi + r]); on return they hold the merged
// numerators.  m_old, l_old, lnl: the lane's slot's state and ln(lambda).
// Returns the merged l; m_new gets the merged m (natural-log units).
template <int kRB, int kAT>
__device__ __forceinline__ float merge_wave(const uint16_t* KL, const uint16_t* RT, const uint16_t* UT,
                                            f32x16 (&acc)[kAT], float m_old, float l_old, float lnl,
                                            int Tn, int q, int lane, float& m_new) {
  constexpr int D = kMergeD, KLS = kMergeKLS, RTS = 32 * kRB + 8;
  const int ln = lane & 31, hi = lane >> 5;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  // S^T = K U^T; element 8 (s % 2) + e of block s / 2 is verified row 16 s + 8 hi + e
  f32x16 sc[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    sc[rb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u16x8*>(&KL[(32 * rb + tile_row(ln)) * KLS + 16 * ks + 8 * hi]));
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const u16x8*>(&UT[ln * KLS + 16 * ks + 8 * hi]));
      sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, sc[rb], 0, 0, 0);
    }
  }

  // softmax of slot j over the new rows in base 2, K-step by K-step (rows
  // 16 s .. 16 s + 15; steps past tau are skipped); the partner lane
  // (lane ^ 32) holds the other 8 rows of each step.  x_ji = a_ji log2(e);
  // a zero decay (ln(lambda) = -inf) enters the bias as -1e30, so every
  // older row's exponent is hugely negative and 0 * bias never occurs.
  constexpr float kLog2e = 1.4426950408889634f;
  const int nks = (Tn + 15) >> 4;
  const float sc2 = kLog2e / sqrtf(float(D));
  const float lb2 = fmaxf(lnl, -1e30f) * kLog2e;
  const float base2 = lnl == -INFINITY ? -INFINITY : fmaf(float(Tn), lnl, m_old) * kLog2e;
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < 2 * kRB; ++s)
    if (s < nks) {
      const int rem = Tn - 16 * s - 8 * hi;         // rows e < rem are new rows
      const float d0 = float(rem - 1);              // distance of e = 0 to row tau-1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // the distance enters as an exact small integer: row tau-1 gets bias 0 exactly
        const float x = fmaf(d0 - float(e), lb2, sc[s >> 1][8 * (s & 1) + e] * sc2);
        sc[s >> 1][8 * (s & 1) + e] = e < rem ? x : -INFINITY;
        mx = fmaxf(mx, sc[s >> 1][8 * (s & 1) + e]);
      }
    }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  // row tau-1 always counts and has a finite exponent, so m2 is finite and
  // 2^(-inf - m2) = 0 needs no test
  const float m2 = fmaxf(base2, mx);
  const float s_old = __builtin_amdgcn_exp2f(base2 - m2);
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < 2 * kRB; ++s)
    if (s < nks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = __builtin_amdgcn_exp2f(sc[s >> 1][8 * (s & 1) + e] - m2);
        sc[s >> 1][8 * (s & 1) + e] = w;
        lsum += w;
      }
    }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float l_new = fmaf(l_old, s_old, lsum);
  m_new = m2 * 0.6931471805599453f;  // back to natural-log units

  // N^T = s N^T + R^T W^T over the K-steps that hold new rows; the weights
  // as bf16 pairs hi = rne(w), lo = rne(w - hi)
#pragma unroll
  for (int t = 0; t < kAT; ++t) acc[t] *= s_old;
#pragma unroll
  for (int s = 0; s < 2 * kRB; ++s) {
    if (s < nks) {
      uint32_t whi[4], wlo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const f32x2 w2 = {sc[s >> 1][8 * (s & 1) + e], sc[s >> 1][8 * (s & 1) + e + 1]};
        const bf16x2 h2 = __builtin_convertvector(w2, bf16x2);
        const f32x2 r2 = w2 - __builtin_convertvector(h2, f32x2);
        whi[e / 2] = __builtin_bit_cast(uint32_t, h2);
        wlo[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
      }
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, uint4{whi[0], whi[1], whi[2], whi[3]});
      const bf16x8 blo = __builtin_bit_cast(bf16x8, uint4{wlo[0], wlo[1], wlo[2], wlo[3]});
#pragma unroll
      for (int t = 0; t < kAT; ++t) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u16x8*>(&RT[((kAT * q + t) * 32 + ln) * RTS + 16 * s + 8 * hi]));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bhi, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, blo, acc[t], 0, 0, 0);
      }
    }
  }
  return l_new;
}

// The pooled slots n / l of the wave's accumulator tiles -> the tile's key
// tile kt (drafter operand order, 32 x d) and value tile vt ([d][32]) in LDS.
// A lane's 4 consecutive entries are 4 consecutive dimensions of its slot:
// one 8-byte write in the key tile, 4 rows of the value tile.
template <int kAT>
__device__ __forceinline__ void pooled_to_lds(const f32x16 (&acc)[kAT], float il, int q, int lane,
                                              uint16_t* kt, uint16_t* vt) {
  constexpr int D = kMergeD;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int ln = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int t = 0; t < kAT; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ent = (kAT * q + t) * 32 + 8 * k + 4 * hi;  // first of the 4 entries
      const bf16x2 p0 = __builtin_convertvector((f32x2{acc[t][4 * k], acc[t][4 * k + 1]} * il), bf16x2);
      const bf16x2 p1 = __builtin_convertvector((f32x2{acc[t][4 * k + 2], acc[t][4 * k + 3]} * il), bf16x2);
      if ((kAT * q + t) * 32 < D) {  // key entries (uniform in the wave)
        *reinterpret_cast<uint2*>(&kt[key_index(0, 32, D, ln, ent)]) =
            uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
      } else {
        const uint32_t w0 = __builtin_bit_cast(uint32_t, p0), w1 = __builtin_bit_cast(uint32_t, p1);
        uint16_t* v = vt + (ent - D) * 32 + ln;
        v[0] = uint16_t(w0);
        v[32] = uint16_t(w0 >> 16);
        v[64] = uint16_t(w1);
        v[96] = uint16_t(w1 >> 16);
      }
    }
}

}  // namespace
}  // namespace ls
