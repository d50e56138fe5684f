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
// bf16, d = 128 (draft_direct).  A workgroup takes one KV head unit, 32 of
// its query rows (two row groups of 16) and one key range; its KPW = 8
// waves (two per SIMD) are 8 key parts.  The keys are cut in 32-key chunks
// that never straddle two views (W and S are multiples of 32; the block
// gets its own chunks), and the chunks of a range are dealt to its waves in
// turn.  Each wave loads every MFMA operand of its window and slot chunks
// straight from memory into registers, with no LDS and no barrier in the
// loop:
//   S^T = K Q^T : A = 16 keys x 32 dimensions; the window and slot keys are
//                 stored in this operand order (tiles of 32 keys), so each
//                 64-lane load is 1 KB contiguous; B = the query rows
//                 (registers, loaded once);
//   O^T += V^T P^T : A = 16 dimensions x 32 keys from the value tiles
//                 [d][32] (1 KB contiguous per load); B = the softmax
//                 weights from the S^T output layout, rounded to bf16.
// A wave holds one chunk's key half and value half (8 loads each); the next
// chunk's keys are requested as soon as the current scores are formed and
// its values as soon as the current P.V is issued, so one chunk is always
// in flight.  No load sits behind a branch, so the compiler waits only for
// the loads a step uses.  Every loaded operand serves both row groups.  The
// verified block arrives token-major from the caller; each of its (at most
// two) chunks is loaded by the wave whose turn it falls on, at the start,
// transposed through that wave's own LDS region and computed first, while
// the wave's other loads are in flight.  The online softmax lives in
// registers (per query row, per lane) in base 2; the key parts merge
// (m, l, O) in LDS at the end, each wave combining 2 of the 16 (row group,
// dimension block) pieces, and key ranges, when there is more than one,
// through the workspace and draft_combine (a kernel boundary, no
// device-scope fence).
// f32 (draft_generic): one workgroup per query row, plain loop (small shapes).
#include "common.hpp"
#include "draft_ops.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;
// Workgroup = (unit, 32 query rows ridx, key range kidx): blockIdx =
// unit + units * (kidx + ksplit * ridx), so the workgroups of one unit sit
// on one XCD when units is a multiple of 8 and the keys they share are
// fetched from HBM once.  The window and slot chunks of key range kidx are
// those with chunk % (ksplit*KPW) in [kidx*KPW, kidx*KPW + KPW); wave kq
// takes residue kidx*KPW + kq.  Block chunk b belongs to key part b (wave b
// of the first key range): the first wave of each SIMD gets its loads into
// the memory pipeline microseconds before the second, so the block chunk
// goes where the chain starts early.  The owner stages it in its own LDS
// slot and computes it before its other chunks, while their first loads are
// in flight.  kEvery: every wave has at least one window or slot
// chunk (checked by the host), so the first loads need no branch.  With
// ksplit = 1 the output is written here, else the range's (m, l, O) go to
// the workspace: [unit][kidx][m[64] | l[64] | O[64][d]].
template <int KPW, bool kEvery>
__global__ __launch_bounds__(64 * KPW, 1) void draft_direct(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ ring_k,
    const uint16_t* __restrict__ ring_v, const int32_t* __restrict__ ring_pos,
    const uint16_t* __restrict__ slot_k, const uint16_t* __restrict__ slot_v,
    uint16_t* __restrict__ out, float* __restrict__ part_out, int Hq, int Hkv, int W, int S, int B,
    int units, int ksplit) {
  constexpr int D = 128;
  static_assert(16 % KPW == 0, "the merge deals 16 (row group, dimension block) pieces to the waves");
  // one LDS slot per wave, touched only by that wave until the merge: first
  // its block chunk (if it owns one), then its (m, l, O) partial
  constexpr int kRedFloats = 2 * 34 * 64;  // per row group: m[64], l[64], O[8 pieces][64 lanes][4]
  constexpr int kSlotElems = (kBlkElems > 2 * kRedFloats) ? kBlkElems : 2 * kRedFloats;
  static_assert(KPW * kSlotElems * 2 <= 160 * 1024, "the wave slots must fit the LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[KPW * kSlotElems];

  const int unit = blockIdx.x % units, split = blockIdx.x / units;
  const int kidx = split % ksplit, ridx = split / ksplit;
  const int c = unit / Hkv, h = unit % Hkv;
  const int G = Hq / Hkv, M = B * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kq = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int ln = lane & 15, kg = lane >> 4;

  const int nring = W / 32, ngl = nring + S / 32, nblk = (B + 31) / 32;
  const int nparts = ksplit * KPW, pidx = kidx * KPW + kq;
  const uint16_t* rk = ring_k + int64_t(unit) * W * D;
  const uint16_t* rv = ring_v + int64_t(unit) * D * W;
  const uint16_t* sk = slot_k + int64_t(unit) * S * D;
  const uint16_t* sv = slot_v + int64_t(unit) * D * S;
  const int32_t* rp = ring_pos + int64_t(c) * W;

  // this wave's window / slot chunks: pidx, pidx + nparts, ...
  const int nmine = ngl > pidx ? (ngl - pidx + nparts - 1) / nparts : 0;
  auto keys_of = [&](Half& x, int j) {
    const int ch = pidx + j * nparts;
    const bool ring = ch < nring;
    load_keys(x, ring ? rk + int64_t(ch) * 32 * D : sk + int64_t(ch - nring) * 32 * D,
              ring ? rp + ch * 32 : kSlotPos, ring, lane);
  };
  auto values_of = [&](Half& x, int j) {
    const int ch = pidx + j * nparts;
    const bool ring = ch < nring;
    load_values(x, ring ? rv + int64_t(ch) * D * 32 : sv + int64_t(ch - nring) * D * 32, lane);
  };

  // the block chunk this wave owns, if any: B <= 47 gives at most 2 block
  // chunks, which land on 2 different waves since there are at least 2
  static_assert(KPW >= 2, "each block chunk gets a wave of its own");
  const int own = pidx < nblk ? pidx : -1;
  const bool owns = own >= 0;
  // the owned block chunk: the key operands straight from the caller's rows
  // (lane (kg, ln) of load mb * 4 + ks: key chunk_key(ln, mb), dimensions
  // 32 ks + 8 kg .. +7), the value rows as 16-byte pieces for LDS; rows past
  // B repeat row B-1 and are masked
  Half bk;
  u16x8 bv_r[8];
  if (owns) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int key = min(own * 32 + chunk_key(ln, mb), B - 1);
        bk.r[mb * 4 + ks] = *reinterpret_cast<const u16x8*>(kb + ((int64_t(c) * B + key) * Hkv + h) * D + ks * 32 + kg * 8);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int piece = lane + 64 * i, row = piece >> 4, col = (piece & 15) * 8;
      const int key = min(own * 32 + row, B - 1);
      bv_r[i] = *reinterpret_cast<const u16x8*>(vb + ((int64_t(c) * B + key) * Hkv + h) * D + col);
    }
  }

  // query operands: lane (row ln of group rg, kg) holds q[row][ks*32+kg*8..+7]
  bf16x8 qb[2][4];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int row = ridx * 32 + rg * 16 + ln;
    const bool ok = row < M;
    const int bq = ok ? row / G : 0, hq = h * G + (ok ? row % G : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(q + ((int64_t(c) * B + bq) * Hq + hq) * D + ks * 32 + kg * 8);
      qb[rg][ks] = as_bf16x8(ok ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
  }

  // the first chunk's halves
  Half hk, hv;
  if (kEvery || nmine > 0) {
    keys_of(hk, 0);
    values_of(hv, 0);
  }

  Softmax st[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    st[rg].m = -INFINITY;
    st[rg].l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st[rg].o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the owned block chunk first: its value rows -> this wave's LDS slot
  // (row-major) -> the [dimension][8 keys] operands by transposed reads; only
  // this wave touches the slot, so a wave barrier orders the writes before
  // the reads.  ds_read_b64_tr_b16 gives lane 4a + b of a 16-lane group
  // element b of the 8-byte reads of lanes a, a+4, a+8, a+12: reader lane ln
  // of group kg reads row 8 kg + ln / 4 (+ 4 for keys 4..7) at dimensions
  // 16 db + 4 (ln % 4) .. +3, so lane ln receives keys 8 kg .. 8 kg + 3 (+4)
  // of dimension 16 db + ln, the layout of a value tile's operand.
  auto block_chunk = [&](int b) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    uint16_t* bv = lds + kq * kSlotElems;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int piece = lane + 64 * i, row = piece >> 4, col = (piece & 15) * 8;
      *reinterpret_cast<u16x8*>(bv + row * kBVS + col) = bv_r[i];
    }
    __builtin_amdgcn_wave_barrier();
    Half xv;
    const uint16_t* rd = bv + (8 * kg + (ln >> 2)) * kBVS + 4 * (ln & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(rd + 16 * db));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(rd + 4 * kBVS + 16 * db));
      xv.r[db] = __builtin_bit_cast(u16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const Half& xk = bk;
    const int nvalid = B - b * 32 - 8 * kg;  // block keys among the lane group's 8
    const uint32_t valid8 = nvalid >= 8 ? 0xFFu : nvalid <= 0 ? 0u : ((1u << nvalid) - 1u);
    f32x4 sc[2][2];
    chunk_scores(sc, xk, qb);
    bf16x8 pk[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) pk[rg] = softmax_chunk(st[rg], sc[rg], valid8, false);
    chunk_pv(st, xv, pk);
  };
  if (owns) block_chunk(own);

  // window / slot chunks: chunk j+1's keys are requested as soon as chunk
  // j's scores are formed, its values as soon as chunk j's P.V is issued,
  // so a chunk is always in flight; the last step requests nothing.
  auto step = [&](bool more, int j) {
    const uint64_t mask = __ballot(hk.pos >= 0);  // bit k (and k+32): key k present
    f32x4 s[2][2];
    chunk_scores(s, hk, qb);
    if (more) keys_of(hk, j + 1);
    const bool full = mask == ~0ull;
    const uint32_t valid8 = uint32_t(mask >> (8 * kg)) & 0xFFu;
    bf16x8 pk[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) pk[rg] = softmax_chunk(st[rg], s[rg], valid8, full);
    chunk_pv(st, hv, pk);
    if (more) values_of(hv, j + 1);
  };
  for (int j = 0; j < nmine - 1; ++j) step(true, j);
  if (nmine > 0) step(false, nmine - 1);

  // merge the key parts: each wave leaves (m, l, O) in its own slot as soon
  // as its chunks are done (per row group: m and l with the lanes contiguous,
  // then the 8 output pieces with each lane's 4 values contiguous, so every
  // access is a wave's 256 bytes or 1 KB in a row); after one barrier each
  // wave combines 16 / KPW of the 16 (row group, dimension block) pieces
  float lt[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    lt[rg] = st[rg].l;
    lt[rg] += __shfl_xor(lt[rg], 16, 64);
    lt[rg] += __shfl_xor(lt[rg], 32, 64);
  }
  auto ml_at = [&](int k, int rg, int e) {
    return reinterpret_cast<float*>(lds + k * kSlotElems) + (rg * 34 + e) * 64 + lane;
  };
  auto o_at = [&](int k, int rg, int mb) {
    return reinterpret_cast<f32x4*>(reinterpret_cast<float*>(lds + k * kSlotElems) + (rg * 34 + 2) * 64) +
           mb * 64 + lane;
  };
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    *ml_at(kq, rg, 0) = st[rg].m;
    *ml_at(kq, rg, 1) = lt[rg];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) *o_at(kq, rg, mb) = st[rg].o[mb];
  }
  __syncthreads();
  constexpr int kPer = 16 / KPW;  // pieces per wave, all in one row group
  static_assert(8 % kPer == 0, "a wave's pieces share their row group");
  const int rgw = (kq * kPer) >> 3;
  // every read of the wave's pieces is issued before the arithmetic, so the
  // LDS round trips overlap instead of forming a chain per key part; the
  // parts' (m, l) and weights serve both pieces
  float pm[KPW], pl[KPW], wk[KPW];
  f32x4 po[kPer][KPW];
#pragma unroll
  for (int k = 0; k < KPW; ++k) {
    pm[k] = *ml_at(k, rgw, 0);
    pl[k] = *ml_at(k, rgw, 1);
  }
#pragma unroll
  for (int pc = 0; pc < kPer; ++pc) {
    const int mb = (kq * kPer + pc) & 7;
#pragma unroll
    for (int k = 0; k < KPW; ++k) po[pc][k] = *o_at(k, rgw, mb);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KPW; ++k) mx = fmaxf(mx, pm[k]);
#pragma unroll
  for (int k = 0; k < KPW; ++k) wk[k] = pm[k] == -INFINITY ? 0.f : exp2_f(pm[k] - mx);
#pragma unroll
  for (int pc = 0; pc < kPer; ++pc) {
    const int mb = (kq * kPer + pc) & 7;
    const int row = ridx * 32 + rgw * 16 + ln;
    float l = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KPW; ++k) {
      l = fmaf(pl[k], wk[k], l);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = fmaf(po[pc][k][r], wk[k], o[r]);
    }
    if (row >= M) continue;
    if (ksplit == 1) {  // the whole key list: write the output
      const float il = 1.0f / l;
      uint16_t* orow = out + ((int64_t(c) * B + row / G) * Hq + h * G + row % G) * D;
      *reinterpret_cast<u16x4*>(orow + mb * 16 + kg * 4) =
          u16x4{bf16_bits(o[0] * il), bf16_bits(o[1] * il), bf16_bits(o[2] * il), bf16_bits(o[3] * il)};
    } else {  // partial of this key range (m in base 2)
      constexpr int Mpad = 64;
      float* pbuf = part_out + (int64_t(unit) * ksplit + kidx) * int64_t(Mpad) * (D + 2);
      if (kg == 0 && mb == 0) {
        pbuf[row] = mx;
        pbuf[Mpad + row] = l;
      }
      *reinterpret_cast<f32x4*>(pbuf + 2 * Mpad + int64_t(row) * D + mb * 16 + kg * 4) = o;
    }
  }
}

// merge the key ranges: one thread per (unit, query row, 4 dimensions)
__global__ __launch_bounds__(kThreads) void draft_combine(
    const float* __restrict__ part, uint16_t* __restrict__ out, int Hq, int Hkv, int B,
    int halves, int Mpad, int units) {
  constexpr int D = 128;
  const int G = Hq / Hkv, M = B * G;
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int e4 = int(idx % (D / 4)) * 4;
  const int row = int((idx / (D / 4)) % Mpad);
  const int unit = int(idx / (int64_t(D / 4) * Mpad));
  if (unit >= units || row >= M) return;
  const int c = unit / Hkv, h = unit % Hkv;
  const int64_t pstride = int64_t(Mpad) * (D + 2);
  const float* ub = part + int64_t(unit) * halves * pstride;
  float ms[4], ls[4];
  f32x4 os[4];
  float mx = -INFINITY;
  for (int s2 = 0; s2 < halves; ++s2) {
    const float* sp = ub + s2 * pstride;
    ms[s2] = sp[row];
    ls[s2] = sp[Mpad + row];
    os[s2] = *reinterpret_cast<const f32x4*>(sp + 2 * Mpad + int64_t(row) * D + e4);
    mx = fmaxf(mx, ms[s2]);
  }
  float l = 0.f;
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < halves; ++s2) {
    const float wgt = ms[s2] == -INFINITY ? 0.f : exp2_f(ms[s2] - mx);
    l = fmaf(ls[s2], wgt, l);
    a += os[s2] * wgt;
  }
  const float il = 1.0f / l;
  uint16_t* orow = out + ((int64_t(c) * B + row / G) * Hq + h * G + row % G) * D + e4;
  *reinterpret_cast<u16x4*>(orow) = u16x4{bf16_bits(a[0] * il), bf16_bits(a[1] * il),
                                          bf16_bits(a[2] * il), bf16_bits(a[3] * il)};
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

  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  __syncthreads();
  for (int k0 = 0; k0 < N; k0 += kThreads) {
    const int key = k0 + tid;
    float a = -INFINITY;
    if (key < N && (key >= W || ring_pos[int64_t(c) * W + key] >= 0)) {
      float dot = 0.f;
      if (key < W) {
        for (int e = 0; e < D; ++e) dot = fmaf(qs[e], Ty::load(ring_k, key_index(unit, W, D, key, e)), dot);
      } else if (key < W + S) {
        for (int e = 0; e < D; ++e)
          dot = fmaf(qs[e], Ty::load(slot_k, key_index(unit, S, D, key - W, e)), dot);
      } else {
        for (int e = 0; e < D; ++e)
          dot = fmaf(qs[e], Ty::load(kb, ((int64_t(c) * B + key - W - S) * Hkv + h) * D + e), dot);
      }
      a = dot * sm_scale;
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
        if (pk == 0.f) continue;
        const int kk = k0 + k;
        float v;  // values of the window and of the slots are key-tiled
        if (kk < W)
          v = Ty::load(ring_v, value_index(unit, W, D, kk, tid));
        else if (kk < W + S)
          v = Ty::load(slot_v, value_index(unit, S, D, kk - W, tid));
        else
          v = Ty::load(vb, ((int64_t(c) * B + kk - W - S) * Hkv + h) * D + tid);
        o = fmaf(pk, v, o);
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
    const int units = d.C * d.Hkv;
    const int rsplit = draft_row_splits(d), ksplit = draft_halves(d);
    float* part = reinterpret_cast<float*>(static_cast<char*>(st.workspace) + ws_layout(d, 1).draft_part);
    const int ngl = d.W / 32 + d.S / 32;  // window and slot chunks
    auto kernel = ngl >= ksplit * kKPW ? draft_direct<kKPW, true> : draft_direct<kKPW, false>;
    hipLaunchKernelGGL(kernel, dim3(units * ksplit * rsplit), dim3(64 * kKPW), 0,
                       stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kb),
                       static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(st.ring_k),
                       static_cast<const uint16_t*>(st.ring_v), st.ring_pos,
                       static_cast<const uint16_t*>(st.slot_k), static_cast<const uint16_t*>(st.slot_v),
                       static_cast<uint16_t*>(out), part, d.Hq, d.Hkv, d.W, d.S, d.B, units, ksplit);
    if (hipGetLastError() != hipSuccess) return LS_ERR_HIP;
    if (ksplit > 1) {
      const int Mpad = 64;
      const int64_t threads = int64_t(units) * Mpad * (128 / 4);
      hipLaunchKernelGGL(draft_combine, dim3(unsigned(cdiv(threads, kThreads))), dim3(kThreads), 0,
                         stream, part, static_cast<uint16_t*>(out), d.Hq, d.Hkv, d.B, ksplit, Mpad, units);
    }
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
