// One drafting round's update and draft attention in a single launch
// (LongSpark paper page, Fig. 2: (a) the target verifies the block, (b) the
// views are updated with the accepted rows, (c) the drafter attends over the
// views; Fig. 3: only the newly retained rows enter the summary).
//
// ls_verify_append_draft = the verification's key pass (ls_verify_keys:
// verify.hip, which also takes the length snapshot and zeroes the arrival
// counters), then update_draft below (ls_update_draft): the same results as ls_verify_append followed by
// ls_draft_attention, in two launches instead of three.  The state comes out
// bit for bit as from the update kernel (the same merge, merge_ops.hpp); the
// attention output equals the draft kernel's up to the order in which the
// softmax visits the keys (the new window rows and the slots are chunks of
// their own here).
//
// Workgroup = (unit (c, h), 32 query rows ridx), 8 waves; the R workgroups
// of a unit are `units` blocks apart, so they run on one XCD and share the
// unit's reads in its L2.  The waves split by role, so that the merge and
// the window reads overlap instead of following each other:
//  * waves 0 .. S/32-1, the updaters: wave t loads slot tile t's state while
//    the rows are staged, merges the tile with the tau new rows, attends over
//    the pooled tile straight from its own LDS output, then over its share
//    of the window chunks (the last chunks of the ring).  Updater S/32-1
//    also takes the chunk of new rows, updater S/32-2 (or 0) the chunk of
//    block rows (k_blk, v_blk; staged in LDS with the verified rows).  The
//    updaters copy the new rows into the ring.
//  * the other waves, the drafters: request their first window chunk at once
//    and run through their chunks (the old rows; the slots (L + i) mod W,
//    i < tau, that the new rows replace are masked, as are empty ones).
// Every workgroup of the unit merges every tile from the state as it was
// before the round (its drafters need all pooled tiles); tile t's state is
// written by the last of the unit's R waves that merged it to finish (a
// counter per (unit, tile), which that wave sets back to zero): a wave
// that starts late must not read a tile that a sibling has already updated.
// Nobody waits: the others skip the stores.  Slot tile t goes out from the
// workgroup with t % R == ridx (the pooled tiles are identical in all of
// them).  The lead workgroup of the sequence writes target_tok, tau,
// ring_pos and seq_len = L + tau (L from the snapshot: no workgroup here
// reads seq_len).  The key parts of the 8 waves merge in LDS as in the
// draft kernel; a wave fills its merge slot as soon as it is done and the
// updaters have counted themselves out of the LDS that the slots overlay.
#include "accept.hpp"
#include "common.hpp"
#include "draft_ops.hpp"
#include "launch.hpp"
#include "merge_ops.hpp"

#include <algorithm>

#ifndef LS_ROUND_UPD_WIN
#define LS_ROUND_UPD_WIN 2
#endif

namespace ls {
namespace {

constexpr int kRoundUpdWin = LS_ROUND_UPD_WIN;  // window chunks per updater wave (at most)

struct RoundKeys {          // the verification's partial keys and its outputs
  const uint64_t* keys;
  int nkeys;
  const int32_t* draft;
  int32_t* target_tok;
  int32_t* tau_out;
  int32_t* arrivals;        // [C*Hkv*S/32], zero at launch; zero again at exit
};

// kTiles: S / 32 slot tiles (2 or 4) = updater waves.  nd_total: the window
// chunks 0 .. nd_total-1 go to the drafters (round robin), the rest to the
// updaters.  Shapes (checked by the host): bf16, d = 128, B + 1 <= 32, W a
// positive multiple of 32, at most 64 query rows per unit.
template <int kTiles>
__global__ __launch_bounds__(64 * kKPW, 1) void update_draft(
    RoundKeys rk, const int32_t* __restrict__ len_snap, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb, uint16_t* __restrict__ ring_k,
    uint16_t* __restrict__ ring_v, int32_t* __restrict__ ring_pos, int32_t* __restrict__ seq_len,
    float* __restrict__ sum_m, float* __restrict__ sum_l, float* __restrict__ sum_n,
    uint16_t* __restrict__ slot_k, uint16_t* __restrict__ slot_v, const uint16_t* __restrict__ u,
    const float* __restrict__ log_lambda, uint16_t* __restrict__ out, int Hq, int Hkv, int W,
    int B, int units, int nd_total) {
  constexpr int D = 128, E = 2 * D, KPW = kKPW, S = 32 * kTiles, ND = KPW - kTiles;
  constexpr int kThreads = 64 * KPW;
  constexpr int RP = 32, KLS = kMergeKLS, RTS = RP + 8;
  static_assert(KPW == 8 && ND >= 1, "updaters and drafters");
  // LDS: the draft kernel's per-wave slots (key-part merge at the end),
  // overlaid until then by the pooled slot tiles, the staged rows, the slot
  // queries and the block rows (k_blk, v_blk) the drafter attends over
  constexpr int kRedFloats = 2 * 34 * 64;
  constexpr int kSlotElems = (kBlkElems > 2 * kRedFloats) ? kBlkElems : 2 * kRedFloats;
  constexpr int kPool = kTiles * 2 * 32 * D;        // pooled key and value tiles
  constexpr int kKL = kPool, kRT = kKL + RP * KLS, kUL = kRT + E * RTS, kBL = kUL + S * KLS;
  constexpr int kKB = kBL + kBlkElems;
  constexpr int kEnd = kKB + RP * KLS;
  constexpr int kLdsElems = kEnd > KPW * kSlotElems ? kEnd : KPW * kSlotElems;
  static_assert(kLdsElems * 2 + 64 * 4 <= 160 * 1024, "one workgroup's LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
  __shared__ int32_t g_tok[64];
  __shared__ int32_t upd_lds_done;  // updaters past their last read of the staged rows / pooled tiles
  uint16_t* pool = lds;
  uint16_t* KL = lds + kKL;
  uint16_t* RT = lds + kRT;
  uint16_t* UL = lds + kUL;
  uint16_t* BV = lds + kBL;  // the block's value rows [32][kBVS]
  uint16_t* KB = lds + kKB;  // and its key rows [32][KLS] (rows past B repeat row B-1)

  const int unit = blockIdx.x % units, ridx = blockIdx.x / units;
  const int R = int(gridDim.x) / units;
  const int c = unit / Hkv, h = unit % Hkv;
  const int G = Hq / Hkv, M = B * G, B1 = B + 1;
  const bool lead = h == 0 && ridx == 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kq = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int ln = lane & 15, kg = lane >> 4;
  const int nring = W / 32;
  const uint16_t* rkt = ring_k + int64_t(unit) * W * D;
  const uint16_t* rvt = ring_v + int64_t(unit) * D * W;
  const int32_t* rp = ring_pos + int64_t(c) * W;
  const int L = len_snap[c];
  const bool upd = kq < kTiles;
  // this wave's window chunks: first + j * stride, j < nmine
  const int nup = nring - nd_total;
  const int first = upd ? nd_total + kq : kq - kTiles;
  const int stride = upd ? kTiles : ND;
  const int nmine = upd ? (nup > kq ? (nup - kq + kTiles - 1) / kTiles : 0)
                        : (nd_total > kq - kTiles ? (nd_total - (kq - kTiles) + ND - 1) / ND : 0);

  bf16x8 qb[2][4];
  auto load_q = [&]() {
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
  };
  auto keys_of = [&](Half& x, int j) {
    const int ch = first + j * stride;
    load_keys(x, rkt + int64_t(ch) * 32 * D, rp + ch * 32, true, lane);
  };
  auto values_of = [&](Half& x, int j) {
    load_values(x, rvt + int64_t(first + j * stride) * D * 32, lane);
  };

  // the unit's B+1 verified rows (row-major keys KL, transposed [k | v] RT,
  // rows past B+1 zero), its S slot queries UL and the drafted block's B rows
  // (row-major KB and BV); the verified rows' argmax tokens into g_tok.
  // Every thread takes part; the caller then meets a barrier.
  // (Requesting these before the role's large loads does not bring that
  // barrier forward: the first ~7 us of the kernel are the whole grid's
  // initial requests, about 200 KB per CU, arriving at the memory's rate.)
  constexpr int kItems = RP * (E / 8) / kThreads;
  static_assert(kItems * kThreads == RP * (E / 8), "whole passes");
  constexpr int kUItems = S * (D / 8) / kThreads;
  static_assert(kUItems * kThreads == S * (D / 8), "whole passes");
  constexpr int kBItems = 2 * RP * (D / 8) / kThreads;  // block keys, then values
  static_assert(kBItems * kThreads == 2 * RP * (D / 8), "whole passes");
  auto stage = [&]() {
    if (tid == 0) upd_lds_done = 0;  // read only after the staging barrier
    u16x8 x[kItems], xu[kUItems], xb[kBItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int p = it * kThreads + tid, row = p % RP, pc = p / RP;
      const int half = pc >> 4, e = pc & 15;
      const int rc = min(row, B1 - 1);  // rows past B+1 load a real row and are zeroed
      x[it] = *reinterpret_cast<const u16x8*>((half ? v_new : k_new) + ((int64_t(c) * B1 + rc) * Hkv + h) * D + 8 * e);
    }
#pragma unroll
    for (int it = 0; it < kUItems; ++it) {
      const int p = it * kThreads + tid, sl = p >> 4, pc = p & 15;
      xu[it] = *reinterpret_cast<const u16x8*>(u + (int64_t(h) * S + sl) * D + 8 * pc);
    }
#pragma unroll
    for (int it = 0; it < kBItems; ++it) {
      const int p = it * kThreads + tid, half = p / (RP * (D / 8)), row = (p >> 4) % RP, pc = p & 15;
      const int key = min(row, B - 1);  // rows past B load a real row; their scores are masked
      xb[it] = *reinterpret_cast<const u16x8*>((half ? vb : kb) + ((int64_t(c) * B + key) * Hkv + h) * D + 8 * pc);
    }
    accept_rows<kThreads>(rk.keys, rk.nkeys, c, B, g_tok, lead ? rk.target_tok : nullptr);
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int p = it * kThreads + tid, row = p % RP, pc = p / RP;
      const int half = pc >> 4, e = pc & 15;
      const u16x8 v = row < B1 ? x[it] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (!half) *reinterpret_cast<u16x8*>(&KL[row * KLS + 8 * e]) = v;
#pragma unroll
      for (int r = 0; r < 8; ++r) RT[(half * D + 8 * e + r) * RTS + row] = v[r];
    }
#pragma unroll
    for (int it = 0; it < kUItems; ++it) {
      const int p = it * kThreads + tid, sl = p >> 4, pc = p & 15;
      *reinterpret_cast<u16x8*>(&UL[sl * KLS + 8 * pc]) = xu[it];
    }
#pragma unroll
    for (int it = 0; it < kBItems; ++it) {
      const int p = it * kThreads + tid, half = p / (RP * (D / 8)), row = (p >> 4) % RP, pc = p & 15;
      *reinterpret_cast<u16x8*>(half ? &BV[row * kBVS + 8 * pc] : &KB[row * KLS + 8 * pc]) = xb[it];
    }
  };

  Softmax st[2];  // started by each role where its attention begins
  auto start_softmax = [&]() {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      st[rg].m = -INFINITY;
      st[rg].l = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) st[rg].o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  const int32_t dj = lane < B ? rk.draft[int64_t(c) * B + lane] : 0;

  // window chunks of this wave: the next chunk's keys are requested once the
  // current scores exist, its values once the current P.V is issued.
  // Present = occupied (ring_pos >= 0) and not replaced this round
  // ((slot - L) mod W >= tau; those slots' rows and positions are being
  // rewritten by the updaters, and their contents do not matter)
  auto window = [&](Half& hk, Half& hv, int Tn) {
    auto step = [&](bool more, int jj) {
      const int slot = (first + jj * stride) * 32 + (lane & 31);
      const int dist = ((slot - L) % W + W) % W;
      const uint64_t mask = __ballot(hk.pos >= 0 && dist >= Tn);
      f32x4 s[2][2];
      chunk_scores(s, hk, qb);
      if (more) keys_of(hk, jj + 1);
      const bool full = mask == ~0ull;
      const uint32_t valid8 = uint32_t(mask >> (8 * kg)) & 0xFFu;
      bf16x8 pk[2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) pk[rg] = softmax_chunk(st[rg], s[rg], valid8, full);
      chunk_pv(st, hv, pk);
      if (more) values_of(hv, jj + 1);
    };
    for (int jj = 0; jj < nmine - 1; ++jj) step(true, jj);
    if (nmine > 0) step(false, nmine - 1);
  };
  // one chunk held in registers (keys in operand order, values [d][32])
  auto lds_chunk = [&](const Half& xk, const Half& xv, uint32_t valid8, bool full) {
    f32x4 sc[2][2];
    chunk_scores(sc, xk, qb);
    bf16x8 pk[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) pk[rg] = softmax_chunk(st[rg], sc[rg], valid8, full);
    chunk_pv(st, xv, pk);
  };

  if (upd) {
    // ---------------- updater: slot tile tl = kq
    const int tl = kq;
    const int l32 = lane & 31, hi = lane >> 5;
    const int j = tl * 32 + l32;                  // this lane's slot
    const int64_t sidx = int64_t(unit) * S + j;
    float* nt = sum_n + (int64_t(unit) * S + tl * 32) * E + lane * 4;
    f32x16 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(nt + (t * 4 + k) * 64 * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][4 * k + r] = v[r];
      }
    const float m_old = sum_m[sidx], l_old = sum_l[sidx], lnl = log_lambda[j];
    stage();
    __syncthreads();  // staging complete
    const int Tn = accept_tau(g_tok, dj, B);
    if (lead && tid == 0) rk.tau_out[c] = Tn;
    // the window: this workgroup's share of the unit's copies (Tn 16-byte
    // key pieces, then 128 Tn value elements, lanes over rows), from the
    // staged rows, by the updater threads
    {
      constexpr int kUT = 64 * kTiles;
      const int nk = Tn * (D / 8), n_all = nk + D * Tn;
      const int per = (n_all + R - 1) / R;
      const int p0 = ridx * per, p1 = min(n_all, p0 + per);
      for (int p = p0 + tid; p < p1; p += kUT) {
        if (p < nk) {
          const int i = p >> 4, e = p & 15;
          const int slot = (L + i) % W;
          *reinterpret_cast<u16x8*>(ring_k + key_index(unit, W, D, slot, 8 * e)) =
              *reinterpret_cast<const u16x8*>(&KL[i * KLS + 8 * e]);
        } else {
          const int qq = p - nk, dim = qq / Tn, i = qq - dim * Tn;
          ring_v[value_index(unit, W, D, (L + i) % W, dim)] = RT[(D + dim) * RTS + i];
        }
      }
      if (lead && tid < Tn) ring_pos[int64_t(c) * W + (L + tid) % W] = L + tid;
      if (lead && tid == 0) seq_len[c] = L + Tn;
    }
    float m_new;
    const float l_new = merge_wave<1, 8>(KL, RT, UL + 32 * tl * KLS, acc, m_old, l_old, lnl, Tn, 0,
                                         lane, m_new);
    // this wave has used its state loads: count it in for tile tl (the
    // empty asm makes the increment depend on the merged accumulators, and so
    // on every state load, so the atomic cannot be issued before they are
    // in); the reply is read after the pooled tile is in LDS
    int32_t before = 0;
    if (R > 1) {
      int one = 1;
      asm volatile("" : "+v"(one)
                   : "v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]), "v"(acc[4]), "v"(acc[5]),
                     "v"(acc[6]), "v"(acc[7]), "v"(l_new));
      if (lane == 0)
        before = __hip_atomic_fetch_add(rk.arrivals + int64_t(unit) * kTiles + tl, one, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    }
    uint16_t* kt = pool + tl * 2 * 32 * D;
    pooled_to_lds<8>(acc, 1.0f / l_new, 0, lane, kt, kt + 32 * D);
    const bool writer = R == 1 || __builtin_amdgcn_readfirstlane(before) == R - 1;
    // the last arrival also rearms the counter for the next launch
    if (R > 1 && writer && lane == 0)
      __hip_atomic_store(rk.arrivals + int64_t(unit) * kTiles + tl, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (writer) {  // every sibling's wave for this tile has read the old state
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          __builtin_nontemporal_store(f32x4{acc[t][4 * k], acc[t][4 * k + 1], acc[t][4 * k + 2], acc[t][4 * k + 3]},
                                      reinterpret_cast<f32x4*>(nt + (t * 4 + k) * 64 * 4));
      if (hi == 0) {
        sum_m[sidx] = m_new;
        sum_l[sidx] = l_new;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (tl % R == ridx) {  // the slot tile, from this wave's own LDS output
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      constexpr int P16 = 32 * D * 2 / 16;  // 16-byte pieces per key (or value) tile
      for (int p = lane; p < 2 * P16; p += 64) {
        const u32x4 val = *reinterpret_cast<const u32x4*>(kt + p * 8);
        u32x4* dst = p < P16 ? reinterpret_cast<u32x4*>(slot_k + key_index(unit, S, D, tl * 32, 0)) + p
                             : reinterpret_cast<u32x4*>(slot_v + value_index(unit, S, D, tl * 32, 0)) + (p - P16);
        __builtin_nontemporal_store(val, dst);
      }
    }
    load_q();
    start_softmax();
    {  // the pooled tile
      Half xk, xv;
#pragma unroll
      for (int i = 0; i < 8; ++i) xk.r[i] = *reinterpret_cast<const u16x8*>(kt + (i * 64 + lane) * 8);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        xv.r[db] = *reinterpret_cast<const u16x8*>(kt + 32 * D + (db * 16 + ln) * 32 + kg * 8);
      lds_chunk(xk, xv, 0xFFu, true);
    }
    if (kq == kTiles - 1) {  // the new rows: keys from KL, values from RT, rows >= tau masked
      Half xk, xv;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          xk.r[mb * 4 + ks] = *reinterpret_cast<const u16x8*>(&KL[chunk_key(ln, mb) * KLS + ks * 32 + kg * 8]);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        xv.r[db] = *reinterpret_cast<const u16x8*>(&RT[(D + db * 16 + ln) * RTS + kg * 8]);
      const int nvalid = Tn - 8 * kg;
      const uint32_t valid8 = nvalid >= 8 ? 0xFFu : nvalid <= 0 ? 0u : ((1u << nvalid) - 1u);
      lds_chunk(xk, xv, valid8, false);
    }
    if (kq == (kTiles > 1 ? kTiles - 2 : 0)) {
      // the drafted block (one chunk: B <= 31), staged with the verified
      // rows: key operands from its row-major keys (as the new rows), value
      // operands by transposed reads of its row-major values
      typedef short i16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      Half bk, xv;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          bk.r[mb * 4 + ks] = *reinterpret_cast<const u16x8*>(&KB[chunk_key(ln, mb) * KLS + ks * 32 + kg * 8]);
      const uint16_t* rd = BV + (8 * kg + (ln >> 2)) * kBVS + 4 * (ln & 3);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(rd + 16 * db));
        const i16x4 hi2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(rd + 4 * kBVS + 16 * db));
        xv.r[db] = __builtin_bit_cast(u16x8, __builtin_shufflevector(lo, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      const int nvalid = B - 8 * kg;
      const uint32_t valid8 = nvalid >= 8 ? 0xFFu : nvalid <= 0 ? 0u : ((1u << nvalid) - 1u);
      lds_chunk(bk, xv, valid8, false);
    }
    // this wave reads no more LDS until the key-part merge: count it out, so
    // that the waves that finish first can fill their merge slots (which
    // overlay the staged rows and the pooled tiles) without waiting for all
    // (one lane: the count is of waves)
    if (lane == 0) __hip_atomic_fetch_add(&upd_lds_done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    Half hk, hv;  // the window chunks last (requested here: no registers to hold them earlier)
    if (nmine > 0) {
      keys_of(hk, 0);
      values_of(hv, 0);
    }
    window(hk, hv, Tn);
  } else {
    // ---------------- drafter
    load_q();
    Half hk, hv;
    if (nmine > 0) {
      keys_of(hk, 0);
      values_of(hv, 0);
    }
    stage();
    __syncthreads();  // staging complete
    const int Tn = accept_tau(g_tok, dj, B);
    start_softmax();
    window(hk, hv, Tn);
  }

  // merge the key parts (as the draft kernel).  Each wave fills its merge
  // slot as soon as its keys are done and every updater has counted out of
  // the LDS chunks that the slots overlay (normally long before; the wait is
  // bounded so that no wave can stay in it), then one barrier.
  float lt[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    lt[rg] = st[rg].l;
    lt[rg] += __shfl_xor(lt[rg], 16, 64);
    lt[rg] += __shfl_xor(lt[rg], 32, 64);
  }
  // wave k's merge slot, per row group rg: m and l (64 lanes each), then
  // the 8 output pieces with each lane's 4 values contiguous (16-byte LDS
  // accesses, a wave's 1 KB contiguous)
  auto ml_at = [&](int k, int rg, int e) {
    return reinterpret_cast<float*>(lds + k * kSlotElems) + (rg * 34 + e) * 64 + lane;
  };
  auto o_at = [&](int k, int rg, int mb) {
    return reinterpret_cast<f32x4*>(reinterpret_cast<float*>(lds + k * kSlotElems) + (rg * 34 + 2) * 64) +
           mb * 64 + lane;
  };
  for (int spin = 0; spin < (1 << 16); ++spin) {
    if (__hip_atomic_load(&upd_lds_done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= kTiles) break;
    __builtin_amdgcn_s_sleep(2);
  }
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
    const float il = 1.0f / l;
    uint16_t* orow = out + ((int64_t(c) * B + row / G) * Hq + h * G + row % G) * D;
    *reinterpret_cast<u16x4*>(orow + mb * 16 + kg * 4) =
        u16x4{bf16_bits(o[0] * il), bf16_bits(o[1] * il), bf16_bits(o[2] * il), bf16_bits(o[3] * il)};
  }
}

}  // namespace

bool round_fusable(const ls_dims& d) {
  return d.dtype == LS_BF16 && d.d == 128 && (d.S == 64 || d.S == 128) && d.B + 1 <= 32 &&
         d.W >= 32 && d.W % 32 == 0 && draft_row_splits(d) <= 2;
}

ls_status launch_round_keys(const ls_dims& d, const ls_state& st, const void* logits,
                            hipStream_t stream) {
  char* ws = static_cast<char*>(st.workspace);
  const WsLayout lay = ws_layout(d, 1);
  return launch_verify_keys(d, logits, ws, st.seq_len, reinterpret_cast<int32_t*>(ws + lay.len_snap),
                            stream, reinterpret_cast<int32_t*>(ws + lay.arrivals));
}

ls_status launch_update_draft(const ls_dims& d, const ls_state& st, const int32_t* draft,
                              int32_t* target_tok, int32_t* tau, const void* k_new,
                              const void* v_new, const void* q, const void* k_blk,
                              const void* v_blk, void* out, hipStream_t stream) {
  if (!round_fusable(d)) {  // the update over the keys, then the draft kernel
    const ls_status s1 = launch_append_from_keys(d, st, draft, target_tok, tau, k_new, v_new, stream);
    return s1 != LS_OK ? s1 : launch_draft(d, st, q, k_blk, v_blk, out, stream);
  }
  char* ws = static_cast<char*>(st.workspace);
  const WsLayout lay = ws_layout(d, 1);
  const RoundKeys rk{reinterpret_cast<const uint64_t*>(ws + lay.verify_part), lay.vsplit, draft,
                     target_tok, tau, reinterpret_cast<int32_t*>(ws + lay.arrivals)};
  const int units = d.C * d.Hkv;
  const int tiles = d.S / 32, nring = d.W / 32;
  // the updaters take up to LS_ROUND_UPD_WIN window chunks each, as long as
  // every drafter keeps one
  const int nd_total = nring - std::min(kRoundUpdWin * tiles, std::max(0, nring - (kKPW - tiles)));
  auto kernel = d.S == 128 ? update_draft<4> : update_draft<2>;
  hipLaunchKernelGGL(kernel, dim3(unsigned(units * draft_row_splits(d))), dim3(64 * kKPW), 0, stream,
                     rk, reinterpret_cast<const int32_t*>(ws + lay.len_snap),
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_blk),
                     static_cast<const uint16_t*>(v_blk), static_cast<uint16_t*>(st.ring_k),
                     static_cast<uint16_t*>(st.ring_v), st.ring_pos, st.seq_len, st.sum_m, st.sum_l,
                     st.sum_n, static_cast<uint16_t*>(st.slot_k), static_cast<uint16_t*>(st.slot_v),
                     static_cast<const uint16_t*>(st.u), st.log_lambda, static_cast<uint16_t*>(out),
                     d.Hq, d.Hkv, d.W, d.B, units, nd_total);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

ls_status launch_verify_append_draft(const ls_dims& d, const ls_state& st, const void* logits,
                                     const int32_t* draft, int32_t* target_tok, int32_t* tau,
                                     const void* k_new, const void* v_new, const void* q,
                                     const void* k_blk, const void* v_blk, void* out,
                                     hipStream_t stream) {
  const ls_status s1 = launch_round_keys(d, st, logits, stream);
  return s1 != LS_OK ? s1
                     : launch_update_draft(d, st, draft, target_tok, tau, k_new, v_new, q, k_blk,
                                           v_blk, out, stream);
}

}  // namespace ls
