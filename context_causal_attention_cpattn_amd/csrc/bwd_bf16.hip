// Block backward of causal ring attention, bf16 inputs, fp32 accumulation, MFMA (gfx950).
//
// For one ring step (local query rows against one KV block at global
// positions) and the FINAL merged LSE and delta = rowsum(dO * O) of the query
// rows, adds into fp32 accumulators (BluScriptCP development log: 2026-04-20
// ring accumulation of dQ/dK/dV; 2026-05-07 an accumulator is never cleared
// between steps; 2026-03-24 the delta term):
//   P  = exp(sigma q k^T - LSE)        (visible pairs only)
//   dV += P^T dO,  dS = P * (dO v^T - delta),  dQ += sigma dS k,  dK += sigma dS^T q.
//
// Two halves, no atomics (bitwise reproducible):
//   * dkdv: a workgroup owns 128 keys and walks the query tiles that can see
//     them. Scores are formed as S = Q K^T so every lane holds one key; P^T
//     and dS^T then feed the A operand of dV += P^T dO and dK += dS^T Q
//     straight from registers, and dO / Q enter as B operands through the
//     transposing LDS read. At D = 64 each of 4 waves owns 32 keys with both
//     accumulators; at D = 128 two waves share 32 keys, each forming P and dS
//     for half of a tile's rows, one accumulating dV and the other dK over the
//     whole tile (8 waves, the halves exchanged through LDS).
//   * dq: a workgroup owns 128 query rows and walks the visible key tiles, like
//     the forward: S^T = K Q^T and dP^T = V dO^T give one query per lane, and
//     dQ^T += K^T dS^T reads K^T with the transposing LDS read.
// Tiles are staged through LDS with direct global->LDS loads into the
// swizzled, unpadded layout of common.h (double buffered, one barrier per tile).

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace cpattn {
namespace {

constexpr int kNW = 4;
constexpr int kTile = 64;  // rows of the streamed tile (queries for dkdv, keys for dq)

template <int D>
struct BCfg {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int TILEB = kTile * ROWB;
  static constexpr int NI = kTile * CPR / (64 * kNW);  // direct loads per wave per tile
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// Per-lane byte offsets into a swizzled tile.
//   row-operand reads (b128): row 32*blk + lq, logical chunk 2c + h  -> base + 32*blk*ROWB + ro[c]
//   transposing reads (b64):  rows 16t + 4h + (l%16)/4 (+8 for hi), columns 32db + 16((l/16)%2) + 4(l%4)
//                             -> base + 16*t*ROWB + tro[hi][db]
template <int D>
struct Offs {
  int ro[D / 16];
  int tro[2][D / 32];
  __device__ __forceinline__ Offs(int l) {
    using C = BCfg<D>;
    const int h = l >> 5, lq = l & 31;
    const int m = swz_mask<D>(lq);
#pragma unroll
    for (int c = 0; c < C::NC; ++c) ro[c] = lq * C::ROWB + (((2 * c + h) ^ m) * 16);
    const int r0 = 4 * h + ((l & 15) >> 2);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = r0 + 8 * hi;
      const int mm = swz_mask<D>(r);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int cc = 4 * db + 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
        tro[hi][db] = r * C::ROWB + ((cc ^ mm) * 16) + (l & 1) * 8;
      }
    }
  }
};

// ------------------------------------------------------------------ dK / dV
constexpr int kKeysPerWG = 32 * kNW;  // 128

template <int D, int NS>
struct DkdvLds {
  alignas(1024) char sq[NS][BCfg<D>::TILEB];
  alignas(1024) char sdo[NS][BCfg<D>::TILEB];
  alignas(16) float slse[NS][kTile];
  alignas(16) float sdelta[NS][kTile];
};

// Workgroup Lg of the dK/dV grid (Lg = bh * n_kt + key tile); 64-wide heads.
template <int D, int NS>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, int Lg, int n_kt, DkdvLds<D, NS>& sm) {
  static_assert(D == 64, "128-wide heads take dkdv_pair_body");
  using C = BCfg<D>;
  auto& sq = sm.sq;
  auto& sdo = sm.sdo;
  auto& slse = sm.slse;
  auto& sdelta = sm.sdelta;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int bh = Lg / n_kt;  // (b, KV head)
  const int kt = Lg - bh * n_kt;
  const int H_kv = a.H / a.G;
  const int b = bh / H_kv, kvh = bh - b * H_kv;
  const int kc0 = kt * kKeysPerWG;         // first key of the workgroup
  const int kw0 = kc0 + 32 * w;            // first key of the wave
  const int key = kw0 + lq;                // this lane's key
  const bool key_ok = key < a.Tk;

  // Positions increase with the local index, so the query rows that see this lane's key
  // are [qlo, Tq); the wave's last key has the largest qlo.
  const int qlo = a.causal ? a.qm.count_lt(a.km.pos(key_ok ? key : a.Tk - 1)) : 0;
  const int wave_last_key = (kw0 + 31 < a.Tk ? kw0 + 31 : a.Tk - 1);
  const int wave_qlo = a.causal ? a.qm.count_lt(a.km.pos(wave_last_key)) : 0;

  // query rows that can see a key of this workgroup
  const int q_first = a.causal ? a.qm.count_lt(a.km.pos(kc0)) : 0;
  const int t_begin = q_first / kTile;
  const int t_end = (a.Tq + kTile - 1) / kTile;
  const int n = t_end - t_begin;  // tiles per query head
  const int n_items = n * a.G;    // (query head of the group, tile), head-major
  const float sl2 = a.scale * kLog2e;

  int ld_row[C::NI], ld_col[C::NI];
  unsigned qo[C::NI], oo[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int p = (w * C::NI + i) * 64 + l;
    ld_row[i] = p / C::CPR;
    ld_col[i] = ((p % C::CPR) ^ swz_mask<D>(p / C::CPR)) * 8;
    qo[i] = (unsigned)((ld_row[i] * a.q.st + ld_col[i]) * 2);
    oo[i] = (unsigned)((ld_row[i] * a.dout.st + ld_col[i]) * 2);
  }
  // LSE and delta rows of a tile: every wave brings 16 of the 64 (lanes 0..15)
  const unsigned lo_lse = (unsigned)((16 * w + (l & 15)) * a.lse.st * 4);
  const unsigned lo_dl = (unsigned)((16 * w + (l & 15)) * a.delta.st * 4);
  // item it = (query head kvh*G + it/n, tile t_begin + it%n)
  auto issue_tile = [&](int it, int buf) {
    const int hq = kvh * a.G + it / n;
    const int t = t_begin + it % n;
    const __bf16* qp = (const __bf16*)a.q.p + b * a.q.sb + hq * a.q.sh;
    const __bf16* dop = (const __bf16*)a.dout.p + b * a.dout.sb + hq * a.dout.sh;
    const float* lp = (const float*)a.lse.p + b * a.lse.sb + hq * a.lse.sh;
    const float* dp = (const float*)a.delta.p + b * a.delta.sb + hq * a.delta.sh;
    const int q0 = t * kTile;
    const char* qbase = (const char*)(qp + (int64_t)q0 * a.q.st);
    const char* obase = (const char*)(dop + (int64_t)q0 * a.dout.st);
    const bool tail = q0 + kTile > a.Tq;  // rows past the end repeat the last row (masked)
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      unsigned q_off = qo[i], o_off = oo[i];
      if (tail) {
        const int r = min(ld_row[i], a.Tq - 1 - q0);
        q_off = (unsigned)((r * a.q.st + ld_col[i]) * 2);
        o_off = (unsigned)((r * a.dout.st + ld_col[i]) * 2);
      }
      load_lds16(qbase, q_off, sq[buf] + (w * C::NI + i) * 1024);
      load_lds16(obase, o_off, sdo[buf] + (w * C::NI + i) * 1024);
    }
    if (l < 16) {
      unsigned l_off = lo_lse, d_off = lo_dl;
      if (tail) {
        const int r = min(16 * w + l, a.Tq - 1 - q0);
        l_off = (unsigned)(r * a.lse.st * 4);
        d_off = (unsigned)(r * a.delta.st * 4);
      }
      load_lds4(lp + (int64_t)q0 * a.lse.st, l_off, &slse[buf][16 * w]);
      load_lds4(dp + (int64_t)q0 * a.delta.st, d_off, &sdelta[buf][16 * w]);
    }
  };

  const Offs<D> off(l);
  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dk[db] = dv[db] = f32x16{};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_items) issue_tile(j, j);

  // K and V rows of this lane's key (B operands: column = key, 8 consecutive d)
  bf16x8 kf[C::NC], vf[C::NC];
  {
    const __bf16* kk = (const __bf16*)a.k.p + b * a.k.sb + kvh * a.k.sh + (int64_t)key * a.k.st;
    const __bf16* vv = (const __bf16*)a.v.p + b * a.v.sb + kvh * a.v.sh + (int64_t)key * a.v.st;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      u32x4 z = {0u, 0u, 0u, 0u};
      kf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(kk + 16 * c + 8 * h) : z);
      vf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(vv + 16 * c + 8 * h) : z);
    }
  }
  // Complete the register loads before the tile loop, so that the compiler's wait for them
  // does not land inside it, where it would also cover later tiles in flight. They are
  // issued after the first tiles' loads so that both take one memory round trip together.
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    asm volatile("" ::"v"(kf[c]));
    asm volatile("" ::"v"(vf[c]));
  }

  // every query head of the group in turn: dK and dV sum over the group in registers
  for (int it = 0; it < n_items; ++it) {
    const int t = t_begin + it % n;
    const int cur = it % NS;
    wait_tiles<2 * C::NI + 2>(min(NS - 2, n_items - 1 - it));
    __syncthreads();
    if (it + NS - 1 < n_items) issue_tile(it + NS - 1, (it + NS - 1) % NS);
    const char* Q = sq[cur];
    const char* DO = sdo[cur];
    const int q0 = t * kTile;
    const bool full = (q0 + kTile <= a.Tq) && (kw0 + 31 < a.Tk) && (q0 >= wave_qlo);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // operands of S = Q K^T and dP = dO V^T for 32 query rows, read as one batch
      f32x16 s = f32x16{}, dpv = f32x16{};
      bf16x8 qa[C::NC], da[C::NC];
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        qa[c] = *(const bf16x8*)(Q + 32 * qb * C::ROWB + off.ro[c]);
        da[c] = *(const bf16x8*)(DO + 32 * qb * C::ROWB + off.ro[c]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        s = mfma32(qa[c], kf[c], s);
        dpv = mfma32(da[c], vf[c], dpv);
      }
      // rows of s / dpv: query 32qb + 8g + 4h + j, column: this lane's key
      f32x4 L4[4], D4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        L4[g] = *(const f32x4*)(slse[cur] + 32 * qb + 8 * g + 4 * h);
        D4[g] = *(const f32x4*)(sdelta[cur] + 32 * qb + 8 * g + 4 * h);
      }
      // raw LSE: -L log2e; a row without any visible key (LSE = -inf) only occurs in
      // tiles that are not full, where the mask below replaces its weights by 0
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(s[r], sl2, L4[r >> 2][r & 3] * -kLog2e));
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
          p[r] = (key_ok && qrow >= qlo && qrow < a.Tq) ? p[r] : 0.f;
        }
      }
      bf16x8 pa[2], dsa[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pa[r >> 3][r & 7] = (__bf16)p[r];
        dsa[r >> 3][r & 7] = (__bf16)(p[r] * (dpv[r] - D4[r >> 2][r & 3]));
      }
      // dV += P^T dO, dK += dS^T Q ; B operand rows = queries 32qb + 16tt + 4h + {0..3}, +8
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int rb = (32 * qb + 16 * tt) * C::ROWB;
        bf16x8 ob[C::NDB], qv[C::NDB];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          ob[db] = cat8(lds_read_tr4((const __bf16*)(DO + rb + off.tro[0][db])),
                        lds_read_tr4((const __bf16*)(DO + rb + off.tro[1][db])));
          qv[db] = cat8(lds_read_tr4((const __bf16*)(Q + rb + off.tro[0][db])),
                        lds_read_tr4((const __bf16*)(Q + rb + off.tro[1][db])));
        }
        __builtin_amdgcn_sched_barrier(0);
        // both accumulators live in AGPRs, away from the working set
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          mfma32_agpr(dv[db], pa[tt], ob[db]);
          mfma32_agpr(dk[db], dsa[tt], qv[db]);
        }
      }
    }
  }

  // no query of this block sees these keys: nothing to add (an overwrite still writes zeros)
  if (n_items <= 0 && a.acc_kv) return;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    mfma_agpr_drain(dk[db]);
    mfma_agpr_drain(dv[db]);
  }
  // accumulate: lane holds column d = 32db + lq, rows key kw0 + 8g + 4h + j. The wave's 32
  // rows go through a buffer resource bounded at its last key, so rows past Tk read as zero
  // and drop their stores with no branch. Each accumulator's old values are all read before
  // its first store: the compiler cannot tell dK from dV apart, so read-add-store pairs in
  // turn would each wait for a full memory round trip.
  const int rows = min(32, a.Tk - kw0);
  auto add_rows = [&](float* base, int64_t st, const f32x16(&acc)[C::NDB], float mul) __attribute__((always_inline)) {
    const int bytes = rows > 0 ? ((rows - 1) * (int)st + D) * 4 : 0;  // rows never overlap: st >= D
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(base + (int64_t)kw0 * st, (short)0, bytes, kBufferFlags);
    // an overwrite reads through an empty range: every read returns 0 and touches no memory
    const auto rl = __builtin_amdgcn_make_buffer_rsrc(base + (int64_t)kw0 * st, (short)0, a.acc_kv ? bytes : 0,
                                                      kBufferFlags);
    auto offset = [&](int db, int r) { return (int)(((8 * (r >> 2) + 4 * h + (r & 3)) * st + lq) * 4) + 128 * db; };
    unsigned old[C::NDB][16];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) old[db][r] = __builtin_amdgcn_raw_buffer_load_b32(rl, offset(db, r), 0, 0);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(unsigned, __builtin_bit_cast(float, old[db][r]) + mul * acc[db][r]), rs, offset(db, r),
            0, 0);
  };
  add_rows(a.dk + b * a.dk_sb + kvh * a.dk_sh, a.dk_st, dk, a.scale);
  add_rows(a.dv + b * a.dv_sb + kvh * a.dv_sh, a.dv_st, dv, 1.f);
}

// ------------------------------------------------------------------ dK / dV, paired waves
// Eight waves, 128 keys per workgroup (one workgroup per CU); waves w and w + 4 own the
// same 32 keys and hold both their K and V rows. Of each 64-row query tile, wave w takes
// rows 0-31 and wave w + 4 rows 32-63: each forms S and dP of its rows, then P and
// dS = P (dP - delta) in bf16. Wave w keeps P and hands dS to its partner through LDS,
// wave w + 4 keeps dS and hands P over; after a barrier wave w accumulates
// dV += P^T dO and wave w + 4 dK += dS^T Q over all 64 rows. Each pair forms each of the
// four products once (8·D flops per pair of the block), both waves do the same work, and
// each holds one accumulator, so two waves fit per SIMD. Two barriers per query tile: the
// tile has landed; the exchanged halves are in LDS. Only waves 0-3 issue the tile loads.
// The arithmetic of every product and of dS is that of dkdv_body, so the results are the
// same bits.

template <int D, int NS, int NP>
struct DkdvPairLds {
  alignas(1024) char sq[NS][BCfg<D>::TILEB];
  alignas(1024) char sdo[NS][BCfg<D>::TILEB];
  alignas(16) float slse[NS][kTile];
  alignas(16) float sdelta[NS][kTile];
  alignas(16) bf16x8 sx[NP][2][2][64];  // [pair][from wave w / w + NP][8-value half][lane]
};

// Chunk (16 bytes) of a staged dS block that holds half i of the 16 values of lane group h
// and key k: chunk 64 i + 32 h + (k ^ 8 (i ^ h)). The XOR spreads the chunks that one
// transposing read of the dQ kernel takes over all LDS banks.
__device__ __forceinline__ int ds_chunk(int i, int h, int k) { return 64 * i + 32 * h + (k ^ (8 * (i ^ h))); }

template <int D, int NS, int NP, bool STAGE>
__device__ __forceinline__ void dkdv_pair_body(const BwdArgs& a, int Lg, int n_kt, DkdvPairLds<D, NS, NP>& sm) {
  using C = BCfg<D>;
  constexpr int NIP = kTile * C::CPR / (64 * NP);  // direct loads per loader wave per tile (Q, dO each)
  constexpr int RL = kTile / NP;                   // rows of LSE and delta a loader wave brings
  static_assert(NIP >= 1 && (NP == 2 || NP == 4), "tile layout");
  auto& sq = sm.sq;
  auto& sdo = sm.sdo;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int hb = w >= NP ? 1 : 0;  // 32-row block of each tile this wave forms; 0: keeps dV
  const int kw = w & (NP - 1);
  const int bh = Lg / n_kt;  // (b, KV head)
  const int kt = Lg - bh * n_kt;
  const int H_kv = a.H / a.G;
  const int b = bh / H_kv, kvh = bh - b * H_kv;
  const int kc0 = kt * 32 * NP;  // first key of the workgroup
  const int kw0 = kc0 + 32 * kw;    // first key of the pair
  const int key = kw0 + lq;         // this lane's key
  const bool key_ok = key < a.Tk;

  const int qlo = a.causal ? a.qm.count_lt(a.km.pos(key_ok ? key : a.Tk - 1)) : 0;
  const int wave_last_key = (kw0 + 31 < a.Tk ? kw0 + 31 : a.Tk - 1);
  const int wave_qlo = a.causal ? a.qm.count_lt(a.km.pos(wave_last_key)) : 0;
  const int q_first = a.causal ? a.qm.count_lt(a.km.pos(kc0)) : 0;
  const int t_begin = q_first / kTile;
  const int t_end = (a.Tq + kTile - 1) / kTile;
  const int n = t_end - t_begin;
  const int n_items = n * a.G;  // (query head of the group, tile), head-major
  const float sl2 = a.scale * kLog2e;

  int ld_row[NIP], ld_col[NIP];
  unsigned qo[NIP], oo[NIP];
#pragma unroll
  for (int i = 0; i < NIP; ++i) {
    const int p = (kw * NIP + i) * 64 + l;
    ld_row[i] = p / C::CPR;
    ld_col[i] = ((p % C::CPR) ^ swz_mask<D>(p / C::CPR)) * 8;
    qo[i] = (unsigned)((ld_row[i] * a.q.st + ld_col[i]) * 2);
    oo[i] = (unsigned)((ld_row[i] * a.dout.st + ld_col[i]) * 2);
  }
  // Only the dV waves (0 .. NP-1) load the tiles: the dK waves go straight from the barrier
  // to their products while the loads queue (a loader brings 64 / NP rows of Q, dO, LSE and
  // delta)
  const int sr = RL * kw + (l % RL);
  auto issue_tile = [&](int it, int buf) {
    if (hb != 0) return;
    const int hq = kvh * a.G + it / n;
    const int t = t_begin + it % n;
    const __bf16* qp = (const __bf16*)a.q.p + b * a.q.sb + hq * a.q.sh;
    const __bf16* dop = (const __bf16*)a.dout.p + b * a.dout.sb + hq * a.dout.sh;
    const float* lp = (const float*)a.lse.p + b * a.lse.sb + hq * a.lse.sh;
    const float* dp = (const float*)a.delta.p + b * a.delta.sb + hq * a.delta.sh;
    const int q0 = t * kTile;
    const char* qbase = (const char*)(qp + (int64_t)q0 * a.q.st);
    const char* obase = (const char*)(dop + (int64_t)q0 * a.dout.st);
    const bool tail = q0 + kTile > a.Tq;  // rows past the end repeat the last row (masked)
#pragma unroll
    for (int i = 0; i < NIP; ++i) {
      unsigned q_off = qo[i], o_off = oo[i];
      if (tail) {
        const int r = min(ld_row[i], a.Tq - 1 - q0);
        q_off = (unsigned)((r * a.q.st + ld_col[i]) * 2);
        o_off = (unsigned)((r * a.dout.st + ld_col[i]) * 2);
      }
      load_lds16(qbase, q_off, sq[buf] + (kw * NIP + i) * 1024);
      load_lds16(obase, o_off, sdo[buf] + (kw * NIP + i) * 1024);
    }
    if (l < RL) {
      const int r = tail ? min(sr, a.Tq - 1 - q0) : sr;
      load_lds4(lp + (int64_t)q0 * a.lse.st, (unsigned)(r * a.lse.st * 4), &sm.slse[buf][RL * kw]);
      load_lds4(dp + (int64_t)q0 * a.delta.st, (unsigned)(r * a.delta.st * 4), &sm.sdelta[buf][RL * kw]);
    }
  };

  const Offs<D> off(l);
  f32x16 acc[C::NDB];  // dV (waves 0-3) or dK (waves 4-7)
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_items) issue_tile(j, j);

  // K and V rows of this lane's key (B operands: column = key, 8 consecutive d)
  bf16x8 kf[C::NC], vf[C::NC];
  {
    const __bf16* kk = (const __bf16*)a.k.p + b * a.k.sb + kvh * a.k.sh + (int64_t)key * a.k.st;
    const __bf16* vv = (const __bf16*)a.v.p + b * a.v.sb + kvh * a.v.sh + (int64_t)key * a.v.st;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      u32x4 z = {0u, 0u, 0u, 0u};
      kf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(kk + 16 * c + 8 * h) : z);
      vf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(vv + 16 * c + 8 * h) : z);
    }
  }
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(kf[c]), "v"(vf[c]));

  for (int it = 0; it < n_items; ++it) {
    const int t = t_begin + it % n;
    const int cur = it % NS;
    wait_tiles<2 * NIP + 2>(min(NS - 2, n_items - 1 - it));
    __syncthreads();  // tile it visible; every wave is done with tile it-1 and the exchange
    if (it + NS - 1 < n_items) issue_tile(it + NS - 1, (it + NS - 1) % NS);
    const char* Q = sq[cur];
    const char* DO = sdo[cur];
    const int q0 = t * kTile;
    const bool full = (q0 + kTile <= a.Tq) && (kw0 + 31 < a.Tk) && (q0 >= wave_qlo);

    // ---- S = Q K^T and dP = dO V^T of this wave's 32 rows (operands streamed from LDS)
    f32x16 s = f32x16{}, dpv = f32x16{};
    {
      constexpr int LA = 4;
      auto rd = [&](int j) {
        return *(const bf16x8*)(((j & 1) ? DO : Q) + 32 * hb * C::ROWB + off.ro[j >> 1]);
      };
      bf16x8 opa[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) opa[j] = rd(j);
#pragma unroll
      for (int j = 0; j < 2 * C::NC; ++j) {
        if (j & 1) dpv = mfma32(opa[j % LA], vf[j >> 1], dpv);
        else s = mfma32(opa[j % LA], kf[j >> 1], s);
        if (j + LA < 2 * C::NC) opa[j % LA] = rd(j + LA);
      }
    }
    // rows of s / dpv: query 32hb + 8g + 4h + j, column: this lane's key
    f32x4 L4[4], D4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      L4[g] = *(const f32x4*)(sm.slse[cur] + 32 * hb + 8 * g + 4 * h);
      D4[g] = *(const f32x4*)(sm.sdelta[cur] + 32 * hb + 8 * g + 4 * h);
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(s[r], sl2, L4[r >> 2][r & 3] * -kLog2e));
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + 32 * hb + 8 * (r >> 2) + 4 * h + (r & 3);
        p[r] = (key_ok && qrow >= qlo && qrow < a.Tq) ? p[r] : 0.f;
      }
    }
    bf16x8 pa[2], dsa[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pa[r >> 3][r & 7] = (__bf16)p[r];
      dsa[r >> 3][r & 7] = (__bf16)(p[r] * (dpv[r] - D4[r >> 2][r & 3]));
    }
    if constexpr (STAGE) {
      // this wave's 32 x 32 block of dS for the dQ kernel (value e of dsa[i]: row
      // 16i + 8(e/4) + 4h + e%4 of the block, key lq), written past the caches (it is read
      // once, by another kernel); blocks past the last row or key are not part of the
      // staging area and are never read. The stores share the vector memory counter with the
      // tile loads: since loads complete in issue order, a wait whose count has dropped by a
      // tile's loads plus these stores still implies that the tile's loads completed.
      const int qr0 = q0 + 32 * hb;
      if (qr0 < a.Tq && kw0 < a.Tk) {
        const int hq = kvh * a.G + it / n;
        char* blk = (char*)a.ds + (((int64_t)(b * a.H + hq) * a.nqb + (qr0 >> 5)) * a.nkb + (kw0 >> 5)) * 2048;
#pragma unroll
        for (int i = 0; i < 2; ++i) __builtin_nontemporal_store(dsa[i], (bf16x8*)(blk + 16 * ds_chunk(i, h, lq)));
      }
    }
    // keep what this wave accumulates (P for dV, dS for dK); hand the other to the partner
    bf16x8 mine[2][2];  // [32-row block][8-value half]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16x8 keep = hb == 0 ? pa[i] : dsa[i];
      const bf16x8 give = hb == 0 ? dsa[i] : pa[i];
      mine[hb][i] = keep;
      sm.sx[kw][hb][i][l] = give;
    }
    __syncthreads();  // the partner's half of the tile in LDS
#pragma unroll
    for (int i = 0; i < 2; ++i) mine[1 - hb][i] = sm.sx[kw][1 - hb][i][l];

    // ---- dV += P^T dO, or dK += dS^T Q ; B operand rows = queries 32qb + 16tt + 4h + {0..3}, +8
    const char* Bsrc = hb == 0 ? DO : Q;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int rb = (32 * qb + 16 * tt) * C::ROWB;
        bf16x8 ob[C::NDB];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          ob[db] = cat8(lds_read_tr4((const __bf16*)(Bsrc + rb + off.tro[0][db])),
                        lds_read_tr4((const __bf16*)(Bsrc + rb + off.tro[1][db])));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) acc[db] = mfma32(mine[qb][tt], ob[db], acc[db]);
      }
    }
  }

  // no query of this block sees these keys: nothing to add (an overwrite still writes zeros)
  if (n_items <= 0 && a.acc_kv) return;
  const bool dv_wave = hb == 0;
  const int rows = min(32, a.Tk - kw0);
  float* base = dv_wave ? a.dv + b * a.dv_sb + kvh * a.dv_sh : a.dk + b * a.dk_sb + kvh * a.dk_sh;
  const int64_t st = dv_wave ? a.dv_st : a.dk_st;
  const float mul = dv_wave ? 1.f : a.scale;
  const int bytes = rows > 0 ? ((rows - 1) * (int)st + D) * 4 : 0;  // rows never overlap: st >= D
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(base + (int64_t)kw0 * st, (short)0, bytes, kBufferFlags);
  const auto rl = __builtin_amdgcn_make_buffer_rsrc(base + (int64_t)kw0 * st, (short)0, a.acc_kv ? bytes : 0,
                                                    kBufferFlags);
  auto offset = [&](int db, int r) { return (int)(((8 * (r >> 2) + 4 * h + (r & 3)) * st + lq) * 4) + 128 * db; };
  unsigned old[C::NDB][16];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) old[db][r] = __builtin_amdgcn_raw_buffer_load_b32(rl, offset(db, r), 0, 0);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(
          __builtin_bit_cast(unsigned, __builtin_bit_cast(float, old[db][r]) + mul * acc[db][r]), rs, offset(db, r), 0,
          0);
}

// ------------------------------------------------------------------ dQ
constexpr int kQPerWG = 32 * kNW;  // 128 query rows per workgroup
constexpr int kKB = 32;            // keys per dQ tile: one 32-key MFMA block

template <int D, int NS, int KS>
struct DqLds {
  alignas(1024) char sk[KS][NS][kKB * BCfg<D>::ROWB];
  alignas(1024) char sv[KS][NS][kKB * BCfg<D>::ROWB];
};

// Workgroup Lg of the dQ grid (Lg = bh * n_qt + heavy-first query tile).
// Software pipeline over the 32-key tiles u of the block (per wave):
//   phase A: P_u, dS_u (VALU)  with  S_u+1^T = K Q^T (and at D = 64 dP_u+1^T = V dO^T) (MFMA)
//   phase B: dQ^T += K_u^T dS_u^T (MFMA), K^T through the transposing LDS read
//            (at D = 128 followed by dP_u+1^T, which keeps phase A within the registers of
//            two waves per SIMD)
// so tiles u and u+1 are read in iteration u, and the LDS ring holds NS >= 3 tiles.
// KS = 2 splits the key tiles of a workgroup between two pairs of waves that own the
// same 64 rows (even tiles to waves 0-1, odd tiles to waves 2-3, each pair with its own
// rings); the odd pair's dQ partial is added to the even pair's through LDS at the end.
template <int D, int NS, int KS>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int Lg, int n_qt, DqLds<D, NS, KS>& sm) {
  using C = BCfg<D>;
  static_assert(NS >= 3 && NS <= 5, "pipeline depth");
  static_assert(KS == 1 || (KS == 2 && D == 64), "key split: 64-wide heads only");
  constexpr int NR = kNW / KS;                        // waves per key share
  constexpr int ROWS = 32 * NR;                       // query rows per workgroup
  constexpr int NIQ = kKB * C::CPR / (64 * NR);       // direct loads per wave per tile (K or V)
  constexpr int kSlotRows = 64 * NR / C::CPR;         // rows between a lane's consecutive slots
  static_assert(NIQ >= 1 && kSlotRows % 16 == 0, "tile layout");

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int rb = w % NR;  // row block of this wave
  const int kh = w / NR;  // key share: tiles kh, kh + KS, ...
  const int bh = Lg / n_qt;
  const int qt = n_qt - 1 - (Lg - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = qt * ROWS;
  const int row = q0 + 32 * rb + lq;
  const bool row_ok = row < a.Tq;

  // ---- key range: the keys row r sees are the prefix [0, lim) of the block
  const int qpos = a.qm.pos(row_ok ? row : a.Tq - 1);
  const int last_row = (q0 + ROWS < a.Tq ? q0 + ROWS : a.Tq) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kKB - 1) / kKB;
  if (n_kt == 0) {  // no key of this block is visible to these rows: nothing to add
    if (!a.acc_q && kh == 0 && row_ok) {  // an overwrite writes zeros
      float* o = a.dq + b * a.dq_sb + hh * a.dq_sh + (int64_t)row * a.dq_st;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(f32x4*)(o + 32 * db + 8 * g + 4 * h) = f32x4{};
    }
    return;
  }
  const int n_jmax = (n_kt + KS - 1) / KS;                    // tiles of the larger share
  const int n_j = n_kt > kh ? (n_kt - kh + KS - 1) / KS : 0;  // tiles of this wave's share
  auto tile = [&](int j) { return KS * j + kh; };
  const int wave_first = q0 + 32 * rb < a.Tq ? q0 + 32 * rb : a.Tq - 1;
  const int lim = a.causal ? min(a.Tk, a.km.count_le(qpos)) : a.Tk;
  const int wave_lim = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(wave_first))) : a.Tk;
  const float sl2 = a.scale * kLog2e;

  const int kvh = hh / a.G;  // the KV head of this query head's group
  const __bf16* kp = (const __bf16*)a.k.p + b * a.k.sb + kvh * a.k.sh;
  const __bf16* vp = (const __bf16*)a.v.p + b * a.v.sb + kvh * a.v.sh;


  // ---- direct global -> LDS loads: wave rb of a share fills 1 KB slots rb + NR*i of that
  // share's tiles; the rows of a lane's slots differ by a multiple of the swizzle period
  // (one lane offset)
  const int ld_r0 = (64 * rb + l) / C::CPR;
  const int ld_col = ((l % C::CPR) ^ swz_mask<D>(ld_r0)) * 8;
  const unsigned ko = (unsigned)((ld_r0 * a.k.st + ld_col) * 2);
  const unsigned vo = (unsigned)((ld_r0 * a.v.st + ld_col) * 2);
  auto issue = [&](const __bf16* base, int64_t st, unsigned off, int kt, char* dst) {
    const char* tb = (const char*)(base + (int64_t)kt * kKB * st);
    if (kt * kKB + kKB <= a.Tk) {
#pragma unroll
      for (int i = 0; i < NIQ; ++i) load_lds16(tb + (int64_t)kSlotRows * i * st * 2, off, dst + (rb + NR * i) * 1024);
    } else {  // rows past the block repeat the last key (masked)
#pragma unroll
      for (int i = 0; i < NIQ; ++i) {
        const int r = min(ld_r0 + kSlotRows * i, a.Tk - 1 - kt * kKB);
        load_lds16(tb, (unsigned)((r * st + ld_col) * 2), dst + (rb + NR * i) * 1024);
      }
    }
  };
  // tile j of this wave's share
  auto issue_tile = [&](int j) {
    issue(kp, a.k.st, ko, tile(j), sm.sk[kh][j % NS]);
    issue(vp, a.v.st, vo, tile(j), sm.sv[kh][j % NS]);
  };

  const Offs<D> off(l);
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

  auto needs_mask = [&](int kt) { return kt * kKB + kKB > wave_lim; };
  // element r of a tile's scores is key kt*kKB + 8(r/4) + 4h + r%4
  auto apply_mask = [&](f32x16& sv, int kt) {
    const int rel = lim - kt * kKB - 4 * h;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = 8 * (r >> 2) + (r & 3) < rel ? sv[r] : -INFINITY;
  };

  // ---- prologue: the share's tiles 0 .. NS-2 in flight, then S and dP of its tile 0. Every
  // wave passes one barrier here and one per tile of the larger share (a share with fewer
  // tiles pads).
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_j) issue_tile(j);
  // ---- Q and dO rows of this lane's query (B operands), LSE and delta of the row
  bf16x8 qf[C::NC], df[C::NC];
  {
    const __bf16* qq = (const __bf16*)a.q.p + b * a.q.sb + hh * a.q.sh + (int64_t)row * a.q.st;
    const __bf16* dd = (const __bf16*)a.dout.p + b * a.dout.sb + hh * a.dout.sh + (int64_t)row * a.dout.st;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8, row_ok ? ldg16(qq + 16 * c + 8 * h) : z);
      df[c] = __builtin_bit_cast(bf16x8, row_ok ? ldg16(dd + 16 * c + 8 * h) : z);
    }
  }
  float lse2 = INFINITY, dl = 0.f;
  if (row_ok) {
    const float L = ((const float*)a.lse.p)[b * a.lse.sb + hh * a.lse.sh + (int64_t)row * a.lse.st];
    lse2 = L == -INFINITY ? INFINITY : L * kLog2e;
    dl = ((const float*)a.delta.p)[b * a.delta.sb + hh * a.delta.sh + (int64_t)row * a.delta.st];
  }
  // complete the register loads before the tile loop; issued after the first tiles' loads,
  // both take one memory round trip together (as in the dK/dV half)
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(qf[c]), "v"(df[c]));
  asm volatile("" ::"v"(lse2), "v"(dl));
  wait_tiles<2 * NIQ>(min(NS - 2, n_j - 1));
  __syncthreads();
  f32x16 sA = f32x16{}, dA = f32x16{}, sB, dB;
  if (n_j > 0) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      sA = mfma32(*(const bf16x8*)(sm.sk[kh][0] + off.ro[c]), qf[c], sA);
      dA = mfma32(*(const bf16x8*)(sm.sv[kh][0] + off.ro[c]), df[c], dA);
    }
    if (needs_mask(tile(0))) apply_mask(sA, tile(0));
  }

  // Tile u of this wave's share: `s`, `dp` hold its S^T (masked) and dP^T; with NEXT, those
  // of tile u+1 are formed into `sn`, `dpn`. Scheduling fences pin the MFMA / vector
  // interleave.
  auto step = [&](int u, f32x16& s, f32x16& dp, f32x16& sn, f32x16& dpn, auto next_tag)
                  __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    if constexpr (NEXT) wait_tiles<2 * NIQ>(min(NS - 3, n_j - 2 - u));  // tile u+1 has landed
    __syncthreads();  // tile u+1 visible; every wave is done with tile u-1
    if (u + NS - 1 < n_j) issue_tile(u + NS - 1);

    // ---- phase A: dS_u = P_u (dP_u - delta) in bf16, with S_u+1 (and dP_u+1) on the matrix cores
    constexpr bool DP_IN_A = D == 64;
    constexpr int NM = (DP_IN_A ? 2 : 1) * C::NC;  // MFMAs of phase A (S and dP chains interleaved)
    constexpr int EA = 16 / NM > 0 ? 16 / NM : 1;
    constexpr int LA = D == 64 ? 4 : 2;  // operand reads in flight ahead of their MFMA
    const char* kn = sm.sk[kh][(u + 1) % NS];
    const char* vn = sm.sv[kh][(u + 1) % NS];
    // operand j of phase A: K row chunk j (S only) or K / V row chunk j/2 (S and dP)
    auto rd = [&](int j) {
      if constexpr (DP_IN_A) return *(const bf16x8*)(((j & 1) ? vn : kn) + off.ro[j >> 1]);
      else return *(const bf16x8*)(kn + off.ro[j]);
    };
    bf16x8 opa[LA];
    if constexpr (NEXT) {
      sn = f32x16{};
      dpn = f32x16{};
#pragma unroll
      for (int j = 0; j < LA; ++j) opa[j] = rd(j);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if constexpr (NEXT) {
        if constexpr (DP_IN_A) {
          if (j & 1) dpn = mfma32(opa[j % LA], df[j >> 1], dpn);
          else sn = mfma32(opa[j % LA], qf[j >> 1], sn);
        } else {
          sn = mfma32(opa[j % LA], qf[j], sn);
        }
        if (j + LA < NM) opa[j % LA] = rd(j + LA);
      }
#pragma unroll
      for (int e = 0; e < EA; ++e) {
        const int r = EA * j + e;
        if (r < 16) {
          const float p = fast_exp2(fmaf(s[r], sl2, -lse2));
          dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase B: dQ^T += K^T dS^T ; K^T operand rows = d, 8 keys 16t + 4h + {0..3}, +8
    const char* K = sm.sk[kh][u % NS];
    bf16x8 kt8[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      kt8[db] = cat8(lds_read_tr4((const __bf16*)(K + off.tro[0][db])), lds_read_tr4((const __bf16*)(K + off.tro[1][db])));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        acc[db] = mfma32(kt8[db], dsb[t], acc[db]);
        if (t == 0)
          kt8[db] = cat8(lds_read_tr4((const __bf16*)(K + 16 * C::ROWB + off.tro[0][db])),
                         lds_read_tr4((const __bf16*)(K + 16 * C::ROWB + off.tro[1][db])));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (NEXT && !DP_IN_A) {
      bf16x8 vb[2];
      vb[0] = *(const bf16x8*)(vn + off.ro[0]);
      vb[1] = *(const bf16x8*)(vn + off.ro[1]);
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        dpn = mfma32(vb[c & 1], df[c], dpn);
        if (c + 2 < C::NC) vb[c & 1] = *(const bf16x8*)(vn + off.ro[c + 2]);
      }
    }
    if constexpr (NEXT)
      if (needs_mask(tile(u + 1))) apply_mask(sn, tile(u + 1));
  };

  using T_ = std::integral_constant<bool, true>;
  // Two tiles per trip so that the score registers alternate instead of being copied. The
  // last tile also forms the scores of a tile past the end from a stale (in-bounds) LDS
  // stage; they are never used, and one code path keeps the loop within the registers.
  int u = 0;
  for (; u + 1 < n_j; u += 2) {
    step(u, sA, dA, sB, dB, T_{});
    step(u + 1, sB, dB, sA, dA, T_{});
  }
  if (u < n_j) step(u, sA, dA, sB, dB, T_{});
  for (int e = n_j; e < n_jmax; ++e) __syncthreads();  // a share with fewer tiles pads

  if constexpr (KS == 2) {
    // ---- add the odd share's dQ^T partial to the even share's (same rows, same layout)
    constexpr int NV = C::NDB * 16;
    static_assert(NR * NV * 64 * 4 <= KS * NS * kKB * C::ROWB, "staging fits the K rings");
    float* cb = (float*)&sm.sk[0][0][0] + rb * NV * 64;
    __syncthreads();  // every wave is done with its rings
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) cb[(16 * db + r) * 64 + l] = acc[db][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] += cb[(16 * db + r) * 64 + l];
  }

  {
    // The wave's 32 rows go through a buffer resource bounded at its last row (rows past
    // Tq read as zero and drop their stores); all old values are read before the stores
    // (one memory round trip), through an empty range when overwriting.
    const int w_row0 = q0 + 32 * rb;
    const int wrows = min(32, a.Tq - w_row0);
    float* base = a.dq + b * a.dq_sb + hh * a.dq_sh + (int64_t)w_row0 * a.dq_st;
    const int bytes = wrows > 0 ? ((wrows - 1) * (int)a.dq_st + D) * 4 : 0;  // rows never overlap: st >= D
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kBufferFlags);
    const auto rl = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, a.acc_q ? bytes : 0, kBufferFlags);
    auto offset = [&](int db, int g) { return (int)((lq * a.dq_st + 32 * db + 8 * g + 4 * h) * 4); };
    u32x4 old[C::NDB][4];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) old[db][g] = __builtin_amdgcn_raw_buffer_load_b128(rl, offset(db, g), 0, 0);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = __builtin_bit_cast(f32x4, old[db][g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] += a.scale * acc[db][4 * g + j];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), rs, offset(db, g), 0, 0);
      }
  }
}

// ------------------------------------------------------------------ dQ from staged dS
template <int D, int NS, int NW>
struct DqStagedLds {
  alignas(1024) char sk[NS][kKB * BCfg<D>::ROWB];
  alignas(1024) char sds[NS][NW][2048];  // each wave's dS block of the tile
};

// Workgroup Lg of the dQ grid (Lg = bh * n_qt + heavy-first query tile), 128-wide heads,
// with the dS blocks the dK/dV kernel staged: per 32-key tile u, wave w takes its block of
// 32 rows x 32 keys (2 KB, one contiguous stream per wave) and the shared K tile into LDS,
// then dQ^T += K^T dS^T with both operands through the transposing LDS read. The operands
// and the order of the products are those of dq_body's phase B.
template <int D, int NS, int NW>
__device__ __forceinline__ void dq_staged_body(const BwdArgs& a, int Lg, int n_qt, DqStagedLds<D, NS, NW>& sm) {
  using C = BCfg<D>;
  static_assert(D == 128, "staged dS: 128-wide heads");
  static_assert(NS >= 2, "pipeline depth");
  constexpr int ROWS = 32 * NW;                  // query rows per workgroup
  constexpr int NIQ = kKB * C::CPR / (64 * NW);  // K loads per wave per tile
  constexpr int kSlotRows = 64 * NW / C::CPR;    // rows between a lane's consecutive K slots
  static_assert(NIQ >= 1 && kSlotRows % 16 == 0, "tile layout");

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int bh = Lg / n_qt;
  const int qt = n_qt - 1 - (Lg - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = qt * ROWS;
  const int w_row0 = q0 + 32 * w;

  const int last_row = (q0 + ROWS < a.Tq ? q0 + ROWS : a.Tq) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kKB - 1) / kKB;
  if (n_kt == 0) {  // no key of this block is visible to these rows: nothing to add
    const int row = w_row0 + lq;
    if (!a.acc_q && row < a.Tq) {  // an overwrite writes zeros
      float* o = a.dq + b * a.dq_sb + hh * a.dq_sh + (int64_t)row * a.dq_st;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(f32x4*)(o + 32 * db + 8 * g + 4 * h) = f32x4{};
    }
    return;
  }
  // tiles of this wave: the keys its last row sees (the dK/dV kernel wrote every such block);
  // blocks of later tiles are re-reads of its last block and are not used
  int n_kw = 0;
  if (w_row0 < a.Tq) {
    const int w_last = min(w_row0 + 31, a.Tq - 1);
    const int w_vis = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(w_last))) : a.Tk;
    n_kw = (w_vis + kKB - 1) / kKB;
  }
  const int qb = min(w_row0 >> 5, a.nqb - 1);  // a wave past the last row re-reads an in-range block
  const char* ds_row = (const char*)a.ds + ((int64_t)(b * a.H + hh) * a.nqb + qb) * a.nkb * 2048;

  const int kvh = hh / a.G;
  const __bf16* kp = (const __bf16*)a.k.p + b * a.k.sb + kvh * a.k.sh;
  const int ld_r0 = (64 * w + l) / C::CPR;
  const int ld_col = ((l % C::CPR) ^ swz_mask<D>(ld_r0)) * 8;
  const unsigned ko = (unsigned)((ld_r0 * a.k.st + ld_col) * 2);
  auto issue_tile = [&](int u) {
    const char* tb = (const char*)(kp + (int64_t)u * kKB * a.k.st);
    char* dst = sm.sk[u % NS];
    if (u * kKB + kKB <= a.Tk) {
#pragma unroll
      for (int i = 0; i < NIQ; ++i)
        load_lds16(tb + (int64_t)kSlotRows * i * a.k.st * 2, ko, dst + (w + NW * i) * 1024);
    } else {  // rows past the block repeat the last key (their dS is zero)
#pragma unroll
      for (int i = 0; i < NIQ; ++i) {
        const int r = min(ld_r0 + kSlotRows * i, a.Tk - 1 - u * kKB);
        load_lds16(tb, (unsigned)((r * a.k.st + ld_col) * 2), dst + (w + NW * i) * 1024);
      }
    }
    const char* src = ds_row + (int64_t)min(u, n_kw > 0 ? n_kw - 1 : 0) * 2048;
    load_lds16_nt(src, (unsigned)(16 * l), sm.sds[u % NS][w]);
    load_lds16_nt(src + 1024, (unsigned)(16 * l), sm.sds[u % NS][w] + 1024);
  };

  const Offs<D> off(l);
  // transposing reads of the dS block: lane l takes row (query) 16((l/16)%2) + l%16 of the
  // wave's 32, keys 16t + 8hi + 4h + {0..3} (the key order of the K^T operand). Source lane
  // s = l%16 addresses key 16t + 8hi + 4h + s/4, rows 16((l/16)%2) + 4(s%4) + {0..3}.
  int dso[2][2];
  {
    const int s = l & 15, e = s >> 2, m = s & 3, G = (l >> 4) & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) dso[t][hi] = 16 * ds_chunk(G, m & 1, 16 * t + 8 * hi + 4 * h + e) + 8 * (m >> 1);
  }
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_kt) issue_tile(j);
  for (int u = 0; u < n_kt; ++u) {
    wait_tiles<NIQ + 2>(min(NS - 2, n_kt - 1 - u));
    __syncthreads();  // tile u visible; every wave is done with tile u-1
    if (u + NS - 1 < n_kt) issue_tile(u + NS - 1);
    if (u < n_kw) {
      const char* K = sm.sk[u % NS];
      const char* S = sm.sds[u % NS][w];
      bf16x8 dsb[2], kt8[C::NDB];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dsb[t] = cat8(lds_read_tr4((const __bf16*)(S + dso[t][0])), lds_read_tr4((const __bf16*)(S + dso[t][1])));
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        kt8[db] = cat8(lds_read_tr4((const __bf16*)(K + off.tro[0][db])), lds_read_tr4((const __bf16*)(K + off.tro[1][db])));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          acc[db] = mfma32(kt8[db], dsb[t], acc[db]);
          if (t == 0)
            kt8[db] = cat8(lds_read_tr4((const __bf16*)(K + 16 * C::ROWB + off.tro[0][db])),
                           lds_read_tr4((const __bf16*)(K + 16 * C::ROWB + off.tro[1][db])));
        }
      }
    }
  }

  {
    const int wrows = min(32, a.Tq - w_row0);
    float* base = a.dq + b * a.dq_sb + hh * a.dq_sh + (int64_t)w_row0 * a.dq_st;
    const int bytes = wrows > 0 ? ((wrows - 1) * (int)a.dq_st + D) * 4 : 0;  // rows never overlap: st >= D
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kBufferFlags);
    const auto rl = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, a.acc_q ? bytes : 0, kBufferFlags);
    auto offset = [&](int db, int g) { return (int)((lq * a.dq_st + 32 * db + 8 * g + 4 * h) * 4); };
    u32x4 old[C::NDB][4];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) old[db][g] = __builtin_amdgcn_raw_buffer_load_b128(rl, offset(db, g), 0, 0);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = __builtin_bit_cast(f32x4, old[db][g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] += a.scale * acc[db][4 * g + j];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), rs, offset(db, g), 0, 0);
      }
  }
}

template <int D, int NS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void dq_staged_kernel(BwdArgs a, int n_qt, int vary) {
  __shared__ DqStagedLds<D, NS, NW> sm;
  int head, rank;
  xcd_tile(blockIdx.x, gridDim.x, n_qt, vary != 0, head, rank);
  dq_staged_body<D, NS, NW>(a, head * n_qt + rank, n_qt, sm);
}

template <int D, int NS>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a, int n_kt) {
  __shared__ DkdvLds<D, NS> sm;
  dkdv_body<D, NS>(a, xcd_remap(blockIdx.x, gridDim.x), n_kt, sm);
}

template <int D, int NS, int NP, bool STAGE>
__global__ __launch_bounds__(128 * NP, 4 / NP) void dkdv_pair_kernel(BwdArgs a, int n_kt) {
  __shared__ DkdvPairLds<D, NS, NP> sm;
  dkdv_pair_body<D, NS, NP, STAGE>(a, xcd_remap(blockIdx.x, gridDim.x), n_kt, sm);
}

template <int D, int NS, int KS>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a, int n_qt, int vary) {
  __shared__ DqLds<D, NS, KS> sm;
  // query tiles heavy first; with `vary` (the tiles' work differs) the heavy tiles of all
  // the heads an XCD holds first
  int head, rank;
  xcd_tile(blockIdx.x, gridDim.x, n_qt, vary != 0, head, rank);
  dq_body<D, NS, KS>(a, head * n_qt + rank, n_qt, sm);
}

// Both halves of the block backward in one grid: the first n_kv workgroups
// (padded to a multiple of 8, the surplus idle) form dK/dV, the rest dQ. The two
// write disjoint outputs, and sharing a grid lets them fill the chip together
// when each alone is too small to. dK/dV workgroups are the longer ones (their
// keys see the query tiles one after another), so they take the low ids, which
// are dispatched first, and the short dQ workgroups fill the slots they leave.
// Workgroups are dealt to the 8 XCDs round-robin by id, so both roles land on
// every XCD; within a role the ids are remapped as in the single-role kernels.
template <int D, int NSK, int NSQ, int KSQ>
__global__ __launch_bounds__(256, 1) void bwd_fused_kernel(BwdArgs a, int n_kt, int n_qt, int n_kv, int n_kv_pad) {
  __shared__ union {
    DkdvLds<D, NSK> kv;
    DqLds<D, NSQ, KSQ> q;
  } sm;
  const int id = blockIdx.x;
  if (id < n_kv_pad) {
    const int L = xcd_remap(id, n_kv_pad);
    if (L < n_kv) dkdv_body<D, NSK>(a, L, n_kt, sm.kv);
  } else {
    dq_body<D, NSQ, KSQ>(a, xcd_remap(id - n_kv_pad, gridDim.x - n_kv_pad), n_qt, sm.q);
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int which, hipStream_t s) {
  constexpr int NSK = D == 64 ? 4 : 3;  // dK/dV: stages of 64 query rows
  constexpr int NSQ = 4;                // dQ: stages of 32 keys
  const int n_kt = (a.Tk + kKeysPerWG - 1) / kKeysPerWG;
  // 128-wide heads: pairs of waves per dK/dV workgroup (32 keys each) and its Q/dO stages
  constexpr int NPP = 4, NSP = NPP == 4 ? 3 : 2;
  const int n_ktp = (a.Tk + 32 * NPP - 1) / (32 * NPP);
  const int n_qt = (a.Tq + kQPerWG - 1) / kQPerWG;
  const int64_t bh = (int64_t)a.B * a.H;           // (b, query head) for dQ
  const int64_t bkv = (int64_t)a.B * (a.H / a.G);  // (b, KV head) for dK / dV
  // fewer than two dQ workgroups per CU: split their keys between two wave pairs
  const bool split = D == 64 && bh * n_qt < 512;
  const int n_qt2 = (a.Tq + kQPerWG / 2 - 1) / (kQPerWG / 2);
  if constexpr (D == 64) {
    // both kernels keep two workgroups per CU at this width, so one grid costs nothing
    if (which == 3) {
      const int nq = split ? n_qt2 : n_qt;
      const int64_t n_kv = bkv * n_kt, n_kv_pad = (n_kv + 7) / 8 * 8;
      const int64_t grid = n_kv_pad + bh * nq;
      if (split)
        hipLaunchKernelGGL((bwd_fused_kernel<D, NSK, NSQ, 2>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, a, n_kt,
                           nq, (int)n_kv, (int)n_kv_pad);
      else
        hipLaunchKernelGGL((bwd_fused_kernel<D, NSK, NSQ, 1>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, a, n_kt,
                           nq, (int)n_kv, (int)n_kv_pad);
      return hipGetLastError();
    }
  }
  // at D = 128, a causal block whose first and last row tiles see different numbers of keys
  const int vary = D == 128 && a.causal &&
                   a.km.count_le(a.qm.pos(std::min(kQPerWG, a.Tq) - 1)) != a.km.count_le(a.qm.pos(a.Tq - 1));
  if constexpr (D == 128) {
    if (which == 3 && a.ds) {  // dQ from the dS blocks the dK/dV kernel stages
      constexpr int NSD = 6, NWD = 8;  // 256 rows per workgroup, 144 KB of LDS
      hipLaunchKernelGGL((dkdv_pair_kernel<D, NSP, NPP, true>), dim3((unsigned)(bkv * n_ktp)), dim3(128 * NPP), 0,
                         s, a, n_ktp);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int rows = 32 * NWD, n_qs = (a.Tq + rows - 1) / rows;
      const int vary_s = a.causal && a.km.count_le(a.qm.pos(std::min(rows, a.Tq) - 1)) != a.km.count_le(a.qm.pos(a.Tq - 1));
      hipLaunchKernelGGL((dq_staged_kernel<D, NSD, NWD>), dim3((unsigned)(bh * n_qs)), dim3(64 * NWD), 0, s, a, n_qs,
                         vary_s);
      return hipGetLastError();
    }
  }
  if (which & 1) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((dkdv_pair_kernel<D, NSP, NPP, false>), dim3((unsigned)(bkv * n_ktp)), dim3(128 * NPP), 0,
                         s, a, n_ktp);
    else
      hipLaunchKernelGGL((dkdv_kernel<D, NSK>), dim3((unsigned)(bkv * n_kt)), dim3(64 * kNW), 0, s, a, n_kt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (which & 2) {
    if constexpr (D == 64) {
      if (split) {
        hipLaunchKernelGGL((dq_kernel<D, NSQ, 2>), dim3((unsigned)(bh * n_qt2)), dim3(64 * kNW), 0, s, a, n_qt2, 0);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((dq_kernel<D, NSQ, 1>), dim3((unsigned)(bh * n_qt)), dim3(64 * kNW), 0, s, a, n_qt, vary);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int which, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, which, s) : launch_d<128>(a, which, s);
}

}  // namespace cpattn
