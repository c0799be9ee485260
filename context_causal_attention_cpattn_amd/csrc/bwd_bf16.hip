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
// Two kernels, no atomics (bitwise reproducible):
//   * dkdv: a workgroup owns 128 keys (32 per wave, kept in registers with
//     their V rows) and walks the query tiles that can see them. Scores are
//     formed as S = Q K^T so every lane holds one key; P^T and dS^T then feed
//     the A operand of dV += P^T dO and dK += dS^T Q straight from registers,
//     and dO / Q enter as B operands through the transposing LDS read.
//   * dq: a workgroup owns 128 query rows and walks the visible key tiles, like
//     the forward: S^T = K Q^T and dP^T = V dO^T give one query per lane, and
//     dQ^T += K^T dS^T reads K^T with the transposing LDS read.
// Tiles are staged through LDS with direct global->LDS loads into the
// swizzled, unpadded layout of common.h (double buffered, one barrier per tile).

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

// Workgroup Lg of the dK/dV grid (Lg = bh * n_kt + key tile).
template <int D, int NS>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, int Lg, int n_kt, DkdvLds<D, NS>& sm) {
  using C = BCfg<D>;
  auto& sq = sm.sq;
  auto& sdo = sm.sdo;
  auto& slse = sm.slse;
  auto& sdelta = sm.sdelta;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int bh = Lg / n_kt;
  const int kt = Lg - bh * n_kt;
  const int b = bh / a.H, hh = bh - b * a.H;
  const int kc0 = kt * kKeysPerWG;         // first key of the workgroup
  const int kw0 = kc0 + 32 * w;            // first key of the wave
  const int key = kw0 + lq;                // this lane's key
  const bool key_ok = key < a.Tk;

  const __bf16* qp = (const __bf16*)a.q.p + b * a.q.sb + hh * a.q.sh;
  const __bf16* dop = (const __bf16*)a.dout.p + b * a.dout.sb + hh * a.dout.sh;
  const float* lp = (const float*)a.lse.p + b * a.lse.sb + hh * a.lse.sh;
  const float* dp = (const float*)a.delta.p + b * a.delta.sb + hh * a.delta.sh;

  // K and V rows of this lane's key (B operands: column = key, 8 consecutive d)
  bf16x8 kf[C::NC], vf[C::NC];
  {
    const __bf16* kk = (const __bf16*)a.k.p + b * a.k.sb + hh * a.k.sh + (int64_t)key * a.k.st;
    const __bf16* vv = (const __bf16*)a.v.p + b * a.v.sb + hh * a.v.sh + (int64_t)key * a.v.st;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      u32x4 z = {0u, 0u, 0u, 0u};
      kf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(kk + 16 * c + 8 * h) : z);
      vf[c] = __builtin_bit_cast(bf16x8, key_ok ? ldg16(vv + 16 * c + 8 * h) : z);
    }
  }
  // complete the register loads before the tile loop (see the forward kernel)
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(kf[c]), "v"(vf[c]));
  // Positions increase with the local index, so the query rows that see this lane's key
  // are [qlo, Tq); the wave's last key has the largest qlo.
  const int qlo = a.causal ? a.qm.count_lt(a.km.pos(key_ok ? key : a.Tk - 1)) : 0;
  const int wave_last_key = (kw0 + 31 < a.Tk ? kw0 + 31 : a.Tk - 1);
  const int wave_qlo = a.causal ? a.qm.count_lt(a.km.pos(wave_last_key)) : 0;

  // query rows that can see a key of this workgroup
  const int q_first = a.causal ? a.qm.count_lt(a.km.pos(kc0)) : 0;
  const int t_begin = q_first / kTile;
  const int t_end = (a.Tq + kTile - 1) / kTile;
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
  auto issue_tile = [&](int t, int buf) {
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
    if (t_begin + j < t_end) issue_tile(t_begin + j, j);

  for (int t = t_begin; t < t_end; ++t) {
    const int cur = (t - t_begin) % NS;
    wait_tiles<2 * C::NI + 2>(min(NS - 2, t_end - 1 - t));
    __syncthreads();
    if (t + NS - 1 < t_end) issue_tile(t + NS - 1, (t - t_begin + NS - 1) % NS);
    const char* Q = sq[cur];
    const char* DO = sdo[cur];
    const int q0 = t * kTile;
    const bool full = (q0 + kTile <= a.Tq) && (kw0 + 31 < a.Tk) && (q0 >= wave_qlo);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // operands of S = Q K^T and dP = dO V^T for 32 query rows, read as one batch
      bf16x8 qa[C::NC], da[C::NC];
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        qa[c] = *(const bf16x8*)(Q + 32 * qb * C::ROWB + off.ro[c]);
        da[c] = *(const bf16x8*)(DO + 32 * qb * C::ROWB + off.ro[c]);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = f32x16{}, dpv = f32x16{};
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
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          mfma32_agpr(dv[db], pa[tt], ob[db]);
          mfma32_agpr(dk[db], dsa[tt], qv[db]);
        }
      }
    }
  }

  if (t_begin >= t_end) return;  // no query of this block sees these keys: nothing to add
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    mfma_agpr_drain(dk[db]);
    mfma_agpr_drain(dv[db]);
  }
  // accumulate: lane holds column d = 32db + lq, rows key kw0 + 8g + 4h + j
  float* dkp = a.dk + b * a.dk_sb + hh * a.dk_sh;
  float* dvp = a.dv + b * a.dv_sb + hh * a.dv_sh;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < a.Tk) {
        float* pk = dkp + (int64_t)kr * a.dk_st + 32 * db + lq;
        float* pv = dvp + (int64_t)kr * a.dv_st + 32 * db + lq;
        *pk += a.scale * dk[db][r];
        *pv += dv[db][r];
      }
    }
}

// ------------------------------------------------------------------ dQ
constexpr int kQPerWG = 32 * kNW;  // 128

template <int D, int NS>
struct DqLds {
  alignas(1024) char sk[NS][BCfg<D>::TILEB];
  alignas(1024) char sv[NS][BCfg<D>::TILEB];
};

// Workgroup Lg of the dQ grid (Lg = bh * n_qt + heavy-first query tile).
template <int D, int NS>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int Lg, int n_qt, DqLds<D, NS>& sm) {
  using C = BCfg<D>;
  auto& sk = sm.sk;
  auto& sv = sm.sv;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int bh = Lg / n_qt;
  const int qt = n_qt - 1 - (Lg - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = qt * kQPerWG;
  const int row = q0 + 32 * w + lq;
  const bool row_ok = row < a.Tq;

  const __bf16* kp = (const __bf16*)a.k.p + b * a.k.sb + hh * a.k.sh;
  const __bf16* vp = (const __bf16*)a.v.p + b * a.v.sb + hh * a.v.sh;

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
  // complete the register loads before the tile loop (see the forward kernel)
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(qf[c]), "v"(df[c]));
  asm volatile("" ::"v"(lse2), "v"(dl));

  const int qpos = a.qm.pos(row_ok ? row : a.Tq - 1);
  const int last_row = (q0 + kQPerWG < a.Tq ? q0 + kQPerWG : a.Tq) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kTile - 1) / kTile;
  // the keys this row sees are the prefix [0, lim) of the block (positions increase)
  const int wave_first = q0 + 32 * w < a.Tq ? q0 + 32 * w : a.Tq - 1;
  const int lim = a.causal ? min(a.Tk, a.km.count_le(qpos)) : a.Tk;
  const int wave_lim = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(wave_first))) : a.Tk;
  const float sl2 = a.scale * kLog2e;

  int ld_row[C::NI], ld_col[C::NI];
  unsigned ko[C::NI], vo[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int p = (w * C::NI + i) * 64 + l;
    ld_row[i] = p / C::CPR;
    ld_col[i] = ((p % C::CPR) ^ swz_mask<D>(p / C::CPR)) * 8;
    ko[i] = (unsigned)((ld_row[i] * a.k.st + ld_col[i]) * 2);
    vo[i] = (unsigned)((ld_row[i] * a.v.st + ld_col[i]) * 2);
  }
  auto issue_tile = [&](int kt, int buf) {
    const char* kbase = (const char*)(kp + (int64_t)kt * kTile * a.k.st);
    const char* vbase = (const char*)(vp + (int64_t)kt * kTile * a.v.st);
    const bool tail = kt * kTile + kTile > a.Tk;  // rows past the block repeat the last key (masked)
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      unsigned k_off = ko[i], v_off = vo[i];
      if (tail) {
        const int r = min(ld_row[i], a.Tk - 1 - kt * kTile);
        k_off = (unsigned)((r * a.k.st + ld_col[i]) * 2);
        v_off = (unsigned)((r * a.v.st + ld_col[i]) * 2);
      }
      load_lds16(kbase, k_off, sk[buf] + (w * C::NI + i) * 1024);
      load_lds16(vbase, v_off, sv[buf] + (w * C::NI + i) * 1024);
    }
  };

  const Offs<D> off(l);
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_kt) issue_tile(j, j);

  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt % NS;
    wait_tiles<2 * C::NI>(min(NS - 2, n_kt - 1 - kt));
    __syncthreads();
    if (kt + NS - 1 < n_kt) issue_tile(kt + NS - 1, (kt + NS - 1) % NS);
    const char* K = sk[cur];
    const char* V = sv[cur];
    const int k0 = kt * kTile;
    const bool full = k0 + kTile <= wave_lim;
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dpv = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        s = mfma32(*(const bf16x8*)(K + 32 * kb * C::ROWB + off.ro[c]), qf[c], s);
        dpv = mfma32(*(const bf16x8*)(V + 32 * kb * C::ROWB + off.ro[c]), df[c], dpv);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(s[r], sl2, -lse2));
        if (!full) {
          const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          p = kk < lim ? p : 0.f;
        }
        dsb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dpv[r] - dl));
      }
    }
    // dQ^T += K^T dS^T ; K^T operand rows = d, 8 keys 16t + 4h + {0..3}, +8
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rb = 16 * t * C::ROWB;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        acc[db] = mfma32(cat8(lds_read_tr4((const __bf16*)(K + rb + off.tro[0][db])),
                              lds_read_tr4((const __bf16*)(K + rb + off.tro[1][db]))),
                         dsb[t], acc[db]);
    }
  }

  if (row_ok) {
    float* o = a.dq + b * a.dq_sb + hh * a.dq_sh + (int64_t)row * a.dq_st;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4* p4 = (f32x4*)(o + 32 * db + 8 * g + 4 * h);
        f32x4 v4 = *p4;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] += a.scale * acc[db][4 * g + j];
        *p4 = v4;
      }
  }
}

template <int D, int NS>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a, int n_kt) {
  __shared__ DkdvLds<D, NS> sm;
  dkdv_body<D, NS>(a, xcd_remap(blockIdx.x, gridDim.x), n_kt, sm);
}

template <int D, int NS>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdArgs a, int n_qt) {
  __shared__ DqLds<D, NS> sm;
  dq_body<D, NS>(a, xcd_remap(blockIdx.x, gridDim.x), n_qt, sm);
}

// Both halves of the block backward in one grid: the first n_dq workgroups (a
// multiple of 8, the surplus idle) form dQ, the rest dK/dV. The two write
// disjoint outputs, and sharing a grid lets them fill the chip together when
// each alone is too small to. Workgroups are dealt to the 8 XCDs round-robin by
// id, so both roles land on every XCD; within a role the ids are remapped as in
// the single-role kernels.
template <int D, int NS>
__global__ __launch_bounds__(256, 1) void bwd_fused_kernel(BwdArgs a, int n_kt, int n_qt, int n_dq, int n_dq_pad) {
  __shared__ union {
    DkdvLds<D, NS> kv;
    DqLds<D, NS> q;
  } sm;
  const int id = blockIdx.x;
  if (id < n_dq_pad) {
    const int L = xcd_remap(id, n_dq_pad);
    if (L < n_dq) dq_body<D, NS>(a, L, n_qt, sm.q);
  } else {
    dkdv_body<D, NS>(a, xcd_remap(id - n_dq_pad, gridDim.x - n_dq_pad), n_kt, sm.kv);
  }
}

#ifndef CPATTN_BWD_NS128
#define CPATTN_BWD_NS128 2
#endif

template <int D>
hipError_t launch_d(const BwdArgs& a, int which, hipStream_t s) {
  constexpr int NS = D == 64 ? 4 : CPATTN_BWD_NS128;
  const int n_kt = (a.Tk + kKeysPerWG - 1) / kKeysPerWG;
  const int n_qt = (a.Tq + kQPerWG - 1) / kQPerWG;
  const int64_t bh = (int64_t)a.B * a.H;
  if constexpr (D == 64) {
    // both kernels keep two workgroups per CU at this width, so one grid costs nothing
    if (which == 3) {
    const int64_t n_dq = bh * n_qt, n_dq_pad = (n_dq + 7) / 8 * 8;
    const int64_t grid = n_dq_pad + bh * n_kt;
    hipLaunchKernelGGL((bwd_fused_kernel<D, NS>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, a, n_kt, n_qt,
                       (int)n_dq, (int)n_dq_pad);
    return hipGetLastError();
    }
  }
  if (which & 1) {
    hipLaunchKernelGGL((dkdv_kernel<D, NS>), dim3((unsigned)(bh * n_kt)), dim3(64 * kNW), 0, s, a, n_kt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (which & 2) {
    hipLaunchKernelGGL((dq_kernel<D, NS>), dim3((unsigned)(bh * n_qt)), dim3(64 * kNW), 0, s, a, n_qt);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int which, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, which, s) : launch_d<128>(a, which, s);
}

}  // namespace cpattn
