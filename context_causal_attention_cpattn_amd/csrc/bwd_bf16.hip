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

#include "internal.h"

namespace cpattn {
namespace {

constexpr int kNW = 4;
constexpr int kPad = 8;

template <int D>
struct BCfg {
  static constexpr int LDP = D + kPad;
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// ------------------------------------------------------------------ dK / dV
constexpr int kKeysPerWG = 32 * kNW;  // 128
constexpr int kQTile = 64;

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a, int n_kt) {
  using C = BCfg<D>;
  constexpr int TILE = kQTile * C::LDP;
  constexpr int CH = kQTile * D / 8 / (64 * kNW);  // 16-byte chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) __bf16 sq[2][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sdo[2][TILE];
  __shared__ __attribute__((aligned(16))) float slse[2][kQTile];
  __shared__ __attribute__((aligned(16))) float sdelta[2][kQTile];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const int Lg = xcd_remap(blockIdx.x, gridDim.x);
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
  const int kpos = a.km.pos(key_ok ? key : a.Tk - 1);
  const int wave_last_key = (kw0 + 31 < a.Tk ? kw0 + 31 : a.Tk - 1);
  const int wave_max_kpos = a.km.pos(wave_last_key < 0 ? 0 : wave_last_key);

  // query rows that can see a key of this workgroup
  const int q_first = a.causal ? a.qm.count_lt(a.km.pos(kc0)) : 0;
  const int t_begin = q_first / kQTile;
  const int t_end = (a.Tq + kQTile - 1) / kQTile;
  const float sl2 = a.scale * kLog2e;

  u32x4 rq[CH], rdo[CH];
  float rl = 0.f, rd = 0.f;
  auto load_tile = [&](int t) {
    const int q0 = t * kQTile;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 64 * kNW * i;
      const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
      const int qrow = q0 + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      rq[i] = rdo[i] = z;
      if (qrow < a.Tq) {
        rq[i] = ldg16(qp + (int64_t)qrow * a.q.st + cc);
        rdo[i] = ldg16(dop + (int64_t)qrow * a.dout.st + cc);
      }
    }
    if (tid < kQTile) {
      const int qrow = q0 + tid;
      rl = INFINITY;  // rows past the end (or without any visible key) give P = 0
      rd = 0.f;
      if (qrow < a.Tq) {
        const float L = lp[(int64_t)qrow * a.lse.st];
        rl = L == -INFINITY ? INFINITY : L * kLog2e;
        rd = dp[(int64_t)qrow * a.delta.st];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 64 * kNW * i;
      const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
      *(u32x4*)(sq[buf] + r * C::LDP + cc) = rq[i];
      *(u32x4*)(sdo[buf] + r * C::LDP + cc) = rdo[i];
    }
    if (tid < kQTile) {
      slse[buf][tid] = rl;
      sdelta[buf][tid] = rd;
    }
  };

  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dk[db] = dv[db] = f32x16{};

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int cur = (t - t_begin) & 1;
    if (t + 1 < t_end) load_tile(t + 1);
    const __bf16* Q = sq[cur];
    const __bf16* DO = sdo[cur];
    const int q0 = t * kQTile;
    const bool full = (q0 + kQTile <= a.Tq) && (key_ok && kw0 + 31 < a.Tk) &&
                      (!a.causal || a.qm.pos(q0) >= wave_max_kpos);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dpv = f32x16{};
      const __bf16* qa = Q + (32 * qb + lq) * C::LDP + 8 * h;
      const __bf16* da = DO + (32 * qb + lq) * C::LDP + 8 * h;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        s = mfma32(*(const bf16x8*)(qa + 16 * c), kf[c], s);
        dpv = mfma32(*(const bf16x8*)(da + 16 * c), vf[c], dpv);
      }
      // rows of s / dpv: query 32qb + 8g + 4h + j, column: this lane's key
      bf16x8 pa[2], dsa[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 L4 = *(const f32x4*)(slse[cur] + 32 * qb + 8 * g + 4 * h);
        const f32x4 D4 = *(const f32x4*)(sdelta[cur] + 32 * qb + 8 * g + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = fast_exp2(fmaf(s[r], sl2, -L4[j]));
          if (!full) {
            const int qrow = q0 + 32 * qb + 8 * g + 4 * h + j;
            const bool vis = key_ok && qrow < a.Tq && (!a.causal || kpos <= a.qm.pos(qrow));
            p = vis ? p : 0.f;
          }
          const float ds = p * (dpv[r] - D4[j]);
          pa[r >> 3][r & 7] = (__bf16)p;
          dsa[r >> 3][r & 7] = (__bf16)ds;
        }
      }
      // dV += P^T dO, dK += dS^T Q ; B operand rows = queries 16tt' + 4h + {0..3}, +8
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int rr = 32 * qb + 16 * tt + 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int col = 32 * db + 16 * ((l >> 4) & 1) + 4 * (l & 3);
          const bf16x8 ob = cat8(lds_read_tr4(DO + rr * C::LDP + col), lds_read_tr4(DO + (rr + 8) * C::LDP + col));
          dv[db] = mfma32(pa[tt], ob, dv[db]);
          const bf16x8 qbv = cat8(lds_read_tr4(Q + rr * C::LDP + col), lds_read_tr4(Q + (rr + 8) * C::LDP + col));
          dk[db] = mfma32(dsa[tt], qbv, dk[db]);
        }
      }
    }
    if (t + 1 < t_end) store_tile(cur ^ 1);
    __syncthreads();
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
constexpr int kKTile = 64;

template <int D>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdArgs a, int n_qt) {
  using C = BCfg<D>;
  constexpr int TILE = kKTile * C::LDP;
  constexpr int CH = kKTile * D / 8 / (64 * kNW);
  __shared__ __attribute__((aligned(16))) __bf16 sk[2][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sv[2][TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const int Lg = xcd_remap(blockIdx.x, gridDim.x);
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
  const int qpos = a.qm.pos(row_ok ? row : a.Tq - 1);
  const int last_row = (q0 + kQPerWG < a.Tq ? q0 + kQPerWG : a.Tq) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kKTile - 1) / kKTile;
  const int wave_first = q0 + 32 * w < a.Tq ? q0 + 32 * w : a.Tq - 1;
  const int wave_min_pos = a.qm.pos(wave_first);
  const float sl2 = a.scale * kLog2e;

  u32x4 rk[CH], rv[CH];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 64 * kNW * i;
      const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
      const int key = kt * kKTile + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      rk[i] = rv[i] = z;
      if (key < a.Tk) {
        rk[i] = ldg16(kp + (int64_t)key * a.k.st + cc);
        rv[i] = ldg16(vp + (int64_t)key * a.v.st + cc);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 64 * kNW * i;
      const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
      *(u32x4*)(sk[buf] + r * C::LDP + cc) = rk[i];
      *(u32x4*)(sv[buf] + r * C::LDP + cc) = rv[i];
    }
  };

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const __bf16* K = sk[cur];
    const __bf16* V = sv[cur];
    const int k0 = kt * kKTile;
    const bool full = (k0 + kKTile <= a.Tk) && (!a.causal || a.km.pos(k0 + kKTile - 1) <= wave_min_pos);
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dpv = f32x16{};
      const __bf16* ka = K + (32 * kb + lq) * C::LDP + 8 * h;
      const __bf16* va = V + (32 * kb + lq) * C::LDP + 8 * h;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        s = mfma32(*(const bf16x8*)(ka + 16 * c), qf[c], s);
        dpv = mfma32(*(const bf16x8*)(va + 16 * c), df[c], dpv);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(s[r], sl2, -lse2));
        if (!full) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool vis = key < a.Tk && (!a.causal || a.km.pos(key) <= qpos);
          p = vis ? p : 0.f;
        }
        dsb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dpv[r] - dl));
      }
    }
    // dQ^T += K^T dS^T ; K^T operand rows = d, 8 keys 16t + 4h + {0..3}, +8
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = 16 * t + 4 * h + ((l & 15) >> 2);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int col = 32 * db + 16 * ((l >> 4) & 1) + 4 * (l & 3);
        const bf16x8 kt8 = cat8(lds_read_tr4(K + rr * C::LDP + col), lds_read_tr4(K + (rr + 8) * C::LDP + col));
        acc[db] = mfma32(kt8, dsb[t], acc[db]);
      }
    }
    if (kt + 1 < n_kt) store_tile(cur ^ 1);
    __syncthreads();
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

template <int D>
hipError_t launch_d(const BwdArgs& a, int which, hipStream_t s) {
  const int n_kt = (a.Tk + kKeysPerWG - 1) / kKeysPerWG;
  const int n_qt = (a.Tq + kQPerWG - 1) / kQPerWG;
  const int64_t bh = (int64_t)a.B * a.H;
  if (which & 1) {
    hipLaunchKernelGGL((dkdv_kernel<D>), dim3((unsigned)(bh * n_kt)), dim3(64 * kNW), 0, s, a, n_kt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (which & 2) {
    hipLaunchKernelGGL((dq_kernel<D>), dim3((unsigned)(bh * n_qt)), dim3(64 * kNW), 0, s, a, n_qt);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int which, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, which, s) : launch_d<128>(a, which, s);
}

}  // namespace cpattn
