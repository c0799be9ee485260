// Block forward of causal ring attention, bf16 inputs, fp32 accumulation, MFMA (gfx950).
//
// Computes, for the local query rows of one ring step against one KV block at
// global positions, the partial output O and its log-sum-exp (BluScriptCP
// development log: 2026-04-20 CP-aware attention with separate query/key
// lengths and offsets; 2026-06-29 requirements: dual-offset global-causal
// mask, log-sum-exp as an output; 2026-07-10: positions through head/tail
// deltas).
//
// Work decomposition
//   * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
//     rows for the whole kernel;
//   * K and V tiles of 64 keys are staged through LDS, double buffered, loaded
//     with coalesced 16-byte global loads;
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16,
//     so every lane holds 16 scores of ONE query row per 32-key block: the row
//     max is an in-lane max3 chain plus one exchange with lane l^32, and the row
//     sum stays a per-lane partial until the epilogue;
//   * the output is accumulated transposed, O^T += V^T P^T: P comes straight
//     from the score registers (same lane = same query), and V^T is read from
//     the row-major V tile with the transposing LDS read (ds_read_b64_tr_b16);
//   * the causal mask is tested only on tiles that straddle the diagonal in
//     global positions; tiles past the last visible key are never loaded;
//   * the softmax max is rescaled lazily: the running max moves only when a new
//     score exceeds it by more than 2^8, so the accumulator is rarely rescaled
//     (exact: O and the row sum always share the same reference max);
//   * workgroup ids are remapped so that the query tiles of one (b, h) run on
//     one XCD and share its K/V in that XCD's L2; heavy (late) tiles go first.

#include "internal.h"

namespace cpattn {
namespace {

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBM = 32 * kNW;   // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr int kPad = 8;         // LDS row padding (elements)
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct Cfg {
  static constexpr int LDP = D + kPad;             // LDS row pitch (elements)
  static constexpr int TILE = kBN * LDP;           // elements per K or V tile
  static constexpr int PAIRS = kBN * (D / 16);     // 16-byte chunk pairs (c, c + D/2) per tile
  static constexpr int PPT = PAIRS / (64 * kNW);   // pairs per thread
  static constexpr int NC = D / 16;                // 16-wide k-chunks of D
  static constexpr int NDB = D / 32;               // 32-row blocks of D in O^T
  static_assert(PAIRS % (64 * kNW) == 0, "tile split");
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

template <int D, bool ROPE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a, int n_qt) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][C::TILE];  // [buf][K,V]

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qt;
  const int qt = n_qt - 1 - (L - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = a.row_begin + qt * kBM;
  const int row = q0 + 32 * w + lq;
  const bool row_ok = row < a.row_end;

  const __bf16* qp = (const __bf16*)a.q.p + b * a.q.sb + hh * a.q.sh;
  const __bf16* kp = (const __bf16*)a.k.p + b * a.k.sb + hh * a.k.sh;
  const __bf16* vp = (const __bf16*)a.v.p + b * a.v.sb + hh * a.v.sh;

  // ---- Q fragment (B operand of S^T): lane holds Q[row][16c + 8h .. +7]
  bf16x8 qf[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (row_ok) t = ldg16(qp + (int64_t)row * a.q.st + 16 * c + 8 * h);
    qf[c] = __builtin_bit_cast(bf16x8, t);
  }
  const int qpos = a.qm.pos(row_ok ? row : a.row_end - 1);
  if constexpr (ROPE) {
    if (row_ok) {
      const float* tb = a.rope + (int64_t)qpos * D;
#pragma unroll
      for (int c = 0; c < C::NC / 2; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 16 * c + 8 * h + e;
          const float cs = tb[2 * i], sn = tb[2 * i + 1];
          const float x1 = (float)qf[c][e], x2 = (float)qf[c + C::NC / 2][e];
          qf[c][e] = (__bf16)(x1 * cs - x2 * sn);
          qf[c + C::NC / 2][e] = (__bf16)(x2 * cs + x1 * sn);
        }
      }
    }
  }

  // ---- key range of this workgroup
  const int last_row = (q0 + kBM < a.row_end ? q0 + kBM : a.row_end) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kBN - 1) / kBN;
  const int wave_first = q0 + 32 * w < a.row_end ? q0 + 32 * w : a.row_end - 1;
  const int wave_min_pos = a.qm.pos(wave_first);

  // ---- global -> register staging of one K/V tile (chunk pairs c, c + D/2 of a row)
  u32x4 kr[2 * C::PPT], vr[2 * C::PPT];
  f32x4 tr[ROPE ? 4 * C::PPT : 1];  // rotary (cos, sin) pairs for the K chunk pairs
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = tid + 64 * kNW * i;
      const int r = p / (D / 16), cp = p % (D / 16);
      const int key = kt * kBN + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      kr[2 * i] = kr[2 * i + 1] = vr[2 * i] = vr[2 * i + 1] = z;
      if (key < a.Tk) {
        const __bf16* kk = kp + (int64_t)key * a.k.st + 8 * cp;
        const __bf16* vv = vp + (int64_t)key * a.v.st + 8 * cp;
        kr[2 * i] = ldg16(kk);
        kr[2 * i + 1] = ldg16(kk + D / 2);
        vr[2 * i] = ldg16(vv);
        vr[2 * i + 1] = ldg16(vv + D / 2);
        if constexpr (ROPE) {
          const f32x4* tb = (const f32x4*)(a.rope + (int64_t)a.km.pos(key) * D + 16 * cp);
#pragma unroll
          for (int j = 0; j < 4; ++j) tr[4 * i + j] = tb[j];
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* ks = smem[buf][0];
    __bf16* vs = smem[buf][1];
#pragma unroll
    for (int i = 0; i < C::PPT; ++i) {
      const int p = tid + 64 * kNW * i;
      const int r = p / (D / 16), cp = p % (D / 16);
      u32x4 k0 = kr[2 * i], k1 = kr[2 * i + 1];
      if constexpr (ROPE) {
        bf16x8 x1 = __builtin_bit_cast(bf16x8, k0), x2 = __builtin_bit_cast(bf16x8, k1);
        bf16x8 y1, y2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = tr[4 * i + e / 2][2 * (e % 2)], sn = tr[4 * i + e / 2][2 * (e % 2) + 1];
          const float f1 = (float)x1[e], f2 = (float)x2[e];
          y1[e] = (__bf16)(f1 * cs - f2 * sn);
          y2[e] = (__bf16)(f2 * cs + f1 * sn);
        }
        k0 = __builtin_bit_cast(u32x4, y1);
        k1 = __builtin_bit_cast(u32x4, y2);
      }
      *(u32x4*)(ks + r * C::LDP + 8 * cp) = k0;
      *(u32x4*)(ks + r * C::LDP + 8 * cp + D / 2) = k1;
      *(u32x4*)(vs + r * C::LDP + 8 * cp) = vr[2 * i];
      *(u32x4*)(vs + r * C::LDP + 8 * cp + D / 2) = vr[2 * i + 1];
    }
  };

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale * kLog2e;

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const __bf16* ks = smem[cur][0];
    const __bf16* vs = smem[cur][1];

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const __bf16* kr0 = ks + (32 * kb + lq) * C::LDP + 8 * h;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) s[kb] = mfma32(*(const bf16x8*)(kr0 + 16 * c), qf[c], s[kb]);
    }

    // ---- mask (tiles that straddle the diagonal or the end of the block)
    const int k0 = kt * kBN;
    const bool full = (k0 + kBN <= a.Tk) && (!a.causal || a.km.pos(k0 + kBN - 1) <= wave_min_pos);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool vis = key < a.Tk && (!a.causal || a.km.pos(key) <= qpos);
          if (!vis) s[kb][r] = -INFINITY;
        }
    }

    // ---- row max (lane + lane^32), lazy rescale
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * sl2;
    const bool need = m_tile > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? m_tile : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_new;
    }
    const float mu = m_run == -INFINITY ? 0.f : m_run;

    // ---- P = exp2(S * sigma * log2e - m), row sum, bf16 pack
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], sl2, -mu));
        l_part += p;
        pb[2 * kb + (r >> 3)][r & 7] = (__bf16)p;
      }

    // ---- O^T += V^T P^T ; V^T operand rows = d, 8 keys: 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int col = 32 * db + 16 * ((l >> 4) & 1) + 4 * (l & 3);
        const int rr = 16 * t + 4 * h + ((l & 15) >> 2);
        const bf16x4 lo = lds_read_tr4(vs + rr * C::LDP + col);
        const bf16x4 hi = lds_read_tr4(vs + (rr + 8) * C::LDP + col);
        acc[db] = mfma32(cat8(lo, hi), pb[t], acc[db]);
      }
    }

    if (kt + 1 < n_kt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (row_ok) {
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    float* op = a.o + b * a.o_sb + hh * a.o_sh + (int64_t)row * a.o_st;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = acc[db][4 * g + j] * inv;
        *(f32x4*)(op + 32 * db + 8 * g + 4 * h) = v4;
      }
    if (h == 0) {
      a.lse[b * a.l_sb + hh * a.l_sh + (int64_t)row * a.l_st] =
          live ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool ROPE>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int rows = a.row_end - a.row_begin;
  const int n_qt = (rows + kBM - 1) / kBM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, ROPE>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const bool rope = a.rope != nullptr;
  if (a.D == 64) return rope ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
  return rope ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace cpattn
