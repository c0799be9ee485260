// Block forward with fused rotary position embedding (the table form of
// cpattn_block_fwd), bf16 inputs, fp32 accumulation, MFMA (gfx950).
//
// The same block attention as fwd_bf16.hip (partial O and log-sum-exp of the
// local query rows against one KV block at global positions; BluScriptCP
// development log, 2026-04-20 and 2026-06-29), with the rotary embedding of
// 2026-06-29 / 2026-07-10 applied inside the kernel at each row's global
// position: Q is rotated once in the prologue; K is staged through registers
// and rotated on its way to LDS (V still goes global -> LDS directly). Work
// split, LDS layout, score/output transposition, masking, lazy rescale and
// workgroup order are those of fwd_bf16.hip; the loop here is not software
// pipelined (the K rotation sits between the tile load and the barrier).
// The ring driver instead rotates Q and each K block once (cpattn_rope_rotate)
// and runs the plain kernel, which is faster when a block meets many query
// tiles; this form needs no workspace.

#include "internal.h"

namespace cpattn {
namespace {

constexpr int kNW = 4;          // waves per workgroup
constexpr int kBM = 32 * kNW;   // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;              // bytes per tile row (no padding)
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = kBN * ROWB;        // bytes per K or V tile
  static constexpr int NI = kBN * CPR / (64 * kNW);  // direct loads per wave per tile
  static constexpr int NC = D / 16;               // 16-wide k-chunks of D
  static constexpr int NDB = D / 32;              // 32-row blocks of D in O^T
  static constexpr int PAIRS = kBN * (D / 16);    // rotary staging: chunk pairs (c, c + D/2) per tile
  static constexpr int PPT = PAIRS / (64 * kNW);
  __device__ static __forceinline__ int mask(int r) { return swz_mask<D>(r); }
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// K is staged through registers (rotated at its global position on the way to
// LDS), V with direct loads; both double buffered.
template <int D>
__global__ __launch_bounds__(256, 2) void fwd_rope_kernel(FwdArgs a, int n_qt) {
  using C = Cfg<D>;
  constexpr int NS = 2;
  __shared__ __attribute__((aligned(1024))) char smem[NS][2][C::TILEB];  // [stage][K,V]

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qt;
  const int qt = n_qt - 1 - (L - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = a.row_begin + qt * kBM;
  const int row = q0 + 32 * w + lq;
  const bool row_ok = row < a.row_end;

  const __bf16* qp = (const __bf16*)a.q.p + b * a.q.sb + hh * a.q.sh;
  const int kvh = hh / a.G;  // the KV head of this query head's group
  const __bf16* kp = (const __bf16*)a.k.p + b * a.k.sb + kvh * a.k.sh;
  const __bf16* vp = (const __bf16*)a.v.p + b * a.v.sb + kvh * a.v.sh;

  // ---- Q fragment (B operand of S^T): lane holds Q[row][16c + 8h .. +7]
  bf16x8 qf[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (row_ok) t = ldg16(qp + (int64_t)row * a.q.st + 16 * c + 8 * h);
    qf[c] = __builtin_bit_cast(bf16x8, t);
  }
  const int qpos = a.qm.pos(row_ok ? row : a.row_end - 1);
  {
    if (row_ok) {
      const float* tb = a.rope + (int64_t)qpos * D;
#pragma unroll
      for (int c = 0; c < C::NC / 2; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 16 * c + 8 * h + e;
          const float cs = tb[2 * i], sn = tb[2 * i + 1];
          const float x1 = (float)qf[c][e], x2 = (float)qf[c + C::NC / 2][e];
          qf[c][e] = (__bf16)rot_lo(x1, x2, cs, sn);
          qf[c + C::NC / 2][e] = (__bf16)rot_hi(x1, x2, cs, sn);
        }
      }
    }
  }

  // Make the Q loads complete here, before the key loop: otherwise the compiler
  // waits for them inside the loop, where the wait would also cover the next
  // tile's in-flight LDS loads.
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(qf[c]));

  // ---- key range of this workgroup
  const int last_row = (q0 + kBM < a.row_end ? q0 + kBM : a.row_end) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kBN - 1) / kBN;
  // Positions increase with the local index, so the keys a query sees are the prefix
  // [0, lim) of the block; the wave's first row has the smallest limit.
  const int wave_first = q0 + 32 * w < a.row_end ? q0 + 32 * w : a.row_end - 1;
  const int lim = a.causal ? min(a.Tk, a.km.count_le(qpos)) : a.Tk;
  const int wave_lim = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(wave_first))) : a.Tk;

  // ---- direct global -> LDS loads: wave w fills 1 KB slots w*NI .. w*NI+NI-1 of each tile.
  // Slot position p = 64*slot + lane is tile row p / CPR, physical chunk p % CPR. The lane's
  // byte offsets from the tile's first key row are fixed; only the (scalar) tile base moves.
  int ld_row[C::NI], ld_col[C::NI];
  unsigned ko[C::NI], vo[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int p = (w * C::NI + i) * 64 + l;
    const int r = p / C::CPR;
    ld_row[i] = r;
    ld_col[i] = ((p % C::CPR) ^ C::mask(r)) * 8;
    ko[i] = (unsigned)((r * a.k.st + ld_col[i]) * 2);
    vo[i] = (unsigned)((r * a.v.st + ld_col[i]) * 2);
  }
  auto issue_tile = [&](int kt, int buf) {
    const char* kbase = (const char*)(kp + (int64_t)kt * kBN * a.k.st);
    const char* vbase = (const char*)(vp + (int64_t)kt * kBN * a.v.st);
    const bool tail = kt * kBN + kBN > a.Tk;  // rows past the block repeat the last key (masked later)
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      unsigned k_off = ko[i], v_off = vo[i];
      if (tail) {
        const int r = min(ld_row[i], a.Tk - 1 - kt * kBN);
        k_off = (unsigned)((r * a.k.st + ld_col[i]) * 2);
        v_off = (unsigned)((r * a.v.st + ld_col[i]) * 2);
      }
      load_lds16(vbase, v_off, smem[buf][1] + (w * C::NI + i) * 1024);
    }
  };
  // rotary: K chunk pairs (c, c + D/2) of a row through registers
  u32x4 kr[2 * C::PPT];
  f32x4 tr[4 * C::PPT];
  auto load_k_regs = [&](int kt) {
    {
#pragma unroll
      for (int i = 0; i < C::PPT; ++i) {
        const int p = tid + 64 * kNW * i;
        const int r = p / (D / 16), cp = p % (D / 16);
        int key = kt * kBN + r;
        key = key < a.Tk ? key : a.Tk - 1;
        const __bf16* kk = kp + (int64_t)key * a.k.st + 8 * cp;
        kr[2 * i] = ldg16(kk);
        kr[2 * i + 1] = ldg16(kk + D / 2);
        const f32x4* tb = (const f32x4*)(a.rope + (int64_t)a.km.pos(key) * D + 16 * cp);
#pragma unroll
        for (int j = 0; j < 4; ++j) tr[4 * i + j] = tb[j];
      }
    }
  };
  auto store_k_regs = [&](int buf) {
    {
      char* ks = smem[buf][0];
#pragma unroll
      for (int i = 0; i < C::PPT; ++i) {
        const int p = tid + 64 * kNW * i;
        const int r = p / (D / 16), cp = p % (D / 16);
        const bf16x8 x1 = __builtin_bit_cast(bf16x8, kr[2 * i]), x2 = __builtin_bit_cast(bf16x8, kr[2 * i + 1]);
        bf16x8 y1, y2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = tr[4 * i + e / 2][2 * (e % 2)], sn = tr[4 * i + e / 2][2 * (e % 2) + 1];
          const float f1 = (float)x1[e], f2 = (float)x2[e];
          y1[e] = (__bf16)rot_lo(f1, f2, cs, sn);
          y2[e] = (__bf16)rot_hi(f1, f2, cs, sn);
        }
        const int m = C::mask(r);
        *(bf16x8*)(ks + r * C::ROWB + ((cp ^ m) * 16)) = y1;
        *(bf16x8*)(ks + r * C::ROWB + (((cp + C::CPR / 2) ^ m) * 16)) = y2;
      }
    }
  };

  // ---- per-lane LDS byte offsets (swizzled)
  // K operand: row 32kb + lq, logical chunk 2c + h
  int koff[C::NC];
  {
    const int m = C::mask(lq);
#pragma unroll
    for (int c = 0; c < C::NC; ++c) koff[c] = lq * C::ROWB + (((2 * c + h) ^ m) * 16);
  }
  // V^T operand (transposing read): rows 16t + 4h + (l%16)/4 (+8), column 32db + 16((l/16)%2) + 4(l%4)
  int voff[2][C::NDB];
  {
    const int r0 = 4 * h + ((l & 15) >> 2);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = r0 + 8 * hi;
      const int m = C::mask(r);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int cc = 4 * db + 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
        voff[hi][db] = r * C::ROWB + ((cc ^ m) * 16) + (l & 1) * 8;
      }
    }
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = a.scale * kLog2e;

  // prologue: tiles 0 .. NS-2 in flight
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_kt) issue_tile(j, j);
  if (n_kt > 0) {
    load_k_regs(0);
    store_k_regs(0);
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt % NS;
    wait_vm0();  // the K registers of tile kt+1 are loaded each iteration: wait for everything
    __syncthreads();  // tile kt visible to every wave; every wave is done with tile kt-1's stage
    if (kt + NS - 1 < n_kt) {
      issue_tile(kt + NS - 1, (kt + NS - 1) % NS);
      load_k_regs(kt + 1);
    }
    const char* ks = smem[cur][0];
    const char* vs = smem[cur][1];

    // ---- S^T = K Q^T for two 32-key blocks (operands read as one batch per block)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 ka[C::NC];
#pragma unroll
      for (int c = 0; c < C::NC; ++c) ka[c] = *(const bf16x8*)(ks + 32 * kb * C::ROWB + koff[c]);
      __builtin_amdgcn_sched_barrier(0);
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) s[kb] = mfma32(ka[c], qf[c], s[kb]);
    }

    // ---- mask: keys at or past this row's limit (only tiles that reach past the wave's smallest limit)
    const int k0 = kt * kBN;
    if (k0 + kBN > wave_lim) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          s[kb][r] = key < lim ? s[kb][r] : -INFINITY;
        }
    }

    // ---- row max (lane + lane^32), lazy rescale
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
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

    // ---- P = exp2(S * sigma * log2e - m), bf16 pack
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pb[2 * kb + (r >> 3)][r & 7] = (__bf16)fast_exp2(fmaf(s[kb][r], sl2, -mu));
      }
    // row sum of the bf16 weights the PV product uses
#pragma unroll
    for (int t = 0; t < 4; ++t) l_part = sum8_bf16(pb[t], l_part);

    // ---- O^T += V^T P^T ; V^T operand rows = d, 8 keys: 16t + 4h + {0..3} and 16t + 8 + 4h + {0..3}
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const char* base = vs + 16 * t * C::ROWB;
      bf16x8 va[C::NDB];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        va[db] = cat8(lds_read_tr4((const __bf16*)(base + voff[0][db])),
                      lds_read_tr4((const __bf16*)(base + voff[1][db])));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) acc[db] = mfma32(va[db], pb[t], acc[db]);
    }

    if (kt + 1 < n_kt) store_k_regs((kt + 1) % NS);
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

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int rows = a.row_end - a.row_begin;
  const int n_qt = (rows + kBM - 1) / kBM;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_rope_kernel<D>), dim3((unsigned)grid), dim3(64 * kNW), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_rope_bf16(const FwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace cpattn
