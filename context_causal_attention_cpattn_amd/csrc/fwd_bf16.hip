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
//   * one workgroup = 4 waves = 128 query rows of one (b, h) at D = 64 (two
//     workgroups per CU), 8 waves = 256 rows at D = 128 (one per CU); each wave
//     owns 32 rows for the whole kernel and keeps them in registers;
//   * K and V tiles of 64 keys are staged through LDS, double buffered. They
//     are loaded with global_load_lds_dwordx4 (16 bytes per lane straight into
//     LDS, no register staging) into an unpadded, XOR-swizzled layout that is
//     free of bank conflicts both for the 16-byte row reads of the K operand and
//     for the transposing reads of the V^T operand. At D = 128 only waves 4..7
//     issue the tile loads: waves 0..3 enter their matrix work straight after
//     the barrier while the loaders queue 32 KB per tile in the address unit,
//     and the K/V bytes loaded per flop are half those of two 4-wave workgroups;
//   * scores are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16,
//     so every lane holds 16 scores of ONE query row per 32-key block: the row
//     max is an in-lane max3 chain plus one swap with lane l^32, and the row
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
//     one XCD and share its K/V in that XCD's L2; heavy (late) tiles go first,
//     on a causal block at D = 128 those of all the heads an XCD holds;
//   * the loop is software pipelined so that each wave keeps its matrix cores
//     and its vector ALUs busy at the same time (see fwd_bf16_kernel).
// The variant with fused rotary embedding lives in fwd_rope_bf16.hip.

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace cpattn {
namespace {

// Max / sum of a lane's value and that of lane l ^ 32. v_permlane32_swap (a vector ALU
// op, no LDS round trip) swaps the upper 32 lanes of its first operand with the lower 32
// of its second; with the same value in both, every lane gets its own value in one
// result and lane l ^ 32's in the other. Max and sum are symmetric in the two, so both
// halves of the wave end with the same bits.
__device__ __forceinline__ float xor32_max(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kNW = 4;          // waves per workgroup at D = 64
constexpr int kBM = 32 * kNW;   // query rows per workgroup at D = 64
constexpr int kBN = 64;         // keys per tile
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;              // bytes per tile row (no padding)
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = kBN * ROWB;        // bytes per K or V tile
  static constexpr int NC = D / 16;               // 16-wide k-chunks of D
  static constexpr int NDB = D / 32;              // 32-row blocks of D in O^T
  __device__ static __forceinline__ int mask(int r) { return swz_mask<D>(r); }
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

// Wait until at most `units * PER` of this wave's vector loads are outstanding
// (loads complete in issue order). `units` is wave-uniform, 0..4.
template <int PER>
__device__ __forceinline__ void wait_units(int units) {
  switch (units) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    case 3: wait_vm<3 * PER>(); break;
    default: wait_vm<4 * PER>(); break;
  }
}

// Software pipeline (per wave, per key tile j):
//   top:     the scores S_j of tile j are already in registers, masked, with their row max;
//            lazy rescale of the accumulator if the max moved
//   phase A: P_j = exp2(S_j sigma log2e - m) (VALU)  interleaved with  S_{j+1} = K_{j+1} Q^T (MFMA)
//   phase B: O^T += V_j^T P_j^T (MFMA)                 interleaved with  row max of S_{j+1} (VALU)
// so that the matrix cores and the vector ALUs of one wave work at the same time.
// LDS holds NS K tiles and NS V tiles. Load group g = {V_g, K_{g+1}} is issued
// (in that order) at the top of iteration g - NS + 1 and consumed in iteration g.
//
// KS = 2 splits the keys of a workgroup between two pairs of waves, for ring
// steps too small to fill the device: waves 0 and 1 own 32 query rows each and
// take the even key tiles, waves 2 and 3 own the same rows and take the odd
// tiles, each pair with its own LDS rings; at the end the odd pair's partial
// results (accumulator, reference max, row sum) are merged into the even pair's
// through LDS. A workgroup then covers 64 rows, so a step has twice as many
// workgroups, each walking half the keys.
//
// NW is the number of waves of a workgroup (4: two workgroups per CU, 8: one).
// With SPLIT_LOAD only the upper half of a key share's waves issue its tile loads.
template <int D, int NS, int KS, int NW, bool SPLIT_LOAD, bool ROTQ>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(FwdArgs a, int n_qt, int vary) {
  using C = Cfg<D>;
  static_assert(NS >= 2 && NS <= 4, "pipeline depth");
  static_assert(KS == 1 || (KS == 2 && D == 64), "key split: 64-wide heads only");
  constexpr int NR = NW / KS;      // waves per key share (one 32-row block each)
  constexpr int ROWS = 32 * NR;    // query rows per workgroup
  __shared__ __attribute__((aligned(1024))) char ksm[KS][NS][C::TILEB];
  __shared__ __attribute__((aligned(1024))) char vsm[KS][NS][C::TILEB];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, h = l >> 5, lq = l & 31;
  const int rb = w % NR;  // row block of this wave
  const int kh = w / NR;  // key share of this wave: tiles kh, kh + KS, kh + 2 KS, ...

  // (head, query tile), heavy tiles first; with `vary` (the tiles' work differs) the heavy
  // tiles of all the heads an XCD holds first
  int bh, rank;
  xcd_tile(blockIdx.x, gridDim.x, n_qt, vary != 0, bh, rank);
  const int qt = n_qt - 1 - rank;
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = a.row_begin + qt * ROWS;
  const int row = q0 + 32 * rb + lq;
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
  if constexpr (ROTQ) {
    // rotary at the row's global position: d and d + D/2 are a pair, both in this lane
    // (chunks c and c + NC/2); the rounding of every kernel that rotates
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
  // waits for them inside the loop, where the wait would also cover the
  // in-flight LDS loads of later tiles.
#pragma unroll
  for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(qf[c]));

  // ---- key range of this workgroup
  const int last_row = (q0 + ROWS < a.row_end ? q0 + ROWS : a.row_end) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kBN - 1) / kBN;   // key tiles of the workgroup
  const int n_jmax = (n_kt + KS - 1) / KS;     // tiles of the larger share
  const int n_j = n_kt > kh ? (n_kt - kh + KS - 1) / KS : 0;  // tiles of this wave's share
  auto tile = [&](int j) { return KS * j + kh; };
  // Positions increase with the local index, so the keys a query sees are the prefix
  // [0, lim) of the block; the wave's first row has the smallest limit.
  const int wave_first = q0 + 32 * rb < a.row_end ? q0 + 32 * rb : a.row_end - 1;
  const int lim = a.causal ? min(a.Tk, a.km.count_le(qpos)) : a.Tk;
  const int wave_lim = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(wave_first))) : a.Tk;
  // keys past the wave's last row's limit are masked for all of its rows: the tiles from
  // there on only keep the workgroup's barriers and loads going
  const int wave_last = min(q0 + 32 * rb + 31, a.row_end - 1);
  const int wave_end = a.causal ? min(a.Tk, a.km.count_le(a.qm.pos(wave_last))) : a.Tk;

  // ---- direct global -> LDS loads: the NL loader waves of a key share fill the 1 KB slots
  // of that share's tiles, loader lw the slots lw + NL*i (i < NIH). Slot position
  // p = 64*slot + lane is tile row p / CPR, physical chunk p % CPR. The rows of a lane's
  // slots differ by 64*NL/CPR, a multiple of the swizzle period, so the lane's byte offset
  // is the same for all of them and only the (scalar) row base moves.
  constexpr int NL = SPLIT_LOAD ? NR / 2 : NR;    // loader waves per key share
  const bool loader = rb >= NR - NL;              // wave-uniform
  const int lw = rb - (NR - NL);                  // loader index
  constexpr int NIH = kBN * C::CPR / (64 * NL);  // loads per loader wave per tile
  constexpr int kSlotRows = 64 * NL / C::CPR;  // rows between a lane's consecutive slots
  const int ld_r0 = (64 * lw + l) / C::CPR;
  const int ld_col = ((l % C::CPR) ^ C::mask(ld_r0)) * 8;
  const unsigned ko = (unsigned)((ld_r0 * a.k.st + ld_col) * 2);
  const unsigned vo = (unsigned)((ld_r0 * a.v.st + ld_col) * 2);
  // rows past the block repeat the last key (masked later)
  static_assert(kSlotRows % 16 == 0, "slot rows must be a multiple of the swizzle period");
  auto issue = [&](const __bf16* base, int64_t st, unsigned off, int kt, char* dst) {
    if (!loader) return;
    const char* tb = (const char*)(base + (int64_t)kt * kBN * st);
    if (kt * kBN + kBN <= a.Tk) {
#pragma unroll
      for (int i = 0; i < NIH; ++i)
        load_lds16(tb + (int64_t)kSlotRows * i * st * 2, off, dst + (lw + NL * i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NIH; ++i) {
        const int r = min(ld_r0 + kSlotRows * i, a.Tk - 1 - kt * kBN);
        load_lds16(tb, (unsigned)((r * st + ld_col) * 2), dst + (lw + NL * i) * 1024);
      }
    }
  };
  // load group j of this share: V of its tile j, then K of its tile j+1
  auto issue_group = [&](int j) {
    if (j < n_j) issue(vp, a.v.st, vo, tile(j), vsm[kh][j % NS]);
    if (j + 1 < n_j) issue(kp, a.k.st, ko, tile(j + 1), ksm[kh][(j + 1) % NS]);
  };
  auto group_units = [&](int j) { return (j < n_j ? 1 : 0) + (j + 1 < n_j ? 1 : 0); };

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

  // S^T block kb of the K tile in `ks` (operands read as one batch, then the MFMA chain)
  auto scores = [&](const char* ks, int kb) {
    bf16x8 ka[C::NC];
#pragma unroll
    for (int c = 0; c < C::NC; ++c) ka[c] = *(const bf16x8*)(ks + 32 * kb * C::ROWB + koff[c]);
    f32x16 r = f32x16{};
#pragma unroll
    for (int c = 0; c < C::NC; ++c) r = mfma32(ka[c], qf[c], r);
    return r;
  };
  // Keys at or past this row's limit get -inf. Only tiles that reach past the
  // wave's smallest limit can hold such keys.
  auto needs_mask = [&](int kt) { return kt * kBN + kBN > wave_lim; };
  // Element r of 32-key block kb is key kt*kBN + 32kb + 8(r/4) + 4h + r%4; with
  // rel = lim - kt*kBN - 4h the test is a compare against a constant.
  auto mask_rel = [&](int kt) { return lim - kt * kBN - 4 * h; };
  auto mask_elem = [](float v, int rel, int kb, int r) {
    return 32 * kb + 8 * (r >> 2) + (r & 3) < rel ? v : -INFINITY;
  };

  // ---- prologue: K of the share's tile 0, groups 0 .. NS-2, then S and its row max. Every
  // wave of the workgroup passes the same number of barriers: one here when the workgroup
  // has any tile, one per tile of the larger share (a share with fewer tiles pads).
  if (n_j > 0) issue(kp, a.k.st, ko, tile(0), ksm[kh][0]);
  int pending = 0;  // load units issued after that K tile
#pragma unroll
  for (int g = 0; g < NS - 1; ++g) {
    issue_group(g);
    pending += group_units(g);
  }
  f32x16 sA[2] = {f32x16{}, f32x16{}}, sB[2];
  float mx = -INFINITY;
  if (n_kt > 0) {
    wait_units<NIH>(pending);
    __syncthreads();
  }
  if (n_j > 0) {
    sA[0] = scores(ksm[kh][0], 0);
    sA[1] = scores(ksm[kh][0], 1);
    if (needs_mask(tile(0))) {
      const int rel = mask_rel(tile(0));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[kb][r] = mask_elem(sA[kb][r], rel, kb, r);
    }
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sA[kb][r]);
    mx = xor32_max(m);
  }

  // Tile j of this wave's share. `sc` holds its S (masked) and `mx` its row max on entry;
  // with NEXT, S of tile j+1 is formed into `sn` (masked) and `mx` becomes its max.
  // The interleaving is fixed by scheduling fences: each MFMA is followed by the
  // slice of vector work that runs while it executes.
  auto step = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2], auto next_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    // group j (V_j, K_j+1) has landed once only groups j+1 .. j+NS-2 are outstanding
    int later = 0;
#pragma unroll
    for (int g = 1; g <= NS - 2; ++g) later += group_units(j + g);
    wait_units<NIH>(later);
    __syncthreads();  // group j visible to its share; every wave is done with V_j-1 and K_j
    issue_group(j + NS - 1);

    // The two waves of a SIMD belong to one 8-wave workgroup and would otherwise run their
    // tiles in step; a wave forming the next scores takes issue priority over one in its
    // PV products, which staggers them.
    if constexpr (NW == 8) __builtin_amdgcn_s_setprio(1);
    // ---- lazy rescale: the running max moves only when a score exceeds it by 2^8
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

    // ---- phase A: P_kt = exp2(S_kt sigma log2e - mu) in bf16 (+ row sum), while the
    // matrix cores form S_kt+1 = K_kt+1 Q^T. The 2*NC K operands are read LA MFMAs ahead.
    constexpr int EA = 16 / C::NC;  // score elements per MFMA slot
    constexpr int LA = 4;
    const char* kn = ksm[kh][(j + 1) % NS];
    auto kread = [&](int jj) { return *(const bf16x8*)(kn + 32 * (jj / C::NC) * C::ROWB + koff[jj % C::NC]); };
    bf16x8 pb[4];
    bf16x8 ka[LA];
    if constexpr (NEXT) {
#pragma unroll
      for (int jj = 0; jj < LA; ++jj) ka[jj] = kread(jj);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc_s = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        if constexpr (NEXT) {
          const int jj = C::NC * kb + c;
          acc_s = mfma32(ka[jj % LA], qf[c], acc_s);
          if (jj + LA < 2 * C::NC) ka[jj % LA] = kread(jj + LA);
        }
#pragma unroll
        for (int e = 0; e < EA; ++e) {
          const int r = EA * c + e;
          pb[2 * kb + (r >> 3)][r & 7] = (__bf16)fast_exp2(fmaf(sc[kb][r], sl2, -mu));
        }
        if (EA * c + EA == 8) l_part = sum8_bf16(pb[2 * kb], l_part);
        if (EA * c + EA == 16) l_part = sum8_bf16(pb[2 * kb + 1], l_part);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NEXT) sn[kb] = acc_s;
    }

    if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
    // ---- phase B: O^T += V^T P^T (V^T rows = d, 8 keys 16t + 4h + {0..3}, +8), while the
    // vector ALUs take the row max of S_kt+1. V^T operands are read one MFMA ahead.
    constexpr int EB = 32 / (4 * C::NDB);  // score elements per MFMA slot
    const char* vs = vsm[kh][j % NS];
    bf16x8 va[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      va[db] = cat8(lds_read_tr4((const __bf16*)(vs + voff[0][db])),
                    lds_read_tr4((const __bf16*)(vs + voff[1][db])));
    float m2 = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        acc[db] = mfma32(va[db], pb[t], acc[db]);
        if (t < 3) {
          const char* base = vs + 16 * (t + 1) * C::ROWB;
          va[db] = cat8(lds_read_tr4((const __bf16*)(base + voff[0][db])),
                        lds_read_tr4((const __bf16*)(base + voff[1][db])));
        }
        if constexpr (NEXT) {
#pragma unroll
          for (int e = 0; e < EB; ++e) {
            const int i = EB * (C::NDB * t + db) + e, kb = i >> 4, r = i & 15;
            m2 = fmaxf(m2, sn[kb][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (NEXT) {
      // a tile that reaches past the wave's smallest limit is masked and its max redone
      asm volatile("" : "+v"(m2));  // keep the unmasked max beside the PV products
      if (needs_mask(tile(j + 1))) {
        const int rel = mask_rel(tile(j + 1));
        m2 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sn[kb][r] = mask_elem(sn[kb][r], rel, kb, r);
            m2 = fmaxf(m2, sn[kb][r]);
          }
      }
      mx = xor32_max(m2);
    }
  };

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  auto run = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
    step(j, sc, sn, T_{});
  };
  // two tiles per trip so that the score registers alternate instead of being copied
  int n_jl = n_j;  // tiles of the share with a key below the wave's end
  if constexpr (KS == 1) n_jl = min(n_j, (wave_end + kBN - 1) / kBN);
  int j = 0;
  for (; j + 2 < n_jl; j += 2) {
    run(j, sA, sB);
    run(j + 1, sB, sA);
  }
  if (j + 1 < n_jl) {
    run(j, sA, sB);
    step(j + 1, sB, sA, F_{});
  } else if (j < n_jl) {
    step(j, sA, sB, F_{});
  }
  for (int jj = n_jl; jj < n_j; ++jj) {  // masked for every row of this wave
    int later = 0;
#pragma unroll
    for (int g = 1; g <= NS - 2; ++g) later += group_units(jj + g);
    wait_units<NIH>(later);
    __syncthreads();
    issue_group(jj + NS - 1);
  }
  for (int e = n_j; e < n_jmax; ++e) __syncthreads();  // a share with fewer tiles pads

  if constexpr (KS == 2) {
    // ---- merge the odd share's partial result into the even share's, rows alike:
    // [NR waves][NDB*16 accumulator values, reference max, row-sum partial][64 lanes]
    constexpr int NV = C::NDB * 16 + 2;
    static_assert(NR * NV * 64 * 4 <= KS * NS * C::TILEB, "merge staging fits the K rings");
    float* cb = (float*)&ksm[0][0][0] + rb * NV * 64;
    __syncthreads();  // every wave is done with its rings
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) cb[(16 * db + r) * 64 + l] = acc[db][r];
      cb[(NV - 2) * 64 + l] = m_run;
      cb[(NV - 1) * 64 + l] = l_part;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = cb[(NV - 2) * 64 + l], l1 = cb[(NV - 1) * 64 + l];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = acc[db][r] * a0 + cb[(16 * db + r) * 64 + l] * a1;
    l_part = l_part * a0 + l1 * a1;
    m_run = mm;
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2; with a.merge the row is folded into
  // the running (O, LSE) instead, with the arithmetic of the merge kernel (merge.hip)
  const float l_tot = xor32_sum(l_part);
  if (row_ok) {
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    const float lb = live ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    float* op = a.o + b * a.o_sb + hh * a.o_sh + (int64_t)row * a.o_st;
    float* lp = a.lse + b * a.l_sb + hh * a.l_sh + (int64_t)row * a.l_st;
    if (a.merge) {
      // both lanes of the row read the running LSE and their half of the running O before
      // any store
      const float lav = *lp;
      f32x4 xa[C::NDB][4];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) xa[db][g] = *(const f32x4*)(op + 32 * db + 8 * g + 4 * h);
      const float m = fmaxf(lav, lb);
      float wa = 0.f, wb = 0.f, lnew = -INFINITY;
      if (m != -INFINITY) {
        const float ea = expf(lav - m), eb = expf(lb - m);
        const float tot = ea + eb;
        const float r = 1.f / tot;
        wa = ea * r;
        wb = eb * r;
        lnew = m + logf(tot);
      }
      const bool dead = m == -INFINITY;  // no key seen in either part: O = 0
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 ob;
#pragma unroll
          for (int j = 0; j < 4; ++j) ob[j] = acc[db][4 * g + j] * inv;
          *(f32x4*)(op + 32 * db + 8 * g + 4 * h) = dead ? f32x4{} : wa * xa[db][g] + wb * ob;
        }
      if (h == 0) *lp = lnew;
    } else {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = acc[db][4 * g + j] * inv;
          *(f32x4*)(op + 32 * db + 8 * g + 4 * h) = v4;
        }
      if (h == 0) *lp = lb;
    }
  }
}

template <int D, bool ROTQ>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int rows = a.row_end - a.row_begin;
  const int64_t bh = (int64_t)a.B * a.H;
  if (rows <= 0 || bh <= 0) return hipSuccess;
  if constexpr (D == 128) {
    constexpr int NW = 8;
    const int n_qt = (rows + 32 * NW - 1) / (32 * NW);
    // a causal block whose first and last row tiles see different numbers of keys
    const int first_last = std::min(a.row_begin + 32 * NW, a.row_end) - 1;
    const int vary = a.causal && a.km.count_le(a.qm.pos(first_last)) != a.km.count_le(a.qm.pos(a.row_end - 1));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 2, 1, NW, true, ROTQ>), dim3((unsigned)(n_qt * bh)), dim3(64 * NW), 0, s, a,
                       n_qt, vary);
    return hipGetLastError();
  } else {
    const int64_t grid1 = (int64_t)((rows + kBM - 1) / kBM) * bh;
    // fewer than two workgroups per CU: split each workgroup's keys between two wave pairs
    if (grid1 < 512) {
      const int n_qt = (rows + kBM / 2 - 1) / (kBM / 2);
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 2, 2, kNW, false, ROTQ>), dim3((unsigned)(n_qt * bh)), dim3(64 * kNW), 0, s,
                         a, n_qt, 0);
      return hipGetLastError();
    }
    const int n_qt = (rows + kBM - 1) / kBM;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 4, 1, kNW, false, ROTQ>), dim3((unsigned)grid1), dim3(64 * kNW), 0, s, a, n_qt,
                       0);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.rope != nullptr && !a.rope_q) return launch_fwd_rope_bf16(a, s);
  if (a.rope != nullptr) return a.D == 64 ? launch_d<64, true>(a, s) : launch_d<128, true>(a, s);
  return a.D == 64 ? launch_d<64, false>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace cpattn
