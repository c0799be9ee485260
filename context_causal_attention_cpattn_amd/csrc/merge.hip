// Bandwidth-bound kernels: the log-sum-exp merge (SDPAMerger) and the
// backward row term delta = rowsum(dO * O).
//
// Merge (BluScriptCP development log, 2026-03-20 SDPAMerger; 2026-05-20 merge
// of a row range): for every row of the range
//   M = max(L_acc, L_blk), L = M + log(exp(L_acc - M) + exp(L_blk - M)),
//   O = exp(L_acc - L) O_acc + exp(L_blk - L) O_blk,  in place into (O_acc, L_acc).
// Each thread owns 16-byte slices of rows; a row's two LSE values are read by
// all lanes that share the row (one cache line per wave). Bytes per row:
// 3 * 4D (two O reads, one O write) + 12 (two LSE reads, one write).

#include <algorithm>

#include "internal.h"

namespace cpattn {
namespace {

// Each thread owns NV 16-byte slices of one row (D/4/NV threads per row): the two LSE
// values and the weights are formed once per thread, and the NV loads of each operand
// are issued together before any arithmetic. Both O operands are read with
// non-temporal loads (each byte is read once; the result is written in place).
constexpr int kMergeNV = 2;  // float4 per thread

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, int64_t n_thr) {
  constexpr int NV = kMergeNV;
  constexpr int TPR = D / 4 / NV;   // threads per row
  const int rows = a.row_end - a.row_begin;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_thr; i += stride) {
    const int64_t rr = i / TPR;
    const int c = (int)(i - rr * TPR) * 4;  // first column; slices c + 4*TPR*v
    const int64_t bh = rr / rows;
    const int row = a.row_begin + (int)(rr - bh * rows);
    const int b = (int)(bh / a.H), hh = (int)(bh - (int64_t)b * a.H);
    float* la = a.l_acc + b * a.la_sb + hh * a.la_sh + (int64_t)row * a.la_st;
    const float lb = a.l_blk[b * a.lb_sb + hh * a.lb_sh + (int64_t)row * a.lb_st];
    const float lav = *la;
    float* oa = a.o_acc + b * a.oa_sb + hh * a.oa_sh + (int64_t)row * a.oa_st + c;
    const float* ob = a.o_blk + b * a.ob_sb + hh * a.ob_sh + (int64_t)row * a.ob_st + c;
    f32x4 xa[NV], xb[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      xa[v] = __builtin_nontemporal_load((const f32x4*)(oa + 4 * TPR * v));
      xb[v] = __builtin_nontemporal_load((const f32x4*)(ob + 4 * TPR * v));
    }
    const float m = fmaxf(lav, lb);
    float wa = 0.f, wb = 0.f, lnew = -INFINITY;
    if (m != -INFINITY) {
      const float ea = expf(lav - m), eb = expf(lb - m);  // exp(-inf) = 0
      const float tot = ea + eb;
      const float inv = 1.f / tot;
      wa = ea * inv;
      wb = eb * inv;
      lnew = m + logf(tot);
    }
    const bool dead = m == -INFINITY;  // no key seen by the row in either part: O = 0
#pragma unroll
    for (int v = 0; v < NV; ++v) *(f32x4*)(oa + 4 * TPR * v) = dead ? f32x4{} : wa * xa[v] + wb * xb[v];
    if (c == 0) *la = lnew;
  }
}

template <int D>
hipError_t merge_d(const MergeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * (a.row_end - a.row_begin);
  const int64_t n_thr = rows * (D / 4 / kMergeNV);
  if (n_thr <= 0) return hipSuccess;
  int64_t blocks = (n_thr + 255) / 256;
  const int64_t cap = 256 * 64;  // 64 workgroups per CU at most; the loop covers the rest
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s, a, n_thr);
  return hipGetLastError();
}

// delta[row] = sum_d dout[row][d] * o[row][d]; 16 lanes per row, 8 elements each (D = 128)
template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_kernel(PreArgs a, int64_t n_rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rr = gid / LPR;
  const int c = (int)(gid % LPR) * 8;
  float sum = 0.f;
  int b = 0, hh = 0, t = 0;
  if (rr < n_rows) {
    const int64_t bh = rr / a.Tq;
    t = (int)(rr - bh * a.Tq);
    b = (int)(bh / a.H);
    hh = (int)(bh - (int64_t)b * a.H);
    const float* op = (const float*)a.o.p + b * a.o.sb + hh * a.o.sh + (int64_t)t * a.o.st + c;
    const f32x4 o0 = *(const f32x4*)op, o1 = *(const f32x4*)(op + 4);
    float g[8];
    if constexpr (BF16) {
      const __bf16* dp = (const __bf16*)a.dout.p + b * a.dout.sb + hh * a.dout.sh + (int64_t)t * a.dout.st + c;
      const bf16x8 x = *(const bf16x8*)dp;
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = (float)x[e];
    } else {
      const float* dp = (const float*)a.dout.p + b * a.dout.sb + hh * a.dout.sh + (int64_t)t * a.dout.st + c;
      const f32x4 x0 = *(const f32x4*)dp, x1 = *(const f32x4*)(dp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { g[e] = x0[e]; g[e + 4] = x1[e]; }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sum = fmaf(g[e], o0[e], sum);
#pragma unroll
    for (int e = 0; e < 4; ++e) sum = fmaf(g[e + 4], o1[e], sum);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (rr < n_rows && c == 0) a.delta[b * a.d_sb + hh * a.d_sh + (int64_t)t * a.d_st] = sum;
}

template <int D>
hipError_t delta_d(const PreArgs& a, hipStream_t s) {
  const int64_t n_rows = (int64_t)a.B * a.H * a.Tq;
  const int64_t threads = n_rows * (D / 8);
  if (threads <= 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (a.bf16)
    hipLaunchKernelGGL((delta_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, s, a, n_rows);
  else
    hipLaunchKernelGGL((delta_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, s, a, n_rows);
  return hipGetLastError();
}

// Rotary table: table[p][i] = (cos, sin)(p * theta^(-2i/D)); angle and reduction in fp64.
__global__ void rope_table_kernel(double theta, int rows, int D, float* table) {
  const int64_t n = (int64_t)rows * (D / 2);
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n; g += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(g / (D / 2)), i = (int)(g % (D / 2));
    const double inv = pow(theta, -2.0 * (double)i / (double)D);
    const double ang = (double)p * inv;
    table[2 * g] = (float)cos(ang);
    table[2 * g + 1] = (float)sin(ang);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 64: return merge_d<64>(a, s);
    case 128: return merge_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_preprocess(const PreArgs& a, hipStream_t s) {
  switch (a.D) {
    case 64: return delta_d<64>(a, s);
    case 128: return delta_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope_table(double theta, int rows, int D, float* table, hipStream_t s) {
  const int64_t n = (int64_t)rows * (D / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, theta, rows, D, table);
  return hipGetLastError();
}

// Rotary embedding of one [B,H,T,D] bf16 tensor at the global positions of its
// rows: (x_i, x_{i+D/2}) -> (x_i cos - x_{i+D/2} sin, x_{i+D/2} cos + x_i sin),
// angle from the table row of the position (half-split pairing), fp32
// arithmetic, bf16 result rounded to nearest even. One thread rotates 8 pairs
// of one position in HG heads (HG = 16 or 4 when the head count allows): four
// 16-byte loads of the table, shared by the HG heads, then two 16-byte loads
// and two 16-byte stores per head. Each thread reads all its elements before
// writing any, so out may alias x. Sharing the table row among four heads took
// the 32k-window rotation from 31.0 to 29.7 us per call, among sixteen 27.0 to
// 25.9 us.
namespace {
template <int HG>
__global__ __launch_bounds__(256) void rope_rotate_kernel(RotArgs a, int64_t n) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  const int per_row = a.D / 16;  // threads per row
  const int hgroups = a.H / HG;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n; g += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(g % per_row);
    const int64_t rowid = g / per_row;
    const int t = (int)(rowid % a.T);
    const int64_t bg = rowid / a.T;
    const int b = (int)(bg / hgroups), h0 = (int)(bg % hgroups) * HG;
    const f32x4* tb = (const f32x4*)(a.table + (int64_t)a.map.pos(t) * a.D + 16 * c);
    f32x4 cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = tb[j];
    bf16x8 x1[HG], x2[HG];
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      const __bf16* xr = (const __bf16*)a.x.p + b * a.x.sb + (h0 + i) * a.x.sh + (int64_t)t * a.x.st;
      x1[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xr + 8 * c));
      x2[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xr + a.D / 2 + 8 * c));
    }
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      bf16x8 y1, y2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float co = cs[e / 2][2 * (e % 2)], si = cs[e / 2][2 * (e % 2) + 1];
        const float f1 = (float)x1[i][e], f2 = (float)x2[i][e];
        y1[e] = (__bf16)rot_lo(f1, f2, co, si);
        y2[e] = (__bf16)rot_hi(f1, f2, co, si);
      }
      __bf16* orow = a.out + b * a.o_sb + (h0 + i) * a.o_sh + (int64_t)t * a.o_st;
      *(u32x4*)(orow + 8 * c) = __builtin_bit_cast(u32x4, y1);
      *(u32x4*)(orow + a.D / 2 + 8 * c) = __builtin_bit_cast(u32x4, y2);
    }
  }
}
}  // namespace

hipError_t launch_rope_rotate(const RotArgs& a, hipStream_t s) {
  const int hg = a.H % 16 == 0 ? 16 : a.H % 4 == 0 ? 4 : 1;
  const int64_t n = (int64_t)a.B * (a.H / hg) * a.T * (a.D / 16);
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 64);
  if (hg == 16)
    hipLaunchKernelGGL(rope_rotate_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, a, n);
  else if (hg == 4)
    hipLaunchKernelGGL(rope_rotate_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, a, n);
  else
    hipLaunchKernelGGL(rope_rotate_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

// Backward through the rotary embedding: the gradient of the unrotated row is
// R(p)^T times the gradient of the rotated row, i.e. the rotation by -a:
// (g_i, g_{i+D/2}) -> (g_i cos + g_{i+D/2} sin, g_{i+D/2} cos - g_i sin), fp32
// in place. One thread handles 4 pairs (16-byte loads and stores).
namespace {
__global__ __launch_bounds__(256) void rope_rotate_grad_kernel(RotGradArgs a, int64_t n) {
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  const int per_row = a.D / 8;  // threads per row
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n; g += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(g % per_row);
    const int64_t rowid = g / per_row;
    const int t = (int)(rowid % a.T);
    const int64_t bh = rowid / a.T;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    float* row = a.g + b * a.sb + h * a.sh + (int64_t)t * a.st;
    const f32x4 g1 = *(const f32x4*)(row + 4 * c);
    const f32x4 g2 = *(const f32x4*)(row + a.D / 2 + 4 * c);
    const f32x4* tb = (const f32x4*)(a.table + (int64_t)a.map.pos(t) * a.D + 8 * c);
    const f32x4 t0 = tb[0], t1 = tb[1];
    const float co[4] = {t0[0], t0[2], t1[0], t1[2]}, si[4] = {t0[1], t0[3], t1[1], t1[3]};
    f32x4 y1, y2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y1[e] = rot_lo(g1[e], g2[e], co[e], -si[e]);
      y2[e] = rot_hi(g1[e], g2[e], co[e], -si[e]);
    }
    *(f32x4*)(row + 4 * c) = y1;
    *(f32x4*)(row + a.D / 2 + 4 * c) = y2;
  }
}
}  // namespace

hipError_t launch_rope_rotate_grad(const RotGradArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.H * a.T * (a.D / 8);
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(rope_rotate_grad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

}  // namespace cpattn
