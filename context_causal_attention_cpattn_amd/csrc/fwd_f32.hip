// Block forward with fp32 inputs and fp32 arithmetic (no bf16 rounding anywhere).
//
// Same operation as the bf16 MFMA kernel (partial O and natural-log LSE of
// local query rows against one KV block at global positions), for inputs whose
// accuracy budget bf16 operands would exceed. Each query row is handled by 4
// lanes that split D into quarters; K/V tiles of 32 keys are staged in LDS and
// read as broadcasts. The softmax is rescaled once per tile with the exact
// (libm) exponential.

#include "internal.h"

namespace cpattn {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (4 lanes each)
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a, int n_qt) {
  constexpr int DQ = D / 4;
  __shared__ __attribute__((aligned(16))) float ks[kKeys][D];
  __shared__ __attribute__((aligned(16))) float vs[kKeys][D];

  const int tid = threadIdx.x;
  const int lr = tid >> 2, part = tid & 3;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / n_qt;
  const int qt = n_qt - 1 - (L - bh * n_qt);
  const int b = bh / a.H, hh = bh - b * a.H;
  const int q0 = a.row_begin + qt * kRows;
  const int row = q0 + lr;
  const bool row_ok = row < a.row_end;

  const float* qp = (const float*)a.q.p + b * a.q.sb + hh * a.q.sh;
  const int kvh = hh / a.G;  // the KV head of this query head's group
  const float* kp = (const float*)a.k.p + b * a.k.sb + kvh * a.k.sh;
  const float* vp = (const float*)a.v.p + b * a.v.sb + kvh * a.v.sh;

  float q[DQ], acc[DQ];
#pragma unroll
  for (int d = 0; d < DQ; ++d) {
    q[d] = row_ok ? qp[(int64_t)row * a.q.st + part * DQ + d] : 0.f;
    acc[d] = 0.f;
  }
  const int qpos = a.qm.pos(row_ok ? row : a.row_end - 1);
  const int last_row = (q0 + kRows < a.row_end ? q0 + kRows : a.row_end) - 1;
  const int n_vis = a.causal ? a.km.count_le(a.qm.pos(last_row)) : a.Tk;
  const int n_kt = (n_vis + kKeys - 1) / kKeys;

  float m = -INFINITY, lsum = 0.f;
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    for (int i = tid; i < kKeys * D / 4; i += 256) {
      const int r = i / (D / 4), c = (i % (D / 4)) * 4;
      const int key = kt * kKeys + r;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < a.Tk) {
        kv = *(const f32x4*)(kp + (int64_t)key * a.k.st + c);
        vv = *(const f32x4*)(vp + (int64_t)key * a.v.st + c);
      }
      *(f32x4*)&ks[r][c] = kv;
      *(f32x4*)&vs[r][c] = vv;
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DQ; ++d) dot = fmaf(q[d], ks[j][part * DQ + d], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const int key = kt * kKeys + j;
      const bool vis = key < a.Tk && (!a.causal || a.km.pos(key) <= qpos);
      s[j] = vis ? dot * a.scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new == -INFINITY) continue;  // nothing visible yet for this row
    const float corr = expf(m - m_new);  // m = -inf -> 0
    lsum *= corr;
#pragma unroll
    for (int d = 0; d < DQ; ++d) acc[d] *= corr;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_new);
      lsum += p;
#pragma unroll
      for (int d = 0; d < DQ; ++d) acc[d] = fmaf(p, vs[j][part * DQ + d], acc[d]);
    }
    m = m_new;
  }
  if (!row_ok) return;
  const bool live = lsum > 0.f;
  float* op = a.o + b * a.o_sb + hh * a.o_sh + (int64_t)row * a.o_st + part * DQ;
#pragma unroll
  for (int d = 0; d < DQ; ++d) op[d] = live ? acc[d] / lsum : 0.f;
  if (part == 0) a.lse[b * a.l_sb + hh * a.l_sh + (int64_t)row * a.l_st] = live ? m + logf(lsum) : -INFINITY;
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const int rows = a.row_end - a.row_begin;
  const int n_qt = (rows + kRows - 1) / kRows;
  const int64_t grid = (int64_t)n_qt * a.B * a.H;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace cpattn
