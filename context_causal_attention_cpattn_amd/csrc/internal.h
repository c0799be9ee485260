// Host-side launch interface between the C ABI (cpattn_abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace cpattn {

struct View {  // [B,H,T,D] (or [B,H,T]) view; D stride 1
  const void* p;
  int64_t sb, sh, st;
};

struct FwdArgs {
  View q, k, v;
  float* o;
  int64_t o_sb, o_sh, o_st;
  float* lse;
  int64_t l_sb, l_sh, l_st;
  int B, H, Tq, Tk, D;
  PosMap qm, km;
  int causal;
  float scale;
  const float* rope;  // [rope_rows][D/2][2] or null
  int rope_rows;
  // with rope: 0 rotates Q and K inside the kernel (K per tile); 1 rotates only the Q rows,
  // as they are loaded into registers (K arrives rotated by its owner)
  int rope_q;
  int row_begin, row_end;
  int G;  // query heads per KV head: query head h reads K and V head h / G
  int merge;  // 1: fold the block result into (o, lse) as the log-sum-exp merge does; 0: write it
};

struct MergeArgs {
  float* o_acc;
  int64_t oa_sb, oa_sh, oa_st;
  float* l_acc;
  int64_t la_sb, la_sh, la_st;
  const float* o_blk;
  int64_t ob_sb, ob_sh, ob_st;
  const float* l_blk;
  int64_t lb_sb, lb_sh, lb_st;
  int B, H, D;
  int row_begin, row_end;
};

struct PreArgs {
  View dout;
  int bf16;
  View o;
  float* delta;
  int64_t d_sb, d_sh, d_st;
  int B, H, Tq, D;
};

struct BwdArgs {
  View q, k, v, dout;
  View lse, delta;
  float* dq;
  int64_t dq_sb, dq_sh, dq_st;
  float* dk;
  int64_t dk_sb, dk_sh, dk_st;
  float* dv;
  int64_t dv_sb, dv_sh, dv_st;
  int B, H, Tq, Tk, D;
  PosMap qm, km;
  int causal;
  float scale;
  int G;  // query heads per KV head; dK / dV are per KV head, summed over its group
  // 1: add into the accumulator; 0: overwrite it (zeros where no pair contributes)
  int acc_q;   // dQ
  int acc_kv;  // dK and dV
  // Staged dS (128-wide heads, both halves): the dK/dV kernel writes every visible dS block
  // of 32 query rows x 32 keys (bf16, 2 KB) here and the dQ kernel contracts them with K
  // instead of forming S and dP again. Block (b * H + h, qb, kb) starts at byte
  // ((b * H + h) * nqb + qb) * nkb + kb) * 2048, nqb = ceil(Tq / 32), nkb = ceil(Tk / 32).
  // Null: the dQ kernel recomputes dS.
  void* ds;
  int nqb, nkb;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_rope_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_bwd_preprocess(const PreArgs& a, hipStream_t s);
// which: 1 = dK/dV kernel, 2 = dQ kernel, 3 = both
hipError_t launch_bwd_bf16(const BwdArgs& a, int which, hipStream_t s);
hipError_t launch_rope_table(double theta, int rows, int D, float* table, hipStream_t s);

// Rotation of bf16 rows at global positions into a (possibly aliasing) output.
struct RotArgs {
  View x;
  __bf16* out;
  int64_t o_sb, o_sh, o_st;
  int B, H, T, D;
  PosMap map;
  const float* table;  // [rows][D/2][2]
};
hipError_t launch_rope_rotate(const RotArgs& a, hipStream_t s);

// R(p)^T applied in place to fp32 gradient rows at global positions.
struct RotGradArgs {
  float* g;
  int64_t sb, sh, st;
  int B, H, T, D;
  PosMap map;
  const float* table;  // [rows][D/2][2]
};
hipError_t launch_rope_rotate_grad(const RotGradArgs& a, hipStream_t s);

// Records `code` and a printf-style message as the thread's last error (what
// cpattn_last_error returns) and returns `code`; for entry points defined
// outside cpattn_abi.cpp.
int api_fail(int code, const char* fmt, ...);

}  // namespace cpattn
