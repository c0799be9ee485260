// The ring backward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// cpattn_ring_bwd keeps one intermediate beyond its inputs and outputs: the
// fp32 row term delta = rowsum(dO * O) of the local rows, in a workspace the
// caller brings. cpattn_ring_bwd_noalloc places it in a file-scope device array
// instead, so the call needs no workspace and allocates nothing. Each GPU the
// library runs on holds its own copy of the array (4 MiB) until the process
// ends. Its device address is looked up once per device, on the first call made
// with that device current, and kept; the host-side name of the array is never
// passed to a kernel.

#include <mutex>

#include "../../include/cpattn.h"
#include "internal.h"

namespace {

constexpr size_t kScratchRows = CPATTN_NOALLOC_MAX_ROWS;
static_assert(kScratchRows % 64 == 0, "whole 256-byte lines");

// fp32 delta of up to kScratchRows local rows (B x H x Tq).
__device__ __align__(256) float scratch[kScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return cpattn::api_fail(CPATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return cpattn::api_fail(CPATTN_EUNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return cpattn::api_fail(CPATTN_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CPATTN_OK;
}

}  // namespace

extern "C" int cpattn_ring_bwd_noalloc(const cpattn_tensor* q, const cpattn_tensor* k_blocks,
                                       const cpattn_tensor* v_blocks, const cpattn_posmap* kmaps, int32_t ring,
                                       int32_t rank, const cpattn_posmap* qmap, int32_t dtype, int64_t B, int64_t H,
                                       int64_t Tq, int64_t Tk, int64_t D, int32_t causal, float scale,
                                       const cpattn_tensor* dout, const cpattn_tensor* o, const cpattn_tensor* lse,
                                       const cpattn_tensor* dq_acc, const cpattn_tensor* dk_blocks,
                                       const cpattn_tensor* dv_blocks, int32_t accumulate, void* stream) {
  if (B <= 0 || H <= 0 || Tq <= 0) return cpattn::api_fail(CPATTN_EINVAL, "B, H, Tq must be positive");
  if (B > (int64_t)kScratchRows || H > (int64_t)kScratchRows || Tq > (int64_t)kScratchRows ||
      B * H * Tq > (int64_t)kScratchRows)
    return cpattn::api_fail(CPATTN_EINVAL,
                            "B*H*Tq = %lld rows exceeds the %zu rows of the static scratch (use cpattn_ring_bwd "
                            "with a workspace)",
                            (long long)(B * H * Tq), kScratchRows);
  void* ws = nullptr;
  if (int st = scratch_address(&ws)) return st;
  // exactly delta's share of the array: the dS staging of a larger workspace is never used here
  return cpattn_ring_bwd(q, k_blocks, v_blocks, kmaps, ring, rank, qmap, dtype, B, H, Tq, Tk, D, causal, scale, dout,
                         o, lse, dq_acc, dk_blocks, dv_blocks, accumulate, ws, cpattn_ring_bwd_workspace_bytes(B, H, Tq),
                         stream);
}
