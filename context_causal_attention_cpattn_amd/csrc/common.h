// Shared device-side definitions for the libcpattn kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Local index -> global position: i + (i < split ? d0 : d1), d1 >= d0.
struct PosMap {
  int len, split, d0, d1;
  __device__ __host__ __forceinline__ int pos(int i) const { return i + (i < split ? d0 : d1); }
  // number of local indices whose position is < P (positions increase with i)
  __device__ __host__ __forceinline__ int count_lt(int P) const {
    int a = P - d0;
    a = a < 0 ? 0 : (a > split ? split : a);
    int b = P - d1 - split;
    int tail = len - split;
    b = b < 0 ? 0 : (b > tail ? tail : b);
    return a + b;
  }
  __device__ __host__ __forceinline__ int count_le(int P) const { return count_lt(P + 1); }
};

// Rotation of the pair (x1, x2) by the angle with cosine c and sine s, in one fixed
// rounding order (the second product rounded, then one fused multiply-add), so that every
// kernel that rotates rows -- once into a buffer or per tile inside the forward -- gives
// the same bits: (x1 c - x2 s, x2 c + x1 s).
__device__ __forceinline__ float rot_lo(float x1, float x2, float c, float s) { return fmaf(x1, c, -(x2 * s)); }
__device__ __forceinline__ float rot_hi(float x1, float x2, float c, float s) { return fmaf(x2, c, x1 * s); }

// One v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] B[16x32].
// Lane l supplies A row (l % 32), B column (l % 32), 8 consecutive k values
// each; the accumulator holds column (l % 32), rows 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the accumulator held in AGPRs (the "a" constraint).
// Used for long-lived accumulators so that they do not compete with the
// working set for VGPRs. The compiler cannot see into the asm, so the wait
// states it would otherwise insert are written here: two before the MFMA (a
// VALU write of an operand VGPR followed by the MFMA read); a dependent MFMA on
// the same accumulator needs none. Before the accumulator is read by anything
// else, call mfma_agpr_drain on it.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 24 wait states after the last MFMA writing `acc` (a 16-pass 32x32 MFMA result
// is read back by a VALU/accvgpr instruction); chained through `acc` so that the
// compiler cannot move the read above it.
__device__ __forceinline__ void mfma_agpr_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Transposing LDS read of a 4-row x 16-column block of 16-bit values.
// Within every group of 16 lanes, output lane i element e is element (i % 4)
// of the 8 bytes addressed by source lane 4*e + i/4. To give lane i the
// column i of rows r0..r0+3 of a row-major tile, source lane s must address
// row r0 + (s % 16) / 4, column c0 + 4 * (s % 4).
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fourth word of a raw buffer resource on this architecture family: data format
// 32-bit (DATA_FORMAT = 4), every other field zero. With stride 0 an access is
// in range when its byte offset + size <= num_records; out-of-range loads return
// zero and out-of-range stores are dropped.
constexpr int kBufferFlags = 0x00020000;

// LDS tiles of 16-bit elements, D per row, stored without padding. The 16-byte
// chunk c of row r sits at physical chunk c ^ swz_mask<D>(r). With 64 banks of
// 4 bytes this is free of bank conflicts for (a) 16-byte reads where 16 lanes
// take the same logical chunk of 16 consecutive rows and (b) transposing
// 8-byte reads where 32 lanes take 4 consecutive rows x 32 bytes, and linear
// 16-byte stores (lane i -> i-th chunk of the tile) stay conflict-free too.
template <int D>
__device__ __forceinline__ int swz_mask(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// 16 bytes per lane from global memory straight into LDS at lds_wave_base +
// 16 * lane (global_load_lds_dwordx4). Issued through inline assembly so that
// the compiler adds no conservative wait before later LDS reads: each kernel
// orders these writes itself (s_waitcnt vmcnt(0), then a barrier, before a
// tile is read). Loads complete in issue order, so these extra loads can only
// make the compiler's own vmcnt waits longer, never shorter. An SALU write of
// M0 followed by an LDS-DMA instruction that reads M0 needs one wait state on
// this architecture family; the compiler's hazard recognizer cannot see inside
// the asm block, so the s_nop is written here.
// `base` is wave-uniform (scalar registers); `off` is the lane's unsigned byte
// offset from it.
__device__ __forceinline__ void load_lds16(const void* base, unsigned off, const void* lds_wave_base) {
  const unsigned lds = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// load_lds16 with the non-temporal hint, for data read once (streams that would otherwise
// evict tiles the other workgroups of an XCD still re-read from its L2).
__device__ __forceinline__ void load_lds16_nt(const void* base, unsigned off, const void* lds_wave_base) {
  const unsigned lds = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Sum of the 8 bf16 values of v, added to acc (v_dot2 against (1, 1)).
__device__ __forceinline__ float sum8_bf16(const bf16x8& v, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 4 bytes per lane into LDS at lds_wave_base + 4 * lane (global_load_lds_dword).
__device__ __forceinline__ void load_lds4(const void* base, unsigned off, const void* lds_wave_base) {
  const unsigned lds = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Wait until at most `later * PER` of this wave's vector loads are outstanding,
// i.e. until every tile issued before the `later` most recent ones has landed
// (loads complete in issue order). `later` is wave-uniform and < 4.
template <int PER>
__device__ __forceinline__ void wait_tiles(int later) {
  if (later <= 0) wait_vm<0>();
  else if (later == 1) wait_vm<PER>();
  else if (later == 2) wait_vm<2 * PER>();
  else wait_vm<3 * PER>();
}

// Workgroup id -> logical tile id so that consecutive logical tiles land on
// the same XCD. Workgroups are dealt to the 8 XCDs round-robin by id, so XCD x
// runs ids x, x+8, x+16, ...; logical tiles [x*per + min(x,rem), ...) go there.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = wg & 7, slot = wg >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

// Workgroup id -> (head, rank) for a grid of heads x n_t tiles each, rank 0 the
// heaviest tile of its head. The tiles of a head run on one XCD, as with
// xcd_remap. When `vary` (the tiles of a head differ in work) and an XCD's share
// of the grid is whole heads, its workgroups take the heaviest tiles of all of
// its heads first (head-minor order), so that no head's heavy tiles are dispatched
// last; otherwise head by head (head-major), keeping one head's tiles together.
__device__ __forceinline__ void xcd_tile(int wg, int n, int n_t, bool vary, int& head, int& rank) {
  const int per = n >> 3, rem = n & 7;
  const int x = wg & 7, slot = wg >> 3;
  const int L0 = x * per + (x < rem ? x : rem), cnt = per + (x < rem ? 1 : 0);
  if (vary && L0 % n_t == 0 && cnt % n_t == 0 && cnt > n_t) {
    const int nh = cnt / n_t;
    head = L0 / n_t + slot % nh;
    rank = slot / nh;
  } else {
    const int L = L0 + slot;
    head = L / n_t;
    rank = L - head * n_t;
  }
}

}  // namespace cpattn
