// C ABI of libcpattn: argument validation, the HeadTail shard map, the ring
// driver and dispatch to the HIP kernels. No exception crosses the boundary;
// every error is a status code plus a thread-local message.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/cpattn.h"
#include "internal.h"

using namespace cpattn;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return CPATTN_OK;
}

}  // namespace

int cpattn::api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

namespace {

constexpr int64_t kIntMax = 2147483647;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A [B,H,T,D] tensor of `esize`-byte elements: non-null, 16-byte aligned,
// strides that keep every row 16-byte aligned.
int check_tensor(const cpattn_tensor* t, const char* name, int esize) {
  if (!t || !t->data) return fail(CPATTN_EINVAL, "%s: null tensor", name);
  if (!aligned16(t->data)) return fail(CPATTN_EINVAL, "%s: pointer not 16-byte aligned", name);
  const int64_t q = 16 / esize;
  if (t->sb % q || t->sh % q || t->st % q)
    return fail(CPATTN_EINVAL, "%s: B/H/T strides must be multiples of %lld elements", name, (long long)q);
  if (t->sb < 0 || t->sh < 0 || t->st < 0) return fail(CPATTN_EINVAL, "%s: negative stride", name);
  // kernels address a 64-row tile with 32-bit byte offsets
  if (t->st * 64 * esize >= (int64_t)1 << 31) return fail(CPATTN_EINVAL, "%s: T stride too large", name);
  return CPATTN_OK;
}

int check_rows(const cpattn_tensor* t, const char* name) {  // [B,H,T] fp32
  if (!t || !t->data) return fail(CPATTN_EINVAL, "%s: null tensor", name);
  if (((uintptr_t)t->data & 3u) != 0) return fail(CPATTN_EINVAL, "%s: pointer not 4-byte aligned", name);
  if (t->sb < 0 || t->sh < 0 || t->st < 0) return fail(CPATTN_EINVAL, "%s: negative stride", name);
  return CPATTN_OK;
}

int check_map(const cpattn_posmap* m, int64_t len, const char* name) {
  if (!m) return fail(CPATTN_EINVAL, "%s: null map", name);
  if (m->len != len) return fail(CPATTN_EINVAL, "%s: len %lld != %lld", name, (long long)m->len, (long long)len);
  if (m->split < 0 || m->split > m->len) return fail(CPATTN_EINVAL, "%s: split outside [0, len]", name);
  if (m->d1 < m->d0) return fail(CPATTN_EINVAL, "%s: d1 < d0 (positions must increase)", name);
  if (m->d0 < 0) return fail(CPATTN_EINVAL, "%s: negative position", name);
  if (m->len + m->d1 >= kIntMax) return fail(CPATTN_EINVAL, "%s: positions exceed 2^31", name);
  return CPATTN_OK;
}

PosMap to_map(const cpattn_posmap* m) {
  return PosMap{(int)m->len, (int)m->split, (int)m->d0, (int)m->d1};
}

View view(const cpattn_tensor* t) { return View{t->data, t->sb, t->sh, t->st}; }

// Largest global position in the map (the last index; positions increase).
int64_t max_pos(const cpattn_posmap* m) {
  if (m->len <= 0) return -1;
  const int64_t i = m->len - 1;
  return i + (i < m->split ? m->d0 : m->d1);
}

int check_dims(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D) {
  if (B <= 0 || H <= 0 || Tq <= 0 || Tk <= 0 || D <= 0)
    return fail(CPATTN_EINVAL, "B, H, Tq, Tk, D must be positive");
  if (B * H > kIntMax || Tq > kIntMax || Tk > kIntMax) return fail(CPATTN_EINVAL, "sizes exceed 2^31");
  if (D != 64 && D != 128) return fail(CPATTN_EUNSUPPORTED, "D = %lld (supported: 64, 128)", (long long)D);
  return CPATTN_OK;
}

int build_fwd(FwdArgs& a, const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int32_t dtype,
              int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap,
              const cpattn_posmap* kmap, int32_t causal, float scale, const float* rope, int64_t rope_rows,
              int64_t row_begin, int64_t row_end, const cpattn_tensor* o, const cpattn_tensor* lse) {
  int st;
  if ((st = check_dims(B, H, Tq, Tk, D))) return st;
  if (dtype != CPATTN_F32 && dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "dtype %d", (int)dtype);
  const int es = dtype == CPATTN_BF16 ? 2 : 4;
  if ((st = check_tensor(q, "q", es)) || (st = check_tensor(k, "k", es)) || (st = check_tensor(v, "v", es)) ||
      (st = check_tensor(o, "o", 4)) || (st = check_rows(lse, "lse")))
    return st;
  if ((st = check_map(qmap, Tq, "qmap")) || (st = check_map(kmap, Tk, "kmap"))) return st;
  if (row_begin < 0 || row_end > Tq || row_begin >= row_end)
    return fail(CPATTN_EINVAL, "row range [%lld, %lld) outside [0, %lld) or empty", (long long)row_begin,
                (long long)row_end, (long long)Tq);
  if (!(scale >= 0.f) || std::isinf(scale)) return fail(CPATTN_EINVAL, "scale must be finite and >= 0");
  if (rope) {
    if (dtype != CPATTN_BF16) return fail(CPATTN_EUNSUPPORTED, "rotary table with fp32 inputs");
    if (((uintptr_t)rope & 15u) != 0) return fail(CPATTN_EINVAL, "rope table not 16-byte aligned");
    if (rope_rows <= 0 || rope_rows > kIntMax) return fail(CPATTN_EINVAL, "rope_rows");
    if (max_pos(qmap) >= rope_rows || max_pos(kmap) >= rope_rows)
      return fail(CPATTN_EINVAL, "a global position is outside the rotary table (%lld rows)", (long long)rope_rows);
  }
  a.q = view(q);
  a.k = view(k);
  a.v = view(v);
  a.o = (float*)o->data;
  a.o_sb = o->sb, a.o_sh = o->sh, a.o_st = o->st;
  a.lse = (float*)lse->data;
  a.l_sb = lse->sb, a.l_sh = lse->sh, a.l_st = lse->st;
  a.B = (int)B, a.H = (int)H, a.Tq = (int)Tq, a.Tk = (int)Tk, a.D = (int)D;
  a.qm = to_map(qmap);
  a.km = to_map(kmap);
  a.causal = causal != 0;
  a.scale = scale == 0.f ? (float)(1.0 / std::sqrt((double)D)) : scale;
  a.rope = rope;
  a.rope_rows = (int)rope_rows;
  a.row_begin = (int)row_begin;
  a.row_end = (int)row_end;
  a.G = 1;
  return CPATTN_OK;
}

// Query heads per KV head for H query heads sharing H_kv KV heads.
int group_of(int64_t H, int64_t H_kv, int* G) {
  if (H_kv <= 0 || H_kv > H || H % H_kv != 0)
    return fail(CPATTN_EINVAL, "H = %lld is not a multiple of H_kv = %lld", (long long)H, (long long)H_kv);
  *G = (int)(H / H_kv);
  return CPATTN_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CPATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int cpattn_version(void) { return CPATTN_ABI_VERSION; }

const char* cpattn_last_error(void) { return g_err; }

int cpattn_headtail_shard(int64_t T, int32_t ring, int32_t rank, cpattn_posmap* map, int32_t* positions) {
  if (!map) return fail(CPATTN_EINVAL, "map is NULL");
  if (T <= 0 || ring <= 0) return fail(CPATTN_EINVAL, "T and ring must be positive");
  if (T >= kIntMax) return fail(CPATTN_EINVAL, "T must be below 2^31");
  if (T % (2 * (int64_t)ring) != 0) return fail(CPATTN_EINVAL, "T %% (2*ring) != 0");
  if (rank < 0 || rank >= ring) return fail(CPATTN_EINVAL, "rank outside [0, ring)");
  const int64_t c = T / (2 * (int64_t)ring);
  map->len = 2 * c;
  map->split = c;
  map->d0 = (int64_t)rank * c;                       // head chunk `rank`
  map->d1 = (int64_t)(2 * ring - 1 - rank) * c - c;  // tail chunk 2*ring-1-rank, local index starts at c
  if (positions)
    for (int64_t i = 0; i < 2 * c; ++i) positions[i] = (int32_t)(i + (i < c ? map->d0 : map->d1));
  return ok();
}

int cpattn_rope_table(double theta, int64_t rows, int64_t D, float* table, void* stream) {
  if (!(theta > 0.0) || std::isinf(theta)) return fail(CPATTN_EINVAL, "theta must be positive");
  if (rows <= 0 || rows > kIntMax || D <= 0 || D % 2 || D > 4096) return fail(CPATTN_EINVAL, "rows / D");
  if (!table) return fail(CPATTN_EINVAL, "table is NULL");
  return launch_status(launch_rope_table(theta, (int)rows, (int)D, table, (hipStream_t)stream), "rope_table");
}

int cpattn_rope_rotate(const cpattn_tensor* x, int32_t dtype, int64_t B, int64_t H, int64_t T, int64_t D,
                       const cpattn_posmap* map, const float* rope_table, int64_t rope_rows,
                       const cpattn_tensor* out, void* stream) {
  int st;
  if ((st = check_dims(B, H, T, T, D))) return st;
  if (dtype != CPATTN_BF16) return fail(CPATTN_EUNSUPPORTED, "rotation of dtype %d (bf16 only)", (int)dtype);
  if ((st = check_tensor(x, "x", 2)) || (st = check_tensor(out, "out", 2))) return st;
  if ((st = check_map(map, T, "map"))) return st;
  if (!rope_table || ((uintptr_t)rope_table & 15u) != 0) return fail(CPATTN_EINVAL, "rope table null or misaligned");
  if (rope_rows <= 0 || rope_rows > kIntMax) return fail(CPATTN_EINVAL, "rope_rows");
  if (max_pos(map) >= rope_rows)
    return fail(CPATTN_EINVAL, "a global position is outside the rotary table (%lld rows)", (long long)rope_rows);
  RotArgs a{};
  a.x = view(x);
  a.out = (__bf16*)out->data;
  a.o_sb = out->sb, a.o_sh = out->sh, a.o_st = out->st;
  a.B = (int)B, a.H = (int)H, a.T = (int)T, a.D = (int)D;
  a.map = to_map(map);
  a.table = rope_table;
  return launch_status(launch_rope_rotate(a, (hipStream_t)stream), "rope_rotate");
}

int cpattn_rope_rotate_grad(const cpattn_tensor* g, int64_t B, int64_t H, int64_t T, int64_t D,
                            const cpattn_posmap* map, const float* rope_table, int64_t rope_rows, void* stream) {
  int st;
  if ((st = check_dims(B, H, T, T, D))) return st;
  if ((st = check_tensor(g, "g", 4))) return st;
  if ((st = check_map(map, T, "map"))) return st;
  if (!rope_table || ((uintptr_t)rope_table & 15u) != 0) return fail(CPATTN_EINVAL, "rope table null or misaligned");
  if (rope_rows <= 0 || rope_rows > kIntMax) return fail(CPATTN_EINVAL, "rope_rows");
  if (max_pos(map) >= rope_rows)
    return fail(CPATTN_EINVAL, "a global position is outside the rotary table (%lld rows)", (long long)rope_rows);
  RotGradArgs a{};
  a.g = (float*)g->data;
  a.sb = g->sb, a.sh = g->sh, a.st = g->st;
  a.B = (int)B, a.H = (int)H, a.T = (int)T, a.D = (int)D;
  a.map = to_map(map);
  a.table = rope_table;
  return launch_status(launch_rope_rotate_grad(a, (hipStream_t)stream), "rope_rotate_grad");
}

int cpattn_block_fwd(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int32_t dtype,
                     int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap,
                     const cpattn_posmap* kmap, int32_t causal, float scale, const float* rope_table,
                     int64_t rope_rows, int64_t row_begin, int64_t row_end, const cpattn_tensor* o,
                     const cpattn_tensor* lse, void* stream) {
  FwdArgs a{};
  int st = build_fwd(a, q, k, v, dtype, B, H, Tq, Tk, D, qmap, kmap, causal, scale, rope_table, rope_rows,
                     row_begin, row_end, o, lse);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  return launch_status(dtype == CPATTN_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s), "block_fwd");
}

int cpattn_block_fwd_gqa(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int32_t dtype,
                         int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t D,
                         const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal, float scale,
                         const float* rope_table, int64_t rope_rows, int64_t row_begin, int64_t row_end,
                         const cpattn_tensor* o, const cpattn_tensor* lse, void* stream) {
  FwdArgs a{};
  int G;
  int st = build_fwd(a, q, k, v, dtype, B, H, Tq, Tk, D, qmap, kmap, causal, scale, rope_table, rope_rows,
                     row_begin, row_end, o, lse);
  if (st || (st = group_of(H, H_kv, &G))) return st;
  a.G = G;
  hipStream_t s = (hipStream_t)stream;
  return launch_status(dtype == CPATTN_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s), "block_fwd_gqa");
}

int cpattn_block_fwd_merge(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int32_t dtype,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t D,
                           const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal, float scale,
                           int64_t row_begin, int64_t row_end, const cpattn_tensor* o_acc,
                           const cpattn_tensor* lse_acc, void* stream) {
  FwdArgs a{};
  int G;
  int st = build_fwd(a, q, k, v, dtype, B, H, Tq, Tk, D, qmap, kmap, causal, scale, nullptr, 0, row_begin, row_end,
                     o_acc, lse_acc);
  if (st || (st = group_of(H, H_kv, &G))) return st;
  if (dtype != CPATTN_BF16) return fail(CPATTN_EUNSUPPORTED, "block_fwd_merge takes bf16 inputs");
  a.G = G;
  a.merge = 1;
  return launch_status(launch_fwd_bf16(a, (hipStream_t)stream), "block_fwd_merge");
}

int cpattn_block_fwd_rotq(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int32_t dtype,
                          int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t D,
                          const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal, float scale,
                          const float* rope_table, int64_t rope_rows, int64_t row_begin, int64_t row_end,
                          int32_t merge, const cpattn_tensor* o, const cpattn_tensor* lse, void* stream) {
  FwdArgs a{};
  int G;
  if (!rope_table) return fail(CPATTN_EINVAL, "rope table is NULL");
  int st = build_fwd(a, q, k, v, dtype, B, H, Tq, Tk, D, qmap, kmap, causal, scale, rope_table, rope_rows,
                     row_begin, row_end, o, lse);
  if (st || (st = group_of(H, H_kv, &G))) return st;
  if (merge != 0 && merge != 1) return fail(CPATTN_EINVAL, "merge must be 0 or 1");
  a.G = G;
  a.rope_q = 1;
  a.merge = merge;
  return launch_status(launch_fwd_bf16(a, (hipStream_t)stream), "block_fwd_rotq");
}

int cpattn_lse_merge(const cpattn_tensor* o_acc, const cpattn_tensor* lse_acc, const cpattn_tensor* o_blk,
                     const cpattn_tensor* lse_blk, int64_t B, int64_t H, int64_t T, int64_t D, int64_t row_begin,
                     int64_t row_end, void* stream) {
  int st;
  if (B <= 0 || H <= 0 || T <= 0 || D <= 0) return fail(CPATTN_EINVAL, "B, H, T, D must be positive");
  if (B * H > kIntMax || T > kIntMax) return fail(CPATTN_EINVAL, "sizes exceed 2^31");
  if (D != 64 && D != 128) return fail(CPATTN_EUNSUPPORTED, "D = %lld (supported: 64, 128)", (long long)D);
  if ((st = check_tensor(o_acc, "o_acc", 4)) || (st = check_tensor(o_blk, "o_blk", 4)) ||
      (st = check_rows(lse_acc, "lse_acc")) || (st = check_rows(lse_blk, "lse_blk")))
    return st;
  if (row_begin < 0 || row_end > T || row_begin >= row_end) return fail(CPATTN_EINVAL, "row range");
  MergeArgs m{};
  m.o_acc = (float*)o_acc->data, m.oa_sb = o_acc->sb, m.oa_sh = o_acc->sh, m.oa_st = o_acc->st;
  m.l_acc = (float*)lse_acc->data, m.la_sb = lse_acc->sb, m.la_sh = lse_acc->sh, m.la_st = lse_acc->st;
  m.o_blk = (const float*)o_blk->data, m.ob_sb = o_blk->sb, m.ob_sh = o_blk->sh, m.ob_st = o_blk->st;
  m.l_blk = (const float*)lse_blk->data, m.lb_sb = lse_blk->sb, m.lb_sh = lse_blk->sh, m.lb_st = lse_blk->st;
  m.B = (int)B, m.H = (int)H, m.D = (int)D;
  m.row_begin = (int)row_begin, m.row_end = (int)row_end;
  return launch_status(launch_merge(m, (hipStream_t)stream), "lse_merge");
}

int cpattn_step_rows(const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal, int64_t* row_begin,
                     int64_t* visible_keys) {
  if (!qmap || !kmap || !row_begin || !visible_keys) return fail(CPATTN_EINVAL, "null argument");
  int st;
  if (qmap->len <= 0 || kmap->len <= 0) return fail(CPATTN_EINVAL, "maps must be non-empty");
  if ((st = check_map(qmap, qmap->len, "qmap")) || (st = check_map(kmap, kmap->len, "kmap"))) return st;
  if (!causal) {
    *row_begin = 0;
    *visible_keys = kmap->len;
    return ok();
  }
  const PosMap qm = to_map(qmap), km = to_map(kmap);
  // rows whose position is below the block's first key position see nothing
  *row_begin = qm.count_lt(km.pos(0));
  *visible_keys = *row_begin < qmap->len ? km.count_le(qm.pos((int)qmap->len - 1)) : 0;
  return ok();
}

// Workspace layout: [fp32 block O][fp32 block LSE] and, with a rotary table, the
// rotated K block in bf16; every part 256-byte aligned.
static size_t ws_part(size_t b) { return (b + 255) / 256 * 256; }

size_t cpattn_ring_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t rope) {
  if (B <= 0 || H <= 0 || Tq <= 0 || Tk <= 0 || D <= 0) return 0;
  size_t n = ws_part((size_t)B * H * Tq * D * 4) + ws_part((size_t)B * H * Tq * 4);
  if (rope) n += ws_part((size_t)B * H * Tk * D * 2);
  return n;
}

int cpattn_ring_fwd(const cpattn_tensor* q, const cpattn_tensor* k_blocks, const cpattn_tensor* v_blocks,
                    const cpattn_posmap* kmaps, int32_t ring, int32_t rank, const cpattn_posmap* qmap,
                    int32_t dtype, int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t causal,
                    float scale, const float* rope_table, int64_t rope_rows, const cpattn_tensor* o_acc,
                    const cpattn_tensor* lse_acc, void* workspace, size_t workspace_bytes, void* stream) {
  if (ring < 1) return fail(CPATTN_EINVAL, "ring must be >= 1");
  if (rank < 0 || rank >= ring) return fail(CPATTN_EINVAL, "rank outside [0, ring)");
  if (!k_blocks || !v_blocks || !kmaps) return fail(CPATTN_EINVAL, "null block arrays");
  // validate every step before launching anything
  int st;
  for (int32_t i = 0; i < ring; ++i) {
    FwdArgs a{};
    if ((st = build_fwd(a, q, &k_blocks[i], &v_blocks[i], dtype, B, H, Tq, Tk, D, qmap, &kmaps[i], causal, scale,
                        rope_table, rope_rows, 0, Tq, o_acc, lse_acc)))
      return st;
  }
  // With a rotary table and bf16 inputs, each K block is rotated once per step into the
  // workspace (every key rotated once instead of once per query tile) and the block kernel
  // rotates the Q rows as it loads them into registers.
  const bool pre = rope_table != nullptr && dtype == CPATTN_BF16;
  const size_t need = cpattn_ring_fwd_workspace_bytes(B, H, Tq, Tk, D, pre ? 1 : 0);
  // bf16 steps merge in the block kernel's epilogue: only fp32 rings and rotary use the workspace
  if ((ring > 1 && dtype != CPATTN_BF16) || pre) {
    if (!workspace || workspace_bytes < need)
      return fail(CPATTN_EINVAL, "workspace of %zu bytes needed", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(CPATTN_EINVAL, "workspace not 256-byte aligned");
  }
  char* wp = (char*)workspace;
  float* o_ws = (float*)wp;
  float* l_ws = (float*)(wp + ws_part((size_t)B * H * Tq * D * 4));
  __bf16* k_rot = (__bf16*)(wp + ws_part((size_t)B * H * Tq * D * 4) + ws_part((size_t)B * H * Tq * 4));
  cpattn_tensor o_blk{o_ws, H * Tq * D, Tq * D, D};
  cpattn_tensor l_blk{l_ws, H * Tq, Tq, 1};
  const cpattn_tensor k_r{k_rot, H * Tk * D, Tk * D, D};
  hipStream_t s = (hipStream_t)stream;
  const float* blk_rope = pre ? nullptr : rope_table;
  // the rotation of Q on load, for the block launches of a pre-rotated ring
  auto rotate_q = [&](FwdArgs& a) {
    if (pre) a.rope = rope_table, a.rope_rows = (int)rope_rows, a.rope_q = 1;
  };
  // the K block a step uses: rotated into the workspace first when pre-rotating
  auto key_block = [&](int32_t src) -> const cpattn_tensor* {
    if (!pre) return &k_blocks[src];
    if (cpattn_rope_rotate(&k_blocks[src], dtype, B, H, Tk, D, &kmaps[src], rope_table, rope_rows, &k_r, stream))
      return nullptr;
    return &k_r;
  };
  for (int32_t step = 0; step < ring; ++step) {
    const int32_t src = ((rank - step) % ring + ring) % ring;
    const cpattn_posmap* km = &kmaps[src];
    int64_t rb = 0, nvis = 0;
    if ((st = cpattn_step_rows(qmap, km, causal, &rb, &nvis))) return st;
    if (step == 0) {
      // step 0 fills every row of the accumulator (rows without a visible key get O = 0, LSE = -inf)
      const cpattn_tensor* kb = key_block(src);
      if (!kb) return CPATTN_EHIP;
      FwdArgs a{};
      build_fwd(a, q, kb, &v_blocks[src], dtype, B, H, Tq, Tk, D, qmap, km, causal, scale, blk_rope, rope_rows, 0, Tq,
                o_acc, lse_acc);
      rotate_q(a);
      hipError_t e = dtype == CPATTN_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s);
      if (e != hipSuccess) return launch_status(e, "ring_fwd step 0");
      continue;
    }
    if (rb >= Tq) continue;  // the whole block is in the future of every local row
    const cpattn_tensor* kb = key_block(src);
    if (!kb) return CPATTN_EHIP;
    if (dtype == CPATTN_BF16 && blk_rope == nullptr) {
      // bf16 without per-tile rotary: the block kernel merges its rows into the accumulator
      // in its epilogue (no block output in the workspace, no merge launch)
      FwdArgs a{};
      build_fwd(a, q, kb, &v_blocks[src], dtype, B, H, Tq, Tk, D, qmap, km, causal, scale, nullptr, 0, rb, Tq,
                o_acc, lse_acc);
      rotate_q(a);
      a.merge = 1;
      hipError_t e = launch_fwd_bf16(a, s);
      if (e != hipSuccess) return launch_status(e, "ring_fwd block merge");
      continue;
    }
    FwdArgs a{};
    build_fwd(a, q, kb, &v_blocks[src], dtype, B, H, Tq, Tk, D, qmap, km, causal, scale, blk_rope, rope_rows, rb, Tq,
              &o_blk, &l_blk);
    hipError_t e = dtype == CPATTN_BF16 ? launch_fwd_bf16(a, s) : launch_fwd_f32(a, s);
    if (e != hipSuccess) return launch_status(e, "ring_fwd block");
    MergeArgs m{};
    m.o_acc = (float*)o_acc->data, m.oa_sb = o_acc->sb, m.oa_sh = o_acc->sh, m.oa_st = o_acc->st;
    m.l_acc = (float*)lse_acc->data, m.la_sb = lse_acc->sb, m.la_sh = lse_acc->sh, m.la_st = lse_acc->st;
    m.o_blk = o_ws, m.ob_sb = o_blk.sb, m.ob_sh = o_blk.sh, m.ob_st = o_blk.st;
    m.l_blk = l_ws, m.lb_sb = l_blk.sb, m.lb_sh = l_blk.sh, m.lb_st = l_blk.st;
    m.B = (int)B, m.H = (int)H, m.D = (int)D;
    m.row_begin = (int)rb, m.row_end = (int)Tq;
    e = launch_merge(m, s);
    if (e != hipSuccess) return launch_status(e, "ring_fwd merge");
  }
  return ok();
}

int cpattn_bwd_preprocess(const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* o,
                          const cpattn_tensor* delta, int64_t B, int64_t H, int64_t Tq, int64_t D, void* stream) {
  int st;
  if ((st = check_dims(B, H, Tq, 1, D))) return st;
  if (dtype != CPATTN_F32 && dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "dtype %d", (int)dtype);
  if ((st = check_tensor(dout, "dout", dtype == CPATTN_BF16 ? 2 : 4)) || (st = check_tensor(o, "o", 4)) ||
      (st = check_rows(delta, "delta")))
    return st;
  PreArgs p{};
  p.dout = view(dout);
  p.bf16 = dtype == CPATTN_BF16;
  p.o = view(o);
  p.delta = (float*)delta->data, p.d_sb = delta->sb, p.d_sh = delta->sh, p.d_st = delta->st;
  p.B = (int)B, p.H = (int)H, p.Tq = (int)Tq, p.D = (int)D;
  return launch_status(launch_bwd_preprocess(p, (hipStream_t)stream), "bwd_preprocess");
}

}  // extern "C"

namespace {

// Checks one block backward's arguments and fills its launch arguments; launches nothing.
// acc_q / acc_kv: 1 adds into dQ / dK and dV, 0 overwrites them.
int build_bwd(BwdArgs& a, const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
              const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse, const cpattn_tensor* delta,
              const cpattn_tensor* dq_acc, const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc, int64_t B,
              int64_t H, int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap,
              int32_t causal, float scale, int32_t acc_q, int32_t acc_kv, int which, int64_t H_kv) {
  int st, G;
  if ((st = check_dims(B, H, Tq, Tk, D))) return st;
  if ((st = group_of(H, H_kv, &G))) return st;
  if (dtype == CPATTN_F32) return fail(CPATTN_EUNSUPPORTED, "block backward takes bf16 inputs");
  if (dtype != CPATTN_BF16) return fail(CPATTN_EINVAL, "dtype %d", (int)dtype);
  if ((st = check_tensor(q, "q", 2)) || (st = check_tensor(k, "k", 2)) || (st = check_tensor(v, "v", 2)) ||
      (st = check_tensor(dout, "dout", 2)) || (st = check_rows(lse, "lse")) || (st = check_rows(delta, "delta")))
    return st;
  if ((which & 2) && (st = check_tensor(dq_acc, "dq_acc", 4))) return st;
  if ((which & 1) && ((st = check_tensor(dk_acc, "dk_acc", 4)) || (st = check_tensor(dv_acc, "dv_acc", 4))))
    return st;
  // accumulator rows must not overlap (the dK/dV epilogue bounds a wave's rows by its last key)
  if (((which & 2) && dq_acc->st < D) || ((which & 1) && (dk_acc->st < D || dv_acc->st < D)))
    return fail(CPATTN_EINVAL, "accumulator T stride below D (rows overlap)");
  if ((st = check_map(qmap, Tq, "qmap")) || (st = check_map(kmap, Tk, "kmap"))) return st;
  if (!(scale >= 0.f) || std::isinf(scale)) return fail(CPATTN_EINVAL, "scale must be finite and >= 0");
  if (acc_q != 0 && acc_q != 1) return fail(CPATTN_EINVAL, "accumulate must be 0 or 1");
  if (acc_kv != 0 && acc_kv != 1) return fail(CPATTN_EINVAL, "accumulate must be 0 or 1");
  a = BwdArgs{};
  a.q = view(q), a.k = view(k), a.v = view(v), a.dout = view(dout);
  a.lse = view(lse), a.delta = view(delta);
  if (which & 2) a.dq = (float*)dq_acc->data, a.dq_sb = dq_acc->sb, a.dq_sh = dq_acc->sh, a.dq_st = dq_acc->st;
  if (which & 1) {
    a.dk = (float*)dk_acc->data, a.dk_sb = dk_acc->sb, a.dk_sh = dk_acc->sh, a.dk_st = dk_acc->st;
    a.dv = (float*)dv_acc->data, a.dv_sb = dv_acc->sb, a.dv_sh = dv_acc->sh, a.dv_st = dv_acc->st;
  }
  a.B = (int)B, a.H = (int)H, a.Tq = (int)Tq, a.Tk = (int)Tk, a.D = (int)D;
  a.qm = to_map(qmap), a.km = to_map(kmap);
  a.causal = causal != 0;
  a.scale = scale == 0.f ? (float)(1.0 / std::sqrt((double)D)) : scale;
  a.G = G;
  a.acc_q = acc_q;
  a.acc_kv = acc_kv;
  return ok();
}

int bwd_common(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, const cpattn_tensor* dout,
               int32_t dtype, const cpattn_tensor* lse, const cpattn_tensor* delta, const cpattn_tensor* dq_acc,
               const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc, int64_t B, int64_t H, int64_t Tq,
               int64_t Tk, int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
               float scale, int32_t accumulate, int which, void* stream, const char* what, int64_t H_kv) {
  BwdArgs a;
  int st = build_bwd(a, q, k, v, dout, dtype, lse, delta, dq_acc, dk_acc, dv_acc, B, H, Tq, Tk, D, qmap, kmap,
                     causal, scale, accumulate, accumulate, which, H_kv);
  if (st) return st;
  return launch_status(launch_bwd_bf16(a, which, (hipStream_t)stream), what);
}

}  // namespace

extern "C" {

int cpattn_block_bwd_gqa(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                         const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                         const cpattn_tensor* delta, const cpattn_tensor* dq_acc, const cpattn_tensor* dk_acc,
                         const cpattn_tensor* dv_acc, int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                         int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                         float scale, int32_t accumulate, void* stream) {
  return bwd_common(q, k, v, dout, dtype, lse, delta, dq_acc, dk_acc, dv_acc, B, H, Tq, Tk, D, qmap, kmap, causal,
                    scale, accumulate, 3, stream, "block_bwd_gqa", H_kv);
}

int cpattn_block_bwd(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                     const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse, const cpattn_tensor* delta,
                     const cpattn_tensor* dq_acc, const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc, int64_t B,
                     int64_t H, int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap,
                     const cpattn_posmap* kmap, int32_t causal, float scale, int32_t accumulate,
                     void* stream) {
  return bwd_common(q, k, v, dout, dtype, lse, delta, dq_acc, dk_acc, dv_acc, B, H, Tq, Tk, D, qmap, kmap, causal,
                    scale, accumulate, 3, stream, "block_bwd", H);
}

int cpattn_block_bwd_dkdv(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                          const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                          const cpattn_tensor* delta, const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc,
                          int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap,
                          const cpattn_posmap* kmap, int32_t causal, float scale, int32_t accumulate,
                          void* stream) {
  return bwd_common(q, k, v, dout, dtype, lse, delta, nullptr, dk_acc, dv_acc, B, H, Tq, Tk, D, qmap, kmap, causal,
                    scale, accumulate, 1, stream, "block_bwd_dkdv", H);
}

int cpattn_block_bwd_dq(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                        const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse, const cpattn_tensor* delta,
                        const cpattn_tensor* dq_acc, int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D,
                        const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal, float scale,
                        int32_t accumulate, void* stream) {
  return bwd_common(q, k, v, dout, dtype, lse, delta, dq_acc, nullptr, nullptr, B, H, Tq, Tk, D, qmap, kmap, causal,
                    scale, accumulate, 2, stream, "block_bwd_dq", H);
}

// Staging area of the dS blocks: one 2 KB block (32 query rows x 32 keys, bf16) per (b, query
// head, 32-row block, 32-key block); 128-wide heads only.
size_t cpattn_block_bwd_staged_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D) {
  if (B <= 0 || H <= 0 || Tq <= 0 || Tk <= 0 || D != 128) return 0;
  return ws_part((size_t)B * H * (size_t)((Tq + 31) / 32) * (size_t)((Tk + 31) / 32) * 2048);
}

int cpattn_block_bwd_staged(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                            const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                            const cpattn_tensor* delta, const cpattn_tensor* dq_acc, const cpattn_tensor* dk_acc,
                            const cpattn_tensor* dv_acc, int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                            int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                            float scale, int32_t accumulate, void* workspace, size_t workspace_bytes,
                            void* stream) {
  BwdArgs a;
  int st = build_bwd(a, q, k, v, dout, dtype, lse, delta, dq_acc, dk_acc, dv_acc, B, H, Tq, Tk, D, qmap, kmap,
                     causal, scale, accumulate, accumulate, 3, H_kv);
  if (st) return st;
  const size_t need = cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D);
  if (need) {
    if (!workspace || workspace_bytes < need) return fail(CPATTN_EINVAL, "workspace of %zu bytes needed", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(CPATTN_EINVAL, "workspace not 256-byte aligned");
    a.ds = workspace;
    a.nqb = (int)((Tq + 31) / 32);
    a.nkb = (int)((Tk + 31) / 32);
  }
  return launch_status(launch_bwd_bf16(a, 3, (hipStream_t)stream), "block_bwd_staged");
}

// Workspace layout: [fp32 delta, B x H x Tq], 256-byte aligned.
size_t cpattn_ring_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Tq) {
  if (B <= 0 || H <= 0 || Tq <= 0) return 0;
  return ws_part((size_t)B * H * Tq * 4);
}

// [fp32 delta | dS staging area of the largest block], both 256-byte aligned.
size_t cpattn_ring_bwd_staged_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D) {
  return cpattn_ring_bwd_workspace_bytes(B, H, Tq) + cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D);
}

int cpattn_ring_bwd(const cpattn_tensor* q, const cpattn_tensor* k_blocks, const cpattn_tensor* v_blocks,
                    const cpattn_posmap* kmaps, int32_t ring, int32_t rank, const cpattn_posmap* qmap,
                    int32_t dtype, int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t causal,
                    float scale, const cpattn_tensor* dout, const cpattn_tensor* o, const cpattn_tensor* lse,
                    const cpattn_tensor* dq_acc, const cpattn_tensor* dk_blocks, const cpattn_tensor* dv_blocks,
                    int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  if (ring < 1) return fail(CPATTN_EINVAL, "ring must be >= 1");
  if (rank < 0 || rank >= ring) return fail(CPATTN_EINVAL, "rank outside [0, ring)");
  if (!k_blocks || !v_blocks || !kmaps || !dk_blocks || !dv_blocks) return fail(CPATTN_EINVAL, "null block arrays");
  int st;
  if ((st = check_dims(B, H, Tq, Tk, D))) return st;
  if ((st = check_tensor(o, "o", 4))) return st;
  const size_t need = cpattn_ring_bwd_workspace_bytes(B, H, Tq);
  if (!workspace || workspace_bytes < need) return fail(CPATTN_EINVAL, "workspace of %zu bytes needed", need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(CPATTN_EINVAL, "workspace not 256-byte aligned");
  const cpattn_tensor delta{workspace, H * Tq, Tq, 1};
  // room for the dS staging area after delta: dQ reuses the dK/dV kernel's dS
  const size_t stage = cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D);
  void* ds = stage && workspace_bytes - need >= stage ? (void*)((char*)workspace + need) : nullptr;
  // validate every step before launching anything
  for (int32_t i = 0; i < ring; ++i) {
    BwdArgs a;
    if ((st = build_bwd(a, q, &k_blocks[i], &v_blocks[i], dout, dtype, lse, &delta, dq_acc, &dk_blocks[i],
                        &dv_blocks[i], B, H, Tq, Tk, D, qmap, &kmaps[i], causal, scale, 1, accumulate, 3, H)))
      return st;
  }
  if ((st = cpattn_bwd_preprocess(dout, dtype, o, &delta, B, H, Tq, D, stream))) return st;
  hipStream_t s = (hipStream_t)stream;
  for (int32_t step = 0; step < ring; ++step) {
    const int32_t src = ((rank - step) % ring + ring) % ring;
    int64_t rb = 0, nvis = 0;
    if ((st = cpattn_step_rows(qmap, &kmaps[src], causal, &rb, &nvis))) return st;
    // dQ takes every step's contribution: only the first step may overwrite it
    const int32_t acc_q = (accumulate || step > 0) ? 1 : 0;
    // no local row sees this block and nothing has to be overwritten: no work
    if (rb >= Tq && acc_q && accumulate) continue;
    BwdArgs a;
    build_bwd(a, q, &k_blocks[src], &v_blocks[src], dout, dtype, lse, &delta, dq_acc, &dk_blocks[src],
              &dv_blocks[src], B, H, Tq, Tk, D, qmap, &kmaps[src], causal, scale, acc_q, accumulate, 3, H);
    if (ds) a.ds = ds, a.nqb = (int)((Tq + 31) / 32), a.nkb = (int)((Tk + 31) / 32);
    hipError_t e = launch_bwd_bf16(a, 3, s);
    if (e != hipSuccess) return launch_status(e, "ring_bwd block");
  }
  return ok();
}

}  // extern "C"
