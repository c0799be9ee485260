/*
 * libcpattn -- one rank's share of causal ring attention under HeadTail
 * load-balanced context parallelism, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the pages on context parallelism (BluScriptCP
 * development log):
 *   - HeadTail shard map: entries of 2026-05-16 (chunk-level HeadTail) and
 *     2026-06-29 / 2026-07-10 (RopeDeltas.h: local index -> global position
 *     through a head delta and a tail delta);
 *   - block attention with separate query/key lengths, global positions for
 *     the causal mask, and the log-sum-exp as an output: entries of
 *     2026-04-20 and 2026-06-29 (kernel requirements);
 *   - the SDPAMerger log-sum-exp merge: entries of 2026-03-20 and 2026-05-20
 *     (merge of a row range);
 *   - the ring forward: entry of 2026-03-20 (ring rotator, per-step SDPA,
 *     merger); the per-block backward with gradients accumulated across ring
 *     steps: entries of 2026-04-20 and 2026-05-07;
 *   - strided Q/K/V/dO/O/LSE/dQ/dK/dV: entry of 2026-04-28;
 *   - rotary embedding at global positions: entries of 2026-06-29 and
 *     2026-07-10.
 *
 * Conventions shared by every call
 *   - Tensors are described by cpattn_tensor: a pointer to element [0,0,0,0]
 *     and element strides for the B, H and T dimensions. The D dimension is
 *     contiguous (stride 1). LSE/delta arrays are [B,H,T] and use sb, sh, st.
 *     Pointers must be aligned to 16 bytes and the B/H/T strides of bf16
 *     tensors must be multiples of 8 elements (of fp32 tensors, multiples of 4).
 *   - Device pointers are HIP device memory owned by the caller. The library
 *     allocates nothing, keeps no device state and never synchronises: every
 *     kernel is launched on the hipStream_t passed as `stream` (NULL = the
 *     default stream). Host arrays are read during the call only.
 *   - Global positions: a cpattn_posmap maps local index i in [0, len) to
 *     global position i + (i < split ? d0 : d1), with 0 <= split <= len and
 *     d1 >= d0 (positions increase with the local index). A contiguous shard
 *     is split = len, d0 = first global position.
 *   - Causal visibility: key j is visible from query p iff
 *     pos_k(j) <= pos_q(p) (self included). causal = 0 makes every key visible.
 *   - The softmax scale is `scale`; pass 0 for 1/sqrt(D).
 *   - LSE is the natural-log log-sum-exp of the scaled scores of the visible
 *     keys. A row with no visible key gets O = 0 and LSE = -inf.
 *   - Return value: CPATTN_OK, or a negative code; cpattn_last_error() then
 *     returns a message (thread-local). Arguments are validated before any
 *     launch; on error nothing is launched. Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - The library sees pointers and strides, not allocations: the caller
 *     guarantees that every tensor holds the elements its sizes and strides
 *     address, in the dtype the call states (inputs in `dtype`, outputs and
 *     accumulators fp32). The Python binding checks each tensor's shape,
 *     dtype and device against these before it calls in.
 *   - Stateless and thread-safe; concurrent calls on different streams must
 *     not write the same memory.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_ABI_VERSION 8

enum {
  CPATTN_OK = 0,
  CPATTN_EINVAL = -1,      /* invalid argument (null pointer, bad shape or stride, bad map) */
  CPATTN_EUNSUPPORTED = -2, /* valid but not implemented (e.g. D not 64 or 128) */
  CPATTN_EHIP = -3          /* a HIP launch failed */
};

enum { CPATTN_F32 = 0, CPATTN_BF16 = 1 };

typedef struct {
  int64_t len, split, d0, d1;
} cpattn_posmap;

typedef struct {
  void* data;
  int64_t sb, sh, st;
} cpattn_tensor;

/* ABI version (CPATTN_ABI_VERSION). */
int cpattn_version(void);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* cpattn_last_error(void);

/*
 * HeadTail shard map (host only, integer, exact).
 * The global sequence of T tokens is cut into 2*ring chunks of c = T/(2*ring)
 * tokens; rank r holds chunk r followed by chunk 2*ring-1-r (BluScriptCP log,
 * 2026-05-16 and 2026-06-29: Megatron's chunk pair [r, 2cp-1-r]; the worked
 * example with two ranks and eight tokens gives rank 0 positions 0, 1, 6, 7).
 *   map        out: len = 2c, split = c, d0 = r*c, d1 = (2*ring-2-r)*c
 *   positions  out, nullable: host int32 array of 2c global positions
 * Errors: EINVAL if T <= 0, ring <= 0, T % (2*ring) != 0, rank outside
 * [0, ring), T >= 2^31, or map is NULL.
 */
int cpattn_headtail_shard(int64_t T, int32_t ring, int32_t rank,
                          cpattn_posmap* map, int32_t* positions);

/*
 * Rotary table: table[p][i] = (cos a, sin a), a = p * theta^(-2i/D), for
 * p in [0, rows), i in [0, D/2); fp32 values of angles computed in fp64 on
 * the device. table is a device array of rows*D floats (interleaved pairs).
 * Reading of the rotary form used with it: dimension i pairs with i + D/2
 * (half-split), as in the Llama-style fused rotary of the BluScriptCP log
 * (2026-07-02), at global positions (2026-06-29).
 * Errors: EINVAL if theta <= 0, rows <= 0, D odd or <= 0, table NULL.
 */
int cpattn_rope_table(double theta, int64_t rows, int64_t D, float* table, void* stream);

/*
 * Rotary embedding applied once: out = x with every row i of every (b, h)
 * rotated by the table row of its global position map(i), half-split pairs
 * (i, i + D/2), fp32 arithmetic, bf16 result rounded to nearest even - the
 * rotation the fused path of cpattn_block_fwd applies to q and k rows. A block
 * rotated this way at its owner's positions can travel the ring as is, and the
 * rotation is paid once per key instead of once per query tile.
 *   x, out      [B,H,T,D] bf16; out may be x itself (in place)
 *   rope_table  device table of cpattn_rope_table, rope_rows rows
 * Errors: EINVAL for null or misaligned tensors or table, a map whose len
 * differs from T, positions outside the table; EUNSUPPORTED for fp32 or D not
 * in {64, 128}.
 */
int cpattn_rope_rotate(const cpattn_tensor* x, int32_t dtype, int64_t B, int64_t H, int64_t T,
                       int64_t D, const cpattn_posmap* map, const float* rope_table,
                       int64_t rope_rows, const cpattn_tensor* out, void* stream);

/*
 * Backward through the rotary embedding, in place: every row i of the fp32
 * gradient g [B,H,T,D] with respect to ROTATED rows becomes the gradient with
 * respect to the unrotated rows, R(p)^T g with p = map(i) (the rotation by the
 * negated angle; each pair rotation is orthogonal). The rotation is linear, so
 * a caller that ran the block backward on rotated q and k applies it once to
 * the accumulated dQ and to each accumulated dK block after the last ring step.
 * Errors: EINVAL for a null or misaligned g or table, a map whose len differs
 * from T, positions outside the table; EUNSUPPORTED for D not in {64, 128}.
 */
int cpattn_rope_rotate_grad(const cpattn_tensor* g, int64_t B, int64_t H, int64_t T, int64_t D,
                            const cpattn_posmap* map, const float* rope_table, int64_t rope_rows,
                            void* stream);

/*
 * Block forward: attention of local query rows [row_begin, row_end) of q
 * ([B,H,Tq,D]) against one KV block k, v ([B,H,Tk,D]) at global positions
 * qmap/kmap. Writes fp32 o [B,H,Tq,D] and lse [B,H,Tq] for those rows only.
 *   dtype       CPATTN_BF16 (bf16 inputs, MFMA with fp32 accumulation) or
 *               CPATTN_F32 (fp32 inputs and arithmetic); q, k, v share it
 *   rope_table  nullable: if set (bf16 only), q and k rows are rotated by the
 *               table row of their global position before the products;
 *               rope_rows = rows in the table, every position must be below it
 * Errors: EINVAL for null tensors, D stride assumptions broken, a map whose
 * len differs from Tq/Tk or with d1 < d0, an empty or out-of-range row range,
 * positions outside the rotary table; EUNSUPPORTED for D not in {64, 128} or
 * a rotary table with fp32 inputs.
 */
int cpattn_block_fwd(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                     int32_t dtype, int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D,
                     const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                     float scale, const float* rope_table, int64_t rope_rows,
                     int64_t row_begin, int64_t row_end,
                     const cpattn_tensor* o, const cpattn_tensor* lse, void* stream);

/*
 * Grouped-query form of cpattn_block_fwd (GQA; MQA when H_kv = 1): q, o and
 * lse have H heads, k and v H_kv heads, and query head h attends with KV head
 * h / (H / H_kv) - the grouping of the BluScriptCP log (2026-07-06: query head
 * hq uses KV head hq / G; 2026-06-29: the ring keeps the KV heads grouped, so
 * blocks travel with H_kv heads only). Every other argument as in
 * cpattn_block_fwd, which is this call with H_kv = H.
 * Errors: as cpattn_block_fwd, plus EINVAL if H is not a multiple of H_kv.
 */
int cpattn_block_fwd_gqa(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                         int32_t dtype, int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                         int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                         float scale, const float* rope_table, int64_t rope_rows,
                         int64_t row_begin, int64_t row_end,
                         const cpattn_tensor* o, const cpattn_tensor* lse, void* stream);

/*
 * SDPAMerger: for rows [row_begin, row_end) of every (b, h), fold the block
 * result (o_blk, lse_blk) into the running result (o_acc, lse_acc), in place:
 *   L = log(exp(L_acc) + exp(L_blk)),
 *   O = exp(L_acc - L) O_acc + exp(L_blk - L) O_blk.
 * A side with LSE = -inf is the identity; both -inf give (0, -inf).
 * All four tensors are fp32: o_* [B,H,T,D], lse_* [B,H,T].
 * Errors: EINVAL for null tensors or a bad row range; EUNSUPPORTED if D % 4.
 */
int cpattn_lse_merge(const cpattn_tensor* o_acc, const cpattn_tensor* lse_acc,
                     const cpattn_tensor* o_blk, const cpattn_tensor* lse_blk,
                     int64_t B, int64_t H, int64_t T, int64_t D,
                     int64_t row_begin, int64_t row_end, void* stream);

/*
 * Block forward fused with the log-sum-exp merge: the result of
 * cpattn_block_fwd_gqa on rows [row_begin, row_end) (H_kv = H for multi-head)
 * is folded into the running fp32 (o_acc, lse_acc) in the kernel's epilogue,
 * with the arithmetic of cpattn_lse_merge (SDPAMerger of the BluScriptCP log,
 * 2026-03-20; partial-row merge, 2026-05-20), instead of being written out
 * and merged by a second launch. Same result as cpattn_block_fwd into a
 * scratch pair followed by cpattn_lse_merge, up to rounding order; it moves
 * about half the bytes (no block output is written and read back) and saves
 * one launch per ring step. Rows outside the range are untouched. A row that
 * sees no key of this block and none before keeps O = 0, LSE = -inf.
 * bf16 inputs only, no rotary table (pass rotated Q and K: cpattn_rope_rotate).
 * Errors: as cpattn_block_fwd_gqa; EUNSUPPORTED for fp32 inputs.
 */
int cpattn_block_fwd_merge(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                           int32_t dtype, int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                           int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap,
                           int32_t causal, float scale, int64_t row_begin, int64_t row_end,
                           const cpattn_tensor* o_acc, const cpattn_tensor* lse_acc, void* stream);

/*
 * Block forward (merge = 0, as cpattn_block_fwd_gqa into o, lse) or block
 * forward fused with the merge (merge = 1, as cpattn_block_fwd_merge into the
 * running o, lse) whose Q rows are rotated at their global positions (qmap)
 * with the rotary table as the kernel loads them into registers; k arrives
 * already rotated, as its owner rotates a block once and sends it (BluScriptCP
 * log, 2026-06-29 and 2026-07-10: rotary at global positions). The rotation is
 * that of cpattn_rope_rotate, so the results equal cpattn_rope_rotate of q
 * followed by the plain call bit for bit, without the pass over Q in HBM.
 * bf16 inputs only; the table as in cpattn_block_fwd (it must cover every
 * position of both maps).
 * Errors: as cpattn_block_fwd_gqa (merge = 0) or cpattn_block_fwd_merge
 * (merge = 1); EINVAL for a NULL table or merge outside {0, 1}; EUNSUPPORTED
 * for fp32 inputs.
 */
int cpattn_block_fwd_rotq(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                          int32_t dtype, int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                          int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap,
                          int32_t causal, float scale, const float* rope_table, int64_t rope_rows,
                          int64_t row_begin, int64_t row_end, int32_t merge, const cpattn_tensor* o,
                          const cpattn_tensor* lse, void* stream);

/*
 * Step classification (host only, integer, exact): the local query rows that
 * see at least one key of a KV block. Positions increase with the local
 * index, so they form the suffix [*row_begin, qmap->len); *visible_keys is the
 * number of keys any of them can see (a prefix of the block). With causal = 0
 * every row sees every key. Under HeadTail this yields the three step shapes
 * of the BluScriptCP log (2026-06-17): the causal diagonal for the own block,
 * all rows against the head half of the keys for an earlier rank's block, and
 * the tail half of the rows against all keys for a later rank's block.
 * A caller that receives blocks one at a time (a real ring) drives each step
 * with cpattn_block_fwd on rows [*row_begin, len) and cpattn_lse_merge, which
 * is what cpattn_ring_fwd does with resident blocks.
 * Errors: EINVAL for null pointers or an invalid map.
 */
int cpattn_step_rows(const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                     int64_t* row_begin, int64_t* visible_keys);

/*
 * Workspace bytes cpattn_ring_fwd needs: an fp32 block output and LSE, and
 * with rope != 0 (a rotary table with bf16 inputs) room for one rotated K
 * block. 0 for non-positive sizes.
 */
size_t cpattn_ring_fwd_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D,
                                       int32_t rope);

/*
 * Ring forward of rank `rank` out of `ring`, all KV blocks resident in HBM.
 * k_blocks[i], v_blocks[i], kmaps[i] describe the block owned by rank i
 * (each [B,H,Tk,D]). At step s the rank holds the block of owner
 * (rank - s) mod ring (blocks travel to the next rank each step). Step 0
 * writes (o_acc, lse_acc) directly; every later step runs the block forward
 * on the rows that see at least one key of that block and merges those rows:
 * with bf16 inputs in the block kernel's epilogue (cpattn_block_fwd_merge, one
 * launch), with fp32 inputs into the workspace and then by cpattn_lse_merge.
 * Steps whose block is invisible to every row are skipped. At most two
 * launches per step, no synchronisation. With a rotary
 * table and bf16 inputs, each step first rotates its K block into the
 * workspace (cpattn_rope_rotate, one more launch per step), then runs the block
 * with its Q rows rotated as they are loaded (cpattn_block_fwd_rotq).
 * workspace: device memory of cpattn_ring_fwd_workspace_bytes(B,H,Tq,Tk,D,
 * rope) bytes, 256-byte aligned; used by fp32 rings (ring > 1) and by the
 * rotary form, may be NULL otherwise (bf16 without rotary, or ring == 1).
 * Other arguments as in cpattn_block_fwd.
 * Errors: as cpattn_block_fwd, plus EINVAL for ring < 1, rank out of range,
 * a short workspace.
 */
int cpattn_ring_fwd(const cpattn_tensor* q, const cpattn_tensor* k_blocks,
                    const cpattn_tensor* v_blocks, const cpattn_posmap* kmaps,
                    int32_t ring, int32_t rank, const cpattn_posmap* qmap, int32_t dtype,
                    int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t causal,
                    float scale, const float* rope_table, int64_t rope_rows,
                    const cpattn_tensor* o_acc, const cpattn_tensor* lse_acc,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward preprocess: delta[b,h,p] = sum_d dout[b,h,p,d] * o[b,h,p,d]
 * (the row term of the softmax backward; BluScriptCP log, 2026-03-24, the
 * Di correction), with o the final merged fp32 output.
 * dout has `dtype` (bf16 or fp32); o, delta fp32.
 */
int cpattn_bwd_preprocess(const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* o,
                          const cpattn_tensor* delta, int64_t B, int64_t H, int64_t Tq, int64_t D,
                          void* stream);

/*
 * Block backward of one ring step: with the FINAL merged lse and delta of the
 * local query rows, recompute P = exp(scale * q k^T - lse) over the visible
 * pairs of this block and ADD into fp32 accumulators:
 *   dv_acc += P^T dout
 *   dS      = P * (dout v^T - delta)
 *   dq_acc += scale * dS k
 *   dk_acc += scale * dS^T q
 * dq_acc is [B,H,Tq,D] (the local rows), dk_acc and dv_acc are [B,H,Tk,D]
 * (the block's rows); their T stride must be at least D (rows never overlap).
 * accumulate = 1 adds as above: the caller zeroes the accumulators once and
 * never between steps. accumulate = 0 overwrites them instead: every row is
 * written, with this block's contribution or 0 where no pair contributes, so
 * the first contribution to an accumulator needs no clearing beforehand (the
 * rank's own diagonal block, which every local row and key takes part in).
 * Other values: EINVAL. bf16 inputs only; rotary is not supported here.
 * Two halves (key-tile-major for dk/dv, query-tile-major for dq), no atomics:
 * results are bitwise reproducible and equal to calling the two halves below.
 * At D = 64 both halves share one grid, so that a small block still fills the
 * device; at D = 128 they are two launches.
 * Errors: as cpattn_block_fwd; EUNSUPPORTED for fp32 inputs.
 */
int cpattn_block_bwd(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                     const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                     const cpattn_tensor* delta, const cpattn_tensor* dq_acc,
                     const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc,
                     int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D,
                     const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                     float scale, int32_t accumulate, void* stream);

/*
 * Grouped-query form of cpattn_block_bwd: q, dout, lse, delta and dq_acc have
 * H heads; k, v, dk_acc and dv_acc have H_kv heads. Query head h reads KV head
 * h / (H / H_kv); the gradient of a KV head adds the contributions of all its
 * query heads, summed in fp32 registers by one workgroup before it is added to
 * dk_acc / dv_acc (the group reduce of the BluScriptCP log, 2026-07-01; no
 * atomics, bitwise reproducible). dQ stays per query head.
 * Errors: as cpattn_block_bwd, plus EINVAL if H is not a multiple of H_kv.
 */
int cpattn_block_bwd_gqa(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                         const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                         const cpattn_tensor* delta, const cpattn_tensor* dq_acc,
                         const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc,
                         int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t D,
                         const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                         float scale, int32_t accumulate, void* stream);

/*
 * The two halves of cpattn_block_bwd, same arguments and accumulate semantics
 * (accumulate applies to the accumulators the half writes):
 * _dkdv adds into dk_acc and dv_acc only (key-tile-major kernel), _dq adds
 * into dq_acc only (query-tile-major kernel). In a real ring the dK/dV
 * partials travel back to their owner while dQ stays local (BluScriptCP log,
 * 2026-03-21 and 2026-06-22 on the dK/dV accumulator that rotates with its
 * block), so launching _dkdv first lets that transfer overlap with _dq.
 * Arguments that a half does not use may be NULL (dq_acc for _dkdv; dk_acc
 * and dv_acc for _dq).
 */
int cpattn_block_bwd_dkdv(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                          const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                          const cpattn_tensor* delta, const cpattn_tensor* dk_acc,
                          const cpattn_tensor* dv_acc, int64_t B, int64_t H, int64_t Tq, int64_t Tk,
                          int64_t D, const cpattn_posmap* qmap, const cpattn_posmap* kmap,
                          int32_t causal, float scale, int32_t accumulate, void* stream);
int cpattn_block_bwd_dq(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                        const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                        const cpattn_tensor* delta, const cpattn_tensor* dq_acc, int64_t B, int64_t H,
                        int64_t Tq, int64_t Tk, int64_t D, const cpattn_posmap* qmap,
                        const cpattn_posmap* kmap, int32_t causal, float scale, int32_t accumulate,
                        void* stream);

/*
 * Block backward with dS staged in HBM: cpattn_block_bwd_gqa (H_kv = H: cpattn_block_bwd)
 * with the same arguments and accumulate semantics, for callers that can lend a workspace.
 * At D = 128 the dK/dV kernel writes every visible block of dS = P * (dout v^T - delta)
 * (bf16, the value its dK product uses) into the workspace, and the dQ kernel forms
 * dq_acc += scale * dS k from those blocks instead of forming P and dS a second time: each
 * of S, dP, dV, dK and dQ is computed once (the FA2 count of 10 D flops per visible pair,
 * against 14 D for cpattn_block_bwd), for 4 bytes of HBM traffic per visible pair (the
 * block written and read back). The dQ kernel contracts the same bf16 dS values in the same
 * order as cpattn_block_bwd's dQ kernel. No atomics: bitwise reproducible.
 * workspace: device memory of cpattn_block_bwd_staged_workspace_bytes(B,H,Tq,Tk,D) bytes,
 * 256-byte aligned, owned by the caller; its contents on entry do not matter and on return
 * are unspecified. At D = 64 that size is 0, workspace may be NULL, and the call is
 * cpattn_block_bwd_gqa.
 * Errors: as cpattn_block_bwd_gqa, plus EINVAL for a short or misaligned workspace.
 */
size_t cpattn_block_bwd_staged_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D);
int cpattn_block_bwd_staged(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                            const cpattn_tensor* dout, int32_t dtype, const cpattn_tensor* lse,
                            const cpattn_tensor* delta, const cpattn_tensor* dq_acc,
                            const cpattn_tensor* dk_acc, const cpattn_tensor* dv_acc, int64_t B,
                            int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t D,
                            const cpattn_posmap* qmap, const cpattn_posmap* kmap, int32_t causal,
                            float scale, int32_t accumulate, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace bytes cpattn_ring_bwd needs: the fp32 delta of the local rows. 0 for non-positive sizes. */
size_t cpattn_ring_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Tq);
/* Workspace bytes with which cpattn_ring_bwd stages dS (delta, then the staging area of one
 * block); equal to cpattn_ring_bwd_workspace_bytes where no staging applies (D != 128). */
size_t cpattn_ring_bwd_staged_workspace_bytes(int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D);

/*
 * Ring backward of rank `rank` out of `ring`, all KV blocks resident in HBM:
 * the backward of cpattn_ring_fwd. It runs cpattn_bwd_preprocess into the
 * workspace, then one cpattn_block_bwd per step in the forward's order (step s
 * uses the block of owner (rank - s) mod ring), each with the final o and lse
 * of the local rows: every step rebuilds its P from the final LSE, which in
 * exact arithmetic equals the per-step saved (O, LSE) with the merge
 * rescaling of the backward (BluScriptCP log, 2026-03-21, the backward merger
 * fix), so no per-step statistics are kept.
 * dq_acc [B,H,Tq,D] fp32 gathers every step's contribution; dk_blocks[i] and
 * dv_blocks[i] [B,H,Tk,D] fp32 get this rank's contribution to block i's
 * gradient (in a real ring that partial travels back to rank i and is summed
 * there with the other ranks' partials).
 * accumulate = 1 adds everything into the accumulators. accumulate = 0
 * overwrites: dq_acc takes the first step's contribution (every row written)
 * and adds the rest; each dk/dv block is written in full by its own step.
 * Steps whose block no local row sees are skipped when accumulate = 1.
 * q, k_blocks, v_blocks, dout bf16 (rotary is not applied here: pass the
 * rotated Q and K blocks that the forward used, then map dq and the dk blocks
 * back with cpattn_rope_rotate_grad); o and lse are cpattn_ring_fwd's outputs.
 * Multi-head only (H_kv = H). ring + 1 launches at most, no synchronisation.
 * workspace: device memory of cpattn_ring_bwd_workspace_bytes(B,H,Tq) bytes,
 * 256-byte aligned. With at least cpattn_ring_bwd_staged_workspace_bytes(B,H,Tq,Tk,D)
 * bytes (D = 128), the workspace also holds the dS staging area of
 * cpattn_block_bwd_staged and every step runs that form (same results, bit for bit;
 * 2 ring + 1 launches at most).
 * Errors: as cpattn_block_bwd for any step (checked before any launch), plus
 * EINVAL for ring < 1, rank out of range, null block arrays, a short or
 * misaligned workspace.
 */
int cpattn_ring_bwd(const cpattn_tensor* q, const cpattn_tensor* k_blocks,
                    const cpattn_tensor* v_blocks, const cpattn_posmap* kmaps,
                    int32_t ring, int32_t rank, const cpattn_posmap* qmap, int32_t dtype,
                    int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t causal,
                    float scale, const cpattn_tensor* dout, const cpattn_tensor* o,
                    const cpattn_tensor* lse, const cpattn_tensor* dq_acc,
                    const cpattn_tensor* dk_blocks, const cpattn_tensor* dv_blocks,
                    int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * cpattn_ring_bwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, semantics, launches and results as
 * cpattn_ring_bwd, bit for bit; the fp32 delta of the local rows lives in a
 * static device array of CPATTN_NOALLOC_MAX_ROWS floats (4 MiB) that each GPU
 * the library runs on holds until the process ends. Its address is looked up
 * on the first call made with a device current (call once outside graph
 * capture before capturing); the stream must belong to the current device.
 * The call allocates nothing and frees nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe. Nothing in the array needs to
 * start at zero (every row of delta is written before it is read).
 * Errors: as cpattn_ring_bwd, plus EINVAL if B*H*Tq > CPATTN_NOALLOC_MAX_ROWS
 * (checked before any launch) and EHIP if the array's address cannot be found.
 */
#define CPATTN_NOALLOC_MAX_ROWS (1 << 20)
int cpattn_ring_bwd_noalloc(const cpattn_tensor* q, const cpattn_tensor* k_blocks,
                            const cpattn_tensor* v_blocks, const cpattn_posmap* kmaps,
                            int32_t ring, int32_t rank, const cpattn_posmap* qmap, int32_t dtype,
                            int64_t B, int64_t H, int64_t Tq, int64_t Tk, int64_t D, int32_t causal,
                            float scale, const cpattn_tensor* dout, const cpattn_tensor* o,
                            const cpattn_tensor* lse, const cpattn_tensor* dq_acc,
                            const cpattn_tensor* dk_blocks, const cpattn_tensor* dv_blocks,
                            int32_t accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
