/*
 * lightning_attn.h -- C ABI of liblightning_attn.so: the Lightning Attention
 * forward pass (causal linear attention, block-tiled) and its constant-cost
 * decode step, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (wiki page "MiniMax-01 Lightning Attention", section
 * "Lightning Attention 设计"; Tencent Cloud article "首个线性注意力架构的大模型
 * 来了…", section 4.1):
 *
 *   o_i = sum_{j <= i} (q_i . k_j) v_j        for every token i of a sequence,
 *
 * with no scale, feature map, normaliser or decay applied inside.  The
 * sequence is cut into blocks of `block_size` tokens; inside a block the
 * masked left product (Q K^T) V is used, across blocks the right product
 * Q S with S = sum of k^T v over all earlier blocks (a d x d state).
 * The decode step is o = q S, then S += k^T v (the state read by o is the
 * one before this token).
 *
 * Plain C: no C++ or HIP types in any signature.  All tensor pointers are
 * DEVICE pointers on the current HIP device; `stream` is a hipStream_t passed
 * as void* (NULL = the default stream).  Every launch is asynchronous on
 * `stream`; nothing synchronises the host.  The library allocates no memory;
 * the only state it keeps is each device's compute-unit count, read once from
 * the device's properties.  Calls are reentrant; calls that share a workspace
 * or a decode state must be ordered by the caller.
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and o. */
#define LA_DTYPE_BF16 0  /* bfloat16 in, fp32 accumulation, bfloat16 out (round to nearest even) */
#define LA_DTYPE_F32  1  /* fp32 in, fp32 accumulation, fp32 out */

/* Status codes. */
#define LA_OK           0  /* success (launches queued on the stream)               */
#define LA_EINVAL       1  /* NULL pointer with work to do, or a negative/zero size */
#define LA_EUNSUPPORTED 2  /* head_dim not 64/128, block_size not 64/128/256, dtype unknown, or a
                              shape past the limits of one launch (more than 2^32 - 1 threads
                              along the grid: over ~4.19M chunks in a prefill, or batch x heads
                              of 2^24 or more in a decode step) */
#define LA_EWORKSPACE   3  /* workspace NULL or smaller than the size query returned */
#define LA_EHIP         4  /* a HIP launch failed; see hipGetLastError semantics     */
#define LA_ESCRATCH     5  /* lightning_attn_fwd_noalloc: the call needs more scratch than
                              LA_NOALLOC_SCRATCH_BYTES */

/*
 * Bytes of device workspace lightning_attn_fwd needs for these arguments
 * (always a multiple of 256; 0 when seq_len == 0).  `varlen` is non-zero when
 * cu_seqlens will be passed; then `batch` is the number of packed sequences
 * and `seq_len` their total token count.  Returns 0 for arguments
 * lightning_attn_fwd would reject.  The work is split to fill the current
 * device's compute units, so query with the device current that will run the
 * pass.  The workspace holds per-chunk fp32 d x d
 * states (Tencent Cloud article, section 4.1: the compact key-value prefix of
 * all earlier blocks) and small tables; its contents need no initialisation
 * and are scratch after the call.
 */
size_t lightning_attn_fwd_workspace_size(int batch, int heads, int64_t seq_len, int head_dim,
                                         int block_size, int varlen, int dtype);

/*
 * Number of tokens one workgroup carries the state across in the forward
 * pass (a multiple of block_size), for the same arguments.  Informational:
 * the result does not depend on it beyond rounding.  0 for rejected arguments.
 */
int64_t lightning_attn_fwd_chunk_tokens(int batch, int heads, int64_t seq_len, int head_dim,
                                        int block_size, int varlen, int dtype);

/*
 * Forward pass (prefill).
 *
 * Dense input (cu_seqlens == NULL): q, k, v, o are contiguous
 *   [batch][heads][seq_len][head_dim]; each (batch, head) is one sequence.
 * Packed variable-length input (cu_seqlens != NULL; wiki page section
 *   "计算优化": data-packing without padding): q, k, v, o are contiguous
 *   [heads][seq_len][head_dim] where seq_len = T is the total token count;
 *   cu_seqlens is a DEVICE int32 array of batch+1 entries with
 *   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[batch] = T.  Sequence s is
 *   tokens [cu_seqlens[s], cu_seqlens[s+1]) of every head and starts from an
 *   empty state.  The device checks these contents before any other work: a
 *   malformed table makes the call compute nothing (o is left as it was);
 *   with the environment variable LA_DEBUG_CHECKS=1 the call also waits for
 *   the stream and returns LA_EINVAL in that case.
 *
 * block_size in {64, 128, 256}; head_dim in {64, 128}; blocks start at each
 * sequence's first token and the last block of a sequence may be short.
 * o has the dtype of q and must not alias q, k, v or the workspace.
 * workspace: device memory of at least lightning_attn_fwd_workspace_size(...)
 * bytes (same arguments, varlen = cu_seqlens != NULL), 256-byte aligned.
 *
 * q, k, v and o must be 16-byte aligned (the kernels move 16-byte vectors),
 * the workspace 256-byte aligned and cu_seqlens 4-byte aligned (else
 * LA_EINVAL).
 * All argument checks happen on the host before any launch (the contents of
 * cu_seqlens, which live on the device, are checked by the first kernel as
 * described above); a rejected call writes nothing.  seq_len == 0 returns LA_OK without touching any pointer.
 * Device-side faults surface at the caller's next synchronisation.
 */
int lightning_attn_fwd(const void *q, const void *k, const void *v, void *o,
                       int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                       const int32_t *cu_seqlens, int dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * lightning_attn_fwd with a state handoff: each sequence may start from a
 * given d x d state and its state after its last token may be returned, so
 * a prefill can hand its state to lightning_attn_decode, or a sequence can
 * be prefilled in pieces (wiki page "MiniMax-01 Lightning Attention", section
 * "Lightning Attention 设计": the KV state carries everything the earlier
 * tokens contribute; Tencent Cloud article, section 4.1).
 *   s_init:  NULL (every sequence starts from zero, as lightning_attn_fwd) or
 *            DEVICE fp32 [batch][heads][head_dim][head_dim], state[a][b] with
 *            a = key dimension, b = value dimension (the decode state layout);
 *            read only.
 *   s_final: NULL (not wanted) or DEVICE fp32, same layout: receives
 *            S_final = s_init + sum over the sequence of k^T v (a sequence of
 *            length 0 gets its s_init, or zero).
 * Then o_i = q_i (s_init + sum_{j <= i} k_j^T v_j).  s_final may be the same
 * buffer as s_init (updated in place); other overlaps between s_final and
 * any buffer are not allowed.  Both must be 16-byte aligned (else LA_EINVAL).
 * All other arguments, checks and rules are those of lightning_attn_fwd; when
 * seq_len == 0 only s_final is written (no workspace is needed).
 */
int lightning_attn_fwd_state(const void *q, const void *k, const void *v, void *o,
                             int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                             const int32_t *cu_seqlens, int dtype,
                             const float *s_init, float *s_final,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * lightning_attn_fwd with stage timing: identical work and results, and in
 * addition records caller-created hipEvent_t handles (passed as void*) on
 * `stream` at the stage boundaries, so a caller can time each kernel on the
 * stream it runs on:
 *   events[0] before the first launch,
 *   events[1] after the chunk/offset tables,
 *   events[2] after the per-chunk K^T V summaries,
 *   events[3] after the exclusive scan of chunk states,
 *   events[4] after the fused intra-block + Q S output kernel.
 * nevents must be LA_FWD_NUM_EVENTS and events non-NULL (else LA_EINVAL); a
 * NULL entry is not recorded, so a caller can bracket only the stages it
 * times (each recorded event takes a little time on the stream).  Stages with
 * nothing to do launch nothing: dense input builds no tables, and a plan of
 * one chunk per sequence runs no summaries or scan.  The events are only
 * recorded, never synchronised or destroyed.
 */
#define LA_FWD_NUM_EVENTS 5
int lightning_attn_fwd_traced(const void *q, const void *k, const void *v, void *o,
                              int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                              const int32_t *cu_seqlens, int dtype,
                              void *workspace, size_t workspace_bytes, void *stream,
                              void *const *events, int nevents);

/*
 * One decode step for batch x heads independent sequences (wiki page section
 * "Lightning Attention 设计": inference only updates the d x d KV state,
 * O(d^2) per token; comparison table row "状态大小").
 *   q, k, v, o: [batch][heads][head_dim] in `dtype`;
 *   state:      fp32 [batch][heads][head_dim][head_dim], state[a][b] with
 *               a = key dimension, b = value dimension; read and updated in
 *               place (caller-owned: a checkpoint is a copy of it).
 *   o = q . state_old ;  state_new = state_old + k^T v .
 * o must not alias the other buffers; state must be 16-byte aligned (else
 * LA_EINVAL).  Checks happen on the host first.
 */
int lightning_attn_decode(const void *q, const void *k, const void *v, float *state, void *o,
                          int batch, int heads, int head_dim, int dtype, void *stream);

/*
 * One decode step over an indexed state table, for serving batches whose
 * sequences come and go while their states stay in a pool (the wiki page's
 * section "计算优化" lists separate prefill and decoding execution and
 * multi-level padding among the inference optimisations): row b of the
 * batch uses pool entry slots[b].
 *   state_pool: fp32 [nslots][heads][head_dim][head_dim] (decode layout);
 *   slots:      DEVICE int32 [batch]; a slot < 0 or >= nslots marks a padding
 *               row: its o is written as zero and no state is touched, so a
 *               caller can pad a batch up to one of a few fixed sizes;
 *   q, k, v, o: [batch][heads][head_dim] in `dtype`.
 * For every non-padding row: o = q . S_old, S_new = S_old + k^T v, with S the
 * pool entry, updated in place.  Two non-padding rows must not name the same
 * slot (precondition, not checked).  state_pool may be NULL only when
 * nslots == 0 (then every row is padding).  Checks happen on the host first.
 */
int lightning_attn_decode_indexed(const void *q, const void *k, const void *v, float *state_pool,
                                  int nslots, const int32_t *slots, void *o, int batch, int heads,
                                  int head_dim, int dtype, void *stream);

/*
 * lightning_attn_fwd_state with rotary position embedding applied to q and k
 * on the way in (wiki page "MiniMax-01 Lightning Attention", section
 * "模型架构": RoPE on half of each head's dims, base frequency 10,000, raised
 * to 10M for the long-context stage).  The page leaves the details open;
 * this library takes: the first rope_dims dims are rotated, dim i
 * (i < rope_dims / 2) paired with dim i + rope_dims / 2, the pair at position
 * p turned by the angle p * rope_base^(-2i / rope_dims); v is not rotated.
 *   rope_dims:  must equal head_dim / 2 (else LA_EUNSUPPORTED);
 *   rope_base:  > 0 and finite (else LA_EINVAL);
 *   pos_offset: NULL (every sequence's first token is at position 0) or a
 *               DEVICE int32 [batch]: token t of sequence s is at position
 *               pos_offset[s] + t (a sequence continued from a handed-over
 *               state continues its positions).
 * q and k are read only (the rotation happens in registers and LDS).  The
 * final state is that of the rotated keys, the state a rotated decode step
 * (lightning_attn_decode_rope) continues.  bf16 kernels rotate in fp32 and
 * round the rotated values to bf16 for the matrix products; fp32 kernels keep
 * them in fp32.  Everything else is as lightning_attn_fwd_state.
 */
int lightning_attn_fwd_rope(const void *q, const void *k, const void *v, void *o,
                            int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                            const int32_t *cu_seqlens, int dtype,
                            int rope_dims, double rope_base, const int32_t *pos_offset,
                            const float *s_init, float *s_final,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefill over an indexed state table, for serving loops that keep every
 * live sequence's state in a pool (the wiki page's section "计算优化" lists
 * separate prefill and decoding execution and multi-level padding among the
 * inference optimisations): sequence s starts from pool entry slots[s] and
 * its state after its last token is written back to that entry, so a prompt
 * can be prefilled in pieces between decode steps
 * (lightning_attn_decode_indexed / lightning_attn_decode_rope on the same
 * pool) without gathering or scattering states.
 *   state_pool: fp32 [nslots][heads][head_dim][head_dim] (decode layout), read
 *               and updated in place; may be NULL only when nslots == 0;
 *   slots:      DEVICE int32 [batch] (required); a slot < 0 or >= nslots makes
 *               the sequence stateless: it starts from zero and its final
 *               state is dropped (padding, or a one-shot prefill).  Two
 *               sequences must not name the same slot (precondition, not
 *               checked).  A sequence of length 0 leaves its entry unchanged.
 *   rope_dims:  0 (no rotation) or head_dim / 2 with rope_base and pos_offset
 *               as in lightning_attn_fwd_rope.
 * Everything else (layouts, cu_seqlens, workspace, checks) is as
 * lightning_attn_fwd.  Then o_i = q_i (S_slot + sum_{j <= i} k_j^T v_j).
 */
int lightning_attn_fwd_indexed(const void *q, const void *k, const void *v, void *o,
                               int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                               const int32_t *cu_seqlens, int dtype,
                               float *state_pool, int nslots, const int32_t *slots,
                               int rope_dims, double rope_base, const int32_t *pos_offset,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step with q and k rotated as in lightning_attn_fwd_rope, row b
 * at position positions[b] (DEVICE int32 [batch], required).  With slots ==
 * NULL the states are [batch][heads][head_dim][head_dim] (as
 * lightning_attn_decode; nslots is ignored); otherwise row b uses pool entry
 * slots[b] of a pool of nslots entries, with padding rows, as
 * lightning_attn_decode_indexed.  rope_dims must equal head_dim / 2;
 * dtype LA_DTYPE_BF16 or LA_DTYPE_F32.  o = (R q) . S_old,
 * S_new = S_old + (R k)^T v.
 */
int lightning_attn_decode_rope(const void *q, const void *k, const void *v, float *state,
                               int nslots, const int32_t *slots, void *o, int batch, int heads,
                               int head_dim, int dtype, int rope_dims, double rope_base,
                               const int32_t *positions, void *stream);

/*
 * Test hooks: the forward pass with the chunking fixed by the caller instead
 * of chosen by the library, so that tests can reach every path of the
 * parallel scan (many chunks per sequence, many summary sub-chunks per chunk,
 * scan tiles starting inside chunks) at small sizes.  The result does not
 * depend on the chunking beyond rounding.  Not for production use: the
 * library's own choice (lightning_attn_fwd and the others) is the fast one.
 *   chunk_tokens: 0 (the library's choice) or the tokens one workgroup walks
 *                 carrying the state: a positive multiple of block_size, at
 *                 most 2^30 / (2 head_dim) tokens, and a multiple of 16384
 *                 when above 16384;
 *   sub_tokens:   0 (the library's choice) or the tokens of one K^T V summary:
 *                 a multiple of block_size dividing the chunk (ignored when
 *                 one chunk covers every dense sequence).
 * Other values are LA_EINVAL, and the size query returns 0 for them.
 *
 * lightning_attn_fwd_planned takes the union of the other forward entry
 * points' options: with slots == NULL, s_init / s_final as
 * lightning_attn_fwd_state (state_pool must be NULL); with slots != NULL, the
 * indexed pool of lightning_attn_fwd_indexed (s_init and s_final must be
 * NULL); rope_dims 0 or head_dim / 2 with rope_base and pos_offset as
 * lightning_attn_fwd_rope.  The workspace must be at least
 * lightning_attn_fwd_workspace_size_planned(...) bytes for the same
 * chunk_tokens and sub_tokens.  Everything else is as lightning_attn_fwd.
 */
size_t lightning_attn_fwd_workspace_size_planned(int batch, int heads, int64_t seq_len, int head_dim,
                                                 int block_size, int varlen, int dtype,
                                                 int64_t chunk_tokens, int64_t sub_tokens);
int lightning_attn_fwd_planned(const void *q, const void *k, const void *v, void *o,
                               int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                               const int32_t *cu_seqlens, int dtype,
                               const float *s_init, float *s_final,
                               float *state_pool, int nslots, const int32_t *slots,
                               int rope_dims, double rope_base, const int32_t *pos_offset,
                               int64_t chunk_tokens, int64_t sub_tokens,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * lightning_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, arguments, layouts, checks and results as
 * lightning_attn_fwd, without the workspace arguments.  The scratch the
 * kernels need (chunk tables and per-sub-chunk fp32 states) lives in a
 * static device array of LA_NOALLOC_SCRATCH_BYTES that each GPU the library
 * runs on holds until the process ends; the call allocates nothing.
 * A call whose lightning_attn_fwd_workspace_size(...) exceeds
 * LA_NOALLOC_SCRATCH_BYTES returns LA_ESCRATCH before any launch (e.g. 64
 * heads x 1,048,576 tokens needs more; the MiniMax layer and packed inputs
 * of a few hundred thousand tokens fit).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  Nothing in the array needs
 * clearing between calls: the kernels write every table and state they read.
 */
#define LA_NOALLOC_SCRATCH_BYTES (128u << 20)
int lightning_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o,
                               int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                               const int32_t *cu_seqlens, int dtype, void *stream);

/* Static, human-readable text for a status code. */
const char *lightning_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */
