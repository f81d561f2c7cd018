/*
 * esm_attn.h -- C ABI of the MI355X (gfx950) attention library for ESM-2-style
 * protein language model training: bidirectional multi-head self-attention
 * with rotary position embedding over packed variable-length sequences,
 * forward and backward.
 *
 * What is computed (for every sequence b and head h):
 *   ESM-2 is a BERT-style model ("BioNeMo Framework: a modular,
 *   high-performance library for AI model development in drug discovery"
 *   review page, Abstract and "proposed method"), so a token attends to all
 *   tokens of its own sequence and to nothing else. Sequences are packed back
 *   to back by the size-aware bucket batching of the same page, with no
 *   padding between them. Inputs and outputs are BF16 (BioNeMo Recipes hub
 *   page, multi-precision training section); products accumulate in FP32
 *   (BioNeMo blog, section 2.3).
 *
 *   p          = t - cu_seqlens[b]          position of token t, 0-based per sequence
 *   theta_j    = rope_base^(-2j/d)          j in [0, d/2)
 *   x~         = R(p) x: (x_j, x_{j+d/2}) turned by the angle p*theta_j
 *                (rotary position embedding, half-split pairing; rope_base = 0
 *                switches it off)
 *   S_ij       = softmax_scale * (q~_i . k~_j)       i, j in the same sequence
 *   LSE_i      = ln sum_j exp(S_ij)
 *   P_ij       = exp(S_ij - LSE_i)
 *   O_i        = sum_j P_ij v_j
 * and, given dO, the gradients of sum(dO * O):
 *   dv_j = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - D_i),  D_i = dO_i . O_i
 *   dq_i = R(p_i)^T (softmax_scale * sum_j dS_ij k~_j)
 *   dk_j = R(p_j)^T (softmax_scale * sum_i dS_ij q~_i)
 * q~ and k~ are rounded once to bf16 before the products (they are operands
 * of bf16 matrix instructions); everything else accumulates in fp32. The
 * rounded query operand carries the softmax scale in log2 units:
 * q^ = bf16(fl32(c * fl32(R(p) q))) with c = fl32(softmax_scale * log2(e)),
 * k^ = bf16(R(p) k), S_ij = ln(2) * (q^_i . k^_j), and dk_j uses
 * ln(2) * sum_i dS_ij q^_i.
 *
 * Layouts
 *   q, k, v, o, d_o, dq, dk, dv : bf16 bit patterns (uint16_t), [T][H][d],
 *                                 row-major, d fastest; token-major packing
 *   lse                         : float, [H][T], natural log
 *   cu_seqlens                  : int32_t, [batch + 1], DEVICE memory
 *   head_dim d                  : 16, 32, 64 or 128
 *   The planned calls also take token row strides (elements between the
 *   starts of consecutive tokens' rows; H*d for the packed layout above): a
 *   fused projection's output [T][3][H][d] is used in place as q, k, v with
 *   stride 3*H*d, and dq, dk, dv can be written into one [T][3][H][d]
 *   gradient the same way. A stride must be >= H*d and a multiple of 8
 *   (else ESM_ATTN_ERR_INVALID_ARGUMENT), and total_tokens * stride < 2^31
 *   (else ESM_ATTN_ERR_UNSUPPORTED).
 *
 * Ownership and execution
 *   The caller allocates every buffer (inputs, outputs, workspace); the library
 *   never allocates or frees memory and keeps no pointer after a call returns.
 *   (One exception: esm_attn_fwd_noalloc works in a fixed buffer the library
 *   itself holds in device global memory, see there.)
 *   Calls are enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   return without waiting; there is no host-device synchronisation and no
 *   device read on the host, so the calls can be captured in a HIP graph.
 *   Workspace contents are undefined before and after a call; concurrent calls
 *   on different streams need different workspaces. Outputs must not alias
 *   inputs or each other.
 *
 * Errors
 *   Problems visible on the host are reported before anything is enqueued and
 *   leave every output untouched. ESM_ATTN_ERR_INVALID_ARGUMENT: null
 *   pointers (allowed when total_tokens is 0), pointers not 16-byte aligned,
 *   batch < 1, num_heads < 1, total_tokens < 0, max_seqlen < 0,
 *   softmax_scale non-finite or with |softmax_scale| * log2(e) beyond the
 *   fp32 range, rope_base negative or non-finite. The scores
 *   softmax_scale * (q~ . k~) must themselves lie in the fp32 range (the
 *   kernels compute them in fp32).
 *   ESM_ATTN_ERR_UNSUPPORTED: max_seqlen > 65536, head_dim not in
 *   {16, 32, 64, 128}, total_tokens*num_heads*head_dim >= 2^31.
 *   ESM_ATTN_ERR_WORKSPACE_TOO_SMALL: workspace smaller than the matching
 *   *_workspace_bytes() result. A failed kernel launch returns
 *   ESM_ATTN_ERR_HIP. Faults during execution surface at the caller's next
 *   synchronisation, as for any HIP work.
 *   The library cannot check the contents of the device-resident cu_seqlens
 *   without a synchronisation; the caller guarantees cu_seqlens[0] = 0,
 *   nondecreasing entries, cu_seqlens[batch] = total_tokens and every length
 *   <= max_seqlen (esm_attn_check_cu_seqlens_host checks a host copy).
 *   Kernels clamp lengths to [0, max_seqlen] and token indices to
 *   [0, total_tokens), so a bad cu_seqlens gives wrong values, never
 *   out-of-bounds accesses. Zero-length sequences are legal; total_tokens = 0
 *   enqueues nothing and returns ESM_ATTN_OK.
 */
#ifndef ESM_ATTN_H
#define ESM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ESM_ATTN_ABI_VERSION 6

typedef int32_t esm_attn_status_t;
#define ESM_ATTN_OK 0
#define ESM_ATTN_ERR_INVALID_ARGUMENT 1
#define ESM_ATTN_ERR_UNSUPPORTED 2
#define ESM_ATTN_ERR_WORKSPACE_TOO_SMALL 3
#define ESM_ATTN_ERR_HIP 4
#define ESM_ATTN_ERR_SCRATCH_TOO_SMALL 5

/* ESM_ATTN_ABI_VERSION of the built library. */
int32_t esm_attn_abi_version(void);

/* Static, never-NULL description of a status code (unknown codes included). */
const char* esm_attn_status_string(esm_attn_status_t status);

/* Workspace bytes that esm_attn_fwd / esm_attn_bwd need for these sizes
 * (a pure host computation; 0 for arguments the calls would reject). The
 * workspace holds the plan (rotary cos/sin table and work-item schedule), the
 * rotated k^ and, for the backward and for the forward at head_dim 128, q^
 * (bf16 [T][H][d] each; the forward up to head_dim 64 rotates q inside the
 * attention kernel, as esm_attn_fwd_rotq_planned) and, for the backward, drow
 * ([H][T] entries of 16 bytes: LSE * log2(e) and the row sum
 * D = rowsum(dO * O), each negated and split into three bf16 values). */
size_t esm_attn_fwd_workspace_bytes(int32_t batch, int32_t total_tokens,
                                    int32_t max_seqlen, int32_t num_heads,
                                    int32_t head_dim);
size_t esm_attn_bwd_workspace_bytes(int32_t batch, int32_t total_tokens,
                                    int32_t max_seqlen, int32_t num_heads,
                                    int32_t head_dim);

/* Forward. q, k, v: pre-rotation inputs, bf16 [T][H][d] (device).
 * cu_seqlens: int32 [batch+1] (device). softmax_scale: usually 1/sqrt(d);
 * any finite value. rope_base: usually 10000; 0 = no rotary embedding.
 * Writes o (bf16 [T][H][d]) and lse (fp32 [H][T], natural log). Runs the
 * planned steps in its workspace (plan; k, or q and k at head_dim 128,
 * rotated by the rotation pass; the forward, which rotates q itself up to
 * head_dim 64), or, when every sequence fits one 128-row work item and
 * head_dim <= 64, one small-batch kernel; the results are the same either
 * way (bitwise for o and lse). */
esm_attn_status_t esm_attn_fwd(
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const int32_t* cu_seqlens,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim,
    float softmax_scale, float rope_base,
    uint16_t* o, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/* Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation as esm_attn_fwd, with the same arguments minus the
 * workspace, which is instead a library-owned buffer of
 * ESM_ATTN_NOALLOC_SCRATCH_BYTES (128 MiB) in device global memory, one copy
 * per GPU, held from the library's load on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine);
 * its first call on a GPU looks up that GPU's copy of the buffer.
 * ESM_ATTN_ERR_SCRATCH_TOO_SMALL when esm_attn_fwd_workspace_bytes() of
 * these sizes exceeds the buffer (it holds the plan and the rotated q^, k^:
 * T*H*d up to about 33 million elements minus the plan); the other errors
 * as for esm_attn_fwd. Every call on one
 * GPU uses that GPU's one buffer, whose contents persist between calls:
 * calls that overlap on one GPU (different streams, or different host
 * threads without stream ordering) race and give wrong results; calls
 * ordered on one stream are safe. Nothing in the buffer needs to start at
 * zero (each call writes every byte it later reads). */
#define ESM_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
esm_attn_status_t esm_attn_fwd_noalloc(
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const int32_t* cu_seqlens,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim,
    float softmax_scale, float rope_base,
    uint16_t* o, float* lse, void* stream);

/* Backward. q, k, v as given to the forward; o and lse as it returned them;
 * d_o: gradient of the loss with respect to o, bf16 [T][H][d].
 * Writes dq, dk, dv (bf16 [T][H][d]): gradients with respect to the
 * pre-rotation q and k and to v. */
esm_attn_status_t esm_attn_bwd(
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const uint16_t* o, const uint16_t* d_o, const float* lse,
    const int32_t* cu_seqlens,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim,
    float softmax_scale, float rope_base,
    uint16_t* dq, uint16_t* dk, uint16_t* dv,
    void* workspace, size_t workspace_bytes, void* stream);

/* ---- plan / execute split ------------------------------------------------
 * esm_attn_fwd and esm_attn_bwd each run three steps on their workspace:
 *   1. plan   : the work-item schedule for cu_seqlens and the rotary cos/sin
 *               table (esm_attn_plan);
 *   2. rotate : q^ = bf16(c R(p) q) and k^ = bf16(R(p) k), once per token
 *               (esm_attn_rotate_planned; c = softmax_scale log2(e); with
 *               rope_base = 0, R(p) is the identity);
 *   3. the attention kernels on q^, k^ (esm_attn_fwd_planned,
 *      esm_attn_bwd_planned), given the same softmax_scale.
 * A caller that runs the forward and backward of one batch can run steps 1
 * and 2 once and keep q^ and k^ (instead of q and k) for the backward. The
 * plan depends only on cu_seqlens, the sizes and rope_base, so one plan
 * serves every layer of a model for that batch (the rotary table is shared
 * across layers); a fused layer rotates q and k in place inside its
 * [T][3][H][d] projection output and keeps that buffer for its backward.
 *
 * The plan buffer is device memory of esm_attn_plan_bytes() bytes, owned by
 * the caller, valid for the sizes, cu_seqlens contents and rope_base it was
 * built with, and read-only for the other planned calls (several may use one
 * plan, on one stream or after proper stream ordering). The planned calls do
 * not read cu_seqlens; they take the same sizes (a different rope_base than
 * the plan's gives wrong values, not an error). */
size_t esm_attn_plan_bytes(int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                           int32_t num_heads, int32_t head_dim);

esm_attn_status_t esm_attn_plan(const int32_t* cu_seqlens, int32_t batch,
                                int32_t total_tokens, int32_t max_seqlen,
                                int32_t num_heads, int32_t head_dim, float rope_base,
                                void* plan, size_t plan_bytes, void* stream);

/* Rotary embedding of q and k (RoFormer's rotation with x_j paired with
 * x_{j+d/2}, angles p * rope_base^(-2j/d) from the plan's table): every
 * element pair is turned in float32 (products and sums rounded one by one);
 * k_rot = bf16(R(p) k) and q_rot = bf16(fl32(c * fl32(R(p) q))) with
 * c = fl32(softmax_scale * log2(e)), each rounded once to bf16, round to
 * nearest even (the attention kernels then exponentiate q_rot . k_rot
 * directly). softmax_scale must be the one later given to the forward and
 * backward on these operands (a different one gives wrong values, not an
 * error); it must be finite with a finite c. Reads q and k with token row
 * stride in_row_stride and writes q_rot and k_rot, bf16, with stride
 * out_row_stride; with rope_base = 0, R(p) is the identity. In place is
 * allowed:
 * q_rot == q and k_rot == k with equal strides (a fused layer rotates q and
 * k inside its [T][3][H][d] projection output); q_rot == q without
 * k_rot == k, or in place with different strides, is
 * ESM_ATTN_ERR_INVALID_ARGUMENT. Otherwise outputs must not overlap inputs.
 * q = q_rot = NULL rotates k alone (for esm_attn_fwd_rotq_planned, which
 * rotates the queries itself); k_rot == k is then in place. */
esm_attn_status_t esm_attn_rotate_planned(
    const uint16_t* q, const uint16_t* k, int32_t in_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float softmax_scale, float rope_base,
    uint16_t* q_rot, uint16_t* k_rot, int32_t out_row_stride,
    const void* plan, size_t plan_bytes, void* stream);

/* Forward on rotated operands: q_rot and k_rot as esm_attn_rotate_planned
 * wrote them with this softmax_scale, and v, all with token row stride
 * qkv_row_stride (they may interleave in one fused buffer). Writes o
 * ([T][H][d], packed) and lse as esm_attn_fwd does. */
esm_attn_status_t esm_attn_fwd_planned(
    const uint16_t* q_rot, const uint16_t* k_rot, const uint16_t* v,
    int32_t qkv_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float softmax_scale,
    uint16_t* o, float* lse,
    const void* plan, size_t plan_bytes, void* stream);

/* Forward that rotates the queries itself: q is the unrotated query, with
 * k_rot (esm_attn_rotate_planned's k_rot, e.g. from its k-alone mode) and v
 * at token row stride qkv_row_stride. Each work item turns and scales its
 * own query rows exactly as esm_attn_rotate_planned does (the plan's table,
 * the same float32 operations, one rounding to bf16), so o and lse are
 * bitwise those of esm_attn_rotate_planned followed by esm_attn_fwd_planned;
 * the rotation pass then moves half the bytes. softmax_scale and rope_base
 * as for esm_attn_rotate_planned (rope_base = 0: no rotation). If q_rot is
 * not NULL, the rotated rows q^ are written there with stride
 * qkv_row_stride, for the backward: rows of tokens inside a sequence's
 * first max_seqlen tokens, bitwise the rotation pass's q_rot (others are not
 * written). q_rot == q rotates in place (each item's query rows are read by
 * that item alone, before it writes them); otherwise q_rot must not overlap
 * an input. The operation is esm_attn_fwd's, defined at the top of this
 * file. */
esm_attn_status_t esm_attn_fwd_rotq_planned(
    const uint16_t* q, const uint16_t* k_rot, const uint16_t* v,
    int32_t qkv_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float softmax_scale, float rope_base,
    uint16_t* o, float* lse, uint16_t* q_rot,
    const void* plan, size_t plan_bytes, void* stream);

/* Split-KV forward: the same result as esm_attn_fwd_planned (to fp32
 * rounding; bitwise equal for n_split = 1) computed as n_split key-range
 * partials per work item and their merge. Each sequence's key blocks are
 * dealt out in n_split contiguous chunks of ceil(blocks / n_split); chunk r of
 * every item is one more workgroup, which fills the chip when a batch has few
 * (sequence, head, query-block) items (few long sequences, few heads: e.g.
 * the local heads of a sequence-parallel shard). Key-range partials and their
 * merge are the per-device half of attention with keys sharded over devices
 * ("Scaling biomolecular modeling with context parallelism in NVIDIA BioNeMo"
 * page, "2D tiling of the pairwise representation").
 *   o_part   : fp32 [n_split][T][H][d], caller-owned scratch; chunk outputs,
 *              each normalised over its own keys (0 for an empty chunk)
 *   lse_part : fp32 [n_split][H][T], chunk LSEs (-inf for an empty chunk)
 *   o, lse   : as esm_attn_fwd_planned.
 * 1 <= n_split <= 64, else ESM_ATTN_ERR_INVALID_ARGUMENT. */
esm_attn_status_t esm_attn_fwd_split_planned(
    const uint16_t* q_rot, const uint16_t* k_rot, const uint16_t* v,
    int32_t qkv_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float softmax_scale,
    int32_t n_split, float* o_part, float* lse_part,
    uint16_t* o, float* lse,
    const void* plan, size_t plan_bytes, void* stream);

/* ---- FP8 (OCP E4M3) forward, inference first ------------------------------
 * The BioNeMo Recipes hub page lists FP8 among its training precisions
 * (multi-precision training section). Here the scores take E4M3 operands on
 * gfx950's 32x32x64 FP8 matrix instruction; softmax, P (bf16) and P V (bf16
 * V) are those of the bf16 forward. head_dim 64 or 128 (else
 * ESM_ATTN_ERR_UNSUPPORTED); q_scale, k_scale finite and > 0 with finite
 * reciprocals (else ESM_ATTN_ERR_INVALID_ARGUMENT).
 *
 * Quantization: q8 = E4M3(clamp(R(p) q * fl32(1 / q_scale), +-448)), k8
 * likewise: the rotation in float32 as esm_attn_rotate_planned (no bf16
 * rounding in between), one float32 product, saturation at the largest E4M3
 * value (448; E4M3 has no infinity), one rounding to nearest even. q and k
 * read with in_row_stride; q8, k8 written packed [T][H][d] bytes. A scale of
 * amax(|q|) * sqrt(2) / 448 avoids saturation (the rotation can grow one
 * component of a pair by at most sqrt(2)). */
esm_attn_status_t esm_attn_quantize_fp8_planned(
    const uint16_t* q, const uint16_t* k, int32_t in_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float rope_base,
    float q_scale, float k_scale, uint8_t* q8, uint8_t* k8,
    const void* plan, size_t plan_bytes, void* stream);

/* Forward on E4M3 q8, k8 (packed, from esm_attn_quantize_fp8_planned with the
 * same scales) and bf16 v (row stride v_row_stride): S = softmax_scale *
 * q_scale * k_scale * (q8 . k8); o and lse as esm_attn_fwd_planned.
 * ESM_ATTN_ERR_INVALID_ARGUMENT also if |softmax_scale| * q_scale * k_scale *
 * log2(e) is not a finite fp32 value. */
esm_attn_status_t esm_attn_fwd_fp8_planned(
    const uint8_t* q8, const uint8_t* k8, const uint16_t* v, int32_t v_row_stride,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim, float softmax_scale,
    float q_scale, float k_scale, uint16_t* o, float* lse,
    const void* plan, size_t plan_bytes, void* stream);

/* Merge of n_parts attention partials of the same queries over disjoint key
 * sets (fp32 o_part [n_parts][T][H][d], lse_part [n_parts][H][T], as the split
 * forward writes them, or as received from other devices):
 *   LSE = log sum_r exp(LSE_r),  O = sum_r exp(LSE_r - LSE) O_r,
 * computed in fp32 (relative to the largest LSE_r); parts with LSE_r = -inf
 * add nothing; rows whose parts are all -inf get O = 0, LSE = -inf. Writes
 * o (bf16 [T][H][d], round to nearest even) and lse (fp32 [H][T]). Needs no
 * plan. 1 <= n_parts <= 64. */
esm_attn_status_t esm_attn_merge_partials(
    const float* o_part, const float* lse_part, int32_t n_parts,
    int32_t total_tokens, int32_t num_heads, int32_t head_dim,
    uint16_t* o, float* lse, void* stream);

/* Backward on rotated operands (q_rot, k_rot, v and their stride as for the
 * forward; o and d_o packed [T][H][d]); dq and dk are still the gradients
 * with respect to the pre-rotation q and k: the kernels apply R(p)^T, for
 * which they need rope_base. dq, dk, dv are written with token row stride
 * grad_row_stride (they may interleave in one [T][3][H][d] gradient; they
 * must not overlap any input). softmax_scale: the one q_rot was made with.
 * drow: caller-provided device buffer of 16 * H * T bytes, 16-byte aligned
 * ([H][T] entries of 16 bytes: -LSE * log2(e), then -D = -rowsum(dO * O),
 * each split into three bf16 values). passes is a
 * bit mask: ESM_ATTN_PASS_DQ runs the dq pass (reads o and lse, writes dq and
 * drow), ESM_ATTN_PASS_DKV the dk/dv pass (reads drow, writes dk and dv);
 * both bits give the full backward. Running the dk/dv pass alone requires a
 * completed dq pass of the same inputs. Pointers a pass does not use may be
 * NULL. */
#define ESM_ATTN_PASS_DQ 1
#define ESM_ATTN_PASS_DKV 2
esm_attn_status_t esm_attn_bwd_planned(
    const uint16_t* q_rot, const uint16_t* k_rot, const uint16_t* v,
    int32_t qkv_row_stride,
    const uint16_t* o, const uint16_t* d_o, const float* lse,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen,
    int32_t num_heads, int32_t head_dim,
    float softmax_scale, float rope_base,
    uint16_t* dq, uint16_t* dk, uint16_t* dv, int32_t grad_row_stride,
    float* drow, int32_t passes,
    const void* plan, size_t plan_bytes, void* stream);

/* Size-aware bucket batching (host only; reads host arrays, enqueues
 * nothing). The "BioNeMo Framework" review page names a size-aware batcher and
 * a bucket batch sampler ("proposed method") and credits them with
 * near-uniform batch sizes and almost no padding ("main findings"); the rule
 * implemented is this reading of them:
 *   buckets   : n_boundaries increasing lengths b_0 < ... < b_{K-1} (each
 *               >= 1) make the buckets [0, b_0), [b_0, b_1), ...,
 *               [b_{K-1}, inf); no boundaries = one bucket;
 *   batcher   : inside each bucket, sequences in input order are appended to
 *               the current batch while its cost stays <= budget; one that
 *               would exceed it starts the next batch (a sequence over budget
 *               alone forms a batch of one). Cost = sum of lengths (padded = 0,
 *               the packed layout) or batch size * longest length (padded = 1);
 *   output    : batches bucket by bucket, in the order formed: batch b is
 *               order[batch_offsets[b] .. batch_offsets[b+1]), indices into
 *               lengths; order has n entries, batch_offsets
 *               batch_capacity + 1 (n batches at most, so batch_capacity = n
 *               always suffices); *n_batches receives the count.
 * Returns ESM_ATTN_ERR_INVALID_ARGUMENT for a negative length, boundaries not
 * increasing or < 1, budget < 1, padded not 0 or 1, a null pointer, or more
 * batches than batch_capacity. */
esm_attn_status_t esm_attn_bucket_batches(const int32_t* lengths, int32_t n,
                                          const int32_t* boundaries, int32_t n_boundaries,
                                          int64_t budget, int32_t padded, int32_t* order,
                                          int32_t* batch_offsets, int32_t batch_capacity,
                                          int32_t* n_batches);

/* Host-only check of a HOST copy of cu_seqlens: cu[0] = 0, nondecreasing,
 * cu[batch] = total_tokens, every length <= max_seqlen. Returns ESM_ATTN_OK or
 * ESM_ATTN_ERR_INVALID_ARGUMENT. Reads batch+1 entries; enqueues nothing. */
esm_attn_status_t esm_attn_check_cu_seqlens_host(const int32_t* cu_host,
                                                 int32_t batch,
                                                 int32_t total_tokens,
                                                 int32_t max_seqlen);

/* Host-only model of the device work-item schedule, for tests and tools.
 * Given a HOST copy of cu_seqlens, builds the schedule the kernels use for
 * items of `block_rows` rows (sequences longest first; the items of one
 * (sequence, head) pair on slots congruent modulo 8, i.e. on one of the
 * chip's eight XCDs under round-robin dispatch) and decodes every launched
 * slot into items[4*s .. 4*s+3] = {sequence start, length, head, block} or
 * {-1, -1, -1, -1} for an idle slot. *n_slots receives the launch size (an
 * upper bound the host computes without reading cu_seqlens); items must hold
 * 4 * items_capacity ints. Returns ESM_ATTN_ERR_INVALID_ARGUMENT if the
 * capacity is too small or an argument is out of range. */
esm_attn_status_t esm_attn_schedule_host(const int32_t* cu_host, int32_t batch,
                                         int32_t total_tokens, int32_t max_seqlen,
                                         int32_t num_heads, int32_t block_rows,
                                         int32_t* items, int32_t items_capacity,
                                         int32_t* n_slots);

#ifdef __cplusplus
}
#endif

#endif /* ESM_ATTN_H */
