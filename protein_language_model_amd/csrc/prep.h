// Launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace esm {

struct PrepArgs {
  const int32_t* cu;
  int32_t B, T, H, max_seqlen, block, head_dim;
  int32_t* sorted;      // [B]
  int32_t* chunk_base;  // [n_chunks + 1]
  int32_t n_chunks;
  Item* items;          // [n_slots]
  int64_t n_slots;
  float2* rope;         // [max_seqlen][head_dim/2], or null
  double rope_base;
  int32_t* pos;         // [T] position of each token in its sequence
};

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);

// Rotation pass: q_rot = bf16(fl32(q_mul * fl32(R(p) q))), k_rot = bf16(R(p) k);
// R(p) is the identity when rope is null.
struct RotArgs {
  const uint16_t* q;    // may equal q_rot (in place, same row stride)
  const uint16_t* k;    // may equal k_rot
  uint16_t* q_rot;      // null: k alone is rotated (q unread)
  uint16_t* k_rot;
  int32_t ld_in;        // elements between consecutive tokens' rows of q, k
  int32_t ld_out;       // ... of q_rot, k_rot
  uint8_t* q8;          // E4M3 quantization: outputs [T][H][d] bytes (packed)
  uint8_t* k8;
  float q_inv, k_inv;   // fl32(1 / scale) of q and k
  float q_mul;          // fl32(softmax_scale * log2(e)): q~ is stored times this
  const float2* rope;   // [max_seqlen][d/2]
  const int32_t* pos;   // [T] token positions (the plan's)
  const Item* items;
  int32_t H, T;
  int32_t max_pos;      // max_seqlen - 1: positions are clamped to [0, max_pos]
};

// Rotation pass over all tokens (token-major: whole token rows, every head).
hipError_t launch_rotate(int head_dim, bool rope, const RotArgs& a, hipStream_t stream);
// q8 = E4M3(R(p) q * q_inv), k8 likewise (saturating, round to nearest even).
hipError_t launch_quantize_fp8(int head_dim, bool rope, const RotArgs& a, int64_t n_slots,
                               hipStream_t stream);

// Everything the attention kernels read. Pointers to bf16 data are uint16_t.
struct AttnArgs {
  const uint16_t* q;    // rotated q~
  const uint16_t* k;    // rotated k~
  const uint16_t* v;
  const uint16_t* o;    // backward: forward output
  const uint16_t* dout; // backward: dO
  uint16_t* out;        // forward: O
  float* lse;           // [H][T]
  const float* lse_in;  // backward: LSE from the forward
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* drow;          // backward: [H][T] x 16 bytes: -LSE log2(e), then -D, each split in 3 bf16
  const float2* rope;   // [max_seqlen][d/2]
  const Item* items;
  int32_t T, H;
  float c;              // FP8 forward: |softmax_scale| q_scale k_scale log2(e)
  float q_sign;         // FP8 forward: sign applied to the E4M3 query bytes
  float scale;          // softmax_scale (signed): dq = R(-p) (scale dQ~)
  int32_t ld_qkv;       // elements between consecutive tokens' rows of q~, k~, v
  int32_t ld_grad;      // ... of dq, dk, dv (o, dO: H * d)
  int32_t n_items;      // split forward: slots with an item record (the grid may be wider)
  int32_t n_split;      // split forward: key chunks per sequence
  float* o_part;        // split forward: [n_split][T][H][d] chunk outputs
  float* lse_part;      // split forward: [n_split][H][T] chunk LSEs
  const uint8_t* q8;    // FP8 forward: E4M3 q~, k~ [T][H][d] bytes, row stride ld8
  const uint8_t* k8;
  int32_t ld8;
  // small-batch path (every sequence at most kSmallMaxLen tokens, d <= 64):
  // one workgroup per (sequence, head) decoded from cu_seqlens, q and k
  // rotated inside the attention kernels (q, k are then the raw inputs)
  const int32_t* cu;    // [B + 1]
  int32_t B, max_seqlen;
  float rope_base;      // 0 = no rotation
  float q_mul;          // fl32(softmax_scale * log2(e)), as in the rotation pass
  // forward that rotates its own query rows (launch_fwd_rotq): q is the raw
  // query, rotated and scaled as the rotation pass does with the table `rope`
  // (always a readable [max_seqlen][d/2] region; rope_base = 0: no rotation)
  // and q_mul; q~ rows are written to q_out when it is not null (same row
  // stride as q; q_out == q is allowed)
  uint16_t* q_out;
};

// Longest sequence of the small-batch path (one 128-row work item).
constexpr int kSmallMaxLen = 128;

// Row pitch, in (cos, sin) entries, of the rotary table the small-batch
// kernels build in LDS: d/2 plus two. Every lane reads the 8 entries of its
// row (64 bytes); at a pitch of d/2 the rows of one ds_read_b128 cycle share
// banks (on gfx950 a cycle serves the quads of a half-wave with one parity
// of the quad index, measured with SQ_LDS_BANK_CONFLICT), at d/2 + 2 they do
// not at d = 16 and hardly at d = 32, 64 (checked against that rule for the
// prologue's, the query rotation's and the epilogue's reads).
template <int D>
constexpr int small_tab_pitch() {
  return D / 2 + 2;
}

hipError_t launch_fwd(int head_dim, const AttnArgs& a, int64_t n_slots, bool split,
                      hipStream_t stream);
hipError_t launch_fwd_fp8(int head_dim, const AttnArgs& a, int64_t n_slots, hipStream_t stream);
// Forward on raw q (each item rotates its own 128 query rows in registers)
// and rotated k~; optionally writes q~ for the backward.
hipError_t launch_fwd_rotq(int head_dim, const AttnArgs& a, int64_t n_slots, hipStream_t stream);
// Small-batch path (max_seqlen <= kSmallMaxLen, head_dim <= 64): one
// workgroup per (sequence, head), B * H of them, no plan, q and k rotated
// inside the kernels. The forward writes o and lse; the backward writes
// dq, dk and dv in one pass (dQ from the dS tile kept in LDS).
hipError_t launch_fwd_small(int head_dim, const AttnArgs& a, hipStream_t stream);
hipError_t launch_bwd_small(int head_dim, const AttnArgs& a, hipStream_t stream);

// O = sum_r exp(LSE_r - LSE) O_r, LSE = log sum_r exp(LSE_r) over n_parts
// partials o_part [n_parts][T][H][d] (fp32), lse_part [n_parts][H][T];
// writes o (bf16, [T][H][d]) and lse ([H][T]).
hipError_t launch_merge(int head_dim, const float* o_part, const float* lse_part, int n_parts,
                        int T, int H, uint16_t* o, float* lse, hipStream_t stream);
hipError_t launch_bwd(int head_dim, bool rope, const AttnArgs& a, int64_t n_slots, bool dq_pass,
                      bool dkv_pass, hipStream_t stream);

// Rows per work item of every kernel (the schedule is built for it).
constexpr int kItemRows = 128;

}  // namespace esm
