// C-ABI entry points of libesm_attn.so: argument validation, workspace layout
// and the launch sequence. Nothing here reads device memory or synchronises.
#include <math.h>
#include <stdint.h>

#include <vector>

#include "esm_attn.h"
#include "prep.h"
#include "schedule.h"

namespace {

using namespace esm;

constexpr size_t kAlign = 256;
constexpr int32_t kMaxSplit = 64;  // key chunks / partials per merge
constexpr size_t kDrowEntryBytes = 16;  // per row of drow (see bwd.hip)
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t rope = 0, sorted = 0, chunk = 0, items = 0, pos = 0, plan = 0;  // the plan
  size_t drow = 0, qrot = 0, krot = 0, total = 0;                // one-shot calls only
  int64_t n_slots = 0;
  int32_t n_chunks = 0;
};

bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// The one-shot forward rotates q inside the attention kernel (and k alone in
// the rotation pass) up to d = 64. At d = 128 the rotary table of a long
// sequence (8192 positions x 512 bytes = 4 MB) no longer stays in L2 next to
// the K/V each XCD streams, and the kernel's table loads cost more than the
// rotation pass's q half (4 x 8192 tokens, H = 40: forward +266 us, rotation
// pass -125 us).
bool fwd_rotates_q(int32_t d) { return d <= 64; }

// Scalar checks shared by the calls and the workspace queries.
esm_attn_status_t check_sizes(int32_t B, int32_t T, int32_t maxL, int32_t H, int32_t d) {
  if (B < 1 || H < 1 || T < 0 || maxL < 0) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (maxL > kMaxSeqlen) return ESM_ATTN_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return ESM_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)T * H * d >= ((int64_t)1 << 31)) return ESM_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)H * d >= ((int64_t)1 << 24)) return ESM_ATTN_ERR_UNSUPPORTED;  // row stride
  if (schedule_num_chunks(B, H) + 1 >= ((int64_t)1 << 31)) return ESM_ATTN_ERR_UNSUPPORTED;
  if (schedule_slot_bound(B, T, H, maxL, kItemRows) >= ((int64_t)1 << 31))
    return ESM_ATTN_ERR_UNSUPPORTED;
  return ESM_ATTN_OK;
}

// Plan = rotary table + schedule. The one-shot calls append the rotated k~,
// q~ (except for a forward that rotates q itself), both [T][H][d] bf16, and
// for the backward drow ([H][T] entries of 16 bytes: -LSE log2 e, then -D,
// each split into three bf16 values).
Layout make_layout(int32_t B, int32_t T, int32_t maxL, int32_t H, int32_t d, bool bwd) {
  Layout l;
  l.n_chunks = (int32_t)schedule_num_chunks(B, H);
  l.n_slots = schedule_slot_bound(B, T, H, maxL, kItemRows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.rope = take((size_t)(maxL > 0 ? maxL : 1) * (d / 2) * sizeof(float2));
  l.sorted = take((size_t)B * sizeof(int32_t));
  l.chunk = take((size_t)(l.n_chunks + 1) * sizeof(int32_t));
  l.items = take((size_t)(l.n_slots > 0 ? l.n_slots : 1) * sizeof(Item));
  l.pos = take((size_t)(T > 0 ? T : 1) * sizeof(int32_t));
  l.plan = off;
  const size_t elems = (size_t)T * H * d;
  if (bwd || !fwd_rotates_q(d)) l.qrot = take(elems * sizeof(uint16_t));
  l.krot = take(elems * sizeof(uint16_t));
  if (bwd) l.drow = take((size_t)T * H * kDrowEntryBytes);
  l.total = off;
  return l;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// E4M3 per-tensor scales: finite, positive, with finite float32 reciprocals
// (the quantization multiplies by them).
esm_attn_status_t check_fp8_scales(float q_scale, float k_scale) {
  const float scales[] = {q_scale, k_scale};
  for (float x : scales)
    if (!(isfinite(x) && x > 0.f && isfinite(1.0f / x))) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  return ESM_ATTN_OK;
}

// A token row stride: at least H*d elements, rows 16-byte aligned, and every
// element offset below 2^31 (the kernels address rows with 32-bit offsets).
esm_attn_status_t check_stride(int32_t ld, int32_t T, int32_t H, int32_t d) {
  if (ld < H * d || ld % 8 != 0) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if ((int64_t)T * ld >= ((int64_t)1 << 31)) return ESM_ATTN_ERR_UNSUPPORTED;
  return ESM_ATTN_OK;
}

esm_attn_status_t check_scalars(float scale, float rope_base) {
  // the kernels work with |scale| * log2(e), which must stay finite too
  if (!isfinite(scale) || !isfinite(fabsf(scale) * kLog2e)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (!isfinite(rope_base) || rope_base < 0.f) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  return ESM_ATTN_OK;
}

void fill_common(AttnArgs* a, int32_t T, int32_t H, float scale) {
  a->T = T;
  a->H = H;
  a->scale = scale;
  a->q_sign = scale < 0.f ? -1.f : 1.f;  // (the bf16 kernels' q~ carries the sign)
}

// The one-shot calls take the small-batch path (one launch each, no plan,
// no rotation pass) when every sequence fits one 128-row work item.
bool small_path(int32_t max_seqlen, int32_t head_dim) {
  return max_seqlen <= kSmallMaxLen && head_dim <= 64;
}

AttnArgs small_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                    int32_t B, int32_t T, int32_t maxL, int32_t H, int32_t d, float scale,
                    float rope_base) {
  AttnArgs a = {};
  a.q = q;  // raw q and k: the small-path kernels rotate them
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.B = B;
  a.max_seqlen = maxL;
  a.rope_base = rope_base;
  a.q_mul = scale * kLog2e;  // as in esm_attn_rotate_planned
  a.ld_qkv = H * d;
  fill_common(&a, T, H, scale);
  return a;
}

esm_attn_status_t run_prep(const int32_t* cu, int32_t B, int32_t T, int32_t maxL, int32_t H,
                           int32_t d, float rope_base, const Layout& l, char* ws,
                           hipStream_t st) {
  PrepArgs p;
  p.cu = cu;
  p.B = B;
  p.T = T;
  p.H = H;
  p.max_seqlen = maxL;
  p.block = kItemRows;
  p.head_dim = d;
  p.sorted = reinterpret_cast<int32_t*>(ws + l.sorted);
  p.chunk_base = reinterpret_cast<int32_t*>(ws + l.chunk);
  p.n_chunks = l.n_chunks;
  p.items = reinterpret_cast<Item*>(ws + l.items);
  p.n_slots = l.n_slots;
  p.rope = rope_base != 0.f ? reinterpret_cast<float2*>(ws + l.rope) : nullptr;
  p.rope_base = rope_base;
  p.pos = reinterpret_cast<int32_t*>(ws + l.pos);
  return launch_prep(p, st) == hipSuccess ? ESM_ATTN_OK : ESM_ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t esm_attn_abi_version(void) { return ESM_ATTN_ABI_VERSION; }

const char* esm_attn_status_string(esm_attn_status_t s) {
  switch (s) {
    case ESM_ATTN_OK: return "esm_attn: success";
    case ESM_ATTN_ERR_INVALID_ARGUMENT: return "esm_attn: invalid argument";
    case ESM_ATTN_ERR_UNSUPPORTED: return "esm_attn: unsupported size or head_dim";
    case ESM_ATTN_ERR_WORKSPACE_TOO_SMALL: return "esm_attn: workspace too small";
    case ESM_ATTN_ERR_HIP: return "esm_attn: HIP launch failed";
    case ESM_ATTN_ERR_SCRATCH_TOO_SMALL:
      return "esm_attn: problem larger than the 128 MiB no-allocation scratch buffer";
    default: return "esm_attn: unknown status";
  }
}

size_t esm_attn_fwd_workspace_bytes(int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                                    int32_t num_heads, int32_t head_dim) {
  if (check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim) != ESM_ATTN_OK) return 0;
  return make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false).total;
}

size_t esm_attn_bwd_workspace_bytes(int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                                    int32_t num_heads, int32_t head_dim) {
  if (check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim) != ESM_ATTN_OK) return 0;
  return make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, true).total;
}

size_t esm_attn_plan_bytes(int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                           int32_t num_heads, int32_t head_dim) {
  if (check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim) != ESM_ATTN_OK) return 0;
  return make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false).plan;
}

esm_attn_status_t esm_attn_plan(const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                                int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                                float rope_base, void* plan, size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(0.f, rope_base)) != ESM_ATTN_OK) return s;
  if (total_tokens == 0 || max_seqlen == 0) return ESM_ATTN_OK;
  if (cu_seqlens == nullptr || !aligned16(cu_seqlens) || plan == nullptr || !aligned16(plan))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  return run_prep(cu_seqlens, batch, total_tokens, max_seqlen, num_heads, head_dim, rope_base, l,
                  static_cast<char*>(plan), reinterpret_cast<hipStream_t>(stream));
}

esm_attn_status_t esm_attn_rotate_planned(const uint16_t* q, const uint16_t* k,
                                          int32_t in_row_stride, int32_t batch,
                                          int32_t total_tokens, int32_t max_seqlen,
                                          int32_t num_heads, int32_t head_dim,
                                          float softmax_scale, float rope_base,
                                          uint16_t* q_rot, uint16_t* k_rot,
                                          int32_t out_row_stride, const void* plan,
                                          size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, rope_base)) != ESM_ATTN_OK) return s;
  if ((s = check_stride(in_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK ||
      (s = check_stride(out_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  // k alone: q and q_rot both null
  const bool k_only = q == nullptr && q_rot == nullptr;
  // in place: both outputs on their inputs (or k_rot on k alone), with the same stride
  const bool qin = k_only ? k_rot == k : q_rot == q, kin = k_rot == k;
  if (qin != kin || (qin && in_row_stride != out_row_stride)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {k, k_rot, plan, k_only ? k : q, k_only ? k_rot : q_rot};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  const char* ws = static_cast<const char*>(plan);
  RotArgs a = {};
  a.q = q;
  a.k = k;
  a.q_rot = q_rot;
  a.k_rot = k_rot;
  a.ld_in = in_row_stride;
  a.ld_out = out_row_stride;
  a.rope = reinterpret_cast<const float2*>(ws + l.rope);
  a.pos = reinterpret_cast<const int32_t*>(ws + l.pos);
  a.H = num_heads;
  a.T = total_tokens;
  a.max_pos = max_seqlen - 1;
  a.q_mul = softmax_scale * kLog2e;  // finite (check_scalars)
  if (launch_rotate(head_dim, rope_base != 0.f, a, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_fwd_planned(const uint16_t* q_rot, const uint16_t* k_rot,
                                       const uint16_t* v, int32_t qkv_row_stride, int32_t batch,
                                       int32_t total_tokens, int32_t max_seqlen,
                                       int32_t num_heads, int32_t head_dim, float softmax_scale,
                                       uint16_t* o, float* lse, const void* plan,
                                       size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, 0.f)) != ESM_ATTN_OK) return s;
  if ((s = check_stride(qkv_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q_rot, k_rot, v, o, lse, plan};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;  // every sequence is empty
  const char* ws = static_cast<const char*>(plan);
  AttnArgs a = {};
  a.q = q_rot;
  a.k = k_rot;
  a.v = v;
  a.out = o;
  a.lse = lse;
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  a.ld_qkv = qkv_row_stride;
  fill_common(&a, total_tokens, num_heads, softmax_scale);
  if (launch_fwd(head_dim, a, l.n_slots, false, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_fwd_rotq_planned(const uint16_t* q, const uint16_t* k_rot,
                                            const uint16_t* v, int32_t qkv_row_stride,
                                            int32_t batch, int32_t total_tokens,
                                            int32_t max_seqlen, int32_t num_heads,
                                            int32_t head_dim, float softmax_scale,
                                            float rope_base, uint16_t* o, float* lse,
                                            uint16_t* q_rot, const void* plan, size_t plan_bytes,
                                            void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, rope_base)) != ESM_ATTN_OK) return s;
  if ((s = check_stride(qkv_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q, k_rot, v, o, lse, plan};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (q_rot != nullptr && !aligned16(q_rot)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;  // every sequence is empty
  const char* ws = static_cast<const char*>(plan);
  AttnArgs a = {};
  a.q = q;  // raw: each item rotates its own query rows
  a.k = k_rot;
  a.v = v;
  a.out = o;
  a.lse = lse;
  a.q_out = q_rot;
  // the table region is always passed (the kernel loads from it unconditionally);
  // rope_base = 0 switches the rotation off
  a.rope = reinterpret_cast<const float2*>(ws + l.rope);
  a.rope_base = rope_base;
  a.q_mul = softmax_scale * kLog2e;  // as in esm_attn_rotate_planned
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  a.ld_qkv = qkv_row_stride;
  fill_common(&a, total_tokens, num_heads, softmax_scale);
  if (launch_fwd_rotq(head_dim, a, l.n_slots, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_fwd_split_planned(const uint16_t* q_rot, const uint16_t* k_rot,
                                             const uint16_t* v, int32_t qkv_row_stride,
                                             int32_t batch, int32_t total_tokens,
                                             int32_t max_seqlen, int32_t num_heads,
                                             int32_t head_dim, float softmax_scale,
                                             int32_t n_split, float* o_part, float* lse_part,
                                             uint16_t* o, float* lse, const void* plan,
                                             size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, 0.f)) != ESM_ATTN_OK) return s;
  if ((s = check_stride(qkv_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (n_split < 1 || n_split > kMaxSplit) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q_rot, k_rot, v, o_part, lse_part, o, lse, plan};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  const char* ws = static_cast<const char*>(plan);
  AttnArgs a = {};
  a.q = q_rot;
  a.k = k_rot;
  a.v = v;
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  a.ld_qkv = qkv_row_stride;
  a.n_split = n_split;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.n_items = (int32_t)l.n_slots;
  fill_common(&a, total_tokens, num_heads, softmax_scale);
  // grid x extent = slots padded to B*H modulo 8: chunk y of group g then
  // runs on XCD (g + y*B*H) mod 8 under round-robin dispatch
  const int64_t groups8 = ((int64_t)batch * num_heads) % 8;
  const int64_t grid_x = l.n_slots + ((groups8 - l.n_slots % 8) + 8) % 8;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (launch_fwd(head_dim, a, grid_x, true, st) != hipSuccess) return ESM_ATTN_ERR_HIP;
  if (launch_merge(head_dim, o_part, lse_part, n_split, total_tokens, num_heads, o, lse, st) !=
      hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_quantize_fp8_planned(const uint16_t* q, const uint16_t* k,
                                               int32_t in_row_stride, int32_t batch,
                                               int32_t total_tokens, int32_t max_seqlen,
                                               int32_t num_heads, int32_t head_dim,
                                               float rope_base, float q_scale, float k_scale,
                                               uint8_t* q8, uint8_t* k8, const void* plan,
                                               size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if (head_dim != 64 && head_dim != 128) return ESM_ATTN_ERR_UNSUPPORTED;
  if ((s = check_scalars(0.f, rope_base)) != ESM_ATTN_OK) return s;
  if ((s = check_fp8_scales(q_scale, k_scale)) != ESM_ATTN_OK) return s;
  const float q_inv = 1.0f / q_scale, k_inv = 1.0f / k_scale;
  if ((s = check_stride(in_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q, k, q8, k8, plan};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  const char* ws = static_cast<const char*>(plan);
  RotArgs a = {};
  a.q = q;
  a.k = k;
  a.ld_in = in_row_stride;
  a.q8 = q8;
  a.k8 = k8;
  a.q_inv = q_inv;
  a.k_inv = k_inv;
  a.rope = reinterpret_cast<const float2*>(ws + l.rope);
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  a.H = num_heads;
  if (launch_quantize_fp8(head_dim, rope_base != 0.f, a, l.n_slots,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_fwd_fp8_planned(const uint8_t* q8, const uint8_t* k8,
                                           const uint16_t* v, int32_t v_row_stride,
                                           int32_t batch, int32_t total_tokens,
                                           int32_t max_seqlen, int32_t num_heads,
                                           int32_t head_dim, float softmax_scale, float q_scale,
                                           float k_scale, uint16_t* o, float* lse,
                                           const void* plan, size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if (head_dim != 64 && head_dim != 128) return ESM_ATTN_ERR_UNSUPPORTED;
  if ((s = check_scalars(softmax_scale, 0.f)) != ESM_ATTN_OK) return s;
  if ((s = check_fp8_scales(q_scale, k_scale)) != ESM_ATTN_OK) return s;
  if (!isfinite(fabsf(softmax_scale) * kLog2e * q_scale * k_scale))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if ((s = check_stride(v_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q8, k8, v, o, lse, plan};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  const char* ws = static_cast<const char*>(plan);
  AttnArgs a = {};
  a.q8 = q8;
  a.k8 = k8;
  a.ld8 = num_heads * head_dim;
  a.v = v;
  a.ld_qkv = v_row_stride;
  a.out = o;
  a.lse = lse;
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  fill_common(&a, total_tokens, num_heads, softmax_scale);
  // scores come out of the E4M3 products in units of 1 / (s_q s_k). A floor
  // of 1e-30 keeps the exp2 factor positive, so that masked scores (-inf)
  // still give exp2(-inf) = 0 when softmax_scale is 0; below the floor every
  // |S c| rounds exp2 to exactly 1 either way.
  a.c = fmaxf(fabsf(softmax_scale) * kLog2e * q_scale * k_scale, 1e-30f);
  if (launch_fwd_fp8(head_dim, a, l.n_slots, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_merge_partials(const float* o_part, const float* lse_part,
                                          int32_t n_parts, int32_t total_tokens,
                                          int32_t num_heads, int32_t head_dim, uint16_t* o,
                                          float* lse, void* stream) {
  if (n_parts < 1 || n_parts > kMaxSplit || total_tokens < 0 || num_heads < 1)
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (!head_dim_ok(head_dim)) return ESM_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)total_tokens * num_heads * head_dim >= ((int64_t)1 << 31))
    return ESM_ATTN_ERR_UNSUPPORTED;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {o_part, lse_part, o, lse};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (launch_merge(head_dim, o_part, lse_part, n_parts, total_tokens, num_heads, o, lse,
                   reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_bwd_planned(const uint16_t* q_rot, const uint16_t* k_rot,
                                       const uint16_t* v, int32_t qkv_row_stride,
                                       const uint16_t* o, const uint16_t* d_o, const float* lse,
                                       int32_t batch, int32_t total_tokens, int32_t max_seqlen,
                                       int32_t num_heads, int32_t head_dim, float softmax_scale,
                                       float rope_base, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                       int32_t grad_row_stride, float* drow, int32_t passes,
                                       const void* plan, size_t plan_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, rope_base)) != ESM_ATTN_OK) return s;
  if ((s = check_stride(qkv_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK ||
      (s = check_stride(grad_row_stride, total_tokens, num_heads, head_dim)) != ESM_ATTN_OK)
    return s;
  if (passes < 1 || passes > (ESM_ATTN_PASS_DQ | ESM_ATTN_PASS_DKV))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const bool pdq = passes & ESM_ATTN_PASS_DQ, pdkv = passes & ESM_ATTN_PASS_DKV;
  const void* common[] = {q_rot, k_rot, v, d_o, drow, plan};
  for (const void* p : common)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (pdq && (o == nullptr || !aligned16(o) || lse == nullptr || !aligned16(lse) ||
              dq == nullptr || !aligned16(dq)))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (pdkv && (dk == nullptr || !aligned16(dk) || dv == nullptr || !aligned16(dv)))
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (plan_bytes < l.plan) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  const char* ws = static_cast<const char*>(plan);
  AttnArgs a = {};
  a.q = q_rot;
  a.k = k_rot;
  a.v = v;
  a.o = o;
  a.dout = d_o;
  a.lse_in = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.drow = drow;
  a.rope = reinterpret_cast<const float2*>(ws + l.rope);
  a.items = reinterpret_cast<const Item*>(ws + l.items);
  a.ld_qkv = qkv_row_stride;
  a.ld_grad = grad_row_stride;
  fill_common(&a, total_tokens, num_heads, softmax_scale);
  if (launch_bwd(head_dim, rope_base != 0.f, a, l.n_slots, pdq, pdkv,
                 reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return ESM_ATTN_ERR_HIP;
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                               int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                               float softmax_scale, float rope_base, uint16_t* o, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, rope_base)) != ESM_ATTN_OK) return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q, k, v, cu_seqlens, o, lse, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, false);
  if (workspace_bytes < l.total) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  if (small_path(max_seqlen, head_dim)) {
    AttnArgs a = small_args(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, num_heads,
                            head_dim, softmax_scale, rope_base);
    a.out = o;
    a.lse = lse;
    return launch_fwd_small(head_dim, a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ESM_ATTN_OK
               : ESM_ATTN_ERR_HIP;
  }
  char* ws = static_cast<char*>(workspace);
  uint16_t* kr = reinterpret_cast<uint16_t*>(ws + l.krot);
  if ((s = esm_attn_plan(cu_seqlens, batch, total_tokens, max_seqlen, num_heads, head_dim,
                         rope_base, ws, l.plan, stream)) != ESM_ATTN_OK)
    return s;
  const int32_t ld = num_heads * head_dim;
  if (fwd_rotates_q(head_dim)) {
    // k~ by the rotation pass; the forward rotates (and scales) its own query rows
    if ((s = esm_attn_rotate_planned(nullptr, k, ld, batch, total_tokens, max_seqlen, num_heads,
                                     head_dim, softmax_scale, rope_base, nullptr, kr, ld, ws,
                                     l.plan, stream)) != ESM_ATTN_OK)
      return s;
    return esm_attn_fwd_rotq_planned(q, kr, v, ld, batch, total_tokens, max_seqlen, num_heads,
                                     head_dim, softmax_scale, rope_base, o, lse, nullptr, ws,
                                     l.plan, stream);
  }
  uint16_t* qr = reinterpret_cast<uint16_t*>(ws + l.qrot);
  if ((s = esm_attn_rotate_planned(q, k, ld, batch, total_tokens, max_seqlen, num_heads,
                                   head_dim, softmax_scale, rope_base, qr, kr, ld, ws, l.plan,
                                   stream)) != ESM_ATTN_OK)
    return s;
  return esm_attn_fwd_planned(qr, kr, v, ld, batch, total_tokens, max_seqlen, num_heads,
                              head_dim, softmax_scale, o, lse, ws, l.plan, stream);
}

esm_attn_status_t esm_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* o, const uint16_t* d_o, const float* lse,
                               const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                               int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                               float softmax_scale, float rope_base, uint16_t* dq, uint16_t* dk,
                               uint16_t* dv, void* workspace, size_t workspace_bytes,
                               void* stream) {
  esm_attn_status_t s = check_sizes(batch, total_tokens, max_seqlen, num_heads, head_dim);
  if (s != ESM_ATTN_OK) return s;
  if ((s = check_scalars(softmax_scale, rope_base)) != ESM_ATTN_OK) return s;
  if (total_tokens == 0) return ESM_ATTN_OK;
  const void* ptrs[] = {q, k, v, o, d_o, lse, cu_seqlens, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const Layout l = make_layout(batch, total_tokens, max_seqlen, num_heads, head_dim, true);
  if (workspace_bytes < l.total) return ESM_ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (max_seqlen == 0) return ESM_ATTN_OK;
  if (small_path(max_seqlen, head_dim)) {
    AttnArgs a = small_args(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, num_heads,
                            head_dim, softmax_scale, rope_base);
    a.o = o;
    a.dout = d_o;
    a.lse_in = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.ld_grad = num_heads * head_dim;
    return launch_bwd_small(head_dim, a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? ESM_ATTN_OK
               : ESM_ATTN_ERR_HIP;
  }
  char* ws = static_cast<char*>(workspace);
  uint16_t* qr = reinterpret_cast<uint16_t*>(ws + l.qrot);
  uint16_t* kr = reinterpret_cast<uint16_t*>(ws + l.krot);
  if ((s = esm_attn_plan(cu_seqlens, batch, total_tokens, max_seqlen, num_heads, head_dim,
                         rope_base, ws, l.plan, stream)) != ESM_ATTN_OK)
    return s;
  const int32_t ld = num_heads * head_dim;
  // the rotation pass also applies softmax_scale log2(e) to q, so it runs
  // with the rotary embedding off too
  if ((s = esm_attn_rotate_planned(q, k, ld, batch, total_tokens, max_seqlen, num_heads,
                                   head_dim, softmax_scale, rope_base, qr, kr, ld, ws, l.plan,
                                   stream)) != ESM_ATTN_OK)
    return s;
  return esm_attn_bwd_planned(qr, kr, v, ld, o, d_o, lse, batch,
                              total_tokens, max_seqlen, num_heads, head_dim, softmax_scale,
                              rope_base, dq, dk, dv, ld, reinterpret_cast<float*>(ws + l.drow),
                              ESM_ATTN_PASS_DQ | ESM_ATTN_PASS_DKV, ws, l.plan, stream);
}

esm_attn_status_t esm_attn_check_cu_seqlens_host(const int32_t* cu, int32_t batch,
                                                 int32_t total_tokens, int32_t max_seqlen) {
  if (cu == nullptr || batch < 1 || total_tokens < 0 || max_seqlen < 0)
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (cu[0] != 0 || cu[batch] != total_tokens) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = (int64_t)cu[b + 1] - cu[b];
    if (L < 0 || L > max_seqlen) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  }
  return ESM_ATTN_OK;
}

esm_attn_status_t esm_attn_schedule_host(const int32_t* cu, int32_t batch, int32_t total_tokens,
                                         int32_t max_seqlen, int32_t num_heads,
                                         int32_t block_rows, int32_t* items,
                                         int32_t items_capacity, int32_t* n_slots) {
  if (cu == nullptr || items == nullptr || n_slots == nullptr || batch < 1 || num_heads < 1 ||
      total_tokens < 0 || max_seqlen < 0 || max_seqlen > kMaxSeqlen || block_rows < 16)
    return ESM_ATTN_ERR_INVALID_ARGUMENT;
  if (ceil_div64(max_seqlen, block_rows) + 1 > kMaxBuckets) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  const int64_t slots = schedule_slot_bound(batch, total_tokens, num_heads, max_seqlen, block_rows);
  if (slots > items_capacity) return ESM_ATTN_ERR_INVALID_ARGUMENT;
  *n_slots = (int32_t)slots;
  // sequences by item count, longest first (ties by index)
  std::vector<int32_t> nblk(batch), sorted;
  sorted.reserve(batch);
  for (int32_t b = 0; b < batch; ++b) {
    int32_t st, L;
    seq_bounds(cu, b, total_tokens, max_seqlen, &st, &L);
    nblk[b] = (L + block_rows - 1) / block_rows;
  }
  for (int32_t k = (int32_t)ceil_div64(max_seqlen, block_rows); k >= 0; --k)
    for (int32_t b = 0; b < batch; ++b)
      if (nblk[b] == k) sorted.push_back(b);
  const int32_t n_chunks = (int32_t)schedule_num_chunks(batch, num_heads);
  std::vector<int32_t> base(n_chunks + 1, 0);
  const int64_t groups = (int64_t)batch * num_heads;
  for (int32_t c = 0; c < n_chunks; ++c) {
    const int64_t g0 = 8 * (int64_t)c;
    const int64_t g1 = (g0 + 8 < groups ? g0 + 8 : groups) - 1;
    int32_t height = 0;
    for (int64_t s = g0 / num_heads; s <= g1 / num_heads; ++s)
      height = nblk[sorted[s]] > height ? nblk[sorted[s]] : height;
    base[c + 1] = base[c] + 8 * height;
  }
  for (int64_t i = 0; i < slots; ++i) {
    int32_t* it = items + 4 * i;
    if (!schedule_decode(i, cu, sorted.data(), base.data(), n_chunks, batch, total_tokens,
                         num_heads, max_seqlen, block_rows, it, it + 1, it + 2, it + 3)) {
      it[0] = it[1] = it[2] = it[3] = -1;
    }
  }
  return ESM_ATTN_OK;
}

}  // extern "C"
