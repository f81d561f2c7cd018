// Per-call preparation kernels: the varlen schedule (see schedule.h) and the
// rotary cos/sin table.
#include "common.h"
#include "prep.h"
#include "schedule.h"

namespace esm {

// Inclusive prefix sum over the 1024 threads of the workgroup: in-register
// within each wave, then over the 16 wave totals. wsum: 16 ints of LDS.
// Every thread must call it; it ends with a barrier.
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int32_t x = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int32_t t = __shfl_up(x, off);
      if (lane >= off) x += t;
    }
    if (lane < 16) wsum[lane] = x;
  }
  __syncthreads();
  if (wid > 0) v += wsum[wid - 1];
  __syncthreads();  // wsum may be reused by the next call
  return v;
}

constexpr int kPlanCache = 4096;  // batches up to this size keep cu and the order in LDS

// One workgroup of 1024 threads. Sorts sequences by item count, longest first
// (counting sort over item counts; order inside a count is arbitrary and
// irrelevant to the results), then writes the chunk bases. For batches of up
// to kPlanCache sequences cu_seqlens and the sorted order live in LDS, so the
// only global-memory round trips are the first read and the final writes.
__global__ __launch_bounds__(1024) void schedule_plan_kernel(
    const int32_t* __restrict__ cu, int32_t B, int32_t T, int32_t H, int32_t max_seqlen,
    int32_t block, int32_t n_buckets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ chunk_base, int32_t n_chunks) {
  __shared__ int32_t hist[kMaxBuckets];
  __shared__ int32_t start[kMaxBuckets];
  __shared__ int32_t cu_s[kPlanCache + 1];
  __shared__ int32_t sorted_s[kPlanCache];
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const bool cached = B <= kPlanCache;
  if (cached)
    for (int i = tid; i <= B; i += 1024) cu_s[i] = cu[i];
  const int32_t* cuv = cached ? cu_s : cu;
  int32_t* srt = cached ? sorted_s : sorted;

  for (int i = tid; i < n_buckets; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += 1024) {
    int32_t s, L;
    seq_bounds(cuv, b, T, max_seqlen, &s, &L);
    atomicAdd(&hist[(L + block - 1) / block], 1);
  }
  __syncthreads();

  // start[k] = number of sequences with more than k items. Thread t owns the
  // four buckets of descending rank 4t .. 4t+3.
  {
    int32_t own = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = n_buckets - 1 - (4 * tid + j);
      if (k >= 0) own += hist[k];
    }
    int32_t run = block_inclusive_scan(own, wsum) - own;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = n_buckets - 1 - (4 * tid + j);
      if (k >= 0) {
        start[k] = run;
        run += hist[k];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < n_buckets; i += 1024) hist[i] = 0;  // reuse as cursors
  __syncthreads();
  for (int b = tid; b < B; b += 1024) {
    int32_t s, L;
    seq_bounds(cuv, b, T, max_seqlen, &s, &L);
    const int k = (L + block - 1) / block;
    srt[start[k] + atomicAdd(&hist[k], 1)] = b;
  }
  if (!cached) __threadfence();
  __syncthreads();
  if (cached)
    for (int i = tid; i < B; i += 1024) sorted[i] = sorted_s[i];

  // chunk heights -> exclusive prefix (chunk_base), 1024 chunks per round
  if (tid == 0) carry = 0;
  __syncthreads();
  const int64_t groups = (int64_t)B * H;
  for (int32_t c0 = 0; c0 < n_chunks; c0 += 1024) {
    const int32_t c = c0 + tid;
    int32_t height = 0;
    if (c < n_chunks) {
      const int64_t g0 = 8 * (int64_t)c;
      const int64_t g1 = (g0 + 8 < groups ? g0 + 8 : groups) - 1;
      for (int64_t s = g0 / H; s <= g1 / H; ++s) {
        int32_t st, L;
        seq_bounds(cuv, srt[s], T, max_seqlen, &st, &L);
        const int32_t n = (L + block - 1) / block;
        height = n > height ? n : height;
      }
    }
    const int32_t incl = block_inclusive_scan(8 * height, wsum);
    const int32_t cbase = carry;
    if (c < n_chunks) chunk_base[c] = cbase + incl - 8 * height;
    __syncthreads();  // every thread has read carry
    if (tid == 1023) carry = cbase + incl;
    __syncthreads();
  }
  if (tid == 0) chunk_base[n_chunks] = carry;
}

// blockIdx.y == 0: decode slots into Item records.
// blockIdx.y == 1: rotary table, table[p * (d/2) + j] = (cos, sin)(p * theta_j),
// theta_j = base^(-2j/d), evaluated in fp64 and rounded once to fp32.
__global__ __launch_bounds__(256) void schedule_fill_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ chunk_base, int32_t n_chunks, int32_t B, int32_t T, int32_t H,
    int32_t max_seqlen, int32_t block, Item* __restrict__ items, int64_t n_slots,
    float2* __restrict__ rope, int32_t head_dim, double rope_base, int32_t* __restrict__ pos,
    int32_t pos_chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.y == 2) {
    // token positions: workgroup x covers tokens 256 c .. 256 c + 255 of
    // sequence b (x = b * pos_chunks + c). Every token of a valid cu_seqlens
    // belongs to exactly one sequence; the readers clamp whatever they read
    // to [0, max_seqlen), so a bad cu_seqlens cannot make them index out of
    // the rotary table.
    const int64_t b = blockIdx.x / pos_chunks;
    if (b >= B) return;
    const int32_t c = (int32_t)(blockIdx.x - b * pos_chunks);
    int32_t st, L;
    seq_bounds(cu, (int32_t)b, T, max_seqlen, &st, &L);
    const int32_t p = 256 * c + (int32_t)threadIdx.x;
    if (p < L) pos[st + p] = p;
    return;
  }
  if (blockIdx.y == 0) {
    if (i >= n_slots) return;
    Item it;
    if (!schedule_decode(i, cu, sorted, chunk_base, n_chunks, B, T, H, max_seqlen, block,
                         &it.seq0, &it.len, &it.head, &it.blk)) {
      it.seq0 = -1;
      it.len = -1;
      it.head = -1;
      it.blk = -1;
    }
    items[i] = it;
  } else {
    const int32_t half = head_dim / 2;
    if (rope == nullptr || i >= (int64_t)max_seqlen * half) return;
    const int32_t p = (int32_t)(i / half);
    const int32_t j = (int32_t)(i - (int64_t)p * half);
    rope[i] = rope_base != 0.0 ? rope_cs(p, j, head_dim, rope_base) : make_float2(1.0f, 0.0f);
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
  const int32_t n_buckets = (int32_t)ceil_div64(a.max_seqlen, a.block) + 1;
  schedule_plan_kernel<<<1, 1024, 0, stream>>>(a.cu, a.B, a.T, a.H, a.max_seqlen, a.block,
                                               n_buckets, a.sorted, a.chunk_base, a.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t table = (int64_t)a.max_seqlen * (a.head_dim / 2);
  const int32_t pos_chunks = (int32_t)ceil_div64(a.max_seqlen > 0 ? a.max_seqlen : 1, 256);
  const int64_t pos_wgs = (int64_t)a.B * pos_chunks;
  int64_t wgs = ceil_div64(a.n_slots > table ? a.n_slots : table, 256);
  if (pos_wgs > wgs) wgs = pos_wgs;
  dim3 grid((unsigned)(wgs > 0 ? wgs : 1), 3);
  schedule_fill_kernel<<<grid, 256, 0, stream>>>(a.cu, a.sorted, a.chunk_base, a.n_chunks, a.B,
                                                 a.T, a.H, a.max_seqlen, a.block, a.items,
                                                 a.n_slots, a.rope, a.head_dim, a.rope_base,
                                                 a.pos, pos_chunks);
  return hipGetLastError();
}

}  // namespace esm
