// Rotary position embedding of q and k, once per token: x~ = bf16(R(p) x).
// The attention kernels then read q~ and k~ directly (a key block is used by
// every query block of its sequence, so rotating it inside those kernels
// would redo the same rotation once per query block).
//
// R(p) turns the pairs (x_j, x_{j+d/2}) by p * theta_j with the float32
// (cos, sin) table of the plan; products and sums are rounded to float32 one
// by one (rotate8) and the result is rounded once to bf16 (round to nearest
// even). Rotary embedding as in RoFormer (Su et al. 2021), with x_j paired
// with x_{j+d/2}. With no rotary table (rope_base = 0) the kernel copies.
// Every element is read and written by one thread, loads first, so the
// outputs may be the inputs themselves (rotation in place).
#include "common.h"
#include "prep.h"

namespace esm {

constexpr int kRotSplit = 2;  // workgroups per 128-row item

// Workgroup (x, y) rotates rows [blk * 128 + y * RR, blk * 128 + (y + 1) * RR)
// (RR = 128 / kRotSplit) of the (sequence, head) of schedule slot x, q and k:
// one 8-pair chunk (16 bytes of the low half, 16 of the high half) per
// thread and tensor, all loads issued before any arithmetic. Many small
// workgroups keep enough loads in flight to stream at close to copy speed
// (grouping several heads per workgroup to share the cos/sin loads measured
// slower: fewer loads in flight).
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void rotate_kernel(RotArgs a) {
  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  constexpr int UPR = D / 16;                        // 8-pair chunks per row
  constexpr int RR = kItemRows / kRotSplit;          // rows per workgroup
  constexpr int NU = (RR * UPR + 255) / 256;         // units per thread
  const int r0 = it.blk * kItemRows + blockIdx.y * RR;
  const int n = min(RR, it.len - r0) * UPR;          // may be <= 0
  const int64_t bin = (int64_t)it.seq0 * a.ld_in + (int64_t)it.head * D;
  const int64_t bout = (int64_t)it.seq0 * a.ld_out + (int64_t)it.head * D;
  u32x4 ql[NU], qh[NU], kl[NU], kh[NU];
  float2 cs[NU][8];
#pragma unroll
  for (int x = 0; x < NU; ++x) {
    const int u = threadIdx.x + 256 * x;
    if (u < n) {
      const int row = u / UPR, j0 = (u % UPR) * 8, pos = r0 + row;
      const int64_t off = bin + (int64_t)pos * a.ld_in + j0;
      ql[x] = ld16(a.q + off);
      qh[x] = ld16(a.q + off + D / 2);
      kl[x] = ld16(a.k + off);
      kh[x] = ld16(a.k + off + D / 2);
      if (ROPE) load_cs8(a.rope, pos * (D / 2) + j0, cs[x]);
    }
  }
#pragma unroll
  for (int x = 0; x < NU; ++x) {
    const int u = threadIdx.x + 256 * x;
    if (u < n) {
      const int row = u / UPR, j0 = (u % UPR) * 8, pos = r0 + row;
      const int64_t off = bout + (int64_t)pos * a.ld_out + j0;
      u32x4 q0 = ql[x], q1 = qh[x], k0 = kl[x], k1 = kh[x];
      if (ROPE) {
        float lo[8], hi[8];
        unpack8(q0, lo);
        unpack8(q1, hi);
        rotate8<false, false>(lo, hi, cs[x]);
        q0 = pack8(lo);
        q1 = pack8(hi);
        unpack8(k0, lo);
        unpack8(k1, hi);
        rotate8<false, false>(lo, hi, cs[x]);
        k0 = pack8(lo);
        k1 = pack8(hi);
      }
      st16(a.q_rot + off, q0);
      st16(a.q_rot + off + D / 2, q1);
      st16(a.k_rot + off, k0);
      st16(a.k_rot + off + D / 2, k1);
    }
  }
}

// E4M3 quantization of the rotated q and k for the FP8 forward: the same
// work split and rotation as rotate_kernel (float32, products and sums
// rounded one by one), then x * fl32(1 / scale) in float32, clamped to
// [-448, 448] (E4M3 has no infinity) and rounded once to E4M3, nearest even.
// Each thread writes 8 + 8 bytes per tensor.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(RotArgs a) {
  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  constexpr int UPR = D / 16;
  constexpr int RR = kItemRows / kRotSplit;
  constexpr int NU = (RR * UPR + 255) / 256;
  const int r0 = it.blk * kItemRows + blockIdx.y * RR;
  const int n = min(RR, it.len - r0) * UPR;
  const int64_t bin = (int64_t)it.seq0 * a.ld_in + (int64_t)it.head * D;
  const int64_t bout = ((int64_t)it.seq0 * a.H + it.head) * D;  // bytes, packed [T][H][d]
  u32x4 ql[NU], qh[NU], kl[NU], kh[NU];
  float2 cs[NU][8];
#pragma unroll
  for (int x = 0; x < NU; ++x) {
    const int u = threadIdx.x + 256 * x;
    if (u < n) {
      const int row = u / UPR, j0 = (u % UPR) * 8, pos = r0 + row;
      const int64_t off = bin + (int64_t)pos * a.ld_in + j0;
      ql[x] = ld16(a.q + off);
      qh[x] = ld16(a.q + off + D / 2);
      kl[x] = ld16(a.k + off);
      kh[x] = ld16(a.k + off + D / 2);
      if (ROPE) load_cs8(a.rope, pos * (D / 2) + j0, cs[x]);
    }
  }
  auto q8 = [](const float* f, float inv) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(f[e] * inv, -448.f), 448.f);
    return u32x2{pack_fp8x4(y[0], y[1], y[2], y[3]), pack_fp8x4(y[4], y[5], y[6], y[7])};
  };
#pragma unroll
  for (int x = 0; x < NU; ++x) {
    const int u = threadIdx.x + 256 * x;
    if (u < n) {
      const int row = u / UPR, j0 = (u % UPR) * 8, pos = r0 + row;
      const int64_t off = bout + (int64_t)pos * a.H * D + j0;
      float lo[8], hi[8];
      unpack8(ql[x], lo);
      unpack8(qh[x], hi);
      if (ROPE) rotate8<false, false>(lo, hi, cs[x]);
      *reinterpret_cast<u32x2*>(a.q8 + off) = q8(lo, a.q_inv);
      *reinterpret_cast<u32x2*>(a.q8 + off + D / 2) = q8(hi, a.q_inv);
      unpack8(kl[x], lo);
      unpack8(kh[x], hi);
      if (ROPE) rotate8<false, false>(lo, hi, cs[x]);
      *reinterpret_cast<u32x2*>(a.k8 + off) = q8(lo, a.k_inv);
      *reinterpret_cast<u32x2*>(a.k8 + off + D / 2) = q8(hi, a.k_inv);
    }
  }
}

template <int D>
static hipError_t launch_rotate_d(bool rope, const RotArgs& a, int64_t n_slots, hipStream_t st) {
  const dim3 grid((unsigned)n_slots, kRotSplit);
  if (rope)
    rotate_kernel<D, true><<<grid, 256, 0, st>>>(a);
  else
    rotate_kernel<D, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_rotate(int head_dim, bool rope, const RotArgs& a, int64_t n_slots,
                         hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_rotate_d<16>(rope, a, n_slots, stream);
    case 32: return launch_rotate_d<32>(rope, a, n_slots, stream);
    case 64: return launch_rotate_d<64>(rope, a, n_slots, stream);
    case 128: return launch_rotate_d<128>(rope, a, n_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_fp8(int head_dim, bool rope, const RotArgs& a, int64_t n_slots,
                               hipStream_t stream) {
  const dim3 grid((unsigned)n_slots, kRotSplit);
  switch (head_dim) {
    case 64:
      if (rope) quantize_fp8_kernel<64, true><<<grid, 256, 0, stream>>>(a);
      else quantize_fp8_kernel<64, false><<<grid, 256, 0, stream>>>(a);
      break;
    case 128:
      if (rope) quantize_fp8_kernel<128, true><<<grid, 256, 0, stream>>>(a);
      else quantize_fp8_kernel<128, false><<<grid, 256, 0, stream>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace esm
