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
#include "common.h"
#include "prep.h"

namespace esm {

// One workgroup per schedule slot: rows [blk * 128, blk * 128 + 128) of one
// (sequence, head), both tensors.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void rotate_kernel(RotArgs a) {
  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int rs = a.H * D;
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)it.head * D;
  const int r0 = it.blk * kItemRows;
  const int rows = min(kItemRows, it.len - r0);
  for (int u = threadIdx.x; u < rows * (D / 16); u += 256) {
    const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, pos = r0 + row;
    const int64_t off = base + (int64_t)pos * rs + j0;
    const u32x4 ql = ld16(a.q + off), qh = ld16(a.q + off + D / 2);
    const u32x4 kl = ld16(a.k + off), kh = ld16(a.k + off + D / 2);
    if (ROPE) {
      float2 cs[8];
      load_cs8(a.rope, pos * (D / 2) + j0, cs);
      float lo[8], hi[8];
      unpack8(ql, lo);
      unpack8(qh, hi);
      rotate8<false, false>(lo, hi, cs);
      st16(a.q_rot + off, pack8(lo));
      st16(a.q_rot + off + D / 2, pack8(hi));
      unpack8(kl, lo);
      unpack8(kh, hi);
      rotate8<false, false>(lo, hi, cs);
      st16(a.k_rot + off, pack8(lo));
      st16(a.k_rot + off + D / 2, pack8(hi));
    } else {
      st16(a.q_rot + off, ql);
      st16(a.q_rot + off + D / 2, qh);
      st16(a.k_rot + off, kl);
      st16(a.k_rot + off + D / 2, kh);
    }
  }
}

template <int D>
static hipError_t launch_rotate_d(bool rope, const RotArgs& a, int64_t n_slots, hipStream_t st) {
  if (rope)
    rotate_kernel<D, true><<<(unsigned)n_slots, 256, 0, st>>>(a);
  else
    rotate_kernel<D, false><<<(unsigned)n_slots, 256, 0, st>>>(a);
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

}  // namespace esm
