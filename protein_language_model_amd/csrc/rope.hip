// Rotary position embedding of q and k, once per token:
//   k~ = bf16(R(p) k),   q~ = bf16(fl32(c * fl32(R(p) q))),  c = fl32(scale log2 e).
// The attention kernels then read q~ and k~ directly (a key block is used by
// every query block of its sequence, so rotating it inside those kernels
// would redo the same rotation once per query block), and q~ . k~ is the
// score in log2 units, ready for exp2 (the kernels fold the subtraction of
// the row reference into their MFMAs, so no per-score multiply is left).
//
// R(p) turns the pairs (x_j, x_{j+d/2}) by p * theta_j with the float32
// (cos, sin) table of the plan; products and sums are rounded to float32 one
// by one (rotate8) and the result is rounded once to bf16 (round to nearest
// even). Rotary embedding as in RoFormer (Su et al. 2021), with x_j paired
// with x_{j+d/2}. With no rotary table (rope_base = 0) R is the identity.
// Every element is read and written by one thread, loads first, so the
// outputs may be the inputs themselves (rotation in place).
#include "common.h"
#include "prep.h"

namespace esm {

constexpr int kRotSplit = 2;  // workgroups per 128-row item (quantization pass)
constexpr int kRotUnits = 4;  // 8-pair units per thread (rotation pass)

// Rotation pass, token-major: unit u (8 rotary pairs: 16 bytes of the low
// half and 16 bytes of the high half of one head row) is token
// u / (H d/16), head and pair offset from the rest, so consecutive threads
// read consecutive bytes of whole token rows (every head of a token in one
// stretch of memory) and the cos/sin row of a position is reused by every
// head of the token. Each thread issues the loads of kRotUnits units before
// any arithmetic. Positions come from the plan (clamped into the table).
// Q false: k alone (the forward that rotates its own query rows needs k~ only).
template <int D, bool ROPE, bool Q>
__global__ __launch_bounds__(256) void rotate_kernel(RotArgs a) {
  constexpr int UPR = D / 16;  // units per head row
  const int upt = a.H * UPR;   // units per token
  const int64_t total = (int64_t)a.T * upt;
  const int64_t u0 = (int64_t)blockIdx.x * 256 * kRotUnits + threadIdx.x;
  u32x4 ql[kRotUnits], qh[kRotUnits], kl[kRotUnits], kh[kRotUnits];
  float2 cs[kRotUnits][8];
  int64_t offo[kRotUnits];
#pragma unroll
  for (int x = 0; x < kRotUnits; ++x) {
    const int64_t u = u0 + 256 * x;
    if (u < total) {
      const int64_t t = u / upt;
      const int rest = (int)(u - t * upt);
      const int h = rest / UPR, j0 = (rest % UPR) * 8;
      const int64_t off = t * a.ld_in + h * D + j0;
      offo[x] = t * a.ld_out + h * D + j0;
      if (Q) {
        ql[x] = ld16(a.q + off);
        qh[x] = ld16(a.q + off + D / 2);
      }
      kl[x] = ld16(a.k + off);
      kh[x] = ld16(a.k + off + D / 2);
      if (ROPE) {
        const int p = min(max(a.pos[t], 0), a.max_pos);
        load_cs8(a.rope, (int64_t)p * (D / 2) + j0, cs[x]);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < kRotUnits; ++x) {
    const int64_t u = u0 + 256 * x;
    if (u < total) {
      u32x4 k0 = kl[x], k1 = kh[x];
      float lo[8], hi[8];
      if (Q) {
        unpack8(ql[x], lo);
        unpack8(qh[x], hi);
        if (ROPE) rotate8<false, false>(lo, hi, cs[x]);
        // q~ = bf16(fl32(q_mul * fl32(R(p) q))): one more fp32 rounding, then one to bf16
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] *= a.q_mul;
          hi[e] *= a.q_mul;
        }
        st16(a.q_rot + offo[x], pack8(lo));
        st16(a.q_rot + offo[x] + D / 2, pack8(hi));
      }
      if (ROPE) {
        unpack8(k0, lo);
        unpack8(k1, hi);
        rotate8<false, false>(lo, hi, cs[x]);
        k0 = pack8(lo);
        k1 = pack8(hi);
      }
      st16(a.k_rot + offo[x], k0);
      st16(a.k_rot + offo[x] + D / 2, k1);
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
static hipError_t launch_rotate_d(bool rope, const RotArgs& a, hipStream_t st) {
  const int64_t units = (int64_t)a.T * a.H * (D / 16);
  const unsigned grid = (unsigned)((units + 256 * kRotUnits - 1) / (256 * kRotUnits));
  if (grid == 0) return hipSuccess;
  const bool q = a.q_rot != nullptr;
  if (rope && q)
    rotate_kernel<D, true, true><<<grid, 256, 0, st>>>(a);
  else if (q)
    rotate_kernel<D, false, true><<<grid, 256, 0, st>>>(a);
  else if (rope)
    rotate_kernel<D, true, false><<<grid, 256, 0, st>>>(a);
  else
    rotate_kernel<D, false, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_rotate(int head_dim, bool rope, const RotArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_rotate_d<16>(rope, a, stream);
    case 32: return launch_rotate_d<32>(rope, a, stream);
    case 64: return launch_rotate_d<64>(rope, a, stream);
    case 128: return launch_rotate_d<128>(rope, a, stream);
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
