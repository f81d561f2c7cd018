// Merge of key-range attention partials: with the softmax over the union of
// the ranges, exp(S_ij - LSE) = exp(LSE_r - LSE) P^r_ij, so
//   LSE = log sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r.
// Context parallelism deals the keys of one long sequence out to devices
// ("Scaling biomolecular modeling with context parallelism in NVIDIA BioNeMo"
// page, "2D tiling of the pairwise representation"); the same combination
// closes the split forward on one device.
//
// One thread per (token, head, 8 consecutive d values): R fp32 LSE loads, R
// 32-byte O loads (consecutive threads read consecutive 32-byte pieces of
// each partial, so every wave reads whole cache lines), one 16-byte bf16
// store. HBM-bound: R*(4d + 4) bytes read and 2d + 4 written per row.
#include "common.h"
#include "prep.h"

namespace esm {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    int n_parts, int T, int H,
                                                    uint16_t* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int CH = D / 8;  // 8-element chunks per row
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)T * H;
  if (u >= rows * CH) return;
  const int64_t row = u / CH;  // t * H + h
  const int c = (int)(u % CH);
  const int64_t t = row / H;
  const int h = (int)(row - t * H);
  // the largest LSE_r, then the weights exp(LSE_r - max)
  float mx = -INFINITY;
  for (int r = 0; r < n_parts; ++r) mx = fmaxf(mx, lse_part[((int64_t)r * H + h) * T + t]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx > -INFINITY) {
    for (int r = 0; r < n_parts; ++r) {
      const float lr = lse_part[((int64_t)r * H + h) * T + t];
      const float wr = fast_exp2((lr - mx) * kLog2e);  // 0 for an empty part
      const f32x4* p = reinterpret_cast<const f32x4*>(o_part + ((int64_t)r * rows + row) * D +
                                                      8 * c);
      const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(wr, x0[e], acc[e]);
        acc[4 + e] = fmaf(wr, x1[e], acc[4 + e]);
      }
      tot += wr;
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  st16(o + row * D + 8 * c, pack8(acc));
  if (c == 0) lse[(int64_t)h * T + t] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

template <int D>
static hipError_t launch_merge_d(const float* o_part, const float* lse_part, int n_parts, int T,
                                 int H, uint16_t* o, float* lse, hipStream_t stream) {
  const int64_t threads = (int64_t)T * H * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (blocks == 0) return hipSuccess;
  merge_kernel<D><<<blocks, 256, 0, stream>>>(o_part, lse_part, n_parts, T, H, o, lse);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const float* o_part, const float* lse_part, int n_parts,
                        int T, int H, uint16_t* o, float* lse, hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_merge_d<16>(o_part, lse_part, n_parts, T, H, o, lse, stream);
    case 32: return launch_merge_d<32>(o_part, lse_part, n_parts, T, H, o, lse, stream);
    case 64: return launch_merge_d<64>(o_part, lse_part, n_parts, T, H, o, lse, stream);
    case 128: return launch_merge_d<128>(o_part, lse_part, n_parts, T, H, o, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace esm
