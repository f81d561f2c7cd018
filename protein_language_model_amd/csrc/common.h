// Shared device helpers for the gfx950 attention kernels: bf16 packing, the
// 32x32x16 bf16 MFMA, register layouts, rotary rotation of 8-element chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace esm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Work item of one workgroup, written by the scheduler: the packed token
// offset of the sequence, its length, the head and the row-block index.
// len <= 0 marks an idle slot.
struct Item {
  int32_t seq0, len, head, blk;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
  return v;
}

__device__ __forceinline__ u32x4 zero4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Register layouts (wave64, lane l, r = l % 32, g = l / 32):
//   A: lane holds row r, 8 values along k;  B: lane holds column r, the same
//   8 k positions. Any assignment of the 16 k positions to (g, slot) works as
//   long as A and B use the same one, which is how every caller feeds them.
//   D: register i of lane l holds row (i/4)*8 + g*4 + (i%4), column r.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// If A-operand row r is loaded from logical row perm_row(r), accumulator
// register i of lane half g holds logical row 16*g + i: each lane then owns 16
// consecutive logical rows.
__device__ __forceinline__ int perm_row(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotary rotation of the pair of 8-element chunks (x_j..x_j+7) and
// (x_{j+d/2}..x_{j+d/2}+7) by the angles whose float32 (cos, sin) pairs are
// cs[0..7]: x' = x c - y s, y' = y c + x s, every product and sum rounded to
// float32 (no fused multiply-add), so that the later rounding of x' and y' to
// bf16 is decided on exactly the float32 values a plain float32 evaluation
// gives. inverse rotates by the negative angles (the transpose). The results
// are multiplied by mul (+1 or -1, exact).
__device__ __forceinline__ void rotate8(float* lo, float* hi, const float2* cs, bool inverse,
                                        float mul) {
#pragma clang fp contract(off)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = cs[e].x;
    const float s = inverse ? -cs[e].y : cs[e].y;
    const float x = lo[e], y = hi[e];
    const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
    lo[e] = (xc - ys) * mul;
    hi[e] = (yc + xs) * mul;
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace esm
