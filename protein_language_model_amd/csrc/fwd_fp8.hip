// FP8 forward attention for gfx950 (inference first): the scores
// S^T = K8 Q8^T run on the 32x32x64 E4M3 matrix instruction from q~ and k~
// quantized once per token (quantize_fp8_kernel, rope.hip: q8 = E4M3(q~ /
// s_q), per-tensor scales); softmax, P (bf16) and O += P V (bf16 V) are those
// of the bf16 forward (fwd.hip), so the kernel's only extra error against
// an oracle on the same E4M3 operands is the bf16 forward's. The BioNeMo
// Recipes hub page lists FP8 among its training precisions (multi-precision
// training section); this variant covers the forward.
//
// Differences from the bf16 forward: a key block's k8 tile is half the bytes
// (rows of d bytes, copied by global_load_lds like a bf16 tile of d/2
// columns, same swizzle), the per-lane queries are 32 bytes per 64-wide
// k-step (d/64 steps), and one E4M3 instruction covers 64 d values where the
// bf16 path needs four. The k8 and v tiles have different shapes and
// strides, so they are copied as two single tiles. head_dim 64 or 128.
#include "common.h"
#include "prep.h"
#include "tile.h"

namespace esm {

template <int D>
struct Fp8Cfg {
  static constexpr int BM = 128;                  // queries per item
  static constexpr int BN = D == 128 ? 32 : 64;   // keys per block
  static constexpr int NS8 = D / 64;              // E4M3 k-steps over d
  static constexpr int ND = D / 32;               // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;              // 32-key tiles per block
  static constexpr int NU = BN / 16;              // bf16 k-steps over keys (P V)
  static constexpr int KTILE = BN * D / 2;        // k8 tile, in uint16 units
  static constexpr int VTILE = BN * D;            // v tile
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int NSTAGE = 3;
  static constexpr int LDS = NSTAGE * STAGE;
  static constexpr int OCC = D == 128 ? 2 : 3;
  using LoaderK = TilePair<D / 2, BN>;            // k8 rows as d/2 uint16
  using LoaderV = TilePair<D, BN>;
  static constexpr int LOADS = LoaderK::PER_TILE + LoaderV::PER_TILE;  // per wave and block
};

constexpr float kLazyBound8 = 65536.0f;  // largest block sum of P kept (as fwd.hip)

template <int D>
__global__ __launch_bounds__(256, Fp8Cfg<D>::OCC) void fwd_fp8_kernel(AttnArgs a) {
  using C = Fp8Cfg<D>;
  static_assert(D == 64 || D == 128, "E4M3 forward: head_dim 64 or 128");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, q0 = it.blk * C::BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  const int rs8 = a.ld8 / 2;  // q8/k8 row stride in uint16 units (ld8 bytes, even)
  const int rsv = a.ld_qkv;   // v row stride; T * stride < 2^31 is checked on the host
  const uint16_t* __restrict__ Kg =
      reinterpret_cast<const uint16_t*>(a.k8 + (int64_t)it.seq0 * a.ld8 + (int64_t)h * D);
  const uint16_t* __restrict__ Vg = a.v + (int64_t)it.seq0 * rsv + (int64_t)h * D;
  const uint8_t* __restrict__ Qg = a.q8 + (int64_t)it.seq0 * a.ld8 + (int64_t)h * D;

  // k8 and v rows of key block kb -> LDS stage `stage`
  const typename C::LoaderK lk(w, lane);
  const typename C::LoaderV lv(w, lane);
  const typename C::LoaderK::Offsets koff = lk.offsets(rs8, w);
  const typename C::LoaderV::Offsets voff = lv.offsets(rsv, w);
  auto issue = [&](int kb, int stage) {
    const int k0 = kb * C::BN;
    uint16_t* Ks = lds + stage * C::STAGE;
    if (k0 + C::BN <= L) {
      lk.load_full_one(Kg + (int64_t)k0 * rs8, koff, Ks, w);
      lv.load_full_one(Vg + (int64_t)k0 * rsv, voff, Ks + C::KTILE, w);
    } else {
      lk.template load_one<1>(Kg + (int64_t)k0 * rs8, rs8, L - k0, Ks, w);
      lv.template load_one<1>(Vg + (int64_t)k0 * rsv, rsv, L - k0, Ks + C::KTILE, w);
    }
  };
  const int nkb = (L + C::BN - 1) / C::BN;
  issue(0, 0);

  // queries: 32 bytes per k-step (d values 64s + 32g ..), zero past the end;
  // a negative softmax scale flips the sign bit of every q8 byte (exact)
  const int qi = q0 + w * 32 + r;
  const bool live = q0 + w * 32 < L;  // wave-uniform
  // (branch-free loads of a clamped row, as in the bf16 forward)
  const uint32_t qflip = a.q_sign < 0.f ? 0x80808080u : 0u;
  const int qc = min(qi, L - 1);
  u32x4 qreg[C::NS8][2];
#pragma unroll
  for (int s = 0; s < C::NS8; ++s)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      qreg[s][hh] = ld16(Qg + (int64_t)qc * a.ld8 + 64 * s + 32 * g + 16 * hh);
#pragma unroll
  for (int s = 0; s < C::NS8; ++s)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[s][hh][e] = qi < L ? qreg[s][hh][e] ^ qflip : 0u;
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nkb) issue(j, j);

  const float c = a.c;  // |scale| s_q s_k log2(e)
  const TrRows<D> vread(lane);
  float m = 0.f, mc = 0.f, l = 0.f;
  f32x16 oacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) oacc[dt] = f32x16{};

  int stage = 0, next = C::NSTAGE - 1;
  auto block = [&](int kb, auto full) {
    constexpr bool FULL = decltype(full)::value;
    if (C::NSTAGE == 3 && kb + 1 < nkb)
      wait_vmem<C::LOADS>();
    else
      wait_vmem<0>();
    block_barrier();
    if (kb + C::NSTAGE - 1 < nkb) issue(kb + C::NSTAGE - 1, next);
    const uint16_t* Ks = lds + stage * C::STAGE;
    const uint16_t* Vs = Ks + C::KTILE;
    stage = stage + 1 == C::NSTAGE ? 0 : stage + 1;
    next = next + 1 == C::NSTAGE ? 0 : next + 1;
    // a wave whose 32 rows all lie past the end of the sequence (the last,
    // partly filled item of a sequence) only takes part in the copies and the
    // barrier: its MFMA and vector work would produce nothing that is stored
    if (!live) return;

    const int lim = L - kb * C::BN;
    f32x16 sacc[C::NT];
    // S^T tile t: k8 row 32t + perm_row(r), 16-byte chunks 4s + 2g and
    // 4s + 2g + 1 of k-step s (the tile is a d/2-column uint16 tile)
    auto scores = [&]() {
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        sacc[t] = f32x16{};
        const int row = 32 * t + prow;
#pragma unroll
        for (int s = 0; s < C::NS8; ++s)
          sacc[t] = mfma32_fp8(ld16(Ks + tile_off<D / 2>(row, 4 * s + 2 * g)),
                               ld16(Ks + tile_off<D / 2>(row, 4 * s + 2 * g + 1)), qreg[s][0],
                               qreg[s][1], sacc[t]);
      }
      if (!FULL) {
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[t][i] = (32 * t + 16 * g + i < lim) ? sacc[t][i] : -INFINITY;
      }
    };
    auto block_max = [&]() {
      float mx = sacc[0][0];
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[t][i]);
      return fmaxf(mx, xor32(mx));
    };
    // P = bf16(exp2(S c - m c)) into preg; returns the sum of those bf16
    // values (l normalises O by the weights its product used, as the bf16
    // forward does)
    u32x4 preg[C::NU];
    auto exponentiate = [&]() {
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[t][i] = fast_exp2(fmaf(sacc[t][i], c, -mc));
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t pp =
                pack_bf16(sacc[t][8 * hh + 2 * e], sacc[t][8 * hh + 2 * e + 1]);
            preg[2 * t + hh][e] = pp;
            sum = add_bf16x2(pp, sum);
          }
      return sum;
    };
    scores();
    if (kb == 0) {
      m = block_max();
      mc = m * c;
    }
    float lb = exponentiate();
    if (wave_any(!(lb <= kLazyBound8))) {
      scores();
      const float mnew = fmaxf(m, block_max());
      const float alpha = fast_exp2((m - mnew) * c);
      m = mnew;
      mc = m * c;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) oacc[dt] *= alpha;
      lb = exponentiate();
    }
    l += lb;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      u32x4 av[C::NU];
      vread.template read<C::NU>(lds_addr(Vs), dt, av);
#pragma unroll
      for (int u = 0; u < C::NU; ++u) oacc[dt] = mfma32(av[u], preg[u], oacc[dt]);
    }
  };
  const int nfull = L / C::BN;
  for (int kb = 0; kb < nfull; ++kb) block(kb, Full{});
  if (nfull < nkb) block(nfull, Ragged{});

  // ---- epilogue (as the bf16 forward)
  l += xor32(l);
  if (qi < L) {
    const float inv = 1.0f / l;
    uint16_t* Og = a.out + (int64_t)(it.seq0 + qi) * (a.H * D) + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      const int d0 = 32 * dt + 16 * g;
      float f[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = oacc[dt][i] * inv;
      st16(Og + d0, pack8(f));
      st16(Og + d0 + 8, pack8(f + 8));
    }
    if (g == 0) a.lse[(int64_t)h * a.T + it.seq0 + qi] = (mc + __log2f(l)) * kLn2;
  }
}

hipError_t launch_fwd_fp8(int head_dim, const AttnArgs& a, int64_t n_slots, hipStream_t stream) {
  const unsigned n = (unsigned)n_slots;
  switch (head_dim) {
    case 64: fwd_fp8_kernel<64><<<n, 256, 0, stream>>>(a); break;
    case 128: fwd_fp8_kernel<128><<<n, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace esm
