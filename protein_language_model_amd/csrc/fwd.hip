// Forward attention kernel for gfx950: one workgroup (4 waves) per work item of
// 128 queries of one (sequence, head); each wave owns 32 queries.
//
// Data flow per item:
//   Q rows (pre-rotation bf16) -> rotated in fp32 with the cos/sin table,
//   rounded once to bf16 -> LDS -> registers (MFMA B operands, kept for the
//   whole item).
//   For each block of 64 keys: K rows are rotated the same way into LDS
//   (row-major, the MFMA A operand) and V rows are stored transposed in LDS
//   (V^T, the A operand of the second product); the next block's global loads
//   are issued before the current block's math and committed to the other
//   LDS buffer after it (double buffering, one barrier per block).
//   S^T = K~ Q~^T on bf16 MFMA (32x32x16, fp32 accumulate). Lane (q, g) of a
//   wave holds the scores of query q against 16 keys per 32-key tile, so the
//   running row maximum is a per-lane max plus one exchange with lane ^ 32.
//   Online softmax (running max m and sum l; rescale of O by exp2 of the max
//   change), P = exp2(S * c - m * c) with c = |scale| * log2(e).
//   O^T += V^T P^T on MFMA: the P registers are already the B operand.
//   Epilogue: O = acc / l -> bf16; LSE = (m c + log2 l) ln 2.
//
// Tiled attention keeps the L x L matrices on chip (BioNeMo blog, section 2.3
// describes the same idea for another GPU); this kernel is written for the
// 64-wide wavefronts, 32x32 MFMA tiles and 160 KB LDS of CDNA4.
#include "common.h"
#include "prep.h"

namespace esm {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;                  // queries per item
  static constexpr int BN = 64;                   // keys per block
  static constexpr int KP = D + 8;                // K~ / Q~ row pitch (bf16)
  static constexpr int VP = BN + 8;               // V^T row pitch
  static constexpr int NS = D / 16;               // k-steps over d
  static constexpr int ND = D >= 32 ? D / 32 : 1; // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;              // 32-key tiles per block
  static constexpr int NU = BN / 16;              // k-steps over keys
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int Q_ELEMS = BM * KP;
  static constexpr int LDS = 2 * STAGE > Q_ELEMS ? 2 * STAGE : Q_ELEMS;
  static constexpr int K_UNITS = BN * (D / 16);       // (key, chunk pair j0 / j0+d/2)
  static constexpr int V_UNITS = (BN / 2) * (D / 8);  // (key pair, 8-wide d chunk)
  static constexpr int KU = (K_UNITS + 255) / 256;
  static constexpr int VU = (V_UNITS + 255) / 256;
};

// Loads (cos, sin) for angles p * theta_{j0 .. j0+7}.
__device__ __forceinline__ void load_cs(const float2* rope, int64_t idx, float2* cs) {
  const u32x4* p = reinterpret_cast<const u32x4*>(rope + idx);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = p[i];
    cs[2 * i] = make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    cs[2 * i + 1] = make_float2(__uint_as_float(v[2]), __uint_as_float(v[3]));
  }
}

template <int D, bool ROPE>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, q0 = it.blk * C::BM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;

  // ---- rotated queries -> LDS -> B-operand registers
  for (int u = tid; u < C::BM * (D / 16); u += 256) {
    const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, qi = q0 + row;
    float lo[8], hi[8];
    if (qi < L) {
      unpack8(ld16(Qg + qi * rs + j0), lo);
      unpack8(ld16(Qg + qi * rs + j0 + D / 2), hi);
      if (ROPE) {
        float2 cs[8];
        load_cs(a.rope, (int64_t)qi * (D / 2) + j0, cs);
        rotate8(lo, hi, cs, false, a.q_sign);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { lo[e] *= a.q_sign; hi[e] *= a.q_sign; }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { lo[e] = 0.f; hi[e] = 0.f; }
    }
    st16(&lds[row * C::KP + j0], pack8(lo));
    st16(&lds[row * C::KP + j0 + D / 2], pack8(hi));
  }
  __syncthreads();
  u32x4 qreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) qreg[s] = ld16(&lds[(w * 32 + r) * C::KP + 16 * s + 8 * g]);
  __syncthreads();

  // ---- K/V block staging (global -> registers -> LDS)
  u32x4 kl[C::KU], kh[C::KU], v0[C::VU], v1[C::VU];
  float2 kcs[C::KU][8];

  auto issue = [&](int kb) {
    const int k0 = kb * C::BN;
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + 256 * x;
      kl[x] = zero4();
      kh[x] = zero4();
      if (u < C::K_UNITS) {
        const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, key = k0 + row;
        if (key < L) {
          kl[x] = ld16(Kg + key * rs + j0);
          kh[x] = ld16(Kg + key * rs + j0 + D / 2);
          if (ROPE) load_cs(a.rope, (int64_t)key * (D / 2) + j0, kcs[x]);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + 256 * x;
      v0[x] = zero4();
      v1[x] = zero4();
      if (u < C::V_UNITS) {
        const int kp = u % (C::BN / 2), nc = u / (C::BN / 2), key = k0 + 2 * kp;
        if (key < L) v0[x] = ld16(Vg + key * rs + 8 * nc);
        if (key + 1 < L) v1[x] = ld16(Vg + (key + 1) * rs + 8 * nc);
      }
    }
  };

  auto commit = [&](int kb, int stage) {
    uint16_t* Ks = lds + stage * C::STAGE;
    uint16_t* Vs = Ks + C::K_ELEMS;
    const int k0 = kb * C::BN;
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + 256 * x;
      if (u < C::K_UNITS) {
        const int row = u / (D / 16), j0 = (u % (D / 16)) * 8;
        u32x4 lo = kl[x], hi = kh[x];
        if (ROPE && k0 + row < L) {
          float fl[8], fh[8];
          unpack8(lo, fl);
          unpack8(hi, fh);
          rotate8(fl, fh, kcs[x], false, 1.0f);
          lo = pack8(fl);
          hi = pack8(fh);
        }
        st16(&Ks[row * C::KP + j0], lo);
        st16(&Ks[row * C::KP + j0 + D / 2], hi);
      }
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + 256 * x;
      if (u < C::V_UNITS) {
        const int kp = u % (C::BN / 2), nc = u / (C::BN / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w0 = v0[x][e >> 1], w1 = v1[x][e >> 1];
          const uint32_t pair = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                        : ((w0 & 0xffffu) | (w1 << 16));
          *reinterpret_cast<uint32_t*>(&Vs[(8 * nc + e) * C::VP + 2 * kp]) = pair;
        }
      }
    }
  };

  const int nkb = (L + C::BN - 1) / C::BN;
  issue(0);
  commit(0, 0);
  __syncthreads();

  const float c = a.c;
  float m = -INFINITY, l = 0.f;
  f32x16 oacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) oacc[dt] = f32x16{};

  for (int kb = 0; kb < nkb; ++kb) {
    const int stage = kb & 1;
    if (kb + 1 < nkb) issue(kb + 1);
    const uint16_t* Ks = lds + stage * C::STAGE;
    const uint16_t* Vs = Ks + C::K_ELEMS;

    // S^T tiles: lane (q = r, g) register i of tile t = key 32t + 16g + i
    f32x16 sacc[C::NT];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      sacc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::NS; ++s)
        sacc[t] = mfma32(ld16(&Ks[(32 * t + prow) * C::KP + 16 * s + 8 * g]), qreg[s], sacc[t]);
    }
    const int lim = L - kb * C::BN;  // valid keys in this block
    const bool ragged = lim < C::BN;
    if (ragged) {
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * t + 16 * g + i >= lim) sacc[t][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[t][i]);
    mx = fmaxf(mx, xor32(mx));
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - mnew) * c);
    const float mc = mnew * c;
    m = mnew;
    float rowsum = 0.f;
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(sacc[t][i], c, -mc));
        if (ragged && 32 * t + 16 * g + i >= lim) p = 0.f;
        sacc[t][i] = p;
        rowsum += p;
      }
    l = fmaf(l, alpha, rowsum);
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) oacc[dt] *= alpha;

    u32x4 preg[C::NU];
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
      const int t = u >> 1, i0 = 8 * (u & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        preg[u][e] = pack_bf16(sacc[t][i0 + 2 * e], sacc[t][i0 + 2 * e + 1]);
    }
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        u32x4 av = zero4();
        if (D >= 32 || prow < D)
          av = ld16(&Vs[(32 * dt + prow) * C::VP + 32 * (u >> 1) + 16 * g + 8 * (u & 1)]);
        oacc[dt] = mfma32(av, preg[u], oacc[dt]);
      }
    }
    if (kb + 1 < nkb) commit(kb + 1, stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  l += xor32(l);
  const int qi = q0 + w * 32 + r;
  if (qi < L) {
    const float inv = 1.0f / l;
    uint16_t* Og = a.out + base + qi * rs;
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      const int d0 = 32 * dt + 16 * g;
      if (d0 < D) {
        float f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = oacc[dt][i] * inv;
        st16(Og + d0, pack8(f));
        st16(Og + d0 + 8, pack8(f + 8));
      }
    }
    if (g == 0) a.lse[(int64_t)h * a.T + it.seq0 + qi] = (m * c + __log2f(l)) * kLn2;
  }
}

template <int D>
static hipError_t launch_fwd_d(bool rope, const AttnArgs& a, int64_t n_slots, hipStream_t st) {
  if (rope)
    fwd_kernel<D, true><<<(unsigned)n_slots, 256, 0, st>>>(a);
  else
    fwd_kernel<D, false><<<(unsigned)n_slots, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(int head_dim, bool rope, const AttnArgs& a, int64_t n_slots,
                      hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_fwd_d<16>(rope, a, n_slots, stream);
    case 32: return launch_fwd_d<32>(rope, a, n_slots, stream);
    case 64: return launch_fwd_d<64>(rope, a, n_slots, stream);
    case 128: return launch_fwd_d<128>(rope, a, n_slots, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace esm
