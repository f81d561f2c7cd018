// Forward attention kernel for gfx950: one workgroup (4 waves) per work item of
// 128 queries of one (sequence, head); each wave owns 32 queries.
//
// Data flow per item:
//   Q rows (pre-rotation bf16) -> rotated in fp32 with the cos/sin table,
//   rounded once to bf16 -> LDS -> registers (MFMA B operands, kept for the
//   whole item).
//   For each block of 64 keys (32 at d = 128): K rows are rotated the same way into a
//   row-major LDS tile (the MFMA A operand of S^T = K~ Q~^T) and V rows are
//   copied row-major into LDS; the A operand of O^T += V^T P^T, which runs
//   along the key (row) axis, is read with the LDS transpose load. The next
//   block's global loads are issued before the current block's math and
//   committed to the other LDS buffer after it (double buffering, one barrier
//   per block).
//   Lane (q, g) of a wave holds the scores of query q against 16 keys per
//   32-key tile, so the block row maximum is a per-lane max plus one exchange
//   with lane ^ 32. Online softmax with a running maximum m that is raised
//   only when a block maximum exceeds it by more than 8 (log2 units): the
//   rescale of O and l by exp2(m_old - m_new) is skipped otherwise, and
//   P = exp2(S c - m c) <= 256 stays well inside bf16/fp32 range.
//   The row sum l accumulates P in fp32; P is rounded once to bf16 for the
//   MFMA. Keys past the end of the sequence get S = -inf, so P = 0.
//   Epilogue: O = acc / l -> bf16; LSE = (m c + log2 l) ln 2.
//
// Tiled attention keeps the L x L matrices on chip (BioNeMo blog, section 2.3
// describes the idea for another GPU); this kernel is laid out for the 64-wide
// wavefronts, 32x32x16 bf16 MFMA and LDS transpose loads of CDNA4.
#include "common.h"
#include "prep.h"

namespace esm {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;                  // queries per item
  static constexpr int BN = D == 128 ? 32 : 64;   // keys per block
  static constexpr int KP = D + 8;                // row pitch of the LDS tiles (bf16)
  static constexpr int NS = D / 16;               // k-steps over d
  static constexpr int ND = D >= 32 ? D / 32 : 1; // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;              // 32-key tiles per block
  static constexpr int NU = BN / 16;              // k-steps over keys
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int STAGE = 2 * K_ELEMS;       // K~ rows + V rows
  static constexpr int Q_ELEMS = BM * KP;
  static constexpr int LDS = 2 * STAGE > Q_ELEMS ? 2 * STAGE : Q_ELEMS;
  static constexpr int K_UNITS = BN * (D / 16);   // (key, chunk pair j0 / j0+d/2)
  static constexpr int V_UNITS = BN * (D / 8);    // (key, 8-wide chunk)
  static constexpr int KU = (K_UNITS + 255) / 256;
  static constexpr int VU = (V_UNITS + 255) / 256;
};

constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D, bool ROPE>
__global__ __launch_bounds__(256, D == 128 ? 2 : 3) void fwd_kernel(AttnArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, q0 = it.blk * C::BM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  const int rs = a.H * D;  // row stride; T*H*d < 2^31 is checked on the host
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const bool qneg = a.q_sign < 0.f;

  // ---- rotated queries -> LDS -> B-operand registers
  for (int u = tid; u < C::BM * (D / 16); u += 256) {
    const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, qi = q0 + row;
    float lo[8], hi[8];
    if (qi < L) {
      unpack8(ld16(Qg + qi * rs + j0), lo);
      unpack8(ld16(Qg + qi * rs + j0 + D / 2), hi);
      if (ROPE) {
        float2 cs[8];
        load_cs8(a.rope, qi * (D / 2) + j0, cs);
        rotate8_signed(lo, hi, cs, qneg);
      } else if (qneg) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { lo[e] = -lo[e]; hi[e] = -hi[e]; }
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
  u32x4 kl[C::KU], kh[C::KU], vv[C::VU];
  float2 kcs[C::KU][8];

  // Rows past the end of the sequence are loaded as copies of its last row
  // (finite values, always in bounds); the softmax gives them P = 0.
  auto issue = [&](int kb) {
    const int k0 = kb * C::BN, lim = L - k0;
    // uniform block bases (scalar registers) + per-lane 32-bit row offsets
    const uint16_t* __restrict__ Kb = Kg + (int64_t)k0 * rs;
    const uint16_t* __restrict__ Vb = Vg + (int64_t)k0 * rs;
    const float2* __restrict__ Rb = a.rope + k0 * (D / 2);
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + 256 * x;
      if (C::K_UNITS % 256 == 0 || u < C::K_UNITS) {
        const int row = min(u / (D / 16), lim - 1), j0 = (u % (D / 16)) * 8;
        kl[x] = ld16(Kb + row * rs + j0);
        kh[x] = ld16(Kb + row * rs + j0 + D / 2);
        if (ROPE) load_cs8(Rb, row * (D / 2) + j0, kcs[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < C::VU; ++x) {
      const int u = tid + 256 * x;
      if (C::V_UNITS % 256 == 0 || u < C::V_UNITS) {
        const int row = min(u / (D / 8), lim - 1), c8 = (u % (D / 8)) * 8;
        vv[x] = ld16(Vb + row * rs + c8);
      }
    }
  };

  auto commit = [&](int stage) {
    uint16_t* Ks = lds + stage * C::STAGE;
    uint16_t* Vs = Ks + C::K_ELEMS;
#pragma unroll
    for (int x = 0; x < C::KU; ++x) {
      const int u = tid + 256 * x;
      if (C::K_UNITS % 256 == 0 || u < C::K_UNITS) {
        const int row = u / (D / 16), j0 = (u % (D / 16)) * 8;
        u32x4 lo = kl[x], hi = kh[x];
        if (ROPE) {
          float fl[8], fh[8];
          unpack8(lo, fl);
          unpack8(hi, fh);
          rotate8<false, false>(fl, fh, kcs[x]);
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
      if (C::V_UNITS % 256 == 0 || u < C::V_UNITS)
        st16(&Vs[(u / (D / 8)) * C::KP + (u % (D / 8)) * 8], vv[x]);
    }
  };

  const int nkb = (L + C::BN - 1) / C::BN;
  issue(0);
  commit(0);
  __syncthreads();

  const float c = a.c;
  float m = 0.f, l = 0.f;
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
    if (lim < C::BN) {  // keys past the end: S = -inf, so P = 0
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sacc[t][i] = (32 * t + 16 * g + i < lim) ? sacc[t][i] : -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[t][i]);
    mx = fmaxf(mx, xor32(mx));
    if (kb == 0) {
      m = mx;  // block 0 holds key 0, so mx is finite
    } else if (wave_any((mx - m) * c > kRescaleThreshold)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2((m - mnew) * c);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) oacc[dt] *= alpha;
    }
    const float mc = m * c;

    u32x4 preg[C::NU];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(fmaf(sacc[t][i], c, -mc));
        l += p[i];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          preg[2 * t + hh][e] = pack_bf16(p[8 * hh + 2 * e], p[8 * hh + 2 * e + 1]);
    }
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        const u32x4 av =
            ld_tr8<(D < 32)>(Vs, C::KP, 32 * (u >> 1) + 8 * (u & 1), 32 * dt, D);
        oacc[dt] = mfma32(av, preg[u], oacc[dt]);
      }
    }
    if (kb + 1 < nkb) commit(stage ^ 1);
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
