// Backward attention kernels for gfx950. P is recomputed from the LSE the
// forward stored (P = exp2(S c - LSE log2 e)), so no L x L matrix is kept.
//
// Two deterministic passes, no atomics:
//   dq pass : one workgroup per 128 queries of a (sequence, head) (lane owns a
//             query). Prologue computes D = rowsum(dO * O) for its queries and
//             stores it for the second pass. Per 64-key block (32 at d=128):
//             S^T = K~ Q~^T, dP^T = V dO^T, dS = P (dP - D),
//             dQ~^T += K~^T dS^T. Epilogue: dq = R(-p) (scale dQ~) -> bf16.
// In the dq pass dP - D comes out of the dP MFMA itself: one extra k-step
// multiplies (1, 1) by (-D_hi, -D_lo) (D split into two bf16 values), which
// replaces one vector subtraction per score. (In the dkv pass D varies along
// the lane's 16 rows; there the extra MFMA measured slower than subtracting.)
//   dkv pass: one workgroup per 128 keys (lane owns a key). Per 64-query block
//             (32 at d=128): S = Q~ K~^T, dP = dO V^T, dS = P (dP - D),
//             dV^T += dO^T P, dK~^T += Q~^T dS. Epilogue: dk = R(-p)(|scale| dK~),
//             dv -> bf16.
// All LDS tiles are row-major (token rows, d columns). Operands that a product
// contracts over the token axis (K~^T, Q~^T, dO^T) are read from those same
// tiles with the LDS transpose load, so nothing is stored twice. The next
// block's global loads are issued before the current block's math
// (double-buffered LDS, one barrier per block).
#include "common.h"
#include "prep.h"

namespace esm {

// =========================================================================
// dq pass
// =========================================================================
template <int D>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = D == 128 ? 32 : 64;
  static constexpr int KP = D + 8;
  static constexpr int NS = D / 16;
  static constexpr int ND = D >= 32 ? D / 32 : 1;
  static constexpr int NT = BN / 32;
  static constexpr int NU = BN / 16;
  static constexpr int K_ELEMS = BN * KP;  // K~ rows
  static constexpr int V_ELEMS = BN * KP;  // V rows
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int PRO = BM * KP;
  static constexpr int EPI = BM * (D + 4) * 2;  // fp32 tile, in uint16 units
  static constexpr int LDS0 = 2 * STAGE > PRO ? 2 * STAGE : PRO;
  static constexpr int LDS = LDS0 > EPI ? LDS0 : EPI;
  static constexpr int K_UNITS = BN * (D / 16);
  static constexpr int V_UNITS = BN * (D / 8);
  static constexpr int KU = (K_UNITS + 255) / 256;
  static constexpr int VU = (V_UNITS + 255) / 256;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(AttnArgs a) {
  using C = DqCfg<D>;
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
  const uint16_t* __restrict__ Og = a.o + base;
  const uint16_t* __restrict__ dOg = a.dout + base;
  const int qi = q0 + w * 32 + r;  // this lane's query
  const bool qvalid = qi < L;
  const bool qneg = a.q_sign < 0.f;

  // ---- prologue: rotated queries (B operands)
  for (int u = tid; u < C::BM * (D / 16); u += 256) {
    const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, qq = q0 + row;
    float lo[8], hi[8];
    if (qq < L) {
      unpack8(ld16(Qg + qq * rs + j0), lo);
      unpack8(ld16(Qg + qq * rs + j0 + D / 2), hi);
      if (ROPE) {
        float2 cs[8];
        load_cs8(a.rope, qq * (D / 2) + j0, cs);
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
  u32x4 qreg[C::NS], doreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) qreg[s] = ld16(&lds[(w * 32 + r) * C::KP + 16 * s + 8 * g]);

  // dO (B operands, straight from global) and D = dO . O for this lane's query
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    doreg[s] = zero4();
    if (qvalid) {
      doreg[s] = ld16(dOg + qi * rs + 16 * s + 8 * g);
      const u32x4 ov = ld16(Og + qi * rs + 16 * s + 8 * g);
      float fo[8], fd[8];
      unpack8(ov, fo);
      unpack8(doreg[s], fd);
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf(fd[e], fo[e], dpart);
    }
  }
  const float Dq = dpart + xor32(dpart);
  // dP - D in one more MFMA k-step: A = (1, 1), B = (-D_hi, -D_lo), in the
  // k slots of lane half 0.
  const u32x4 a_one = {g == 0 ? kBf16OnePair : 0u, 0u, 0u, 0u};
  const u32x4 b_negd = {g == 0 ? neg_bf16_pair(Dq) : 0u, 0u, 0u, 0u};
  const int64_t rowidx = (int64_t)h * a.T + it.seq0 + qi;
  float lse2 = 0.f;
  if (qvalid) {
    lse2 = a.lse_in[rowidx] * kLog2e;
    if (g == 0) a.drow[rowidx] = Dq;
  }
  __syncthreads();

  // ---- K/V staging
  u32x4 kl[C::KU], kh[C::KU], vv[C::VU];
  float2 kcs[C::KU][8];
  // Rows past the end of the sequence are loaded as copies of its last row
  // (finite, in bounds); the ragged block masks their P to 0.
  auto issue = [&](int kb) {
    const int k0 = kb * C::BN, lim = L - k0;
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
  f32x16 dqacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) dqacc[dt] = f32x16{};

  for (int kb = 0; kb < nkb; ++kb) {
    const int stage = kb & 1;
    if (kb + 1 < nkb) issue(kb + 1);
    const uint16_t* Ks = lds + stage * C::STAGE;
    const uint16_t* Vs = Ks + C::K_ELEMS;
    const int lim = L - kb * C::BN;  // valid keys in this block

    u32x4 dsreg[C::NU];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int off = (32 * t + prow) * C::KP + 16 * s + 8 * g;
        sacc = mfma32(ld16(&Ks[off]), qreg[s], sacc);
        pacc = mfma32(ld16(&Vs[off]), doreg[s], pacc);
      }
      pacc = mfma32(a_one, b_negd, pacc);  // pacc = dP - D
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[i], c, -lse2));
        dsv[i] = p * pacc[i];
      }
      if (lim < C::BN) {  // keys past the end: dS = 0
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * t + 16 * g + i >= lim) dsv[i] = 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dsreg[2 * t + hh][e] = pack_bf16(dsv[8 * hh + 2 * e], dsv[8 * hh + 2 * e + 1]);
    }
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        const u32x4 at =
            ld_tr8<(D < 32)>(Ks, C::KP, 32 * (u >> 1) + 8 * (u & 1), 32 * dt, D);
        dqacc[dt] = mfma32(at, dsreg[u], dqacc[dt]);
      }
    }
    if (kb + 1 < nkb) commit(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: dq~ (fp32) -> LDS -> inverse rotation -> bf16
  float* F = reinterpret_cast<float*>(lds);
  constexpr int FP = D + 4;
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    const int d0 = 32 * dt + 16 * g;
    if (d0 < D) {
#pragma unroll
      for (int i = 0; i < 16; ++i) F[(w * 32 + r) * FP + d0 + i] = dqacc[dt][i] * a.scale;
    }
  }
  __syncthreads();
  store_rows<D, ROPE>(F, C::BM, q0, L, a.dq + base, rs, a.rope, true, tid);
}

// =========================================================================
// dk / dv pass
// =========================================================================
template <int D>
struct DkvCfg {
  static constexpr int BK = 128;
  static constexpr int BQ = D == 128 ? 32 : 64;
  static constexpr int KP = D + 8;
  static constexpr int NS = D / 16;
  static constexpr int ND = D >= 32 ? D / 32 : 1;
  static constexpr int NT = BQ / 32;
  static constexpr int NU = BQ / 16;
  static constexpr int Q_ELEMS = BQ * KP;   // Q~ rows
  static constexpr int O_ELEMS = BQ * KP;   // dO rows
  static constexpr int F_ELEMS = 4 * BQ;    // lse2[BQ], D[BQ] as fp32
  static constexpr int STAGE = Q_ELEMS + O_ELEMS + F_ELEMS;
  static constexpr int PRO = 2 * BK * KP;
  static constexpr int EPI = BK * (D + 4) * 2;
  static constexpr int LDS0 = 2 * STAGE > PRO ? 2 * STAGE : PRO;
  static constexpr int LDS = LDS0 > EPI ? LDS0 : EPI;
  static constexpr int Q_UNITS = BQ * (D / 16);
  static constexpr int O_UNITS = BQ * (D / 8);
  static constexpr int QU = (Q_UNITS + 255) / 256;
  static constexpr int OU = (O_UNITS + 255) / 256;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(AttnArgs a) {
  using C = DkvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, k0 = it.blk * C::BK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  const int rs = a.H * D;  // row stride; T*H*d < 2^31 is checked on the host
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const uint16_t* __restrict__ dOg = a.dout + base;
  const int64_t row0 = (int64_t)h * a.T + it.seq0;
  const bool qneg = a.q_sign < 0.f;

  // ---- prologue: rotated keys and values -> LDS -> B-operand registers
  {
    uint16_t* Ks = lds;
    uint16_t* Vs = lds + C::BK * C::KP;
    for (int u = tid; u < C::BK * (D / 16); u += 256) {
      const int row = u / (D / 16), j0 = (u % (D / 16)) * 8, key = k0 + row;
      float lo[8], hi[8];
      u32x4 vlo = zero4(), vhi = zero4();
      if (key < L) {
        unpack8(ld16(Kg + key * rs + j0), lo);
        unpack8(ld16(Kg + key * rs + j0 + D / 2), hi);
        if (ROPE) {
          float2 cs[8];
          load_cs8(a.rope, key * (D / 2) + j0, cs);
          rotate8<false, false>(lo, hi, cs);
        }
        vlo = ld16(Vg + key * rs + j0);
        vhi = ld16(Vg + key * rs + j0 + D / 2);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { lo[e] = 0.f; hi[e] = 0.f; }
      }
      st16(&Ks[row * C::KP + j0], pack8(lo));
      st16(&Ks[row * C::KP + j0 + D / 2], pack8(hi));
      st16(&Vs[row * C::KP + j0], vlo);
      st16(&Vs[row * C::KP + j0 + D / 2], vhi);
    }
  }
  __syncthreads();
  u32x4 kreg[C::NS], vreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    kreg[s] = ld16(&lds[(w * 32 + r) * C::KP + 16 * s + 8 * g]);
    vreg[s] = ld16(&lds[C::BK * C::KP + (w * 32 + r) * C::KP + 16 * s + 8 * g]);
  }
  __syncthreads();

  // ---- Q / dO staging
  u32x4 ql[C::QU], qh[C::QU], ov[C::OU];
  float2 qcs[C::QU][8];
  float fl_lse = 0.f, fl_d = 0.f;
  // Rows past the end of the sequence are loaded as copies of its last row
  // (finite, in bounds); their LSE is set to +inf so that P = 0.
  auto issue = [&](int qb) {
    const int q0 = qb * C::BQ, lim = L - q0;
    const uint16_t* __restrict__ Qb = Qg + (int64_t)q0 * rs;
    const uint16_t* __restrict__ Ob = dOg + (int64_t)q0 * rs;
    const float2* __restrict__ Rb = a.rope + q0 * (D / 2);
#pragma unroll
    for (int x = 0; x < C::QU; ++x) {
      const int u = tid + 256 * x;
      if (C::Q_UNITS % 256 == 0 || u < C::Q_UNITS) {
        const int row = min(u / (D / 16), lim - 1), j0 = (u % (D / 16)) * 8;
        ql[x] = ld16(Qb + row * rs + j0);
        qh[x] = ld16(Qb + row * rs + j0 + D / 2);
        if (ROPE) load_cs8(Rb, row * (D / 2) + j0, qcs[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < C::OU; ++x) {
      const int u = tid + 256 * x;
      if (C::O_UNITS % 256 == 0 || u < C::O_UNITS) {
        const int row = min(u / (D / 8), lim - 1), c8 = (u % (D / 8)) * 8;
        ov[x] = ld16(Ob + row * rs + c8);
      }
    }
    if (tid < C::BQ) {
      const int qq = q0 + tid;
      fl_lse = INFINITY;
      fl_d = 0.f;
      if (qq < L) {
        fl_lse = a.lse_in[row0 + qq] * kLog2e;
        fl_d = a.drow[row0 + qq];
      }
    }
  };
  auto commit = [&](int stage) {
    uint16_t* Qs = lds + stage * C::STAGE;
    uint16_t* Os = Qs + C::Q_ELEMS;
    float* Fs = reinterpret_cast<float*>(Os + C::O_ELEMS);
#pragma unroll
    for (int x = 0; x < C::QU; ++x) {
      const int u = tid + 256 * x;
      if (C::Q_UNITS % 256 == 0 || u < C::Q_UNITS) {
        const int row = u / (D / 16), j0 = (u % (D / 16)) * 8;
        float fl[8], fh[8];
        unpack8(ql[x], fl);
        unpack8(qh[x], fh);
        if (ROPE) {
          rotate8_signed(fl, fh, qcs[x], qneg);
        } else if (qneg) {
#pragma unroll
          for (int e = 0; e < 8; ++e) { fl[e] = -fl[e]; fh[e] = -fh[e]; }
        }
        st16(&Qs[row * C::KP + j0], pack8(fl));
        st16(&Qs[row * C::KP + j0 + D / 2], pack8(fh));
      }
    }
#pragma unroll
    for (int x = 0; x < C::OU; ++x) {
      const int u = tid + 256 * x;
      if (C::O_UNITS % 256 == 0 || u < C::O_UNITS)
        st16(&Os[(u / (D / 8)) * C::KP + (u % (D / 8)) * 8], ov[x]);
    }
    if (tid < C::BQ) {
      Fs[tid] = fl_lse;
      Fs[C::BQ + tid] = fl_d;
    }
  };

  const int nqb = (L + C::BQ - 1) / C::BQ;
  issue(0);
  commit(0);
  __syncthreads();

  const float c = a.c;
  f32x16 dvacc[C::ND], dkacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    dvacc[dt] = f32x16{};
    dkacc[dt] = f32x16{};
  }

  for (int qb = 0; qb < nqb; ++qb) {
    const int stage = qb & 1;
    if (qb + 1 < nqb) issue(qb + 1);
    const uint16_t* Qs = lds + stage * C::STAGE;
    const uint16_t* Os = Qs + C::Q_ELEMS;
    const float* Fs = reinterpret_cast<const float*>(Os + C::O_ELEMS);

    u32x4 preg[C::NU], dsreg[C::NU];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int off = (32 * t + prow) * C::KP + 16 * s + 8 * g;
        sacc = mfma32(ld16(&Qs[off]), kreg[s], sacc);
        pacc = mfma32(ld16(&Os[off]), vreg[s], pacc);
      }
      // queries 32t + 16g + i, i = 0..15
      float lse2[16], dd[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 x = ld16(&Fs[32 * t + 16 * g + 4 * j]);
        const u32x4 y = ld16(&Fs[C::BQ + 32 * t + 16 * g + 4 * j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lse2[4 * j + e] = __uint_as_float(x[e]);
          dd[4 * j + e] = __uint_as_float(y[e]);
        }
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = fast_exp2(fmaf(sacc[i], c, -lse2[i]));
        dsv[i] = pv[i] * (pacc[i] - dd[i]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          preg[2 * t + hh][e] = pack_bf16(pv[8 * hh + 2 * e], pv[8 * hh + 2 * e + 1]);
          dsreg[2 * t + hh][e] = pack_bf16(dsv[8 * hh + 2 * e], dsv[8 * hh + 2 * e + 1]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        const int k0 = 32 * (u >> 1) + 8 * (u & 1);
        const u32x4 ao = ld_tr8<(D < 32)>(Os, C::KP, k0, 32 * dt, D);
        const u32x4 aq = ld_tr8<(D < 32)>(Qs, C::KP, k0, 32 * dt, D);
        dvacc[dt] = mfma32(ao, preg[u], dvacc[dt]);
        dkacc[dt] = mfma32(aq, dsreg[u], dkacc[dt]);
      }
    }
    if (qb + 1 < nqb) commit(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: dk = R(-p) |scale| dK~, dv
  float* F = reinterpret_cast<float*>(lds);
  constexpr int FP = D + 4;
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    const int d0 = 32 * dt + 16 * g;
    if (d0 < D) {
#pragma unroll
      for (int i = 0; i < 16; ++i) F[(w * 32 + r) * FP + d0 + i] = dkacc[dt][i] * a.scale_abs;
    }
  }
  __syncthreads();
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dk + base, rs, a.rope, true, tid);
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    const int d0 = 32 * dt + 16 * g;
    if (d0 < D) {
#pragma unroll
      for (int i = 0; i < 16; ++i) F[(w * 32 + r) * FP + d0 + i] = dvacc[dt][i];
    }
  }
  __syncthreads();
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dv + base, rs, a.rope, false, tid);
}

template <int D, bool ROPE>
static hipError_t launch_bwd_dr(const AttnArgs& a, int64_t n_slots, bool dq_pass, bool dkv_pass,
                                hipStream_t st) {
  if (dq_pass) {
    bwd_dq_kernel<D, ROPE><<<(unsigned)n_slots, 256, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dkv_pass) {
    bwd_dkv_kernel<D, ROPE><<<(unsigned)n_slots, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_d(bool rope, const AttnArgs& a, int64_t n_slots, bool dq_pass,
                               bool dkv_pass, hipStream_t st) {
  return rope ? launch_bwd_dr<D, true>(a, n_slots, dq_pass, dkv_pass, st)
              : launch_bwd_dr<D, false>(a, n_slots, dq_pass, dkv_pass, st);
}

hipError_t launch_bwd(int head_dim, bool rope, const AttnArgs& a, int64_t n_slots, bool dq_pass,
                      bool dkv_pass, hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_bwd_d<16>(rope, a, n_slots, dq_pass, dkv_pass, stream);
    case 32: return launch_bwd_d<32>(rope, a, n_slots, dq_pass, dkv_pass, stream);
    case 64: return launch_bwd_d<64>(rope, a, n_slots, dq_pass, dkv_pass, stream);
    case 128: return launch_bwd_d<128>(rope, a, n_slots, dq_pass, dkv_pass, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace esm
