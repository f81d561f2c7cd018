// Backward attention kernels for gfx950. P is recomputed from the LSE the
// forward stored (P = exp2(S c - LSE log2 e)), so no L x L matrix is kept.
//
// Two deterministic passes, no atomics:
//   dq pass : one workgroup per 128 queries of a (sequence, head) (lane owns a
//             query). Prologue computes D = rowsum(dO * O) for its queries and
//             stores it, with LSE log2 e, for the second pass. Per 64-key
//             block (32 at d=128): S^T = K~ Q~^T, dP^T = V dO^T,
//             dS = P (dP - D), dQ~^T += K~^T dS^T.
//             Epilogue: dq = R(-p) (scale dQ~) -> bf16.
//             dP - D comes out of the dP MFMA itself: one extra k-step
//             multiplies (1, 1) by (-D_hi, -D_lo) (D split into two bf16
//             values), which replaces one vector subtraction per score.
//   dkv pass: one workgroup per 128 keys (lane owns a key). Per 64-query block
//             (32 at d=128): S = Q~ K~^T, dP = dO V^T, dS = P (dP - D),
//             dV^T += dO^T P, dK~^T += Q~^T dS. Epilogue: dk = R(-p)(scale dK~),
//             dv -> bf16. (Here D varies along the lane's 16 rows; an extra
//             MFMA for dP - D measured slower than the subtraction.)
// q~ and k~ come rotated from the rotation pass. The streamed operands (k~
// and v in the dq pass; q~, dO, LSE and D in the dkv pass) are copied from
// global memory into swizzled LDS tiles by global_load_lds, in a ring of
// three LDS stages (the copy of block b + 2 is issued right after the barrier
// that opens block b). Products that contract over the token axis (K~^T, Q~^T,
// dO^T) read the same row-major tiles with the LDS transpose load.
#include "common.h"
#include "prep.h"
#include "tile.h"

namespace esm {

// =========================================================================
// dq pass
// =========================================================================
template <int D>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = D == 128 ? 32 : 64;
  static constexpr int NS = D / 16;
  static constexpr int ND = D >= 32 ? D / 32 : 1;
  static constexpr int NT = BN / 32;
  static constexpr int NU = BN / 16;
  static constexpr int TILE = BN * D;           // k~ tile, then v tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NSTAGE = 3;              // LDS ring of key blocks
  static constexpr int EPI = BM * (D + 4) * 2;  // fp32 tile, in uint16 units
  static constexpr int LDS = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
  static constexpr int OCC = 2;
  using Loader = TilePair<D, BN>;
  static constexpr int LOADS = Loader::LOADS_PER_WAVE;  // per wave and block
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256, DqCfg<D>::OCC) void bwd_dq_kernel(AttnArgs a) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, q0 = it.blk * C::BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  // row strides (T * stride < 2^31 is checked on the host): q~, k~, v; o, dO
  const int rs = a.ld_qkv, rso = a.H * D;
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const int64_t baseo = (int64_t)it.seq0 * rso + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const uint16_t* __restrict__ Og = a.o + baseo;
  const uint16_t* __restrict__ dOg = a.dout + baseo;

  // k~ and v rows of key block kb -> LDS stage `stage` (offsets kept in
  // registers for blocks with every key present)
  const typename C::Loader loader(w, lane);
  const typename C::Loader::Offsets koff = loader.offsets(rs, w);
  auto issue = [&](int kb, int stage) {
    const int k0 = kb * C::BN;
    uint16_t* Ks = lds + stage * C::STAGE;
    if (k0 + C::BN <= L)
      loader.load_full(Kg + (int64_t)k0 * rs, Vg + (int64_t)k0 * rs, koff, Ks, Ks + C::TILE, w);
    else
      loader.template load<1>(Kg + (int64_t)k0 * rs, rs, Vg + (int64_t)k0 * rs, rs, L - k0, Ks,
                              Ks + C::TILE, w);
  };
  const int nkb = (L + C::BN - 1) / C::BN;
  issue(0, 0);

  // ---- prologue: q~ and dO (B operands), D = dO . O, LSE (log2 units)
  const int qi = q0 + w * 32 + r;  // this lane's query
  const bool qvalid = qi < L;
  const uint32_t qflip = a.q_sign < 0.f ? 0x80008000u : 0u;
  // Every load reads a clamped row and is issued before any is used (loads
  // under a branch would each be awaited at the branch's end); rows past the
  // end are zeroed afterwards.
  const int qc = min(qi, L - 1);
  const int64_t rowidx = (int64_t)h * a.T + it.seq0 + qi;
  const float lse_raw = a.lse_in[(int64_t)h * a.T + it.seq0 + qc];
  u32x4 qreg[C::NS], doreg[C::NS], oreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    qreg[s] = ld16(Qg + qc * rs + 16 * s + 8 * g);
    doreg[s] = ld16(dOg + qc * rso + 16 * s + 8 * g);
    oreg[s] = ld16(Og + qc * rso + 16 * s + 8 * g);
  }
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    float fo[8], fd[8];
    unpack8(oreg[s], fo);
    unpack8(doreg[s], fd);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf(fd[e], fo[e], dpart);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qreg[s][e] = qvalid ? qreg[s][e] ^ qflip : 0u;
      doreg[s][e] = qvalid ? doreg[s][e] : 0u;
    }
  }
  if (!qvalid) dpart = 0.f;
  const float Dq = dpart + xor32(dpart);
  // dP - D in one more MFMA k-step: A = (1, 1), B = (-D_hi, -D_lo), in the
  // k slots of lane half 0.
  const u32x4 a_one = {g == 0 ? kBf16OnePair : 0u, 0u, 0u, 0u};
  const u32x4 b_negd = {g == 0 ? neg_bf16_pair(Dq) : 0u, 0u, 0u, 0u};
  const float lse2 = qvalid ? lse_raw * kLog2e : 0.f;
  if (qvalid && g == 0) {
    a.drow[rowidx] = Dq;
    a.drow[(int64_t)a.H * a.T + rowidx] = lse2;
  }

  // blocks 1 .. NSTAGE-2 after the prologue's global loads (see the wait below)
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nkb) issue(j, j);

  const float c = a.c;
  const int xk = swz<D>(prow);
  const TrRows<D> kread(lane);  // transposed reads of the k~ tile
  f32x16 dqacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) dqacc[dt] = f32x16{};

  int stage = 0, next = C::NSTAGE - 1;
  // One key block; only the last block of a ragged sequence (FULL false)
  // carries the masking code.
  auto block = [&](int kb, auto full) {
    constexpr bool FULL = decltype(full)::value;
    // block kb's copies are done once at most the next block's are
    // outstanding; the barrier publishes them and frees stage `next`
    if (C::NSTAGE == 3 && kb + 1 < nkb)
      wait_vmem<C::LOADS>();
    else
      wait_vmem<0>();
    block_barrier();
    if (kb + C::NSTAGE - 1 < nkb) issue(kb + C::NSTAGE - 1, next);
    const uint16_t* Ks = lds + stage * C::STAGE;
    const uint16_t* Vs = Ks + C::TILE;
    stage = stage + 1 == C::NSTAGE ? 0 : stage + 1;
    next = next + 1 == C::NSTAGE ? 0 : next + 1;
    const int lim = L - kb * C::BN;  // valid keys in this block

    u32x4 dsreg[C::NU];
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const int rowoff = (32 * t + prow) * D;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int off = rowoff + 8 * ((2 * s + g) ^ xk);
        sacc = mfma32(ld16(Ks + off), qreg[s], sacc);
        pacc = mfma32(ld16(Vs + off), doreg[s], pacc);
      }
      pacc = mfma32(a_one, b_negd, pacc);  // pacc = dP - D
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[i], c, -lse2));
        dsv[i] = p * pacc[i];
      }
      if (!FULL) {  // keys past the end: dS = 0
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
      u32x4 at[C::NU];
      kread.template read<C::NU>(lds_addr(Ks), dt, at);
#pragma unroll
      for (int u = 0; u < C::NU; ++u) dqacc[dt] = mfma32(at[u], dsreg[u], dqacc[dt]);
    }
  };
  const int nfull = L / C::BN;
  for (int kb = 0; kb < nfull; ++kb) block(kb, Full{});
  if (nfull < nkb) block(nfull, Ragged{});
  __syncthreads();  // every wave is done with the tiles

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
  store_rows<D, ROPE>(F, C::BM, q0, L, a.dq + (int64_t)it.seq0 * a.ld_grad + (int64_t)h * D,
                     a.ld_grad, a.rope, true, tid);
}

// =========================================================================
// dk / dv pass
// =========================================================================
template <int D>
struct DkvCfg {
  static constexpr int BK = 128;
  static constexpr int BQ = D == 128 ? 32 : 64;
  static constexpr int NS = D / 16;
  static constexpr int ND = D >= 32 ? D / 32 : 1;
  static constexpr int NT = BQ / 32;
  static constexpr int TILE = BQ * D;           // q~ tile, then dO tile
  static constexpr int STAGE = 2 * TILE + 4 * BQ;  // + lse2[BQ], D[BQ] as fp32
  static constexpr int NSTAGE = 3;              // LDS ring of query blocks
  static constexpr int EPI = BK * (D + 4) * 2;
  static constexpr int LDS = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
  static constexpr int OCC = D == 128 ? 2 : 3;
  static constexpr bool FOLD_D = D <= 64;          // dP - D folded into an MFMA
  using Loader = TilePair<D, BQ>;
  static constexpr int LOADS = Loader::LOADS_PER_WAVE + 1;  // + a half row of lse2 or D
};

template <int D, bool ROPE>
__global__ __launch_bounds__(256, DkvCfg<D>::OCC) void bwd_dkv_kernel(AttnArgs a) {
  using C = DkvCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS];

  const Item it = a.items[blockIdx.x];
  if (it.len <= 0) return;
  const int L = it.len, h = it.head, k0 = it.blk * C::BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  // row strides (T * stride < 2^31 is checked on the host): q~, k~, v; dO
  const int rs = a.ld_qkv, rso = a.H * D;
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  const uint16_t* __restrict__ Kg = a.k + base;
  const uint16_t* __restrict__ Vg = a.v + base;
  const uint16_t* __restrict__ dOg = a.dout + (int64_t)it.seq0 * rso + (int64_t)h * D;
  const int64_t row0 = (int64_t)h * a.T + it.seq0;
  // waves 0-1 copy halves of the lse2 row, waves 2-3 halves of the D row
  const float* __restrict__ Fg =
      a.drow + (w < 2 ? (int64_t)a.H * a.T : (int64_t)0) + row0;

  // q~, dO, lse2 and D rows of query block qb -> LDS stage `stage`
  const typename C::Loader loader(w, lane);
  auto issue = [&](int qb, int stage) {
    const int q0 = qb * C::BQ, lim = L - q0;
    uint16_t* Qs = lds + stage * C::STAGE;
    float* Fs = reinterpret_cast<float*>(Qs + 2 * C::TILE) + (w < 2 ? 0 : C::BQ);
    loader.load(Qg + (int64_t)q0 * rs, rs, dOg + (int64_t)q0 * rso, rso, lim, Qs, Qs + C::TILE,
                w);
    load_half_row_f32(Fg + q0, C::BQ, lim, Fs, w & 1);
  };
  const int nqb = (L + C::BQ - 1) / C::BQ;
  issue(0, 0);

  // ---- prologue: this lane's key k~ and v (B operands). A negative softmax
  // scale is applied as a sign flip of k~ in S (exact); dK~ then takes the
  // signed scale.
  const int kj = k0 + w * 32 + r;
  const uint32_t kflip = a.q_sign < 0.f ? 0x80008000u : 0u;
  // (branch-free loads of a clamped row, zeroed past the end: see the dq pass)
  const int kc = min(kj, L - 1);
  u32x4 kreg[C::NS], vreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    kreg[s] = ld16(Kg + kc * rs + 16 * s + 8 * g);
    vreg[s] = ld16(Vg + kc * rs + 16 * s + 8 * g);
  }
#pragma unroll
  for (int s = 0; s < C::NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kreg[s][e] = kj < L ? kreg[s][e] ^ kflip : 0u;
      vreg[s][e] = kj < L ? vreg[s][e] : 0u;
    }

  // blocks 1 .. NSTAGE-2 after the prologue's global loads (see the wait below)
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nqb) issue(j, j);

  const float c = a.c;
  const int xq = swz<D>(prow);
  const TrRows<D> tread(lane);  // transposed reads of the q~ and dO tiles
  f32x16 dvacc[C::ND], dkacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    dvacc[dt] = f32x16{};
    dkacc[dt] = f32x16{};
  }

  int stage = 0, next = C::NSTAGE - 1;
  // One query block; only the last block of a ragged sequence (FULL false)
  // carries the masking code.
  auto block = [&](int qb, auto full) {
    constexpr bool FULL = decltype(full)::value;
    // block qb's copies are done once at most the next block's are
    // outstanding; the barrier publishes them and frees stage `next`
    if (C::NSTAGE == 3 && qb + 1 < nqb)
      wait_vmem<C::LOADS>();
    else
      wait_vmem<0>();
    block_barrier();
    if (qb + C::NSTAGE - 1 < nqb) issue(qb + C::NSTAGE - 1, next);
    const uint16_t* Qs = lds + stage * C::STAGE;
    const uint16_t* Os = Qs + C::TILE;
    stage = stage + 1 == C::NSTAGE ? 0 : stage + 1;
    next = next + 1 == C::NSTAGE ? 0 : next + 1;
    const float* Fs = reinterpret_cast<const float*>(Qs + 2 * C::TILE);
    const int lim = L - qb * C::BQ;  // valid queries in this block

    // One 32-query tile at a time: S and dP, then P and dS, then the tile's
    // dV / dK products (keeps one tile's P and dS live, not the block's).
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const int rowoff = (32 * t + prow) * D;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        const int off = rowoff + 8 * ((2 * s + g) ^ xq);
        sacc = mfma32(ld16(Qs + off), kreg[s], sacc);
        pacc = mfma32(ld16(Os + off), vreg[s], pacc);
      }
      // dP - D on the matrix core (d <= 64; at d = 128 the extra operands
      // would spill): one more k-step whose A column pair holds -D of the
      // query row as a bf16 hi + lo split and whose B pair is (1, 1), so
      // every key column gets -D added in fp32
      if (C::FOLD_D) {
        const u32x4 a_negd = {g == 0 ? neg_bf16_pair(Fs[C::BQ + 32 * t + prow]) : 0u, 0u, 0u, 0u};
        const u32x4 b_one = {g == 0 ? kBf16OnePair : 0u, 0u, 0u, 0u};
        pacc = mfma32(a_negd, b_one, pacc);
      }
      // queries 32t + 16g + i, i = 0..15; P and dS overwrite S and dP
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 x = ld16(&Fs[32 * t + 16 * g + 4 * j]);
        u32x4 y = zero4();
        if (!C::FOLD_D) y = ld16(&Fs[C::BQ + 32 * t + 16 * g + 4 * j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          sacc[i] = fast_exp2(fmaf(sacc[i], c, -__uint_as_float(x[e])));
          pacc[i] = sacc[i] * (C::FOLD_D ? pacc[i] : pacc[i] - __uint_as_float(y[e]));
        }
      }
      if (!FULL) {  // queries past the end (copies of the last row): P = dS = 0
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * t + 16 * g + i >= lim) {
            sacc[i] = 0.f;
            pacc[i] = 0.f;
          }
      }
      u32x4 preg[2], dsreg[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          preg[hh][e] = pack_bf16(sacc[8 * hh + 2 * e], sacc[8 * hh + 2 * e + 1]);
          dsreg[hh][e] = pack_bf16(pacc[8 * hh + 2 * e], pacc[8 * hh + 2 * e + 1]);
        }
      // rows 32t .. 32t + 31 of the dO and q~ tiles, read along the rows
      const uint32_t orow = lds_addr(Os) + 32 * t * 2 * D, qrow = lds_addr(Qs) + 32 * t * 2 * D;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) {
        u32x4 ao[2], aq[2];
        tread.template read<2>(orow, dt, ao);
#pragma unroll
        for (int u = 0; u < 2; ++u) dvacc[dt] = mfma32(ao[u], preg[u], dvacc[dt]);
        tread.template read<2>(qrow, dt, aq);
#pragma unroll
        for (int u = 0; u < 2; ++u) dkacc[dt] = mfma32(aq[u], dsreg[u], dkacc[dt]);
      }
    }
  };
  const int nfull = L / C::BQ;
  for (int qb = 0; qb < nfull; ++qb) block(qb, Full{});
  if (nfull < nqb) block(nfull, Ragged{});
  __syncthreads();  // every wave is done with the tiles

  // ---- epilogue: dk = R(-p) scale dK~, dv
  float* F = reinterpret_cast<float*>(lds);
  constexpr int FP = D + 4;
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    const int d0 = 32 * dt + 16 * g;
    if (d0 < D) {
#pragma unroll
      for (int i = 0; i < 16; ++i) F[(w * 32 + r) * FP + d0 + i] = dkacc[dt][i] * a.scale;
    }
  }
  __syncthreads();
  const int64_t baseg = (int64_t)it.seq0 * a.ld_grad + (int64_t)h * D;
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dk + baseg, a.ld_grad, a.rope, true, tid);
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
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dv + baseg, a.ld_grad, a.rope, false, tid);
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
