// Backward attention kernels for gfx950. P is recomputed from the LSE the
// forward stored, so no L x L matrix is kept. q~ (from the rotation pass, or
// written by the forward that rotates its own query rows) carries
// softmax_scale * log2(e), so S' = q~ . k~ is the score in log2 units and
// P = exp2(S' - LSE log2 e).
//
// Two deterministic passes, no atomics:
//   dq pass : one workgroup per 128 queries of a (sequence, head) (lane owns a
//             query). Prologue computes D = rowsum(dO * O) for its queries and
//             stores it, with LSE log2 e, for the second pass. Per 64-key
//             block (32 at d=128): S'^T = K~ Q~^T, dP^T = V dO^T,
//             dS = P (dP - D), dQ~^T += K~^T dS^T.
//             Epilogue: dq = R(-p) (scale dQ~) -> bf16.
//   dkv pass: one workgroup per 128 keys (lane owns a key). Per 64-query block
//             (32 at d=128): S' = Q~ K~^T, dP = dO V^T, dS = P (dP - D),
//             dV^T += dO^T P, dK~^T += Q~^T dS. Epilogue:
//             dk = R(-p)(ln 2 dK~) (q~ carries the scale), dv -> bf16.
// Folds: S' - LSE log2 e and dP - D come out of the MFMAs themselves. One
// extra k-step multiplies (1, 1, 1) by the per-row (or per-column) value
// split into three bf16 values (k-slots 0..2), which replaces one vector
// FMA or subtraction per score: an MFMA blocks vector issue for fewer cycles
// than the 16 vector instructions of a 32x32 tile. In the dkv pass the
// values vary along the lane's 16 rows, so the dq pass stores them already
// split (drow: one 16-byte entry per row, -lse2 then -D) and the dkv pass
// reads them from LDS.
// q~ and k~ arrive rotated. The streamed operands (k~
// and v in the dq pass; q~, dO, LSE and D in the dkv pass) are copied from
// global memory into swizzled LDS tiles by global_load_lds, in a ring of
// three LDS stages (the copy of block b + 2 is issued right after the barrier
// that opens block b). Products that contract over the token axis (K~^T, Q~^T,
// dO^T) read the same row-major tiles with the LDS transpose load.
#include "common.h"
#include "prep.h"
#include "schedule.h"
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
  // launch bound (minimum workgroups per CU the register budget must allow);
  // up to d = 64 the pass fits three per CU anyway (152 VGPRs at d = 64)
  static constexpr int OCC = D == 128 ? 2 : 3;
  using Loader = TilePair<D, BN>;
  static constexpr int LOADS = Loader::LOADS_PER_WAVE;  // per wave and block
  // k-steps per batch of A-row reads (k~ and v rows, one wait per batch); at
  // d = 128 the rows are read one k-step at a time (no registers to spare)
  static constexpr int RB = D == 128 ? 0 : (NS < 4 ? NS : 4);
};

// (A wave whose rows all lie past the end skips the block work through a
// separate copies-and-barriers loop after the prologue, not an early exit
// inside the block body: that exit raised the pass's register use at d = 64
// from 152 to 174 VGPRs, three resident waves per SIMD to two.)
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
      qreg[s][e] = qvalid ? qreg[s][e] : 0u;
      doreg[s][e] = qvalid ? doreg[s][e] : 0u;
    }
  }
  if (!qvalid) dpart = 0.f;
  const float Dq = dpart + xor32(dpart);
  const float lse2 = qvalid ? lse_raw * kLog2e : 0.f;
  // S' - lse2 and dP - D in one more MFMA k-step each: A = (1, 1, 1), B = the
  // three-way bf16 split of -lse2 or -D, in the k-slots of lane half 0
  const u32x4 a_one = fold_ones(g);
  const u32x2 tlse = neg_bf16_triple(lse2), td = neg_bf16_triple(Dq);
  const u32x4 b_neglse = fold_operand(tlse, g), b_negd = fold_operand(td, g);
  if (qvalid && g == 0)  // -lse2 and -D, split, for the dkv pass's folds
    reinterpret_cast<u32x4*>(a.drow)[rowidx] = u32x4{tlse[0], tlse[1], td[0], td[1]};

  // blocks 1 .. NSTAGE-2 after the prologue's global loads (see the wait below)
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nkb) issue(j, j);

  const int xk = swz<D>(prow);
  // byte offset in a tile of the lane's A-operand row chunk for k-step s
  uint32_t lrow[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) lrow[s] = 2 * (prow * D + 8 * ((2 * s + g) ^ xk));
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
    const uint16_t* Ks = lds + stage * C::STAGE;  // then the v tile (+ TILE)
    stage = stage + 1 == C::NSTAGE ? 0 : stage + 1;
    next = next + 1 == C::NSTAGE ? 0 : next + 1;
    const int lim = L - kb * C::BN;  // valid keys in this block

    u32x4 dsreg[C::NU];
    // lane addresses of the A rows (keys prow of tile 0) of each k-step
    uint32_t arow[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) arow[s] = lds_addr(Ks) + lrow[s];
    auto tile = [&](auto tt) {
      constexpr int t = decltype(tt)::value;
      f32x16 sacc = mfma32(a_one, b_neglse, f32x16{});  // -lse2, then + S'
      f32x16 pacc = f32x16{};
      // S'^T += K~ Q~^T and dP^T += V dO^T: k~ rows of tile t, v rows (the next tile)
      if constexpr (C::RB > 0) {
        mfma_rows2<C::NS, C::RB, 64 * D * t, 2 * C::TILE + 64 * D * t>(arow, qreg, doreg, sacc,
                                                                        pacc);
      } else {
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
          const int off = (32 * t + prow) * D + 8 * ((2 * s + g) ^ xk);
          sacc = mfma32(ld16(Ks + off), qreg[s], sacc);
          pacc = mfma32(ld16(Ks + C::TILE + off), doreg[s], pacc);
        }
      }
      pacc = mfma32(a_one, b_negd, pacc);  // pacc = dP - D
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) dsv[i] = fast_exp2(sacc[i]) * pacc[i];
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
    };
    tile(std::integral_constant<int, 0>{});
    if constexpr (C::NT == 2) tile(std::integral_constant<int, 1>{});
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      u32x4 at[C::NU];
      kread.template read<C::NU>(lds_addr(Ks), dt, at);
#pragma unroll
      for (int u = 0; u < C::NU; ++u) dqacc[dt] = mfma32(at[u], dsreg[u], dqacc[dt]);
    }
  };
  const int nfull = L / C::BN;
  if (q0 + w * 32 < L) {
    for (int kb = 0; kb < nfull; ++kb) block(kb, Full{});
    if (nfull < nkb) block(nfull, Ragged{});
  } else {
    // a wave whose 32 queries all lie past the end of the sequence only takes
    // part in the copies and the barriers (the same waits, barriers and
    // issues as block(), one per key block); kept out of block() because an
    // early exit there raised the pass's register use by an occupancy level
    for (int kb = 0; kb < nkb; ++kb) {
      if (C::NSTAGE == 3 && kb + 1 < nkb)
        wait_vmem<C::LOADS>();
      else
        wait_vmem<0>();
      block_barrier();
      if (kb + C::NSTAGE - 1 < nkb) issue(kb + C::NSTAGE - 1, next);
      next = next + 1 == C::NSTAGE ? 0 : next + 1;
    }
  }
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
  // + the block's -lse2 and -D rows, split into three bf16 values (8 bytes)
  static constexpr int STAGE = 2 * TILE + 8 * BQ;
  static constexpr int NSTAGE = 3;              // LDS ring of query blocks
  static constexpr int EPI = BK * (D + 4) * 2;
  static constexpr int LDS = NSTAGE * STAGE > EPI ? NSTAGE * STAGE : EPI;
  static constexpr int OCC = D == 128 ? 2 : 3;
  using Loader = TilePair<D, BQ>;
  static constexpr int LOADS = Loader::LOADS_PER_WAVE + 1;  // + a quarter of the drow entries
  // k-steps per batch of A-row reads (q~ and dO rows, one wait per batch); at
  // d = 128 the rows are read one k-step at a time (no registers to spare)
  static constexpr int RB = D == 128 ? 0 : 1;
};

// Small-batch prologue of the dk/dv kernel (see SMALL below): the rotary
// table of positions 0 .. L-1 in LDS; for every row p < 128 the rotated
// q~ (times q_mul, as the rotation pass makes it) and dO into query stage
// p / 64, the rotated k~ into the k~ tile; the dS tile cleared; and per
// query row the fold operands -lse2 and -D formed exactly as the dq pass
// forms them (D = dO . O summed over d = 16 s + e, then over d = 16 s + 8 + e,
// then the two parts added). Rows past the end are zero.
template <int D, typename C>
__device__ __forceinline__ void small_prologue(const AttnArgs& a, uint16_t* lds, uint16_t* KTs,
                                               uint16_t* DSs, int L, int seq0, int h, int tid) {
  constexpr int TP = small_tab_pitch<D>();
  float2* tab = reinterpret_cast<float2*>(DSs + kSmallMaxLen * kSmallMaxLen);
  const bool rope = a.rope_base != 0.f;
  for (int i = tid; i < L * (D / 2); i += 256)
    tab[(i / (D / 2)) * TP + i % (D / 2)] =
        rope ? rope_cs(i / (D / 2), i % (D / 2), D, (double)a.rope_base)
             : make_float2(1.f, 0.f);
  for (int i = tid; i < kSmallMaxLen * kSmallMaxLen / 8; i += 256) st16(DSs + 8 * i, zero4());
  __syncthreads();
  const int rs = a.ld_qkv, rso = a.H * D;
  const uint16_t* __restrict__ Qg = a.q + (int64_t)seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Kg = a.k + (int64_t)seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ dOg = a.dout + (int64_t)seq0 * rso + (int64_t)h * D;
  const uint16_t* __restrict__ Og = a.o + (int64_t)seq0 * rso + (int64_t)h * D;
  for (int u = tid; u < kSmallMaxLen * (D / 16); u += 256) {
    const int p = u / (D / 16), c = u % (D / 16), j0 = 8 * c;
    u32x4 ql = zero4(), qh = zero4(), kl = zero4(), kh = zero4(), ol = zero4(), oh = zero4();
    if (p < L) {
      ql = ld16(Qg + p * rs + j0);
      qh = ld16(Qg + p * rs + j0 + D / 2);
      kl = ld16(Kg + p * rs + j0);
      kh = ld16(Kg + p * rs + j0 + D / 2);
      ol = ld16(dOg + p * rso + j0);
      oh = ld16(dOg + p * rso + j0 + D / 2);
      float lo[8], hi[8];
      unpack8(ql, lo);
      unpack8(qh, hi);
      if (rope) rotate8<false, false>(lo, hi, tab + p * TP + j0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] *= a.q_mul;
        hi[e] *= a.q_mul;
      }
      ql = pack8(lo);
      qh = pack8(hi);
      if (rope) {
        unpack8(kl, lo);
        unpack8(kh, hi);
        rotate8<false, false>(lo, hi, tab + p * TP + j0);
        kl = pack8(lo);
        kh = pack8(hi);
      }
    }
    uint16_t* Qs = lds + (p / C::BQ) * C::STAGE;
    const int row = p % C::BQ;
    st_row_halves<D>(Qs, row, c, ql, qh);
    st_row_halves<D>(Qs + C::TILE, row, c, ol, oh);
    st_row_halves<D>(KTs, p, c, kl, kh);
  }
  for (int p = tid; p < kSmallMaxLen; p += 256) {
    float lse2 = 0.f, Dq = 0.f;
    if (p < L) {
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          float fo[8], fd[8];
          unpack8(ld16(Og + p * rso + 16 * s + 8 * gg), fo);
          unpack8(ld16(dOg + p * rso + 16 * s + 8 * gg), fd);
#pragma unroll
          for (int e = 0; e < 8; ++e) part[gg] = fmaf(fd[e], fo[e], part[gg]);
        }
      Dq = part[0] + part[1];
      lse2 = a.lse_in[(int64_t)h * a.T + seq0 + p] * kLog2e;
    }
    const u32x2 tl = neg_bf16_triple(lse2), td = neg_bf16_triple(Dq);
    float* Fs = reinterpret_cast<float*>(lds + (p / C::BQ) * C::STAGE + 2 * C::TILE);
    reinterpret_cast<u32x4*>(Fs)[entry_slot(p % C::BQ)] = u32x4{tl[0], tl[1], td[0], td[1]};
  }
  __syncthreads();
}

// SMALL: the small-batch path (every sequence at most 128 tokens, d <= 64):
// one workgroup per (sequence, head), read from cu_seqlens, computes dq as
// well, so no dq pass runs. q and k are the raw inputs, rotated here as the
// rotation pass does (rotary table in LDS); the prologue also forms D and
// the fold operands the dq pass would have stored. The bf16 dS of every
// (key, query) pair is kept in an LDS tile [128 keys][128 queries]; after
// the query loop wave w computes dQ~^T of queries 32w .. 32w+31 as
// K~^T dS^T over all 128 keys, in the key order of the dq pass.
template <int D, bool ROPE, bool SMALL = false>
__global__ __launch_bounds__(256, SMALL ? 1 : DkvCfg<D>::OCC) void bwd_dkv_kernel(AttnArgs a) {
  using C = DkvCfg<D>;
  static_assert(!SMALL || (C::BQ == 64 && C::BK == kSmallMaxLen && C::NSTAGE >= 2), "small path");
  constexpr int KT = SMALL ? kSmallMaxLen * D : 0;                    // k~ tile [128][D]
  constexpr int DS = SMALL ? kSmallMaxLen * kSmallMaxLen : 0;         // dS tile [128][128]
  constexpr int TP = small_tab_pitch<D>();
  constexpr int TAB = SMALL ? kSmallMaxLen * TP * 4 : 0;              // float2 [128][TP]
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS + KT + DS + TAB];

  Item it;
  if constexpr (SMALL) {
    const int b = (int)blockIdx.x / a.H;
    it.head = (int)blockIdx.x - b * a.H;
    it.blk = 0;
    seq_bounds(a.cu, b, a.T, a.max_seqlen, &it.seq0, &it.len);
    it.len = min(it.len, kSmallMaxLen);
  } else {
    it = a.items[blockIdx.x];
  }
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
  const float* __restrict__ Fg = a.drow + 4 * row0;  // 16-byte (-lse2, -D) entries

  // q~, dO, lse2 and D rows of query block qb -> LDS stage `stage`
  const typename C::Loader loader(w, lane);
  auto issue = [&](int qb, int stage) {
    if constexpr (SMALL) return;  // every block is in LDS from the prologue
    const int q0 = qb * C::BQ, lim = L - q0;
    uint16_t* Qs = lds + stage * C::STAGE;
    float* Fs = reinterpret_cast<float*>(Qs + 2 * C::TILE);
    loader.load(Qg + (int64_t)q0 * rs, rs, dOg + (int64_t)q0 * rso, rso, lim, Qs, Qs + C::TILE,
                w);
    load_entries16(Fg + 4 * q0, C::BQ, lim, Fs, w);
  };
  const int nqb = (L + C::BQ - 1) / C::BQ;
  uint16_t* const KTs = lds + C::LDS;            // small path: k~ tile
  uint16_t* const DSs = KTs + KT;                // small path: dS tile
  const float2* const tab = reinterpret_cast<const float2*>(DSs + DS);
  if constexpr (SMALL) small_prologue<D, C>(a, lds, KTs, DSs, L, it.seq0, it.head, tid);
  else issue(0, 0);

  // ---- prologue: this lane's key k~ and v (B operands)
  const int kj = k0 + w * 32 + r;
  const bool live = k0 + w * 32 < L;  // wave-uniform
  // (branch-free loads of a clamped row, zeroed past the end: see the dq pass)
  const int kc = min(kj, L - 1);
  u32x4 kreg[C::NS], vreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    kreg[s] = SMALL ? ld16(KTs + tile_off<D>(kj, 2 * s + g)) : ld16(Kg + kc * rs + 16 * s + 8 * g);
    vreg[s] = ld16(Vg + kc * rs + 16 * s + 8 * g);
  }
#pragma unroll
  for (int s = 0; s < C::NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kreg[s][e] = kj < L ? kreg[s][e] : 0u;
      vreg[s][e] = kj < L ? vreg[s][e] : 0u;
    }

  // blocks 1 .. NSTAGE-2 after the prologue's global loads (see the wait below)
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nqb) issue(j, j);

  const int xq = swz<D>(prow);
  // byte offset in a tile of the lane's A-operand row chunk for k-step s
  uint32_t lrow[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) lrow[s] = 2 * (prow * D + 8 * ((2 * s + g) ^ xq));
  const TrRows<D> tread(lane);  // transposed reads of the q~ and dO tiles
  const u32x4 b_one = fold_ones(g);
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
    // a wave whose 32 rows all lie past the end of the sequence (the last,
    // partly filled item of a sequence) only takes part in the copies and the
    // barrier: its MFMA and vector work would produce nothing that is stored
    if (!live) return;
    const float* Fs = reinterpret_cast<const float*>(Qs + 2 * C::TILE);
    const int lim = L - qb * C::BQ;  // valid queries in this block

    // lane addresses of the A rows (queries prow of tile 0) of each k-step
    uint32_t arow[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) arow[s] = lds_addr(Qs) + lrow[s];

    // One 32-query tile at a time: S and dP, then P and dS, then the tile's
    // dV / dK products (keeps one tile's P and dS live, not the block's).
    auto tile = [&](auto tt) {
      constexpr int t = decltype(tt)::value;
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      {  // the A rows (queries 32t + prow) bring -lse2 and -D
        const u32x4 e = reinterpret_cast<const u32x4*>(Fs)[32 * t + entry_slot(prow)];
        sacc = mfma32(fold_operand(u32x2{e[0], e[1]}, g), b_one, sacc);
        pacc = mfma32(fold_operand(u32x2{e[2], e[3]}, g), b_one, pacc);
      }
      // S' += Q~ K~^T and dP += dO V^T: q~ rows of tile t, dO rows (the next tile)
      if constexpr (C::RB > 0) {
        mfma_rows2<C::NS, C::RB, 64 * D * t, 2 * C::TILE + 64 * D * t>(arow, kreg, vreg, sacc,
                                                                        pacc);
      } else {
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
          const int off = (32 * t + prow) * D + 8 * ((2 * s + g) ^ xq);
          sacc = mfma32(ld16(Qs + off), kreg[s], sacc);
          pacc = mfma32(ld16(Os + off), vreg[s], pacc);
        }
      }
      // queries 32t + 16g + i, i = 0..15; P and dS overwrite S' and dP
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = fast_exp2(sacc[i]);
        pacc[i] = sacc[i] * pacc[i];
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
      if constexpr (SMALL) {  // dS of key kj, queries 64 qb + 32 t + 16 g + 0..15
        if (kj < L) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            st16(DSs + tile_off<kSmallMaxLen>(kj, 8 * qb + 4 * t + 2 * g + hh), dsreg[hh]);
        }
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
    };
    tile(std::integral_constant<int, 0>{});
    if constexpr (C::NT == 2) tile(std::integral_constant<int, 1>{});
  };
  const int nfull = L / C::BQ;
  for (int qb = 0; qb < nfull; ++qb) block(qb, Full{});
  if (nfull < nqb) block(nfull, Ragged{});
  __syncthreads();  // every wave is done with the tiles

  float* F = reinterpret_cast<float*>(lds);
  constexpr int FP = D + 4;
  const float2* const rope = SMALL ? tab : a.rope;
  if constexpr (SMALL) {
    // dQ~^T of queries 32 w + perm_row(r) (B columns read through the
    // transposed dS tile) = K~^T dS^T over keys 0..63, then 64..127
    f32x16 qacc[C::ND];
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) qacc[dt] = f32x16{};
    if (32 * w < L) {
      const TrRows<kSmallMaxLen> dsread(lane);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 bs[4];
        dsread.template read<4>(lds_addr(DSs) + kb * 64 * 2 * kSmallMaxLen, w, bs);
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt) {
          u32x4 ak[4];
          tread.template read<4>(lds_addr(KTs) + kb * 64 * 2 * D, dt, ak);
#pragma unroll
          for (int u = 0; u < 4; ++u) qacc[dt] = mfma32(ak[u], bs[u], qacc[dt]);
        }
      }
    }
    __syncthreads();  // the tiles under F are no longer read
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      const int d0 = 32 * dt + 16 * g;
      if (d0 < D) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          F[(w * 32 + perm_row(r)) * FP + d0 + i] = qacc[dt][i] * a.scale;
      }
    }
    __syncthreads();
    store_rows<D, ROPE>(F, kSmallMaxLen, 0, L,
                        a.dq + (int64_t)it.seq0 * a.ld_grad + (int64_t)h * D, a.ld_grad, rope,
                        true, tid, TP);
    __syncthreads();
  }

  // ---- epilogue: dk = R(-p) ln2 dK~ (q~ carries softmax_scale log2 e), dv
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) {
    const int d0 = 32 * dt + 16 * g;
    if (d0 < D) {
#pragma unroll
      for (int i = 0; i < 16; ++i) F[(w * 32 + r) * FP + d0 + i] = dkacc[dt][i] * kLn2;
    }
  }
  __syncthreads();
  const int64_t baseg = (int64_t)it.seq0 * a.ld_grad + (int64_t)h * D;
  constexpr int rope_pitch = SMALL ? TP : D / 2;
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dk + baseg, a.ld_grad, rope, true, tid, rope_pitch);
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
  store_rows<D, ROPE>(F, C::BK, k0, L, a.dv + baseg, a.ld_grad, rope, false, tid, rope_pitch);
}

hipError_t launch_bwd_small(int head_dim, const AttnArgs& a, hipStream_t st) {
  const unsigned n = (unsigned)((int64_t)a.B * a.H);
  const bool rope = a.rope_base != 0.f;
  switch (head_dim) {
    case 16:
      if (rope) bwd_dkv_kernel<16, true, true><<<n, 256, 0, st>>>(a);
      else bwd_dkv_kernel<16, false, true><<<n, 256, 0, st>>>(a);
      break;
    case 32:
      if (rope) bwd_dkv_kernel<32, true, true><<<n, 256, 0, st>>>(a);
      else bwd_dkv_kernel<32, false, true><<<n, 256, 0, st>>>(a);
      break;
    case 64:
      if (rope) bwd_dkv_kernel<64, true, true><<<n, 256, 0, st>>>(a);
      else bwd_dkv_kernel<64, false, true><<<n, 256, 0, st>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
