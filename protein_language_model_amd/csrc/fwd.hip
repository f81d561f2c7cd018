// Forward attention kernel for gfx950: one workgroup (4 waves) per work item of
// 128 queries of one (sequence, head); each wave owns 32 queries.
//
// Data flow per item:
//   q~ rows (rotated once per token by the rotation pass, or rotated here in
//   the ROTQ mode below) sit in the MFMA B-operand registers for the whole
//   item.
//   For each block of 64 keys (32 at d = 128) the k~ and v rows are copied
//   from global memory into swizzled LDS tiles by global_load_lds (no register
//   staging, no vector instructions), in a ring of two LDS stages: the copy
//   of block kb + 1 is issued right after the barrier that opens block kb.
//   With two 16 KB stages and at most 128 VGPRs, four workgroups (four waves
//   per SIMD) are resident per CU at d <= 64. The MFMA phases (scores, P V)
//   run at raised wave priority, so a wave that reaches its matrix products
//   issues them ahead of the other waves' exponentials.
//   S^T = K~ Q~^T reads k~ rows; O^T += V^T P^T reads the v tile along its
//   key (row) axis with the LDS transpose load.
//   Lane (q, g) of a wave holds the scores of query q against 16 keys per
//   32-key tile; a row's values are split over lanes q and q + 32.
//
// Scores in log2 units: q~ is already multiplied by softmax_scale * log2(e)
// (by the rotation pass or the ROTQ prologue), so S' = q~ . k~ = S log2(e)
// and P = exp2(S' - m).
//
// Softmax (online, one pass over the keys). The running reference m is the
// exact row maximum of the first key block. Later blocks are exponentiated
// against it without computing their maximum: P = exp2(S' - m), and their
// sum l_blk is accumulated. The subtraction of m runs on the matrix core:
// one more MFMA per 32-key tile multiplies (1, 1, 1) by -m split into three
// bf16 values (k-slots 0..2), so the accumulator comes out as S' - m and each
// score costs one exp2, one add and half a conversion on the vector ALU (an
// MFMA blocks vector issue for fewer cycles than the 16 FMAs it replaces).
// Only if some lane's l_blk exceeds 2^16 (a score rose far above m, or exp2
// overflowed) does the wave compute the block maximum, raise m, rescale O
// and l by exp2(m_old - m_new) and redo the block. So every P ever used is
// at most 2^16, l and O stay far from fp32 overflow. P is rounded once to
// bf16 for the MFMA, and l sums exactly those bf16 values (dot2 against
// (1, 1)), so O is the weighted mean of v under the weights the product
// used: a dominant key's rounding (up to 2^-8 relative) cancels in O instead
// of scaling it, and the LSE is the log of that same normaliser, within
// ln(1 + 2^-8) of the exact one. Keys past the end of the sequence get
// S' = -inf, so P = 0. Epilogue: O = acc / l -> bf16; LSE = (m + log2 l) ln 2.
//
// Tiled attention keeps the L x L matrices on chip (BioNeMo blog, section 2.3
// describes the idea for another GPU); this kernel is laid out for the 64-wide
// wavefronts, 32x32x16 bf16 MFMA, LDS DMA and LDS transpose loads of CDNA4.
#include "common.h"
#include "prep.h"
#include "schedule.h"
#include "tile.h"

namespace esm {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;                  // queries per item
  static constexpr int BN = D == 128 ? 32 : 64;   // keys per block
  static constexpr int NS = D / 16;               // k-steps over d
  static constexpr int ND = D >= 32 ? D / 32 : 1; // 32-row d tiles of O^T
  static constexpr int NT = BN / 32;              // 32-key tiles per block
  static constexpr int NU = BN / 16;              // k-steps over keys
  static constexpr int TILE = BN * D;             // elements of one k~ or v tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NSTAGE = 2;                // LDS ring of key blocks
  static constexpr int LDS = NSTAGE * STAGE;
  // workgroups per CU: four at d <= 64 (two LDS stages of 16 KB, at most 128
  // VGPRs), two at d = 128
  static constexpr int OCC = D == 128 ? 2 : 4;
  using Loader = TilePair<D, BN>;
  // k-steps per batch of k~ row reads (both tiles' rows, one wait per batch)
  static constexpr int RB = NS < 2 ? NS : 2;
};

constexpr float kLazyBound = 65536.0f;  // 2^16: largest block sum of P kept

// SPLIT: key-range partials. Workgroup (x, y) attends the queries of item x
// to key chunk y of its sequence (the sequence's key blocks dealt out in
// n_split contiguous runs of ceil(blocks / n_split)) and writes the chunk's
// own normalised O_y (fp32) and LSE_y; an empty chunk writes 0 and -inf.
// merge_kernel then combines the chunks (split-KV: more work items when a
// batch has too few for the chip, and the per-device half of attention
// with keys sharded over devices). The grid's x extent is padded to
// B*H modulo 8 (padding workgroups exit), so that under round-robin
// dispatch chunk y of (sequence, head) group g runs on XCD (g + y*B*H) mod 8:
// few groups still spread over all eight XCDs, and each chunk's keys stay in
// one XCD's L2.
//
// SMALL: the small-batch path (every sequence at most 128 tokens, d <= 64),
// one launch with no plan: workgroup x is (sequence x / H, head x % H), read
// from cu_seqlens; q, k are the raw inputs, rotated here exactly as the
// rotation pass does (the rotary table built in LDS with the plan's formula),
// and the at most two key blocks of the sequence sit in the two LDS stages
// for the whole item.
//
// ROTQ: q is the raw query; each item rotates and scales its own query rows
// in registers with the plan's rotary table, the same float32 operations as
// the rotation pass (so O and LSE are bitwise those of the rotation pass
// followed by the plain forward), and writes those q~ rows to q_out when
// asked (for the backward), right after the first block's barrier so that
// the writes drain under the block's work. Only k then needs the rotation
// pass. q_out may be q itself: an item's query rows are read by no other
// workgroup, and its own waves load them before the first block barrier and
// store them after it.
template <int D, bool SPLIT, bool SMALL = false, bool ROTQ = false>
__global__ __launch_bounds__(256, SMALL ? 2 : FwdCfg<D>::OCC) void fwd_kernel(AttnArgs a) {
  using C = FwdCfg<D>;
  static_assert((int)SPLIT + (int)SMALL + (int)ROTQ <= 1, "one mode");
  static_assert(!SMALL || (C::BN == 64 && C::NSTAGE * C::BN >= kSmallMaxLen), "small path");
  // (the small path adds the rotary table of its positions: float2 [128][D/2])
  constexpr int TP = small_tab_pitch<D>();
  constexpr int TAB = SMALL ? kSmallMaxLen * TP * 4 : 0;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS + TAB];

  if (SPLIT && (int)blockIdx.x >= a.n_items) return;  // grid padding
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
  const int L = it.len, h = it.head, q0 = it.blk * C::BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5, prow = perm_row(r);
  const int rs = a.ld_qkv;  // row stride of q~, k~, v; T * rs < 2^31 is checked on the host
  const int64_t base = (int64_t)it.seq0 * rs + (int64_t)h * D;
  const uint16_t* __restrict__ Qg = a.q + base;
  // keys kbase .. kbase + Lk - 1 of the sequence (all of them unless SPLIT)
  int kbase = 0, Lk = L;
  if (SPLIT) {
    const int per = (((L + C::BN - 1) / C::BN) + a.n_split - 1) / a.n_split;  // blocks per chunk
    kbase = min((int)blockIdx.y * per * C::BN, L);
    Lk = min(per * C::BN, L - kbase);
  }
  const uint16_t* __restrict__ Kg = a.k + base + (int64_t)kbase * rs;
  const uint16_t* __restrict__ Vg = a.v + base + (int64_t)kbase * rs;
  const int qi = q0 + w * 32 + r;  // this lane's query
  const bool live = q0 + w * 32 < L;  // wave-uniform
  if (SPLIT && Lk <= 0) {  // empty chunk: O_y = 0, LSE_y = -inf
    if (qi < L) {
      float* Op = a.o_part + (((int64_t)blockIdx.y * a.T + it.seq0 + qi) * a.H + h) * D;
      for (int d0 = 16 * g; d0 < D; d0 += 32)
#pragma unroll
        for (int e = 0; e < 16; e += 4) *reinterpret_cast<f32x4*>(Op + d0 + e) = f32x4{};
      if (g == 0) a.lse_part[((int64_t)blockIdx.y * a.H + h) * a.T + it.seq0 + qi] = -INFINITY;
    }
    return;
  }

  // k~ and v rows of key block kb -> LDS stage `stage` (offsets kept in
  // registers for blocks with every key present)
  const typename C::Loader loader(w, lane);
  const typename C::Loader::Offsets koff = loader.offsets(rs, w);
  auto issue = [&](int kb, int stage) {
    if constexpr (SMALL) return;  // every block is in LDS from the prologue
    const int k0 = kb * C::BN;
    uint16_t* Ks = lds + stage * C::STAGE;
    if (k0 + C::BN <= Lk)
      loader.load_full(Kg + (int64_t)k0 * rs, Vg + (int64_t)k0 * rs, koff, Ks, Ks + C::TILE, w);
    else
      loader.template load<1>(Kg + (int64_t)k0 * rs, rs, Vg + (int64_t)k0 * rs, rs, Lk - k0, Ks,
                              Ks + C::TILE, w);
  };
  const int nkb = (Lk + C::BN - 1) / C::BN;
  const float2* tab = reinterpret_cast<const float2*>(lds + C::LDS);
  if constexpr (SMALL) {
    // rotary table of positions 0 .. L-1, then the rotated k~ rows and the v
    // rows of key block kb into stage kb (rows past the end zero)
    float2* tw = reinterpret_cast<float2*>(lds + C::LDS);
    const bool rope = a.rope_base != 0.f;
    for (int i = tid; i < L * (D / 2); i += 256)
      tw[(i / (D / 2)) * TP + i % (D / 2)] =
          rope ? rope_cs(i / (D / 2), i % (D / 2), D, (double)a.rope_base)
               : make_float2(1.f, 0.f);
    __syncthreads();
    for (int u = tid; u < nkb * C::BN * (D / 16); u += 256) {
      const int p = u / (D / 16), c = u % (D / 16), j0 = 8 * c;
      uint16_t* Ks = lds + (p / C::BN) * C::STAGE;
      const int row = p % C::BN;
      u32x4 kl = zero4(), kh = zero4(), vl = zero4(), vh = zero4();
      if (p < L) {
        kl = ld16(Kg + p * rs + j0);
        kh = ld16(Kg + p * rs + j0 + D / 2);
        vl = ld16(Vg + p * rs + j0);
        vh = ld16(Vg + p * rs + j0 + D / 2);
        if (rope) {
          float lo[8], hi[8];
          unpack8(kl, lo);
          unpack8(kh, hi);
          rotate8<false, false>(lo, hi, tab + p * TP + j0);
          kl = pack8(lo);
          kh = pack8(hi);
        }
      }
      st_row_halves<D>(Ks, row, c, kl, kh);
      st_row_halves<D>(Ks + C::TILE, row, c, vl, vh);
    }
  } else {
    issue(0, 0);
  }

  // queries: B operands (8 d values per k-step); rows past the end are zero.
  // The loads read a clamped row and are selected away afterwards: loads
  // under a branch would each be awaited at the branch's end, one memory
  // round trip per k-step.
  const int qc = min(qi, L - 1);
  u32x4 qreg[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) qreg[s] = ld16(Qg + qc * rs + 16 * s + 8 * g);
  // lane (r, g) holds d = 16 s + 8 g + e, whose rotary partner d + D/2 is in
  // k-step s + NS/2 of the same lane (d >= 32) or in lane ^ 32 (d = 16); the
  // pairs of rotation step s start at j = 16 s + 8 g (j = 0 at d = 16). The
  // position of row qc is qc itself (< max_seqlen, the table's rows).
  constexpr int NR = (C::NS + 1) / 2;  // rotation steps
  auto pair0 = [&](int s) { return C::NS == 1 ? 0 : 16 * s + 8 * g; };
  // ROTQ: the (cos, sin) of the lane's pairs come from the plan's table in
  // global memory. They are loaded here, next to the q rows and outside any
  // branch, so that the prologue waits for both at once (a load under a
  // branch is awaited at the branch's end: one more memory round trip per
  // item each). The table pointer is always valid memory; with the rotation
  // off its contents are not used.
  float2 csq[ROTQ ? NR : 1][8];
  if constexpr (ROTQ) {
#pragma unroll
    for (int s = 0; s < NR; ++s) load_cs8(a.rope, (int64_t)qc * (D / 2) + pair0(s), csq[s]);
    // (an empty asm that takes the values keeps the compiler from sinking
    // the loads into the branch below)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(csq[s][e].x), "+v"(csq[s][e].y));
  }
  if constexpr (SMALL || ROTQ) {
    // q~ = bf16(fl32(q_mul fl32(R(p) q))), as the rotation pass computes it
    const bool rope = a.rope_base != 0.f;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      u32x4 xl = qreg[s], xh;
      if constexpr (C::NS == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) xh[e] = __shfl_xor(xl[e], 32);
        if (g == 1) {
          const u32x4 t = xl;
          xl = xh;
          xh = t;
        }
      } else {
        xh = qreg[s + C::NS / 2];
      }
      float lo[8], hi[8];
      unpack8(xl, lo);
      unpack8(xh, hi);
      if (rope) rotate8<false, false>(lo, hi, SMALL ? tab + qc * TP + pair0(s) : csq[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] *= a.q_mul;
        hi[e] *= a.q_mul;
      }
      if constexpr (C::NS == 1) {
        qreg[0] = g == 0 ? pack8(lo) : pack8(hi);
      } else {
        qreg[s] = pack8(lo);
        qreg[s + C::NS / 2] = pack8(hi);
      }
    }
    if constexpr (SMALL) __syncthreads();  // the prologue's LDS tiles are complete
  }
#pragma unroll
  for (int s = 0; s < C::NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) qreg[s][e] = qi < L ? qreg[s][e] : 0u;
  // Blocks 1 .. NSTAGE-2 are issued after the q~ loads, so that the first
  // wait below (which lets one block's loads stay in flight) covers those.
#pragma unroll
  for (int j = 1; j < C::NSTAGE - 1; ++j)
    if (j < nkb) issue(j, j);

  const int xk = swz<D>(prow);  // swizzle of the lane's k~ rows 32t + prow
  // byte offset in the k~ tile of the lane's A-operand row chunk for k-step s
  uint32_t lrow[C::NS];
#pragma unroll
  for (int s = 0; s < C::NS; ++s) lrow[s] = 2 * (prow * D + 8 * ((2 * s + g) ^ xk));
  const TrRows<D> vread(lane);  // transposed reads of the v tile
  const u32x4 a_one = fold_ones(g);
  float m = 0.f, l = 0.f;       // m in log2 units
  u32x4 b_negm = u32x4{0u, 0u, 0u, 0u};  // -m in k-slots 0..2 (0 until block 0 sets m)
  f32x16 oacc[C::ND];
#pragma unroll
  for (int dt = 0; dt < C::ND; ++dt) oacc[dt] = f32x16{};

  int stage = 0;                 // LDS stage of block kb
  int next = C::NSTAGE - 1;      // LDS stage of block kb + NSTAGE - 1
  // One key block; FULL blocks have no key past the end of the sequence, so
  // only the last block of a ragged sequence carries the masking code.
  auto block = [&](int kb, auto full) {
    constexpr bool FULL = decltype(full)::value;
    // This wave's copies of block kb are done once at most the loads of the
    // blocks after it (NSTAGE - 2 of them, when they exist) are outstanding;
    // the barrier then publishes every wave's copies, and also tells that
    // stage `next` (last read for block kb - 1) is free again.
    if (C::NSTAGE == 3 && kb + 1 < nkb)
      wait_vmem<C::Loader::LOADS_PER_WAVE>();
    else
      wait_vmem<0>();
    block_barrier();
    if (kb + C::NSTAGE - 1 < nkb) issue(kb + C::NSTAGE - 1, next);
    if constexpr (ROTQ) {
      // q~ rows for the backward, written under the first block's work (at
      // the item's end they measured as an extra serial cost); every wave
      // has consumed its own q loads before this barrier, so in place is safe
      if (kb == 0 && a.q_out != nullptr && qi < L) {
        uint16_t* Qo = a.q_out + base + (int64_t)qi * rs;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) st16(Qo + 16 * s + 8 * g, qreg[s]);
      }
    }
    const uint16_t* Ks = lds + stage * C::STAGE;
    const uint16_t* Vs = Ks + C::TILE;
    stage = stage + 1 == C::NSTAGE ? 0 : stage + 1;
    next = next + 1 == C::NSTAGE ? 0 : next + 1;
    // a wave whose 32 rows all lie past the end of the sequence (the last,
    // partly filled item of a sequence) only takes part in the copies and the
    // barrier: its MFMA and vector work would produce nothing that is stored
    if (!live) return;

    // S'^T - m tiles: lane (q = r, g) register i of tile t = key 32t + 16g + i.
    // Keys past the end of the sequence get -inf, so P = 0.
    const int lim = Lk - kb * C::BN;  // valid keys in this block
    f32x16 sacc[C::NT];
    auto scores = [&]() {
      if constexpr (C::NT == 2) {
        // both 32-key tiles at once: k~ rows prow and 32 + prow of each k-step
        uint32_t arow[C::NS];
#pragma unroll
        for (int s = 0; s < C::NS; ++s) arow[s] = lds_addr(Ks) + lrow[s];
        sacc[0] = mfma32(a_one, b_negm, f32x16{});
        sacc[1] = sacc[0];
        mfma_rows2<C::NS, C::RB, 0, 64 * D>(arow, qreg, qreg, sacc[0], sacc[1]);
      } else {
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          sacc[t] = mfma32(a_one, b_negm, f32x16{});
          const uint16_t* Kr = Ks + (32 * t + prow) * D;
#pragma unroll
          for (int s = 0; s < C::NS; ++s)
            sacc[t] = mfma32(ld16(Kr + 8 * ((2 * s + g) ^ xk)), qreg[s], sacc[t]);
        }
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
    // P = bf16(exp2(acc - shift)) into preg (no subtraction at all on the
    // common path, NoShift); returns this lane's sum of those bf16 values
    u32x4 preg[C::NU];
    auto exponentiate = [&](auto shift) {
      constexpr bool SHIFT = !std::is_same<decltype(shift), NoShift>::value;
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sacc[t][i];
          if constexpr (SHIFT) x -= (float)shift;
          sacc[t][i] = fast_exp2(x);
        }
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
    wave_priority<1>();  // (MFMA phases at raised priority, see below)
    scores();
    wave_priority<0>();
    float lb;
    if (kb == 0) {  // no reference yet: the accumulator holds S'
      m = block_max();  // block 0 holds key 0, so m is finite
      b_negm = fold_operand(neg_bf16_triple(m), g);
      lb = exponentiate(m);
    } else {
      lb = exponentiate(NoShift{});
    }
    if (wave_any(!(lb <= kLazyBound))) {
      // rare: recompute S' - m, raise the reference to the new maximum, redo P
      scores();
      const float up = fmaxf(block_max(), 0.f);
      const float alpha = fast_exp2(-up);
      m += up;
      b_negm = fold_operand(neg_bf16_triple(m), g);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) oacc[dt] *= alpha;
      lb = exponentiate(up);
    }
    l += lb;

    wave_priority<1>();
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      u32x4 av[C::NU];
      vread.template read<C::NU>(lds_addr(Vs), dt, av);
#pragma unroll
      for (int u = 0; u < C::NU; ++u) oacc[dt] = mfma32(av[u], preg[u], oacc[dt]);
    }
    wave_priority<0>();
  };
  const int nfull = Lk / C::BN;
  for (int kb = 0; kb < nfull; ++kb) block(kb, Full{});
  if (nfull < nkb) block(nfull, Ragged{});

  // ---- epilogue
  l += xor32(l);
  if (SPLIT) {  // the chunk's O_y (fp32) and LSE_y
    if (qi < L) {
      const float inv = 1.0f / l;
      float* Op = a.o_part + (((int64_t)blockIdx.y * a.T + it.seq0 + qi) * a.H + h) * D;
#pragma unroll
      for (int dt = 0; dt < C::ND; ++dt) {
        const int d0 = 32 * dt + 16 * g;
        if (d0 < D) {
#pragma unroll
          for (int e = 0; e < 16; e += 4)
            *reinterpret_cast<f32x4*>(Op + d0 + e) =
                f32x4{oacc[dt][e] * inv, oacc[dt][e + 1] * inv, oacc[dt][e + 2] * inv,
                      oacc[dt][e + 3] * inv};
        }
      }
      if (g == 0)
        a.lse_part[((int64_t)blockIdx.y * a.H + h) * a.T + it.seq0 + qi] =
            (m + __log2f(l)) * kLn2;
    }
    return;
  }
  if (qi < L) {
    const float inv = 1.0f / l;
    const int rso = a.H * D;
    uint16_t* Og = a.out + (int64_t)(it.seq0 + qi) * rso + (int64_t)h * D;
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
    if (g == 0) a.lse[(int64_t)h * a.T + it.seq0 + qi] = (m + __log2f(l)) * kLn2;
  }
}

template <int D>
static void launch_fwd_d(const AttnArgs& a, unsigned n, int n_split, hipStream_t stream) {
  if (n_split > 0)
    fwd_kernel<D, true><<<dim3(n, (unsigned)n_split), 256, 0, stream>>>(a);
  else
    fwd_kernel<D, false><<<n, 256, 0, stream>>>(a);
}

hipError_t launch_fwd_small(int head_dim, const AttnArgs& a, hipStream_t stream) {
  const unsigned n = (unsigned)((int64_t)a.B * a.H);
  switch (head_dim) {
    case 16: fwd_kernel<16, false, true><<<n, 256, 0, stream>>>(a); break;
    case 32: fwd_kernel<32, false, true><<<n, 256, 0, stream>>>(a); break;
    case 64: fwd_kernel<64, false, true><<<n, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd_rotq(int head_dim, const AttnArgs& a, int64_t n_slots, hipStream_t stream) {
  const unsigned n = (unsigned)n_slots;
  switch (head_dim) {
    case 16: fwd_kernel<16, false, false, true><<<n, 256, 0, stream>>>(a); break;
    case 32: fwd_kernel<32, false, false, true><<<n, 256, 0, stream>>>(a); break;
    case 64: fwd_kernel<64, false, false, true><<<n, 256, 0, stream>>>(a); break;
    case 128: fwd_kernel<128, false, false, true><<<n, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(int head_dim, const AttnArgs& a, int64_t n_slots, bool split,
                      hipStream_t stream) {
  const unsigned n = (unsigned)n_slots;
  const int ns = split ? a.n_split : 0;
  switch (head_dim) {
    case 16: launch_fwd_d<16>(a, n, ns, stream); break;
    case 32: launch_fwd_d<32>(a, n, ns, stream); break;
    case 64: launch_fwd_d<64>(a, n, ns, stream); break;
    case 128: launch_fwd_d<128>(a, n, ns, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace esm
