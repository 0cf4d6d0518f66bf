// fa_bob.hip -- bf16 backward-over-backward passes for gfx950 with LDS DMA
// staging and transposing operand reads (fa_lds.h).
//
// Source: [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward
// for Softmax Attention", section 4.2 (affine fusion, Proposition 4.1 and the
// corrections (8)), section 4.3 (Algorithm 1, two passes), appendix D (final
// assembled identities).
//
// Work split: one workgroup = 4 waves = 128 resident rows (32 per wave, the
// N index of v_mfma_f32_32x32x16_bf16); the other side is streamed through
// LDS in tiles of TS rows, double buffered, filled by DMA.  Inside a tile the
// 32-row sub-tiles are software pipelined: while the elementwise work of
// sub-tile s runs on the VALU, the MFMA pipe computes the scores of s + 1 and
// the accumulations of s - 1.
#include <type_traits>

#include "fa_lds.h"
#include <utility>

namespace fa {

// Bias rows of the score chains: 0 for streamed rows < N, -inf past N (so
// that exp2 gives P = 0 there), for the tile starting at row0.
template <int TS>
__device__ inline void fill_bias(float* b, int row0, int N) {
  for (int x = threadIdx.x; x < TS; x += kThreads) b[x] = (row0 + x < N) ? 0.0f : -INFINITY;
}

// ---------------------------------------------------------------------------
// Matrix-core steps as inline assembly, so that the register class of every
// operand is fixed: score chains in VGPRs (the VALU consumes them), the
// output accumulators in AGPRs for the whole kernel, resident operands in
// AGPRs.  The wait states the hardware needs around v_mfma_f32_32x32x16_bf16
// (the same counts the compiler inserts for the builtin on gfx950) are
// explicit:
//   * a VALU write of an operand -> the MFMA reading it: 2 (s_nop 1 in front
//     of every MFMA whose B operand the VALU produced);
//   * an MFMA result -> a VALU or memory read of it: 12 (mfma_fence());
//   * an MFMA reading a VGPR as C -> a VALU write of it: 7 (C is always the
//     tied destination here, so the fence above covers it);
//   * back-to-back accumulation into the same registers needs none.

// d = a * b (a chain start; C = 0).
__device__ inline f32x16 mfma_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
// The same two with the two wait states of a VALU write in front: for kernels
// where the compiler, short of VGPRs, may copy a resident B operand back from
// AGPRs (v_accvgpr_read, a VALU instruction) right before the MFMA.
__device__ inline f32x16 mfma_first_w(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ inline void mfma_v_w(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// d = a * b (C = 0) with b resident in AGPRs.
__device__ inline f32x16 mfma_first_a(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
// d += a * b, d in VGPRs, b resident in AGPRs.
__device__ inline void mfma_va(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// d += a * b, all operands in VGPRs.
__device__ inline void mfma_v(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// acc += a * b, acc in AGPRs, b produced by the VALU.
__device__ inline void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Results of the chains above may be read by the VALU after this.
__device__ inline void mfma_fence(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
template <int NDB>
__device__ inline void acc_fence(f32x16 (&a)[NDB], f32x16 (&b)[NDB], f32x16 (&c)[NDB], f32x16 (&d)[NDB]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[db]), "+a"(b[db]), "+a"(c[db]), "+a"(d[db]));
}

template <int NDB>
__device__ inline void acc_fence1(f32x16 (&a)[NDB]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[db]));
}

template <int NDB>
__device__ inline void acc_fence2(f32x16 (&a)[NDB], f32x16 (&b)[NDB]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[db]), "+a"(b[db]));
}

// ---------------------------------------------------------------------------
// Pass 1 (row-major).  Resident per wave: query rows i with q_i, u_Q,i
// (scaled by pow2), do_i, L_i, D_i.  Streamed: K, V, U_K, U_V.  Per 32 x 32
// sub-tile (streamed index j on M):
//   S^T = K Q^T,  F^T = K U_Q^T + U_K Q^T,  dP^T = V dO^T,  C^T = U_V dO^T,
//   P = exp(tau S - L),  dPD = dP - D,  P~ = C + F dPD  (d~P before the
//   alpha correction), and the alpha-free accumulators of Proposition 4.1:
//     alpha += sum_j P F            E° += sum_j P P~
//     G     += P U_V + (P F) V      (d~(dO) before the correction)
//     Om    += (P P~) K + dS U_K    with dS = P dPD
//     R'    += dS K                 Bk += P K
// Epilogue (the corrections (8); R = R' + D Bk, so alpha R + E Bk =
// alpha R' + E° Bk):
//     E = E° - alpha D,  gdo = G - alpha o,  gq = tau (Om - alpha R' - E° Bk).
//
// Schedule of one tile (NSUB sub-tiles): scores(0); then for each sub-tile s
// the elementwise work of s interleaved with the accumulations of s - 1, and
// the scores of s + 1.
//
// SCHED = 1 is the second sweep of the three-pass schedule ([FlashBoB]
// appendix G.1): alpha is known (written by bob_alpha_dma_kernel), so
//   d~P = C + F dPD - alpha dP,  h = F - alpha,  E = sum_j P d~P directly,
//   G  += P U_V + (P h) V        (= gdo, no correction),
//   Om += (P d~P) K + dS U_K,    Bk += P K,      gq = tau (Om - E Bk)
// (the delayed E-correction), with one accumulation fewer than SCHED = 0.
//
// DROP (two-pass only): dropout with the forward's scaled keep mask g
// ([FlashBoB] appendix G, analytical dropout extension): dP and C become
// g dP and g C, and the products with V and U_V (the accumulator G) take
// P g and P F g; alpha, E°, Om, R' and Bk keep P.  The mask of each pair of
// sub-tiles comes from one shared generator call per lane (DropRow), issued
// while the score MFMAs of the first of them are in flight.
// KSPLIT: the key-split instance (a.ks > 1, see key_range): a range of the
// keys and raw partial sums instead of the epilogue.  Its own instance, so
// that the unsplit kernels keep their register allocation.
template <int D, int TS, bool RHO1, bool SPLIT, bool CAUSAL, int SCHED = 0, bool DROP = false, bool KSPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bob_pass1_dma_kernel(Args a) {
  static_assert(!(DROP && SCHED != 0), "the three-pass schedule has no dropout variant");
  static_assert(!KSPLIT || (!CAUSAL && SCHED == 0 && !DROP), "the key split serves the two-pass schedule only");
  static_assert(!DROP || TS % 64 == 0, "the mask comes in pairs of sub-tiles");
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int NSLICE = 2 * NDB;  // (d-block, k-step) pairs of one accumulation
  constexpr int STAGE = 4 * W::BYTES;
  static_assert(NSLICE == 4 || NSLICE == 8, "slices");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float kbias[TS];  // chain init of a ragged last tile
  // At d = 128 with dropout the mask words and the fifth operand chain leave
  // too few VGPRs for the resident U_Q rows (the AGPRs hold the four output
  // accumulators): each lane parks its U_Q fragments in LDS and reads them
  // back where the F chain takes them, instead of the compiler spilling to
  // scratch inside the tile loop.  That fills the 160 KB of LDS exactly, so
  // this instance masks a ragged last tile element by element instead of
  // keeping the bias row.
  constexpr int NPARK = DROP && D == 128 ? NKS : 0;
  __shared__ __attribute__((aligned(16))) bf16x8 uq_park[NPARK ? NPARK * kThreads : 1];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> q = head_of<bf16>(a.q, wk.b, wk.h), uq = head_of<bf16>(a.uq, wk.b, wk.h),
                      dout = head_of<bf16>(a.dout, wk.b, wk.h);
  HeadPtr<bf16> src[4] = {head_of<bf16>(a.k, wk.b, wk.hk), head_of<bf16>(a.v, wk.b, wk.hk),
                          head_of<bf16>(a.uk, wk.b, wk.hk), head_of<bf16>(a.uv, wk.b, wk.hk)};
  const int nt = (N + TS - 1) / TS;
  // Key tiles [t_begin, t_end).  Causal: key tiles past this row block's last
  // row are skipped, and the tiles from t_diag on cross the diagonal and are
  // masked element by element.  Key split (two-pass, no dropout): this
  // workgroup's range of the keys.
  int t_begin = 0, t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  if constexpr (KSPLIT) key_range(a, wk.kk, nt, t_begin, t_end);
  const int t_diag = CAUSAL ? wk.rb * kResRows / TS : nt;
  const bool ragged = !CAUSAL && (N % TS) != 0 && t_end == nt;

  // Start the first tile's copy before anything else.
  Dma<D, TS, 4> dma;
  dma.init(src);
  dma.copy(t_begin * TS, N, lds + (t_begin & 1) * STAGE);
  if constexpr (NPARK == 0) fill_bias<TS>(kbias, (nt - 1) * TS, N);

  bf16x8 qf[NKS], uqf[NKS], df[NKS];
  load_resident<bf16, D>(qf, q.p, q.sn, row, N, a.pow2);
  load_resident<bf16, D>(uqf, uq.p, uq.sn, row, N, a.pow2);
  load_resident<bf16, D>(df, dout.p, dout.sn, row, N, 1.0f);
#pragma unroll
  for (int ks = 0; ks < NPARK; ++ks) uq_park[ks * kThreads + threadIdx.x] = uqf[ks];
  // U_Q fragment ks: from the registers, or read back from this lane's own
  // LDS slot (volatile, so that the reads stay where they are used).
  auto uq_frag = [&](int ks) {
    if (ks < NPARK) return *reinterpret_cast<volatile bf16x8*>(&uq_park[ks * kThreads + threadIdx.x]);
    return uqf[ks];
  };
  const int64_t rv = (int64_t)wk.bh * N;
  const float Li = row < N ? a.lse[rv + row] : 0.0f;
  // Two-pass: D is computed here (no separate row-scalar kernel) and written
  // for the column pass; the three-pass row sweep reads the row-scalar kernel's.
  const float Di = SCHED == 0 ? resident_rowdot<D>(df, head_of<float>(a.o, wk.b, wk.h), row, N)
                              : (row < N ? a.D[rv + row] : 0.0f);
  const float nl2 = -Li * kLog2e;
  const float Ai = (SCHED == 1 && row < N) ? a.alpha[rv + row] : 0.0f;  // known alpha (three-pass)

  Reader<D, TS> rd;
  rd.init();

  f32x16 ag[NDB], aom[NDB], ar[NDB], abk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ag[db] = aom[db] = ar[db] = abk[db] = zero16();
    asm volatile("" : "+a"(ag[db]), "+a"(aom[db]), "+a"(ar[db]), "+a"(abk[db]));
  }
  // eob_p: E° summed from the bf16-rounded products P t0 that the matrix core
  // accumulates into Omega.  gQ = tau (Omega - alpha R' - E° B) uses it, so the
  // rounded operands cancel the way the exact ones do (Sum_j (P t0 - E° P) = 0;
  // on a row whose P sits on one key those terms cancel exactly).  E and the column
  // pass keep the unrounded E°.
  float alpha_p = 0.0f, eo_p = 0.0f, eob_p = 0.0f;
  // No load of the compiler's own may be outstanding inside the loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // Tile modes: 0 = every key valid, 1 = ragged last tile (chain init from
  // kbias), 2 = causal diagonal tile (chain init -inf where key > query).
  auto tile_body = [&](int t, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tk = lds + (t & 1) * STAGE;
    const char* tv = tk + W::BYTES;
    const char* tuk = tk + 2 * W::BYTES;
    const char* tuv = tk + 3 * W::BYTES;

    // The dropout instance runs short of VGPRs: its score MFMAs carry the
    // wait states of a VALU write themselves (see mfma_first_w).
    auto first = [&](bf16x8 x, bf16x8 y) { return DROP ? mfma_first_w(x, y) : mfma_first(x, y); };
    auto macc = [&](f32x16& z, bf16x8 x, bf16x8 y) {
      if constexpr (DROP) {
        mfma_v_w(z, x, y);
      } else {
        mfma_v(z, x, y);
      }
    };
    auto scores = [&](int sub, f32x16& s, f32x16& f, f32x16& dp, f32x16& c) {
      if constexpr (MODE == 1 && NPARK == 0) {
        s = row_init<TS>(kbias, sub);
      } else if constexpr (MODE == 1) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) s[idx] = (t * TS + sub * 32 + acc_pos(idx, hh) < N) ? 0.0f : -INFINITY;
        asm volatile("s_nop 1" : "+v"(s));  // VALU write -> MFMA read of C
      } else if constexpr (MODE == 2) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          s[idx] = (t * TS + sub * 32 + acc_pos(idx, hh) <= row) ? 0.0f : -INFINITY;
        asm volatile("s_nop 1" : "+v"(s));  // VALU write -> MFMA read of C
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 xk = rd_row<D, TS>(tk, rd, sub, ks);
        const bf16x8 xuk = rd_row<D, TS>(tuk, rd, sub, ks);
        const bf16x8 xv = rd_row<D, TS>(tv, rd, sub, ks);
        const bf16x8 xuv = rd_row<D, TS>(tuv, rd, sub, ks);
        if (MODE == 0 && ks == 0) {
          s = first(xk, qf[0]);
        } else {
          macc(s, xk, qf[ks]);
        }
        if (ks == 0) {
          f = first(xk, uq_frag(0));
          dp = first(xv, df[0]);
          c = first(xuv, df[0]);
        } else {
          macc(f, xk, uq_frag(ks));
          macc(dp, xv, df[ks]);
          macc(c, xuv, df[ks]);
        }
        macc(f, xuk, qf[ks]);
      }
    };
    // One (d-block, k-step) slice of the accumulations of sub-tile `sub`.
    // With DROP, cpf carries P F g and cpg P g (the operands of G).
    auto acc_slice = [&](int sub, int db, int s2, const Chain<bf16>& cp, const Chain<bf16>& cpf,
                         const Chain<bf16>& cpt, const Chain<bf16>& cds, const Chain<bf16>& cpg) {
      const bf16x8 xuv = rd_tr<D, TS>(tuv, rd, sub, db, s2);
      const bf16x8 xv = rd_tr<D, TS>(tv, rd, sub, db, s2);
      const bf16x8 xk = rd_tr<D, TS>(tk, rd, sub, db, s2);
      const bf16x8 xuk = rd_tr<D, TS>(tuk, rd, sub, db, s2);
      mfma_acc(ag[db], xuv, DROP ? cpg.f[s2] : cp.f[s2]);
      mfma_acc(ag[db], xv, cpf.f[s2]);
      mfma_acc(aom[db], xk, cpt.f[s2]);
      mfma_acc(aom[db], xuk, cds.f[s2]);
      if constexpr (SCHED == 0) mfma_acc(ar[db], xk, cds.f[s2]);
      mfma_acc(abk[db], xk, cp.f[s2]);
    };
    // Elementwise work on elements 4*part .. 4*part+3 of the current sub-tile.
    auto elementwise = [&](int part, const f32x16& s, const f32x16& f, const f32x16& dp, const f32x16& c,
                           Chain<bf16>& cp, Chain<bf16>& cpf, Chain<bf16>& cpt, Chain<bf16>& cds, Chain<bf16>& cpg,
                           const DropRow<2>& dm, int gsub) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * part + e;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], a.c1, nl2));
        const float F = RHO1 ? f[idx] : f[idx] * a.rho;
        if constexpr (DROP) {
          const float g = dm.at(a, gsub, idx);
          const float dpd = fmaf(g, dp[idx], -Di);
          const float pf = p * F, pt = p * fmaf(F, dpd, g * c[idx]);
          alpha_p += pf;
          eo_p += pt;
          const bf16 ptb = (bf16)pt;
          eob_p += (float)ptb;
          cp.f[idx >> 3][idx & 7] = (bf16)p;
          cpf.f[idx >> 3][idx & 7] = (bf16)(pf * g);
          cpt.f[idx >> 3][idx & 7] = ptb;
          cds.f[idx >> 3][idx & 7] = (bf16)(p * dpd);
          cpg.f[idx >> 3][idx & 7] = (bf16)(p * g);
          continue;
        }
        const float dpd = dp[idx] - Di;
        const float t0 = fmaf(F, dpd, c[idx]);
        if constexpr (SCHED == 0) {
          const float pf = p * F, pt = p * t0;
          alpha_p += pf;
          eo_p += pt;
          const bf16 ptb = (bf16)pt;
          eob_p += (float)ptb;
          cp.f[idx >> 3][idx & 7] = (bf16)p;
          cpf.f[idx >> 3][idx & 7] = (bf16)pf;
          cpt.f[idx >> 3][idx & 7] = ptb;
          cds.f[idx >> 3][idx & 7] = (bf16)(p * dpd);
        } else {
          // cpf carries P h, cpt carries P d~P; E is summed directly.
          const float pt = p * fmaf(-Ai, dp[idx], t0);
          eo_p += pt;
          const bf16 ptb = (bf16)pt;
          eob_p += (float)ptb;
          cp.f[idx >> 3][idx & 7] = (bf16)p;
          cpf.f[idx >> 3][idx & 7] = (bf16)(p * (F - Ai));
          cpt.f[idx >> 3][idx & 7] = ptb;
          cds.f[idx >> 3][idx & 7] = (bf16)(p * dpd);
        }
      }
    };

    f32x16 s, f, dp, c;
    scores(0, s, f, dp, c);
    Chain<bf16> pp, ppf, ppt, pds, ppg;  // chains of the previous sub-tile
    DropRow<2> dm;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      if constexpr (DROP) {
        if (sub % 2 == 0) dm.init(a, wk.bh, row, t * TS + sub * 32);
      }
      mfma_fence(s, f, dp, c);
      Chain<bf16> cp, cpf, cpt, cds, cpg;
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        elementwise(part, s, f, dp, c, cp, cpf, cpt, cds, cpg, dm, sub & 1);
        if constexpr (SPLIT) {
          // Parts 0-1 overlap the k-step-1 half of sub - 1; parts 2-3 the
          // k-step-0 half of this sub-tile (its chains come from parts 0-1).
          constexpr int H = NDB / 2;
          if (part < 2) {
            if (sub > 0) {
#pragma unroll
              for (int db = part * H; db < (part + 1) * H; ++db) acc_slice(sub - 1, db, 1, pp, ppf, ppt, pds, ppg);
            }
          } else {
#pragma unroll
            for (int db = (part - 2) * H; db < (part - 1) * H; ++db) acc_slice(sub, db, 0, cp, cpf, cpt, cds, cpg);
          }
        } else if (sub > 0) {
#pragma unroll
          for (int sl = part * NSLICE / 4; sl < (part + 1) * NSLICE / 4; ++sl)
            acc_slice(sub - 1, sl >> 1, sl & 1, pp, ppf, ppt, pds, ppg);
        }
      }
      pp = cp;
      ppf = cpf;
      ppt = cpt;
      pds = cds;
      if constexpr (DROP) ppg = cpg;
      if (sub + 1 < NSUB) scores(sub + 1, s, f, dp, c);
    }
    if constexpr (SPLIT) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_slice(NSUB - 1, db, 1, pp, ppf, ppt, pds, ppg);
    } else {
#pragma unroll
      for (int sl = 0; sl < NSLICE; ++sl) acc_slice(NSUB - 1, sl >> 1, sl & 1, pp, ppf, ppt, pds, ppg);
    }
  };

  // Tiles [t0, t1) in one mode.  Each mode is its own loop, so the
  // accumulators keep one register assignment per loop; the fence at the end
  // covers any copy the compiler places between loops.
  auto run = [&](int t0, int t1, auto mode_c) {
    for (int t = t0; t < t1; ++t) {
      // This wave's copies of tile t are done; the barrier makes every
      // wave's copies visible and guarantees that no wave still reads the
      // other stage.
      dma_wait();
      __syncthreads();
      if (t + 1 < t_end) dma.copy((t + 1) * TS, N, lds + ((t + 1) & 1) * STAGE);
      tile_body(t, mode_c);
    }
    acc_fence<NDB>(ag, aom, ar, abk);
  };
  if constexpr (CAUSAL) {
    run(0, t_diag, std::integral_constant<int, 0>{});
    run(t_diag, t_end, std::integral_constant<int, 2>{});
  } else {
    run(t_begin, ragged ? nt - 1 : t_end, std::integral_constant<int, 0>{});
    if (ragged) run(nt - 1, nt, std::integral_constant<int, 1>{});
  }

  acc_fence<NDB>(ag, aom, ar, abk);
  // SCHED 0: alpha and E° from the sweep; SCHED 1: alpha known, E summed.
  const float alpha = SCHED == 0 ? half_sum(alpha_p) : Ai;
  const float esum = half_sum(eo_p);
  const float eo = SCHED == 0 ? esum : esum + Ai * Di;  // E° = E + alpha D
  const float eob = half_sum(eob_p);
  if constexpr (KSPLIT) {
    // Key split: this key range's raw sums; bob_ksplit_sum_kernel does the rest.
    if (row < N && hh == 0) {
      kpart_rowsum(a, wk.kk, 0, wk.bh)[row] = alpha;
      kpart_rowsum(a, wk.kk, 1, wk.bh)[row] = eo;
      kpart_rowsum(a, wk.kk, 2, wk.bh)[row] = eob;
      if (wk.kk == 0) a.D[rv + row] = Di;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      store_out(kpart_acc<D>(a, wk.kk, 0, wk.bh), D, row, N, db, [&](int idx) { return ag[db][idx]; });
      store_out(kpart_acc<D>(a, wk.kk, 1, wk.bh), D, row, N, db, [&](int idx) { return aom[db][idx]; });
      store_out(kpart_acc<D>(a, wk.kk, 2, wk.bh), D, row, N, db, [&](int idx) { return ar[db][idx]; });
      store_out(kpart_acc<D>(a, wk.kk, 3, wk.bh), D, row, N, db, [&](int idx) { return abk[db][idx]; });
    }
    return;
  }
  if (row < N && hh == 0) {
    if constexpr (SCHED == 0) {
      a.alpha[rv + row] = alpha;
      a.D[rv + row] = Di;
    }
    a.E[rv + row] = SCHED == 0 ? eo - alpha * Di : esum;
  }
  if (hh == 0) {
    // Chain inits of the column pass for this row (see bob_pass2_dma_kernel):
    // -L/rho, -D, -alpha/rho, -(alpha D + E) = -E°; rows past N get
    // (-inf, 0, 0, 0), which masks them there.
    float* ps = a.ps + ((int64_t)wk.bh * ((N + kPsRows - 1) / kPsRows) + row / kPsRows) * 4 * kPsRows + row % kPsRows;
    const bool ok = row < N;
    const float irho = 1.0f / a.rho;
    ps[0] = ok ? -Li * irho : -INFINITY;
    ps[kPsRows] = ok ? -Di : 0.0f;
    ps[2 * kPsRows] = ok ? -alpha * irho : 0.0f;
    ps[3 * kPsRows] = ok ? -eo : 0.0f;
  }
  const HeadPtr<float> o = head_of<float>(a.o, wk.b, wk.h);
  float* gq = head_out(a.r0, wk.b, wk.h);
  float* gdo = head_out(a.r3, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    if constexpr (SCHED == 0) {
      float ov[16];
      if (row < N) {
        const float* orow = o.p + (int64_t)row * o.sn + db * 32 + 4 * hh;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(orow + 8 * b4);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[4 * b4 + e] = x[e];
        }
      }
      store_out(gdo, a.r3.sn, row, N, db, [&](int idx) { return ag[db][idx] - alpha * ov[idx]; });
      store_out(gq, a.r0.sn, row, N, db,
                [&](int idx) { return a.tau * (aom[db][idx] - alpha * ar[db][idx] - eob * abk[db][idx]); });
    } else {
      store_out(gdo, a.r3.sn, row, N, db, [&](int idx) { return ag[db][idx]; });
      store_out(gq, a.r0.sn, row, N, db, [&](int idx) { return a.tau * (aom[db][idx] - eob * abk[db][idx]); });
    }
  }
}


// ---------------------------------------------------------------------------
// alpha sweep: the first pass of the three-pass schedule ([FlashBoB]
// appendix G.1), kept for the schedule ablation.  Streams only K and U_K
// (the operands of F):  alpha_i = sum_j P_ij F_ij  with
//   S^T = K Q^T,  F^T = K U_Q^T + U_K Q^T,  P = exp(tau S - L).
// The score chains of sub-tile s + 1 are issued before the elementwise work
// of sub-tile s, so the matrix cores and the VALU overlap.
template <int D, int TS, bool RHO1, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bob_alpha_dma_kernel(Args a) {
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NSUB = TS / 32;
  constexpr int STAGE = 2 * W::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float kbias[TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> q = head_of<bf16>(a.q, wk.b, wk.h), uq = head_of<bf16>(a.uq, wk.b, wk.h);
  HeadPtr<bf16> src[2] = {head_of<bf16>(a.k, wk.b, wk.hk), head_of<bf16>(a.uk, wk.b, wk.hk)};
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  const int t_diag = CAUSAL ? wk.rb * kResRows / TS : nt;
  const bool ragged = !CAUSAL && (N % TS) != 0;

  Dma<D, TS, 2> dma;
  dma.init(src);
  dma.copy(0, N, lds);
  fill_bias<TS>(kbias, (nt - 1) * TS, N);

  bf16x8 qf[NKS], uqf[NKS];
  load_resident<bf16, D>(qf, q.p, q.sn, row, N, a.pow2);
  load_resident<bf16, D>(uqf, uq.p, uq.sn, row, N, a.pow2);
  const int64_t rv = (int64_t)wk.bh * N;
  const float Li = row < N ? a.lse[rv + row] : 0.0f;
  const float nl2 = -Li * kLog2e;

  Reader<D, TS> rd;
  rd.init();
  float alpha_p = 0.0f;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load of the compiler's own in the loop

  auto tile_body = [&](int t, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tk = lds + (t & 1) * STAGE;
    const char* tuk = tk + W::BYTES;
    auto scores = [&](int sub, f32x16& s, f32x16& f) {
      if constexpr (MODE == 1) {
        s = row_init<TS>(kbias, sub);
      } else if constexpr (MODE == 2) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          s[idx] = (t * TS + sub * 32 + acc_pos(idx, hh) <= row) ? 0.0f : -INFINITY;
        asm volatile("s_nop 1" : "+v"(s));  // VALU write -> MFMA read of C
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 xk = rd_row<D, TS>(tk, rd, sub, ks);
        const bf16x8 xuk = rd_row<D, TS>(tuk, rd, sub, ks);
        if (MODE == 0 && ks == 0) {
          s = mfma_first(xk, qf[0]);
        } else {
          mfma_v(s, xk, qf[ks]);
        }
        if (ks == 0) {
          f = mfma_first(xk, uqf[0]);
        } else {
          mfma_v(f, xk, uqf[ks]);
        }
        mfma_v(f, xuk, qf[ks]);
      }
    };
    f32x16 s[2], f[2];
    scores(0, s[0], f[0]);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x16& sc = s[sub & 1];
      f32x16& fc = f[sub & 1];
      asm volatile("s_nop 7\n\ts_nop 4" : "+v"(sc), "+v"(fc));  // MFMA result -> VALU read
      if (sub + 1 < NSUB) scores(sub + 1, s[(sub + 1) & 1], f[(sub + 1) & 1]);
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[idx], a.c1, nl2));
        alpha_p = fmaf(p, RHO1 ? fc[idx] : fc[idx] * a.rho, alpha_p);
      }
    }
  };
  auto run = [&](int t0, int t1, auto mode_c) {
    for (int t = t0; t < t1; ++t) {
      dma_wait();
      __syncthreads();
      if (t + 1 < t_end) dma.copy((t + 1) * TS, N, lds + ((t + 1) & 1) * STAGE);
      tile_body(t, mode_c);
    }
  };
  if constexpr (CAUSAL) {
    run(0, t_diag, std::integral_constant<int, 0>{});
    run(t_diag, t_end, std::integral_constant<int, 2>{});
  } else {
    run(0, ragged ? nt - 1 : nt, std::integral_constant<int, 0>{});
    if (ragged) run(nt - 1, nt, std::integral_constant<int, 1>{});
  }
  const float alpha = half_sum(alpha_p);
  if (row < N && hh == 0) a.alpha[rv + row] = alpha;
}

// ---------------------------------------------------------------------------
// Pass 2 (column-major).  Resident per wave: 32 key rows j with k_j, u_K,j
// (scaled by pow2), v_j, u_V,j.  Streamed: Q, dO, U_Q, and per streamed row
// the chain inits written by pass 1: -L/rho, -D, -alpha/rho, -(alpha D + E).
// Per 32 x 32 sub-tile (streamed index i on M):
//   s = (tau S - L)/rho,  h/rho = (F - alpha)/rho,  dPD = dP - D,
//   C' = C - alpha D - E,
//   P = exp(tau S - L),   d~P - E = C' + h dPD,
//   d~S = P (d~P - E),    dS = P dPD,    W = P h,
//   gk += d~S^T Q + dS^T U_Q (times tau at the end),  gv += W^T dO.
// Same tile schedule as pass 1.
//
// DROP (split schedule only): dropout with the forward's scaled keep mask g
// ([FlashBoB] appendix G, analytical dropout extension): dP = g (dO V^T) - D
// and C' = g (dO U_V^T) - alpha D - E, so these two chains start at 0 and take
// their staged scalars after the mask; W = P g h.  The mask of each pair of
// sub-tiles comes from one shared generator call per lane (DropCol).
// TWO: two waves per SIMD (two workgroups per CU, 256 registers a wave), for
// the split schedule at d = 64 (with dropout only without the causal mask);
// the launch uses it only for grids of whole multiples of 512 workgroups.
template <int D, int TS, bool RHO1, bool SPLIT, bool RESA, bool CAUSAL, bool DROP = false, bool TWO = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TWO ? 2 : 1, TWO ? 2 : 1))) void
bob_pass2_dma_kernel(Args a) {
  static_assert(!DROP || (SPLIT && TS % 64 == 0), "dropout runs the split schedule on pairs of sub-tiles");
  static_assert(!TWO || (D == 64 && SPLIT && !(DROP && CAUSAL)), "the two-wave instance is the d = 64 split schedule");
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int NSLICE = 2 * NDB;
  constexpr int TBYTES = 3 * W::BYTES;
  constexpr int SBYTES = 4 * TS * 4;
  constexpr int STAGE = TBYTES + SBYTES;
  static_assert(kPsRows % TS == 0 && (TS == 64 || TS == 128), "tiles split the staged scalar blocks");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

  const Work wk = work_item_cols(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int col = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> k = head_of<bf16>(a.k, wk.b, wk.hk), v = head_of<bf16>(a.v, wk.b, wk.hk),
                      uk = head_of<bf16>(a.uk, wk.b, wk.hk), uv = head_of<bf16>(a.uv, wk.b, wk.hk);
  // Streamed: the G query heads of this key/value head in sequence (the
  // key-side outputs sum over the group, [FlashBoB] section 4.3).
  HeadPtr<bf16> src[3] = {head_of<bf16>(a.q, wk.b, wk.h), head_of<bf16>(a.dout, wk.b, wk.h),
                          head_of<bf16>(a.uq, wk.b, wk.h)};
  const int64_t hstride[3] = {a.q.sh, a.dout.sh, a.uq.sh};
  const int nt = (N + TS - 1) / TS;
  const int64_t ps_head = (int64_t)((N + kPsRows - 1) / kPsRows) * 4 * kPsRows;  // floats per query head
  const float* ps0 = a.ps + ((int64_t)wk.b * a.H + wk.h) * ps_head;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  Dma<D, TS, 3> dma;
  dma.init(src, hstride);
  // Tile t of query head h + g into dst.
  auto copy_tile = [&](int g, int t, const char* dst) {
    dma.copy(t * TS, N, dst, g);
    // The tile's chain inits, [4][TS] floats: TS / 64 wave-wide copies.  Lane l
    // of copy w moves rows 4 (l % 16) .. +3 of init (4 w + l / 16) % 4 ...
    if (wave < SBYTES / 1024) {
      const int r0 = t * TS;
      const int e = (wave * 64 + l) * 4;  // float index inside the [4][TS] block
      const int kk = e / TS, rr = e % TS;
      const float* src_ps = ps0 + g * ps_head + ((int64_t)(r0 / kPsRows) * 4 + kk) * kPsRows + r0 % kPsRows + rr;
      dma16(src_ps, lds_addr(dst + TBYTES + wave * 1024));
    }
  };
  // Causal: query tiles before this key block's first key are skipped; tiles
  // below t_diag cross the diagonal and are masked element by element.
  // A row split (non-causal only) gives this workgroup tiles [t_begin, t_end)
  // of every query head; its key-side sums are one partial of the block's.
  const int t_begin = CAUSAL ? wk.rb * kResRows / TS : (int)((int64_t)nt * wk.rr / a.rs);
  const int t_end = CAUSAL ? nt : (int)((int64_t)nt * (wk.rr + 1) / a.rs);
  const int t_diag = CAUSAL ? (wk.rb * kResRows + kResRows + TS - 1) / TS : 0;
  copy_tile(0, t_begin, lds);

  bf16x8 kf[NKS], ukf[NKS], vf[NKS], uvf[NKS];
  load_resident<bf16, D>(kf, k.p, k.sn, col, N, a.pow2);
  load_resident<bf16, D>(ukf, uk.p, uk.sn, col, N, a.pow2);
  load_resident<bf16, D>(vf, v.p, v.sn, col, N, 1.0f);
  load_resident<bf16, D>(uvf, uv.p, uv.sn, col, N, 1.0f);
  if constexpr (RESA) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(vf[ks]), "+a"(uvf[ks]));
  }
  if constexpr (!SPLIT) {
    // The woven schedule reads every resident operand from AGPRs, so that
    // the compiler has no reason to copy one into VGPRs in front of an MFMA.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(ukf[ks]), "+a"(vf[ks]), "+a"(uvf[ks]));
  }

  Reader<D, TS> rd;
  rd.init();

  f32x16 ak[NDB], av[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ak[db] = av[db] = zero16();
    asm volatile("" : "+a"(ak[db]), "+a"(av[db]));
  }
  // No load of the compiler's own may be outstanding inside the loop.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // Tile modes: 0 = rows masked only through the staged inits, 2 = causal
  // diagonal tile (also -inf where query < key).
  // Tile t in LDS buffer buf.
  // Tile t of query head wk.h + gq in LDS buffer buf.
  auto tile_body = [&](int t, int buf, int gq, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tq = lds + buf * STAGE;
    const char* tdo = tq + W::BYTES;
    const char* tuq = tq + 2 * W::BYTES;
    const float* sc = reinterpret_cast<const float*>(tq + TBYTES);

    auto scores = [&](int sub, f32x16& s, f32x16& f, f32x16& dp, f32x16& c) {
      s = row_init<TS>(sc, sub);
      if constexpr (MODE == 2) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          if (t * TS + sub * 32 + acc_pos(idx, hh) < col) s[idx] = -INFINITY;
        asm volatile("s_nop 1" : "+v"(s));  // VALU write -> MFMA read of C
      }
      // With DROP the dP and C chains start at 0: their first MFMA takes the
      // literal 0 as C, so no zero-filled registers (which the compiler
      // would copy in with a VALU write right before the MFMA) are read.
      if constexpr (!DROP) {
        dp = row_init<TS>(sc + TS, sub);
        c = row_init<TS>(sc + 3 * TS, sub);
      }
      f = row_init<TS>(sc + 2 * TS, sub);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 xq = rd_row<D, TS>(tq, rd, sub, ks);
        const bf16x8 xuq = rd_row<D, TS>(tuq, rd, sub, ks);
        const bf16x8 xd = rd_row<D, TS>(tdo, rd, sub, ks);
        // The causal and the dropout two-wave instances, short of registers,
        // copy K and U_K back from AGPRs right before these: their MFMAs
        // carry the wait.
        if constexpr (TWO && (CAUSAL || DROP)) {
          mfma_v_w(s, xq, kf[ks]);
          mfma_v_w(f, xuq, kf[ks]);
          mfma_v_w(f, xq, ukf[ks]);
        } else {
          mfma_v(s, xq, kf[ks]);
          mfma_v(f, xuq, kf[ks]);
          mfma_v(f, xq, ukf[ks]);
        }
        if (DROP && ks == 0) {
          dp = RESA ? mfma_first_a(xd, vf[0]) : mfma_first(xd, vf[0]);
          c = RESA ? mfma_first_a(xd, uvf[0]) : mfma_first(xd, uvf[0]);
        } else if constexpr (RESA) {
          mfma_va(dp, xd, vf[ks]);
          mfma_va(c, xd, uvf[ks]);
        } else {
          mfma_v(dp, xd, vf[ks]);
          mfma_v(c, xd, uvf[ks]);
        }
      }
    };
    auto acc_slice = [&](int sub, int db, int s2, const Chain<bf16>& cdt, const Chain<bf16>& cds,
                         const Chain<bf16>& cw) {
      const bf16x8 xq = rd_tr<D, TS>(tq, rd, sub, db, s2);
      const bf16x8 xuq = rd_tr<D, TS>(tuq, rd, sub, db, s2);
      const bf16x8 xd = rd_tr<D, TS>(tdo, rd, sub, db, s2);
      mfma_acc(ak[db], xq, cdt.f[s2]);
      mfma_acc(ak[db], xuq, cds.f[s2]);
      mfma_acc(av[db], xd, cw.f[s2]);
    };
    // With DROP, dm holds the mask of the sub-tile pair and the part's four
    // staged -D and -(alpha D + E) are read from the tile's chain inits here
    // (one 16-byte LDS read each), not held for the whole sub-tile.
    auto elementwise = [&](int part, const f32x16& s, const f32x16& f, const f32x16& dp, const f32x16& c,
                           Chain<bf16>& cdt, Chain<bf16>& cds, Chain<bf16>& cw, int sub,
                           const DropCol<2>& dm) {
      f32x4 nd, nc;
      if constexpr (DROP) {
        const int o = sub * 32 + sig(8 * part + 4 * hh);
        nd = *reinterpret_cast<const f32x4*>(sc + TS + o);
        nc = *reinterpret_cast<const f32x4*>(sc + 3 * TS + o);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * part + e;
        const float p = __builtin_amdgcn_exp2f(s[idx] * a.c1);
        const float h = RHO1 ? f[idx] : f[idx] * a.rho;
        if constexpr (DROP) {
          const float g = dm.at(a, sub & 1, idx);
          const float dpx = fmaf(g, dp[idx], nd[e]);
          cdt.f[idx >> 3][idx & 7] = (bf16)(p * fmaf(h, dpx, fmaf(g, c[idx], nc[e])));
          cds.f[idx >> 3][idx & 7] = (bf16)(p * dpx);
          cw.f[idx >> 3][idx & 7] = (bf16)(p * g * h);
          continue;
        }
        const float x = fmaf(h, dp[idx], c[idx]);
        cdt.f[idx >> 3][idx & 7] = (bf16)(p * x);
        cds.f[idx >> 3][idx & 7] = (bf16)(p * dp[idx]);
        cw.f[idx >> 3][idx & 7] = (bf16)(p * h);
      }
    };

    // Woven schedule (d = 64, one wave per SIMD).  The wave issues in order,
    // so the matrix core only stays busy if the work between two MFMAs takes
    // no longer than one MFMA (32 cycles).  Per sub-tile sub the MFMAs are
    // the accumulations of sub-tile sub - 1 (12) and then the scores of
    // sub-tile sub + 1 (20); the elementwise work of sub-tile sub is cut into
    // 32 parts of at most six VALU instructions, one after each MFMA:
    //   E(e)  P of element e (one exp),
    //   A(j)  the P x chain of element pair j,
    //   B(j)  the P dP and P h chains of pair j,
    // in the order E0..E3, then A(j) B(j) E(2j+4) E(2j+5) for j = 0..5, then
    // A6 B6 A7 B7, so that every exp has two slots to finish before its P is
    // used.  Scheduling barriers hold this order.  The LDS operands of an MFMA
    // are loaded at least three MFMAs ahead: the transposed operands of the
    // accumulations two slices ahead (across sub-tiles), the score rows one
    // k-step ahead, and the chain inits of sub-tile sub + 1 during the
    // accumulations.  Score sets and operand chains alternate between two
    // register sets by sub-tile parity.
    auto woven = [&]() {
      f32x16 cs[2][4];        // [set][S, F, dP, C]
      Chain<bf16> ch[2][3];   // [set][P x, P dP, P h]
      float pv[16];           // P of the sub-tile in work
      bf16x8 ta[2][3];        // transposed operands of two slices: [slice & 1][Q, U_Q, dO]
      bf16x8 xr[3];           // score operands of one k-step: [Q, U_Q, dO]

      // Transposed operand k of slice sl (d-block sl % NDB, half sl / NDB) of
      // sub-tile sub into ta[sl & 1][k].
      auto load_tr = [&](int sub, int sl, int k) {
        const char* tile = k == 0 ? tq : (k == 1 ? tuq : tdo);
        ta[sl & 1][k] = rd_tr<D, TS>(tile, rd, sub, sl % NDB, sl / NDB);
      };
      auto load_row = [&](int sub, int ks, int k) {
        const char* tile = k == 0 ? tq : (k == 1 ? tuq : tdo);
        xr[k] = rd_row<D, TS>(tile, rd, sub, ks);
      };
      // Chain init c (0 S, 1 F, 2 dP, 3 C) of sub-tile sub into z.
      auto load_init = [&](int sub, f32x16 (&z)[4], int c) {
        z[c] = row_init<TS>(sc + (c == 0 ? 0 : c == 1 ? 2 * TS : c == 2 ? TS : 3 * TS), sub);
      };
      auto mask_init = [&](int sub, f32x16 (&z)[4]) {
        if constexpr (MODE == 2) {
#pragma unroll
          for (int idx = 0; idx < 16; ++idx)
            if (t * TS + sub * 32 + acc_pos(idx, hh) < col) z[0][idx] = -INFINITY;
          asm volatile("s_nop 1" : "+v"(z[0]));  // VALU write -> MFMA read of C
        }
      };

      // Elementwise part Q (0..31) of the sub-tile in set z / chains c.
      auto part = [&](const f32x16 (&z)[4], Chain<bf16> (&c)[3], auto qc) {
        constexpr int q = decltype(qc)::value;
        auto E = [&](auto ec) {
          constexpr int e = decltype(ec)::value;
          pv[e] = __builtin_amdgcn_exp2f(z[0][e] * a.c1);
        };
        auto hv = [&](int e) { return RHO1 ? z[1][e] : z[1][e] * a.rho; };
        auto A = [&](auto jc) {
          constexpr int e0 = 2 * decltype(jc)::value, e1 = e0 + 1;
          c[0].f[e0 >> 3][e0 & 7] = (bf16)(pv[e0] * fmaf(hv(e0), z[2][e0], z[3][e0]));
          c[0].f[e1 >> 3][e1 & 7] = (bf16)(pv[e1] * fmaf(hv(e1), z[2][e1], z[3][e1]));
        };
        auto Bc = [&](auto jc) {
          constexpr int e0 = 2 * decltype(jc)::value, e1 = e0 + 1;
          c[1].f[e0 >> 3][e0 & 7] = (bf16)(pv[e0] * z[2][e0]);
          c[1].f[e1 >> 3][e1 & 7] = (bf16)(pv[e1] * z[2][e1]);
          c[2].f[e0 >> 3][e0 & 7] = (bf16)(pv[e0] * hv(e0));
          c[2].f[e1 >> 3][e1 & 7] = (bf16)(pv[e1] * hv(e1));
        };
        if constexpr (q < 4) {
          E(std::integral_constant<int, q>{});
        } else if constexpr (q < 28) {
          constexpr int j = (q - 4) >> 2, r = (q - 4) & 3;
          if constexpr (r == 0) A(std::integral_constant<int, j>{});
          else if constexpr (r == 1) Bc(std::integral_constant<int, j>{});
          else E(std::integral_constant<int, 2 * j + 2 + r>{});
        } else {
          constexpr int j = 6 + ((q - 28) >> 1);
          if constexpr ((q & 1) == 0) A(std::integral_constant<int, j>{});
          else Bc(std::integral_constant<int, j>{});
        }
      };

      // One sub-tile iteration: MFMAs of acc(sub - 1) then scores(sub + 1),
      // elementwise parts of sub after them (PRE parts before the first MFMA
      // when there is no accumulation, to cover the first loads).
      auto iteration = [&](auto subc) {
        constexpr int sub = decltype(subc)::value;
        constexpr int P = sub & 1, Q = P ^ 1;
        constexpr bool has_acc = sub > 0, has_sc = sub + 1 < NSUB;
        constexpr int NA = has_acc ? 3 * NSLICE : 0, NSC = has_sc ? 5 * NKS : 0;
        constexpr int PRE = has_acc ? 0 : 4, M = NA + NSC;
        mfma_fence(cs[P][0], cs[P][1], cs[P][2], cs[P][3]);
        auto run_parts = [&](auto q0c, auto q1c) {
          __builtin_amdgcn_sched_barrier(0);
          static_for<decltype(q0c)::value, decltype(q1c)::value>([&](auto qc) { part(cs[P], ch[P], qc); });
          __builtin_amdgcn_sched_barrier(0);
        };
        // Parts after MFMA I of this iteration.
        auto after = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          run_parts(std::integral_constant<int, PRE + (32 - PRE) * i / M>{},
                    std::integral_constant<int, PRE + (32 - PRE) * (i + 1) / M>{});
        };
        if constexpr (!has_acc) {
          // No accumulation ahead of the scores: their first loads, then the
          // first parts while they land.
          static_for<0, 4>([&](auto cc) { load_init(sub + 1, cs[Q], cc); });
          static_for<0, 3>([&](auto k) { load_row(sub + 1, 0, k); });
          run_parts(std::integral_constant<int, 0>{}, std::integral_constant<int, PRE>{});
          mask_init(sub + 1, cs[Q]);
        }
        if constexpr (has_acc) {
          const Chain<bf16>(&cp)[3] = ch[Q];
          static_for<0, NSLICE>([&](auto slc) {
            constexpr int sl = decltype(slc)::value;
            constexpr int db = sl % NDB, s2 = sl / NDB;
            // Slice sl + 2 of this sub-tile, else slice sl + 2 - NSLICE of the
            // next accumulation (sub-tile sub), which follows in the next
            // iteration or after the last one.
            constexpr bool nxt = sl + 2 < NSLICE;
            constexpr int lsub = nxt ? sub - 1 : sub, lsl = nxt ? sl + 2 : sl + 2 - NSLICE;
            mfma_acc(ak[db], ta[sl & 1][0], cp[0].f[s2]);
            load_tr(lsub, lsl, 0);
            if constexpr (has_sc && sl == 0) load_init(sub + 1, cs[Q], 0);
            if constexpr (has_sc && sl == 1) load_init(sub + 1, cs[Q], 2);
            if constexpr (has_sc && sl == 2) load_row(sub + 1, 0, 0);
            if constexpr (has_sc && sl == 3) load_row(sub + 1, 0, 2);
            after(std::integral_constant<int, 3 * sl>{});
            mfma_acc(av[db], ta[sl & 1][2], cp[2].f[s2]);
            load_tr(lsub, lsl, 2);
            if constexpr (has_sc && sl == 0) load_init(sub + 1, cs[Q], 1);
            if constexpr (has_sc && sl == 1) load_init(sub + 1, cs[Q], 3);
            if constexpr (has_sc && sl == 2) load_row(sub + 1, 0, 1);
            after(std::integral_constant<int, 3 * sl + 1>{});
            mfma_acc(ak[db], ta[sl & 1][1], cp[1].f[s2]);
            load_tr(lsub, lsl, 1);
            if constexpr (has_sc && sl == 3) mask_init(sub + 1, cs[Q]);
            after(std::integral_constant<int, 3 * sl + 2>{});
          });
        }
        if constexpr (has_sc) {
          f32x16(&z)[4] = cs[Q];
          static_for<0, NKS>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            constexpr bool more = ks + 1 < NKS;
            constexpr int i0 = NA + 5 * ks;
            mfma_va(z[1], xr[1], kf[ks]);
            if constexpr (more) load_row(sub + 1, ks + 1, 1);
            after(std::integral_constant<int, i0>{});
            mfma_va(z[0], xr[0], kf[ks]);
            after(std::integral_constant<int, i0 + 1>{});
            mfma_va(z[1], xr[0], ukf[ks]);
            if constexpr (more) load_row(sub + 1, ks + 1, 0);
            after(std::integral_constant<int, i0 + 2>{});
            mfma_va(z[2], xr[2], vf[ks]);
            after(std::integral_constant<int, i0 + 3>{});
            mfma_va(z[3], xr[2], uvf[ks]);
            if constexpr (more) load_row(sub + 1, ks + 1, 2);
            after(std::integral_constant<int, i0 + 4>{});
          });
        }
      };

      // Tile head: scores of sub-tile 0 (nothing to overlap), with the first
      // two slices of the first accumulation loaded behind them.
      static_for<0, 4>([&](auto cc) { load_init(0, cs[0], cc); });
      static_for<0, 3>([&](auto k) { load_row(0, 0, k); });
      mask_init(0, cs[0]);
      static_for<0, NKS>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr bool more = ks + 1 < NKS;
        mfma_va(cs[0][1], xr[1], kf[ks]);
        if constexpr (more) load_row(0, ks + 1, 1);
        mfma_va(cs[0][0], xr[0], kf[ks]);
        mfma_va(cs[0][1], xr[0], ukf[ks]);
        if constexpr (more) load_row(0, ks + 1, 0);
        mfma_va(cs[0][2], xr[2], vf[ks]);
        mfma_va(cs[0][3], xr[2], uvf[ks]);
        if constexpr (more) load_row(0, ks + 1, 2);
      });
      static_for<0, 2>([&](auto sl) { static_for<0, 3>([&](auto k) { load_tr(0, sl, k); }); });
      static_for<0, NSUB>([&](auto subc) { iteration(subc); });
      // Tail: accumulation of the last sub-tile (its first two slices are
      // already loaded).
      {
        const Chain<bf16>(&cp)[3] = ch[(NSUB - 1) & 1];
        static_for<0, NSLICE>([&](auto slc) {
          constexpr int sl = decltype(slc)::value;
          constexpr int db = sl % NDB, s2 = sl / NDB;
          constexpr bool nxt = sl + 2 < NSLICE;
          mfma_acc(ak[db], ta[sl & 1][0], cp[0].f[s2]);
          if constexpr (nxt) load_tr(NSUB - 1, sl + 2, 0);
          mfma_acc(av[db], ta[sl & 1][2], cp[2].f[s2]);
          if constexpr (nxt) load_tr(NSUB - 1, sl + 2, 2);
          mfma_acc(ak[db], ta[sl & 1][1], cp[1].f[s2]);
          if constexpr (nxt) load_tr(NSUB - 1, sl + 2, 1);
        });
      }
    };

    if constexpr (SPLIT) {
    f32x16 s, f, dp, c;
    scores(0, s, f, dp, c);
    Chain<bf16> pdt, pds, pw;  // chains of the previous sub-tile
    DropCol<2> dm;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      if constexpr (DROP) {
        if (sub % 2 == 0) dm.init(a, (int64_t)wk.b * a.H + wk.h + gq, t * TS + sub * 32, col);
      }
      mfma_fence(s, f, dp, c);
      Chain<bf16> cdt, cds, cw;
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        elementwise(part, s, f, dp, c, cdt, cds, cw, sub, dm);
        if constexpr (SPLIT) {
          constexpr int H = NDB / 2;
          if (part < 2) {
            if (sub > 0) {
#pragma unroll
              for (int db = part * H; db < (part + 1) * H; ++db) acc_slice(sub - 1, db, 1, pdt, pds, pw);
            }
          } else {
#pragma unroll
            for (int db = (part - 2) * H; db < (part - 1) * H; ++db) acc_slice(sub, db, 0, cdt, cds, cw);
          }
        }
      }
      pdt = cdt;
      pds = cds;
      pw = cw;
      if (sub + 1 < NSUB) scores(sub + 1, s, f, dp, c);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_slice(NSUB - 1, db, 1, pdt, pds, pw);
    } else {
      woven();
    }
  };

  // u counts the tiles of all heads (it picks the LDS buffer); the copy of
  // the next tile, possibly the next head's first, overlaps the current one.
  int u = 0;
  for (int g = 0; g < a.gs; ++g) {
    auto run = [&](int t0, int t1, auto mode_c) {
      for (int t = t0; t < t1; ++t) {
        dma_wait();
        __syncthreads();
        // The next tile: t + 1 of this head, else the next head's first.
        const bool wrap = t + 1 >= t_end;
        const int gn = wrap ? g + 1 : g, tn = wrap ? t_begin : t + 1;
        if (gn < a.gs) copy_tile(gn, tn, lds + ((u + 1) & 1) * STAGE);
        tile_body(t, u & 1, g, mode_c);
        ++u;
      }
      acc_fence2<NDB>(ak, av);
    };
    if constexpr (CAUSAL) run(t_begin, min(t_diag, nt), std::integral_constant<int, 2>{});
    run(CAUSAL ? min(t_diag, nt) : t_begin, t_end, std::integral_constant<int, 0>{});
  }

  acc_fence2<NDB>(ak, av);
  const KeyOut out = key_out<D>(a, wk);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    store_out(out.k, out.sk, col, N, db, [&](int idx) { return a.tau * ak[db][idx]; });
    store_out(out.v, out.sv, col, N, db, [&](int idx) { return av[db][idx]; });
  }
}

}  // namespace fa
