// fa_fwd_bwd.hip -- bf16 forward and first backward on the LDS-DMA path
// (fa_lds.h), for gfx950.
//
// Sources: [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward
// for Softmax Attention", section 3 (forward, L, first backward);
// [FA2-triton] "FlashAttention-2 from PyTorch to Triton" (online softmax);
// [FA2-recompute] "Why does FlashAttention-2's backward pass recompute
// attention ...": P = exp(S - L), D = rowsum(dO * O).
//
// Same work split as the BoB passes: 4 waves x 32 resident rows, the other
// side streamed in tiles of TS rows (two LDS stages filled by DMA, one
// barrier per tile), score chains with the streamed index on M so their
// accumulator values feed the next product as B operands, transposed
// operands read with ds_read_b64_tr_b16.  The output accumulators live in
// VGPRs here: the forward rescales them by the online-softmax factor, which
// the VALU cannot do in AGPRs.
#include <type_traits>

#include "fa_lds.h"

namespace fa {

// d += a * b, every operand in VGPRs; the s_nop covers a VALU write of b or
// of d (rescale) just before.
__device__ inline void mfma_vacc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ inline void vfence1(f32x16& a) { asm volatile("s_nop 7\n\ts_nop 4" : "+v"(a)); }
// d = a * b + c with b resident in AGPRs and c in its own registers (kept):
// the matrix core reads c after issue, so a write of c's registers must wait
// 7 wait states, which the instruction carries.
__device__ inline f32x16 mfma_init_a(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 6" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
  return d;
}

// ---------------------------------------------------------------------------
// Forward: O = softmax(tau Q K^T) V with the online softmax, L = log-sum-exp.
// Per 32-key sub-tile: S^T = K Q^T (keys on M); a reference maximum m (log2
// domain) and the sum l; O <- O * exp2(m_old - m_new) + V^T P.  The softmax
// is the same for any reference, so m moves only when a row's exponentials
// against it would exceed 2^16 (or it is still -inf): in the common case a
// sub-tile costs one FMA, one exp2, one add and half a conversion per score,
// with no maximum, no rescale and no second exp2.  The scores of sub-tile
// s + 1 are issued before the elementwise work of s, so the matrix cores and
// the VALU overlap.
//
// DROP: dropout with the scaled keep mask g ([FlashBoB] appendix G): O takes
// (P g) V while the row sum and L keep P.  The mask of each pair of sub-tiles
// comes from one shared generator call per lane (DropRow), issued behind the
// score MFMAs of the next sub-tile.
// WPE: waves per SIMD (2; 3 for the d = 64 instances with 64-key tiles, 122
// registers, 162 with the mask, and the d = 128 one with 32-key tiles, 166;
// each 33 KB of LDS a workgroup: three workgroups per CU).
// Largest partial row sum (16 exponentials of one lane) accepted against a
// stale reference maximum; it bounds every exponential by 2^16.
constexpr float kLazyBound = 65536.0f;

template <int D, int TS, bool CAUSAL, bool DROP = false, int WPE = 2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void fwd_dma_kernel(Args a) {
  static_assert(!DROP || TS % 64 == 0, "the mask comes in pairs of sub-tiles");
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int STAGE = 2 * W::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float kbias[TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> q = head_of<bf16>(a.q, wk.b, wk.h);
  HeadPtr<bf16> src[2] = {head_of<bf16>(a.k, wk.b, wk.hk), head_of<bf16>(a.v, wk.b, wk.hk)};
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  const int t_diag = CAUSAL ? wk.rb * kResRows / TS : nt;
  const bool ragged = !CAUSAL && (N % TS) != 0;

  Dma<D, TS, 2> dma;
  dma.init(src);
  dma.copy(0, N, lds);
  fill_bias<TS>(kbias, (nt - 1) * TS, N);

  bf16x8 qf[NKS];
  load_resident<bf16, D>(qf, q.p, q.sn, row, N, a.pow2);
  Reader<D, TS> rd;
  rd.init();

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  float m = -INFINITY, lsum = 0.0f;  // running maximum of S * c1 (log2 domain) and sum of exp2
  const float c1 = a.c1;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load of the compiler's own in the loop

  auto tile_body = [&](int t, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tk = lds + (t & 1) * STAGE;
    const char* tv = tk + W::BYTES;
    auto scores = [&](int sub, f32x16& s) {
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
        if (MODE == 0 && ks == 0) {
          s = mfma_first(xk, qf[0]);
        } else {
          mfma_v(s, xk, qf[ks]);
        }
      }
    };
    f32x16 sb[2];
    scores(0, sb[0]);
    DropRow<2> dm;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x16& s = sb[sub & 1];
      vfence1(s);
      if (sub + 1 < NSUB) scores(sub + 1, sb[(sub + 1) & 1]);
      if constexpr (DROP) {
        if (sub % 2 == 0) dm.init(a, wk.bh, row, t * TS + sub * 32);
      }
      Chain<bf16> cp;
      float ps;
      auto expo = [&](float ref) {
        ps = 0.0f;
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], c1, -ref));
          ps += p;
          cp.f[idx >> 3][idx & 7] = (bf16)(DROP ? p * dm.at(a, sub & 1, idx) : p);
        }
      };
      // Lazy maximum: the exponentials are taken against the reference m
      // of the earlier tiles.  Only when some row's partial sum leaves
      // (0, kLazyBound] -- a score far above m, or m still -inf -- does the
      // wave take the maximum of the sub-tile, move m and rescale.
      expo(m);
      if (__any(!(ps <= kLazyBound))) {
        float mx = s[0];
#pragma unroll
        for (int idx = 1; idx < 16; ++idx) mx = fmaxf(mx, s[idx]);
        mx = half_max(mx);
        const float mn = fmaxf(m, mx * c1);
        const float ms = (mn == -INFINITY) ? 0.0f : mn;
        const float sc = __builtin_amdgcn_exp2f(m - ms);
        expo(ms);
        lsum *= sc;
        m = mn;
        if (__any(sc != 1.0f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            vfence1(acc[db]);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] *= sc;
          }
        }
      }
      lsum += ps;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) mfma_vacc(acc[db], rd_tr<D, TS>(tv, rd, sub, db, s2), cp.f[s2]);
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
#pragma unroll
  for (int db = 0; db < NDB; ++db) vfence1(acc[db]);
  const float lt = half_sum(lsum);
  const float inv = 1.0f / lt;
  float* o = head_out(a.r0, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_out(o, a.r0.sn, row, N, db, [&](int idx) { return acc[db][idx] * inv; });
  if (row < N && hh == 0) a.lse_out[(int64_t)wk.bh * N + row] = kLn2 * (m + __log2f(lt));
}

// ---------------------------------------------------------------------------
// First backward, row side: dQ = tau dS K with dS = P (dP - D).  Resident per
// wave: q_i (scaled by pow2), do_i, L_i, D_i; streamed K, V.  Per 32-key
// sub-tile: S^T = K Q^T and dP^T = V dO^T (keys on M), P = exp(tau S - L),
// dS = P (dP - D), and dQ^T += K^T dS^T (transposed K from LDS).  DROP: dP is
// g (dO V^T) ([FlashBoB] appendix G), so dS = P (g dP - D).
template <int D, int TS, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_dma_kernel(Args a) {
  static_assert(!DROP || TS % 64 == 0, "the mask comes in pairs of sub-tiles");
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int STAGE = 2 * W::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float kbias[TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> q = head_of<bf16>(a.q, wk.b, wk.h), dout = head_of<bf16>(a.dout, wk.b, wk.h);
  HeadPtr<bf16> src[2] = {head_of<bf16>(a.k, wk.b, wk.hk), head_of<bf16>(a.v, wk.b, wk.hk)};
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  const int t_diag = CAUSAL ? wk.rb * kResRows / TS : nt;
  const bool ragged = !CAUSAL && (N % TS) != 0;

  Dma<D, TS, 2> dma;
  dma.init(src);
  dma.copy(0, N, lds);
  fill_bias<TS>(kbias, (nt - 1) * TS, N);

  // Resident operands in AGPRs (the matrix core reads B from there), which
  // leaves the VGPRs to the score chains at two waves per SIMD.
  bf16x8 qf[NKS], df[NKS];
  load_resident<bf16, D>(qf, q.p, q.sn, row, N, a.pow2);
  load_resident<bf16, D>(df, dout.p, dout.sn, row, N, 1.0f);
  const int64_t rv = (int64_t)wk.bh * N;
  const float Li = row < N ? a.lse[rv + row] : 0.0f;
  // d = 64: D = rowsum(dO * O) from the resident dO rows (no row-scalar
  // kernel); this kernel also stages the dK/dV kernel's chain inits of its
  // rows, -L/rho and -D ((-inf, 0) on the padding rows of the last block),
  // which that kernel, launched after it, reads.  d = 128 reads them from the
  // row-scalar kernel (with its registers it would spill in the dropout
  // instance, measured 14 % slower there and no faster without dropout).
  constexpr bool OWN_D = D == 64;
  const float Di = OWN_D ? resident_rowdot<D>(df, head_of<float>(a.o, wk.b, wk.h), row, N)
                         : (row < N ? a.D[rv + row] : 0.0f);
  if (OWN_D && hh == 0) {
    const bool ok = row < N;
    if (ok) a.D[rv + row] = Di;
    const int nblk = (N + kPsRows - 1) / kPsRows;
    float* st = a.bs + ((int64_t)wk.bh * nblk + row / kPsRows) * 2 * kPsRows + row % kPsRows;
    st[0] = ok ? -Li / a.rho : -INFINITY;
    st[kPsRows] = ok ? -Di : 0.0f;
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(qf[ks]), "+a"(df[ks]));
  const float nl2 = -Li * kLog2e;
  // At d = 64 without dropout the dP chains start from -D (the MFMA's C
  // operand), so dP - D comes out of the matrix core (fa_bwd 2-3 % faster;
  // at d = 128 it measured no faster and is not used).
  constexpr bool NEGD = D == 64 && !DROP;
  f32x16 negd;
#pragma unroll
  for (int e = 0; e < 16; ++e) negd[e] = -Di;
  Reader<D, TS> rd;
  rd.init();

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acc[db] = zero16();
    asm volatile("" : "+a"(acc[db]));
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load of the compiler's own in the loop

  auto tile_body = [&](int t, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tk = lds + (t & 1) * STAGE;
    const char* tv = tk + W::BYTES;
    auto scores = [&](int sub, f32x16& s, f32x16& dp) {
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
        const bf16x8 xv = rd_row<D, TS>(tv, rd, sub, ks);
        if (MODE == 0 && ks == 0) {
          s = mfma_first_a(xk, qf[0]);
        } else {
          mfma_va(s, xk, qf[ks]);
        }
        if (ks == 0) {
          dp = NEGD ? mfma_init_a(xv, df[0], negd) : mfma_first_a(xv, df[0]);
        } else {
          mfma_va(dp, xv, df[ks]);
        }
      }
    };
    f32x16 sb[2], pb[2];
    scores(0, sb[0], pb[0]);
    DropRow<2> dm;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x16& s = sb[sub & 1];
      f32x16& dp = pb[sub & 1];
      asm volatile("s_nop 7\n\ts_nop 4" : "+v"(s), "+v"(dp));  // MFMA result -> VALU read
      if (sub + 1 < NSUB) scores(sub + 1, sb[(sub + 1) & 1], pb[(sub + 1) & 1]);
      if constexpr (DROP) {
        if (sub % 2 == 0) dm.init(a, wk.bh, row, t * TS + sub * 32);
      }
      Chain<bf16> cds;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], a.c1, nl2));
        cds.f[idx >> 3][idx & 7] =
            (bf16)(p * (DROP ? fmaf(dm.at(a, sub & 1, idx), dp[idx], -Di) : NEGD ? dp[idx] : dp[idx] - Di));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) mfma_acc(acc[db], rd_tr<D, TS>(tk, rd, sub, db, s2), cds.f[s2]);
    }
  };
  auto run = [&](int t0, int t1, auto mode_c) {
    for (int t = t0; t < t1; ++t) {
      dma_wait();
      __syncthreads();
      if (t + 1 < t_end) dma.copy((t + 1) * TS, N, lds + ((t + 1) & 1) * STAGE);
      tile_body(t, mode_c);
    }
    acc_fence1<NDB>(acc);
  };
  if constexpr (CAUSAL) {
    run(0, t_diag, std::integral_constant<int, 0>{});
    run(t_diag, t_end, std::integral_constant<int, 2>{});
  } else {
    run(0, ragged ? nt - 1 : nt, std::integral_constant<int, 0>{});
    if (ragged) run(nt - 1, nt, std::integral_constant<int, 1>{});
  }
  acc_fence1<NDB>(acc);
  float* dq = head_out(a.r0, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_out(dq, a.r0.sn, row, N, db, [&](int idx) { return a.tau * acc[db][idx]; });
}

// ---------------------------------------------------------------------------
// First backward, column side: dK = tau dS^T Q, dV = P^T dO.  Resident per
// wave: k_j (scaled by pow2), v_j; streamed Q, dO and, per streamed row, the
// chain inits -L/rho, -D written by the row-scalar kernel.  Per 32-row
// sub-tile (queries on M): S = Q K^T, dP - D = dO V^T - D, P = exp(tau S - L),
// dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.  The G query heads of a
// key/value head are streamed one after another into the same accumulators.
// DROP ([FlashBoB] appendix G): dP - D = g (dO V^T) - D, so that chain starts
// at 0 and takes -D after the mask, and dV^T += dO^T (P g).  At d = 64 two
// waves share a SIMD (each within 128 VGPRs and 128 AGPRs; the chains of the
// other wave hide this one's latencies), at d = 128 one.
template <int D, int TS, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1))) void
bwd_dkdv_dma_kernel(Args a) {
  static_assert(!DROP || TS % 64 == 0, "the mask comes in pairs of sub-tiles");
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int TBYTES = 2 * W::BYTES;
  constexpr int SBYTES = 2 * TS * 4;                       // [2][TS] floats of chain inits
  constexpr int SROOM = SBYTES < 1024 ? 1024 : SBYTES;     // LDS room: one wave copies 1 KB
  constexpr int STAGE = TBYTES + SROOM;
  static_assert(kPsRows % TS == 0 && SBYTES % 512 == 0 && SBYTES <= 1024, "staged inits: one wave-wide copy");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

  const Work wk = work_item_cols(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int col = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<bf16> k = head_of<bf16>(a.k, wk.b, wk.hk), v = head_of<bf16>(a.v, wk.b, wk.hk);
  HeadPtr<bf16> src[2] = {head_of<bf16>(a.q, wk.b, wk.h), head_of<bf16>(a.dout, wk.b, wk.h)};
  const int64_t hstride[2] = {a.q.sh, a.dout.sh};
  const int nt = (N + TS - 1) / TS;
  const int64_t bs_head = (int64_t)((N + kPsRows - 1) / kPsRows) * 2 * kPsRows;  // floats per query head
  const float* bs0 = a.bs + ((int64_t)wk.b * a.H + wk.h) * bs_head;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  Dma<D, TS, 2> dma;
  dma.init(src, hstride);
  // Tile t of query head h + g into dst: Q, dO and the [2][TS] inits (wave 0;
  // lane l moves 4 floats of init e / TS, rows e % TS .., e = 4 l).
  auto copy_tile = [&](int g, int t, const char* dst) {
    dma.copy(t * TS, N, dst, g);
    if (wave == 0 && l * 16 < SBYTES) {
      const int r0 = t * TS;
      const int e = l * 4;
      const int kk = e / TS, rr = e % TS;
      const float* s_ = bs0 + g * bs_head + ((int64_t)(r0 / kPsRows) * 2 + kk) * kPsRows + r0 % kPsRows + rr;
      dma16(s_, lds_addr(dst + TBYTES));
    }
  };
  const int t_begin = CAUSAL ? wk.rb * kResRows / TS : 0;
  const int t_diag = CAUSAL ? (wk.rb * kResRows + kResRows + TS - 1) / TS : 0;
  copy_tile(0, t_begin, lds);

  bf16x8 kf[NKS], vf[NKS];
  load_resident<bf16, D>(kf, k.p, k.sn, col, N, a.pow2);
  load_resident<bf16, D>(vf, v.p, v.sn, col, N, 1.0f);
  Reader<D, TS> rd;
  rd.init();

  f32x16 ak[NDB], av[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ak[db] = av[db] = zero16();
    asm volatile("" : "+a"(ak[db]), "+a"(av[db]));
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // Tile t of query head wk.h + gq in LDS buffer buf.
  auto tile_body = [&](int t, int buf, int gq, auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    const char* tq = lds + buf * STAGE;
    const char* tdo = tq + W::BYTES;
    const float* sc = reinterpret_cast<const float*>(tq + TBYTES);
    auto scores = [&](int sub, f32x16& s, f32x16& dp) {
      s = row_init<TS>(sc, sub);
      if constexpr (MODE == 2) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx)
          if (t * TS + sub * 32 + acc_pos(idx, hh) < col) s[idx] = -INFINITY;
      }
      dp = DROP ? zero16() : row_init<TS>(sc + TS, sub);
      asm volatile("s_nop 1" : "+v"(s), "+v"(dp));  // VALU write -> MFMA read of C
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (D == 64) {
          // Two waves per SIMD: short of VGPRs the compiler keeps K and V in
          // AGPRs and copies them back (a VALU write) right before an MFMA.
          mfma_v_w(s, rd_row<D, TS>(tq, rd, sub, ks), kf[ks]);
          mfma_v_w(dp, rd_row<D, TS>(tdo, rd, sub, ks), vf[ks]);
        } else {
          mfma_v(s, rd_row<D, TS>(tq, rd, sub, ks), kf[ks]);
          mfma_v(dp, rd_row<D, TS>(tdo, rd, sub, ks), vf[ks]);
        }
      }
    };
    f32x16 sb[2], pb[2];
    scores(0, sb[0], pb[0]);
    DropCol<2> dm;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x16& s = sb[sub & 1];
      f32x16& dp = pb[sub & 1];
      asm volatile("s_nop 7\n\ts_nop 4" : "+v"(s), "+v"(dp));  // MFMA result -> VALU read
      if (sub + 1 < NSUB) scores(sub + 1, sb[(sub + 1) & 1], pb[(sub + 1) & 1]);
      f32x16 nd;
      if constexpr (DROP) {
        if (sub % 2 == 0) dm.init(a, (int64_t)wk.b * a.H + wk.h + gq, t * TS + sub * 32, col);
        nd = row_init<TS>(sc + TS, sub);
      }
      Chain<bf16> cp, cds;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(s[idx] * a.c1);
        if constexpr (DROP) {
          const float g = dm.at(a, sub & 1, idx);
          cp.f[idx >> 3][idx & 7] = (bf16)(p * g);
          cds.f[idx >> 3][idx & 7] = (bf16)(p * fmaf(g, dp[idx], nd[idx]));
        } else {
          cp.f[idx >> 3][idx & 7] = (bf16)p;
          cds.f[idx >> 3][idx & 7] = (bf16)(p * dp[idx]);
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          mfma_acc(av[db], rd_tr<D, TS>(tdo, rd, sub, db, s2), cp.f[s2]);
          mfma_acc(ak[db], rd_tr<D, TS>(tq, rd, sub, db, s2), cds.f[s2]);
        }
    }
  };

  int u = 0;  // tiles of all heads so far (picks the LDS buffer)
  for (int g = 0; g < a.gs; ++g) {
    auto run = [&](int t0, int t1, auto mode_c) {
      for (int t = t0; t < t1; ++t) {
        dma_wait();
        __syncthreads();
        const bool wrap = t + 1 >= nt;
        const int gn = wrap ? g + 1 : g, tn = wrap ? t_begin : t + 1;
        if (gn < a.gs) copy_tile(gn, tn, lds + ((u + 1) & 1) * STAGE);
        tile_body(t, u & 1, g, mode_c);
        ++u;
      }
      acc_fence2<NDB>(ak, av);
    };
    if constexpr (CAUSAL) run(t_begin, min(t_diag, nt), std::integral_constant<int, 2>{});
    run(CAUSAL ? min(t_diag, nt) : 0, nt, std::integral_constant<int, 0>{});
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
