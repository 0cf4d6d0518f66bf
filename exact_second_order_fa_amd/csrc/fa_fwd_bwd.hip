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

// ---------------------------------------------------------------------------
// Forward: O = softmax(tau Q K^T) V with the online softmax, L = log-sum-exp.
// Per 32-key sub-tile: S^T = K Q^T (keys on M); the running maximum m (log2
// domain) and sum l; O <- O * exp2(m_old - m_new) + V^T P.  The rescale is
// skipped when no row's maximum moved, which after the first tiles is the
// common case.  The scores of sub-tile s + 1 are issued before the
// elementwise work of s, so the matrix cores and the VALU overlap.
template <int D, int TS, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_dma_kernel(Args a) {
  typedef SwTile<D, TS> W;
  constexpr int NKS = D / 16, NDB = D / 32, NSUB = TS / 32;
  constexpr int STAGE = 2 * W::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float kbias[TS];

  const Work wk = work_item(a);
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
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x16& s = sb[sub & 1];
      vfence1(s);
      if (sub + 1 < NSUB) scores(sub + 1, sb[(sub + 1) & 1]);
      float mx = s[0];
#pragma unroll
      for (int idx = 1; idx < 16; ++idx) mx = fmaxf(mx, s[idx]);
      mx = half_max(mx);
      const float mn = fmaxf(m, mx * c1);
      const float ms = (mn == -INFINITY) ? 0.0f : mn;
      const float sc = __builtin_amdgcn_exp2f(m - ms);
      Chain<bf16> cp;
      float ps = 0.0f;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], c1, -ms));
        ps += p;
        cp.f[idx >> 3][idx & 7] = (bf16)p;
      }
      lsum = fmaf(lsum, sc, ps);
      m = mn;
      if (__any(sc != 1.0f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          vfence1(acc[db]);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][e] *= sc;
        }
      }
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

}  // namespace fa
