// fa_kernels.hip -- gfx950 kernels: forward, first backward, and the two-pass
// exact backward-over-backward of softmax attention.
//
// Sources (page title, section):
//   [FlashBoB]      "FlashBoB: I/O-Efficient Exact Backward-over-Backward for
//                   Softmax Attention": section 3 (forward, L, first
//                   backward), sections 4.2-4.3 (affine fusion, two-pass
//                   schedule), appendix D (final assembled identities).
//   [FA2-recompute] "Why does FlashAttention-2's backward pass recompute
//                   attention ...": D = rowsum(dO * O), P = exp(S - L).
//   [FA2-triton]    "FlashAttention-2 from PyTorch to Triton": online softmax
//                   forward, masking of a ragged last key tile.
//
// Every kernel: 256 threads (4 waves), 32 resident rows per wave, streamed
// tiles of TS rows double-buffered in LDS (see fa_tile.h for the operand
// layouts).  The softmax scale is split as tau = pow2 * rho with pow2 an
// exact power of two folded into the resident operands and rho in [1, 2)
// applied in fp32 (rho == 1 at d = 64).
#include "fa_tile.h"

namespace fa {

struct TDesc {
  const void* p;
  int64_t sb, sh, sn;
};

struct Args {
  TDesc q, k, v, o, dout, uq, uk, uv;  // inputs (o: fp32)
  TDesc r0, r1, r2, r3;                // outputs (fp32), kernel specific
  const float* lse;                    // [B,H,N] saved log-normaliser (input)
  float* lse_out;                      // [B,H,N] (fa_fwd output)
  float* D;                            // [B,H,N] rowsum(dO * O)
  float* alpha;                        // [B,H,N] BoB row scalar alpha
  float* E;                            // [B,H,N] BoB row scalar E
  float* ps;                           // [B*H][ceil(N/128)][4][128] column-pass chain inits
  float* bs;                           // [B*H][ceil(N/128)][2][128] first-backward column chain inits (or null)
  float* part;                         // key-side partial sums of a split group (or null), see GroupSplit
  float* kpart;                        // row-pass partial sums of a key split (or null), see KeySplit
  int B, H, N;
  int Hk, G;                 // key/value heads and query heads per key/value head (H = Hk * G)
  int gs, nsplit;            // column kernels: query heads per workgroup and partial sums per key block
  int rs;                    // column kernels: query-row ranges per head subset (nsplit = G / gs * rs)
  int ks;                    // two-pass row pass: key ranges per row block (1: no key split)
  float tau, pow2, rho, c1;  // c1 = log2(e) * rho
  uint64_t seed;             // dropout: generator key
  uint32_t drop_thr;         // dropout: keep an element iff its byte >= drop_thr (1..255)
  float drop_scale;          // dropout: 256 / (256 - drop_thr), the kept elements' factor
};

template <typename T>
__device__ inline HeadPtr<T> head_of(const TDesc& t, int b, int h) {
  HeadPtr<T> r;
  r.p = reinterpret_cast<const T*>(t.p) + (int64_t)b * t.sb + (int64_t)h * t.sh;
  r.sn = t.sn;
  return r;
}

__device__ inline float* head_out(const TDesc& t, int b, int h) {
  return reinterpret_cast<float*>(const_cast<void*>(t.p)) + (int64_t)b * t.sb + (int64_t)h * t.sh;
}

// One workgroup's share: batch b, row block rb and
//   * row-side kernels (a block of query rows): query head h, bh = b * H + h,
//     and the key/value head hk = h / G its keys come from;
//   * column-side kernels (a block of key rows): key/value head hk,
//     bh = b * Hk + hk; its G query heads are hk * G .. hk * G + G - 1, the
//     first of them in h ([FlashBoB] section 4.3: the key-side outputs sum
//     over the group inside one workgroup).
struct Work {
  int bh, b, h, hk, rb;
  int sp;  // column kernels: which partial sum of the key block (0 without a split)
  int rr;  // column kernels: which range of the query rows (0 without a row split)
  int kk;  // row pass: which range of the keys (0 without a key split)
};

// heavy_first: causal row-side kernels do work proportional to rb + 1; the
// blocks are taken in descending rb (longest_first) so the largest ones start
// first and the last wave of workgroups is made of the small ones.
__device__ inline Work work_item(const Args& a, bool heavy_first = false) {
  const int nblk = (a.N + kResRows - 1) / kResRows;
  const int w0 = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.B * a.H * nblk;
  Work r;
  r.kk = w0 / per;  // the key range is the slowest index (0 unless a key split)
  const int w = w0 - r.kk * per;
  if (heavy_first) {
    int k;
    longest_first(w, gridDim.x, nblk, r.bh, k);
    r.rb = nblk - 1 - k;
  } else {
    r.bh = w / nblk;
    r.rb = w % nblk;
  }
  r.b = r.bh / a.H;
  r.h = r.bh % a.H;
  r.hk = r.h / a.G;
  return r;
}

// With a group split (nsplit > 1: few key blocks, many query heads per
// key/value head) workgroup sp of a key block takes query heads
// hk * G + sp * gs .. + gs - 1 and leaves its sums in a.part; the split index
// is the slowest, so the workgroups streaming the same query heads sit on one
// XCD.
// causal: key block rb streams the rows from 128 rb on, so rb = 0 is the
// longest; without a split the blocks are taken longest first.
__device__ inline Work work_item_cols(const Args& a, bool causal = false) {
  const int nblk = (a.N + kResRows - 1) / kResRows;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.B * a.Hk * nblk;
  Work r;
  r.sp = w / per;
  const int w2 = w - r.sp * per;
  if (causal && a.nsplit == 1) {
    longest_first(w2, gridDim.x, nblk, r.bh, r.rb);
  } else {
    r.bh = w2 / nblk;
    r.rb = w2 % nblk;
  }
  r.b = r.bh / a.Hk;
  r.hk = r.bh % a.Hk;
  const int sh = r.sp / a.rs;  // subset of the group's query heads
  r.rr = r.sp - sh * a.rs;
  r.h = r.hk * a.G + sh * a.gs;
  return r;
}

// Key-side output rows of a column workgroup: the caller's tensor, or with a
// group split this split's slab of a.part ([2][nsplit][B * Hk][N][D] floats:
// first the d~K sums, then the d~V sums).
struct KeyOut {
  float* k;
  float* v;
  int64_t sk, sv;
};
template <int D>
__device__ inline KeyOut key_out(const Args& a, const Work& wk) {
  KeyOut o;
  if (a.part) {
    const int64_t slab = (int64_t)a.B * a.Hk * a.N * D;
    o.k = a.part + ((int64_t)wk.sp * a.B * a.Hk + wk.bh) * a.N * D;
    o.v = o.k + a.nsplit * slab;
    o.sk = o.sv = D;
  } else {
    o.k = head_out(a.r1, wk.b, wk.hk);
    o.v = head_out(a.r2, wk.b, wk.hk);
    o.sk = a.r1.sn;
    o.sv = a.r2.sn;
  }
  return o;
}

// Sum of the nsplit partial key-side outputs, in split order (deterministic),
// into the caller's tensors: one thread per 4 consecutive floats of a row.
template <int D>
__global__ __launch_bounds__(256) void group_sum_kernel(Args a) {
  const int64_t rows = (int64_t)a.B * a.Hk * a.N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * rows * (D / 4)) return;
  const int which = (int)(i / (rows * (D / 4)));  // 0: d~K, 1: d~V
  const int64_t j = i - (int64_t)which * rows * (D / 4);
  const int64_t row = j / (D / 4);
  const int c = (int)(j % (D / 4)) * 4;
  const int64_t slab = rows * D;
  const float* src = a.part + (int64_t)which * a.nsplit * slab + row * D + c;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int sp = 1; sp < a.nsplit; ++sp) acc += *reinterpret_cast<const f32x4*>(src + sp * slab);
  const int b = (int)(row / ((int64_t)a.Hk * a.N));
  const int hk = (int)(row / a.N % a.Hk);
  const int n = (int)(row % a.N);
  const TDesc& t = which ? a.r2 : a.r1;
  float* dst = head_out(t, b, hk) + (int64_t)n * t.sn + c;
  *reinterpret_cast<f32x4*>(dst) = acc;
}

// Key split of the two-pass row pass (KeySplit).  Row-side workgroups are
// too few to fill the chip when B * H * ceil(N / 128) < 256 (multi-query at
// N = 2048: 128); then each row block's keys are cut into ks ranges of whole
// tiles, workgroup kk takes tiles [nt kk / ks, nt (kk + 1) / ks), and instead
// of the epilogue it stores its raw sums -- alpha, E°, the E° of the
// bf16-rounded operands, and the four accumulators G, Omega, R', B -- all
// linear in the keys.  a.kpart holds [ks][3][B*H][N] row sums, then
// [ks][4][B*H][N][D] accumulators; bob_ksplit_sum_kernel adds them in order.
__device__ inline void key_range(const Args& a, int kk, int nt, int& t0, int& t1) {
  t0 = (int)((int64_t)nt * kk / a.ks);
  t1 = (int)((int64_t)nt * (kk + 1) / a.ks);
}
__device__ inline float* kpart_rowsum(const Args& a, int kk, int j, int64_t bh) {
  return a.kpart + (((int64_t)kk * 3 + j) * a.B * a.H + bh) * a.N;
}
template <int D>
__device__ inline float* kpart_acc(const Args& a, int kk, int m, int64_t bh) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  return a.kpart + (int64_t)a.ks * 3 * rows + (((int64_t)kk * 4 + m) * a.B * a.H + bh) * a.N * D;
}

// The row pass's epilogue over the key-split partial sums, in split order
// (deterministic): one thread per 4 consecutive floats of a row (rows padded
// to whole 128-row blocks, whose chain inits it also writes).  Same outputs
// as the unsplit row pass: gdO = G - alpha O, gQ = tau (Omega - alpha R' -
// E°_b B), alpha, E = E° - alpha D (D stored by key range 0), and the chain
// inits -L/rho, -D, -alpha/rho, -E° ((-inf, 0, 0, 0) past N).
template <int D>
__global__ __launch_bounds__(256) void bob_ksplit_sum_kernel(Args a) {
  constexpr int CH = D / 4;
  const int nblk = (a.N + kPsRows - 1) / kPsRows;
  const int64_t prow = (int64_t)nblk * kPsRows;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.H * prow * CH) return;
  const int c = (int)(i % CH) * 4;
  const int64_t rr = i / CH;
  const int64_t bh = rr / prow;
  const int row = (int)(rr % prow);
  const bool ok = row < a.N;
  float alpha = 0.0f, eo = 0.0f, eob = 0.0f;
  if (ok) {
    for (int kk = 0; kk < a.ks; ++kk) {
      alpha += kpart_rowsum(a, kk, 0, bh)[row];
      eo += kpart_rowsum(a, kk, 1, bh)[row];
      eob += kpart_rowsum(a, kk, 2, bh)[row];
    }
  }
  const int64_t rv = bh * a.N;
  const float Di = ok ? a.D[rv + row] : 0.0f;
  if (c == 0) {
    if (ok) {
      a.alpha[rv + row] = alpha;
      a.E[rv + row] = eo - alpha * Di;
    }
    float* ps = a.ps + (bh * nblk + row / kPsRows) * 4 * kPsRows + row % kPsRows;
    const float irho = 1.0f / a.rho;
    ps[0] = ok ? -a.lse[rv + row] * irho : -INFINITY;
    ps[kPsRows] = ok ? -Di : 0.0f;
    ps[2 * kPsRows] = ok ? -alpha * irho : 0.0f;
    ps[3 * kPsRows] = ok ? -eo : 0.0f;
  }
  if (!ok) return;
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc[m] = *reinterpret_cast<const f32x4*>(kpart_acc<D>(a, 0, m, bh) + (int64_t)row * D + c);
    for (int kk = 1; kk < a.ks; ++kk) acc[m] += *reinterpret_cast<const f32x4*>(kpart_acc<D>(a, kk, m, bh) + (int64_t)row * D + c);
  }
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const HeadPtr<float> o = head_of<float>(a.o, b, h);
  const f32x4 ov = *reinterpret_cast<const f32x4*>(o.p + (int64_t)row * o.sn + c);
  float* gq = head_out(a.r0, b, h) + (int64_t)row * a.r0.sn + c;
  float* gdo = head_out(a.r3, b, h) + (int64_t)row * a.r3.sn + c;
  *reinterpret_cast<f32x4*>(gdo) = acc[0] - alpha * ov;
  *reinterpret_cast<f32x4*>(gq) = a.tau * (acc[1] - alpha * acc[2] - eob * acc[3]);
}

// Row scalars of a streamed tile, staged into LDS next to the operand tiles.
// NS scalars per streamed row; Fn maps (global row) -> values and Pad gives
// the values of rows past N.  The scalars enter the score chains as MFMA
// accumulator initial values, and a -inf there is what masks a ragged tile
// (exp2(-inf) = 0), so no per-element select is needed in the inner loop.
template <int TS, int NS>
struct ScalarStager {
  float v[NS];
  bool active;
  template <typename Fn, typename Pad>
  __device__ inline void load(int row0, int N, Fn fn, Pad pad) {
    active = threadIdx.x < TS;
    if (active) {
      const int row = row0 + threadIdx.x;
      if (row < N) {
        fn(row, v);
      } else {
        pad(v);
      }
    }
  }
  __device__ inline void store(float* lds) const {
    if (active) {
#pragma unroll
      for (int e = 0; e < NS; ++e) lds[e * TS + threadIdx.x] = v[e];
    }
  }
};

// ---------------------------------------------------------------------------
// Dropout ([FlashBoB] appendix G, analytical dropout extension): the forward
// multiplies P by a scaled keep mask g before the product with V, and the
// first backward and the BoB take the same g.  Every pass recomputes g from a
// counter-based generator instead of storing it: Philox4x64-10 (Salmon,
// Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC
// 2011), ten rounds that each take the 128-bit products of counter words 0
// and 2 with two fixed odd multipliers, the key advancing by two Weyl
// constants between rounds.  Element (i, j) of query head bh (= b H + h) uses
// byte j % 8 of output word i % 4 of the block for counter (i / 4, j / 8, bh,
// 0) and key (seed, 0); it is kept iff that byte is >= t = round(256 p), and
// kept elements are scaled by 256 / (256 - t).
struct U64x4 {
  uint64_t w0, w1, w2, w3;
};
// High and low words of the 128-bit product a * m from four 32 x 32 -> 64-bit
// partial products, each one v_mad_u64_u32 with the carry of the previous one
// as its addend (none of the sums can exceed 64 bits).
__device__ inline void mulhilo64(uint64_t a, uint64_t m, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32), m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
  const uint64_t p00 = (uint64_t)a0 * m0;
  const uint64_t p01 = (uint64_t)a0 * m1 + (p00 >> 32);
  const uint64_t p10 = (uint64_t)a1 * m0 + (uint32_t)p01;
  const uint64_t p11 = (uint64_t)a1 * m1 + (p01 >> 32);
  lo = (p10 << 32) | (uint32_t)p00;
  hi = p11 + (p10 >> 32);
}
__device__ inline U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(c0, M0, hi0, lo0);
    mulhilo64(c2, M1, hi1, lo1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return {c0, c1, c2, c3};
}
__device__ inline float keep_byte(const Args& a, uint32_t w, int byte) {
  return ((w >> (8 * byte)) & 0xffu) >= a.drop_thr ? a.drop_scale : 0.0f;
}

// The wave shares the generator's work.  A 32 x 32 sub-tile covers 32 blocks
// (8 groups of four query rows x 4 groups of eight keys); a row-side lane's 16
// elements lie in two of them, which the other three rows of its group of
// four use too, and a column-side lane's in four, which the other seven keys
// of its group of eight use too.  So instead of each lane running every block
// it touches, each lane runs ONE block per granule of NS sub-tiles (NS = 2:
// every block of the granule exactly once; NS = 1: each block by two lanes)
// and the words move to the lanes that use them by lane exchanges inside
// groups of M lanes (xor_transpose): 4-8x fewer generator calls.

// Lanes g = lane % M of a group each hold items A[q] (K dwords each), q =
// 0..M-1, of their own block; afterwards lane g holds in A[s] item g of lane
// s's block.  One stage per lane bit: a lane keeps the items whose index has
// that bit equal to its own, swaps the others with the lane that differs in
// that bit, and re-slots both by the bit of the lane they came from.
template <int M, int K>
__device__ inline void xor_transpose(uint32_t (&A)[M][K]) {
  // Every index is a compile-time constant (static_for), so the array stays
  // in registers: with loop-variable indices the compiler may place it in LDS
  // before unrolling, one row per lane, which bank-conflicts.
  constexpr int LOGM = M == 2 ? 1 : M == 4 ? 2 : 3;
  static_assert(M == (1 << LOGM), "group of 2, 4 or 8 lanes");
  const int g = lane_id() & (M - 1);
  static_for<0, LOGM>([&](auto bc) {
    constexpr int bit = 1 << decltype(bc)::value;
    const bool up = (g & bit) != 0;
    static_for<0, M>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr ((s & bit) == 0) {
        static_for<0, K>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          const uint32_t send = up ? A[s][k] : A[s | bit][k];
          const uint32_t recv = (uint32_t)__shfl_xor((int)send, bit);
          A[s][k] = up ? recv : A[s][k];
          A[s | bit][k] = up ? A[s | bit][k] : recv;
        });
      }
    });
  });
}

// Row side: this lane's query row i (i % 4 = lane % 4) and NS sub-tiles of 32
// keys from s0 (a multiple of 32).  Element idx of sub-tile sub sits at key
// s0 + 32 sub + 16 (b / 2) + 8 hh + 4 (b % 2) + e (b = idx / 4, e = idx % 4):
// block (i / 4, s0 / 8 + 4 sub + 2 (b / 2) + hh), word i % 4, byte 4 (b % 2)
// + e.  Lane r = i % 4 of the quad runs the block of sub = r / 2 (NS = 2),
// b / 2 = r % 2; the quad then swaps words so that lane r holds word r of
// all four.
template <int NS>
struct DropRow {
  static_assert(NS == 1 || NS == 2, "granule of one or two sub-tiles");
  uint32_t w[4][2];  // [lane of the quad that ran the block][low / high dword of word i % 4]
  __device__ inline void init(const Args& a, int64_t bh, int i, int s0) {
    const int hh = lane_id() >> 5, r = lane_id() & 3;
    const int sub = NS == 2 ? r >> 1 : 0;
    const U64x4 x = philox4x64_10((uint32_t)(i >> 2), (uint32_t)(s0 / 8 + 4 * sub + 2 * (r & 1) + hh),
                                  (uint32_t)bh, 0, a.seed, 0);
    const uint64_t ww[4] = {x.w0, x.w1, x.w2, x.w3};
    static_for<0, 4>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      w[q][0] = (uint32_t)ww[q];
      w[q][1] = (uint32_t)(ww[q] >> 32);
    });
    xor_transpose<4, 2>(w);
  }
  // g of element idx (0..15) of sub-tile sub of the granule.  The word is
  // picked by selects over constant indices (see xor_transpose).
  __device__ inline float at(const Args& a, int sub, int idx) const {
    const int b = idx >> 2, q = (NS == 2 ? 2 * sub : 0) + (b >> 1), h = b & 1;
    auto wq = [&](auto qc) {
      constexpr int c = decltype(qc)::value;
      return h ? w[c][1] : w[c][0];
    };
    const uint32_t d = q == 0   ? wq(std::integral_constant<int, 0>{})
                       : q == 1 ? wq(std::integral_constant<int, 1>{})
                       : q == 2 ? wq(std::integral_constant<int, 2>{})
                                : wq(std::integral_constant<int, 3>{});
    return keep_byte(a, d, idx & 3);
  }
  __device__ inline void get(const Args& a, int sub, float (&g)[16]) const {
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) g[idx] = at(a, sub, idx);
  }
};

// Column side: this lane's key j (j % 8 = lane % 8) and NS sub-tiles of 32
// query rows from s0 (a multiple of 32).  Element idx of sub-tile sub sits at
// row s0 + 32 sub + 16 (b / 2) + 8 hh + 4 (b % 2) + e: block (s0 / 4 + 8 sub
// + 4 (b / 2) + 2 hh + b % 2, j / 8), word e, byte j % 8.  Lane r = j % 8 of
// the group of eight runs the block of sub = r / 4 (NS = 2), b = r % 4,
// packs byte q of its four words into item q, and the group swaps items so
// that lane r holds item r of all eight blocks.
template <int NS>
struct DropCol {
  static_assert(NS == 1 || NS == 2, "granule of one or two sub-tiles");
  uint32_t w[8][1];  // [lane of the group that ran the block]: byte e = word e's byte j % 8
  __device__ inline void init(const Args& a, int64_t bh, int s0, int j) {
    const int hh = lane_id() >> 5, r = lane_id() & 7;
    const int sub = NS == 2 ? r >> 2 : 0, b = r & 3;
    const U64x4 x = philox4x64_10((uint32_t)(s0 / 4 + 8 * sub + 4 * (b >> 1) + 2 * hh + (b & 1)),
                                  (uint32_t)(j >> 3), (uint32_t)bh, 0, a.seed, 0);
    const uint64_t ww[4] = {x.w0, x.w1, x.w2, x.w3};
    static_for<0, 8>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      uint32_t item = 0;
      static_for<0, 4>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        item |= (uint32_t)((ww[e] >> (8 * q)) & 0xffu) << (8 * e);
      });
      w[q][0] = item;
    });
    xor_transpose<8, 1>(w);
  }
  // g of element idx (0..15) of sub-tile sub of the granule.  The word is
  // picked by selects over constant indices (see xor_transpose).
  __device__ inline float at(const Args& a, int sub, int idx) const {
    const int q = (NS == 2 ? 4 * sub : 0) + (idx >> 2);
    uint32_t d = w[0][0];
    static_for<1, 2 * 4>([&](auto qc) {
      constexpr int c = decltype(qc)::value;
      d = q == c ? w[c][0] : d;
    });
    return keep_byte(a, d, idx & 3);
  }
  __device__ inline void get(const Args& a, int sub, float (&g)[16]) const {
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) g[idx] = at(a, sub, idx);
  }
};

// Chain-initial value of a score-shaped accumulator from a staged per-row
// scalar array: element idx gets sc[sub*32 + acc_pos(idx, hh)].
template <int TS>
__device__ inline f32x16 row_init(const float* sc, int sub) {
  const int hh = lane_id() >> 5;
  f32x16 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(sc + sub * 32 + sig(8 * b + 4 * hh));
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * b + e] = x[e];
  }
  return r;
}

// Causal attention ([FlashBoB] section 3, B_mask = -inf for key > query):
// the S-chain init of a sub-tile with keys streamed (row-side kernels) or
// queries streamed (column-side kernels) gets -inf on the masked entries.
template <int TS, bool CAUSAL>
__device__ inline f32x16 key_init(const float* kb, int sub, int key0, int row) {
  f32x16 r = row_init<TS>(kb, sub);
  if constexpr (CAUSAL) {
    const int hh = lane_id() >> 5;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx)
      if (key0 + sub * 32 + acc_pos(idx, hh) > row) r[idx] = -INFINITY;
  }
  return r;
}
template <int TS, bool CAUSAL>
__device__ inline f32x16 query_init(const float* sc, int sub, int q0, int col) {
  f32x16 r = row_init<TS>(sc, sub);
  if constexpr (CAUSAL) {
    const int hh = lane_id() >> 5;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx)
      if (q0 + sub * 32 + acc_pos(idx, hh) < col) r[idx] = -INFINITY;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Row-scalar preprocessing: D_i = sum_c dO_ic O_ic ([FA2-recompute]; the
// first backward's D_i = sum_j P_ij dP_ij).  HBM-bound: D/8 lanes per row,
// eight elements each, reduced with lane shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void rowscalar_kernel(Args a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  // With a.bs the launch also covers the padding rows of each head's last
  // 128-row block, which get the masking inits (-inf, 0).
  const int NP = a.bs ? (a.N + kPsRows - 1) / kPsRows * kPsRows : a.N;
  const int64_t total = (int64_t)a.B * a.H * NP;
  const int64_t gr = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c0 = (threadIdx.x % LPR) * 8;
  const int64_t bh = gr / NP;
  const int i = (int)(gr % NP);
  const bool valid = gr < total && i < a.N;
  float acc = 0.0f;
  if (valid) {
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const HeadPtr<T> dout = head_of<T>(a.dout, b, h);
    const HeadPtr<float> o = head_of<float>(a.o, b, h);
    const T* dr = dout.p + (int64_t)i * dout.sn + c0;
    const float* orow = o.p + (int64_t)i * o.sn + c0;
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(orow);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(orow + 4);
    float dv[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(dr);
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] = (float)x[e];
    } else {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(dr);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(dr + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dv[e] = x0[e];
        dv[e + 4] = x1[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(dv[e], o0[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(dv[e + 4], o1[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (gr < total && (threadIdx.x % LPR) == 0) {
    const int64_t rv = bh * a.N + i;
    if (valid) a.D[rv] = acc;
    if (a.bs) {
      // Chain inits of the first-backward column pass: -L/rho, -D.
      float* st = a.bs + (bh * (NP / kPsRows) + i / kPsRows) * 2 * kPsRows + i % kPsRows;
      st[0] = valid ? -a.lse[rv] / a.rho : -INFINITY;
      st[kPsRows] = valid ? -acc : 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Forward ([FlashBoB] section 3; online softmax as in [FA2-triton]).
// Resident: 32 query rows per wave.  Streamed: K (row copy, for S^T = K Q^T)
// and V (transposed copy, for O^T += V^T P^T).  Running max in base-2 units.
template <typename T, int D, int TS, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_kernel(Args a) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  constexpr int NKS = D / E::KS, NDB = D / 32, NSUB = TS / 32, KS32 = ksteps32<T>();
  __shared__ __attribute__((aligned(16))) T lds[2][2 * S::ELEMS];
  __shared__ __attribute__((aligned(16))) float kbias[2][TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<T> q = head_of<T>(a.q, wk.b, wk.h);
  HeadPtr<T> src[2] = {head_of<T>(a.k, wk.b, wk.hk), head_of<T>(a.v, wk.b, wk.hk)};

  typename E::frag qf[NKS];
  load_resident<T, D>(qf, q.p, q.sn, row, N, a.pow2);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  float m = -INFINITY, lsum = 0.0f;

  Stager<T, D, TS, 2> st;
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  ScalarStager<TS, 1> ks;
  auto kvalid = [](int, float* o) { o[0] = 0.0f; };
  auto kpad = [](float* o) { o[0] = -INFINITY; };
  st.load(src, 0, N);
  ks.load(0, N, kvalid, kpad);
  st.store(lds[0]);
  ks.store(kbias[0]);
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    if (t + 1 < t_end) {
      st.load(src, (t + 1) * TS, N);
      ks.load((t + 1) * TS, N, kvalid, kpad);
    }
    const float* kb = kbias[t & 1];
    const T* kr = lds[t & 1];
    const T* vt = lds[t & 1] + S::ELEMS + S::ROW_ELEMS;
    DropRow<NSUB> dm;
    if constexpr (DROP) dm.init(a, wk.bh, row, t * TS);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const f32x16 s = mm_row<T, D, TS>(kr, sub, qf, key_init<TS, CAUSAL>(kb, sub, t * TS, row));
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        z[idx] = s[idx] * a.c1;
        mx = fmaxf(mx, z[idx]);
      }
      mx = half_max(mx);
      const float mn = fmaxf(m, mx);
      const float ms = (mn == -INFINITY) ? 0.0f : mn;
      const float sc = __builtin_amdgcn_exp2f(m - ms);
      float p[16];
      float ps = 0.0f;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        p[idx] = __builtin_amdgcn_exp2f(z[idx] - ms);
        ps += p[idx];
      }
      lsum = lsum * sc + ps;
      m = mn;
      Chain<T> cp;
      if constexpr (DROP) {
        // O = (P * g) V; the row sum (and L) is over P.
        float g[16];
        dm.get(a, sub, g);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) g[idx] *= p[idx];
        cp.set(g);
      } else {
        cp.set(p);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= sc;
#pragma unroll
        for (int s2 = 0; s2 < KS32; ++s2) acc[db] = E::mma(tr_frag<T, D, TS>(vt, db, sub, s2), cp.f[s2], acc[db]);
      }
    }
    if (t + 1 < t_end) {
      st.store(lds[(t + 1) & 1]);
      ks.store(kbias[(t + 1) & 1]);
    }
    __syncthreads();
  }
  const float lt = half_sum(lsum);
  const float inv = 1.0f / lt;
  float* o = head_out(a.r0, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_out(o, a.r0.sn, row, N, db, [&](int idx) { return acc[db][idx] * inv; });
  if (row < N && hh == 0) a.lse_out[(int64_t)wk.bh * N + row] = kLn2 * (m + __log2f(lt));
}

// ---------------------------------------------------------------------------
// First backward, row side: dQ = tau dS K with dS = P (dP - D)
// ([FlashBoB] section 3).  Resident: query rows.  Streamed: K, V.
template <typename T, int D, int TS, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dq_kernel(Args a) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  constexpr int NKS = D / E::KS, NDB = D / 32, NSUB = TS / 32, KS32 = ksteps32<T>();
  __shared__ __attribute__((aligned(16))) T lds[2][2 * S::ELEMS];
  __shared__ __attribute__((aligned(16))) float kbias[2][TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<T> q = head_of<T>(a.q, wk.b, wk.h), dout = head_of<T>(a.dout, wk.b, wk.h);
  HeadPtr<T> src[2] = {head_of<T>(a.k, wk.b, wk.hk), head_of<T>(a.v, wk.b, wk.hk)};

  typename E::frag qf[NKS], df[NKS];
  load_resident<T, D>(qf, q.p, q.sn, row, N, a.pow2);
  load_resident<T, D>(df, dout.p, dout.sn, row, N, 1.0f);
  const int64_t rv = (int64_t)wk.bh * N;
  const float Li = row < N ? a.lse[rv + row] : 0.0f;
  const float Di = row < N ? a.D[rv + row] : 0.0f;
  const float nl2 = -Li * kLog2e;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  Stager<T, D, TS, 2> st;
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  ScalarStager<TS, 1> ks;
  auto kvalid = [](int, float* o) { o[0] = 0.0f; };
  auto kpad = [](float* o) { o[0] = -INFINITY; };
  st.load(src, 0, N);
  ks.load(0, N, kvalid, kpad);
  st.store(lds[0]);
  ks.store(kbias[0]);
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    if (t + 1 < t_end) {
      st.load(src, (t + 1) * TS, N);
      ks.load((t + 1) * TS, N, kvalid, kpad);
    }
    const float* kb = kbias[t & 1];
    const T* kr = lds[t & 1];
    const T* kt = kr + S::ROW_ELEMS;
    const T* vr = kr + S::ELEMS;
    DropRow<NSUB> dm;
    if constexpr (DROP) dm.init(a, wk.bh, row, t * TS);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const f32x16 s = mm_row<T, D, TS>(kr, sub, qf, key_init<TS, CAUSAL>(kb, sub, t * TS, row));
      const f32x16 dp = mm_row<T, D, TS>(vr, sub, df, zero16());
      float ds[16], g[16];
      if constexpr (DROP) dm.get(a, sub, g);
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], a.c1, nl2));
        // With dropout dP becomes g * (dO V^T).
        ds[idx] = p * ((DROP ? g[idx] * dp[idx] : dp[idx]) - Di);
      }
      Chain<T> cds;
      cds.set(ds);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < KS32; ++s2) acc[db] = E::mma(tr_frag<T, D, TS>(kt, db, sub, s2), cds.f[s2], acc[db]);
    }
    if (t + 1 < t_end) {
      st.store(lds[(t + 1) & 1]);
      ks.store(kbias[(t + 1) & 1]);
    }
    __syncthreads();
  }
  float* dq = head_out(a.r0, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_out(dq, a.r0.sn, row, N, db, [&](int idx) { return a.tau * acc[db][idx]; });
}

// First backward, column side: dV = P^T dO, dK = tau dS^T Q
// ([FlashBoB] section 3).  Resident: key rows.  Streamed: Q, dO and the row
// scalars (-L/rho, -D).
template <typename T, int D, int TS, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(Args a) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  constexpr int NKS = D / E::KS, NDB = D / 32, NSUB = TS / 32, KS32 = ksteps32<T>();
  __shared__ __attribute__((aligned(16))) T lds[2][2 * S::ELEMS];
  __shared__ __attribute__((aligned(16))) float scl[2][2 * TS];

  const Work wk = work_item_cols(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int col = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<T> k = head_of<T>(a.k, wk.b, wk.hk), v = head_of<T>(a.v, wk.b, wk.hk);
  HeadPtr<T> src[2];

  typename E::frag kf[NKS], vf[NKS];
  load_resident<T, D>(kf, k.p, k.sn, col, N, a.pow2);
  load_resident<T, D>(vf, v.p, v.sn, col, N, 1.0f);
  int64_t rv = 0;  // row-vector base of the query head being staged
  const float irho = 1.0f / a.rho;
  auto scal = [&](int row, float* o) {
    o[0] = -a.lse[rv + row] * irho;
    o[1] = -a.D[rv + row];
  };
  auto pad = [](float* o) {
    o[0] = -INFINITY;
    o[1] = 0.0f;
  };

  f32x16 ak[NDB], av[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) ak[db] = av[db] = zero16();

  Stager<T, D, TS, 2> st;
  ScalarStager<TS, 2> ss;
  // Row tiles of the G query heads of this key/value head in sequence, all
  // into the same accumulators: tile u is row tile t_begin + u % ntq of query
  // head h + u / ntq.
  const int nt = (N + TS - 1) / TS;
  const int t_begin = CAUSAL ? wk.rb * kResRows / TS : 0;
  const int ntq = nt - t_begin, nu = a.G * ntq;
  auto load_tile = [&](int u) {
    const int hq = wk.h + u / ntq, t = t_begin + u % ntq;
    src[0] = head_of<T>(a.q, wk.b, hq);
    src[1] = head_of<T>(a.dout, wk.b, hq);
    rv = ((int64_t)wk.b * a.H + hq) * N;
    st.load(src, t * TS, N);
    ss.load(t * TS, N, scal, pad);
  };
  load_tile(0);
  st.store(lds[0]);
  ss.store(scl[0]);
  __syncthreads();
  for (int u = 0; u < nu; ++u) {
    const int t = t_begin + u % ntq;
    if (u + 1 < nu) load_tile(u + 1);
    const T* qr = lds[u & 1];
    const T* qt = qr + S::ROW_ELEMS;
    const T* dr = qr + S::ELEMS;
    const T* dt = dr + S::ROW_ELEMS;
    const float* sc = scl[u & 1];
    DropCol<NSUB> dm;
    if constexpr (DROP) dm.init(a, (int64_t)wk.b * a.H + wk.h + u / ntq, t * TS, col);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const f32x16 s = mm_row<T, D, TS>(qr, sub, kf, query_init<TS, CAUSAL>(sc, sub, t * TS, col));
      // Without dropout dP starts from -D; with it dP = g * (dO V^T) - D.
      const f32x16 dp = mm_row<T, D, TS>(dr, sub, vf, DROP ? zero16() : row_init<TS>(sc + TS, sub));
      float p[16], ds[16], g[16];
      f32x16 nd = zero16();
      if constexpr (DROP) {
        dm.get(a, sub, g);
        nd = row_init<TS>(sc + TS, sub);
      }
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float pp = __builtin_amdgcn_exp2f(s[idx] * a.c1);
        p[idx] = DROP ? pp * g[idx] : pp;
        ds[idx] = pp * (DROP ? fmaf(g[idx], dp[idx], nd[idx]) : dp[idx]);
      }
      Chain<T> cp, cds;
      cp.set(p);
      cds.set(ds);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < KS32; ++s2) {
          av[db] = E::mma(tr_frag<T, D, TS>(dt, db, sub, s2), cp.f[s2], av[db]);
          ak[db] = E::mma(tr_frag<T, D, TS>(qt, db, sub, s2), cds.f[s2], ak[db]);
        }
    }
    if (u + 1 < nu) {
      st.store(lds[(u + 1) & 1]);
      ss.store(scl[(u + 1) & 1]);
    }
    __syncthreads();
  }
  float* dk = head_out(a.r1, wk.b, wk.hk);
  float* dv = head_out(a.r2, wk.b, wk.hk);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    store_out(dk, a.r1.sn, col, N, db, [&](int idx) { return a.tau * ak[db][idx]; });
    store_out(dv, a.r2.sn, col, N, db, [&](int idx) { return av[db][idx]; });
  }
}

// ---------------------------------------------------------------------------
// BoB pass 1 (row-major; [FlashBoB] section 4.3, Algorithm 1's first pass).
// Resident per wave: 32 query rows i with q_i, u_Q,i (scaled by pow2), do_i,
// and the row scalars L_i, D_i.  Streamed: K, V, U_K, U_V.  Per 32 x 32
// tile (streamed index j on M):
//   S^T = K Q^T,  F^T = K U_Q^T + U_K Q^T,  dP^T = V dO^T,  C^T = U_V dO^T
//   P = exp(tau S - L),  dPD = dP - D,  P~ = C + F dPD   (d~P before the
//   alpha correction), then the alpha-free accumulators of the affine
//   fusion (section 4.2):
//     alpha += sum_j P F            E° += sum_j P P~
//     G     += P U_V + (P F) V      (d~(dO) before the correction)
//     Om    += (P P~) K + dS U_K    with dS = P dPD
//     R'    += dS K                 Bk += P K
// Epilogue (the corrections of section 4.2, with R = R' + D Bk so that
// alpha R + E Bk = alpha R' + E° Bk):
//     E = E° - alpha D,  gdo = G - alpha o,  gq = tau (Om - alpha R' - E° Bk).
template <typename T, int D, int TS, bool RHO1, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bob_pass1_kernel(Args a) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  constexpr int NKS = D / E::KS, NDB = D / 32, NSUB = TS / 32, KS32 = ksteps32<T>();
  __shared__ __attribute__((aligned(16))) T lds[2][4 * S::ELEMS];
  __shared__ __attribute__((aligned(16))) float kbias[2][TS];

  const Work wk = work_item(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int row = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<T> q = head_of<T>(a.q, wk.b, wk.h), uq = head_of<T>(a.uq, wk.b, wk.h),
                   dout = head_of<T>(a.dout, wk.b, wk.h);
  HeadPtr<T> src[4] = {head_of<T>(a.k, wk.b, wk.hk), head_of<T>(a.v, wk.b, wk.hk), head_of<T>(a.uk, wk.b, wk.hk),
                       head_of<T>(a.uv, wk.b, wk.hk)};

  typename E::frag qf[NKS], uqf[NKS], df[NKS];
  load_resident<T, D>(qf, q.p, q.sn, row, N, a.pow2);
  load_resident<T, D>(uqf, uq.p, uq.sn, row, N, a.pow2);
  load_resident<T, D>(df, dout.p, dout.sn, row, N, 1.0f);
  const int64_t rv = (int64_t)wk.bh * N;
  const float Li = row < N ? a.lse[rv + row] : 0.0f;
  const float Di = row < N ? a.D[rv + row] : 0.0f;
  const float nl2 = -Li * kLog2e;

  f32x16 ag[NDB], aom[NDB], ar[NDB], abk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) ag[db] = aom[db] = ar[db] = abk[db] = zero16();
  float alpha_p = 0.0f, eo_p = 0.0f;

  Stager<T, D, TS, 4> st;
  const int nt = (N + TS - 1) / TS;
  const int t_end = CAUSAL ? min(nt, (wk.rb * kResRows + kResRows + TS - 1) / TS) : nt;
  ScalarStager<TS, 1> ks;
  auto kvalid = [](int, float* o) { o[0] = 0.0f; };
  auto kpad = [](float* o) { o[0] = -INFINITY; };
  st.load(src, 0, N);
  ks.load(0, N, kvalid, kpad);
  st.store(lds[0]);
  ks.store(kbias[0]);
  __syncthreads();
  for (int t = 0; t < t_end; ++t) {
    if (t + 1 < t_end) {
      st.load(src, (t + 1) * TS, N);
      ks.load((t + 1) * TS, N, kvalid, kpad);
    }
    const float* kb = kbias[t & 1];
    const T* kr = lds[t & 1];
    const T* kt = kr + S::ROW_ELEMS;
    const T* vr = kr + S::ELEMS;
    const T* vt = vr + S::ROW_ELEMS;
    const T* ukr = kr + 2 * S::ELEMS;
    const T* ukt = ukr + S::ROW_ELEMS;
    const T* uvr = kr + 3 * S::ELEMS;
    const T* uvt = uvr + S::ROW_ELEMS;
    DropRow<NSUB> dm;
    if constexpr (DROP) dm.init(a, wk.bh, row, t * TS);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const f32x16 s = mm_row<T, D, TS>(kr, sub, qf, key_init<TS, CAUSAL>(kb, sub, t * TS, row));
      f32x16 f = mm_row<T, D, TS>(kr, sub, uqf, zero16());
      f = mm_row<T, D, TS>(ukr, sub, qf, f);
      const f32x16 dp = mm_row<T, D, TS>(vr, sub, df, zero16());
      const f32x16 c = mm_row<T, D, TS>(uvr, sub, df, zero16());
      // Dropout (the analytical extension of [FlashBoB] appendix G): dP and
      // C become g * (dO V^T) and g * (dO U_V^T); the products with V and
      // U_V (the d~(dO) accumulator G) take P * g; alpha, E°, Om, R' and Bk
      // keep P.
      float P[16], PF[16], PT[16], DS[16], g[16];
      if constexpr (DROP) dm.get(a, sub, g);
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[idx], a.c1, nl2));
        const float F = RHO1 ? f[idx] : f[idx] * a.rho;
        const float dpd = (DROP ? g[idx] * dp[idx] : dp[idx]) - Di;
        const float t0 = fmaf(F, dpd, DROP ? g[idx] * c[idx] : c[idx]);
        P[idx] = p;
        PF[idx] = p * F;
        PT[idx] = p * t0;
        DS[idx] = p * dpd;
        alpha_p += PF[idx];
        eo_p += PT[idx];
      }
      Chain<T> cp, cpf, cpt, cds, cpg, cpfg;
      cp.set(P);
      cpf.set(PF);
      cpt.set(PT);
      cds.set(DS);
      if constexpr (DROP) {
        float PG[16], PFG[16];
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          PG[idx] = P[idx] * g[idx];
          PFG[idx] = PF[idx] * g[idx];
        }
        cpg.set(PG);
        cpfg.set(PFG);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < KS32; ++s2) {
          const typename E::frag xuv = tr_frag<T, D, TS>(uvt, db, sub, s2);
          const typename E::frag xv = tr_frag<T, D, TS>(vt, db, sub, s2);
          const typename E::frag xk = tr_frag<T, D, TS>(kt, db, sub, s2);
          const typename E::frag xuk = tr_frag<T, D, TS>(ukt, db, sub, s2);
          ag[db] = E::mma(xuv, DROP ? cpg.f[s2] : cp.f[s2], ag[db]);
          ag[db] = E::mma(xv, DROP ? cpfg.f[s2] : cpf.f[s2], ag[db]);
          aom[db] = E::mma(xk, cpt.f[s2], aom[db]);
          aom[db] = E::mma(xuk, cds.f[s2], aom[db]);
          ar[db] = E::mma(xk, cds.f[s2], ar[db]);
          abk[db] = E::mma(xk, cp.f[s2], abk[db]);
        }
    }
    if (t + 1 < t_end) {
      st.store(lds[(t + 1) & 1]);
      ks.store(kbias[(t + 1) & 1]);
    }
    __syncthreads();
  }

  const float alpha = half_sum(alpha_p);
  const float eo = half_sum(eo_p);
  if (row < N && hh == 0) {
    a.alpha[rv + row] = alpha;
    a.E[rv + row] = eo - alpha * Di;
  }
  const HeadPtr<float> o = head_of<float>(a.o, wk.b, wk.h);
  float* gq = head_out(a.r0, wk.b, wk.h);
  float* gdo = head_out(a.r3, wk.b, wk.h);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
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
              [&](int idx) { return a.tau * (aom[db][idx] - alpha * ar[db][idx] - eo * abk[db][idx]); });
  }
}

// ---------------------------------------------------------------------------
// BoB pass 2 (column-major; [FlashBoB] section 4.3, Algorithm 1's second
// pass).  Resident per wave: 32 key rows j with k_j, u_K,j (scaled by pow2),
// v_j, u_V,j.  Streamed: Q, dO, U_Q and the row scalars L, D, alpha, E,
// staged as MFMA chain initial values -L/rho, -D, -alpha/rho,
// -(alpha D + E).  Per tile (streamed index i on M):
//   s = (tau S - L)/rho,  h/rho = (F - alpha)/rho,  dPD = dP - D,
//   C' = C - alpha D - E,
//   P = exp(tau S - L),   d~P - E = C' + h dPD,
//   d~S = P (d~P - E),    dS = P dPD,    W = P h,
//   gk += d~S^T Q + dS^T U_Q (times tau at the end),  gv += W^T dO.
template <typename T, int D, int TS, bool RHO1, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bob_pass2_kernel(Args a) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  constexpr int NKS = D / E::KS, NDB = D / 32, NSUB = TS / 32, KS32 = ksteps32<T>();
  __shared__ __attribute__((aligned(16))) T lds[2][3 * S::ELEMS];
  __shared__ __attribute__((aligned(16))) float scl[2][4 * TS];

  const Work wk = work_item_cols(a, CAUSAL);
  const int N = a.N;
  const int l = lane_id(), hh = l >> 5;
  const int col = wk.rb * kResRows + (threadIdx.x >> 6) * 32 + (l & 31);
  const HeadPtr<T> k = head_of<T>(a.k, wk.b, wk.hk), v = head_of<T>(a.v, wk.b, wk.hk),
                   uk = head_of<T>(a.uk, wk.b, wk.hk), uv = head_of<T>(a.uv, wk.b, wk.hk);
  HeadPtr<T> src[3];

  typename E::frag kf[NKS], vf[NKS], ukf[NKS], uvf[NKS];
  load_resident<T, D>(kf, k.p, k.sn, col, N, a.pow2);
  load_resident<T, D>(ukf, uk.p, uk.sn, col, N, a.pow2);
  load_resident<T, D>(vf, v.p, v.sn, col, N, 1.0f);
  load_resident<T, D>(uvf, uv.p, uv.sn, col, N, 1.0f);
  int64_t rv = 0;  // row-vector base of the query head being staged
  const float irho = 1.0f / a.rho;
  auto scal = [&](int row, float* o) {
    const float L = a.lse[rv + row], Dd = a.D[rv + row], al = a.alpha[rv + row], Ee = a.E[rv + row];
    o[0] = -L * irho;
    o[1] = -Dd;
    o[2] = -al * irho;
    o[3] = -fmaf(al, Dd, Ee);
  };
  auto pad = [](float* o) {
    o[0] = -INFINITY;
    o[1] = o[2] = o[3] = 0.0f;
  };

  f32x16 ak[NDB], av[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) ak[db] = av[db] = zero16();

  Stager<T, D, TS, 3> st;
  ScalarStager<TS, 4> ss;
  // Row tiles of the G query heads of this key/value head in sequence (see
  // bwd_dkdv_kernel).
  const int nt = (N + TS - 1) / TS;
  const int t_begin = CAUSAL ? wk.rb * kResRows / TS : 0;
  const int ntq = nt - t_begin, nu = a.G * ntq;
  auto load_tile = [&](int u) {
    const int hq = wk.h + u / ntq, t = t_begin + u % ntq;
    src[0] = head_of<T>(a.q, wk.b, hq);
    src[1] = head_of<T>(a.dout, wk.b, hq);
    src[2] = head_of<T>(a.uq, wk.b, hq);
    rv = ((int64_t)wk.b * a.H + hq) * N;
    st.load(src, t * TS, N);
    ss.load(t * TS, N, scal, pad);
  };
  load_tile(0);
  st.store(lds[0]);
  ss.store(scl[0]);
  __syncthreads();
  for (int u = 0; u < nu; ++u) {
    const int t = t_begin + u % ntq;
    if (u + 1 < nu) load_tile(u + 1);
    const T* qr = lds[u & 1];
    const T* qt = qr + S::ROW_ELEMS;
    const T* dr = qr + S::ELEMS;
    const T* dt = dr + S::ROW_ELEMS;
    const T* uqr = qr + 2 * S::ELEMS;
    const T* uqt = uqr + S::ROW_ELEMS;
    const float* sc = scl[u & 1];
    DropCol<NSUB> dm;
    if constexpr (DROP) dm.init(a, (int64_t)wk.b * a.H + wk.h + u / ntq, t * TS, col);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const f32x16 s = mm_row<T, D, TS>(qr, sub, kf, query_init<TS, CAUSAL>(sc, sub, t * TS, col));
      f32x16 f = mm_row<T, D, TS>(uqr, sub, kf, row_init<TS>(sc + 2 * TS, sub));
      f = mm_row<T, D, TS>(qr, sub, ukf, f);
      // Dropout: dP = g * (dO V^T) - D and C' = g * (dO U_V^T) - alpha D - E,
      // so the chains start at 0 and take the row scalars after g; W = P g h.
      f32x16 dp = mm_row<T, D, TS>(dr, sub, vf, DROP ? zero16() : row_init<TS>(sc + TS, sub));
      f32x16 c = mm_row<T, D, TS>(dr, sub, uvf, DROP ? zero16() : row_init<TS>(sc + 3 * TS, sub));
      float g[16];
      if constexpr (DROP) {
        dm.get(a, sub, g);
        const f32x16 nd = row_init<TS>(sc + TS, sub), nc = row_init<TS>(sc + 3 * TS, sub);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          dp[idx] = fmaf(g[idx], dp[idx], nd[idx]);
          c[idx] = fmaf(g[idx], c[idx], nc[idx]);
        }
      }
      float DT[16], DS[16], W[16];
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const float p = __builtin_amdgcn_exp2f(s[idx] * a.c1);
        const float h = RHO1 ? f[idx] : f[idx] * a.rho;
        const float x = fmaf(h, dp[idx], c[idx]);
        DT[idx] = p * x;
        DS[idx] = p * dp[idx];
        W[idx] = DROP ? p * g[idx] * h : p * h;
      }
      Chain<T> cdt, cds, cw;
      cdt.set(DT);
      cds.set(DS);
      cw.set(W);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < KS32; ++s2) {
          ak[db] = E::mma(tr_frag<T, D, TS>(qt, db, sub, s2), cdt.f[s2], ak[db]);
          ak[db] = E::mma(tr_frag<T, D, TS>(uqt, db, sub, s2), cds.f[s2], ak[db]);
          av[db] = E::mma(tr_frag<T, D, TS>(dt, db, sub, s2), cw.f[s2], av[db]);
        }
    }
    if (u + 1 < nu) {
      st.store(lds[(u + 1) & 1]);
      ss.store(scl[(u + 1) & 1]);
    }
    __syncthreads();
  }
  float* gk = head_out(a.r1, wk.b, wk.hk);
  float* gv = head_out(a.r2, wk.b, wk.hk);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    store_out(gk, a.r1.sn, col, N, db, [&](int idx) { return a.tau * ak[db][idx]; });
    store_out(gv, a.r2.sn, col, N, db, [&](int idx) { return av[db][idx]; });
  }
}

}  // namespace fa
