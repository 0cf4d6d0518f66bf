// fa_bob_ws.hip -- warp-specialised bf16 row pass of the backward-over-
// backward for gfx950, d = 64.
//
// Source: [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward
// for Softmax Attention", section 4.2 (Proposition 4.1: six row accumulators
// and the corrections (8)), section 4.3 (Algorithm 1, pass 1).
//
// One workgroup = 8 waves = 128 query rows, two waves per SIMD (waves w and
// w + 4 share one):
//   * producer wave i (waves 0-3) owns rows 32 i .. 32 i + 31 of the block:
//     it computes the score chains S, F, dP, C of each 32-key tile on the
//     matrix cores, does the elementwise work (P, the row sums alpha and E°)
//     and writes the bf16 B operands P, P F, P P~, dS to LDS;
//   * consumer wave i (waves 4-7) holds the four d-wide accumulators of the
//     same rows and runs the 24 accumulation MFMAs of each tile from those
//     operands and the transposed K, V, U_K, U_V tiles.
// The roles meet in LDS once per 32-key slot, separated by a workgroup
// barrier:
//   slot s: producer: scores(s) into register set s % 2, interleaved with
//                     elementwise(s - 1) from set (s - 1) % 2 -> operands
//                     buffer (s - 1) % 2;
//           consumer: accumulations(s - 2) from operands buffer s % 2 and
//                     key tile s - 2;
//           everyone: copies of key tile s + 2 (LDS DMA), five tile stages.
// Inside a producer slot every score MFMA is followed by the VALU work of one
// element of the previous tile (scheduling barriers keep that order), so the
// producer's matrix-core and vector work overlap, and the consumer's MFMAs
// fill the matrix core while the producer's VALU runs.
#include <type_traits>

#include "fa_lds.h"

namespace fa {

// d += a * b with every operand in VGPRs (no AGPRs in this kernel: the two
// waves of a SIMD share 512 registers).  W: with the two wait states of a
// VALU write in front, for the key-split instance, whose register allocation
// gathers some operands with v_mov right before the MFMA.
template <bool W = false>
__device__ inline void mfma_vv(f32x16& d, bf16x8 a, bf16x8 b) {
  if constexpr (W)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
template <bool W = false>
__device__ inline f32x16 mfma_vv_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  if constexpr (W)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
// d = a * b + c, with c in its own registers (kept).  The matrix core reads
// c after issue, so a write of c's registers must wait 7 wait states; the
// compiler does not know that about an asm MFMA (it may reuse them right
// after the last one), so the wait is part of the instruction here.
template <bool W = false>
__device__ inline f32x16 mfma_vv_init(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  if constexpr (W)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 6" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 6" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ inline void vfence4(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// acc += x at this point of the instruction stream (a scheduling barrier does
// not hold plain arithmetic, which the compiler would otherwise gather at the
// end of the slot, keeping every addend live until then).
__device__ inline void add_here(float& acc, float x) { asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(x)); }

// Two floats as a packed pair of bf16 (element 0 in the low half).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(bf16)lo, (bf16)hi};
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  asm("" : "+v"(u));  // one conversion for both halves, also where only one half is read back
  return u;
}

typedef const __attribute__((address_space(3))) char* lds_cp;
typedef __attribute__((address_space(3))) char* lds_p;

// LDS offsets inside the stage region are masked to its size, so that the
// compiler can prove the base of an LDS access non-negative and fold the
// constant part of the address into the instruction's offset field.
constexpr uint32_t kStageMask = 0x1ffff;

// Copies of one 32-row key tile of K, V, U_K, U_V (4 x 4 KB = 16 blocks of
// 64 granules) by 8 waves, two blocks each.  Rows at or past N are read from
// row N - 1 (masked to P = 0 by the producer).  Full tiles advance two
// wave-uniform row pointers; only a ragged last tile computes its rows.
struct WsDma {
  typedef SwTile<64, 32> W;
  const char* base[2];  // tensors t0 and t0 + 2 (selected once: no dynamic indexing)
  const char* next[2];  // block b of the next tile
  int64_t rs[2];
  uint32_t offt[2];     // per-lane offset inside a block
  int jl, b, t0;

  // row_start: the first row the copies start from (a multiple of 32).
  __device__ inline void init(const HeadPtr<bf16>* src, int row_start) {
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    b = wave & 3;      // block (8 rows) inside each tensor tile
    t0 = wave >> 2;    // this wave copies tensors t0 and t0 + 2
    jl = lane >> 3;
    const int q = (lane & 7) ^ swz<8>(b * 8 + jl);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const HeadPtr<bf16> h = t0 ? src[2 * k + 1] : src[2 * k];
      base[k] = reinterpret_cast<const char*>(h.p);
      rs[k] = h.sn * 2;
      offt[k] = (uint32_t)(jl * (int)rs[k] + 16 * q);
      next[k] = base[k] + (int64_t)(row_start + b * 8) * rs[k];
    }
  }

  // Copy the tile of rows row0 .. row0 + 31.  Tiles are copied in order,
  // each once.
  __device__ inline void copy(int row0, int N, const char* dst) {
    const uint32_t lbase = lds_addr(dst);
    const int r0 = row0 + b * 8;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t lds = lbase + (t0 + 2 * k) * W::BYTES + b * 1024;
      if (r0 + 8 <= N) {
        dma16_so(next[k], offt[k], lds);
      } else {
        const int row = min(r0 + jl, N - 1);
        dma16(base[k] + row * rs[k] + (offt[k] - jl * (int)rs[k]), lds);
      }
      next[k] += 32 * rs[k];
    }
  }
};

// KSPLIT: the key-split instance (a.ks > 1, see key_range): a range of the
// keys and raw partial sums instead of the epilogue, in its own instance so
// that the unsplit kernel is compiled without it.
template <bool RHO1, bool CAUSAL, bool KSPLIT = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bob_pass1_ws_kernel(Args a) {
  static_assert(!(KSPLIT && CAUSAL), "the key split is not causal");
  constexpr int D = 64, TS = 32, NKS = 4, NDB = 2;
  typedef SwTile<D, TS> W;
  constexpr int NSTAGE = 5;
  constexpr int STAGE = 4 * W::BYTES;    // 16 KB
  constexpr int OPB = 4 * 2 * 64 * 16;   // operands of one wave and tile: 8 KB
  // Operand buffer of a wave: word w (0..7) of the four chains (P, P F, P P~,
  // dS) of a lane as one 16-byte group, lane-contiguous ([w][lane][k] words):
  // the producer writes the four words of an element pair with one 128-bit
  // store and the consumer reads four of them with one 128-bit load, both
  // free of bank conflicts.
  auto op_off = [](int w) { return w * 64 * 16; };
  static_assert(NSTAGE * STAGE <= (int)kStageMask + 1, "stage region larger than its offset mask");
  __shared__ __attribute__((aligned(1024))) char stages[NSTAGE * STAGE];
  __shared__ __attribute__((aligned(1024))) char ops[2][4 * OPB];
  __shared__ float rowx[4][32];  // alpha handed from producer to consumer

  const int nblk = (a.N + kResRows - 1) / kResRows;
  const int wid0 = xcd_remap(blockIdx.x, gridDim.x);
  const int kk = KSPLIT ? wid0 / (a.B * a.H * nblk) : 0;  // key range
  const int wid = wid0 - kk * (a.B * a.H * nblk);
  // Causal: the largest row blocks of a head first (see work_item).
  int bh, rb;
  if constexpr (CAUSAL) {
    int k;
    longest_first(wid, gridDim.x, nblk, bh, k);
    rb = nblk - 1 - k;
  } else {
    bh = wid / nblk;
    rb = wid % nblk;
  }
  const int bb = bh / a.H, hd = bh % a.H, hk = hd / a.G;
  const int N = a.N;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool producer = wave < 4;
  const int wi = wave & 3;
  const int l = lane_id(), hh = l >> 5;
  const int r0 = rb * kResRows;
  const int row = r0 + wi * 32 + (l & 31);

  HeadPtr<bf16> src[4] = {head_of<bf16>(a.k, bb, hk), head_of<bf16>(a.v, bb, hk), head_of<bf16>(a.uk, bb, hk),
                          head_of<bf16>(a.uv, bb, hk)};
  // Key tiles kt0 .. kt0 + nt - 1; slot and tile numbers below count from kt0.
  int kt0 = 0, nt = CAUSAL ? min((N + TS - 1) / TS, (r0 + kResRows) / TS) : (N + TS - 1) / TS;
  if constexpr (KSPLIT) {
    int kt1;
    key_range(a, kk, nt, kt0, kt1);
    nt = kt1 - kt0;
  }
  WsDma dma;
  dma.init(src, kt0 * TS);
  dma.copy(kt0 * TS, N, stages);
  if (nt > 1) dma.copy((kt0 + 1) * TS, N, stages + STAGE);

  Reader<D, TS> rd;
  const int64_t rv = (int64_t)bh * N;
  // Stage offset of key tile t.
  auto stage_off = [](int t) { return (uint32_t)((t % NSTAGE) * STAGE); };
  // LDS address rel + lane_off inside the stage region, formed once per use
  // (opaque to the optimiser, which would otherwise keep one precomputed
  // address per stage and lane offset live) and masked so that constant
  // offsets added to it fold into the instruction.
  auto stage_ptr = [&](uint32_t rel, int lane_off) {
    uint32_t r = rel + (uint32_t)lane_off;
    asm volatile("" : "+v"(r));
    return (lds_cp)stages + (r & kStageMask);
  };
  // End of a slot: this slot's copies may stay in flight unless they are the
  // last ones; operand writes and stage reads are complete at the barrier.
  auto end_slot = [&](int sl) {
    if (sl + 2 < nt) {
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  };

  if (producer) {
    // ------------------------------------------------------------ producer
    const HeadPtr<bf16> q = head_of<bf16>(a.q, bb, hd), uq = head_of<bf16>(a.uq, bb, hd),
                        dout = head_of<bf16>(a.dout, bb, hd);
    bf16x8 qf[NKS], uqf[NKS], df[NKS];
    load_resident<bf16, D>(qf, q.p, q.sn, row, N, a.pow2);
    load_resident<bf16, D>(uqf, uq.p, uq.sn, row, N, a.pow2);
    load_resident<bf16, D>(df, dout.p, dout.sn, row, N, 1.0f);
    const float Li = row < N ? a.lse[rv + row] : 0.0f;
    // D = rowsum(dO * O) of this row, computed here and written for the column pass.
    const float Di = resident_rowdot<D>(df, head_of<float>(a.o, bb, hd), row, N);
    // The dP chains start from -D (the MFMA's C operand), so dP - D comes out
    // of the matrix core.
    f32x16 negd;
#pragma unroll
    for (int e = 0; e < 16; ++e) negd[e] = -Di;
    const float nl2 = -Li * kLog2e;
    float alpha_p = 0.0f, eo_p = 0.0f;
    rd.init();
    f32x16 S[2], F[2], DP[2], C[2];  // score chains, double buffered across slots
    const lds_p ob0 = (lds_p)ops[0] + wi * OPB + 16 * l;  // this wave's operand buffers
    const lds_p ob1 = (lds_p)ops[1] + wi * OPB + 16 * l;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // the compiler's own loads are done before the loop
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // A operand `which` (0 K, 1 V, 2 U_K, 3 U_V) of a k-step whose rows start
    // at b (one address per k-step; the tensors sit at constant offsets).
    auto rd_a = [&](lds_cp b, int which) {
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(b + which * W::BYTES);
    };
    // Scores of key tile t into set P: per k-step ks, S += K q, F += K u_q,
    // dP += V do, C += U_V do, F += U_K q; group(g) runs after MFMA g
    // (g = 0..19).  Each A operand of k-step ks + 1 is read into the
    // registers of k-step ks right after the last MFMA that uses them.
    auto scores = [&](auto Pc, int t, auto&& group) {
      constexpr int P = decltype(Pc)::value;
      const uint32_t rel = stage_off(t);
      lds_cp bk = stage_ptr(rel, rd.row[0]);
      bf16x8 xk = rd_a(bk, 0), xv = rd_a(bk, 1), xuk = rd_a(bk, 2), xuv = rd_a(bk, 3);
      sched_fence();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bool more = ks + 1 < NKS;
        if (ks == 0) {
          S[P] = mfma_vv_first<KSPLIT>(xk, qf[0]);
          group(0);
          sched_fence();
          F[P] = mfma_vv_first<KSPLIT>(xk, uqf[0]);
        } else {
          mfma_vv<KSPLIT>(S[P], xk, qf[ks]);
          group(5 * ks);
          sched_fence();
          mfma_vv<KSPLIT>(F[P], xk, uqf[ks]);
        }
        if (more) {
          bk = stage_ptr(rel, rd.row[ks + 1]);
          xk = rd_a(bk, 0);
        }
        group(5 * ks + 1);
        sched_fence();
        if (ks == 0) {
          DP[P] = mfma_vv_init<KSPLIT>(xv, df[0], negd);
        } else {
          mfma_vv<KSPLIT>(DP[P], xv, df[ks]);
        }
        if (more) xv = rd_a(bk, 1);
        group(5 * ks + 2);
        sched_fence();
        if (ks == 0) {
          C[P] = mfma_vv_first<KSPLIT>(xuv, df[0]);
        } else {
          mfma_vv<KSPLIT>(C[P], xuv, df[ks]);
        }
        if (more) xuv = rd_a(bk, 3);
        group(5 * ks + 3);
        sched_fence();
        mfma_vv<KSPLIT>(F[P], xuk, qf[ks]);
        if (more) xuk = rd_a(bk, 2);
        group(5 * ks + 4);
        sched_fence();
      }
    };
    // Keys past N (ragged end) or past the row (causal) of key tile t get
    // P = 0 through S = -inf.
    auto mask_tile = [&](auto Pc, int t) {
      constexpr int P = decltype(Pc)::value;
      const int key0 = (kt0 + t) * TS;
      if ((key0 + TS > N) || (CAUSAL && key0 + TS - 1 > r0 + wi * 32)) {
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          const int key = key0 + acc_pos(idx, hh);
          S[P][idx] = (key < N && (!CAUSAL || key <= row)) ? S[P][idx] : -INFINITY;
        }
      }
    };
    // Elementwise work on element idx of set P.  Each pair of elements is
    // packed to bf16 and written to the operand buffer at once (one word per
    // chain: P, P F, P P~, dS).
    auto element = [&](auto Pc, int idx, float (&pair)[4], lds_p obuf) {
      constexpr int P = decltype(Pc)::value;
      const float p = __builtin_amdgcn_exp2f(fmaf(S[P][idx], a.c1, nl2));
      const float Fv = RHO1 ? F[P][idx] : F[P][idx] * a.rho;
      const float dpd = DP[P][idx];
      const float t0 = fmaf(Fv, dpd, C[P][idx]);
      const float pf = p * Fv, pt = p * t0, ds = p * dpd;
      add_here(alpha_p, pf);
      add_here(eo_p, pt);
      if ((idx & 1) == 0) {
        pair[0] = p;
        pair[1] = pf;
        pair[2] = pt;
        pair[3] = ds;
      } else {
        const int w = idx >> 1;  // word w of each chain: k-half w / 4, word w % 4
        const uint32_t wp = pack_bf16(pair[0], p), wpf = pack_bf16(pair[1], pf), wpt = pack_bf16(pair[2], pt),
                       wds = pack_bf16(pair[3], ds);
        typedef __attribute__((address_space(3))) u32x4* wptr;
        const u32x4 words = {wp, wpf, wpt, wds};
        *reinterpret_cast<wptr>(obuf + op_off(w)) = words;
      }
    };
    // Slot sl in 1 .. nt - 1: scores of tile sl into set P, elementwise of
    // tile sl - 1 from the other set.
    auto steady = [&](auto Pc, int sl) {
      constexpr int P = decltype(Pc)::value;
      constexpr std::integral_constant<int, 1 - P> Qc{};
      if (sl + 2 < nt) dma.copy((kt0 + sl + 2) * TS, N, stages + stage_off(sl + 2));
      vfence4(S[1 - P], F[1 - P], DP[1 - P], C[1 - P]);
      mask_tile(Qc, sl - 1);
      float pair[4];
      const lds_p obuf = ((sl - 1) & 1) ? ob1 : ob0;
      scores(Pc, sl, [&](int g) {
        if (g < 16) element(Qc, g, pair, obuf);
      });
    };
    // Slot nt: elementwise of the last tile only.
    auto last = [&](auto Qc) {
      constexpr int Pq = decltype(Qc)::value;
      vfence4(S[Pq], F[Pq], DP[Pq], C[Pq]);
      mask_tile(Qc, nt - 1);
      float pair[4];
      const lds_p obuf = ((nt - 1) & 1) ? ob1 : ob0;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) element(Qc, idx, pair, obuf);
    };

    // Slot 0: scores of tile 0.
    if (2 < nt) dma.copy((kt0 + 2) * TS, N, stages + 2 * STAGE);
    scores(std::integral_constant<int, 0>{}, 0, [](int) {});
    end_slot(0);
    int sl = 1;
    for (; sl + 1 < nt; sl += 2) {
      steady(std::integral_constant<int, 1>{}, sl);
      end_slot(sl);
      steady(std::integral_constant<int, 0>{}, sl + 1);
      end_slot(sl + 1);
    }
    if (sl < nt) {
      steady(std::integral_constant<int, 1>{}, sl);
      end_slot(sl);
    }
    if ((nt - 1) & 1) {
      last(std::integral_constant<int, 1>{});
    } else {
      last(std::integral_constant<int, 0>{});
    }
    end_slot(nt);
    end_slot(nt + 1);  // the consumer's last tile

    const float alpha = half_sum(alpha_p);
    const float eo = half_sum(eo_p);
    if constexpr (KSPLIT) {
      // Key split: this key range's row sums; the sum kernel does the rest.
      if (hh == 0 && row < N) {
        kpart_rowsum(a, kk, 0, bh)[row] = alpha;
        kpart_rowsum(a, kk, 1, bh)[row] = eo;
        if (kk == 0) a.D[rv + row] = Di;
      }
    } else if (hh == 0) {
      rowx[wi][l] = alpha;
      if (row < N) {
        a.alpha[rv + row] = alpha;
        a.E[rv + row] = eo - alpha * Di;
        a.D[rv + row] = Di;
      }
      // Chain inits of the column pass (see bob_pass2_dma_kernel).
      float* ps = a.ps + ((int64_t)bh * nblk + row / kPsRows) * 4 * kPsRows + row % kPsRows;
      const bool ok = row < N;
      const float irho = 1.0f / a.rho;
      ps[0] = ok ? -Li * irho : -INFINITY;
      ps[kPsRows] = ok ? -Di : 0.0f;
      ps[2 * kPsRows] = ok ? -alpha * irho : 0.0f;
      ps[3 * kPsRows] = ok ? -eo : 0.0f;
    }
    __syncthreads();
  } else {
    // ------------------------------------------------------------ consumer
    f32x16 ag[NDB], aom[NDB], ar[NDB], abk[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) ag[db] = aom[db] = ar[db] = abk[db] = zero16();
    const lds_cp ob0 = (lds_cp)ops[0] + wi * OPB + 16 * l;
    const lds_cp ob1 = (lds_cp)ops[1] + wi * OPB + 16 * l;
    rd.init();
    float eob_c = 0.0f;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int sl = 0; sl < nt + 2; ++sl) {
      if (sl + 2 < nt) dma.copy((kt0 + sl + 2) * TS, N, stages + stage_off(sl + 2));
      if (sl >= 2) {
        const int kt = sl - 2;
        const uint32_t rel = stage_off(kt);
        lds_cp trb[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) trb[db][kh] = stage_ptr(rel, rd.tr[db][kh]);
        // A operand of tensor t (0 K, 1 V, 2 U_K, 3 U_V): d-columns db*32..,
        // keys 16 s2 ..
        auto tr = [&](int t, int db, int s2) {
          const int off = t * W::BYTES + s2 * 16 * D * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(trb[db][0] + off));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(trb[db][1] + off));
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          return __builtin_bit_cast(bf16x8, v);
        };
        const lds_cp o = (kt & 1) ? ob1 : ob0;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          // B operand of chain k: words 4 s2 .. 4 s2 + 3 (keys 16 s2 + 8 hh ..),
          // word k of the groups 4 s2 + j.
          typedef const __attribute__((address_space(3))) u32x4* rp;
          u32x4 grp[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) grp[j] = *reinterpret_cast<rp>(o + op_off(4 * s2 + j));
          // E° from the bf16-rounded products P t0 that the matrix core
          // accumulates into Omega: gQ = tau (Omega - alpha R' - E° B) uses
          // it, so the rounded operands cancel the way the exact ones do
          // (Sum_j (P t0 - E° P) = 0; on a row whose P sits on one key those
          // terms cancel exactly).  E and the column pass keep the unrounded
          // E°.  This lane holds 16 of the row's keys per tile; the other
          // half of the wave holds the rest.
#pragma unroll
          for (int j = 0; j < 4; ++j)
            eob_c += __builtin_bit_cast(float, grp[j][2] << 16) + __builtin_bit_cast(float, grp[j][2] & 0xffff0000u);
          auto opnd = [&](int k) {
            const u32x4 v = {grp[0][k], grp[1][k], grp[2][k], grp[3][k]};
            return __builtin_bit_cast(bf16x8, v);
          };
          const bf16x8 bp = opnd(0), bpf = opnd(1), bpt = opnd(2), bds = opnd(3);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 xuv = tr(3, db, s2);
            const bf16x8 xv = tr(1, db, s2);
            const bf16x8 xk = tr(0, db, s2);
            const bf16x8 xuk = tr(2, db, s2);
            mfma_vv<KSPLIT>(ag[db], xuv, bp);
            mfma_vv<KSPLIT>(ag[db], xv, bpf);
            mfma_vv<KSPLIT>(aom[db], xk, bpt);
            mfma_vv<KSPLIT>(aom[db], xuk, bds);
            mfma_vv<KSPLIT>(ar[db], xk, bds);
            mfma_vv<KSPLIT>(abk[db], xk, bp);
          }
        }
      }
      end_slot(sl);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) vfence4(ag[db], aom[db], ar[db], abk[db]);
    __syncthreads();  // alpha and E° of the producers are in LDS
    const float eob = half_sum(eob_c);
    if constexpr (KSPLIT) {
      // Key split: this key range's accumulators and E°_b, raw.
      if (hh == 0 && row < N) kpart_rowsum(a, kk, 2, bh)[row] = eob;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        store_out(kpart_acc<D>(a, kk, 0, bh), D, row, N, db, [&](int idx) { return ag[db][idx]; });
        store_out(kpart_acc<D>(a, kk, 1, bh), D, row, N, db, [&](int idx) { return aom[db][idx]; });
        store_out(kpart_acc<D>(a, kk, 2, bh), D, row, N, db, [&](int idx) { return ar[db][idx]; });
        store_out(kpart_acc<D>(a, kk, 3, bh), D, row, N, db, [&](int idx) { return abk[db][idx]; });
      }
      return;
    }
    const float alpha = rowx[wi][l & 31];
    const HeadPtr<float> o = head_of<float>(a.o, bb, hd);
    float* gq = head_out(a.r0, bb, hd);
    float* gdo = head_out(a.r3, bb, hd);
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
                [&](int idx) { return a.tau * (aom[db][idx] - alpha * ar[db][idx] - eob * abk[db][idx]); });
    }
  }
}

}  // namespace fa
