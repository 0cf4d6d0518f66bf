// fa_lds.h -- LDS staging of streamed bf16 tiles for the gfx950 BoB passes.
//
//   * Tiles are copied HBM -> LDS with global_load_lds_dwordx4: every lane
//     moves one 16-byte granule and the wave's 64 granules land contiguously
//     at the LDS address the instruction names, so no VGPR holds tile data.
//   * A tile is TS rows of D bf16 (G = D/8 granules per row) with no padding;
//     granule q of row j sits at position q ^ swz<G>(j) of the row, which
//     keeps both read patterns below free of LDS bank conflicts.  The swizzle
//     is applied on the HBM side: the lane that fills LDS position p fetches
//     the granule that belongs there.
//   * Bank model (measured on gfx950 with SQ_LDS_BANK_CONFLICT): 64 banks of
//     4 bytes; ds_read_b128 serves 16 lanes per cycle, ds_read_b64 32 lanes,
//     so each group must cover 256 distinct bytes modulo 256.
//   * Products that contract over d read their A operand (32 streamed rows x
//     8 consecutive d per lane) with ds_read_b128.
//   * Products that contract over the streamed index need the transposed
//     operand (32 d-columns x 8 consecutive streamed rows per lane).  It is
//     read from the same row-major tile with two ds_read_b64_tr_b16: within
//     each group of 16 lanes, lane r names an 8-byte piece of row r of a 16 x 4
//     block and receives element (r % 4) of the pieces named by lanes
//     4k + r / 4, k = 0..3.
#pragma once

#include "fa_tile.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Position of granule q inside row j is q ^ swz<G>(j).
//   * Row-major reads: one 16-lane group reads the same granule of 16
//     consecutive rows.  G = 8 (d = 64, two rows per 256 bytes): the eight
//     even rows and the eight odd rows of a 16-row block need distinct swz;
//     G = 16 (one row per 256 bytes): all sixteen rows do.
//   * Transposing reads: one 32-lane group reads granules 4c .. 4c+3 of four
//     consecutive rows 4m .. 4m+3, so those rows must map the aligned block of
//     four granules onto disjoint blocks: for G = 8, rows 4m and 4m+2 (and
//     4m+1, 4m+3) differ in bit 2 of swz; for G = 16 the four rows differ in
//     bits 2-3.
template <int G>
__host__ __device__ constexpr int swz(int j) {
  if constexpr (G == 8) {
    return ((j & 2) << 1) | ((j >> 2) & 3);
  } else {
    return ((j & 3) << 2) | ((j >> 2) & 3);
  }
}

template <int D, int TS>
struct SwTile {
  static constexpr int G = D / 8;             // granules per row
  static constexpr int BYTES = TS * D * 2;    // bytes per tensor tile
  static constexpr int BLOCKS = TS * G / 64;  // wave-wide DMA copies per tensor tile
  static_assert((TS * G) % 64 == 0, "a tile must be a whole number of wave copies");
  static_assert(64 % G == 0, "a wave copy must cover whole rows");
  static constexpr int ROWS_PER_BLOCK = 64 / G;

  // Byte offset of (row j, granule q).
  static_assert(G == 8 || G == 16, "d = 64 or 128");
  __host__ __device__ static constexpr int off(int j, int q) { return (j * G + (q ^ swz<G>(j))) * 16; }
};

// One wave-wide HBM -> LDS copy: lane i moves 16 bytes to lds_base + 16 i.
// Issued as inline assembly so that the compiler does not treat the
// in-flight copy as a pending write to every LDS location (it would otherwise
// wait for the copy before the first LDS read of the current tile); the
// kernels await completion explicitly with dma_wait() before the barrier that
// publishes a tile.  M0 holds the LDS base for the instruction.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Source = uniform 64-bit base + per-lane 32-bit byte offset.
__device__ inline void dma16_so(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(off), "s"(base)
               : "memory", "m0");
}
// Source = per-lane 64-bit address.
__device__ inline void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until every copy this wave issued has landed in LDS.
__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// HBM -> LDS copies of rows [row0, row0 + TS) of NT streamed tensors of one
// head into NT consecutive tiles.  Wave w copies blocks w, w + NW, ... of
// every tensor (a block = 64 granules = ROWS_PER_BLOCK rows).  Rows at or
// past N are read from row N - 1 instead (in bounds; the caller masks their
// scores to P = 0).
template <int D, int TS, int NT>
struct Dma {
  typedef SwTile<D, TS> W;
  static constexpr int NW = kThreads / 64;
  static constexpr int RPB = W::ROWS_PER_BLOCK;
  static constexpr int PER_WAVE = W::BLOCKS / NW;
  static_assert(W::BLOCKS % NW == 0, "blocks per tensor must split evenly over the waves");
  // Rows of one wave's blocks are 16 apart, and the swizzle depends on the
  // row modulo 16 only, so it is fixed per lane and wave.
  static_assert((NW * RPB) % 16 == 0, "block stride must keep the row swizzle");

  const char* base[NT];  // head base pointers (uniform)
  int64_t rs[NT];        // row strides in bytes (uniform)
  int64_t hs[NT];        // head strides in bytes (uniform; copy() may step over heads)
  uint32_t off[NT];      // per-lane byte offset inside a block: jl * rs + 16 q
  int jl, wave;

  // src: the tensors' first heads; hstride: their head strides in elements
  // (needed only by copies with g != 0).
  __device__ inline void init(const HeadPtr<bf16>* src, const int64_t* hstride = nullptr) {
    const int lane = lane_id();
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    jl = lane / W::G;
    const int q = (lane % W::G) ^ swz<W::G>(wave * RPB + jl);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      base[t] = reinterpret_cast<const char*>(src[t].p);
      rs[t] = src[t].sn * 2;
      hs[t] = hstride ? hstride[t] * 2 : 0;
      off[t] = (uint32_t)(jl * (int)rs[t] + 16 * q);
    }
  }

  // Rows row0 .. row0 + TS - 1 of head g (counted from the heads passed to
  // init) of every tensor.
  __device__ inline void copy(int row0, int N, const char* dst, int g = 0) const {
    const uint32_t lbase = lds_addr(dst);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const char* hb = base[t] + g * hs[t];
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int b = i * NW + wave;
        const int r0 = row0 + b * RPB;
        const uint32_t lds = lbase + t * W::BYTES + b * 1024;
        if (r0 + RPB <= N) {
          dma16_so(hb + r0 * rs[t], off[t], lds);
        } else {
          const int row = min(r0 + jl, N - 1);
          dma16(hb + row * rs[t] + (off[t] - jl * (int)rs[t]), lds);
        }
      }
    }
  }
};

// Per-lane byte offsets (inside one tile) of the two operand read patterns.
template <int D, int TS>
struct Reader {
  typedef SwTile<D, TS> W;
  static constexpr int NKS = D / 16;  // k-steps of a contraction over d
  static constexpr int NDB = D / 32;  // 32-column blocks of d
  int row[NKS];                       // ds_read_b128 for k-step ks, sub-tile 0
  int tr[NDB][2];                     // ds_read_b64_tr_b16 for d-block db, half koff/4

  __device__ inline void init() {
    const int l = lane_id();
    const int m = l & 31, h = l >> 5;
    const int j = sig(m);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) row[ks] = W::off(j, 2 * ks + h);
    const int g = l >> 4, r = l & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int jj = 8 * (g >> 1) + 4 * kh + (r >> 2);
        const int q = 4 * db + 2 * (g & 1) + ((r & 3) >> 1);
        tr[db][kh] = W::off(jj, q) + 8 * (r & 1);
      }
  }
};

// A operand of a contraction over d: streamed rows sub*32 + sig(m), k-step ks.
template <int D, int TS>
__device__ inline bf16x8 rd_row(const char* tile, const Reader<D, TS>& rd, int sub, int ks) {
  return *reinterpret_cast<const bf16x8*>(tile + rd.row[ks] + sub * 32 * D * 2);
}

// A operand of a contraction over the streamed rows: d-columns db*32 + m,
// streamed rows sub*32 + 16*s + 8*h + e, e = 0..7.
template <int D, int TS>
__device__ inline bf16x8 rd_tr(const char* tile, const Reader<D, TS>& rd, int sub, int db, int s) {
  const int base = (sub * 32 + 16 * s) * D * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + rd.tr[db][0] + base));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + rd.tr[db][1] + base));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// D_i = rowsum(dO * O)_i ([FA2-recompute]) of this lane's resident row, from
// its resident bf16 dO operands (k-step ks holds d-columns 16 ks + 8 hh ..
// + 7) and the matching fp32 O values; the two halves of the wave hold the
// two halves of the row.
template <int D>
__device__ inline float resident_rowdot(const bf16x8 (&df)[D / 16], const HeadPtr<float>& o, int row, int N) {
  const int hh = lane_id() >> 5;
  float acc = 0.0f;
  if (row < N) {
    const float* orow = o.p + (int64_t)row * o.sn + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(orow + 16 * ks);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(orow + 16 * ks + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf((float)df[ks][e], x0[e], acc);
        acc = fmaf((float)df[ks][e + 4], x1[e], acc);
      }
    }
  }
  return half_sum(acc);
}

}  // namespace fa
