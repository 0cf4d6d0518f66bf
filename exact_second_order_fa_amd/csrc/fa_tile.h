// fa_tile.h -- wave-level tile machinery shared by the gfx950 attention kernels.
//
// Geometry (CDNA4, wave64, v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32):
//
//   * Every kernel keeps one block of "resident" rows per workgroup (4 waves x
//     32 rows) and streams tiles of the other side through LDS.  A wave's
//     resident rows are the N index of its MFMAs; the streamed rows are M.
//   * Accumulator element idx (0..15) of lane l sits at column n = l % 32 and
//     row m = 8*(idx/4) + 4*(l/32) + idx%4.
//   * Scores are produced with the streamed index on M.  Reading the A rows of
//     that product through the permutation sig() (swap of bits 2 and 3) makes
//     the eight accumulator values a lane feeds into each k-step of the NEXT
//     product (a contraction over the streamed index) land on eight
//     consecutive streamed positions: 16*s + 8*(l/32) + e.  So score tiles are
//     re-used as MFMA B operands straight from registers (after rounding to
//     the input type), and the matching A operand is one 16-byte LDS read
//     from the transposed copy of the streamed tile.
//   * Each streamed tensor is staged twice in LDS: row-major [row][d] (A
//     operand of products that contract over d) and transposed [d][row] (A
//     operand of products that contract over the streamed rows).  Both copies
//     are written from one 16-byte-per-row register block per thread; the
//     transposed copy comes from an in-register transpose of that block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kResRows = 32 * kWaves;  // resident rows per workgroup
constexpr int kPsRows = 128;           // row granule of the staged column-pass scalars
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  static constexpr int KS = 16;  // contraction length of one MFMA
  static constexpr int KL = 8;   // contraction elements held per lane
  static constexpr int VEC = 8;  // elements per 16-byte vector
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // Scale eight elements by an exact power of two (re-rounding is exact).
  __device__ static inline frag scale(frag x, float s) {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)((float)x[e] * s);
    return r;
  }
  __device__ static inline frag zero() {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)0.0f;
    return r;
  }
  __device__ static inline float to_f32(bf16 x) { return (float)x; }
};

template <>
struct Elem<float> {
  static constexpr int KS = 2;
  static constexpr int KL = 1;
  static constexpr int VEC = 4;
  typedef float frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const float* p) { return *p; }
  __device__ static inline frag scale(frag x, float s) { return x * s; }
  __device__ static inline frag zero() { return 0.0f; }
  __device__ static inline float to_f32(float x) { return x; }
};

__device__ inline int lane_id() { return threadIdx.x & 63; }

// f(integral_constant<int, i>) for i = B .. E - 1, in order: the index is a
// compile-time constant inside f, whatever the unroller decides.
template <int B, int... I, typename F>
__device__ inline void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, B + I>{}), ...);
}
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (E > B) static_for_impl<B>(std::make_integer_sequence<int, E - B>{}, f);
}

// Swap bits 2 and 3 (an involution on 0..31).
__host__ __device__ constexpr int sig(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Streamed position (0..31 inside a 32-row sub-tile) of accumulator element
// idx held by a lane in half hh (= lane / 32).
__host__ __device__ constexpr int acc_pos(int idx, int hh) { return sig(8 * (idx >> 2) + 4 * hh + (idx & 3)); }

// Row (0..31) of accumulator element idx: 8*(idx/4) + 4*hh + idx%4.
__host__ __device__ constexpr int acc_row(int idx, int hh) { return 8 * (idx >> 2) + 4 * hh + (idx & 3); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

// Workgroup id -> work item, grouping consecutive work items (same head) on
// one XCD: workgroups are dispatched round-robin over the 8 XCDs.
__device__ inline int xcd_remap(int g, int total) {
  if (total % 8) return g;
  return (g % 8) * (total / 8) + g / 8;
}

// Causal work items (after xcd_remap): block k of a head, k = 0 the longest,
// does work that falls with k.  Head-major order, each head's blocks longest
// first, keeps the workgroups an XCD runs at once on few heads, whose
// streamed tiles then hit its L2, but puts the long blocks of its last heads
// near the end.  With at most 32 blocks per head (N <= 4096: every head's
// tiles fit the L2 together, and each compute unit runs few workgroups, so
// the tail weighs most) and whole heads per XCD (its total / 8 items a
// multiple of nblk), the XCD runs its heads block-major instead -- every
// head's longest block, then every head's second -- so its last items are
// the shortest of all its heads.
__device__ inline void longest_first(int w, int total, int nblk, int& head, int& k) {
  const int per_xcd = total / 8;
  if (nblk <= 32 && total % 8 == 0 && per_xcd % nblk == 0) {
    const int hx = per_xcd / nblk, x = w / per_xcd, i = w - x * per_xcd;
    head = x * hx + i % hx;
    k = i / hx;
  } else {
    head = w / nblk;
    k = w % nblk;
  }
}

// ---------------------------------------------------------------------------
// LDS layout of one staged tensor: row copy [TS][D + VEC], transposed copy
// [D][TS + VEC] (the pad keeps 16-byte alignment and spreads banks).
template <typename T, int D, int TS>
struct Stage {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int LDR = D + VEC;
  static constexpr int LDT = TS + VEC;
  static constexpr int ROW_ELEMS = TS * LDR;
  static constexpr int TR_ELEMS = D * LDT;
  static constexpr int ELEMS = ROW_ELEMS + TR_ELEMS;
  static constexpr int BYTES = ELEMS * (int)sizeof(T);
  static constexpr int BLK_PER_TENSOR = (TS / VEC) * (D / VEC);
};

// Descriptor of one streamed tensor for one head: base pointer (already
// offset to the head) and row stride in elements.
template <typename T>
struct HeadPtr {
  const T* p;
  int64_t sn;
};

// A register block: VEC rows x 16 bytes.
struct RegBlock {
  u32x4 r[8];
};

// Load this thread's blocks of NT streamed tensors, rows [row0, row0+TS).
// Rows >= N read as zero.
template <typename T, int D, int TS, int NT>
struct Stager {
  typedef Stage<T, D, TS> S;
  static constexpr int VEC = S::VEC;
  static constexpr int TOTAL = NT * S::BLK_PER_TENSOR;
  static constexpr int NB = (TOTAL + kThreads - 1) / kThreads;

  RegBlock blk[NB];

  __device__ inline void load(const HeadPtr<T>* src, int row0, int N) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int bi = threadIdx.x + b * kThreads;
      if (TOTAL % kThreads == 0 || bi < TOTAL) {
        const int t = bi / S::BLK_PER_TENSOR;
        const int w = bi % S::BLK_PER_TENSOR;
        const int rb = w / (D / VEC), cb = w % (D / VEC);
        const T* base = src[t].p + (int64_t)cb * VEC;
#pragma unroll
        for (int rr = 0; rr < VEC; ++rr) {
          const int row = row0 + rb * VEC + rr;
          if (row < N) {
            blk[b].r[rr] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * src[t].sn);
          } else {
            blk[b].r[rr] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
  }

  // lds points at NT consecutive Stage<T,D,TS> regions.
  __device__ inline void store(T* lds) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int bi = threadIdx.x + b * kThreads;
      if (TOTAL % kThreads == 0 || bi < TOTAL) {
        const int t = bi / S::BLK_PER_TENSOR;
        const int w = bi % S::BLK_PER_TENSOR;
        const int rb = w / (D / VEC), cb = w % (D / VEC);
        T* rowc = lds + t * S::ELEMS;
        T* trc = rowc + S::ROW_ELEMS;
#pragma unroll
        for (int rr = 0; rr < VEC; ++rr)
          *reinterpret_cast<u32x4*>(rowc + (rb * VEC + rr) * S::LDR + cb * VEC) = blk[b].r[rr];
        // transposed copy: column cb*VEC+cc, rows rb*VEC .. rb*VEC+VEC-1
#pragma unroll
        for (int cc = 0; cc < VEC; ++cc) {
          u32x4 o;
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
              const uint32_t x = blk[b].r[2 * wd][cc >> 1];
              const uint32_t y = blk[b].r[2 * wd + 1][cc >> 1];
              o[wd] = (cc & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
            }
          } else {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) o[wd] = blk[b].r[wd][cc];
          }
          *reinterpret_cast<u32x4*>(trc + (cb * VEC + cc) * S::LDT + rb * VEC) = o;
        }
      }
    }
  }
};

// Resident B operand: rows row0 + lane%32 of a head tensor, contraction over
// the D columns, scaled by the exact power of two `s`.
template <typename T, int D>
__device__ inline void load_resident(typename Elem<T>::frag (&f)[D / Elem<T>::KS], const T* p,
                                     int64_t sn, int row, int N, float s) {
  typedef Elem<T> E;
  const int hh = lane_id() >> 5;
  if (row < N) {
    const T* r = p + (int64_t)row * sn + hh * E::KL;
#pragma unroll
    for (int ks = 0; ks < D / E::KS; ++ks) {
      typename E::frag x = E::load(r + ks * E::KS);
      f[ks] = (s == 1.0f) ? x : E::scale(x, s);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < D / E::KS; ++ks) f[ks] = E::zero();
  }
}

// acc[m][n] += sum_c A[sub*32 + sig(m)][c] * Bres[n][c]: A from the row copy,
// B resident.  M = streamed rows of sub-tile `sub`, N = resident rows.
template <typename T, int D, int TS>
__device__ inline f32x16 mm_row(const T* rowc, int sub, const typename Elem<T>::frag (&b)[D / Elem<T>::KS],
                                f32x16 acc) {
  typedef Elem<T> E;
  typedef Stage<T, D, TS> S;
  const int l = lane_id();
  const T* a = rowc + (sub * 32 + sig(l & 31)) * S::LDR + (l >> 5) * E::KL;
#pragma unroll
  for (int ks = 0; ks < D / E::KS; ++ks) acc = E::mma(E::load(a + ks * E::KS), b[ks], acc);
  return acc;
}

// Column (within the transposed copy) of the k-step s operand of a lane in
// half hh, for streamed sub-tile `sub`.
template <typename T>
__device__ inline int tr_col(int sub, int s, int hh) {
  if constexpr (sizeof(T) == 2) {
    return sub * 32 + 16 * s + 8 * hh;
  } else {
    return sub * 32 + 16 * (s >> 3) + 8 * hh + (s & 7);
  }
}

// Number of k-steps for a contraction over one 32-row streamed sub-tile.
template <typename T>
constexpr int ksteps32() { return 32 / Elem<T>::KS; }

// A operand from the transposed copy: rows d = db*32 + lane%32, k-step s.
template <typename T, int D, int TS>
__device__ inline typename Elem<T>::frag tr_frag(const T* trc, int db, int sub, int s) {
  typedef Stage<T, D, TS> S;
  const int l = lane_id();
  return Elem<T>::load(trc + (db * 32 + (l & 31)) * S::LDT + tr_col<T>(sub, s, l >> 5));
}

// B operand frags of a contraction over the streamed sub-tile, built from the
// 16 per-lane values of a score-shaped accumulator (rounded to T).
template <typename T>
struct Chain {
  typename Elem<T>::frag f[ksteps32<T>()];
  __device__ inline void set(const float (&v)[16]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[s][e] = (bf16)v[8 * s + e];
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) f[s] = v[s];
    }
  }
};

// Cross-half (lane ^ 32) sum, for row sums whose 32 streamed positions are
// split over the two halves of the wave.
__device__ inline float half_sum(float x) { return x + __shfl_xor(x, 32); }
__device__ inline float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// Store the 16 values of an output accumulator (M = d rows db*32.., N =
// resident row `row`) as fp32 with an element-wise transform.
template <typename Fn>
__device__ inline void store_out(float* out, int64_t sn, int row, int N, int db, Fn fn) {
  if (row >= N) return;
  const int hh = lane_id() >> 5;
  float* r = out + (int64_t)row * sn + db * 32 + 4 * hh;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x4 v;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) v[rr] = fn(4 * b + rr);
    *reinterpret_cast<f32x4*>(r + 8 * b) = v;
  }
}

}  // namespace fa
