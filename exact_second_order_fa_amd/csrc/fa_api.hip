// fa_api.hip -- the C ABI declared in include/fa.h: host-side validation and
// kernel launches.  No allocation and no synchronisation; the only state is
// the per-device address of fa_bob_noalloc's static scratch array.
#include <math.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_kernels.hip"
#include "fa_bob.hip"
#include "fa_bob_ws.hip"
#include "fa_fwd_bwd.hip"

namespace {

using fa::Args;
using fa::bf16;
using fa::TDesc;

constexpr int kVersion = 1 * 10000 + 4 * 100 + 0;  // 1.1: fa_problem.H_kv; 1.2: dropout, seed;
                                                   // 1.3: fa_bob_noalloc; 1.4: split partial sums in
                                                   // fa_bob's workspace, 64 MiB no-alloc array

struct Ctx {
  int64_t B, H, N, d;
  int64_t Hkv, G;  // key/value heads, query heads per key/value head
  size_t esize;  // input element size
  bool bf;
  bool causal;
  float tau, pow2, rho;
  bool drop;            // dropout with a threshold > 0
  uint32_t drop_thr;    // round(256 p)
  float drop_scale;     // 256 / (256 - drop_thr)
  uint64_t seed;
};

fa_status check_problem(const fa_problem* p, Ctx* c) {
  if (!p) return FA_ERR_NULL;
  if (p->B < 1 || p->H < 1 || p->N < 1) return FA_ERR_SHAPE;
  const int64_t hkv = p->H_kv == 0 ? p->H : p->H_kv;
  if (hkv < 1 || hkv > p->H || p->H % hkv) return FA_ERR_SHAPE;
  if (p->in_dtype != FA_BF16 && p->in_dtype != FA_FP32) return FA_ERR_DTYPE;
  if (p->d != 64 && p->d != 128) return FA_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return FA_ERR_UNSUPPORTED;
  // fp32 inputs are built for d = 64 only (register budget of the fp32 MFMA path).
  if (p->in_dtype == FA_FP32 && p->d != 64) return FA_ERR_UNSUPPORTED;
  // Row vectors are indexed with 64-bit offsets, sequence positions and grid
  // sizes with 32-bit ints.
  if (p->N > (int64_t(1) << 30)) return FA_ERR_SHAPE;
  const int64_t bh = p->B * p->H;
  if (p->B > (int64_t(1) << 30) || p->H > (int64_t(1) << 30) || bh > (int64_t(1) << 30)) return FA_ERR_SHAPE;
  const int64_t nblk = (p->N + fa::kResRows - 1) / fa::kResRows;
  if (bh * nblk > (int64_t(1) << 31) - 1) return FA_ERR_SHAPE;
  if (bh * p->N > (int64_t(1) << 40)) return FA_ERR_SHAPE;
  float tau = p->scale;
  if (!(tau > 0.0f)) {
    if (tau != tau) return FA_ERR_UNSUPPORTED;  // NaN
    tau = 1.0f / sqrtf((float)p->d);
  }
  if (!isfinite(tau)) return FA_ERR_UNSUPPORTED;
  // Dropout rate p in [0, 1); the kernels keep an element with probability
  // 1 - t / 256, t = round(256 p), which must stay below 256.
  if (!(p->dropout >= 0.0f && p->dropout < 1.0f)) return FA_ERR_UNSUPPORTED;
  const int thr = (int)floorf(p->dropout * 256.0f + 0.5f);
  if (thr > 255) return FA_ERR_UNSUPPORTED;
  c->drop = thr > 0;
  c->drop_thr = (uint32_t)thr;
  c->drop_scale = 256.0f / (float)(256 - thr);
  c->seed = p->seed;
  int ex = 0;
  const float m = frexpf(tau, &ex);  // tau = m * 2^ex, m in [0.5, 1)
  c->B = p->B;
  c->H = p->H;
  c->Hkv = hkv;
  c->G = p->H / hkv;
  c->N = p->N;
  c->d = p->d;
  c->bf = p->in_dtype == FA_BF16;
  c->causal = p->causal != 0;
  c->esize = c->bf ? 2 : 4;
  c->tau = tau;
  c->pow2 = ldexpf(1.0f, ex - 1);
  c->rho = 2.0f * m;
  if (!(c->pow2 > 0.0f) || !isfinite(c->pow2)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status check_tensor(const Ctx& c, const fa_tensor& t, size_t esize) {
  if (!t.ptr) return FA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(t.ptr) % 16) return FA_ERR_STRIDE;
  const int64_t vec = 16 / (int64_t)esize;
  if (t.stride_n < c.d || t.stride_h < 0 || t.stride_b < 0) return FA_ERR_STRIDE;
  if (t.stride_n % vec || t.stride_h % vec || t.stride_b % vec) return FA_ERR_STRIDE;
  // Tile copies address a few rows with 32-bit byte offsets.
  if (t.stride_n > (int64_t(1) << 26)) return FA_ERR_STRIDE;
  return FA_OK;
}

fa_status check_vec(const void* p) {
  if (!p) return FA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(p) % 4) return FA_ERR_STRIDE;
  return FA_OK;
}

TDesc desc(const fa_tensor& t) {
  TDesc r;
  r.p = t.ptr;
  r.sb = t.stride_b;
  r.sh = t.stride_h;
  r.sn = t.stride_n;
  return r;
}

Args base_args(const Ctx& c) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.B = (int)c.B;
  a.H = (int)c.H;
  a.Hk = (int)c.Hkv;
  a.G = (int)c.G;
  a.gs = (int)c.G;
  a.nsplit = 1;
  a.rs = 1;
  a.ks = 1;
  a.part = nullptr;
  a.kpart = nullptr;
  a.N = (int)c.N;
  a.tau = c.tau;
  a.pow2 = c.pow2;
  a.rho = c.rho;
  a.c1 = fa::kLog2e * c.rho;
  a.seed = c.seed;
  a.drop_thr = c.drop_thr;
  a.drop_scale = c.drop_scale;
  return a;
}

unsigned grid_rows(const Ctx& c) {
  return (unsigned)(c.B * c.H * ((c.N + fa::kResRows - 1) / fa::kResRows));
}

// Column-side kernels: one workgroup per (batch, key/value head, key block);
// each streams the rows of the group's G query heads.
unsigned grid_cols(const Ctx& c) {
  return (unsigned)(c.B * c.Hkv * ((c.N + fa::kResRows - 1) / fa::kResRows));
}

// Rows per head padded to whole 128-row blocks (the staged chain-init layout).
int64_t padded_rows(const Ctx& c) { return (c.N + fa::kPsRows - 1) / fa::kPsRows * fa::kPsRows; }

// Group split of the bf16 column kernels.  A column workgroup streams the
// rows of its key/value head's G query heads, so grouped-query attention
// with few key blocks launches few workgroups (multi-query at N = 2048: 16
// for 256 CUs).  Then each key block's G query heads are split over nsplit
// workgroups (the smallest divisor of G that gives one per CU, else G), each
// leaving its sums in the workspace, and a sum kernel adds the nsplit
// partial results in a fixed order and writes each output block once.
int group_split(const Ctx& c) {
  if (!c.bf || c.G == 1) return 1;
  const int64_t cols = c.B * c.Hkv * ((c.N + fa::kResRows - 1) / fa::kResRows);
  if (cols >= 256) return 1;
  for (int s = 2; s < c.G; ++s)
    if (c.G % s == 0 && cols * s >= 256) return s;
  return (int)c.G;
}

// Row split of the BoB column pass, on top of the group split g: still fewer
// than 256 workgroups (few key blocks and few query heads per key/value head,
// e.g. multi-query attention at N = 2048: 16 x 8) and not causal, each
// query head's rows are cut into r ranges of at least two 128-row blocks
// (r the smallest power of two that reaches 256), whose key-side sums are
// further partials of the block's.
int row_split(const Ctx& c, int g) {
  if (!c.bf || c.causal) return 1;
  const int64_t nblk = (c.N + fa::kResRows - 1) / fa::kResRows;
  const int64_t cols = c.B * c.Hkv * nblk * g;
  int r = 1;
  while (cols * r < 256 && nblk / (2 * r) >= 2) r *= 2;
  return r;
}
int bob_nsplit(const Ctx& c) {
  const int g = group_split(c);
  return g * row_split(c, g);
}

// Key split of the bf16 two-pass row pass (no dropout, not causal): with
// fewer than 256 row workgroups (B * H * ceil(N / 128); multi-query at
// N = 2048: 128) each row block's keys are cut into k ranges of at least two
// 128-key blocks (k the smallest power of two reaching 256), whose raw sums a
// sum kernel adds and finishes (bob_ksplit_sum_kernel).
int key_split(const Ctx& c) {
  if (!c.bf || c.causal || c.drop) return 1;
  const int64_t nblk = (c.N + fa::kResRows - 1) / fa::kResRows;
  const int64_t rows = c.B * c.H * nblk;
  int k = 1;
  while (rows * k < 256 && nblk / (2 * k) >= 2) k *= 2;
  return k;
}
// Floats of the key-split partial sums: [k][3][B*H][N] row sums and
// [k][4][B*H][N][d] accumulators.
size_t ksplit_floats(const Ctx& c, int k) {
  return k > 1 ? (size_t)k * (size_t)(c.B * c.H * c.N) * (3 + 4 * (size_t)c.d) : 0;
}

// Floats of the partial key-side sums of a group split: [2][nsplit][B * H_kv][N][d].
size_t split_floats(const Ctx& c, int nsplit) {
  return nsplit > 1 ? 2 * (size_t)nsplit * (size_t)(c.B * c.Hkv * c.N) * (size_t)c.d : 0;
}

// Workspace offsets in floats: fa_bob [D | alpha | E | chain inits | partial
// sums], fa_bwd [D | chain inits | partial sums]; the partial sums start on a
// 256-byte boundary.
size_t align64(size_t f) { return (f + 63) / 64 * 64; }
size_t bob_part_offset(const Ctx& c) {
  return align64(3 * (size_t)(c.B * c.H * c.N) + 4 * (size_t)(c.B * c.H) * (size_t)padded_rows(c));
}
size_t bob_kpart_offset(const Ctx& c) { return align64(bob_part_offset(c) + split_floats(c, bob_nsplit(c))); }
size_t bwd_part_offset(const Ctx& c) {
  return align64((size_t)(c.B * c.H * c.N) + 2 * (size_t)(c.B * c.H) * (size_t)padded_rows(c));
}

// Launch of the partial-sum kernel after a split column kernel.
template <int D>
void launch_group_sum(const Ctx& c, const fa::Args& a, hipStream_t st) {
  if (a.nsplit <= 1) return;
  const int64_t threads = 2 * (int64_t)(c.B * c.Hkv * c.N) * (D / 4);
  hipLaunchKernelGGL((fa::group_sum_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
}

// staged: the launch also covers each head's padding rows (fa_bwd's column
// chain inits).
unsigned grid_rowscalar(const Ctx& c, bool staged = false) {
  const int64_t rpb = 256 / (c.d / 8);
  return (unsigned)((c.B * c.H * (staged ? padded_rows(c) : c.N) + rpb - 1) / rpb);
}

#define FA_CHECK(x)                 \
  do {                              \
    const fa_status s_ = (x);       \
    if (s_ != FA_OK) return s_;     \
  } while (0)

fa_status launched() { return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP; }

template <typename T, int D>
void launch_rowscalar(const Ctx& c, const Args& a, hipStream_t st) {
  hipLaunchKernelGGL((fa::rowscalar_kernel<T, D>), dim3(grid_rowscalar(c)), dim3(256), 0, st, a);
}

// Streamed tile rows per LDS stage of the portable kernels (fp32 inputs).
template <typename T, int D>
struct Tiles {
  static_assert(sizeof(T) == 4, "bf16 inputs run the LDS-DMA kernels");
  static constexpr int TS = 32;
};

// Dropout: the LDS-DMA kernels with their DROP flag for bf16 inputs, the
// portable kernels (register-staged tiles, one wave per SIMD) for fp32.
template <typename T, int D, bool C>
void launch_fwd(const Ctx& c, const Args& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // Three waves per SIMD (64-key tiles at d = 64, 32-key tiles at d = 128
    // without dropout) on grids of at least two full rounds of three
    // workgroups per CU; below that the CUs of a last partial round would sit
    // idle longer than the third wave gains.
    auto go = [&](auto drop_c) {
      constexpr bool DR = decltype(drop_c)::value;
      if constexpr (D == 64) {
        if (grid_rows(c) >= 1536) {
          hipLaunchKernelGGL((fa::fwd_dma_kernel<D, 64, C, DR, 3>), dim3(grid_rows(c)), dim3(fa::kThreads), 0, st, a);
          return;
        }
      } else if constexpr (!DR) {
        if (grid_rows(c) >= 1536) {
          hipLaunchKernelGGL((fa::fwd_dma_kernel<D, 32, C, DR, 3>), dim3(grid_rows(c)), dim3(fa::kThreads), 0, st, a);
          return;
        }
      }
      hipLaunchKernelGGL((fa::fwd_dma_kernel<D, D == 64 ? 128 : 64, C, DR>), dim3(grid_rows(c)), dim3(fa::kThreads),
                         0, st, a);
    };
    if (c.drop)
      go(std::true_type{});
    else
      go(std::false_type{});
  } else if (c.drop)
    hipLaunchKernelGGL((fa::fwd_kernel<T, D, Tiles<T, D>::TS, C, true>), dim3(grid_rows(c)), dim3(fa::kThreads), 0,
                       st, a);
  else
    hipLaunchKernelGGL((fa::fwd_kernel<T, D, Tiles<T, D>::TS, C>), dim3(grid_rows(c)), dim3(fa::kThreads), 0, st, a);
}

template <typename T, int D, bool C>
void launch_bwd(const Ctx& c, const Args& a, hipStream_t st) {
  if constexpr (sizeof(T) != 2) {
    if (c.drop) {
      Args b = a;
      b.bs = nullptr;
      launch_rowscalar<T, D>(c, b, st);
      hipLaunchKernelGGL((fa::bwd_dq_kernel<T, D, Tiles<T, D>::TS, C, true>), dim3(grid_rows(c)),
                         dim3(fa::kThreads), 0, st, b);
      hipLaunchKernelGGL((fa::bwd_dkdv_kernel<T, D, Tiles<T, D>::TS, C, true>), dim3(grid_cols(c)),
                         dim3(fa::kThreads), 0, st, b);
      return;
    }
  }
  if constexpr (sizeof(T) == 2) {
    // Row scalars D plus the staged chain inits (-L/rho, -D) of the column
    // kernel: at d = 64 from the dQ kernel (which the column kernel follows),
    // at d = 128 from the row-scalar kernel.
    if constexpr (D != 64)
      hipLaunchKernelGGL((fa::rowscalar_kernel<T, D>), dim3(grid_rowscalar(c, true)), dim3(256), 0, st, a);
    constexpr int TS = D == 64 ? 128 : 64;
    const dim3 gc(grid_cols(c) * a.nsplit);
    if (c.drop) {
      hipLaunchKernelGGL((fa::bwd_dq_dma_kernel<D, TS, C, true>), dim3(grid_rows(c)), dim3(fa::kThreads), 0, st, a);
      hipLaunchKernelGGL((fa::bwd_dkdv_dma_kernel<D, TS, C, true>), gc, dim3(fa::kThreads), 0, st, a);
    } else {
      hipLaunchKernelGGL((fa::bwd_dq_dma_kernel<D, TS, C>), dim3(grid_rows(c)), dim3(fa::kThreads), 0, st, a);
      hipLaunchKernelGGL((fa::bwd_dkdv_dma_kernel<D, TS, C>), gc, dim3(fa::kThreads), 0, st, a);
    }
    launch_group_sum<D>(c, a, st);
  } else {
    Args b = a;
    b.bs = nullptr;
    launch_rowscalar<T, D>(c, b, st);
    hipLaunchKernelGGL((fa::bwd_dq_kernel<T, D, Tiles<T, D>::TS, C>), dim3(grid_rows(c)), dim3(fa::kThreads), 0,
                       st, b);
    hipLaunchKernelGGL((fa::bwd_dkdv_kernel<T, D, Tiles<T, D>::TS, C>), dim3(grid_cols(c)), dim3(fa::kThreads), 0,
                       st, b);
  }
}

// Schedules of the BoB ([FlashBoB] section 4.3 and appendix G.1):
//   0: two-pass (row-scalar kernel, row pass, column pass), the production path;
//   1: two-pass with the single-wave row pass at bf16, d = 64 (the same kernels
//      as 0 elsewhere), the baseline of the schedule ablation;
//   2: three-pass (row scalars, alpha sweep, row pass with known alpha, column
//      pass), bf16 only.
// phase < 0 runs the whole schedule; otherwise only that kernel.
template <typename T, int D, bool RHO1, bool C>
void launch_bob(const Ctx& c, const Args& a, hipStream_t st, int schedule, int phase) {
  const dim3 g(grid_rows(c)), b(fa::kThreads), gc(grid_cols(c) * a.nsplit);
  auto want = [&](int ph) { return phase < 0 || phase == ph; };
  if (c.drop) {  // two-pass schedule (schedule 2 is refused earlier)
    if constexpr (sizeof(T) == 2) {
      // bf16: the LDS-DMA row pass (which computes D itself) and the column
      // pass's split schedule, both with the mask; at d = 64 without the
      // causal mask the column pass runs two waves per SIMD when the grid
      // gives every CU its two workgroups.
      if (want(1)) {
        if constexpr (D == 64)
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 128, RHO1, false, C, 0, true>), g, b, 0, st, a);
        else
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 64, RHO1, true, C, 0, true>), g, b, 0, st, a);
      }
      if (want(2)) {
        if constexpr (D == 64) {
          if (!C && gc.x % 512 == 0)
            hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 64, RHO1, true, true, false, true, true>), gc, b, 0, st, a);
          else
            hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 128, RHO1, true, false, C, true>), gc, b, 0, st, a);
        } else
          hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 64, RHO1, true, true, C, true>), gc, b, 0, st, a);
        launch_group_sum<D>(c, a, st);
      }
    } else {
      if (want(0)) launch_rowscalar<T, D>(c, a, st);
      if (want(1)) hipLaunchKernelGGL((fa::bob_pass1_kernel<T, D, Tiles<T, D>::TS, RHO1, C, true>), g, b, 0, st, a);
      if (want(2)) hipLaunchKernelGGL((fa::bob_pass2_kernel<T, D, Tiles<T, D>::TS, RHO1, C, true>), gc, b, 0, st, a);
    }
    return;
  }
  // The bf16 two-pass row passes compute D themselves; phase 0 then launches nothing.
  if (want(0) && !(sizeof(T) == 2 && schedule != 2)) launch_rowscalar<T, D>(c, a, st);
  const int col_phase = schedule == 2 ? 3 : 2;
  if constexpr (sizeof(T) == 2) {
    if (schedule == 2) {
      if (want(1)) {
        if constexpr (D == 64)
          hipLaunchKernelGGL((fa::bob_alpha_dma_kernel<D, 128, RHO1, C>), g, b, 0, st, a);
        else
          hipLaunchKernelGGL((fa::bob_alpha_dma_kernel<D, 64, RHO1, C>), g, b, 0, st, a);
      }
      if (want(2)) {
        if constexpr (D == 64)
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 128, RHO1, false, C, 1>), g, b, 0, st, a);
        else
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 64, RHO1, true, C, 1>), g, b, 0, st, a);
      }
    } else if (want(1)) {
      // Two-pass row pass, a.ks workgroups per row block (key split).
      const dim3 gk(grid_rows(c) * a.ks);
      if constexpr (D == 64) {
        if (schedule == 0 && a.ks > 1) {  // never causal (key_split)
          if constexpr (!C)
            hipLaunchKernelGGL((fa::bob_pass1_ws_kernel<RHO1, C, true>), gk, dim3(2 * fa::kThreads), 0, st, a);
        } else if (schedule == 0)
          hipLaunchKernelGGL((fa::bob_pass1_ws_kernel<RHO1, C>), g, dim3(2 * fa::kThreads), 0, st, a);
        else
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 128, RHO1, false, C>), gk, b, 0, st, a);
      } else if (a.ks > 1) {  // never causal (key_split)
        if constexpr (!C)
          hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 64, RHO1, true, C, 0, false, true>), gk, b, 0, st, a);
      } else {
        hipLaunchKernelGGL((fa::bob_pass1_dma_kernel<D, 64, RHO1, true, C>), g, b, 0, st, a);
      }
      if (a.ks > 1) {
        const int64_t threads = (int64_t)(c.B * c.H) * padded_rows(c) * (D / 4);
        hipLaunchKernelGGL((fa::bob_ksplit_sum_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, a);
      }
    }
    if (want(col_phase)) {
      if constexpr (D == 64) {
        // Two workgroups per CU (64-row tiles, split schedule) when the grid
        // fills every CU's two slots evenly, else the woven one-wave kernel.
        if (gc.x % 512 == 0)
          hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 64, RHO1, true, true, C, false, true>), gc, b, 0, st, a);
        else
          hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 128, RHO1, false, false, C>), gc, b, 0, st, a);
      } else {
        hipLaunchKernelGGL((fa::bob_pass2_dma_kernel<D, 64, RHO1, true, true, C>), gc, b, 0, st, a);
      }
      launch_group_sum<D>(c, a, st);
    }
  } else {
    if (want(1)) hipLaunchKernelGGL((fa::bob_pass1_kernel<T, D, Tiles<T, D>::TS, RHO1, C>), g, b, 0, st, a);
    if (want(2)) hipLaunchKernelGGL((fa::bob_pass2_kernel<T, D, Tiles<T, D>::TS, RHO1, C>), gc, b, 0, st, a);
  }
}

// Dispatch on (input type, d, causal).
template <template <typename, int, bool> class L, typename... X>
void dispatch3(const Ctx& c, X&&... x) {
  if (c.bf) {
    if (c.d == 64) {
      if (c.causal) L<bf16, 64, true>::run(c, x...);
      else L<bf16, 64, false>::run(c, x...);
    } else {
      if (c.causal) L<bf16, 128, true>::run(c, x...);
      else L<bf16, 128, false>::run(c, x...);
    }
  } else {
    if (c.causal) L<float, 64, true>::run(c, x...);
    else L<float, 64, false>::run(c, x...);
  }
}

template <typename T, int D, bool C>
struct FwdL {
  static void run(const Ctx& c, const Args& a, hipStream_t st) { launch_fwd<T, D, C>(c, a, st); }
};
template <typename T, int D, bool C>
struct BwdL {
  static void run(const Ctx& c, const Args& a, hipStream_t st) { launch_bwd<T, D, C>(c, a, st); }
};
template <typename T, int D, bool C>
struct BobL {
  static void run(const Ctx& c, const Args& a, hipStream_t st, int schedule, int phase) {
    if (c.rho == 1.0f) launch_bob<T, D, true, C>(c, a, st, schedule, phase);
    else launch_bob<T, D, false, C>(c, a, st, schedule, phase);
  }
};

}  // namespace

// Workspace of fa_bob_noalloc: a device array that every call on one GPU
// shares (each GPU holds its own copy for the life of the process).  Host
// code never uses its name as an address: the per-device address comes from
// hipGetSymbolAddress on the first call made with that device current.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Address of the current device's scratch array (looked up once per device).
fa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape";
    case FA_ERR_STRIDE: return "invalid stride or alignment";
    case FA_ERR_DTYPE: return "invalid dtype";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t fa_bwd_workspace_bytes(const fa_problem* p) {
  Ctx c;
  if (check_problem(p, &c) != FA_OK) return 0;
  return (bwd_part_offset(c) + split_floats(c, group_split(c))) * sizeof(float);
}

size_t fa_bob_workspace_bytes(const fa_problem* p) {
  Ctx c;
  if (check_problem(p, &c) != FA_OK) return 0;
  return (bob_kpart_offset(c) + ksplit_floats(c, key_split(c))) * sizeof(float);
}

fa_status fa_fwd(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                 void* stream) {
  Ctx c;
  FA_CHECK(check_problem(p, &c));
  FA_CHECK(check_tensor(c, q, c.esize));
  FA_CHECK(check_tensor(c, k, c.esize));
  FA_CHECK(check_tensor(c, v, c.esize));
  FA_CHECK(check_tensor(c, o, 4));
  FA_CHECK(check_vec(lse));
  Args a = base_args(c);
  a.q = desc(q);
  a.k = desc(k);
  a.v = desc(v);
  a.r0 = desc(o);
  a.lse_out = lse;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch3<FwdL>(c, a, st);
  return launched();
}

fa_status fa_bwd(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, const float* lse,
                 fa_tensor dout, fa_tensor dq, fa_tensor dk, fa_tensor dv, void* workspace, size_t workspace_bytes,
                 void* stream) {
  Ctx c;
  FA_CHECK(check_problem(p, &c));
  FA_CHECK(check_tensor(c, q, c.esize));
  FA_CHECK(check_tensor(c, k, c.esize));
  FA_CHECK(check_tensor(c, v, c.esize));
  FA_CHECK(check_tensor(c, dout, c.esize));
  FA_CHECK(check_tensor(c, o, 4));
  FA_CHECK(check_tensor(c, dq, 4));
  FA_CHECK(check_tensor(c, dk, 4));
  FA_CHECK(check_tensor(c, dv, 4));
  FA_CHECK(check_vec(lse));
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16) return FA_ERR_WORKSPACE;
  if (workspace_bytes < fa_bwd_workspace_bytes(p)) return FA_ERR_WORKSPACE;
  Args a = base_args(c);
  a.q = desc(q);
  a.k = desc(k);
  a.v = desc(v);
  a.o = desc(o);
  a.dout = desc(dout);
  a.r0 = desc(dq);
  a.r1 = desc(dk);
  a.r2 = desc(dv);
  a.lse = lse;
  a.D = reinterpret_cast<float*>(workspace);
  a.bs = a.D + (size_t)(c.B * c.H * c.N);
  a.nsplit = group_split(c);
  a.gs = (int)(c.G / a.nsplit);
  a.part = a.nsplit > 1 ? a.D + bwd_part_offset(c) : nullptr;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch3<BwdL>(c, a, st);
  return launched();
}

static fa_status bob_impl(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o,
                          const float* lse, fa_tensor dout, fa_tensor uq, fa_tensor uk, fa_tensor uv, fa_tensor gq,
                          fa_tensor gk, fa_tensor gv, fa_tensor gdo, void* workspace, size_t workspace_bytes,
                          int schedule, int phase, void* stream, bool use_scratch = false) {
  Ctx c;
  FA_CHECK(check_problem(p, &c));
  if (schedule < 0 || schedule > 2) return FA_ERR_UNSUPPORTED;
  if (schedule == 2 && (!c.bf || c.drop)) return FA_ERR_UNSUPPORTED;
  if (phase < -1 || phase > (schedule == 2 ? 3 : 2)) return FA_ERR_UNSUPPORTED;
  FA_CHECK(check_tensor(c, q, c.esize));
  FA_CHECK(check_tensor(c, k, c.esize));
  FA_CHECK(check_tensor(c, v, c.esize));
  FA_CHECK(check_tensor(c, dout, c.esize));
  FA_CHECK(check_tensor(c, uq, c.esize));
  FA_CHECK(check_tensor(c, uk, c.esize));
  FA_CHECK(check_tensor(c, uv, c.esize));
  FA_CHECK(check_tensor(c, o, 4));
  FA_CHECK(check_tensor(c, gq, 4));
  FA_CHECK(check_tensor(c, gk, 4));
  FA_CHECK(check_tensor(c, gv, 4));
  FA_CHECK(check_tensor(c, gdo, 4));
  FA_CHECK(check_vec(lse));
  if (use_scratch) {  // fa_bob_noalloc: the static array, once the arguments passed
    if (fa_bob_workspace_bytes(p) > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
    FA_CHECK(scratch_of_current_device(&workspace));
    workspace_bytes = FA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16) return FA_ERR_WORKSPACE;
  if (workspace_bytes < fa_bob_workspace_bytes(p)) return FA_ERR_WORKSPACE;
  Args a = base_args(c);
  a.q = desc(q);
  a.k = desc(k);
  a.v = desc(v);
  a.o = desc(o);
  a.dout = desc(dout);
  a.uq = desc(uq);
  a.uk = desc(uk);
  a.uv = desc(uv);
  a.r0 = desc(gq);
  a.r1 = desc(gk);
  a.r2 = desc(gv);
  a.r3 = desc(gdo);
  a.lse = lse;
  const size_t nrow = (size_t)(c.B * c.H * c.N);
  a.D = reinterpret_cast<float*>(workspace);
  a.alpha = a.D + nrow;
  a.E = a.D + 2 * nrow;
  a.ps = a.D + 3 * nrow;
  const int gsplit = group_split(c);
  a.gs = (int)(c.G / gsplit);
  a.rs = row_split(c, gsplit);
  a.nsplit = gsplit * a.rs;
  a.part = a.nsplit > 1 ? a.D + bob_part_offset(c) : nullptr;
  // Only the two-pass schedule's row passes split their keys (not the
  // single-wave baseline of the ablation nor the three-pass schedule).
  a.ks = schedule == 0 ? key_split(c) : 1;
  a.kpart = a.ks > 1 ? a.D + bob_kpart_offset(c) : nullptr;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch3<BobL>(c, a, st, schedule, phase);
  return launched();
}

fa_status fa_bob(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, const float* lse,
                 fa_tensor dout, fa_tensor uq, fa_tensor uk, fa_tensor uv, fa_tensor gq, fa_tensor gk, fa_tensor gv,
                 fa_tensor gdo, void* workspace, size_t workspace_bytes, void* stream) {
  return bob_impl(p, q, k, v, o, lse, dout, uq, uk, uv, gq, gk, gv, gdo, workspace, workspace_bytes, 0, -1, stream);
}

fa_status fa_bob_noalloc(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o,
                         const float* lse, fa_tensor dout, fa_tensor uq, fa_tensor uk, fa_tensor uv, fa_tensor gq,
                         fa_tensor gk, fa_tensor gv, fa_tensor gdo, void* stream) {
  return bob_impl(p, q, k, v, o, lse, dout, uq, uk, uv, gq, gk, gv, gdo, nullptr, 0, 0, -1, stream, true);
}

fa_status fa_bob_phase(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, const float* lse,
                       fa_tensor dout, fa_tensor uq, fa_tensor uk, fa_tensor uv, fa_tensor gq, fa_tensor gk,
                       fa_tensor gv, fa_tensor gdo, void* workspace, size_t workspace_bytes, int32_t phase,
                       void* stream) {
  if (phase < 0 || phase > 2) return FA_ERR_UNSUPPORTED;
  return bob_impl(p, q, k, v, o, lse, dout, uq, uk, uv, gq, gk, gv, gdo, workspace, workspace_bytes, 0, phase, stream);
}

fa_status fa_bob_schedule(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o,
                          const float* lse, fa_tensor dout, fa_tensor uq, fa_tensor uk, fa_tensor uv, fa_tensor gq,
                          fa_tensor gk, fa_tensor gv, fa_tensor gdo, void* workspace, size_t workspace_bytes,
                          int32_t schedule, int32_t phase, void* stream) {
  return bob_impl(p, q, k, v, o, lse, dout, uq, uk, uv, gq, gk, gv, gdo, workspace, workspace_bytes, schedule,
                  phase, stream);
}

}  // extern "C"
