/*
 * fa.h -- C ABI of the MI355X (gfx950) attention library: forward, first
 * backward and exact backward-over-backward (BoB) of softmax attention.
 *
 * Sources cited below by page title and section:
 *   [FlashBoB]      "FlashBoB: I/O-Efficient Exact Backward-over-Backward for
 *                   Softmax Attention" (Givans, Crawshaw, Liu).
 *   [FA2-recompute] "Why does FlashAttention-2's backward pass recompute
 *                   attention, and what exactly does the forward pass save
 *                   for it?"
 *   [FA2-triton]    "FlashAttention-2 from PyTorch to Triton".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Problem: B batches x H query heads, sequence length N (queries = keys),
 * head dimension d, softmax scale tau, full or causal attention.  Causal adds
 * the mask term B_mask = -inf for key j > query i to S ([FlashBoB] section 3);
 * key tiles entirely above the diagonal are skipped.  One attention head is
 * the (b, h) slice.
 *
 * Grouped-query / multi-query attention ([FlashBoB] section 4.3, the
 * paragraph after Algorithm 1): H_kv key/value heads, H_kv dividing H, G =
 * H / H_kv.  Query head h attends to key/value head h / G (consecutive query
 * heads share a head).  K, V, U_K, U_V and the key-side outputs dK, dV, gK,
 * gV have H_kv heads; every key-side output is the sum over its group's G
 * query heads, accumulated inside one workgroup (no atomics).  H_kv = 0 or
 * H_kv = H is multi-head attention.
 *
 * Tensors: every N x d operand is passed as an fa_tensor: a DEVICE pointer
 * plus element strides for the batch, head and sequence dimensions; the head
 * dimension is contiguous (stride 1).  Element (b, h, n, c) lives at
 * ptr[b*stride_b + h*stride_h + n*stride_n + c].  Pointers must be 16-byte
 * aligned and stride_n, stride_h, stride_b must be multiples of 16 bytes
 * (8 bf16 or 4 fp32 elements); d <= stride_n <= 2^26.  Inputs Q, K, V, dO, U_Q,
 * U_K, U_V use the problem's input dtype (bf16 or fp32).  O and every
 * output are fp32.
 *
 * Row vectors (L, and D / alpha / E in the workspace) are contiguous
 * [B, H, N] fp32 device arrays.
 *
 * Ownership: the caller allocates and frees every buffer.  The library never
 * allocates, frees or synchronises; it enqueues kernels on `stream` (a
 * hipStream_t; NULL means the default stream) and returns.  It keeps no
 * state between calls and is reentrant.
 *
 * Errors: every argument is validated on the host before anything is
 * launched; a failed validation returns the status and enqueues nothing.  A
 * launch error reported by the HIP runtime returns FA_ERR_HIP.  Outputs must
 * not alias inputs or each other.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, H or N < 1, H_kv not 0 or a divisor of H, or sizes overflow */
  FA_ERR_STRIDE = 3,      /* stride or alignment rule violated */
  FA_ERR_DTYPE = 4,       /* unknown input dtype */
  FA_ERR_UNSUPPORTED = 5, /* d not in {64, 128} (fp32 inputs: d = 64 only), causal not 0/1,
                             a NaN or +inf scale (any scale <= 0, -inf included, selects
                             1/sqrt(d)), or a dropout rate outside [0, 255.5/256) */
  FA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
  FA_ERR_HIP = 7          /* the HIP runtime reported a launch error */
} fa_status;

typedef enum fa_dtype {
  FA_BF16 = 0, /* bfloat16 inputs; contractions on bf16 MFMA, fp32 accumulate */
  FA_FP32 = 1  /* fp32 inputs (d = 64); contractions on fp32 MFMA */
} fa_dtype;

typedef struct fa_problem {
  int64_t B, H, N, d;
  float scale;      /* tau; a value <= 0 selects 1/sqrt(d) */
  int32_t causal;   /* 0: full attention; 1: causal (key j > query i masked) */
  int32_t in_dtype; /* an fa_dtype */
  int64_t H_kv;     /* key/value heads: 0 (= H) or a divisor of H */
  float dropout;    /* dropout rate p in [0, 1); 0 = none (see below) */
  int32_t reserved; /* set to 0 */
  uint64_t seed;    /* dropout generator key */
} fa_problem;

/*
 * Dropout ([FlashBoB] appendix G, "Analytical dropout extension"): the
 * forward multiplies P by a scaled keep mask g before the product with V,
 *   O = (P * g) V,   L unchanged (over P),
 * the first backward uses dP = g * (dO V^T) and dV = (P * g)^T dO, and fa_bob
 * returns the BoB of that first backward: the pages' identities with
 * A = g * (dO V^T) in place of dP, C = g * (dO U_V^T), h = F - alpha, and
 * P * g in the products with V and dO (d~(V) = (P g h)^T dO,
 * d~(dO) = (P g) U_V + (P g h) V).
 * g is not stored: every pass regenerates it from Philox4x64-10 (Salmon et
 * al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with key
 * (seed, 0).  Element (i, j) of query head bh = b * H + h takes byte j % 8
 * of output word i % 4 of the block for counter (i / 4, j / 8, bh, 0); with
 * t = round(256 p) (t <= 255, else FA_ERR_UNSUPPORTED) it is kept iff that
 * byte is >= t, and kept elements are scaled by 256 / (256 - t).  p rounds
 * to a multiple of 1/256; t = 0 means no dropout.  The same (p, seed) must be
 * passed to fa_fwd, fa_bwd and fa_bob.  With bf16 inputs dropout runs on
 * the same LDS-DMA kernels as the dropout-free path (about 1.4x the
 * dropout-free fa_bob time); fp32 inputs use the portable register-staged
 * kernels.  The three-pass schedule of fa_bob_schedule does not support it.
 */

typedef struct fa_tensor {
  void* ptr; /* device pointer */
  int64_t stride_b, stride_h, stride_n; /* element strides; head dim stride is 1 */
} fa_tensor;

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

/* Static text for a status code (never NULL). */
const char* fa_status_str(fa_status s);

/*
 * fa_fwd -- softmax attention forward, [FlashBoB] section 3:
 *   S = tau Q K^T,  P = softmax(S) row-wise,  O = P V,
 *   L_i = log sum_j exp(S_ij)   (natural log; the saved row statistic from
 *                                which P_ij = exp(S_ij - L_i) is rebuilt,
 *                                [FA2-recompute]).
 * In:  q, k, v  (in_dtype).
 * Out: o (fp32, N x d per head), lse (fp32 [B,H,N]).
 * Online softmax over key tiles ([FA2-triton]); nothing N x N is stored.
 */
fa_status fa_fwd(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                 fa_tensor o, float* lse, void* stream);

/* Workspace bytes fa_bwd needs: the row vector D (B*H*N fp32, first), then
 * 8 * B*H*ceil(N/128)*128 bytes of per-row chain inits for the key-side
 * kernel (an internal layout). */
size_t fa_bwd_workspace_bytes(const fa_problem* p);

/*
 * fa_bwd -- first backward at output cotangent dO, [FlashBoB] section 3:
 *   dP = dO V^T, dV = P^T dO, dS_ij = P_ij (dP_ij - D_i),
 *   dQ = tau dS K, dK = tau dS^T Q,
 * with D_i = rowsum(dO * O)_i ([FA2-recompute]), computed by a row-scalar
 * kernel into the workspace (first B*H*N floats; the rest is internal).
 * In:  q, k, v, dout (in_dtype); o (fp32) and lse (fp32) from fa_fwd.
 * Out: dq (H heads), dk, dv (H_kv heads: sums over each group) in fp32.
 * Deterministic: every output block has one writer.
 */
fa_status fa_bwd(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                 fa_tensor o, const float* lse, fa_tensor dout,
                 fa_tensor dq, fa_tensor dk, fa_tensor dv,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bob needs: D, alpha, E, each B*H*N fp32, in that order,
 * then 16 * B*H*ceil(N/128)*128 bytes of per-row chain inits the row pass
 * leaves for the column pass (an internal layout).  Problems too small to
 * give every compute unit a workgroup (fewer than 256 row or column blocks
 * of 128) add the partial sums of the kernels that are then split over
 * several workgroups (an internal layout too). */
size_t fa_bob_workspace_bytes(const fa_problem* p);

/*
 * fa_bob -- exact backward-over-backward, [FlashBoB] sections 4.1-4.3 and
 * appendix D ("Final assembled identities").  With cotangents U_Q, U_K, U_V
 * on the first-backward outputs dQ, dK, dV, the functional
 *   Phi = <dQ, U_Q> + <dK, U_K> + <dV, U_V>
 * is differentiated with respect to Q, K, V and dO (total derivatives: O and
 * L are functions of Q, K, V):
 *   F = tau (U_Q K^T + Q U_K^T),  alpha_i = sum_j P_ij F_ij,  C = dO U_V^T,
 *   d~P = C + F (dP - D) - alpha dP,  E_i = sum_j P_ij d~P_ij,
 *   d~S = P (d~P - E),  h = F - alpha,
 *   gq  = tau (d~S K + dS U_K),     gk  = tau (d~S^T Q + dS^T U_Q),
 *   gv  = (P h)^T dO,               gdo = P U_V + (P h) V.
 * Schedule ([FlashBoB] section 4.3): D = rowsum(dO * O) (computed inside the
 * row pass for bf16 inputs, by a row-scalar kernel for fp32); a row-major
 * pass accumulates the row outputs with the affine corrections of section 4.2
 * and writes gq, gdo, alpha, E (and D) once per row block; a
 * column-major pass writes gk, gv once per column block.  No N x N tensor is
 * written anywhere and no atomics are used, so results are deterministic.
 * In:  q, k, v, dout, uq, uk, uv (in_dtype); o (fp32), lse (fp32) from fa_fwd;
 *      k, v, uk, uv have H_kv heads.
 * Out: gq, gdo (H heads), gk, gv (H_kv heads) in fp32.  Workspace: [D | alpha | E | internal], D,
 *      alpha, E each contiguous [B,H,N] fp32 (this part of the layout is part
 *      of the ABI); the internal tail carries per-row values from the row pass
 *      to the column pass.
 */
fa_status fa_bob(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                 fa_tensor o, const float* lse, fa_tensor dout,
                 fa_tensor uq, fa_tensor uk, fa_tensor uv,
                 fa_tensor gq, fa_tensor gk, fa_tensor gv, fa_tensor gdo,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bob_noalloc -- fa_bob for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as fa_bob without the
 * workspace: D, alpha, E and the row pass's per-row values live in a static
 * device array of FA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on
 * each GPU it runs on until the process ends, so D, alpha and E are not
 * returned.  Nothing in the array needs clearing: the row pass writes every
 * value the column pass reads.  The array's address on the current device is
 * looked up on the first call made with that device current; call with the
 * stream's device current.
 * Limit: fa_bob_workspace_bytes(p) <= FA_NOALLOC_SCRATCH_BYTES, i.e. about
 * B*H*N <= 2.39 million rows when nothing is split (N = 262,144 with B*H = 8
 * fits); small problems whose kernels split (see fa_bob_workspace_bytes)
 * also hold their partial sums there (multi-query, 8 heads, N = 2048, d =
 * 64: 52 MiB).  A larger problem returns FA_ERR_WORKSPACE before anything is
 * launched.
 * Calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering) share the array and race: serialise them.
 * Allocates nothing, no torch or library allocator included.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fa_status fa_bob_noalloc(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                         fa_tensor o, const float* lse, fa_tensor dout,
                         fa_tensor uq, fa_tensor uk, fa_tensor uv,
                         fa_tensor gq, fa_tensor gk, fa_tensor gv, fa_tensor gdo,
                         void* stream);

/*
 * fa_bob_phase -- one kernel of fa_bob, for per-kernel timing and profiling.
 * Same arguments as fa_bob plus `phase`: 0 launches the row-scalar kernel
 * (writes D; with bf16 inputs the row pass computes D itself and phase 0
 * launches nothing), 1 the row-major pass (writes gq, gdo, alpha, E and, for
 * bf16, D), 2 the column-major pass (reads D, alpha, E; writes gk, gv).  Calling phases 0, 1,
 * 2 in that order on one stream is exactly fa_bob.  A phase outside 0..2
 * returns FA_ERR_UNSUPPORTED.
 */
fa_status fa_bob_phase(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                       fa_tensor o, const float* lse, fa_tensor dout,
                       fa_tensor uq, fa_tensor uk, fa_tensor uv,
                       fa_tensor gq, fa_tensor gk, fa_tensor gv, fa_tensor gdo,
                       void* workspace, size_t workspace_bytes, int32_t phase,
                       void* stream);

/* Schedules of fa_bob_schedule. */
typedef enum fa_schedule {
  FA_SCHED_TWO_PASS = 0,       /* what fa_bob runs */
  FA_SCHED_TWO_PASS_1WAVE = 1, /* two-pass with the single-wave row pass (bf16, d = 64; else = 0) */
  FA_SCHED_THREE_PASS = 2      /* three-pass schedule of [FlashBoB] appendix G.1 (bf16 only) */
} fa_schedule;

/*
 * fa_bob_schedule -- fa_bob under a chosen schedule, for the schedule
 * ablation of [FlashBoB] appendix G.1 ("Three-pass versus two-pass").  Every
 * schedule computes the same outputs and workspace values (D, alpha, E) up to
 * rounding; they differ in how many sweeps stream the key side:
 *   FA_SCHED_TWO_PASS, FA_SCHED_TWO_PASS_1WAVE: phases 0 (row scalars D; bf16:
 *     nothing, the row pass computes D), 1 (row pass: gq, gdo, alpha, E with
 *     the affine corrections of section 4.2), 2 (column pass: gk, gv);
 *   FA_SCHED_THREE_PASS: phases 0 (D), 1 (alpha-only row sweep, streams K and
 *     U_K), 2 (row pass with alpha known: gq by the delayed E-correction, gdo,
 *     E), 3 (column pass).
 * phase = -1 runs the whole schedule; calling its phases in order on one
 * stream is the same.  Arguments otherwise as fa_bob.  Errors: an unknown
 * schedule, a phase outside the schedule, or FA_SCHED_THREE_PASS with fp32
 * inputs return FA_ERR_UNSUPPORTED before anything is launched.
 */
fa_status fa_bob_schedule(const fa_problem* p, fa_tensor q, fa_tensor k, fa_tensor v,
                          fa_tensor o, const float* lse, fa_tensor dout,
                          fa_tensor uq, fa_tensor uk, fa_tensor uv,
                          fa_tensor gq, fa_tensor gk, fa_tensor gv, fa_tensor gdo,
                          void* workspace, size_t workspace_bytes, int32_t schedule,
                          int32_t phase, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
