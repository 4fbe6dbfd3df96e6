/* attn.h -- C ABI of libattn: tiled causal / key-padded self-attention, forward and backward,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (notation of the CS336 Assignment 2 (systems) handout: eq. 1 in §4.1 "Optimizing
 * Attention with FlashAttention-2", everything else in §4.2.2 "FlashAttention-2 forward pass"):
 *   forward  (eq. 1, eqs. 4-6, eq. 12, Algorithm 1):
 *     S = scale * Q K^T, masked entries removed, P = row softmax(S), O = P V,
 *     L_i = log sum_j exp(S_ij) over the unmasked entries of row i (natural log).
 *   backward (eqs. 13-19, "backward pass with recomputation"):
 *     D_i = sum_c O_ic dO_ic, P_ij = exp(S_ij - L_i), dV = P^T dO, dP = dO V^T,
 *     dS_ij = P_ij (dP_ij - D_i), dQ = scale dS K, dK = scale dS^T Q.
 *   masks: causal (Problem (flash_forward)(c)): key j is masked for query i when j > i, with
 *     equal query and key lengths N; key padding: keys j >= kv_len[b] are masked for every
 *     query of batch row b.  Queries are never masked.
 *
 * Layout: Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] (d fastest) in the
 * element type `dtype`; L and D are dense [B, H, N] float32.  `kv_len` is a device int32[B] or
 * NULL (no padding).  All pointers are device pointers, 16-byte aligned, owned by the caller;
 * the library allocates nothing and keeps no per-call state.
 *
 * Execution: every call only enqueues kernels on `stream` (NULL = the default stream) and
 * returns without synchronising the host; faults inside a kernel surface at the caller's next
 * synchronisation.  Results are bitwise reproducible (no atomics).
 *
 * Errors: each call validates its arguments before launching anything and returns an
 * attn_status; on any negative status nothing has been enqueued (except ATTN_E_LAUNCH, which
 * reports the HIP launch error of a kernel).  No exception crosses the ABI.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,    /* a required pointer is NULL */
  ATTN_E_SHAPE = -2,   /* B, H, N or d < 1, B*H*N*d >= 2^31 elements, or one head's N*d elements
                          span 2^31 bytes or more (the kernels' per-head 32-bit buffer offsets) */
  ATTN_E_HEADDIM = -3, /* no kernel for this head dim (supported: 16, 32, 64, 80, 128) */
  ATTN_E_DTYPE = -4,   /* dtype is not an attn_dtype */
  ATTN_E_ALIGN = -5,   /* a pointer is not 16-byte aligned */
  ATTN_E_ALIAS = -6,   /* an output buffer overlaps an input or another output */
  ATTN_E_LAUNCH = -7,  /* a kernel launch failed (HIP error) */
  ATTN_E_SCALE = -8,   /* scale is not a finite number > 0 */
  ATTN_E_SCRATCH = -9  /* attn_bwd_noalloc: the shape needs more than ATTN_NOALLOC_SCRATCH_BYTES */
} attn_status;

/* Forward pass (Algorithm 1 of the handout, §4.2.2, with the causal flag of Problem
 * (flash_forward)(c)).
 *   Q, K, V  in : [B,H,N,d] dtype
 *   O        out: [B,H,N,d] dtype, softmax(mask(scale Q K^T)) V
 *   L        out: [B,H,N] float32, natural-log logsumexp of the scaled, masked scores
 *   causal      : 0 or non-zero
 *   scale       : softmax scale, finite and > 0; normally 1/sqrt(d)
 *   kv_len      : device int32[B], 1 <= kv_len[b] <= N (values outside are clamped), or NULL
 * O and L must not overlap any input or each other. */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N, int d,
             int causal, float scale, int dtype, const int32_t* kv_len, hipStream_t stream);

/* Backward pass (eqs. 13-19 of the handout, §4.2.2; the two-kernel split of §4.2.3 that
 * recomputes P once for dK/dV and once for dQ).
 *   Q, K, V, O, dO in : [B,H,N,d] dtype (O and L as returned by attn_fwd for the same inputs)
 *   L              in : [B,H,N] float32
 *   dQ, dK, dV     out: [B,H,N,d] dtype
 *   D              out: [B,H,N] float32 workspace, receives rowsum(O o dO)
 * Other arguments as for attn_fwd.  Outputs must not overlap inputs or each other. */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
             void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
             int dtype, const int32_t* kv_len, hipStream_t stream);

/* The backward's first step alone: D_i = sum_c O_ic dO_ic in float32 (handout §4.2.2, the D
 * vector of the backward pass with recomputation).  O, dO: [B,H,N,d] dtype; D: [B,H,N] float32. */
int attn_bwd_rowdot(const void* O, const void* dO, float* D, int B, int H, int N, int d, int dtype,
                    hipStream_t stream);

/* The backward's second step alone: dK and dV for every key tile (eqs. 13-17 and 19 of the
 * handout, §4.2.2), P recomputed from L, D taken from attn_bwd_rowdot (or from attn_bwd_dq called
 * with O).  Arguments as for attn_bwd; D is an input here. */
int attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* L, const float* D,
                  void* dK, void* dV, int B, int H, int N, int d, int causal, float scale, int dtype,
                  const int32_t* kv_len, hipStream_t stream);

/* dQ for every query tile (eqs. 13-14, 16-18 of the handout's §4.2.2), P recomputed a second time
 * so that no two workgroups write the same output (§4.2.3).
 *   O   in, optional: [B,H,N,d] dtype forward output.  When non-NULL the kernel first computes
 *       D = rowsum(O o dO) for its own query rows and writes it to D (D is then an output, and this
 *       call replaces attn_bwd_rowdot); when NULL, D is an input (from attn_bwd_rowdot).
 *   D   [B,H,N] float32, see O.
 * attn_bwd = attn_bwd_dq with O, then attn_bwd_dkdv.  Other arguments as for attn_bwd. */
int attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const void* O, const float* L,
                float* D, void* dQ, int B, int H, int N, int d, int causal, float scale, int dtype,
                const int32_t* kv_len, hipStream_t stream);

/* Block-sparse forward ("Notes on flashattention", section Block-sparse Flashattention): as
 * attn_fwd, with the scores further restricted to the support of a mask that is constant on
 * 64 x 64 blocks, and blocks outside it skipped entirely (neither loaded nor computed).
 *   block_mask in: device uint8 [TB][TB], TB = ceil(N / 64), row-major, shared by every (batch,
 *                  head); entry (r, c) != 0 lets queries 64r .. 64r+63 attend keys 64c .. 64c+63.
 *                  Combined (AND) with the causal and key-padding masks.  NULL = attn_fwd.
 * A query row left with no key at all gets O = 0 and L = -inf.  Requires N <= 65536
 * (ATTN_E_SHAPE otherwise).  Outputs must not overlap any input, the mask included. */
int attn_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N,
                         int d, int causal, float scale, int dtype, const int32_t* kv_len, const uint8_t* block_mask,
                         hipStream_t stream);

/* Bytes of workspace attn_fwd_ex can use for this shape: non-zero when B*H*ceil(N/128) query
 * tiles are too few to fill the chip, in which case the key range of each query tile is split
 * over several workgroups (partial results in the workspace, merged by a second kernel with the
 * online-softmax rescaling of the handout's Algorithm 1).  0 on bad arguments. */
size_t attn_fwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/* attn_fwd with every option: block_mask as for attn_fwd_blocksparse (NULL = none), and a
 * caller-owned device workspace.  With workspace_bytes >= attn_fwd_workspace_bytes(...) the split
 * path runs; with a smaller (or NULL) workspace the plain single launch runs.  The results agree
 * with attn_fwd to rounding (the split sums in a different order); both are deterministic.  The
 * workspace must be 16-byte aligned and must not overlap any input or output; its contents are
 * scratch (not read before written). */
int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N, int d,
                int causal, float scale, int dtype, const int32_t* kv_len, const uint8_t* block_mask,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Block-sparse backward: attn_bwd under the same block mask as attn_fwd_blocksparse (O and L must
 * come from that call).  Rows without keys get dQ = 0 and contribute nothing to dK, dV; D is
 * still rowsum(O o dO).  NULL block_mask = attn_bwd.  Other arguments as for attn_bwd. */
int attn_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                         void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
                         int dtype, const int32_t* kv_len, const uint8_t* block_mask, hipStream_t stream);

/* Bytes of workspace attn_bwd_ex can use for this shape: non-zero when the dQ or dK/dV grid is
 * too small to fill the chip, in which case each workgroup's chain (key tiles for dQ, query tiles
 * for dK/dV) is split over several workgroups whose float32 partials a sum kernel adds up in a
 * fixed order.  0 on bad arguments. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/* attn_bwd with every option: block_mask as for attn_bwd_blocksparse (NULL = none) and a
 * caller-owned device workspace, used as for attn_fwd_ex (split path when workspace_bytes >=
 * attn_bwd_workspace_bytes(...), the plain launches otherwise).  Deterministic either way; the
 * split path agrees with attn_bwd to rounding. */
int attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
                int dtype, const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* Size of the static device scratch behind attn_bwd_noalloc (64 MiB per GPU the library runs on). */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* attn_bwd_ex without a caller workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Where attn_bwd_ex would
 * split the workgroup chains of a small grid (attn_bwd_workspace_bytes(...) > 0), the partial sums go
 * to a file-scope device array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the call itself calls no hipMalloc, hipFree or allocating library
 * routine.  Results are bitwise those of attn_bwd_ex given a workspace of at least
 * attn_bwd_workspace_bytes(...) bytes.
 *   Arguments as for attn_bwd_ex (no workspace).  The scratch is that of the device `stream` belongs
 *   to (the current device for the NULL stream).
 *   ATTN_E_SCRATCH when attn_bwd_workspace_bytes(B, H, N, d, dtype) > ATTN_NOALLOC_SCRATCH_BYTES
 *   (nothing is enqueued); other errors as for attn_bwd_ex.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents (each call
 * writes every partial it later reads, so nothing needs clearing): calls whose kernels can overlap
 * on one GPU (different streams, or different host threads without ordering) race and must not be
 * issued. */
int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                     void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
                     int dtype, const int32_t* kv_len, const uint8_t* block_mask, hipStream_t stream);

/* How many kernels attn_bwd launches for this problem: 1 when the dQ and dK/dV work share one
 * launch (small bfloat16 problems with d <= 80, where the grid would otherwise leave CUs idle),
 * 2 otherwise (attn_bwd_dq with O, then attn_bwd_dkdv).  Negative attn_status on bad arguments. */
int attn_bwd_launches(int B, int H, int N, int d, int dtype);

/* Static text for a status code (never NULL). */
const char* attn_status_string(int status);

/* 1 if a kernel exists for (dtype, d), else 0. */
int attn_supported(int dtype, int d);

/* ABI version: 10000 * major + 100 * minor + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
