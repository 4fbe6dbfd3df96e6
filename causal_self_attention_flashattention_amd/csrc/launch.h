// Host-side launchers for the attention kernels (internal to libattn; the public C ABI is
// include/attn.h).  Each launcher only enqueues work on `stream`; it returns hipSuccess, or
// hipErrorInvalidValue when no kernel exists for the (dtype, head dim) pair, or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

enum Dtype { kF32 = 0, kBF16 = 1 };

struct Problem {
  int B, H, N, d;
  int causal;
  float scale;
  const int32_t* kv_len;  // device int32[B] or nullptr
  const uint8_t* bmask;   // block-sparse mask, device uint8[TB][TB] (TB = ceil(N / 64)), or nullptr
};

bool fwd_supported(int dtype, int d);
bool bwd_supported(int dtype, int d);

// Forward.  With a workspace of at least fwd_workspace_bytes(dtype, p) bytes (non-zero only for
// grids too small to fill the chip) the key range of every query tile is split over several
// workgroups whose partial results a second kernel merges; otherwise one launch.
constexpr int kMaxSplits = 16;
hipError_t launch_fwd(int dtype, const Problem& p, const void* Q, const void* K, const void* V,
                      void* O, float* L, hipStream_t stream, void* workspace = nullptr, size_t workspace_bytes = 0);
int fwd_splits(int dtype, const Problem& p);
size_t fwd_workspace_bytes(int dtype, const Problem& p);

hipError_t launch_rowdot(int dtype, const Problem& p, const void* O, const void* dO, float* Dv,
                         hipStream_t stream);

// dK/dV and dQ.  With a workspace of at least bwd_workspace_bytes(dtype, p) bytes (non-zero only
// for grids too small to fill the chip) each workgroup chain is split into chunks whose float32
// partials a sum kernel adds in fixed order; the two calls may share one workspace (dQ's sum runs
// before dK/dV's partials are written, on the same stream).
size_t bwd_workspace_bytes(int dtype, const Problem& p);
hipError_t launch_dkdv(int dtype, const Problem& p, const void* Q, const void* K, const void* V,
                       const void* dO, const float* L, const float* Dv, void* dK, void* dV,
                       hipStream_t stream, void* workspace = nullptr, size_t workspace_bytes = 0);

// dQ; with O != nullptr it also computes D = rowsum(O o dO) for its rows and stores it to Dv
// (which is then an output), else it reads D from Dv.
hipError_t launch_dq(int dtype, const Problem& p, const void* Q, const void* K, const void* V,
                     const void* dO, const void* O, const float* L, float* Dv, void* dQ, hipStream_t stream,
                     void* workspace = nullptr, size_t workspace_bytes = 0);

// Small problems: the dQ and dK/dV work of attn_bwd in a single launch (both halves independent;
// D stored by the dQ half).  bwd_small_applies tells when this path is used.
bool bwd_small_applies(int dtype, const Problem& p);
hipError_t launch_bwd_small(int dtype, const Problem& p, const void* Q, const void* K, const void* V,
                            const void* dO, const void* O, const float* L, float* Dv, void* dQ, void* dK,
                            void* dV, hipStream_t stream);

// attn_bwd_ex split in two: argument validation (returns an attn_status, launches nothing) and
// dispatch of the kernels (returns ATTN_OK or ATTN_E_LAUNCH); the C ABI runs both.
int bwd_ex_check(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                 void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, float scale, int dtype,
                 const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes);
int bwd_ex_run(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L, void* dQ,
               void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale, int dtype,
               const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

}  // namespace attn
