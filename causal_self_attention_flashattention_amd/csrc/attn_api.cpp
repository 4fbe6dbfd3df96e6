// C ABI of libattn (declared in include/attn.h): argument validation, then dispatch to the
// kernel launchers.  Nothing here allocates memory or synchronises the host.
#include "../../include/attn.h"

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == ATTN_DTYPE_BF16 ? 2 : 4; }

// Block-sparse masks hold one byte per 64 x 64 block; the kernels keep one row of it in LDS.
constexpr int kMaxBlockSparseN = 65536;
int mask_blocks(int N) { return (N + 63) / 64; }

int check_common(int B, int H, int N, int d, int dtype, float scale, bool need_scale) {
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_E_DTYPE;
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_E_SHAPE;
  const int64_t elems = (int64_t)B * H * N * d;
  if (elems >= ((int64_t)1 << 31)) return ATTN_E_SHAPE;
  // The kernels address one head of a tensor through a 32-bit buffer resource with signed 32-bit
  // byte offsets, so a head (N * d elements) must span fewer than 2^31 bytes.
  if ((int64_t)N * d * (int64_t)elem_size(dtype) >= ((int64_t)1 << 31)) return ATTN_E_SHAPE;
  if (!attn::fwd_supported(dtype, d)) return ATTN_E_HEADDIM;
  // The kernels take row maxima of the unscaled scores and mask before scaling, both of which
  // assume scale > 0.
  if (need_scale && !(std::isfinite(scale) && scale > 0.f)) return ATTN_E_SCALE;
  return ATTN_OK;
}

// Every output range must be disjoint from every input range and from the other outputs.
int check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (ins[j].lo != ins[j].hi && overlap(outs[i], ins[j])) return ATTN_E_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_E_ALIAS;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_version(void) { return 10000; }

int attn_bwd_launches(int B, int H, int N, int d, int dtype) {
  const int st = check_common(B, H, N, d, dtype, 1.0f, false);
  if (st != ATTN_OK) return st;
  const attn::Problem p{B, H, N, d, 1, 1.0f, nullptr};
  return attn::bwd_small_applies(dtype, p) ? 1 : 2;
}

int attn_supported(int dtype, int d) {
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return 0;
  return attn::fwd_supported(dtype, d) && attn::bwd_supported(dtype, d) ? 1 : 0;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "B, H, N and d must be >= 1, B*H*N*d < 2^31 and one head (N*d elements) < 2^31 bytes";
    case ATTN_E_HEADDIM: return "unsupported head dim (supported: 16, 32, 64, 80, 128)";
    case ATTN_E_DTYPE: return "unknown dtype (0 = float32, 1 = bfloat16)";
    case ATTN_E_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_E_ALIAS: return "an output buffer overlaps an input or another output";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_SCALE: return "scale is not a finite number greater than 0";
    case ATTN_E_SCRATCH:
      return "the shape needs more scratch than attn_bwd_noalloc's static buffer holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N, int d,
             int causal, float scale, int dtype, const int32_t* kv_len, hipStream_t stream) {
  return attn_fwd_ex(Q, K, V, O, L, B, H, N, d, causal, scale, dtype, kv_len, nullptr, nullptr, 0, stream);
}

size_t attn_fwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_common(B, H, N, d, dtype, 1.0f, false) != ATTN_OK) return 0;
  const attn::Problem p{B, H, N, d, 1, 1.0f, nullptr};
  return attn::fwd_workspace_bytes(dtype, p);
}

int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N, int d,
                int causal, float scale, int dtype, const int32_t* kv_len, const uint8_t* block_mask,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!Q || !K || !V || !O || !L) return ATTN_E_NULL;
  int st = check_common(B, H, N, d, dtype, scale, true);
  if (st != ATTN_OK) return st;
  if (block_mask && N > kMaxBlockSparseN) return ATTN_E_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(L)) return ATTN_E_ALIGN;
  if (workspace && !aligned16(workspace)) return ATTN_E_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const size_t mb = block_mask ? (size_t)mask_blocks(N) * mask_blocks(N) : 0;
  const Range outs[3] = {range_of(O, tb), range_of(L, lb),
                         workspace ? range_of(workspace, workspace_bytes) : Range{0, 0}};
  const Range ins[5] = {range_of(Q, tb), range_of(K, tb), range_of(V, tb),
                        kv_len ? range_of(kv_len, (size_t)B * 4) : Range{0, 0}, range_of(block_mask, mb)};
  st = check_alias(outs, workspace ? 3 : 2, ins, 5);
  if (st != ATTN_OK) return st;
  const attn::Problem p{B, H, N, d, causal ? 1 : 0, scale, kv_len, block_mask};
  if (attn::launch_fwd(dtype, p, Q, K, V, O, L, stream, workspace, workspace ? workspace_bytes : 0) != hipSuccess)
    return ATTN_E_LAUNCH;
  return ATTN_OK;
}

int attn_bwd_rowdot(const void* O, const void* dO, float* D, int B, int H, int N, int d, int dtype,
                    hipStream_t stream) {
  if (!O || !dO || !D) return ATTN_E_NULL;
  int st = check_common(B, H, N, d, dtype, 1.0f, false);
  if (st != ATTN_OK) return st;
  if (!aligned16(O) || !aligned16(dO) || !aligned16(D)) return ATTN_E_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const Range outs[1] = {range_of(D, (size_t)B * H * N * sizeof(float))};
  const Range ins[2] = {range_of(O, tb), range_of(dO, tb)};
  st = check_alias(outs, 1, ins, 2);
  if (st != ATTN_OK) return st;
  const attn::Problem p{B, H, N, d, 0, 1.0f, nullptr};
  if (attn::launch_rowdot(dtype, p, O, dO, D, stream) != hipSuccess) return ATTN_E_LAUNCH;
  return ATTN_OK;
}

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
             void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
             int dtype, const int32_t* kv_len, hipStream_t stream) {
  return attn_bwd_ex(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, causal, scale, dtype, kv_len, nullptr, nullptr, 0,
                     stream);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_common(B, H, N, d, dtype, 1.0f, false) != ATTN_OK) return 0;
  const attn::Problem p{B, H, N, d, 1, 1.0f, nullptr};
  return attn::bwd_workspace_bytes(dtype, p);
}

}  // extern "C"

namespace attn {

int bwd_ex_check(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                 void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, float scale, int dtype,
                 const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes) {
  if (!Q || !K || !V || !O || !dO || !L || !dQ || !dK || !dV || !D) return ATTN_E_NULL;
  int st = check_common(B, H, N, d, dtype, scale, true);
  if (st != ATTN_OK) return st;
  if (block_mask && N > kMaxBlockSparseN) return ATTN_E_SHAPE;
  const void* ptrs[] = {Q, K, V, O, dO, L, dQ, dK, dV, D};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_E_ALIGN;
  if (workspace && !aligned16(workspace)) return ATTN_E_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const size_t mb = block_mask ? (size_t)mask_blocks(N) * mask_blocks(N) : 0;
  const Range outs[5] = {range_of(dQ, tb), range_of(dK, tb), range_of(dV, tb), range_of(D, lb),
                         workspace ? range_of(workspace, workspace_bytes) : Range{0, 0}};
  const Range ins[8] = {range_of(Q, tb), range_of(K, tb), range_of(V, tb), range_of(O, tb), range_of(dO, tb),
                        range_of(L, lb), kv_len ? range_of(kv_len, (size_t)B * 4) : Range{0, 0},
                        range_of(block_mask, mb)};
  return check_alias(outs, workspace ? 5 : 4, ins, 8);
}

int bwd_ex_run(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L, void* dQ,
               void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale, int dtype,
               const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  const attn::Problem p{B, H, N, d, causal ? 1 : 0, scale, kv_len, block_mask};
  const size_t need = attn::bwd_workspace_bytes(dtype, p);
  const bool split = need > 0 && workspace && workspace_bytes >= need;
  if (!split && attn::bwd_small_applies(dtype, p)) {
    // Small grids: dQ and dK/dV side by side in one launch.
    if (attn::launch_bwd_small(dtype, p, Q, K, V, dO, O, L, D, dQ, dK, dV, stream) != hipSuccess)
      return ATTN_E_LAUNCH;
    return ATTN_OK;
  }
  // The dQ kernel computes D for its query rows on the way (replacing the separate pre-pass), so it
  // runs first; the dK/dV kernel then reads D.  With a large enough workspace both split their
  // workgroup chains (the two phases reuse the workspace one after the other).
  void* ws = split ? workspace : nullptr;
  const size_t wb = split ? workspace_bytes : 0;
  if (attn::launch_dq(dtype, p, Q, K, V, dO, O, L, D, dQ, stream, ws, wb) != hipSuccess) return ATTN_E_LAUNCH;
  if (attn::launch_dkdv(dtype, p, Q, K, V, dO, L, D, dK, dV, stream, ws, wb) != hipSuccess) return ATTN_E_LAUNCH;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

int attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
                int dtype, const int32_t* kv_len, const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  const int st = attn::bwd_ex_check(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, scale, dtype, kv_len, block_mask,
                                    workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  return attn::bwd_ex_run(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, causal, scale, dtype, kv_len, block_mask,
                          workspace, workspace_bytes, stream);
}

int attn_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H, int N,
                         int d, int causal, float scale, int dtype, const int32_t* kv_len, const uint8_t* block_mask,
                         hipStream_t stream) {
  return attn_fwd_ex(Q, K, V, O, L, B, H, N, d, causal, scale, dtype, kv_len, block_mask, nullptr, 0, stream);
}

int attn_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                         void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d, int causal, float scale,
                         int dtype, const int32_t* kv_len, const uint8_t* block_mask, hipStream_t stream) {
  return attn_bwd_ex(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, causal, scale, dtype, kv_len, block_mask, nullptr,
                     0, stream);
}

int attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* L, const float* D,
                  void* dK, void* dV, int B, int H, int N, int d, int causal, float scale, int dtype,
                  const int32_t* kv_len, hipStream_t stream) {
  if (!Q || !K || !V || !dO || !L || !D || !dK || !dV) return ATTN_E_NULL;
  int st = check_common(B, H, N, d, dtype, scale, true);
  if (st != ATTN_OK) return st;
  const void* ptrs[] = {Q, K, V, dO, L, D, dK, dV};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_E_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const Range outs[2] = {range_of(dK, tb), range_of(dV, tb)};
  const Range ins[7] = {range_of(Q, tb), range_of(K, tb), range_of(V, tb), range_of(dO, tb),
                        range_of(L, lb), range_of(D, lb), kv_len ? range_of(kv_len, (size_t)B * 4) : Range{0, 0}};
  st = check_alias(outs, 2, ins, 7);
  if (st != ATTN_OK) return st;
  const attn::Problem p{B, H, N, d, causal ? 1 : 0, scale, kv_len};
  if (attn::launch_dkdv(dtype, p, Q, K, V, dO, L, D, dK, dV, stream) != hipSuccess) return ATTN_E_LAUNCH;
  return ATTN_OK;
}

int attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const void* O, const float* L,
                float* D, void* dQ, int B, int H, int N, int d, int causal, float scale, int dtype,
                const int32_t* kv_len, hipStream_t stream) {
  if (!Q || !K || !V || !dO || !L || !D || !dQ) return ATTN_E_NULL;
  int st = check_common(B, H, N, d, dtype, scale, true);
  if (st != ATTN_OK) return st;
  const void* ptrs[] = {Q, K, V, dO, L, D, dQ};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_E_ALIGN;
  if (O && !aligned16(O)) return ATTN_E_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  // D is an output when O is given, an input otherwise.
  const Range outs[2] = {range_of(dQ, tb), range_of(D, lb)};
  const Range ins[7] = {range_of(Q, tb), range_of(K, tb), range_of(V, tb), range_of(dO, tb),
                        range_of(L, lb), O ? range_of(O, tb) : Range{0, 0},
                        kv_len ? range_of(kv_len, (size_t)B * 4) : Range{0, 0}};
  st = O ? check_alias(outs, 2, ins, 7) : check_alias(outs, 1, ins, 7);
  if (st != ATTN_OK) return st;
  if (!O && overlap(outs[0], outs[1])) return ATTN_E_ALIAS;
  const attn::Problem p{B, H, N, d, causal ? 1 : 0, scale, kv_len};
  if (attn::launch_dq(dtype, p, Q, K, V, dO, O, L, D, dQ, stream) != hipSuccess) return ATTN_E_LAUNCH;
  return ATTN_OK;
}

}  // extern "C"
