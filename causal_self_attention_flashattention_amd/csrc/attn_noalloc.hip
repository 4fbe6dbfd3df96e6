// attn_bwd_noalloc: the backward of attn_bwd_ex with the split-chain partial sums in a static device
// array instead of a caller workspace, for callers that cannot allocate device memory.
//
// The array `scratch` lives in this module's device memory on every GPU the library runs on, for
// the life of the process.  In host code its name only stands for the device symbol; the device
// address comes from hipGetSymbolAddress, looked up once per device with that device current and
// kept per device, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of `scratch` on device `dev`, or nullptr if it cannot be looked up.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess) return nullptr;
  g_scratch[dev] = p;
  return p;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                const float* L, void* dQ, void* dK, void* dV, float* D, int B, int H, int N, int d,
                                int causal, float scale, int dtype, const int32_t* kv_len,
                                const uint8_t* block_mask, hipStream_t stream) {
  int st = attn::bwd_ex_check(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, scale, dtype, kv_len, block_mask,
                              nullptr, 0);
  if (st != ATTN_OK) return st;
  const attn::Problem p{B, H, N, d, causal ? 1 : 0, scale, kv_len, block_mask};
  const size_t need = attn::bwd_workspace_bytes(dtype, p);
  if (need > kScratchBytes) return ATTN_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return ATTN_E_LAUNCH;
    ws = scratch_on(dev);
    if (!ws) return ATTN_E_LAUNCH;
  }
  return attn::bwd_ex_run(Q, K, V, O, dO, L, dQ, dK, dV, D, B, H, N, d, causal, scale, dtype, kv_len, block_mask, ws,
                          ws ? kScratchBytes : 0, stream);
}
