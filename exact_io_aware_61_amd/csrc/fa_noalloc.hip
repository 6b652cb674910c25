// fa_bwd for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same three
// backward stages on the same kernels, with their per-row workspace (D_i and
// LSE_i log2(e), 8 bytes per query row) in a fixed device array of this library
// instead of a caller-supplied buffer.
//
// The array lives in this file's code object, one copy per GPU the library runs
// on, held until the process ends. In host code its name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and cached; kernels only ever
// receive that address. Every call on one GPU shares the GPU's copy: calls that
// overlap on one GPU (two streams, or two host threads) race. Nothing in it must
// start at zero: the preprocess stage writes every row the later stages read.
#include <mutex>

#include "fa.h"
#include "fa_kernels.hpp"

constexpr size_t kScratchBytes = size_t(16) << 20;   // B*H*ceil(N/128)*128 <= 2^21 rows

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Device address of this device's copy of `scratch`; `dev` is made current for
// the lookup and the previous current device restored.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, float scale, const fa_mask_t* mask,
                              void* stream) {
  size_t need = 0;
  const int rc = fa_bwd_workspace_size(B, H, N, d, &need);
  if (rc != FA_OK) return rc;
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  if ((int64_t)B * H * N == 0) return FA_OK;
  // the device the stream's work runs on (the current device for the null stream)
  int dev = 0;
  if (stream != nullptr) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
      return FA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FA_ERR_HIP;
  }
  void* ws = nullptr;
  const int got = scratch_on(dev, &ws);
  if (got != FA_OK) return got;
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, mask, ws, kScratchBytes,
                stream);
}
