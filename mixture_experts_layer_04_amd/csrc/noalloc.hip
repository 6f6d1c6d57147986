// moe_layer_noalloc: moe_layer on a scratch array that the library holds in
// device memory, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: each GPU that loads the
// library holds its own copy, at its own address, until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host
// that name is a stand-in, not a device address): the first call on a device
// looks the device address up with hipGetSymbolAddress, with that device
// current, and every later call on the device uses the address kept here.
//
// Contents: the array is the moe_layer workspace.  Its first 64 KiB are the
// control block, whose counters must be zero when a call starts; every call
// leaves them at zero, and the first call on a device clears them (a fill
// kernel on the caller's stream) before its own kernels.  Everything else
// the layer writes before it reads.  Calls that overlap in time on one GPU
// share the array and race: a caller serialises them (one stream, or events).

#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;   // device address of this device's `scratch`
  bool cleared = false;  // its control block was cleared by a call outside a capture
};

std::mutex g_mutex;
DeviceScratch g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// The device that `stream` runs on (the current device for the null stream).
moe_status stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev) == hipSuccess ? MOE_OK : MOE_E_HIP;
  hipDevice_t d = 0;
  if (hipStreamGetDevice(stream, &d) != hipSuccess) return MOE_E_HIP;
  *dev = (int)d;
  return MOE_OK;
}

// This device's scratch address, looked up on the first call with the
// device current.
moe_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch& s = g_scratch[dev];
  if (!s.ptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_E_HIP;
    if (e != hipSuccess || p == nullptr) return MOE_E_HIP;
    s.ptr = p;
  }
  *out = s.ptr;
  return MOE_OK;
}

// Clears this device's control block until a clear has been enqueued
// outside a stream capture (a clear recorded into a graph runs only when the
// graph does, so calls keep enqueueing it until one runs eagerly).
moe_status clear_until_done(int dev, void* ptr, hipStream_t stream) {
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev].cleared) return MOE_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return MOE_E_HIP;
  constexpr int words = (int)(moe::kCtrlBytes / 4);
  clear_words_kernel<<<words / (256 * 4), 256, 0, stream>>>(static_cast<uint32_t*>(ptr), words);
  MOE_CHECK_LAUNCH();
  if (cap == hipStreamCaptureStatusNone) {
    std::lock_guard<std::mutex> lock(g_mutex);
    g_scratch[dev].cleared = true;
  }
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_noalloc(const void* x, const void* gate, int gate_is_fp32, const float* bias,
                                        int wformat,
                                        const void* w13, const void* w13_scale, const void* w2,
                                        const void* w2_scale, int T, int H, int E, int F, int k, int n_shared,
                                        int n_group, int topk_group, int scoring, int renormalize,
                                        float routed_scale, int block_m, float swiglu_limit, void* y,
                                        int32_t* topk_ids_out, float* topk_weights_out, hipStream_t stream) {
  // host checks first: nothing is looked up or enqueued for a call that
  // fails them or that the scratch array cannot hold
  moe_status st = moe::layer_validate(x, gate, gate_is_fp32, wformat, w13, w13_scale, w2, w2_scale, T, H, E, F, k,
                                      n_shared, n_group, topk_group, scoring, block_m, swiglu_limit, y);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (moe::layer_workspace_bytes(T, H, E, F, k, n_shared, block_m, wformat) > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_E_WORKSPACE;
  int dev = 0;
  st = stream_device(stream, &dev);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != MOE_OK) return st;
  st = clear_until_done(dev, ws, stream);
  if (st != MOE_OK) return st;
  return moe::layer_enqueue(x, gate, gate_is_fp32, bias, wformat, w13, w13_scale, w2, w2_scale, T, H, E, F, k,
                            n_shared, n_group,
                            topk_group, scoring, renormalize, routed_scale, block_m, swiglu_limit, y, topk_ids_out,
                            topk_weights_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
