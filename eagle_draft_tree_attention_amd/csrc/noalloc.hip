// eagle_verify_spec_accept_noalloc: multi-round speculative sampling for
// callers that cannot allocate device memory (code that a caller captures
// into a HIP graph, tight serving loops, harnesses that forbid hipMalloc).
//
// It runs the same kernels as eagle_verify_spec_accept.  Their scratch (node
// states, chunk statistics, round partials, publication and round words)
// lives in `scratch`, a fixed-size array in device memory that the code
// object provides on every GPU the library runs on, instead of a handle's
// workspace.  Host code reaches the array only through the device address
// hipGetSymbolAddress returns for the current device, looked up once per
// device on its first call.
//
// Every call first clears the part of the array it uses with a fill kernel
// on the caller's stream (no hipMemsetAsync, which a captured graph must not
// hold), so nothing carries over from the previous call.  Calls that overlap
// on one GPU share the array and race: the caller serialises them (one
// stream, or events between streams).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <mutex>

#include "ev_internal.h"

namespace {

// scratch of one call: 8 MiB covers, e.g., 32 sequences of 64 rows at
// V = 32000, or 8 sequences of 64 rows at V = 128256
constexpr size_t kScratchBytes = size_t(8) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  bool ready = false;
  unsigned char* ptr = nullptr;   // device address of `scratch` on that device
  int fused_cap[2] = {0, 0};      // co-resident fused-acceptance workgroups (f32, bf16)
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ __launch_bounds__(256) void scratch_zero(uint4* p, size_t n16) {
  const uint4 z = {0u, 0u, 0u, 0u};
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = z;
}

eagle_status fail(const char* msg) {
  ev::set_thread_error(msg);
  return EAGLE_ERR_ARG;
}

}  // namespace

extern "C" EAGLE_API eagle_status eagle_verify_spec_accept_noalloc(const eagle_verify_desc* desc,
                                                                    const eagle_spec_accept_args* a,
                                                                    void* hip_stream) {
  char msg[512] = {0};
  eagle_status st = ev::check_desc(desc, msg, sizeof(msg));
  if (st == EAGLE_OK) st = ev::check_spec_accept(desc, a, msg, sizeof(msg));
  if (st != EAGLE_OK) {
    ev::set_thread_error(msg);
    return st;
  }
  // the layout of this call: its own batch and row count
  const int NC = ev::vocab_chunks(desc->vocab_size);
  const size_t need = ev::accept_layout(a->batch, a->tree_rows, NC, 0, nullptr, nullptr);
  if (need > kScratchBytes) {
    std::snprintf(msg, sizeof(msg),
                  "spec_accept_noalloc: %d sequences of %d rows over %d vocabulary chunks need %zu bytes of "
                  "scratch, more than the %zu available",
                  a->batch, a->tree_rows, NC, need, kScratchBytes);
    ev::set_thread_error(msg);
    return EAGLE_ERR_CAPACITY;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    std::snprintf(msg, sizeof(msg), "hipGetDevice failed: %s", hipGetErrorString(e));
    ev::set_thread_error(msg);
    return EAGLE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return fail("spec_accept_noalloc: device index out of range");
  DeviceScratch ds;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch& d = g_dev[dev];
    if (!d.ready) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr) {
        std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        ev::set_thread_error(msg);
        return EAGLE_ERR_HIP;
      }
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = ev::kDefaultCUs;
      d.ptr = static_cast<unsigned char*>(ptr);
      d.fused_cap[0] = ev::fused_accept_capacity(0, cus);
      d.fused_cap[1] = ev::fused_accept_capacity(1, cus);
      d.ready = true;
    }
    ds = d;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const size_t n16 = need / 16;   // the layout is a multiple of 256 bytes
  const unsigned grid = static_cast<unsigned>(std::min<size_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(scratch_zero, dim3(grid), dim3(256), 0, stream, reinterpret_cast<uint4*>(ds.ptr), n16);
  e = hipGetLastError();
  if (e != hipSuccess) {
    std::snprintf(msg, sizeof(msg), "scratch clear launch failed: %s", hipGetErrorString(e));
    ev::set_thread_error(msg);
    return EAGLE_ERR_HIP;
  }
  ev::Workspace ws;
  ev::accept_layout(a->batch, a->tree_rows, NC, 0, reinterpret_cast<char*>(ds.ptr), &ws);
  ev::AcceptCallState cs;   // fresh: the cleared scratch holds no earlier epoch
  const int64_t cap = ds.fused_cap[desc->logits_dtype == EAGLE_BF16 ? 1 : 0];
  st = ev::run_spec_accept(*desc, ws, a->batch, a->tree_rows, cap, &cs, a, hip_stream, msg, sizeof(msg),
                           ev::spin_limit_from_env(), ev::cooperative_from_env());
  ev::set_thread_error(st == EAGLE_OK ? "" : msg);
  return st;
}
