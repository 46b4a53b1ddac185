// muon_step_noalloc: muon_step_ex for callers that cannot allocate device
// memory.  The step's workspace is a file-scope device array of a fixed
// size instead of a caller buffer, and the launch tables reach it through
// kernel arguments (copied by the runtime at launch) instead of pinned
// staging, so the call makes no allocation of any kind.  The kernels are the
// ones muon_step_ex launches; they take the array's device address as their
// workspace pointer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "elem.hpp"
#include "muon.h"
#include "plan.hpp"

namespace {

constexpr size_t kScratchBytes = MUON_NOALLOC_SCRATCH_BYTES;

// The workspace of every allocation-free step on a device.  In host code
// `scratch` is only a stand-in for the device array: its device address
// comes from hipGetSymbolAddress (per device, below), and only that address
// is ever handed to a kernel or a copy.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's scratch array, looked up once per device
// with that device current.
muon_status scratch_ptr(char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    muon::set_error(std::string("muon_step_noalloc: hipGetDevice: ") + hipGetErrorString(e));
    return MUON_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    muon::set_error("muon_step_noalloc: device index beyond " + std::to_string(kMaxDevices));
    return MUON_ERR_UNSUPPORTED;
  }
  std::call_once(g_once[dev], [dev] {
    void *ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_err[dev] != hipSuccess || !g_ptr[dev]) {
    muon::set_error(std::string("muon_step_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(g_err[dev]));
    return MUON_ERR_HIP;
  }
  *out = static_cast<char *>(g_ptr[dev]);
  return MUON_OK;
}

// One piece of the launch tables, carried in the kernel's arguments.
constexpr int kChunkWords = 768;  // 3 KB per launch, under the 4 KB argument limit
struct TableChunk {
  uint64_t offset;  // byte offset of the piece in the workspace
  uint32_t nwords;
  uint32_t pad_;
  uint32_t w[kChunkWords];
};
constexpr size_t kMaxTableBytes = 32 * kChunkWords * 4;  // 96 KB: at most 32 launches

__global__ __launch_bounds__(256) void k_put_tables(char *ws, TableChunk c) {
  uint32_t *dst = reinterpret_cast<uint32_t *>(ws + c.offset);
  for (uint32_t i = threadIdx.x; i < c.nwords; i += 256) dst[i] = c.w[i];
}

}  // namespace

extern "C" muon_status muon_step_noalloc(muon_plan *p, const void *const *grads, float *const *momenta,
                                         float *const *partitions, const int32_t *skip_flag, float grad_scale,
                                         void *stream) {
  if (!p) { muon::set_error("muon_step_noalloc: NULL plan"); return MUON_ERR_INVALID_ARG; }
  if ((size_t)p->ws_bytes > kScratchBytes) {
    muon::set_error("muon_step_noalloc: the plan needs " + std::to_string(p->ws_bytes) +
                    " bytes of workspace, the static scratch holds " + std::to_string(kScratchBytes) +
                    " (cap it with max_inflight_bytes, or use muon_step_ex with a workspace)");
    return MUON_ERR_WORKSPACE;
  }
  const size_t tb = p->host_tables.size();
  if (tb > kMaxTableBytes || tb % 4 != 0) {
    muon::set_error("muon_step_noalloc: launch tables of " + std::to_string(tb) + " bytes exceed the " +
                    std::to_string(kMaxTableBytes) + " the kernel-argument upload carries");
    return MUON_ERR_UNSUPPORTED;
  }
  char *wsb = nullptr;
  muon_status st = scratch_ptr(&wsb);
  if (st != MUON_OK) return st;
  st = muon::step_check(p, grads, momenta, partitions, skip_flag, grad_scale, wsb, kScratchBytes);
  if (st != MUON_OK) return st;

  // the plan's tables with this call's pointers, into the plan's own host
  // buffer (sized at plan creation), then into the scratch by value
  muon::step_patch(p, p->patch_host.data(), grads, momenta, partitions, wsb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TableChunk c;
  const size_t nw = tb / 4;
  for (size_t w0 = 0; w0 < nw; w0 += kChunkWords) {
    const size_t n = std::min<size_t>(kChunkWords, nw - w0);
    c.offset = (uint64_t)(w0 * 4);
    c.nwords = (uint32_t)n;
    c.pad_ = 0;
    std::memcpy(c.w, p->patch_host.data() + w0 * 4, n * 4);
    hipLaunchKernelGGL(k_put_tables, dim3(1), dim3(256), 0, s, wsb, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      muon::set_error(std::string("muon_step_noalloc: table upload: ") + hipGetErrorString(e));
      return MUON_ERR_HIP;
    }
  }
  st = muon::step_launch(p, skip_flag, grad_scale, wsb, stream, false, false);
  if (st != MUON_OK) return st;
  muon::step_count(p, skip_flag, wsb);
  return MUON_OK;
}
