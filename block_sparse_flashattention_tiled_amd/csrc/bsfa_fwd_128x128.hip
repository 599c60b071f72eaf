// Forward, diagnostic and tile-maximum kernels for 128 x 128 tiles
// (B_M = 128 query rows, B_N = 128 keys), both head dimensions.
#include <atomic>
#include <mutex>

#include "bsfa_fwd_kernels.h"

namespace bsfa {

// Work counters of the persistent pipelined launches: a ring of slots of 8
// 64-bit counters (one per XCD queue) that the library holds in device
// memory, a copy per device.  Each launch takes the next slot and zeroes it on its own stream
// before the kernel; a slot comes round again after kWorkSlots launches, so at
// most that many launches may be in flight at once on one device.
constexpr int kWorkSlots = 1024;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned long long work_ring[kWorkSlots][8];

__global__ void zero_work_slot(unsigned long long* w) {
  if (threadIdx.x < 8) w[threadIdx.x] = 0;
}

unsigned long long* pipe_work_slot(hipStream_t stream, int* n_cu) {
  static std::mutex mu;
  static unsigned long long* ring[kMaxDevices];  // the ring's device address on each device
  static int cus[kMaxDevices];
  static std::atomic<unsigned> next{0};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!ring[dev]) {
      void* ptr = nullptr;
      int c = 0;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(work_ring)) != hipSuccess || !ptr) return nullptr;
      if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return nullptr;
      cus[dev] = c;
      ring[dev] = static_cast<unsigned long long*>(ptr);
    }
    *n_cu = cus[dev];
  }
  unsigned long long* slot = ring[dev] + 8 * (next.fetch_add(1, std::memory_order_relaxed) % kWorkSlots);
  hipLaunchKernelGGL(zero_work_slot, dim3(1), dim3(64), 0, stream, slot);
  if (hipGetLastError() != hipSuccess) return nullptr;
  return slot;
}

int launch_fwd_128x128(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t stream) {
  return launch_tile<128, 128>(p, head_dim, causal, mode, stream);
}

}  // namespace bsfa
