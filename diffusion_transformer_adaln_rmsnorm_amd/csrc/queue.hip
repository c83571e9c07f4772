// Tile-queue counters of the persistent GEMM launches.
//
// Each persistent launch takes one counter set from a static device pool (a set per launch,
// in rotation).  A set starts at zero (the pool is zero when the module loads) and the last
// workgroup of the launch that used it puts it back to zero when it finishes, so no kernel or
// memset has to clear it and the launch can be captured in a HIP graph as it is.  Launches that
// overlap in time get different sets as long as fewer than kQueueSlots of them are in flight
// at once; the one case that shares a set is two replays of the same captured graph running at
// the same time (the set is fixed at capture).
//
// The pool is a file-scope __device__ array: each GPU the library runs on holds its own copy.
// Host code never names it in a kernel argument (there the name is a host-side stand-in, not a
// device address): on the first call on a device, with that device current,
// hipGetSymbolAddress gives that device's copy, which is kept per device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {
namespace {

constexpr int kQueueSlots = 4096;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint32_t g_tile_queues[kQueueSlots * gemm::kTileQueueWords];

std::mutex g_mu;
uint32_t* g_pool[kMaxDevices];     // device address of the pool on each device, once looked up
int g_grid[kMaxDevices];           // persistent grid: the device's CUs, a multiple of kXcds
std::atomic<uint64_t> g_seq{0};

hipError_t device_state(uint32_t** pool, int* grid) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_pool[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_tile_queues));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus -= cus % gemm::kXcds;
        if (cus <= 0) return hipErrorInvalidDevice;
        g_grid[dev] = cus;
        g_pool[dev] = static_cast<uint32_t*>(p);
    }
    *pool = g_pool[dev];
    *grid = g_grid[dev];
    return hipSuccess;
}

}  // namespace

hipError_t tile_queue(hipStream_t stream, uint32_t** counters, int* grid) {
    uint32_t* pool = nullptr;
    hipError_t e = device_state(&pool, grid);
    if (e != hipSuccess) return e;
    (void)stream;
    const uint64_t slot = g_seq.fetch_add(1, std::memory_order_relaxed) % kQueueSlots;
    *counters = pool + slot * gemm::kTileQueueWords;
    return hipSuccess;
}

}  // namespace dit
