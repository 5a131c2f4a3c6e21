// The update for callers that cannot allocate (lso_adam_step_noalloc).
//
// lso_adam_step keeps the block table of a call with more than kInline
// blocks in device memory it allocates (and caches).  This entry point
// keeps it instead in one file-scope device array per GPU, `scratch`, of
// fixed size, written on the call's stream by a small kernel whose
// arguments carry the table (so nothing is read from host memory after the
// call returns, and no host buffer has to outlive it).  The fused kernel
// then finds each workgroup's block by a binary search over that table (no
// per-chunk index: it would not fit a fixed array).  Nothing here calls
// hipMalloc, hipFree or any other allocating routine.
//
// Every call on a GPU shares that GPU's array and leaves its table there:
// calls that overlap on one GPU (on different streams, or from several
// threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "lso_internal.h"
#include "lso_runtime.h"

namespace lso {
namespace {

constexpr size_t kScratchBlocks = LSO_NOALLOC_MAX_BLOCKS;
static_assert(kScratchBlocks * sizeof(DevBlock) == 256 * 1024, "scratch is 256 KiB");

// The table of the call's launches, per device.  In host code this name is
// a host-side stand-in; kernels get the device address taken below.
static __device__ __align__(256) DevBlock scratch[kScratchBlocks];

// Table entries per writer launch: the kernel arguments stay under 4 KiB.
constexpr uint32_t kWriteBlocks = 56;

struct TablePart {
    DevBlock* dst;
    uint32_t count;
    uint32_t pad;
    DevBlock src[kWriteBlocks];
};
static_assert(sizeof(TablePart) <= 4000, "writer arguments");

__global__ void __launch_bounds__(64) table_write_kernel(const TablePart part)
{
    // one entry per lane, eight 8-byte vector stores each
    if (threadIdx.x < part.count) part.dst[threadIdx.x] = part.src[threadIdx.x];
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DevBlock* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

}  // namespace

lso_status noalloc_scratch(DevBlock** out, void* stream)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LSO_E_INVALID, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev] && stream) {
        // the address is looked up once per device, outside any capture (the
        // lookup may load the code object, which a capture cannot hold)
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        err = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs);
        if (err != hipSuccess) return hip_fail(err, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone)
            return fail(LSO_E_INVALID, "the first lso_adam_step_noalloc call on device %d is under stream capture: "
                        "make one call (any table of more than 4 blocks, or lso_adam_step) before capturing", dev);
    }
    if (!g_scratch[dev]) {
        // once per device, with that device current
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p) return hip_fail(err, "hipGetSymbolAddress(scratch)");
        g_scratch[dev] = static_cast<DevBlock*>(p);
    }
    *out = g_scratch[dev];
    return LSO_OK;
}

lso_status noalloc_write_table(DevBlock* dst, const DevBlock* tab, size_t count, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t k = 0; k < count; k += kWriteBlocks) {
        TablePart part{};
        part.dst = dst + k;
        part.count = static_cast<uint32_t>(count - k < kWriteBlocks ? count - k : kWriteBlocks);
        for (uint32_t j = 0; j < part.count; ++j) part.src[j] = tab[k + j];
        hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(64), 0, s, part);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return hip_fail(err, "table write launch");
    }
    return LSO_OK;
}

}  // namespace lso

extern "C" lso_status lso_adam_step_noalloc(const lso_block* blocks, size_t n, void* stream)
{
    lso::clear_error();
    return lso::enqueue_update_noalloc(blocks, n, stream);
}
