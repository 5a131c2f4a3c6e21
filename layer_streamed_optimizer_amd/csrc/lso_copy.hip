// Host <-> device block copies issued by the shader cores.
//
// The layer stream moves each piece with one copy per direction.  By
// default both run on two SDMA engines it names (lso_sdma.h); this kernel
// serves the other modes: D2H when the engines cannot be named (H2D then
// goes to a runtime-chosen DMA engine, which on its own would often share
// one engine with the D2H and halve it), or both directions on request.
// Done by a kernel, the two directions run at about 46-47 GB/s each way on
// this part's PCIe Gen5 x16 link whatever else the process has queued.
// One 16-byte vector per lane and iteration; 128 workgroups keep the link
// busy -- more keep so many long-latency host reads queued that the update
// kernel running beside them slows down.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lso_copy.h"

namespace lso {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
block_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint64_t n16,
                  const unsigned char* __restrict__ src_tail, unsigned char* __restrict__ dst_tail,
                  uint32_t ntail)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    const uint64_t first = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (uint64_t i = first; i < n16; i += stride) dst[i] = src[i];
    if (first < ntail) dst_tail[first] = src_tail[first];
}

}  // namespace

int launch_block_copy(void* dst, const void* src, uint64_t bytes, unsigned max_grid, void* stream)
{
    if (bytes == 0) return 0;
    const uint64_t n16 = bytes / 16;
    const uint32_t ntail = static_cast<uint32_t>(bytes % 16);
    const uint64_t want = (n16 + 255) / 256;
    const uint64_t cap = max_grid ? max_grid : kCopyGrid;
    const unsigned grid = static_cast<unsigned>(want < cap ? (want ? want : 1) : cap);
    hipLaunchKernelGGL(block_copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16,
                       static_cast<const unsigned char*>(src) + n16 * 16,
                       static_cast<unsigned char*>(dst) + n16 * 16, ntail);
    return static_cast<int>(hipGetLastError());
}

}  // namespace lso
