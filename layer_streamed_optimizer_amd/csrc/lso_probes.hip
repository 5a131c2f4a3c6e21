// Measurement and verification probes (not part of the update path).
//
//  lso_probe_copy      plain 16-byte-vector device copy: the HBM ceiling a
//                      read+write stream reaches, and the reference for
//                      scaling the FETCH_SIZE / WRITE_SIZE counters.
//  lso_probe_bf16_rne  the fused kernel's BF16 rounding applied to a range
//                      of FP32 bit patterns, so a test can compare it with
//                      the host definition over all 2^32 patterns.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lso_bf16.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LSO_GLOBAL __attribute__((address_space(1)))

// One 16-byte vector per lane, non-temporal both ways (the fastest plain
// copy measured on this part: one pass, nothing reused).
__global__ void __launch_bounds__(256)
copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint64_t n16)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 x = __builtin_nontemporal_load(
            reinterpret_cast<const LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(src + i)));
        __builtin_nontemporal_store(x, reinterpret_cast<LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(dst + i)));
    }
}

__global__ void __launch_bounds__(256)
bf16_probe_kernel(uint32_t first, uint64_t count, uint16_t* __restrict__ out)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t bits = first + static_cast<uint32_t>(i);
        out[i] = static_cast<uint16_t>(lso::bf16_rne(__uint_as_float(bits)));
    }
}

}  // namespace

extern "C" {

// Copy bytes (a multiple of 16; both pointers 16-byte aligned) on stream
// with `grid` workgroups of 256 lanes (0: one vector per lane, as many
// workgroups as that takes, at most 2^24).  Returns a hipError_t.
int lso_probe_copy(const void* src, void* dst, uint64_t bytes, unsigned grid, void* stream)
{
    if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return static_cast<int>(hipErrorInvalidValue);
    if (bytes == 0) return 0;
    if (grid == 0) {
        const uint64_t want = (bytes / 16 + 255) / 256;
        grid = static_cast<unsigned>(want < (1ull << 24) ? want : (1ull << 24));
    }
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return static_cast<int>(hipGetLastError());
}

// out[i] = BF16 RNE of the FP32 pattern first + i, for i < count
// (first + count <= 2^32).  Returns a hipError_t.
int lso_probe_bf16_rne(uint32_t first, uint64_t count, uint16_t* out, void* stream)
{
    if (count == 0) return 0;
    if (static_cast<uint64_t>(first) + count > (uint64_t(1) << 32) || !out)
        return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(bf16_probe_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                       first, count, out);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
