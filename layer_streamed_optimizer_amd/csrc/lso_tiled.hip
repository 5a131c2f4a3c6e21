// Conversions between planar FP32 master/m/v arrays and the tiled state
// region (tiles of LSO_TILE_ELEMS elements, [master | m | v] per tile).
// One element per lane, grid-stride; bounded by n on both sides.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lso_runtime.h"

namespace lso {
namespace {

constexpr uint64_t kT = LSO_TILE_ELEMS;

__device__ __forceinline__ uint64_t tiled_index(uint64_t i, int which)
{
    // element i, array `which` (0 master, 1 m, 2 v) inside the region
    return (i / kT) * 3 * kT + static_cast<uint64_t>(which) * kT + (i % kT);
}

__global__ void __launch_bounds__(256)
pack_kernel(float* __restrict__ state, const float* __restrict__ master, const float* __restrict__ m,
            const float* __restrict__ v, uint64_t n)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        state[tiled_index(i, 0)] = master[i];
        state[tiled_index(i, 1)] = m ? m[i] : 0.0f;
        state[tiled_index(i, 2)] = v ? v[i] : 0.0f;
    }
}

__global__ void __launch_bounds__(256)
unpack_kernel(const float* __restrict__ state, float* __restrict__ master, float* __restrict__ m,
              float* __restrict__ v, uint64_t n)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (master) master[i] = state[tiled_index(i, 0)];
        if (m) m[i] = state[tiled_index(i, 1)];
        if (v) v[i] = state[tiled_index(i, 2)];
    }
}

unsigned grid_for(uint64_t n)
{
    const uint64_t want = (n + 255) / 256;
    return static_cast<unsigned>(want < 8192 ? (want ? want : 1) : 8192);
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace
}  // namespace lso

extern "C" {

lso_status lso_tiled_pack(void* state, const float* master, const float* m, const float* v, uint64_t n,
                          void* stream)
{
    lso::clear_error();
    if (n == 0) return LSO_OK;
    if (!state || !master) return lso::fail(LSO_E_INVALID, "state and master must be non-NULL");
    if (!lso::aligned16(state) || !lso::aligned16(master) || (m && !lso::aligned16(m)) ||
        (v && !lso::aligned16(v)))
        return lso::fail(LSO_E_ALIGN, "arrays must be 16-byte aligned");
    hipLaunchKernelGGL(lso::pack_kernel, dim3(lso::grid_for(n)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<float*>(state), master, m, v, n);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? LSO_OK : lso::hip_fail(err, "tiled pack launch");
}

lso_status lso_tiled_unpack(const void* state, float* master, float* m, float* v, uint64_t n, void* stream)
{
    lso::clear_error();
    if (n == 0) return LSO_OK;
    if (!state) return lso::fail(LSO_E_INVALID, "state must be non-NULL");
    if (!lso::aligned16(state) || (master && !lso::aligned16(master)) || (m && !lso::aligned16(m)) ||
        (v && !lso::aligned16(v)))
        return lso::fail(LSO_E_ALIGN, "arrays must be 16-byte aligned");
    hipLaunchKernelGGL(lso::unpack_kernel, dim3(lso::grid_for(n)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float*>(state), master, m, v, n);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? LSO_OK : lso::hip_fail(err, "tiled unpack launch");
}

}  // extern "C"
