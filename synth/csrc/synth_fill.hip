// Seeded synthetic inputs, device side (gfx950).
//
// Holds none of the optimizer's arithmetic.  Independent implementation of
// the generator that synth_host.c implements for the host: Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, SC'11) keyed by (seed, stream) with counter
// (index lo, index hi, block, purpose<<24 | step); the centred Irwin-Hall sum
// of the eight 16-bit halves of one output, times one FP32 scale, is the
// normal deviate; BF16 values are the truncated upper half of that pattern.
// Integer work plus one correctly rounded FP32 multiply, so host and device
// agree bit for bit (checked by a GPU test).
//
// The gradient callback below fills one layer's BF16 gradient buffer on the
// compute stream; it stands in for the backward pass of that layer.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

__device__ __forceinline__ int32_t centred_ih8(uint64_t index, uint32_t seed, uint32_t stream,
                                               uint32_t block, uint32_t ctr3)
{
    uint32_t c0 = static_cast<uint32_t>(index), c1 = static_cast<uint32_t>(index >> 32);
    uint32_t c2 = block, c3 = ctr3;
    uint32_t k0 = seed, k1 = stream;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
        const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += kW0; k1 += kW1;
    }
    const int32_t s = static_cast<int32_t>((c0 & 0xFFFFu) + (c0 >> 16) + (c1 & 0xFFFFu) + (c1 >> 16) +
                                           (c2 & 0xFFFFu) + (c2 >> 16) + (c3 & 0xFFFFu) + (c3 >> 16));
    return s - 262140;
}

__global__ void __launch_bounds__(256)
fill_normal_f32_kernel(float* __restrict__ out, uint64_t n, uint64_t i0, uint32_t seed,
                       uint32_t stream, uint32_t block, uint32_t ctr3, float scale)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += stride) {
        const int32_t x = centred_ih8(i0 + k, seed, stream, block, ctr3);
        out[k] = __fmul_rn(static_cast<float>(x), scale);
    }
}

__global__ void __launch_bounds__(256)
fill_normal_bf16_kernel(uint16_t* __restrict__ out, uint64_t n, uint64_t i0, uint32_t seed,
                        uint32_t stream, uint32_t block, uint32_t ctr3, float scale)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += stride) {
        const int32_t x = centred_ih8(i0 + k, seed, stream, block, ctr3);
        const float f = __fmul_rn(static_cast<float>(x), scale);
        out[k] = static_cast<uint16_t>(__float_as_uint(f) >> 16);
    }
}

__global__ void __launch_bounds__(256)
fill_zero_kernel(uint4* __restrict__ out16, uint64_t n16, unsigned char* __restrict__ tail, uint64_t ntail)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    const uint64_t first = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (uint64_t k = first; k < n16; k += stride) out16[k] = make_uint4(0u, 0u, 0u, 0u);
    if (first < ntail) tail[first] = 0;
}

unsigned grid_for(uint64_t n)
{
    const uint64_t want = (n + 255) / 256;
    const uint64_t cap = 256ull * 32ull;   // 32 workgroups per CU is plenty for a fill
    return static_cast<unsigned>(want < 1 ? 1 : (want > cap ? cap : want));
}

uint32_t ctr3_of(uint32_t purpose, uint32_t step) { return (purpose << 24) | (step & 0x00FFFFFFu); }

}  // namespace

extern "C" {

// Fill out[0..n) with deviates for indices start..start+n-1.  Async on stream.
// Returns 0, or the hipError_t of the launch.
int synth_fill_normal_f32(float* out, uint64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                          uint32_t block, uint32_t purpose, uint32_t step, float scale, hipStream_t s)
{
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_normal_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, start,
                       seed, stream, block, ctr3_of(purpose, step), scale);
    return static_cast<int>(hipGetLastError());
}

int synth_fill_normal_bf16(uint16_t* out, uint64_t n, uint64_t start, uint32_t seed, uint32_t stream,
                           uint32_t block, uint32_t purpose, uint32_t step, float scale, hipStream_t s)
{
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_normal_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, start,
                       seed, stream, block, ctr3_of(purpose, step), scale);
    return static_cast<int>(hipGetLastError());
}

// Zero nbytes at ptr with a kernel (kept out of memset so it can sit in a
// captured graph).  ptr must be 16-byte aligned.
int synth_fill_zero(void* ptr, uint64_t nbytes, hipStream_t s)
{
    if (nbytes == 0) return 0;
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
    const uint64_t n16 = nbytes / 16, ntail = nbytes % 16;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16 > ntail ? n16 : ntail)), dim3(256), 0, s,
                       static_cast<uint4*>(ptr), n16, static_cast<unsigned char*>(ptr) + n16 * 16, ntail);
    return static_cast<int>(hipGetLastError());
}

struct synth_fill_params {
    uint32_t seed, stream, purpose, step;
    float scale;
    uint32_t block_base;
};

// Gradient producer for a layer stream: fills layer `layer`'s BF16 gradient
// buffer (n elements) with the deviates of block block_base + layer at the
// step in params.  Enqueue only; never synchronises.
int synth_grad_fn(void* user, size_t layer, void* dev_grad_bf16, uint64_t n, hipStream_t s)
{
    const synth_fill_params* p = static_cast<const synth_fill_params*>(user);
    if (!p || !dev_grad_bf16) return 1;
    return synth_fill_normal_bf16(static_cast<uint16_t*>(dev_grad_bf16), n, 0, p->seed, p->stream,
                                  p->block_base + static_cast<uint32_t>(layer), p->purpose, p->step,
                                  p->scale, s) == 0 ? 0 : 6;
}

// The same producer for layers whose gradients are FP32: the deviates before
// their BF16 rounding (synth_fill_normal_f32 with the same counters).
int synth_grad_fn_f32(void* user, size_t layer, void* dev_grad_f32, uint64_t n, hipStream_t s)
{
    const synth_fill_params* p = static_cast<const synth_fill_params*>(user);
    if (!p || !dev_grad_f32) return 1;
    return synth_fill_normal_f32(static_cast<float*>(dev_grad_f32), n, 0, p->seed, p->stream,
                                 p->block_base + static_cast<uint32_t>(layer), p->purpose, p->step,
                                 p->scale, s) == 0 ? 0 : 6;
}

}  // extern "C"
