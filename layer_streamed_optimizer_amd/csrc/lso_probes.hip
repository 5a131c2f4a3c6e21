// Measurement and verification probes (not part of the update path).
//
//  lso_probe_copy      plain 16-byte-vector device copy: the HBM ceiling a
//                      read+write stream reaches, and the reference for
//                      scaling the FETCH_SIZE / WRITE_SIZE counters.
//  lso_probe_copy_shaped  the update's memory access pattern with no
//                      arithmetic: per element 2 + 12 bytes read, 12 + 2
//                      written, in the planar or tiled state layout, one
//                      1,024-element chunk per workgroup -- the ceiling of
//                      the update's own traffic shape.
//  lso_probe_copy_variant  other shapes of the same 1:1 read/write
//                      stream (direct-to-LDS loads with a read phase and a
//                      write phase per workgroup, several vectors in flight
//                      per lane, cache-policy bits, in-place, read-only and
//                      write-only streams), to find the part's ceiling for
//                      the update's traffic
//  lso_probe_link_mode / lso_probe_link_sdma  host-link rates, each
//                      direction alone and both at once, per copy engine
//  lso_probe_bf16_rne  the fused kernel's BF16 rounding applied to a range
//                      of FP32 bit patterns, so a test can compare it with
//                      the host definition over all 2^32 patterns.
//  lso_probe_sqrt      the fused kernel's FP32 square root (__builtin_sqrtf
//                      under the same build flags) over a range of bit
//                      patterns, for an exhaustive check of its rounding.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>

#include "lso_bf16.h"
#include "lso_sdma.h"

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

// Copy between page-locked host memory and device memory by the shader
// cores (PCIe reads or writes issued by the kernel itself).
__global__ void __launch_bounds__(256)
link_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint64_t n16)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T ld_nt(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p)));
}

template <typename T>
__device__ __forceinline__ void st_nt(void* p, T v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p)));
}

constexpr uint32_t kShapedChunk = 1024;   // elements per workgroup: 256 lanes x 4
constexpr uint32_t kShapedTile = 8192;    // elements per state tile

// Each lane reads four BF16 "gradients" and four FP32 each of master, m and
// v, and writes the three FP32 quads back in place (bits mixed so nothing
// is a no-op) and four BF16 "weights".
template <bool kTiled>
__global__ void __launch_bounds__(256)
shaped_copy_kernel(float* __restrict__ state, const uint16_t* __restrict__ grad,
                   uint16_t* __restrict__ weight, uint64_t n)
{
    const uint64_t e0 = static_cast<uint64_t>(blockIdx.x) * kShapedChunk;
    float *p, *m, *v;
    if (kTiled) {
        p = state + 3 * (e0 / kShapedTile) * kShapedTile + e0 % kShapedTile;
        m = p + kShapedTile;
        v = m + kShapedTile;
    } else {
        p = state + e0;
        m = state + n + e0;
        v = state + 2 * n + e0;
    }
    const uint32_t i = threadIdx.x * 4;
    const u32x2 g = ld_nt<u32x2>(grad + e0 + i);
    f32x4 a = ld_nt<f32x4>(p + i), b = ld_nt<f32x4>(m + i), c = ld_nt<f32x4>(v + i);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    u32x4v ai = __builtin_bit_cast(u32x4v, a) ^ g.x, bi = __builtin_bit_cast(u32x4v, b) ^ g.y;
    u32x4v ci = __builtin_bit_cast(u32x4v, c) ^ (g.x + g.y);
    st_nt<f32x4>(p + i, __builtin_bit_cast(f32x4, ai));
    st_nt<f32x4>(m + i, __builtin_bit_cast(f32x4, bi));
    st_nt<f32x4>(v + i, __builtin_bit_cast(f32x4, ci));
    const u32x2 w = {(ai.x >> 16) | (ai.y & 0xFFFF0000u), (ai.z >> 16) | (ai.w & 0xFFFF0000u)};
    st_nt<u32x2>(weight + e0 + i, w);
}

// ---- copy variants (lso_probe_copy_variant) ----

#define LSO_LDS __attribute__((address_space(3)))

// Read phase then write phase per workgroup: the workgroup's KB kilobytes
// are loaded straight into LDS (global_load_lds_dwordx4: no VGPRs held by
// the loads, so all of them are in flight at once), then written out from
// LDS.  Lane t of wave w's load k lands at LDS vector k*256 + w*64 + t.
template <int KB>
__global__ void __launch_bounds__(256)
copy_lds_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst)
{
    constexpr int kVec = KB * 1024 / 16;   // vectors per workgroup
    constexpr int kPer = kVec / 256;       // per lane
    __shared__ u32x4 buf[kVec];
    const uint64_t base = static_cast<uint64_t>(blockIdx.x) * kVec;
    const int wave0 = threadIdx.x & ~63;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const u32x4* s = src + base + k * 256 + threadIdx.x;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const LSO_GLOBAL void*>(reinterpret_cast<uintptr_t>(s)),
                                         (LSO_LDS void*)(&buf[k * 256 + wave0]), 16, 0, 2 /* nt */);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        st_nt<u32x4>(dst + base + k * 256 + threadIdx.x, buf[k * 256 + threadIdx.x]);
}

// P vectors per lane: all P loads, then all P stores (a workgroup covers
// 256 * P consecutive vectors, lane-interleaved).
template <int P>
__global__ void __launch_bounds__(256)
copy_regs_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst)
{
    const uint64_t base = static_cast<uint64_t>(blockIdx.x) * 256 * P;
    u32x4 x[P];
#pragma unroll
    for (int k = 0; k < P; ++k) x[k] = ld_nt<u32x4>(src + base + k * 256 + threadIdx.x);
#pragma unroll
    for (int k = 0; k < P; ++k) st_nt<u32x4>(dst + base + k * 256 + threadIdx.x, x[k]);
}

// One vector per lane with the cache-policy bits of the load (L) and the
// store (S): 0 none, 1 nt, 2 sc1, 3 nt sc1, 4 sc0 sc1, 5 sc0 sc1 nt.  Every
// inline-assembly store ends with s_nop 0: the compiler cannot see the wait
// state a store's data registers need before a vector-ALU write to them.
#define LSO_CPOL_LOAD(ms) \
    asm volatile("global_load_dwordx4 %0, %1, off " ms "\n\ts_waitcnt vmcnt(0)" : "=v"(x) : "v"(s) : "memory")
#define LSO_CPOL_STORE(ms) asm volatile("global_store_dwordx4 %0, %1, off " ms "\n\ts_nop 0" : : "v"(d), "v"(x) : "memory")

template <int L, int S>
__global__ void __launch_bounds__(256)
copy_cpol_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst)
{
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    const LSO_GLOBAL u32x4* s = reinterpret_cast<const LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(src + i));
    LSO_GLOBAL u32x4* d = reinterpret_cast<LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(dst + i));
    u32x4 x;
    if (L == 0) LSO_CPOL_LOAD("");
    else if (L == 1) LSO_CPOL_LOAD("nt");
    else if (L == 2) LSO_CPOL_LOAD("sc1");
    else if (L == 3) LSO_CPOL_LOAD("nt sc1");
    else if (L == 4) LSO_CPOL_LOAD("sc0 sc1");
    else LSO_CPOL_LOAD("sc0 sc1 nt");
    if (S == 0) LSO_CPOL_STORE("");
    else if (S == 1) LSO_CPOL_STORE("nt");
    else if (S == 2) LSO_CPOL_STORE("sc1");
    else if (S == 3) LSO_CPOL_STORE("nt sc1");
    else if (S == 4) LSO_CPOL_STORE("sc0 sc1");
    else LSO_CPOL_STORE("sc0 sc1 nt");
}

// The update's tiled traffic shape (shaped_copy_kernel<true>) with the
// cache-policy bits S of its stores (as copy_cpol_kernel's).
#define LSO_CPOL_ST16(ms, addr, val) asm volatile("global_store_dwordx4 %0, %1, off " ms "\n\ts_nop 0" : : "v"(addr), "v"(val) : "memory")
#define LSO_CPOL_ST8(ms, addr, val) asm volatile("global_store_dwordx2 %0, %1, off " ms "\n\ts_nop 0" : : "v"(addr), "v"(val) : "memory")

template <int S>
__device__ __forceinline__ void st16_cpol(float* p, f32x4 x)
{
    LSO_GLOBAL f32x4* a = reinterpret_cast<LSO_GLOBAL f32x4*>(reinterpret_cast<uintptr_t>(p));
    if (S == 0) LSO_CPOL_ST16("", a, x);
    else if (S == 1) LSO_CPOL_ST16("nt", a, x);
    else if (S == 2) LSO_CPOL_ST16("sc1", a, x);
    else if (S == 3) LSO_CPOL_ST16("nt sc1", a, x);
    else if (S == 4) LSO_CPOL_ST16("sc0 sc1", a, x);
    else LSO_CPOL_ST16("sc0 sc1 nt", a, x);
}

template <int S>
__device__ __forceinline__ void st8_cpol(uint16_t* p, u32x2 x)
{
    LSO_GLOBAL u32x2* a = reinterpret_cast<LSO_GLOBAL u32x2*>(reinterpret_cast<uintptr_t>(p));
    if (S == 0) LSO_CPOL_ST8("", a, x);
    else if (S == 1) LSO_CPOL_ST8("nt", a, x);
    else if (S == 2) LSO_CPOL_ST8("sc1", a, x);
    else if (S == 3) LSO_CPOL_ST8("nt sc1", a, x);
    else if (S == 4) LSO_CPOL_ST8("sc0 sc1", a, x);
    else LSO_CPOL_ST8("sc0 sc1 nt", a, x);
}

template <int S>
__global__ void __launch_bounds__(256)
shaped_cpol_kernel(float* __restrict__ state, const uint16_t* __restrict__ grad, uint16_t* __restrict__ weight)
{
    const uint64_t e0 = static_cast<uint64_t>(blockIdx.x) * kShapedChunk;
    float* p = state + 3 * (e0 / kShapedTile) * kShapedTile + e0 % kShapedTile;
    float* m = p + kShapedTile;
    float* v = m + kShapedTile;
    const uint32_t i = threadIdx.x * 4;
    const u32x2 g = ld_nt<u32x2>(grad + e0 + i);
    f32x4 a = ld_nt<f32x4>(p + i), b = ld_nt<f32x4>(m + i), c = ld_nt<f32x4>(v + i);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    u32x4v ai = __builtin_bit_cast(u32x4v, a) ^ g.x, bi = __builtin_bit_cast(u32x4v, b) ^ g.y;
    u32x4v ci = __builtin_bit_cast(u32x4v, c) ^ (g.x + g.y);
    st16_cpol<S>(p + i, __builtin_bit_cast(f32x4, ai));
    st16_cpol<S>(m + i, __builtin_bit_cast(f32x4, bi));
    st16_cpol<S>(v + i, __builtin_bit_cast(f32x4, ci));
    const u32x2 w = {(ai.x >> 16) | (ai.y & 0xFFFF0000u), (ai.z >> 16) | (ai.w & 0xFFFF0000u)};
    st8_cpol<S>(weight + e0 + i, w);
}

// In place: every vector read and written back to the same address (bits
// flipped), as the update does with its state.
__global__ void __launch_bounds__(256)
inplace_kernel(u32x4* __restrict__ buf)
{
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    const u32x4 x = ld_nt<u32x4>(buf + i);
    st_nt<u32x4>(buf + i, ~x);
}

// In place with nt loads and the store cache-policy bits S (as
// copy_cpol_kernel's): the update's own state traffic, each vector read and
// written back to its address (bits flipped).
template <int S>
__global__ void __launch_bounds__(256)
inplace_cpol_kernel(u32x4* __restrict__ buf)
{
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    const LSO_GLOBAL u32x4* s = reinterpret_cast<const LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(buf + i));
    LSO_GLOBAL u32x4* d = reinterpret_cast<LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(buf + i));
    u32x4 x;
    LSO_CPOL_LOAD("nt");
    x = ~x;
    if (S == 0) LSO_CPOL_STORE("");
    else if (S == 1) LSO_CPOL_STORE("nt");
    else if (S == 2) LSO_CPOL_STORE("sc1");
    else if (S == 3) LSO_CPOL_STORE("nt sc1");
    else if (S == 4) LSO_CPOL_STORE("sc0 sc1");
    else LSO_CPOL_STORE("sc0 sc1 nt");
}

// One W-byte vector per lane (W = 4, 8 or 16), nt loads and nt sc1 stores
// (the update's bits): how the access width alone moves the stream.
template <int W>
__global__ void __launch_bounds__(256)
copy_width_kernel(const char* __restrict__ src, char* __restrict__ dst)
{
    const uint64_t off = (static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x) * W;
    if (W == 16) {
        const u32x4 x = ld_nt<u32x4>(src + off);
        LSO_GLOBAL u32x4* d = reinterpret_cast<LSO_GLOBAL u32x4*>(reinterpret_cast<uintptr_t>(dst + off));
        asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 0" : : "v"(d), "v"(x) : "memory");
    } else if (W == 8) {
        const u32x2 x = ld_nt<u32x2>(src + off);
        LSO_GLOBAL u32x2* d = reinterpret_cast<LSO_GLOBAL u32x2*>(reinterpret_cast<uintptr_t>(dst + off));
        asm volatile("global_store_dwordx2 %0, %1, off nt sc1\n\ts_nop 0" : : "v"(d), "v"(x) : "memory");
    } else {
        const uint32_t x = ld_nt<uint32_t>(src + off);
        LSO_GLOBAL uint32_t* d = reinterpret_cast<LSO_GLOBAL uint32_t*>(reinterpret_cast<uintptr_t>(dst + off));
        asm volatile("global_store_dword %0, %1, off nt sc1\n\ts_nop 0" : : "v"(d), "v"(x) : "memory");
    }
}

// Read-only: every vector read; one word per workgroup written so the
// loads stay.
__global__ void __launch_bounds__(256)
read_only_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink)
{
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    const u32x4 x = ld_nt<u32x4>(src + i);
    const uint32_t r = x.x ^ x.y ^ x.z ^ x.w;
    if (r == 0x9E3779B9u) sink[blockIdx.x] = r;   // practically never
}

// Write-only: every vector written.
__global__ void __launch_bounds__(256)
write_only_kernel(u32x4* __restrict__ dst)
{
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    const uint32_t v = static_cast<uint32_t>(i);
    st_nt<u32x4>(dst + i, u32x4{v, v, v, v});
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

__global__ void __launch_bounds__(256)
sqrt_probe_kernel(uint32_t first, uint64_t count, float* __restrict__ out)
{
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
        out[i] = __builtin_sqrtf(__uint_as_float(first + static_cast<uint32_t>(i)));
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

// The update's traffic shape with no arithmetic, over n elements (a
// multiple of 8192, at most 2^34): state is 12n bytes (planar: master, m,
// v arrays of n FP32 back to back; tiled: 8192-element [master|m|v] tiles),
// grad and weight n BF16 each; all 16-byte aligned.  State and weight are
// overwritten with mixed bits.  Returns a hipError_t.
int lso_probe_copy_shaped(void* state, const void* grad, void* weight, uint64_t n, int tiled, void* stream)
{
    if (n % kShapedTile != 0 || n > (uint64_t(1) << 34) || !state || !grad || !weight ||
        reinterpret_cast<uintptr_t>(state) % 16 != 0 || reinterpret_cast<uintptr_t>(grad) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(weight) % 16 != 0)
        return static_cast<int>(hipErrorInvalidValue);
    if (n == 0) return 0;
    const dim3 grid(static_cast<unsigned>(n / kShapedChunk));
    auto* st = static_cast<float*>(state);
    auto* g = static_cast<const uint16_t*>(grad);
    auto* w = static_cast<uint16_t*>(weight);
    if (tiled)
        hipLaunchKernelGGL(shaped_copy_kernel<true>, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           st, g, w, n);
    else
        hipLaunchKernelGGL(shaped_copy_kernel<false>, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           st, g, w, n);
    return static_cast<int>(hipGetLastError());
}

// One variant of the device copy of lso_probe_copy over `bytes` (a multiple
// of 64 KiB; src and dst 16-byte aligned, not overlapping, at most 2^36
// bytes), one chunk per workgroup, no grid loop:
//   0  one vector per lane, nt load and store (lso_probe_copy's shape)
//   1  direct-to-LDS read phase, then write phase; param = KB per workgroup
//      (4, 8, 16, 32 or 64)
//   2  param vectors per lane in registers (1, 2, 4 or 8)
//   3  cache-policy bits: param = load policy + 8 * store policy (0..5 each,
//      see copy_cpol_kernel)
//   4  in place over src (dst unused): read and write the same addresses
//   5  read-only over src (dst receives at most a few words)
//   6  write-only over dst
//   7  in place over src with nt loads; param = store policy (0..5, see
//      copy_cpol_kernel)
//   8  param bytes (4, 8 or 16) per lane, nt loads, nt sc1 stores
// Returns a hipError_t (hipErrorInvalidValue for a bad variant, param or
// size).
int lso_probe_copy_variant(int variant, int param, const void* src, void* dst, uint64_t bytes, void* stream)
{
    if (bytes == 0 || bytes % (64 << 10) != 0 || bytes > (uint64_t(1) << 36) || !src || !dst ||
        reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return static_cast<int>(hipErrorInvalidValue);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const auto* s = static_cast<const u32x4*>(src);
    auto* d = static_cast<u32x4*>(dst);
    const uint64_t n16 = bytes / 16;
    const dim3 t(256);
    const unsigned g1 = static_cast<unsigned>(n16 / 256);   // one vector per lane
    switch (variant) {
    case 0: hipLaunchKernelGGL(copy_kernel, dim3(g1), t, 0, st, s, d, n16); break;
    case 1:
        switch (param) {
        case 4: hipLaunchKernelGGL(copy_lds_kernel<4>, dim3(bytes / (4 << 10)), t, 0, st, s, d); break;
        case 8: hipLaunchKernelGGL(copy_lds_kernel<8>, dim3(bytes / (8 << 10)), t, 0, st, s, d); break;
        case 16: hipLaunchKernelGGL(copy_lds_kernel<16>, dim3(bytes / (16 << 10)), t, 0, st, s, d); break;
        case 32: hipLaunchKernelGGL(copy_lds_kernel<32>, dim3(bytes / (32 << 10)), t, 0, st, s, d); break;
        case 64: hipLaunchKernelGGL(copy_lds_kernel<64>, dim3(bytes / (64 << 10)), t, 0, st, s, d); break;
        default: return static_cast<int>(hipErrorInvalidValue);
        }
        break;
    case 2:
        switch (param) {
        case 1: hipLaunchKernelGGL(copy_regs_kernel<1>, dim3(g1), t, 0, st, s, d); break;
        case 2: hipLaunchKernelGGL(copy_regs_kernel<2>, dim3(g1 / 2), t, 0, st, s, d); break;
        case 4: hipLaunchKernelGGL(copy_regs_kernel<4>, dim3(g1 / 4), t, 0, st, s, d); break;
        case 8: hipLaunchKernelGGL(copy_regs_kernel<8>, dim3(g1 / 8), t, 0, st, s, d); break;
        default: return static_cast<int>(hipErrorInvalidValue);
        }
        break;
    case 3: {
        const int L = param % 8, S = param / 8;
        if (L > 5 || S > 5 || param < 0) return static_cast<int>(hipErrorInvalidValue);
#define LSO_CPOL_CASE(l, s_) \
    if (L == l && S == s_) hipLaunchKernelGGL((copy_cpol_kernel<l, s_>), dim3(g1), t, 0, st, s, d)
#define LSO_CPOL_ROW(l) \
    LSO_CPOL_CASE(l, 0); LSO_CPOL_CASE(l, 1); LSO_CPOL_CASE(l, 2); LSO_CPOL_CASE(l, 3); LSO_CPOL_CASE(l, 4); \
    LSO_CPOL_CASE(l, 5)
        LSO_CPOL_ROW(0); LSO_CPOL_ROW(1); LSO_CPOL_ROW(2); LSO_CPOL_ROW(3); LSO_CPOL_ROW(4); LSO_CPOL_ROW(5);
#undef LSO_CPOL_ROW
#undef LSO_CPOL_CASE
        break;
    }
    case 4: hipLaunchKernelGGL(inplace_kernel, dim3(g1), t, 0, st, const_cast<u32x4*>(s)); break;
    case 5: hipLaunchKernelGGL(read_only_kernel, dim3(g1), t, 0, st, s, static_cast<uint32_t*>(dst)); break;
    case 6: hipLaunchKernelGGL(write_only_kernel, dim3(g1), t, 0, st, d); break;
    case 7: {
        auto* b = const_cast<u32x4*>(s);
        switch (param) {
        case 0: hipLaunchKernelGGL(inplace_cpol_kernel<0>, dim3(g1), t, 0, st, b); break;
        case 1: hipLaunchKernelGGL(inplace_cpol_kernel<1>, dim3(g1), t, 0, st, b); break;
        case 2: hipLaunchKernelGGL(inplace_cpol_kernel<2>, dim3(g1), t, 0, st, b); break;
        case 3: hipLaunchKernelGGL(inplace_cpol_kernel<3>, dim3(g1), t, 0, st, b); break;
        case 4: hipLaunchKernelGGL(inplace_cpol_kernel<4>, dim3(g1), t, 0, st, b); break;
        case 5: hipLaunchKernelGGL(inplace_cpol_kernel<5>, dim3(g1), t, 0, st, b); break;
        default: return static_cast<int>(hipErrorInvalidValue);
        }
        break;
    }
    case 8: {
        const auto* cs = static_cast<const char*>(src);
        auto* cd = static_cast<char*>(dst);
        switch (param) {
        case 4: hipLaunchKernelGGL(copy_width_kernel<4>, dim3(bytes / 1024), t, 0, st, cs, cd); break;
        case 8: hipLaunchKernelGGL(copy_width_kernel<8>, dim3(bytes / 2048), t, 0, st, cs, cd); break;
        case 16: hipLaunchKernelGGL(copy_width_kernel<16>, dim3(bytes / 4096), t, 0, st, cs, cd); break;
        default: return static_cast<int>(hipErrorInvalidValue);
        }
        break;
    }
    default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

// The tiled update-shaped copy of lso_probe_copy_shaped with the store
// cache-policy bits `store_cpol` (0 none, 1 nt, 2 sc1, 3 nt sc1, 4 sc0 sc1,
// 5 sc0 sc1 nt); same buffer rules.  Returns a hipError_t.
int lso_probe_copy_shaped_cpol(void* state, const void* grad, void* weight, uint64_t n, int store_cpol,
                               void* stream)
{
    if (n % kShapedTile != 0 || n > (uint64_t(1) << 34) || !state || !grad || !weight || store_cpol < 0 ||
        store_cpol > 5 || reinterpret_cast<uintptr_t>(state) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(grad) % 16 != 0 || reinterpret_cast<uintptr_t>(weight) % 16 != 0)
        return static_cast<int>(hipErrorInvalidValue);
    if (n == 0) return 0;
    const dim3 grid(static_cast<unsigned>(n / kShapedChunk));
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* sp = static_cast<float*>(state);
    auto* g = static_cast<const uint16_t*>(grad);
    auto* w = static_cast<uint16_t*>(weight);
    switch (store_cpol) {
    case 0: hipLaunchKernelGGL(shaped_cpol_kernel<0>, grid, dim3(256), 0, st, sp, g, w); break;
    case 1: hipLaunchKernelGGL(shaped_cpol_kernel<1>, grid, dim3(256), 0, st, sp, g, w); break;
    case 2: hipLaunchKernelGGL(shaped_cpol_kernel<2>, grid, dim3(256), 0, st, sp, g, w); break;
    case 3: hipLaunchKernelGGL(shaped_cpol_kernel<3>, grid, dim3(256), 0, st, sp, g, w); break;
    case 4: hipLaunchKernelGGL(shaped_cpol_kernel<4>, grid, dim3(256), 0, st, sp, g, w); break;
    default: hipLaunchKernelGGL(shaped_cpol_kernel<5>, grid, dim3(256), 0, st, sp, g, w); break;
    }
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

// out[i] = FP32 square root of the pattern first + i, for i < count
// (first + count <= 2^32).  Returns a hipError_t.
int lso_probe_sqrt(uint32_t first, uint64_t count, float* out, void* stream)
{
    if (count == 0) return 0;
    if (static_cast<uint64_t>(first) + count > (uint64_t(1) << 32) || !out)
        return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(sqrt_probe_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                       first, count, out);
    return static_cast<int>(hipGetLastError());
}

// Host-link rates with page-locked buffers of `bytes` each: out[0] H2D
// alone, out[1] D2H alone, out[2] H2D and out[3] D2H while both run at once
// on two streams (best of `reps`), in GB/s.  mode selects the copy engine
// per direction: bit 0 set = H2D by a copy kernel (else DMA engine), bit 1
// set = D2H by a copy kernel; grid = workgroups of such a kernel.
// Returns a hipError_t.
int lso_probe_link_mode(uint64_t bytes, int reps, int mode, unsigned grid, double out[4]);

// The same four rates with the layer stream's default engines: H2D and
// D2H on the two SDMA engines lso::sdma_open names (engines[0], engines[1]
// get their masks).  Returns a hipError_t, or -1 if the engines cannot be
// named, -2 if a copy fails.
int lso_probe_link_sdma(uint64_t bytes, int reps, uint32_t engines[2], double out[4]);

int lso_probe_link(uint64_t bytes, int reps, double out[4])
{
    return lso_probe_link_mode(bytes, reps, 0, 0, out);
}

int lso_probe_link_mode(uint64_t bytes, int reps, int mode, unsigned grid, double out[4])
{
    if (bytes % 16 != 0 || bytes == 0) return static_cast<int>(hipErrorInvalidValue);
    if (grid == 0) grid = 256;
    void *h1 = nullptr, *h2 = nullptr, *d1 = nullptr, *d2 = nullptr;
    hipStream_t s1 = nullptr, s2 = nullptr;
    hipError_t err = hipSuccess;
    auto now = [] { return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count(); };
    auto best = [&](auto fn) {
        double b = 1e30;
        for (int r = 0; r < reps && err == hipSuccess; ++r) {
            if ((err = hipDeviceSynchronize()) != hipSuccess) break;
            const double t0 = now();
            fn();
            if ((err = hipDeviceSynchronize()) != hipSuccess) break;
            const double dt = now() - t0;
            b = dt < b ? dt : b;
        }
        return b;
    };
    if ((err = hipHostMalloc(&h1, bytes, hipHostMallocDefault)) != hipSuccess) goto done;
    if ((err = hipHostMalloc(&h2, bytes, hipHostMallocDefault)) != hipSuccess) goto done;
    if ((err = hipMalloc(&d1, bytes)) != hipSuccess) goto done;
    if ((err = hipMalloc(&d2, bytes)) != hipSuccess) goto done;
    if ((err = hipStreamCreateWithFlags(&s1, hipStreamNonBlocking)) != hipSuccess) goto done;
    if ((err = hipStreamCreateWithFlags(&s2, hipStreamNonBlocking)) != hipSuccess) goto done;
    {
        auto h2d = [&] {
            if (mode & 1) {
                hipLaunchKernelGGL(link_copy_kernel, dim3(grid), dim3(256), 0, s1,
                                   static_cast<const u32x4*>(h1), static_cast<u32x4*>(d1), bytes / 16);
                err = hipGetLastError();
            } else {
                err = hipMemcpyAsync(d1, h1, bytes, hipMemcpyHostToDevice, s1);
            }
        };
        auto d2h = [&] {
            if (mode & 2) {
                hipLaunchKernelGGL(link_copy_kernel, dim3(grid), dim3(256), 0, s2,
                                   static_cast<const u32x4*>(d2), static_cast<u32x4*>(h2), bytes / 16);
                err = hipGetLastError();
            } else {
                err = hipMemcpyAsync(h2, d2, bytes, hipMemcpyDeviceToHost, s2);
            }
        };
        const double th = best(h2d);
        const double td = best(d2h);
        // concurrent: time each direction by its own stream's completion
        double bh = 1e30, bd = 1e30;
        for (int r = 0; r < reps && err == hipSuccess; ++r) {
            if ((err = hipDeviceSynchronize()) != hipSuccess) break;
            const double t0 = now();
            h2d();
            if (err != hipSuccess) break;
            d2h();
            if (err != hipSuccess) break;
            double t1 = 0, t2 = 0;
            bool f1 = false, f2 = false;
            while (!(f1 && f2)) {
                if (!f1 && hipStreamQuery(s1) == hipSuccess) { f1 = true; t1 = now() - t0; }
                if (!f2 && hipStreamQuery(s2) == hipSuccess) { f2 = true; t2 = now() - t0; }
            }
            bh = t1 < bh ? t1 : bh;
            bd = t2 < bd ? t2 : bd;
        }
        if (err == hipSuccess) {
            out[0] = bytes / th / 1e9;
            out[1] = bytes / td / 1e9;
            out[2] = bytes / bh / 1e9;
            out[3] = bytes / bd / 1e9;
        }
    }
done:
    if (s1) (void)hipStreamDestroy(s1);
    if (s2) (void)hipStreamDestroy(s2);
    if (d1) (void)hipFree(d1);
    if (d2) (void)hipFree(d2);
    if (h1) (void)hipHostFree(h1);
    if (h2) (void)hipHostFree(h2);
    return static_cast<int>(err);
}

int lso_probe_link_sdma(uint64_t bytes, int reps, uint32_t engines[2], double out[4])
{
    if (bytes % 16 != 0 || bytes == 0) return static_cast<int>(hipErrorInvalidValue);
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return static_cast<int>(err);
    lso::SdmaLink link;
    if (!lso::sdma_open(dev, &link)) return -1;
    engines[0] = link.h2d_engine;
    engines[1] = link.d2h_engine;
    void *h1 = nullptr, *h2 = nullptr, *d1 = nullptr, *d2 = nullptr;
    hsa_signal_t sh{}, sd{};
    int rc = 0;
    auto now = [] { return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count(); };
    // the copies' completion times, from t0; false if a copy failed
    auto run = [&](bool in, bool outw, double t0, double& th, double& td) {
        if (in && lso::sdma_copy(link, d1, h1, bytes, true, nullptr, sh) != HSA_STATUS_SUCCESS) return false;
        if (outw && lso::sdma_copy(link, h2, d2, bytes, false, nullptr, sd) != HSA_STATUS_SUCCESS) {
            while (in && lso::sdma_state(sh) > 0) {}
            return false;
        }
        bool fh = !in, fd = !outw, ok = true;
        while (!(fh && fd)) {
            if (!fh) {
                const int64_t v = lso::sdma_state(sh);
                if (v <= 0) { fh = true; th = now() - t0; ok &= v == 0; }
            }
            if (!fd) {
                const int64_t v = lso::sdma_state(sd);
                if (v <= 0) { fd = true; td = now() - t0; ok &= v == 0; }
            }
        }
        return ok;
    };
    double bh1 = 1e30, bd1 = 1e30, bh = 1e30, bd = 1e30;
    if ((err = hipHostMalloc(&h1, bytes, hipHostMallocDefault)) != hipSuccess ||
        (err = hipHostMalloc(&h2, bytes, hipHostMallocDefault)) != hipSuccess ||
        (err = hipMalloc(&d1, bytes)) != hipSuccess || (err = hipMalloc(&d2, bytes)) != hipSuccess) {
        rc = static_cast<int>(err);
        goto done;
    }
    if (hsa_signal_create(0, 0, nullptr, &sh) != HSA_STATUS_SUCCESS ||
        hsa_signal_create(0, 0, nullptr, &sd) != HSA_STATUS_SUCCESS) {
        rc = -1;
        goto done;
    }
    for (int r = 0; r < reps && rc == 0; ++r) {
        double th = 0, td = 0;
        if (!run(true, false, now(), th, td)) { rc = -2; break; }
        bh1 = th < bh1 ? th : bh1;
        if (!run(false, true, now(), th, td)) { rc = -2; break; }
        bd1 = td < bd1 ? td : bd1;
        if (!run(true, true, now(), th, td)) { rc = -2; break; }
        bh = th < bh ? th : bh;
        bd = td < bd ? td : bd;
    }
    if (rc == 0) {
        out[0] = bytes / bh1 / 1e9;
        out[1] = bytes / bd1 / 1e9;
        out[2] = bytes / bh / 1e9;
        out[3] = bytes / bd / 1e9;
    }
done:
    if (sh.handle) (void)hsa_signal_destroy(sh);
    if (sd.handle) (void)hsa_signal_destroy(sd);
    if (d1) (void)hipFree(d1);
    if (d2) (void)hipFree(d2);
    if (h1) (void)hipHostFree(h1);
    if (h2) (void)hipHostFree(h2);
    lso::sdma_close(&link);
    return rc;
}

}  // extern "C"
