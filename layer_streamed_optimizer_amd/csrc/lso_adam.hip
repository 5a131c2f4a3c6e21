// Fused mixed-precision Adam for gfx950: one HBM pass per element.
//
// Per element (frozen-incremental page, section "The Math"; training-memory
// article, "Optimizer states"): read the BF16 gradient and the FP32 master,
// m and v; update the two moments; form the bias-corrected step with eps
// outside the root; add it to the master (the additive write-back); store
// master, m, v and the BF16 round-to-nearest-even re-cast of the new master.
// 14 bytes read + 14 bytes written per parameter and nothing else: no
// scratch, no second pass.
//
// Ragged multi-tensor launch: one grid walks the concatenated chunk space of
// every block of the call; a workgroup finds the block that owns its chunk by
// a uniform (scalar) binary search over the table's chunk starts.
//
// Built with -ffp-contract=off: every FMA below is an explicit fmaf, every
// other operator rounds once, so the SGD path is exactly fl(W + fl(-(lr*g))).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lso_bf16.h"
#include "lso_internal.h"

namespace lso {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Explicit address spaces: state arrays are global memory (so the compiler
// emits global_* rather than flat_* accesses), and the block table is
// read-only for the kernel's lifetime (constant space, scalar loads).
#define LSO_GLOBAL __attribute__((address_space(1)))
#define LSO_CONST __attribute__((address_space(4)))

template <typename T>
__device__ __forceinline__ T ld(const void* p)
{
    return *reinterpret_cast<const LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p));
}

template <typename T>
__device__ __forceinline__ void st(void* p, const T& v)
{
    *reinterpret_cast<LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p)) = v;
}

__device__ __forceinline__ void adam_elem(const Coef& c, float g, float& master, float& m, float& v)
{
    const float m1 = fmaf(c.b1, m, c.c1 * g);
    const float v1 = fmaf(c.b2, v, c.c2 * (g * g));   // g*g is exact: g has 8 significant bits
    const float den = fmaf(__fsqrt_rn(v1), c.r, c.e);  // sqrt(v_hat) + eps, v_hat = v1 * r^2
    const float delta = -__fdiv_rn(c.s * m1, den);
    master = master + delta;
    m = m1;
    v = v1;
}

__device__ __forceinline__ void sgd_elem(const Coef& c, float g, float& master)
{
    const float delta = -(c.s * g);
    master = master + delta;
}

// Eight consecutive elements held by one lane.
struct Group {
    u32x4 g;          // 8 BF16
    f32x4 p0, p1;     // master
    f32x4 m0, m1;
    f32x4 v0, v1;
};

template <bool kSgd>
__device__ __forceinline__ void load_group(const DevBlock& b, uint64_t e, Group& x)
{
    x.g = ld<u32x4>(b.g + e);
    x.p0 = ld<f32x4>(b.master + e);
    x.p1 = ld<f32x4>(b.master + e + 4);
    if (!kSgd) {
        x.m0 = ld<f32x4>(b.m + e);
        x.m1 = ld<f32x4>(b.m + e + 4);
        x.v0 = ld<f32x4>(b.v + e);
        x.v1 = ld<f32x4>(b.v + e + 4);
    }
}

template <bool kSgd>
__device__ __forceinline__ void compute_group(const Coef& c, Group& x, u32x4& wout)
{
    float gs[8], ps[8], ms[8], vs[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t word = x.g[k];
        gs[2 * k] = bf16_widen(word & 0xFFFFu);
        gs[2 * k + 1] = bf16_widen(word >> 16);
        ps[k] = x.p0[k];
        ps[k + 4] = x.p1[k];
        if (!kSgd) {
            ms[k] = x.m0[k];
            ms[k + 4] = x.m1[k];
            vs[k] = x.v0[k];
            vs[k + 4] = x.v1[k];
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (kSgd) sgd_elem(c, gs[k], ps[k]);
        else adam_elem(c, gs[k], ps[k], ms[k], vs[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x.p0[k] = ps[k];
        x.p1[k] = ps[k + 4];
        if (!kSgd) {
            x.m0[k] = ms[k];
            x.m1[k] = ms[k + 4];
            x.v0[k] = vs[k];
            x.v1[k] = vs[k + 4];
        }
        wout[k] = bf16_rne(ps[2 * k]) | (bf16_rne(ps[2 * k + 1]) << 16);
    }
}

template <bool kSgd>
__device__ __forceinline__ void store_group(const DevBlock& b, uint64_t e, const Group& x,
                                            const u32x4& wout, bool has_w)
{
    st<f32x4>(b.master + e, x.p0);
    st<f32x4>(b.master + e + 4, x.p1);
    if (!kSgd) {
        st<f32x4>(b.m + e, x.m0);
        st<f32x4>(b.m + e + 4, x.m1);
        st<f32x4>(b.v + e, x.v0);
        st<f32x4>(b.v + e + 4, x.v1);
    }
    if (has_w) st<u32x4>(b.w + e, wout);
}

// Elements [e, n) of a block, fewer than eight: scalar accesses.
template <bool kSgd>
__device__ void tail_elems(const DevBlock& b, const Coef& c, uint64_t e, uint64_t n, bool has_w)
{
    for (uint64_t i = e; i < n; ++i) {
        const float g = bf16_widen(ld<uint16_t>(b.g + i));
        float p = ld<float>(b.master + i);
        if (kSgd) {
            sgd_elem(c, g, p);
        } else {
            float m = ld<float>(b.m + i), v = ld<float>(b.v + i);
            adam_elem(c, g, p, m, v);
            st<float>(b.m + i, m);
            st<float>(b.v + i, v);
        }
        st<float>(b.master + i, p);
        if (has_w) st<uint16_t>(b.w + i, static_cast<uint16_t>(bf16_rne(p)));
    }
}

template <bool kSgd>
__device__ __forceinline__ void run_chunk(const DevBlock& b, const Coef& c, uint64_t e0)
{
    const bool has_w = (b.flags & kFlagWeight) != 0;
    const uint64_t n = b.n;
    if (e0 + kChunk <= n) {
        // full chunk: all loads first, then arithmetic, then stores
        Group x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            load_group<kSgd>(b, e0 + (static_cast<uint64_t>(u) * kThreads + threadIdx.x) * kVec, x[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            u32x4 w;
            compute_group<kSgd>(c, x[u], w);
            store_group<kSgd>(b, e0 + (static_cast<uint64_t>(u) * kThreads + threadIdx.x) * kVec, x[u], w, has_w);
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t e = e0 + (static_cast<uint64_t>(u) * kThreads + threadIdx.x) * kVec;
        if (e + kVec <= n) {
            Group x;
            u32x4 w;
            load_group<kSgd>(b, e, x);
            compute_group<kSgd>(c, x, w);
            store_group<kSgd>(b, e, x, w, has_w);
        } else if (e < n) {
            tail_elems<kSgd>(b, c, e, n, has_w);
        }
    }
}

// The block owning global chunk `chunk`: the last block whose chunk0 <=
// chunk.  Uniform across the workgroup; the table lives in constant space
// so the search and the block fields are scalar loads.
__device__ __forceinline__ DevBlock find_block(const LSO_CONST DevBlock* blocks, uint32_t nblocks,
                                               uint64_t chunk)
{
    uint32_t lo = 0, hi = nblocks;   // blocks[lo].chunk0 <= chunk < blocks[hi].chunk0
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (blocks[mid].chunk0 <= chunk) lo = mid;
        else hi = mid;
    }
    const LSO_CONST DevBlock* p = blocks + lo;
    DevBlock b;
    b.master = p->master;
    b.m = p->m;
    b.v = p->v;
    b.g = p->g;
    b.w = p->w;
    b.n = p->n;
    b.chunk0 = p->chunk0;
    b.group = p->group;
    b.flags = p->flags;
    return b;
}

// Same for the few blocks passed by value: fully unrolled selects.
__device__ __forceinline__ DevBlock find_inline(const KernelArgs& a, uint64_t chunk)
{
    DevBlock b = a.inl[0];
#pragma unroll
    for (int k = 1; k < kInline; ++k)
        if (static_cast<uint32_t>(k) < a.nblocks && a.inl[k].chunk0 <= chunk) b = a.inl[k];
    return b;
}

__device__ __forceinline__ void run_block_chunk(const KernelArgs& args, const DevBlock& b, uint64_t chunk)
{
    const Coef c = args.coef[b.group];
    const uint64_t e0 = (chunk - b.chunk0) * kChunk;
    if (b.flags & kFlagSgd) run_chunk<true>(b, c, e0);
    else run_chunk<false>(b, c, e0);
}

__global__ void __launch_bounds__(kThreads) fused_adam_kernel(const KernelArgs args)
{
    if (args.blocks) {
        const LSO_CONST DevBlock* table =
            reinterpret_cast<const LSO_CONST DevBlock*>(reinterpret_cast<uintptr_t>(args.blocks));
        for (uint64_t chunk = blockIdx.x; chunk < args.total_chunks; chunk += gridDim.x)
            run_block_chunk(args, find_block(table, args.nblocks, chunk), chunk);
    } else {
        for (uint64_t chunk = blockIdx.x; chunk < args.total_chunks; chunk += gridDim.x)
            run_block_chunk(args, find_inline(args, chunk), chunk);
    }
}

}  // namespace

unsigned default_grid(uint64_t total_chunks)
{
    // 256 CUs; eight resident workgroups of 256 lanes per CU keeps enough
    // 16-byte requests in flight to cover HBM latency.
    const uint64_t cap = 256ull * 8ull;
    return static_cast<unsigned>(total_chunks < cap ? total_chunks : cap);
}

int launch_fused_adam(const KernelArgs& args, unsigned grid, void* stream)
{
    if (args.total_chunks == 0) return 0;
    if (grid == 0) grid = default_grid(args.total_chunks);
    hipLaunchKernelGGL(fused_adam_kernel, dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), args);
    return static_cast<int>(hipGetLastError());
}

}  // namespace lso
