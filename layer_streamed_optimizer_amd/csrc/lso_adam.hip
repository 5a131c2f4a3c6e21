// Fused mixed-precision Adam for gfx950: one HBM pass per element.
//
// Per element (frozen-incremental page, section "The Math"; training-memory
// article, "Optimizer states"): read the BF16 gradient and the FP32 master,
// m and v; update the two moments; form the bias-corrected step with eps
// outside the root; add it to the master (the additive write-back); store
// master, m, v and the BF16 round-to-nearest-even re-cast of the new master.
// 14 bytes read + 14 bytes written per parameter (16 + 14 with FP32
// gradients) and nothing else: no scratch, no second pass.  The norm
// variant also sums g^2 while the gradient is in registers (one FP64 per
// wave and chunk, 1/250 of the traffic or less) for progressive layer
// locking; a small second kernel adds each block's wave sums in a fixed
// order.
//
// Memory access: a lane owns groups of four consecutive elements, so every
// FP32 access is one 128-bit load or store, and each wave instruction covers
// one contiguous run (1 KB of FP32, 512 B of BF16).  A lane's own BF16
// gradients and weights are 64 bits; on full tiled chunks and full planar
// chunks of big calls they move 128 bits per lane instead (half of each
// wave, or row pairs) and reach their lanes by ds_bpermute (run_chunk).  All
// state is touched exactly once, so loads and stores are non-temporal
// (streamed past the caches); tiled chunks store with device scope too
// (inline assembly, each block of stores closed by a wait state).
//
// Two layouts of the FP32 state: planar (three arrays) or tiled (master, m
// and v interleaved in tiles of LSO_TILE_ELEMS elements): in the tiled one
// the three arrays of a workgroup's chunk sit in one 96 KB tile instead of
// three streams far apart, which the HBM serves about 10% faster.  A tile
// is split over eight workgroups of 1024 elements each (a grid of about a
// million small workgroups for a 1B-parameter call); measured 3% faster
// than one workgroup per tile.
//
// Ragged multi-tensor launch: one grid covers the concatenated chunk space
// of every block of the call, one chunk per workgroup.  A workgroup finds
// its block through a per-chunk block index (one scalar load), through a
// binary search over the table when the call has too many chunks for an
// index, or among the few blocks passed by value in the kernel arguments.
//
// Built with -ffp-contract=off: every FMA below is an explicit fmaf and every
// other operator rounds once, so the SGD path is exactly fl(W + fl(-(lr*g))).
// Built with -fhip-fp32-correctly-rounded-divide-sqrt: FP32 division and
// sqrtf are correctly rounded (HIP's __fsqrt_rn is the hardware's 1-ulp root
// unless the rounded-operation library is selected, so it is not used).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lso_bf16.h"
#include "lso_internal.h"

namespace lso {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// State arrays are global memory (global_* rather than flat_* accesses);
// the block table and chunk index are read-only while the kernel runs
// (constant space: scalar loads).
#define LSO_GLOBAL __attribute__((address_space(1)))
#define LSO_CONST __attribute__((address_space(4)))

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

// Stores of a tiled chunk carry the cache-policy bits nt (streaming) and
// sc1 (device scope).  Measured on this part, alternating libraries on one
// machine: c3 (LLaMA-7B, tiled) 28.75 ms against 29.71 ms with nt alone over
// six runs each, c1 tiled 4.75 against 4.87 ms; planar chunks (four quads
// per lane) were 3% slower with them, so they keep plain nt stores.  No
// compiler builtin sets sc1 on a global store, hence the inline assembly.
// The compiler does not count these stores in its waits; on this
// architecture vector-memory operations complete in order and share one
// counter, and every lane issues them after all its loads of the chunk, so
// each wait the compiler emits only becomes longer, never shorter.
// Nor does it see the hazard of a store's data registers: a store of more
// than 8 bytes reads them one cycle after issue, so a vector-ALU write to
// them in the next cycle needs a wait state between the two, which the
// compiler inserts after stores it emits itself but not after inline
// assembly.  Every asm block of stores here therefore ends with s_nop 0
// (one wait state); the 8-byte form gets one too.  (Without it, a build
// whose second quad's arithmetic followed the first quad's stores wrote
// corrupted m values.)  A quad's master, m and v go out in one block with
// one s_nop: a wait state after each store measured 0.4% slower on c3.
__device__ __forceinline__ void st_nt_sc1(const void* p, f32x4 v)
{
    const LSO_GLOBAL f32x4* a = reinterpret_cast<const LSO_GLOBAL f32x4*>(reinterpret_cast<uintptr_t>(p));
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 0" : : "v"(a), "v"(v) : "memory");
}

__device__ __forceinline__ void st_nt_sc1(const void* p, u32x2 v)
{
    const LSO_GLOBAL u32x2* a = reinterpret_cast<const LSO_GLOBAL u32x2*>(reinterpret_cast<uintptr_t>(p));
    asm volatile("global_store_dwordx2 %0, %1, off nt sc1\n\ts_nop 0" : : "v"(a), "v"(v) : "memory");
}

template <typename T>
__device__ __forceinline__ T ld(const void* p)
{
    return *reinterpret_cast<const LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p));
}

template <typename T>
__device__ __forceinline__ void st(void* p, T v)
{
    *reinterpret_cast<LSO_GLOBAL T*>(reinterpret_cast<uintptr_t>(p)) = v;
}

__device__ __forceinline__ void adam_elem(const Coef& c, float g, float& master, float& m, float& v)
{
    const float m1 = fmaf(c.b1, m, c.c1 * g);
    const float v1 = fmaf(c.b2, v, c.c2 * (g * g));   // g*g is exact for BF16 g (8 significant bits)
    const float den = fmaf(__builtin_sqrtf(v1), c.r, c.e);  // sqrt(v_hat) + eps, v_hat = v1 * r^2
    const float delta = -((c.s * m1) / den);
    master = master + delta;
    m = m1;
    v = v1;
}

__device__ __forceinline__ void sgd_elem(const Coef& c, float g, float& master)
{
    const float delta = -(c.s * g);
    master = master + delta;
}

// Four consecutive elements held by one lane.
struct Quad {
    u32x2 g;     // 4 BF16 gradients
    f32x4 gf;    // or 4 FP32 gradients
    f32x4 p;     // master
    f32x4 m;
    f32x4 v;
};

// One chunk as seen by a workgroup: pointers to its first element in each
// array, and how many of its elements exist (the rest of a ragged last chunk
// is skipped).  A planar chunk points into the block's three arrays; a tiled
// chunk is one state tile, whose master, m and v runs are back to back.
struct Chunk {
    float* p;
    float* m;
    float* v;
    const uint16_t* g;   // BF16 gradients
    const float* gf;     // FP32 gradients
    uint16_t* w;
    uint32_t n;   // valid elements in this chunk
};

template <bool kSgd, bool kG32>
__device__ __forceinline__ void load_quad(const Chunk& ch, uint32_t e, Quad& x)
{
    if (kG32) x.gf = ld_nt<f32x4>(ch.gf + e);
    else x.g = ld_nt<u32x2>(ch.g + e);
    x.p = ld_nt<f32x4>(ch.p + e);
    if (!kSgd) {
        x.m = ld_nt<f32x4>(ch.m + e);
        x.v = ld_nt<f32x4>(ch.v + e);
    }
}

// The state of a quad alone (its gradients come separately).
__device__ __forceinline__ void load_state(const Chunk& ch, uint32_t e, Quad& x)
{
    x.p = ld_nt<f32x4>(ch.p + e);
    x.m = ld_nt<f32x4>(ch.m + e);
    x.v = ld_nt<f32x4>(ch.v + e);
}

// Value v of lane src_lane of this wave.
__device__ __forceinline__ uint32_t lane_take(uint32_t v, int src_lane)
{
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(v)));
}

template <bool kSgd, bool kG32, bool kNorm>
__device__ __forceinline__ u32x2 compute_quad(const Coef& c, Quad& x, float& sq)
{
    u32x2 w;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float g0 = kG32 ? x.gf[2 * k] : bf16_widen(x.g[k] & 0xFFFFu);
        const float g1 = kG32 ? x.gf[2 * k + 1] : bf16_widen(x.g[k] >> 16);
        if (kNorm) {
            sq = fmaf(g0, g0, sq);
            sq = fmaf(g1, g1, sq);
        }
        float p0 = x.p[2 * k], p1 = x.p[2 * k + 1];
        if (kSgd) {
            sgd_elem(c, g0, p0);
            sgd_elem(c, g1, p1);
        } else {
            float m0 = x.m[2 * k], m1 = x.m[2 * k + 1];
            float v0 = x.v[2 * k], v1 = x.v[2 * k + 1];
            adam_elem(c, g0, p0, m0, v0);
            adam_elem(c, g1, p1, m1, v1);
            x.m[2 * k] = m0;
            x.m[2 * k + 1] = m1;
            x.v[2 * k] = v0;
            x.v[2 * k + 1] = v1;
        }
        x.p[2 * k] = p0;
        x.p[2 * k + 1] = p1;
        w[k] = bf16_rne(p0) | (bf16_rne(p1) << 16);
    }
    return w;
}

template <bool kSgd, bool kSc1>
__device__ __forceinline__ void store_quad(const Chunk& ch, uint32_t e, const Quad& x, u32x2 w, bool has_w)
{
    if (kSc1 && !kSgd) {
        // master, m and v back to back, then the one wait state
        const LSO_GLOBAL f32x4* ap = reinterpret_cast<const LSO_GLOBAL f32x4*>(reinterpret_cast<uintptr_t>(ch.p + e));
        const LSO_GLOBAL f32x4* am = reinterpret_cast<const LSO_GLOBAL f32x4*>(reinterpret_cast<uintptr_t>(ch.m + e));
        const LSO_GLOBAL f32x4* av = reinterpret_cast<const LSO_GLOBAL f32x4*>(reinterpret_cast<uintptr_t>(ch.v + e));
        asm volatile("global_store_dwordx4 %0, %3, off nt sc1\n\t"
                     "global_store_dwordx4 %1, %4, off nt sc1\n\t"
                     "global_store_dwordx4 %2, %5, off nt sc1\n\t"
                     "s_nop 0"
                     : : "v"(ap), "v"(am), "v"(av), "v"(x.p), "v"(x.m), "v"(x.v) : "memory");
        if (has_w) st_nt_sc1(ch.w + e, w);
        return;
    }
    if (kSc1) {
        st_nt_sc1(ch.p + e, x.p);
        if (has_w) st_nt_sc1(ch.w + e, w);
        return;
    }
    st_nt<f32x4>(ch.p + e, x.p);
    if (!kSgd) {
        st_nt<f32x4>(ch.m + e, x.m);
        st_nt<f32x4>(ch.v + e, x.v);
    }
    if (has_w) st_nt<u32x2>(ch.w + e, w);
}

// Elements [e, n) of a chunk, fewer than four: scalar accesses.
template <bool kSgd, bool kG32, bool kNorm>
__device__ void tail_elems(const Chunk& ch, const Coef& c, uint32_t e, uint32_t n, bool has_w, float& sq)
{
    for (uint32_t i = e; i < n; ++i) {
        const float g = kG32 ? ld<float>(ch.gf + i) : bf16_widen(ld<uint16_t>(ch.g + i));
        if (kNorm) sq = fmaf(g, g, sq);
        float p = ld<float>(ch.p + i);
        if (kSgd) {
            sgd_elem(c, g, p);
        } else {
            float m = ld<float>(ch.m + i), v = ld<float>(ch.v + i);
            adam_elem(c, g, p, m, v);
            st<float>(ch.m + i, m);
            st<float>(ch.v + i, v);
        }
        st<float>(ch.p + i, p);
        if (has_w) st<uint16_t>(ch.w + i, static_cast<uint16_t>(bf16_rne(p)));
    }
}

// One chunk of kThreads * kQuad * U elements.  Returns this lane's sum of
// g^2 (norm variant; 0 otherwise).
template <int U, bool kSgd, bool kG32, bool kNorm, bool kSc1>
__device__ __forceinline__ float run_chunk(const Chunk& ch, const Coef& c, bool has_w)
{
    constexpr uint32_t kChunkU = static_cast<uint32_t>(kThreads) * kQuad * U;
    float sq = 0.0f;
    if (ch.n == kChunkU && kSc1 && !kSgd) {
        // full tiled chunk: a wave's BF16 gradients and weights are each one
        // 512-byte run, moved 16 bytes per lane by lanes 0-31 and handed to
        // the lanes of their quads by ds_bpermute (a lane's own quad is only
        // 8 bytes of each); FP32 gradients are 16 bytes per lane already and
        // load as they are.  Measured against 8-byte accesses: c3 28.71
        // against 28.89 ms, c1 4.681 against 4.699 ms, c1 with FP32
        // gradients 5.041 against 5.048-5.127 ms (two alternating runs
        // each).
        const uint32_t lane = threadIdx.x & 63u;
        Quad x[U];
        u32x4 gw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t we = (u * kThreads + (threadIdx.x & ~63u)) * kQuad;   // the wave's first element
            gw[u] = u32x4{0u, 0u, 0u, 0u};
            if (kG32) x[u].gf = ld_nt<f32x4>(ch.gf + (u * kThreads + threadIdx.x) * kQuad);
            else if (lane < 32u) gw[u] = ld_nt<u32x4>(ch.g + we + 8u * lane);
            load_state(ch, (u * kThreads + threadIdx.x) * kQuad, x[u]);
        }
#pragma unroll
        for (int u = 0; u < U && !kG32; ++u) {
            // lane l's quad is the first or second half of lane l/2's load
            const int from = static_cast<int>(lane >> 1);
            const uint32_t a0 = lane_take(gw[u].x, from), a1 = lane_take(gw[u].y, from);
            const uint32_t a2 = lane_take(gw[u].z, from), a3 = lane_take(gw[u].w, from);
            x[u].g = (lane & 1u) ? u32x2{a2, a3} : u32x2{a0, a1};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x2 w = compute_quad<kSgd, kG32, kNorm>(c, x[u], sq);
            store_quad<kSgd, kSc1>(ch, (u * kThreads + threadIdx.x) * kQuad, x[u], w, false);
            if (has_w) {
                // lane l < 32 stores the weights of lanes 2l and 2l + 1
                const int s0 = static_cast<int>((2u * lane) & 63u), s1 = static_cast<int>((2u * lane + 1u) & 63u);
                const u32x4 ww = {lane_take(w.x, s0), lane_take(w.y, s0), lane_take(w.x, s1), lane_take(w.y, s1)};
                const uint32_t we = (u * kThreads + (threadIdx.x & ~63u)) * kQuad;
                if (lane < 32u) st_nt_sc1(ch.w + we + 8u * lane, __builtin_bit_cast(f32x4, ww));
            }
        }
        return sq;
    }
    if (ch.n == kChunkU && !kSc1 && U % 2 == 0 && !kG32 && !kSgd) {
        // full planar chunk of a big call (four quads per lane), BF16
        // gradients: rows are paired, lanes 0-31 moving row 2k's 512-byte
        // gradient and weight runs and lanes 32-63 row 2k+1's, 16 bytes per
        // lane, handed over by ds_bpermute.  Planar c3 33.96 against 34.21
        // ms, c1 5.44 against 5.46-5.51 ms.  Small planar calls (one quad per
        // lane, half of each wave moving) were slower with it (c0 +5%, c2
        // +1.5%) and keep the 8-byte accesses below.
        const uint32_t lane = threadIdx.x & 63u;
        Quad x[U];
        u32x4 gw[U / 2 > 0 ? U / 2 : 1];
#pragma unroll
        for (int k = 0; k < U / 2; ++k) {
            const uint32_t r = 2u * k + (lane >> 5);   // lanes 0-31: row 2k, 32-63: row 2k+1
            const uint32_t we = (r * kThreads + (threadIdx.x & ~63u)) * kQuad;
            gw[k] = ld_nt<u32x4>(ch.g + we + 8u * (lane & 31u));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) load_state(ch, (u * kThreads + threadIdx.x) * kQuad, x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int from = static_cast<int>((lane >> 1) + 32u * (u & 1));
            const u32x4 g4 = gw[u / 2];
            const uint32_t a0 = lane_take(g4.x, from), a1 = lane_take(g4.y, from);
            const uint32_t a2 = lane_take(g4.z, from), a3 = lane_take(g4.w, from);
            x[u].g = (lane & 1u) ? u32x2{a2, a3} : u32x2{a0, a1};
        }
        u32x2 wq[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wq[u] = compute_quad<kSgd, kG32, kNorm>(c, x[u], sq);
            store_quad<kSgd, kSc1>(ch, (u * kThreads + threadIdx.x) * kQuad, x[u], wq[u], false);
        }
        if (has_w) {
#pragma unroll
            for (int k = 0; k < U / 2; ++k) {
                // lane l stores 8 weights of row 2k + l/32: those of lanes
                // 2(l%32) and 2(l%32) + 1
                const int s0 = static_cast<int>(2u * (lane & 31u)), s1 = s0 + 1;
                const u32x2 w0 = wq[2 * k], w1 = wq[2 * k + 1];
                const uint32_t b0 = lane_take(w0.x, s0), b1 = lane_take(w0.y, s0), b2 = lane_take(w0.x, s1), b3 = lane_take(w0.y, s1);
                const uint32_t c0 = lane_take(w1.x, s0), c1 = lane_take(w1.y, s0), c2 = lane_take(w1.x, s1), c3 = lane_take(w1.y, s1);
                const u32x4 ww = (lane < 32u) ? u32x4{b0, b1, b2, b3} : u32x4{c0, c1, c2, c3};
                const uint32_t r = 2u * k + (lane >> 5);
                const uint32_t we = (r * kThreads + (threadIdx.x & ~63u)) * kQuad;
                st_nt<u32x4>(ch.w + we + 8u * (lane & 31u), ww);
            }
        }
        return sq;
    }
    if (ch.n == kChunkU) {
        // full chunk: every load of the lane first, then arithmetic and stores
        Quad x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) load_quad<kSgd, kG32>(ch, (u * kThreads + threadIdx.x) * kQuad, x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x2 w = compute_quad<kSgd, kG32, kNorm>(c, x[u], sq);
            store_quad<kSgd, kSc1>(ch, (u * kThreads + threadIdx.x) * kQuad, x[u], w, has_w);
        }
        return sq;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t e = (u * kThreads + threadIdx.x) * kQuad;
        if (e + kQuad <= ch.n) {
            Quad x;
            load_quad<kSgd, kG32>(ch, e, x);
            const u32x2 w = compute_quad<kSgd, kG32, kNorm>(c, x, sq);
            store_quad<kSgd, kSc1>(ch, e, x, w, has_w);
        } else if (e < ch.n) {
            tail_elems<kSgd, kG32, kNorm>(ch, c, e, ch.n, has_w, sq);
        }
    }
    return sq;
}

constexpr int kWaves = kThreads / 64;

// Sum of v over the wave by an xor butterfly (fixed order; every lane ends
// with the same value).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum of v over a workgroup of kN threads in a fixed order (lanes by xor
// butterfly, then the waves in order); the result is valid in thread 0.
// Every thread of the workgroup must call it.
template <int kN>
__device__ __forceinline__ double workgroup_sum(double v)
{
    __shared__ double per_wave[kN / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) per_wave[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < kN / 64; ++k) s += per_wave[k];
    }
    __syncthreads();   // per_wave may be rewritten by the next call
    return s;
}

// A table entry in one 64-byte scalar load (fields loaded one by one let
// the compiler fetch the constant-set index first and wait for it).
__device__ __forceinline__ DevBlock load_block(const LSO_CONST DevBlock* p)
{
    typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
    const u32x16 raw = *reinterpret_cast<const LSO_CONST u32x16*>(p);
    return __builtin_bit_cast(DevBlock, raw);
}

// The last block whose chunk0 <= chunk (uniform across the workgroup).
__device__ __forceinline__ uint32_t search_block(const LSO_CONST DevBlock* blocks, uint32_t nblocks,
                                                 uint64_t chunk)
{
    uint32_t lo = 0, hi = nblocks;   // blocks[lo].chunk0 <= chunk < blocks[hi].chunk0
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (blocks[mid].chunk0 <= chunk) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Same for the few blocks passed by value, with their constants (block k
// of a by-value launch uses coef[k]): the blocks' first chunks load in one
// round from fixed places in the kernel arguments, the pick is a few scalar
// selects, and the picked block and its constants load in a second round --
// a one-round grid (a small call) reaches its data after two rounds of
// scalar loads instead of a chain of them.
__device__ __forceinline__ void find_inline(const KernelArgs& a, uint64_t chunk, DevBlock& b, Coef& c)
{
    uint32_t sel = 0;
#pragma unroll
    for (int k = 1; k < kInline; ++k)
        sel = (static_cast<uint32_t>(k) < a.nblocks && a.inl[k].chunk0 <= chunk) ? static_cast<uint32_t>(k) : sel;
    c = a.coef[sel];
    b = a.inl[sel];
}

template <int U, bool kTiled, bool kG32, bool kNorm>
__device__ __forceinline__ void run_block_chunk(const KernelArgs& args, const DevBlock& b, const Coef& c,
                                                uint64_t chunk)
{
    constexpr uint64_t kChunkU = static_cast<uint64_t>(kThreads) * kQuad * U;
    const uint64_t k = chunk - b.chunk0;   // chunk index inside the block
    const uint64_t e0 = k * kChunkU;       // its first element
    const uint64_t left = b.n - e0;
    Chunk ch;
    ch.n = static_cast<uint32_t>(left < kChunkU ? left : kChunkU);
    ch.g = b.g + e0;
    ch.gf = reinterpret_cast<const float*>(b.g) + e0;
    ch.w = b.w ? b.w + e0 : nullptr;
    if (kTiled) {
        // tile e0 / T holds [master | m | v], T elements each; the chunk is
        // a part of one tile (three short runs a tile-length apart)
        constexpr uint64_t T = LSO_TILE_ELEMS;
        ch.p = b.master + 3 * (e0 / T) * T + (e0 % T);
        ch.m = ch.p + T;
        ch.v = ch.m + T;
    } else {
        ch.p = b.master + e0;
        ch.m = b.m ? b.m + e0 : nullptr;
        ch.v = b.v ? b.v + e0 : nullptr;
    }
    const bool has_w = (b.flags & kFlagWeight) != 0;
    const float sq = (!kTiled && (b.flags & kFlagSgd)) ? run_chunk<U, true, kG32, kNorm, false>(ch, c, has_w)
                                                       : run_chunk<U, false, kG32, kNorm, kTiled>(ch, c, has_w);
    if (kNorm) {
        // one sum per wave (no barrier in the update kernel); the reduce
        // kernel adds a block's wave sums in order
        const double s = static_cast<double>(wave_sum(sq));
        if ((threadIdx.x & 63) == 0) st<double>(args.partials + chunk * kWaves + (threadIdx.x >> 6), s);
    }
}

// kTable: the blocks are in a device table (found by the per-chunk index or
// by a binary search), else in the kernel arguments; kOne: a by-value call
// of one block, whose fields and constants load in a single round with no
// pick.  The grid never exceeds the chunk count, so every workgroup has a
// first chunk: the loop only tests the count for grids smaller than the
// call (very large calls).
template <int U, bool kTiled, bool kG32, bool kNorm, bool kTable, bool kOne>
__global__ void __launch_bounds__(kThreads) fused_adam_kernel(const KernelArgs args)
{
    uint64_t chunk = blockIdx.x;
    if (kTable) {
        const LSO_CONST DevBlock* table =
            reinterpret_cast<const LSO_CONST DevBlock*>(reinterpret_cast<uintptr_t>(args.blocks));
        const LSO_CONST uint32_t* index =
            reinterpret_cast<const LSO_CONST uint32_t*>(reinterpret_cast<uintptr_t>(args.chunk_block));
        // one constant set for the whole launch (the usual case): its load
        // does not wait for the block's
        const Coef c0 = args.coef[0];
        do {
            const uint32_t bi = index ? index[chunk] : search_block(table, args.nblocks, chunk);
            const DevBlock b = load_block(table + bi);
            Coef c = c0;
            if (args.ngroups != 1) c = args.coef[b.group];
            run_block_chunk<U, kTiled, kG32, kNorm>(args, b, c, chunk);
            chunk += args.grid;
        } while (chunk < args.total_chunks);
    } else if (kOne) {
        const DevBlock b = args.inl[0];
        const Coef c = args.coef[0];
        do {
            run_block_chunk<U, kTiled, kG32, kNorm>(args, b, c, chunk);
            chunk += args.grid;
        } while (chunk < args.total_chunks);
    } else {
        do {
            DevBlock b;
            Coef c;
            find_inline(args, chunk, b, c);
            run_block_chunk<U, kTiled, kG32, kNorm>(args, b, c, chunk);
            chunk += args.grid;
        } while (chunk < args.total_chunks);
    }
}

// One workgroup per block of the launch: the block's wave sums added in a
// fixed order, written to sq_norms[the block's position in the call].  A
// large block has hundreds of thousands of them: 1024 threads with eight
// independent loads in flight each keep the pass short.
constexpr int kReduceThreads = 1024;
constexpr int kReduceLoads = 8;

template <int U>
__global__ void __launch_bounds__(kReduceThreads) norm_reduce_kernel(const KernelArgs args, double* sq_norms)
{
    constexpr uint64_t kChunkU = static_cast<uint64_t>(kThreads) * kQuad * U;
    DevBlock b;
    if (args.blocks) {
        const LSO_CONST DevBlock* table =
            reinterpret_cast<const LSO_CONST DevBlock*>(reinterpret_cast<uintptr_t>(args.blocks));
        b = load_block(table + blockIdx.x);
    } else {
        b = args.inl[0];
#pragma unroll
        for (int k = 1; k < kInline; ++k)
            if (static_cast<uint32_t>(k) == blockIdx.x) b = args.inl[k];
    }
    const uint64_t nparts = (b.n + kChunkU - 1) / kChunkU * kWaves;
    const double* parts = args.partials + b.chunk0 * kWaves;
    constexpr uint64_t R = kReduceThreads;
    double acc[kReduceLoads];
#pragma unroll
    for (int j = 0; j < kReduceLoads; ++j) acc[j] = 0.0;
    uint64_t k = threadIdx.x;
    for (; k + (kReduceLoads - 1) * R < nparts; k += kReduceLoads * R) {
#pragma unroll
        for (int j = 0; j < kReduceLoads; ++j) acc[j] += ld<double>(parts + k + j * R);
    }
    for (int j = 0; k < nparts; k += R, ++j) acc[j] += ld<double>(parts + k);   // j < kReduceLoads - 1
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kReduceLoads; ++j) s += acc[j];
    s = workgroup_sum<kReduceThreads>(s);
    if (threadIdx.x == 0) st<double>(sq_norms + (b.flags >> kIndexShift), s);
}

template <int U, bool kTiled, bool kG32>
void launch_variant(const KernelArgs& args, dim3 g, hipStream_t s)
{
    const dim3 t(kThreads);
    if (args.blocks) {
        if (args.partials) hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, true, true, false>), g, t, 0, s, args);
        else hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, false, true, false>), g, t, 0, s, args);
    } else if (args.nblocks == 1) {
        if (args.partials) hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, true, false, true>), g, t, 0, s, args);
        else hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, false, false, true>), g, t, 0, s, args);
    } else {
        if (args.partials) hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, true, false, false>), g, t, 0, s, args);
        else hipLaunchKernelGGL((fused_adam_kernel<U, kTiled, kG32, false, false, false>), g, t, 0, s, args);
    }
}

}  // namespace

int launch_fused_adam(const KernelArgs& args, int unroll, bool tiled, bool grad_f32, void* stream)
{
    if (args.total_chunks == 0) return 0;
    // one chunk per workgroup; a call too large for one grid loops.  The
    // stride travels as an ordinary argument: it then loads with the rest
    // of the first round, where the grid size would be a second one.
    KernelArgs a = args;
    a.grid = args.total_chunks < kMaxGrid ? args.total_chunks : kMaxGrid;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(static_cast<unsigned>(a.grid));
    if (grad_f32) {
        if (tiled) launch_variant<kUnrollTiled, true, true>(a, g, s);
        else if (unroll == kUnrollLarge) launch_variant<kUnrollLarge, false, true>(a, g, s);
        else launch_variant<kUnrollSmall, false, true>(a, g, s);
    } else {
        if (tiled) launch_variant<kUnrollTiled, true, false>(a, g, s);
        else if (unroll == kUnrollLarge) launch_variant<kUnrollLarge, false, false>(a, g, s);
        else launch_variant<kUnrollSmall, false, false>(a, g, s);
    }
    return static_cast<int>(hipGetLastError());
}

// the tiled chunk size is the small planar one, so one instance serves both
static_assert(kUnrollTiled == kUnrollSmall, "norm_reduce_kernel<kUnrollSmall> serves tiled launches");

int launch_norm_reduce(const KernelArgs& args, int unroll, double* sq_norms, void* stream)
{
    if (args.nblocks == 0 || !args.partials) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(args.nblocks), t(kReduceThreads);
    if (unroll == kUnrollLarge) hipLaunchKernelGGL((norm_reduce_kernel<kUnrollLarge>), g, t, 0, s, args, sq_norms);
    else hipLaunchKernelGGL((norm_reduce_kernel<kUnrollSmall>), g, t, 0, s, args, sq_norms);
    return static_cast<int>(hipGetLastError());
}

}  // namespace lso
