// Internal types shared by the host runtime and the fused kernel.
#pragma once

#include <cstdint>

#include "lso.h"

namespace lso {

// Work decomposition of the fused kernel.  A workgroup of kThreads lanes
// handles one chunk of consecutive elements of one block; each lane owns U
// groups of kQuad consecutive elements (U = kUnrollLarge for big calls,
// kUnrollSmall for small ones, where more, smaller chunks spread the work
// over all 256 CUs).
constexpr int kThreads = 256;
constexpr int kQuad = 4;
constexpr int kUnrollLarge = 4;
constexpr int kUnrollSmall = 1;
constexpr int kUnrollTiled = 1;   // a tile's 8192 elements over 8 workgroups
constexpr uint64_t kSmallCallElems = 32ull << 20;   // below this, kUnrollSmall
constexpr uint64_t kMaxGrid = 1ull << 24;            // workgroups per launch
constexpr uint64_t kMaxIndexChunks = 1ull << 22;     // per-chunk block index up to this

constexpr uint64_t chunk_elems(int unroll) { return static_cast<uint64_t>(kThreads) * kQuad * unroll; }
constexpr uint64_t kNormPartsPerChunk = kThreads / 64;   // one FP64 per wave
static_assert(LSO_TILE_ELEMS % chunk_elems(kUnrollTiled) == 0, "a tiled chunk lies inside one state tile");

// At most this many distinct constant sets travel by value in one launch.
constexpr int kMaxGroups = 16;

enum : uint32_t { kFlagSgd = 1u, kFlagWeight = 2u, kFlagTiled = 4u, kFlagGradF32 = 8u };

// One block as the kernel sees it (64 bytes, lives in a device table).
// Tiled blocks: master is the tiled state region, m and v are unused.
struct DevBlock {
    float* master;
    float* m;
    float* v;
    const uint16_t* g;   // BF16 gradients (FP32 ones when kFlagGradF32)
    uint16_t* w;
    uint64_t n;
    uint64_t chunk0;     // first global chunk index of this block
    uint32_t group;      // index into KernelArgs::coef
    uint32_t flags;      // kFlag* in bits 0-7; the block's position in the
                         // caller's array in bits 8-31
};
constexpr int kIndexShift = 8;
constexpr uint64_t kMaxBlocksPerCall = 1ull << 24;
static_assert(sizeof(DevBlock) == 64, "DevBlock layout");

// FP32 constants of one (opt, t, lr, beta1, beta2, eps) set.
struct Coef {
    float b1, c1, b2, c2;   // beta1, 1-beta1, beta2, 1-beta2
    float s;                // Adam: lr/(1-beta1^t); SGD: lr
    float r;                // 1/sqrt(1-beta2^t)
    float e;                // eps
    float pad;
};
static_assert(sizeof(Coef) == 32, "Coef layout");

// Up to this many blocks travel by value in the kernel arguments (no
// device table, no upload, no dependent table load).
constexpr int kInline = 4;

struct KernelArgs {
    const DevBlock* blocks;        // device table, or nullptr: use inl[]
    const uint32_t* chunk_block;   // block index per chunk, or nullptr: search
    double* partials;              // norm variant: sum of g^2 per wave and chunk of this launch
    uint64_t total_chunks;
    uint64_t grid;                 // workgroups of the launch (set by launch_fused_adam)
    uint32_t nblocks;
    uint32_t ngroups;              // constant sets in coef[] (table launches)
    Coef coef[kMaxGroups];         // by-value launches: coef[k] is inl[k]'s
    DevBlock inl[kInline];
};

// Enqueue the fused kernel (defined in lso_adam.hip) with chunks of
// chunk_elems(unroll) elements (unroll: kUnrollSmall or kUnrollLarge
// planar, kUnrollTiled tiled); tiled launches the tiled variant (every
// block of the launch tiled); grad_f32 the FP32-gradient variant (every
// block of the launch).  With args.partials set, the norm
// variant also writes each wave's sum of g^2 to
// args.partials[chunk * kNormPartsPerChunk + wave].
// Returns the hipError_t.
int launch_fused_adam(const KernelArgs& args, int unroll, bool tiled, bool grad_f32, void* stream);

// Sum the chunk partials of each block of the launch (one workgroup per
// block, fixed order) into sq_norms[the block's position in the call].
// Returns the hipError_t.
int launch_norm_reduce(const KernelArgs& args, int unroll, double* sq_norms, void* stream);

}  // namespace lso
