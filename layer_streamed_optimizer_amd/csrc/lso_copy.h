// Block copies between page-locked host memory and device memory by a copy
// kernel (lso_copy.hip), used by the layer stream.
#pragma once

#include <cstdint>

namespace lso {

constexpr unsigned kCopyGrid = 128;   // default workgroups of a block copy

// Copy bytes on stream with at most max_grid workgroups (0: kCopyGrid);
// both pointers 16-byte aligned.  Returns the hipError_t of the launch.
int launch_block_copy(void* dst, const void* src, uint64_t bytes, unsigned max_grid, void* stream);

}  // namespace lso
