// Host-runtime pieces shared between the resident and the streamed paths.
#pragma once

#include <cstddef>
#include <cstdint>

#include "lso.h"

namespace lso {

// Record a message for lso_last_error() and return s.
lso_status fail(lso_status s, const char* fmt, ...);
lso_status hip_fail(int hip_error, const char* what);
void clear_error();

// Count one fused-update kernel launch (lso_kernel_launches).
void count_launch();

// Bytes of the tiled state region of n parameters.
uint64_t tiled_bytes(uint64_t n);

lso_status check_hyper(uint32_t opt, uint64_t t, double lr, double beta1, double beta2, double eps,
                       size_t index);

// Where the norm variant puts its results: sq_norms[i] = sum of g^2 of
// block i (device, n doubles); workspace: device, norm_workspace_bytes().
struct NormOut {
    double* sq_norms = nullptr;
    double* workspace = nullptr;
    uint64_t workspace_bytes = 0;
};

// Device workspace the norm variant needs for these blocks: one double per
// chunk of every launch of the call.
uint64_t norm_workspace_bytes(const lso_block* blocks, size_t n);

// Checks of the norm variant's outputs: non-NULL, aligned, workspace
// large enough, and neither overlapping the other or any array of the call.
lso_status validate_norm_buffers(const lso_block* blocks, size_t n, const NormOut& o);

// Validate (unless geometry_checked) and enqueue one update of the blocks
// on stream; with norms, also each block's sum of g^2.
lso_status enqueue_update(const lso_block* blocks, size_t n, void* stream, bool geometry_checked,
                          const NormOut* norms = nullptr);

struct DevBlock;

// The current device's fixed scratch array of LSO_NOALLOC_MAX_BLOCKS
// DevBlocks (lso_noalloc.hip); its address is looked up once per device.
// stream: the call's stream, checked for capture before the first lookup
// (NULL skips the check).
lso_status noalloc_scratch(DevBlock** out, void* stream);

// Enqueue on stream the writes of count table entries to dst (inside the
// scratch array), carried in kernel arguments.
lso_status noalloc_write_table(DevBlock* dst, const DevBlock* tab, size_t count, void* stream);

// lso_adam_step_noalloc: validate every call, and keep the block tables of
// the call's launches in the device's fixed scratch array instead of
// allocated, cached device tables (no allocation of any kind).
lso_status enqueue_update_noalloc(const lso_block* blocks, size_t n, void* stream);

}  // namespace lso
