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

// Bytes of the tiled state region of n parameters.
uint64_t tiled_bytes(uint64_t n);

lso_status check_hyper(uint32_t opt, uint64_t t, double lr, double beta1, double beta2, double eps,
                       size_t index);

// Validate (unless geometry_checked) and enqueue one update of the blocks
// on stream.
lso_status enqueue_update(const lso_block* blocks, size_t n, void* stream, bool geometry_checked);

}  // namespace lso
