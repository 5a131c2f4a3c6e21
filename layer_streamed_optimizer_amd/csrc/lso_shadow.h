// Shadow regions for crash-consistent write-back (LSO_FILE_SHADOW): the
// header format and the reads and writes around it.  Host code only.
#pragma once

#include <cstddef>
#include <cstdint>

#include "lso.h"

namespace lso {

constexpr uint64_t kShadowCopy = 4096;   // bytes of one header copy

struct ShadowState {
    uint64_t epoch = 0;
    uint64_t t = 0;
};

// Absolute file offsets inside the region at `off` with data blocks of
// `bytes`: the data slot and the header copy of an epoch.
inline uint64_t shadow_slot(uint64_t off, uint64_t bytes, uint64_t epoch)
{
    return off + LSO_SHADOW_HEADER_BYTES + (epoch % 2) * bytes;
}
inline uint64_t shadow_header(uint64_t off, uint64_t epoch) { return off + (epoch % 2) * kShadowCopy; }

// One header copy (kShadowCopy bytes, the rest zero) for (epoch, bytes, t).
void shadow_encode(char* buf, uint64_t epoch, uint64_t bytes, uint64_t t);

// The committed state: the valid copy with the highest epoch.  Errors:
// LSO_E_IO (read failure, or no valid copy), with a message.
lso_status shadow_read(int fd, uint64_t off, uint64_t bytes, ShadowState* st);

}  // namespace lso
