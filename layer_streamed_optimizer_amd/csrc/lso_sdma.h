// Host-link copies on SDMA engines chosen explicitly (ROCr).
//
// The GPU's SDMA engines come in pairs that share a path to the host link.
// Measured on MI355X with page-locked buffers, both directions running at
// once: H2D on one engine of a pair and D2H on its partner move 57 and 49
// GB/s; on engines of different pairs 46 and 52; on one engine the two
// directions take turns (D2H 29).  hipMemcpyAsync lets the runtime pick
// the engine per copy, and which of these cases a stream gets depends on
// what else was copying when it chose, so the layer stream names its two
// engines itself.
#pragma once

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <cstdint>

namespace lso {

struct SdmaLink {
    bool ok = false;
    hsa_agent_t gpu{};
    hsa_agent_t cpu{};
    uint32_t h2d_engine = 0;   // one hsa_amd_sdma_engine_id_t bit each
    uint32_t d2h_engine = 0;
};

// Initialises ROCr (reference-counted), finds the agent of HIP device
// `device` and a CPU agent, and picks the engines: H2D on the runtime's
// preferred host-to-device engine (else the lowest available), D2H on the
// preferred device-to-host engine other than that one (else its pair
// partner).  LSO_STREAM_SDMA="h,d" (engine numbers) overrides the choice.
// Returns false (with link->ok false and ROCr released) when any of that
// fails; the caller then moves blocks another way.
bool sdma_open(int device, SdmaLink* link);
void sdma_close(SdmaLink* link);

// Copies bytes between page-locked host memory and device memory on the
// link's engine for that direction.  done is set to 1 here and drops to 0
// when the copy ends (negative on failure); dep, if non-null, must reach 0
// before the copy starts.  Returns the ROCr status of the submission.
hsa_status_t sdma_copy(const SdmaLink& link, void* dst, const void* src, uint64_t bytes, bool to_device,
                       const hsa_signal_t* dep, hsa_signal_t done);

// 1 while a copy is pending, 0 once it ended, negative if it failed.
inline int64_t sdma_state(hsa_signal_t s) { return hsa_signal_load_scacquire(s); }

}  // namespace lso
