// Host-link copies on SDMA engines chosen explicitly (see lso_sdma.h).
#include "lso_sdma.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace lso {
namespace {

struct AgentSearch {
    uint32_t domain = 0;
    uint32_t bdf = 0;   // bus << 8 | device << 3 | function
    bool gpu_found = false, cpu_found = false;
    hsa_agent_t gpu{}, cpu{};
};

hsa_status_t visit_agent(hsa_agent_t a, void* data)
{
    auto* s = static_cast<AgentSearch*>(data);
    hsa_device_type_t type;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
    if (type == HSA_DEVICE_TYPE_CPU && !s->cpu_found) {
        s->cpu = a;
        s->cpu_found = true;
    } else if (type == HSA_DEVICE_TYPE_GPU && !s->gpu_found) {
        uint32_t bdf = 0, domain = 0;
        if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) ==
                HSA_STATUS_SUCCESS &&
            hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &domain) ==
                HSA_STATUS_SUCCESS &&
            bdf == s->bdf && domain == s->domain) {
            s->gpu = a;
            s->gpu_found = true;
        }
    }
    return HSA_STATUS_SUCCESS;
}

uint32_t lowest_bit(uint32_t m) { return m & (~m + 1u); }

}  // namespace

bool sdma_open(int device, SdmaLink* link)
{
    *link = SdmaLink{};
    char bus_id[64] = {};
    if (hipDeviceGetPCIBusId(bus_id, static_cast<int>(sizeof bus_id), device) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    unsigned dom = 0, bus = 0, dev = 0, fn = 0;
    if (std::sscanf(bus_id, "%x:%x:%x.%x", &dom, &bus, &dev, &fn) != 4) return false;
    if (hsa_init() != HSA_STATUS_SUCCESS) return false;
    AgentSearch s;
    s.domain = dom;
    s.bdf = (bus << 8) | (dev << 3) | fn;
    uint32_t avail_in = 0, avail_out = 0, pref_in = 0, pref_out = 0;
    if (hsa_iterate_agents(visit_agent, &s) != HSA_STATUS_SUCCESS || !s.gpu_found || !s.cpu_found ||
        hsa_amd_memory_copy_engine_status(s.gpu, s.cpu, &avail_in) != HSA_STATUS_SUCCESS ||
        hsa_amd_memory_copy_engine_status(s.cpu, s.gpu, &avail_out) != HSA_STATUS_SUCCESS) {
        (void)hsa_shut_down();
        return false;
    }
    // a runtime without a preference leaves the masks at 0
    (void)hsa_amd_memory_get_preferred_copy_engine(s.gpu, s.cpu, &pref_in);
    (void)hsa_amd_memory_get_preferred_copy_engine(s.cpu, s.gpu, &pref_out);
    uint32_t h = lowest_bit(pref_in & avail_in);
    if (!h) h = lowest_bit(avail_in);
    uint32_t d = lowest_bit(pref_out & avail_out & ~h);
    if (!d) {
        // engines 2k and 2k + 1 form a pair
        const uint32_t partner = (h & 0x55555555u) ? h << 1 : h >> 1;
        d = (partner & avail_out) ? partner : lowest_bit(avail_out & ~h);
    }
    if (const char* e = std::getenv("LSO_STREAM_SDMA")) {
        int a = -1, b = -1;
        if (std::sscanf(e, "%d,%d", &a, &b) == 2 && a >= 0 && a < 16 && b >= 0 && b < 16) {
            h = 1u << a;
            d = 1u << b;
        }
    }
    if (!h || !d || !(h & avail_in) || !(d & avail_out)) {
        (void)hsa_shut_down();
        return false;
    }
    link->gpu = s.gpu;
    link->cpu = s.cpu;
    link->h2d_engine = h;
    link->d2h_engine = d;
    link->ok = true;
    return true;
}

void sdma_close(SdmaLink* link)
{
    if (link->ok) (void)hsa_shut_down();
    *link = SdmaLink{};
}

hsa_status_t sdma_copy(const SdmaLink& link, void* dst, const void* src, uint64_t bytes, bool to_device,
                       const hsa_signal_t* dep, hsa_signal_t done)
{
    hsa_signal_store_screlease(done, 1);
    const hsa_agent_t dst_agent = to_device ? link.gpu : link.cpu;
    const hsa_agent_t src_agent = to_device ? link.cpu : link.gpu;
    const uint32_t engine = to_device ? link.h2d_engine : link.d2h_engine;
    return hsa_amd_memory_async_copy_on_engine(dst, dst_agent, src, src_agent, bytes, dep ? 1u : 0u, dep, done,
                                               static_cast<hsa_amd_sdma_engine_id_t>(engine), false);
}

}  // namespace lso
