// Host runtime of the C ABI: validation, FP64 -> FP32 constants, the
// multi-tensor launch plan, the device-table cache and lso_adam_step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "lso_internal.h"
#include "lso_runtime.h"

namespace lso {

// Fused-update launches enqueued by this process (lso_kernel_launches).
static std::atomic<uint64_t> g_launches{0};

void count_launch() { g_launches.fetch_add(1, std::memory_order_relaxed); }

// ------------------------------------------------------------------ errors

static thread_local char t_last_error[512] = "";

lso_status fail(lso_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(t_last_error, sizeof t_last_error, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { t_last_error[0] = '\0'; }

lso_status hip_fail(int err, const char* what)
{
    return fail(LSO_E_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
}

// ------------------------------------------------------------- validation
// Field checks (dtypes, optimizer, hyper-parameters) run on every call;
// address checks (NULL, alignment, overlap) run when a block table is new.

lso_status check_hyper(uint32_t opt, uint64_t t, double lr, double beta1, double beta2, double eps,
                       size_t index)
{
    if (opt != LSO_OPT_ADAM && opt != LSO_OPT_SGD)
        return fail(LSO_E_DTYPE, "block %zu: unknown optimizer %u", index, opt);
    if (!std::isfinite(lr)) return fail(LSO_E_INVALID, "block %zu: lr is not finite", index);
    if (opt == LSO_OPT_SGD) return LSO_OK;
    if (t < 1) return fail(LSO_E_INVALID, "block %zu: t must be >= 1 (got %llu)", index,
                           static_cast<unsigned long long>(t));
    if (!(beta1 >= 0.0 && beta1 < 1.0))
        return fail(LSO_E_INVALID, "block %zu: beta1 must be in [0, 1)", index);
    if (!(beta2 >= 0.0 && beta2 < 1.0))
        return fail(LSO_E_INVALID, "block %zu: beta2 must be in [0, 1)", index);
    if (!(std::isfinite(eps) && eps >= 0.0))
        return fail(LSO_E_INVALID, "block %zu: eps must be finite and >= 0", index);
    return LSO_OK;
}

uint64_t tiled_bytes(uint64_t n)
{
    return 12ull * LSO_TILE_ELEMS * ((n + LSO_TILE_ELEMS - 1) / LSO_TILE_ELEMS);
}

namespace {

struct Interval {
    uintptr_t lo, hi;   // [lo, hi)
    bool written;
    size_t block;
};

lso_status check_overlap(std::vector<Interval>& iv)
{
    std::sort(iv.begin(), iv.end(), [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
    uintptr_t end_all = 0, end_written = 0;
    size_t blk_all = 0, blk_written = 0;
    for (const Interval& x : iv) {
        if (x.lo < end_written)
            return fail(LSO_E_OVERLAP, "block %zu: an array overlaps a written array of block %zu",
                        x.block, blk_written);
        if (x.written && x.lo < end_all)
            return fail(LSO_E_OVERLAP, "block %zu: a written array overlaps an array of block %zu",
                        x.block, blk_all);
        if (x.hi > end_all) { end_all = x.hi; blk_all = x.block; }
        if (x.written && x.hi > end_written) { end_written = x.hi; blk_written = x.block; }
    }
    return LSO_OK;
}

bool add_array(std::vector<Interval>& iv, uintptr_t addr, uint64_t bytes, bool written, size_t block)
{
    if (addr + bytes < addr) return false;   // wraps
    iv.push_back({addr, addr + bytes, written, block});
    return true;
}

}  // namespace

namespace {

// Every used array of the call as an interval (NULL, alignment and wrap
// checks on the way).
lso_status collect_geometry(const lso_block* blocks, size_t n, std::vector<Interval>& iv)
{
    iv.reserve(iv.size() + n * 5);
    for (size_t i = 0; i < n; ++i) {
        const lso_block& b = blocks[i];
        if (b.n == 0) continue;
        if (b.n > (UINT64_MAX / 8)) return fail(LSO_E_INVALID, "block %zu: n too large", i);
        const uintptr_t base = reinterpret_cast<uintptr_t>(b.base);
        const bool adam = b.opt == LSO_OPT_ADAM;
        const bool tiled = b.layout == LSO_LAYOUT_TILED;
        struct A { uint64_t off; uint64_t bytes; bool used; bool written; const char* name; } arr[5] = {
            {b.off_master, tiled ? tiled_bytes(b.n) : 4 * b.n, true, true, tiled ? "tiled state" : "master"},
            {b.off_m, 4 * b.n, adam && !tiled, true, "m"},
            {b.off_v, 4 * b.n, adam && !tiled, true, "v"},
            {b.off_grad, (b.grad_dtype == LSO_DT_F32 ? 4 : 2) * b.n, true, false, "grad"},
            {b.off_weight, 2 * b.n, b.weight_dtype == LSO_DT_BF16, true, "weight"},
        };
        for (const A& a : arr) {
            if (!a.used) continue;
            const uintptr_t addr = base + a.off;
            if (addr == 0) return fail(LSO_E_INVALID, "block %zu: %s address is NULL", i, a.name);
            if (addr % 16 != 0)
                return fail(LSO_E_ALIGN, "block %zu: %s address %#llx is not 16-byte aligned", i, a.name,
                            static_cast<unsigned long long>(addr));
            if (!add_array(iv, addr, a.bytes, a.written, i))
                return fail(LSO_E_INVALID, "block %zu: %s range wraps the address space", i, a.name);
        }
    }
    return LSO_OK;
}

}  // namespace

lso_status validate_geometry(const lso_block* blocks, size_t n)
{
    thread_local std::vector<Interval> iv;   // reused: no allocation once grown
    iv.clear();
    lso_status s = collect_geometry(blocks, n, iv);
    if (s != LSO_OK) return s;
    return check_overlap(iv);
}

lso_status validate_norm_buffers(const lso_block* blocks, size_t n, const NormOut& o)
{
    if (!o.sq_norms || !o.workspace) return fail(LSO_E_INVALID, "sq_norms and workspace must be non-NULL");
    if (reinterpret_cast<uintptr_t>(o.sq_norms) % 8 != 0 || reinterpret_cast<uintptr_t>(o.workspace) % 8 != 0)
        return fail(LSO_E_ALIGN, "sq_norms and workspace must be 8-byte aligned");
    const uint64_t need = norm_workspace_bytes(blocks, n);
    if (o.workspace_bytes < need)
        return fail(LSO_E_INVALID, "workspace of %llu bytes is smaller than the %llu this call needs",
                    static_cast<unsigned long long>(o.workspace_bytes), static_cast<unsigned long long>(need));
    lso_status s = validate_geometry(blocks, n);
    if (s != LSO_OK) return s;
    std::vector<Interval> iv;
    s = collect_geometry(blocks, n, iv);
    if (s != LSO_OK) return s;
    // both are written
    if (!add_array(iv, reinterpret_cast<uintptr_t>(o.sq_norms), 8ull * n, true, n) ||
        (need > 0 && !add_array(iv, reinterpret_cast<uintptr_t>(o.workspace), need, true, n)))
        return fail(LSO_E_INVALID, "sq_norms or workspace range wraps the address space");
    s = check_overlap(iv);
    if (s != LSO_OK) fail(s, "sq_norms or workspace overlaps an array of the call, or each other");
    return s;
}

lso_status check_fields(const lso_block& b, size_t i)
{
    if (b.layout != LSO_LAYOUT_PLANAR && b.layout != LSO_LAYOUT_TILED)
        return fail(LSO_E_INVALID, "block %zu: unknown layout %u", i, b.layout);
    if (b.layout == LSO_LAYOUT_TILED && b.opt != LSO_OPT_ADAM)
        return fail(LSO_E_DTYPE, "block %zu: the tiled state layout is for Adam only", i);
    if (b.grad_dtype != LSO_DT_BF16 && b.grad_dtype != LSO_DT_F32)
        return fail(LSO_E_DTYPE, "block %zu: gradient dtype must be BF16 or F32", i);
    if (b.weight_dtype != LSO_DT_BF16 && b.weight_dtype != LSO_DT_NONE)
        return fail(LSO_E_DTYPE, "block %zu: weight dtype must be BF16 or NONE", i);
    return check_hyper(b.opt, b.t, b.lr, b.beta1, b.beta2, b.eps, i);
}

lso_status validate_all(const lso_block* blocks, size_t n)
{
    if (n > 0 && !blocks) return fail(LSO_E_INVALID, "blocks is NULL");
    for (size_t i = 0; i < n; ++i) {
        lso_status s = check_fields(blocks[i], i);
        if (s != LSO_OK) return s;
    }
    return validate_geometry(blocks, n);
}

// --------------------------------------------------------------- constants

Coef make_coef(uint32_t opt, uint64_t t, double lr, double beta1, double beta2, double eps)
{
    Coef c{};
    if (opt == LSO_OPT_SGD) {
        c.s = static_cast<float>(lr);
        return c;
    }
    // Everything in FP64, rounded once to FP32: 1 - beta in FP32 would be
    // off by ~1e-5 relative for beta2 = 0.999.
    const double td = static_cast<double>(t);
    c.b1 = static_cast<float>(beta1);
    c.c1 = static_cast<float>(1.0 - beta1);
    c.b2 = static_cast<float>(beta2);
    c.c2 = static_cast<float>(1.0 - beta2);
    c.s = static_cast<float>(lr / (1.0 - std::pow(beta1, td)));
    c.r = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(beta2, td)));
    c.e = static_cast<float>(eps);
    return c;
}

// ------------------------------------------------------------------- plan

namespace {

struct HyperKey {
    uint32_t opt;
    uint64_t t;
    double lr, beta1, beta2, eps;
    bool operator==(const HyperKey& o) const
    {
        return opt == o.opt && t == o.t && lr == o.lr && beta1 == o.beta1 && beta2 == o.beta2 && eps == o.eps;
    }
};

HyperKey key_of(const lso_block& b)
{
    if (b.opt == LSO_OPT_SGD) return {b.opt, 0, b.lr, 0, 0, 0};
    return {b.opt, b.t, b.lr, b.beta1, b.beta2, b.eps};
}

// Device copies of block tables of more than kInline blocks (plus their
// per-chunk block index), cached by content so a training loop that passes
// the same blocks every step uploads its table once.  Per device; at most
// kCacheCap entries and kCacheBytes of device memory.  Uploads go through
// one page-locked staging buffer per device, reused (a new table waits
// until the previous upload has read it), so the cache holds no host
// memory.  Least recently used entries are evicted after a device
// synchronisation, because queued kernels on any stream may still read
// them; a loop that cycles through more tables than the cache holds pays
// that synchronisation on every new one.
struct TableEntry {
    std::vector<DevBlock> key;
    int unroll = 0;
    void* dev = nullptr;          // [DevBlock x n | uint32 index x chunks]
    size_t bytes = 0;
    hipEvent_t ready = nullptr;   // recorded after the upload
    bool ready_seen = false;
    void* upload_stream = nullptr;
    uint64_t tick = 0;
    bool has_index = false;
};

constexpr size_t kCacheCap = 256;
constexpr size_t kCacheBytes = 512ull << 20;

struct DeviceTables {
    std::vector<TableEntry> entries;
    uint64_t tick = 0;
    size_t bytes = 0;                    // device bytes of all entries
    void* staging = nullptr;             // page-locked upload buffer
    size_t staging_bytes = 0;
    hipEvent_t staging_read = nullptr;   // the last upload from it has been read
    bool staging_busy = false;
};

std::mutex g_mu;
std::unordered_map<int, DeviceTables> g_tables;

void free_entry(TableEntry& e)
{
    if (e.dev) (void)hipFree(e.dev);
    if (e.ready) (void)hipEventDestroy(e.ready);
    e = TableEntry{};
}

// The device's staging buffer, at least `bytes` large and no longer read by
// an earlier upload.
lso_status staging_for(DeviceTables& dt, size_t bytes)
{
    hipError_t err;
    if (!dt.staging_read) {
        err = hipEventCreateWithFlags(&dt.staging_read, hipEventDisableTiming);
        if (err != hipSuccess) { dt.staging_read = nullptr; return hip_fail(err, "hipEventCreateWithFlags"); }
    }
    if (dt.staging_busy) {
        err = hipEventSynchronize(dt.staging_read);
        if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize (table staging)");
        dt.staging_busy = false;
    }
    if (dt.staging_bytes < bytes) {
        if (dt.staging) (void)hipHostFree(dt.staging);
        dt.staging = nullptr;
        dt.staging_bytes = 0;
        const size_t want = (bytes + (1u << 20) - 1) & ~size_t((1u << 20) - 1);
        if (hipHostMalloc(&dt.staging, want, hipHostMallocDefault) != hipSuccess) {
            dt.staging = nullptr;
            return fail(LSO_E_NOMEM, "hipHostMalloc of a %zu-byte table staging buffer failed", want);
        }
        dt.staging_bytes = want;
    }
    return LSO_OK;
}

bool same_table(const TableEntry& e, const std::vector<DevBlock>& tab, int unroll)
{
    return e.unroll == unroll && e.key.size() == tab.size() &&
           std::memcmp(e.key.data(), tab.data(), tab.size() * sizeof(DevBlock)) == 0;
}

// Find the cached device table for tab, or validate the call's addresses,
// upload tab (and its chunk index) on stream and cache it.
lso_status device_table(const lso_block* blocks, size_t n, bool geometry_checked,
                        const std::vector<DevBlock>& tab, uint64_t total_chunks, int unroll,
                        void* stream, KernelArgs& args)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceTables& dt = g_tables[dev];
    ++dt.tick;
    for (TableEntry& e : dt.entries) {
        if (!same_table(e, tab, unroll)) continue;
        e.tick = dt.tick;
        if (!e.ready_seen) {
            if (hipEventQuery(e.ready) == hipSuccess) {
                e.ready_seen = true;
            } else if (stream != e.upload_stream) {
                err = hipStreamWaitEvent(static_cast<hipStream_t>(stream), e.ready, 0);
                if (err != hipSuccess) return hip_fail(err, "hipStreamWaitEvent");
            }
        }
        args.blocks = static_cast<const DevBlock*>(e.dev);
        args.chunk_block = e.has_index
            ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(e.dev) + tab.size() * sizeof(DevBlock))
            : nullptr;
        return LSO_OK;
    }
    // a new table: its addresses are checked once, here
    if (!geometry_checked) {
        lso_status s = validate_geometry(blocks, n);
        if (s != LSO_OK) return s;
    }
    const bool has_index = total_chunks <= kMaxIndexChunks;
    const size_t tab_bytes = tab.size() * sizeof(DevBlock);
    const size_t bytes = tab_bytes + (has_index ? total_chunks * sizeof(uint32_t) : 0);
    if (dt.entries.size() >= kCacheCap || (!dt.entries.empty() && dt.bytes + bytes > kCacheBytes)) {
        err = hipDeviceSynchronize();
        if (err != hipSuccess) return hip_fail(err, "hipDeviceSynchronize (table eviction)");
        while (!dt.entries.empty() && (dt.entries.size() >= kCacheCap || dt.bytes + bytes > kCacheBytes)) {
            auto lru = std::min_element(dt.entries.begin(), dt.entries.end(),
                                        [](const TableEntry& a, const TableEntry& b) { return a.tick < b.tick; });
            dt.bytes -= lru->bytes;
            free_entry(*lru);
            dt.entries.erase(lru);
        }
    }
    lso_status st = staging_for(dt, bytes);
    if (st != LSO_OK) return st;
    TableEntry e;
    e.key = tab;
    e.unroll = unroll;
    e.tick = dt.tick;
    e.upload_stream = stream;
    e.has_index = has_index;
    e.bytes = bytes;
    if (hipMalloc(&e.dev, bytes) != hipSuccess) {
        free_entry(e);
        return fail(LSO_E_NOMEM, "hipMalloc of a %zu-byte block table failed", bytes);
    }
    std::memcpy(dt.staging, tab.data(), tab_bytes);
    if (e.has_index) {
        uint32_t* idx = reinterpret_cast<uint32_t*>(static_cast<char*>(dt.staging) + tab_bytes);
        for (size_t k = 0; k < tab.size(); ++k) {
            const uint64_t end = k + 1 < tab.size() ? tab[k + 1].chunk0 : total_chunks;
            for (uint64_t c = tab[k].chunk0; c < end; ++c) idx[c] = static_cast<uint32_t>(k);
        }
    }
    err = hipEventCreateWithFlags(&e.ready, hipEventDisableTiming);
    if (err != hipSuccess) { free_entry(e); return hip_fail(err, "hipEventCreateWithFlags"); }
    err = hipMemcpyAsync(e.dev, dt.staging, bytes, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) { free_entry(e); return hip_fail(err, "hipMemcpyAsync (block table)"); }
    err = hipEventRecord(e.ready, static_cast<hipStream_t>(stream));
    if (err == hipSuccess) err = hipEventRecord(dt.staging_read, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        // the copy is queued: let it finish before its buffers go
        (void)hipStreamSynchronize(static_cast<hipStream_t>(stream));
        free_entry(e);
        return hip_fail(err, "hipEventRecord");
    }
    dt.staging_busy = true;
    dt.bytes += bytes;
    args.blocks = static_cast<const DevBlock*>(e.dev);
    args.chunk_block = e.has_index
        ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(e.dev) + tab_bytes)
        : nullptr;
    dt.entries.push_back(std::move(e));
    return LSO_OK;
}

}  // namespace

namespace {

int kind_of(const lso_block& b)
{
    return (b.layout == LSO_LAYOUT_TILED ? 1 : 0) + (b.grad_dtype == LSO_DT_F32 ? 2 : 0);
}

// Chunk size of each launch kind of a call: planar chunks by the planar
// work of the call (small calls take small chunks to fill the chip), tiled
// chunks are one state tile.
int planar_unroll_of(const lso_block* blocks, size_t n)
{
    uint64_t planar_elems = 0;
    for (size_t i = 0; i < n; ++i)
        if (blocks[i].layout != LSO_LAYOUT_TILED) planar_elems += blocks[i].n;
    return planar_elems < kSmallCallElems ? kUnrollSmall : kUnrollLarge;
}

}  // namespace

uint64_t norm_workspace_bytes(const lso_block* blocks, size_t n)
{
    if (!blocks) return 0;
    const uint64_t planar_chunk = chunk_elems(planar_unroll_of(blocks, n));
    uint64_t chunks = 0;
    for (size_t i = 0; i < n; ++i) {
        const uint64_t c = blocks[i].layout == LSO_LAYOUT_TILED ? chunk_elems(kUnrollTiled) : planar_chunk;
        chunks += (blocks[i].n + c - 1) / c;
    }
    return chunks * kNormPartsPerChunk * sizeof(double);
}

namespace {

// The update of one call: one launch per (launch kind, 16 constant sets).
// A launch's table of more than kInline blocks lives in a cached device
// table (allocated on first sight), or with noalloc in the device's fixed
// scratch array (written on the stream every call).
lso_status enqueue_impl(const lso_block* blocks, size_t n, void* stream, bool geometry_checked,
                        const NormOut* norms, bool noalloc)
{
    if (n == 0) return LSO_OK;
    if (!blocks) return fail(LSO_E_INVALID, "blocks is NULL");
    if (n > kMaxBlocksPerCall) return fail(LSO_E_INVALID, "more than 2^24 blocks in one call");
    // per-thread scratch, reused across calls (no allocation in steady state)
    thread_local std::vector<HyperKey> sets;
    thread_local std::vector<uint32_t> set_of;
    thread_local std::vector<DevBlock> tab;
    sets.clear();
    set_of.resize(n);
    for (size_t i = 0; i < n; ++i) {
        lso_status s = check_fields(blocks[i], i);
        if (s != LSO_OK) return s;
        const HyperKey k = key_of(blocks[i]);
        size_t j = 0;
        while (j < sets.size() && !(sets[j] == k)) ++j;
        if (j == sets.size()) sets.push_back(k);
        set_of[i] = static_cast<uint32_t>(j);
    }
    // launches: one per launch kind ((tiled or planar) x (BF16 or FP32
    // gradients)) and per 16 constant sets
    bool present[4] = {false, false, false, false};
    for (size_t i = 0; i < n; ++i) present[kind_of(blocks[i])] = true;
    const int kinds = present[0] + present[1] + present[2] + present[3];
    const int planar_unroll = planar_unroll_of(blocks, n);
    uint64_t part_offset = 0;   // norm variant: this launch's first partial
    const size_t set_groups = (sets.size() + kMaxGroups - 1) / kMaxGroups;
    const size_t launches = set_groups * static_cast<size_t>(kinds);
    bool checked = geometry_checked;
    DevBlock* scratch = nullptr;
    size_t scratch_used = 0;
    if (noalloc) {
        // every table of the call must fit the scratch array; checked (with
        // the addresses) before anything is enqueued
        size_t need = 0;
        for (int kind = 0; kind < 4; ++kind) {
            if (!present[kind]) continue;
            for (size_t L = 0; L < set_groups; ++L) {
                size_t cnt = 0;
                for (size_t i = 0; i < n; ++i)
                    cnt += blocks[i].n != 0 && kind_of(blocks[i]) == kind && set_of[i] / kMaxGroups == L;
                if (cnt > static_cast<size_t>(kInline)) need += cnt;
            }
        }
        if (need > LSO_NOALLOC_MAX_BLOCKS)
            return fail(LSO_E_INVALID, "%zu block-table entries exceed the %u of lso_adam_step_noalloc", need,
                        static_cast<unsigned>(LSO_NOALLOC_MAX_BLOCKS));
        if (!checked) {
            lso_status s = validate_geometry(blocks, n);
            if (s != LSO_OK) return s;
            checked = true;
        }
        if (need > 0) {
            lso_status s = noalloc_scratch(&scratch, stream);
            if (s != LSO_OK) return s;
        }
    }
    if (launches > 1 && !checked) {
        // overlaps across the launches of one call are checked up front, so
        // an error never follows a launch already enqueued
        lso_status s = validate_geometry(blocks, n);
        if (s != LSO_OK) return s;
        checked = true;
    }
    for (int kind = 0; kind < 4; ++kind) {   // one pass per launch kind present
        if (!present[kind]) continue;
        const bool tiled_pass = (kind & 1) != 0;
        const bool g32_pass = (kind & 2) != 0;
        const int unroll = tiled_pass ? kUnrollTiled : planar_unroll;
        const uint64_t chunk = chunk_elems(unroll);
        for (size_t L = 0; L < set_groups; ++L) {
            KernelArgs args{};
            tab.clear();
            uint64_t chunks = 0;
            for (size_t i = 0; i < n; ++i) {
                if (set_of[i] / kMaxGroups != L) continue;
                const lso_block& b = blocks[i];
                if (kind_of(b) != kind) continue;
                if (b.n == 0) continue;
                const uintptr_t base = reinterpret_cast<uintptr_t>(b.base);
                DevBlock d{};
                d.master = reinterpret_cast<float*>(base + b.off_master);
                if (b.opt == LSO_OPT_ADAM && !tiled_pass) {
                    d.m = reinterpret_cast<float*>(base + b.off_m);
                    d.v = reinterpret_cast<float*>(base + b.off_v);
                }
                d.g = reinterpret_cast<const uint16_t*>(base + b.off_grad);
                d.w = b.weight_dtype == LSO_DT_BF16 ? reinterpret_cast<uint16_t*>(base + b.off_weight) : nullptr;
                d.n = b.n;
                d.chunk0 = chunks;
                d.group = set_of[i] % kMaxGroups;
                d.flags = (b.opt == LSO_OPT_SGD ? kFlagSgd : 0u) | (d.w ? kFlagWeight : 0u) |
                          (tiled_pass ? kFlagTiled : 0u) | (g32_pass ? kFlagGradF32 : 0u) |
                          (static_cast<uint32_t>(i) << kIndexShift);
                chunks += (b.n + chunk - 1) / chunk;
                tab.push_back(d);
            }
            for (size_t j = L * kMaxGroups; j < sets.size() && j < (L + 1) * kMaxGroups; ++j) {
                const HyperKey& k = sets[j];
                args.coef[j % kMaxGroups] = make_coef(k.opt, k.t, k.lr, k.beta1, k.beta2, k.eps);
            }
            args.ngroups = static_cast<uint32_t>(std::min<size_t>(kMaxGroups, sets.size() - L * kMaxGroups));
            if (tab.empty()) continue;
            args.total_chunks = chunks;
            args.nblocks = static_cast<uint32_t>(tab.size());
            if (tab.size() <= static_cast<size_t>(kInline)) {
                // The address checks of a by-value table are remembered per
                // thread: a loop passing the same few blocks every step skips
                // them (the table holds every address and size they look at).
                thread_local DevBlock last_ok[kInline];
                thread_local size_t last_ok_n = 0;
                const bool same = last_ok_n == tab.size() &&
                                  std::memcmp(last_ok, tab.data(), tab.size() * sizeof(DevBlock)) == 0;
                if (!checked && !same) {
                    lso_status s = validate_geometry(blocks, n);
                    if (s != LSO_OK) return s;
                    checked = true;
                }
                if (launches == 1) {
                    std::memcpy(last_ok, tab.data(), tab.size() * sizeof(DevBlock));
                    last_ok_n = tab.size();
                }
                // by value, block j carries its constants in coef[j]
                Coef mine[kInline];
                for (size_t j = 0; j < tab.size(); ++j) mine[j] = args.coef[tab[j].group];
                for (size_t j = 0; j < tab.size(); ++j) {
                    args.inl[j] = tab[j];
                    args.inl[j].group = static_cast<uint32_t>(j);
                    args.coef[j] = mine[j];
                }
            } else if (noalloc) {
                lso_status s = noalloc_write_table(scratch + scratch_used, tab.data(), tab.size(), stream);
                if (s != LSO_OK) return s;
                args.blocks = scratch + scratch_used;
                args.chunk_block = nullptr;   // the kernel searches the table
                scratch_used += tab.size();
            } else {
                lso_status s = device_table(blocks, n, checked, tab, chunks, unroll, stream, args);
                if (s != LSO_OK) return s;
            }
            if (norms) args.partials = norms->workspace + part_offset * kNormPartsPerChunk;
            int err = launch_fused_adam(args, unroll, tiled_pass, g32_pass, stream);
            if (err != 0) return hip_fail(err, "fused Adam launch");
            count_launch();
            if (norms) {
                err = launch_norm_reduce(args, unroll, norms->sq_norms, stream);
                if (err != 0) return hip_fail(err, "norm reduction launch");
                part_offset += chunks;
            }
        }
    }
    return LSO_OK;
}

}  // namespace

lso_status enqueue_update(const lso_block* blocks, size_t n, void* stream, bool geometry_checked,
                          const NormOut* norms)
{
    return enqueue_impl(blocks, n, stream, geometry_checked, norms, false);
}

lso_status enqueue_update_noalloc(const lso_block* blocks, size_t n, void* stream)
{
    return enqueue_impl(blocks, n, stream, false, nullptr, true);
}

}  // namespace lso

// ================================================================== C ABI

extern "C" {

lso_status lso_adam_step(const lso_block* blocks, size_t n, void* stream)
{
    lso::clear_error();
    lso_status s = lso::enqueue_update(blocks, n, stream, false);
    if (s == LSO_OK && n > 0) {
        // so a caller that captures lso_adam_step_noalloc later finds the
        // allocation-free path's array already looked up on this device
        thread_local int looked_up = -1;
        int dev = -1;
        if (hipGetDevice(&dev) == hipSuccess && dev != looked_up) {
            lso::DevBlock* p = nullptr;
            if (lso::noalloc_scratch(&p, stream) == LSO_OK) looked_up = dev;
            lso::clear_error();
        }
    }
    return s;
}

uint64_t lso_norm_workspace_bytes(const lso_block* blocks, size_t n)
{
    return lso::norm_workspace_bytes(blocks, n);
}

lso_status lso_adam_step_norms(const lso_block* blocks, size_t n, double* sq_norms, void* workspace,
                               uint64_t workspace_bytes, void* stream)
{
    lso::clear_error();
    if (n == 0) return LSO_OK;
    if (!blocks) return lso::fail(LSO_E_INVALID, "blocks is NULL");
    lso::NormOut o;
    o.sq_norms = sq_norms;
    o.workspace = static_cast<double*>(workspace);
    o.workspace_bytes = workspace_bytes;
    for (size_t i = 0; i < n; ++i) {
        lso_status s = lso::check_fields(blocks[i], i);
        if (s != LSO_OK) return s;
    }
    lso_status s = lso::validate_norm_buffers(blocks, n, o);   // covers the blocks' geometry
    if (s != LSO_OK) return s;
    return lso::enqueue_update(blocks, n, stream, true, &o);
}

uint64_t lso_tiled_state_bytes(uint64_t n) { return lso::tiled_bytes(n); }

uint64_t lso_kernel_launches(void) { return lso::g_launches.load(std::memory_order_relaxed); }

lso_status lso_validate_blocks(const lso_block* blocks, size_t n)
{
    lso::clear_error();
    return lso::validate_all(blocks, n);
}

lso_status lso_block_constants(const lso_block* block, float out[8])
{
    lso::clear_error();
    if (!block || !out) return lso::fail(LSO_E_INVALID, "NULL argument");
    lso_status s = lso::check_hyper(block->opt, block->t, block->lr, block->beta1, block->beta2,
                                    block->eps, 0);
    if (s != LSO_OK) return s;
    const lso::Coef c = lso::make_coef(block->opt, block->t, block->lr, block->beta1, block->beta2,
                                       block->eps);
    const float v[8] = {c.b1, c.c1, c.b2, c.c2, c.s, c.r, c.e, 0.0f};
    std::memcpy(out, v, sizeof v);
    return LSO_OK;
}

lso_status lso_host_alloc(uint64_t bytes, void** out)
{
    lso::clear_error();
    if (!out || bytes == 0) return lso::fail(LSO_E_INVALID, "bytes must be > 0 and out non-NULL");
    *out = nullptr;
    void* p = nullptr;
    hipError_t err = hipHostMalloc(&p, bytes, hipHostMallocDefault);
    if (err != hipSuccess || !p)
        return lso::fail(LSO_E_NOMEM, "hipHostMalloc(%llu) failed: %s", static_cast<unsigned long long>(bytes),
                         hipGetErrorString(err));
    *out = p;
    return LSO_OK;
}

lso_status lso_host_free(void* p)
{
    lso::clear_error();
    if (!p) return LSO_OK;
    hipError_t err = hipHostFree(p);
    return err == hipSuccess ? LSO_OK : lso::hip_fail(err, "hipHostFree");
}

const char* lso_status_string(lso_status s)
{
    // a C caller may pass any int; read it as one (a C++ load of an enum
    // holding a value outside its range is undefined)
    int code = 0;
    static_assert(sizeof code == sizeof s, "lso_status is int-sized");
    std::memcpy(&code, &s, sizeof code);
    switch (code) {
    case LSO_OK: return "ok";
    case LSO_E_INVALID: return "invalid argument";
    case LSO_E_ALIGN: return "misaligned array";
    case LSO_E_DTYPE: return "unsupported dtype or optimizer";
    case LSO_E_OVERLAP: return "overlapping arrays";
    case LSO_E_NOMEM: return "out of memory";
    case LSO_E_HIP: return "HIP runtime error";
    case LSO_E_CALLBACK: return "gradient producer failed";
    case LSO_E_IO: return "file read or write failed";
    }
    return "unknown status";
}

const char* lso_last_error(void) { return lso::t_last_error; }

}  // extern "C"
