// Layer streaming: CPU-authoritative state, GPU as a transient update engine.
//
// MegaTrain summary (blog.hotdry.top), section on streaming execution and
// the double-buffered pipeline: each layer's state is one contiguous,
// page-aligned host block moved by one burst DMA; two sets of staging
// buffers (CPU side and GPU side) alternate so the next layer loads while
// the current one computes; three streams (weight transfer H2D, compute,
// transfer back D2H) are tied only by events -- weights-ready, backward-done
// (here: step-done) and buffer-free -- with no host barrier in the GPU
// pipeline; the slot size is the largest layer (section on key engineering
// parameters).  The write-back of each layer is the frozen-incremental
// page's "stored W += delta": the device computes master + delta and the
// updated block overwrites the authoritative host copy.
//
// Per layer i, slot s = i % 2:
//   H2D:     wait buffer-free[s]; copy src[i] -> slot[s]; record weights-ready[s]
//   compute: wait weights-ready[s]; gradient producer; fused update;
//            record step-done[s]
//   D2H:     wait step-done[s]; copy slot[s] -> dst[i]; record buffer-free[s]
// Every wait refers to an event recorded earlier in host order.
//
// Each copy is one burst over the whole block, issued by a copy kernel on
// the transfer stream (lso_copy.hip says why not the DMA engines; set
// LSO_STREAM_COPY=dma to use them).
//
// Two kinds of host block:
//  - pinned (page-locked, e.g. lso_host_alloc): src = dst = the block itself,
//    one copy each way, and the host thread never waits inside the loop;
//  - pageable: the DMA engines cannot reach it, so the block goes through
//    the context's two pinned CPU-side staging buffers; worker threads copy
//    it in before its H2D and back out after its D2H (the host waits for
//    that D2H only, two layers behind the one it is issuing).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "lso_copy.h"
#include "lso_runtime.h"

namespace {

// A fixed pool that splits one memcpy over all its threads.
class CopyPool {
public:
    explicit CopyPool(unsigned n) : n_(n ? n : 1)
    {
        for (unsigned k = 1; k < n_; ++k) workers_.emplace_back([this, k] { run(k); });
    }
    ~CopyPool()
    {
        {
            std::lock_guard<std::mutex> l(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : workers_) t.join();
    }
    // dst[0..bytes) = src[0..bytes), split in n contiguous parts.
    void copy(void* dst, const void* src, uint64_t bytes)
    {
        {
            std::lock_guard<std::mutex> l(mu_);
            dst_ = static_cast<char*>(dst);
            src_ = static_cast<const char*>(src);
            bytes_ = bytes;
            pending_ = n_ - 1;
            ++gen_;
        }
        cv_.notify_all();
        part(0);
        std::unique_lock<std::mutex> l(mu_);
        done_cv_.wait(l, [this] { return pending_ == 0; });
    }

private:
    void part(unsigned k)
    {
        const uint64_t per = (bytes_ / n_ + 4095) & ~uint64_t(4095);
        const uint64_t lo = std::min<uint64_t>(bytes_, per * k);
        const uint64_t hi = std::min<uint64_t>(bytes_, lo + per);
        if (hi > lo) std::memcpy(dst_ + lo, src_ + lo, hi - lo);
    }
    void run(unsigned k)
    {
        uint64_t seen = 0;
        for (;;) {
            {
                std::unique_lock<std::mutex> l(mu_);
                cv_.wait(l, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
            }
            part(k);
            {
                std::lock_guard<std::mutex> l(mu_);
                if (--pending_ == 0) done_cv_.notify_one();
            }
        }
    }
    unsigned n_;
    std::vector<std::thread> workers_;
    std::mutex mu_;
    std::condition_variable cv_, done_cv_;
    bool stop_ = false;
    uint64_t gen_ = 0;
    unsigned pending_ = 0;
    char* dst_ = nullptr;
    const char* src_ = nullptr;
    uint64_t bytes_ = 0;
};

}  // namespace

constexpr int kMaxSlots = 4;

// Which engine moves each direction of a layer block.
enum CopyMode { kCopyKernels = 0, kCopyDma = 1, kCopyDmaIn = 2 };

struct lso_stream_ctx {
    int device = 0;
    uint64_t max_bytes = 0;
    uint64_t max_params = 0;
    lso_grad_fn fn = nullptr;
    void* user = nullptr;
    int nslots = 2;
    hipStream_t h2d = nullptr, compute = nullptr, d2h = nullptr;
    void* slot_state[kMaxSlots] = {};
    void* slot_grad[kMaxSlots] = {};
    void* slot_weight[kMaxSlots] = {};
    void* staging[kMaxSlots + 1] = {};   // pinned, allocated on first pageable layer
    hipEvent_t weights_ready[kMaxSlots] = {};
    hipEvent_t step_done[kMaxSlots] = {};
    hipEvent_t buffer_free[kMaxSlots] = {};
    hipEvent_t d2h_done[kMaxSlots + 1] = {};   // per staging buffer: its layer's D2H ended
    CopyPool* pool = nullptr;
    int copy_mode = kCopyKernels;
    unsigned copy_grid = lso::kCopyGrid;
};

namespace {

uint64_t round16(uint64_t x) { return (x + 15) & ~uint64_t(15); }

void release(lso_stream_ctx* c)
{
    if (!c) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    for (hipStream_t s : {c->h2d, c->compute, c->d2h})
        if (s) (void)hipStreamSynchronize(s);
    for (int s = 0; s <= kMaxSlots; ++s) {
        if (c->staging[s]) (void)hipHostFree(c->staging[s]);
        if (c->d2h_done[s]) (void)hipEventDestroy(c->d2h_done[s]);
    }
    for (int s = 0; s < kMaxSlots; ++s) {
        if (c->slot_state[s]) (void)hipFree(c->slot_state[s]);
        if (c->slot_grad[s]) (void)hipFree(c->slot_grad[s]);
        if (c->slot_weight[s]) (void)hipFree(c->slot_weight[s]);
        if (c->weights_ready[s]) (void)hipEventDestroy(c->weights_ready[s]);
        if (c->step_done[s]) (void)hipEventDestroy(c->step_done[s]);
        if (c->buffer_free[s]) (void)hipEventDestroy(c->buffer_free[s]);
    }
    for (hipStream_t s : {c->h2d, c->compute, c->d2h})
        if (s) (void)hipStreamDestroy(s);
    delete c->pool;
    (void)hipSetDevice(prev);
    delete c;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        (void)hipSetDevice(dev);
    }
    ~DeviceGuard()
    {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// True if the DMA engines can reach the whole block (page-locked host
// memory registered with HIP); false for ordinary pageable memory.
bool is_pinned(const void* p, uint64_t bytes)
{
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();   // pageable memory is not an error here
        return false;
    }
    if (a.type != hipMemoryTypeHost) return false;
    // the block must lie inside one allocation; check its last byte too
    hipPointerAttribute_t b{};
    const void* last = static_cast<const char*>(p) + (bytes - 1);
    if (hipPointerGetAttributes(&b, last) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return b.type == hipMemoryTypeHost;
}

lso_status check_layer(const lso_stream_ctx* c, const lso_host_layer& L, size_t i)
{
    using lso::fail;
    if (!L.host_base) return fail(LSO_E_INVALID, "layer %zu: host_base is NULL", i);
    if (L.layout != LSO_LAYOUT_PLANAR && L.layout != LSO_LAYOUT_TILED)
        return fail(LSO_E_INVALID, "layer %zu: unknown layout %u", i, L.layout);
    if (L.layout == LSO_LAYOUT_TILED && L.opt != LSO_OPT_ADAM)
        return fail(LSO_E_DTYPE, "layer %zu: the tiled state layout is for Adam only", i);
    lso_status s = lso::check_hyper(L.opt, L.t, L.lr, L.beta1, L.beta2, L.eps, i);
    if (s != LSO_OK) return s;
    if (L.bytes == 0 || L.bytes > c->max_bytes)
        return fail(LSO_E_INVALID, "layer %zu: bytes %llu outside (0, %llu]", i,
                    static_cast<unsigned long long>(L.bytes), static_cast<unsigned long long>(c->max_bytes));
    if (L.n > c->max_params)
        return fail(LSO_E_INVALID, "layer %zu: %llu params exceed the context's %llu", i,
                    static_cast<unsigned long long>(L.n), static_cast<unsigned long long>(c->max_params));
    if (reinterpret_cast<uintptr_t>(L.host_base) % 16 != 0)
        return fail(LSO_E_ALIGN, "layer %zu: host block is not 16-byte aligned", i);
    if (L.dev_weight && reinterpret_cast<uintptr_t>(L.dev_weight) % 16 != 0)
        return fail(LSO_E_ALIGN, "layer %zu: dev_weight is not 16-byte aligned", i);
    if (L.layout == LSO_LAYOUT_TILED) {
        const uint64_t rb = lso::tiled_bytes(L.n);
        if (L.off_master % 16 != 0) return fail(LSO_E_ALIGN, "layer %zu: state offset not 16-byte aligned", i);
        if (L.off_master > L.bytes || rb > L.bytes - L.off_master)
            return fail(LSO_E_INVALID, "layer %zu: the tiled state runs past the block's bytes", i);
        return LSO_OK;
    }
    const bool adam = L.opt == LSO_OPT_ADAM;
    const uint64_t arr_bytes = 4 * L.n;
    const uint64_t offs[3] = {L.off_master, L.off_m, L.off_v};
    const int used = adam ? 3 : 1;
    for (int k = 0; k < used; ++k) {
        if (offs[k] % 16 != 0) return fail(LSO_E_ALIGN, "layer %zu: array offset not 16-byte aligned", i);
        if (offs[k] > L.bytes || arr_bytes > L.bytes - offs[k])
            return fail(LSO_E_INVALID, "layer %zu: an array runs past the block's bytes", i);
    }
    for (int a = 0; a < used; ++a)
        for (int b = a + 1; b < used; ++b)
            if (L.n > 0 && offs[a] < offs[b] + arr_bytes && offs[b] < offs[a] + arr_bytes)
                return fail(LSO_E_OVERLAP, "layer %zu: master/m/v overlap inside the block", i);
    return LSO_OK;
}

// Staging buffers: one more than device slots, so a layer can be copied in
// while the layer two slots back is still on its way out.
int staging_count(const lso_stream_ctx* c) { return c->nslots + 1; }

lso_status ensure_staging(lso_stream_ctx* c)
{
    for (int s = 0; s < staging_count(c); ++s) {
        if (c->staging[s]) continue;
        if (hipHostMalloc(&c->staging[s], c->max_bytes, hipHostMallocDefault) != hipSuccess) {
            (void)hipGetLastError();
            c->staging[s] = nullptr;
            return lso::fail(LSO_E_NOMEM, "pinned staging buffer of %llu bytes",
                             static_cast<unsigned long long>(c->max_bytes));
        }
    }
    if (!c->pool) {
        unsigned n = std::thread::hardware_concurrency();
        c->pool = new (std::nothrow) CopyPool(std::min(n ? n : 1u, 16u));
        if (!c->pool) return lso::fail(LSO_E_NOMEM, "copy pool");
    }
    return LSO_OK;
}

// One block copy between a page-locked host buffer and a device slot: a
// copy kernel by default (full duplex), or the DMA engines.
hipError_t copy_block(const lso_stream_ctx* c, void* dst, const void* src, uint64_t bytes,
                      hipMemcpyKind kind, hipStream_t st)
{
    const bool dma = c->copy_mode == kCopyDma ||
                     (c->copy_mode == kCopyDmaIn && kind == hipMemcpyHostToDevice);
    if (dma) return hipMemcpyAsync(dst, src, bytes, kind, st);
    return static_cast<hipError_t>(lso::launch_block_copy(dst, src, bytes, c->copy_grid, st));
}

// Enqueue H2D, gradient producer, update and D2H of layer i (slot i % nslots).
// src/dst: where the H2D reads and the D2H writes (the block itself when
// pinned, the slot's staging buffer otherwise).
lso_status issue_layer(lso_stream_ctx* c, const lso_host_layer& h, size_t i, void* src, void* dst)
{
    const int s = static_cast<int>(i % c->nslots);
    hipError_t err;
    // StreamIn: the device slot is free once the layer that used it last
    // (nslots layers ago) has been copied back.
    if ((err = hipStreamWaitEvent(c->h2d, c->buffer_free[s], 0)) != hipSuccess ||
        (err = copy_block(c, c->slot_state[s], src, h.bytes, hipMemcpyHostToDevice, c->h2d)) != hipSuccess ||
        (err = hipEventRecord(c->weights_ready[s], c->h2d)) != hipSuccess)
        return lso::hip_fail(err, "H2D stage");
    // Compute: gradients of this layer, then the fused update on the slot.
    if ((err = hipStreamWaitEvent(c->compute, c->weights_ready[s], 0)) != hipSuccess)
        return lso::hip_fail(err, "hipStreamWaitEvent(weights-ready)");
    const int rc = c->fn(c->user, i, c->slot_grad[s], h.n, c->compute);
    if (rc != 0) return lso::fail(LSO_E_CALLBACK, "gradient producer returned %d at layer %zu", rc, i);
    lso_block b{};
    const uintptr_t base = reinterpret_cast<uintptr_t>(c->slot_state[s]);
    b.base = nullptr;   // absolute addresses below
    b.n = h.n;
    b.off_master = base + h.off_master;
    b.off_m = base + h.off_m;
    b.off_v = base + h.off_v;
    b.off_grad = reinterpret_cast<uintptr_t>(c->slot_grad[s]);
    b.off_weight = reinterpret_cast<uintptr_t>(h.dev_weight ? h.dev_weight : c->slot_weight[s]);
    b.grad_dtype = LSO_DT_BF16;
    b.weight_dtype = LSO_DT_BF16;
    b.opt = h.opt;
    b.layout = h.layout;
    b.t = h.t;
    b.lr = h.lr;
    b.beta1 = h.beta1;
    b.beta2 = h.beta2;
    b.eps = h.eps;
    lso_status st = lso::enqueue_update(&b, 1, c->compute, false);
    if (st != LSO_OK) return st;
    if ((err = hipEventRecord(c->step_done[s], c->compute)) != hipSuccess)
        return lso::hip_fail(err, "hipEventRecord(step-done)");
    // Offload: the updated block goes back over the authoritative copy.
    if ((err = hipStreamWaitEvent(c->d2h, c->step_done[s], 0)) != hipSuccess ||
        (err = copy_block(c, dst, c->slot_state[s], h.bytes, hipMemcpyDeviceToHost, c->d2h)) != hipSuccess ||
        (err = hipEventRecord(c->buffer_free[s], c->d2h)) != hipSuccess ||
        (err = hipEventRecord(c->d2h_done[i % (c->nslots + 1)], c->d2h)) != hipSuccess)
        return lso::hip_fail(err, "D2H stage");
    return LSO_OK;
}

}  // namespace

extern "C" {

lso_status lso_stream_create(uint64_t max_layer_bytes, uint64_t max_layer_params, lso_grad_fn fn,
                             void* user, int device, lso_stream_ctx** out)
{
    lso::clear_error();
    if (!out) return lso::fail(LSO_E_INVALID, "out is NULL");
    *out = nullptr;
    if (max_layer_bytes == 0 || !fn)
        return lso::fail(LSO_E_INVALID, "max_layer_bytes must be > 0 and fn non-NULL");
    int ndev = 0;
    hipError_t err = hipGetDeviceCount(&ndev);
    if (err != hipSuccess) return lso::hip_fail(err, "hipGetDeviceCount");
    if (device < 0 || device >= ndev) return lso::fail(LSO_E_INVALID, "device %d out of range", device);
    DeviceGuard guard(device);
    auto* c = new (std::nothrow) lso_stream_ctx;
    if (!c) return lso::fail(LSO_E_NOMEM, "context allocation failed");
    c->device = device;
    c->max_bytes = max_layer_bytes;
    c->max_params = max_layer_params;
    c->fn = fn;
    c->user = user;
    if (const char* e = std::getenv("LSO_STREAM_COPY")) {
        if (!std::strcmp(e, "dma")) c->copy_mode = kCopyDma;
        else if (!std::strcmp(e, "dma-in")) c->copy_mode = kCopyDmaIn;
    }
    if (const char* e = std::getenv("LSO_STREAM_SLOTS")) {
        const int k = std::atoi(e);
        if (k >= 2 && k <= kMaxSlots) c->nslots = k;
    }
    if (const char* e = std::getenv("LSO_STREAM_COPY_GRID")) {
        const int k = std::atoi(e);
        if (k >= 1 && k <= 4096) c->copy_grid = static_cast<unsigned>(k);
    }
    // default priority on all three (different priorities are not used)
    for (hipStream_t* s : {&c->h2d, &c->compute, &c->d2h}) {
        err = hipStreamCreateWithFlags(s, hipStreamNonBlocking);
        if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipStreamCreateWithFlags"); }
    }
    const uint64_t pbytes = round16(2 * (max_layer_params ? max_layer_params : 1));
    for (int s = 0; s < c->nslots; ++s) {
        if (hipMalloc(&c->slot_state[s], max_layer_bytes) != hipSuccess ||
            hipMalloc(&c->slot_grad[s], pbytes) != hipSuccess ||
            hipMalloc(&c->slot_weight[s], pbytes) != hipSuccess) {
            release(c);
            return lso::fail(LSO_E_NOMEM, "slot allocation (%llu + 2 x %llu bytes) failed",
                             static_cast<unsigned long long>(max_layer_bytes),
                             static_cast<unsigned long long>(pbytes));
        }
        for (hipEvent_t* e : {&c->weights_ready[s], &c->step_done[s], &c->buffer_free[s]}) {
            err = hipEventCreateWithFlags(e, hipEventDisableTiming);
            if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipEventCreateWithFlags"); }
        }
    }
    for (int s = 0; s <= c->nslots; ++s) {
        err = hipEventCreateWithFlags(&c->d2h_done[s], hipEventDisableTiming);
        if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipEventCreateWithFlags"); }
    }
    *out = c;
    return LSO_OK;
}

lso_status lso_stream_layers(lso_stream_ctx* c, const lso_host_layer* L, size_t n_layers)
{
    lso::clear_error();
    if (!c) return lso::fail(LSO_E_INVALID, "ctx is NULL");
    if (n_layers == 0) return LSO_OK;
    if (!L) return lso::fail(LSO_E_INVALID, "host_blocks is NULL");
    for (size_t i = 0; i < n_layers; ++i) {
        lso_status s = check_layer(c, L[i], i);
        if (s != LSO_OK) return s;
    }
    DeviceGuard guard(c->device);
    std::vector<char> pinned(n_layers);
    bool any_pageable = false;
    for (size_t i = 0; i < n_layers; ++i) {
        pinned[i] = is_pinned(L[i].host_base, L[i].bytes);
        any_pageable |= !pinned[i];
    }
    if (any_pageable) {
        lso_status s = ensure_staging(c);
        if (s != LSO_OK) return s;
    }
    lso_status result = LSO_OK;
    hipError_t err = hipSuccess;
    // Host order: issue layers ahead while a staging buffer is free, else
    // retire the oldest layer.  retire(i) waits for layer i's D2H and copies
    // a staged layer back out of its staging buffer, which frees that buffer
    // for layer i + nstage; with one more staging buffer than device slots
    // the copy-in of a layer overlaps the D2H of the layer before it.  A
    // pinned layer needs no staging and its retire does not wait.
    const size_t nst = static_cast<size_t>(staging_count(c));
    size_t issued = 0, retired = 0;
    auto issue = [&](size_t i) -> lso_status {
        void* blk = L[i].host_base;
        if (!pinned[i]) {
            void* stg = c->staging[i % nst];
            c->pool->copy(stg, blk, L[i].bytes);   // stage in
            blk = stg;
        }
        return issue_layer(c, L[i], i, blk, blk);
    };
    auto retire = [&](size_t i) -> lso_status {
        if (pinned[i]) return LSO_OK;
        // d2h_done[i % nst] still refers to layer i: layer i + nst, which
        // re-records it, is issued only after this retire
        hipError_t e = hipEventSynchronize(c->d2h_done[i % nst]);
        if (e != hipSuccess) return lso::hip_fail(e, "hipEventSynchronize(buffer-free)");
        c->pool->copy(L[i].host_base, c->staging[i % nst], L[i].bytes);   // stage out
        return LSO_OK;
    };
    while (retired < n_layers) {
        if (issued < n_layers && issued < retired + nst) {
            result = issue(issued);
            if (result != LSO_OK) break;
            ++issued;
        } else {
            result = retire(retired);
            if (result != LSO_OK) break;
            ++retired;
        }
    }
    // Drain: every enqueued stage finishes (on error too, so no copy into a
    // host block is still running when the caller looks at it); a staged
    // layer whose D2H was enqueued is still copied out.
    for (hipStream_t st : {c->h2d, c->compute, c->d2h}) {
        err = hipStreamSynchronize(st);
        if (err != hipSuccess && result == LSO_OK) result = lso::hip_fail(err, "hipStreamSynchronize");
    }
    if (result == LSO_E_CALLBACK || result == LSO_E_HIP) {
        // layers whose D2H completed are whole; copy the staged ones out
        // (a failed layer never reached its D2H, so it is not among them)
        const size_t failed = issued;   // the layer that failed was not counted
        for (size_t i = retired; i < failed; ++i)
            if (!pinned[i]) c->pool->copy(L[i].host_base, c->staging[i % nst], L[i].bytes);
    }
    return result;
}

void* lso_stream_slot_weight(lso_stream_ctx* c, int slot)
{
    if (!c || slot < 0 || slot >= c->nslots) return nullptr;
    return c->slot_weight[slot];
}

lso_status lso_stream_destroy(lso_stream_ctx* c)
{
    lso::clear_error();
    release(c);
    return LSO_OK;
}

}  // extern "C"
