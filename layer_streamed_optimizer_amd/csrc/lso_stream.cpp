// Layer streaming: CPU-authoritative state, GPU as a transient update engine.
//
// MegaTrain summary (blog.hotdry.top), section on streaming execution and
// the double-buffered pipeline: each layer's state is one contiguous,
// page-aligned host block moved by one burst DMA; two staging slots
// alternate so the next layer loads while the current one computes; three
// streams (weight transfer H2D, compute, transfer back D2H) are tied only by
// events -- weights-ready, backward-done (here: step-done) and buffer-free --
// with no host barrier in the layer loop; the slot size is the largest
// layer (section on key engineering parameters).  The write-back of each
// layer is the frozen-incremental page's "stored W += delta": the device
// computes master + delta and the updated block overwrites the host copy.
//
// Per layer i, slot s = i % 2:
//   H2D:     wait buffer-free[s]; copy host[i] -> slot[s]; record weights-ready[s]
//   compute: wait weights-ready[s]; gradient producer; fused update;
//            record step-done[s]
//   D2H:     wait step-done[s]; copy slot[s] -> host[i]; record buffer-free[s]
// Every wait refers to an event recorded earlier in host order, so the loop
// enqueues everything without blocking and the GPU runs H2D of layer i+1 and
// D2H of layer i-1 under the update of layer i.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "lso_runtime.h"

struct lso_stream_ctx {
    int device = 0;
    uint64_t max_bytes = 0;
    uint64_t max_params = 0;
    lso_grad_fn fn = nullptr;
    void* user = nullptr;
    hipStream_t h2d = nullptr, compute = nullptr, d2h = nullptr;
    void* slot_state[2] = {nullptr, nullptr};
    void* slot_grad[2] = {nullptr, nullptr};
    void* slot_weight[2] = {nullptr, nullptr};
    hipEvent_t weights_ready[2] = {nullptr, nullptr};
    hipEvent_t step_done[2] = {nullptr, nullptr};
    hipEvent_t buffer_free[2] = {nullptr, nullptr};
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
    for (int s = 0; s < 2; ++s) {
        if (c->slot_state[s]) (void)hipFree(c->slot_state[s]);
        if (c->slot_grad[s]) (void)hipFree(c->slot_grad[s]);
        if (c->slot_weight[s]) (void)hipFree(c->slot_weight[s]);
        if (c->weights_ready[s]) (void)hipEventDestroy(c->weights_ready[s]);
        if (c->step_done[s]) (void)hipEventDestroy(c->step_done[s]);
        if (c->buffer_free[s]) (void)hipEventDestroy(c->buffer_free[s]);
    }
    for (hipStream_t s : {c->h2d, c->compute, c->d2h})
        if (s) (void)hipStreamDestroy(s);
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

lso_status check_layer(const lso_stream_ctx* c, const lso_host_layer& L, size_t i)
{
    using lso::fail;
    if (!L.host_base) return fail(LSO_E_INVALID, "layer %zu: host_base is NULL", i);
    if (L.reserved != 0) return fail(LSO_E_INVALID, "layer %zu: reserved field must be 0", i);
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
    // default priority on all three (different priorities are not used)
    for (hipStream_t* s : {&c->h2d, &c->compute, &c->d2h}) {
        err = hipStreamCreateWithFlags(s, hipStreamNonBlocking);
        if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipStreamCreateWithFlags"); }
    }
    const uint64_t pbytes = round16(2 * (max_layer_params ? max_layer_params : 1));
    for (int s = 0; s < 2; ++s) {
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
    lso_status result = LSO_OK;
    hipError_t err = hipSuccess;
    for (size_t i = 0; i < n_layers; ++i) {
        const int s = static_cast<int>(i & 1);
        const lso_host_layer& h = L[i];
        // StreamIn: the slot is free once the layer that used it two steps
        // ago has been copied back.
        if ((err = hipStreamWaitEvent(c->h2d, c->buffer_free[s], 0)) != hipSuccess ||
            (err = hipMemcpyAsync(c->slot_state[s], h.host_base, h.bytes, hipMemcpyHostToDevice, c->h2d)) != hipSuccess ||
            (err = hipEventRecord(c->weights_ready[s], c->h2d)) != hipSuccess) {
            result = lso::hip_fail(err, "H2D stage");
            break;
        }
        // Compute: gradients of this layer, then the fused update on the slot.
        if ((err = hipStreamWaitEvent(c->compute, c->weights_ready[s], 0)) != hipSuccess) {
            result = lso::hip_fail(err, "hipStreamWaitEvent(weights-ready)");
            break;
        }
        const int rc = c->fn(c->user, i, c->slot_grad[s], h.n, c->compute);
        if (rc != 0) {
            result = lso::fail(LSO_E_CALLBACK, "gradient producer returned %d at layer %zu", rc, i);
            break;
        }
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
        b.t = h.t;
        b.lr = h.lr;
        b.beta1 = h.beta1;
        b.beta2 = h.beta2;
        b.eps = h.eps;
        result = lso::enqueue_update(&b, 1, c->compute, false);
        if (result != LSO_OK) break;
        if ((err = hipEventRecord(c->step_done[s], c->compute)) != hipSuccess) {
            result = lso::hip_fail(err, "hipEventRecord(step-done)");
            break;
        }
        // Offload: write the updated block back over the authoritative copy.
        if ((err = hipStreamWaitEvent(c->d2h, c->step_done[s], 0)) != hipSuccess ||
            (err = hipMemcpyAsync(h.host_base, c->slot_state[s], h.bytes, hipMemcpyDeviceToHost, c->d2h)) != hipSuccess ||
            (err = hipEventRecord(c->buffer_free[s], c->d2h)) != hipSuccess) {
            result = lso::hip_fail(err, "D2H stage");
            break;
        }
    }
    // Drain: every enqueued stage finishes (on error too, so no copy into a
    // host block is still running when the caller looks at it).
    for (hipStream_t st : {c->h2d, c->compute, c->d2h}) {
        err = hipStreamSynchronize(st);
        if (err != hipSuccess && result == LSO_OK) result = lso::hip_fail(err, "hipStreamSynchronize");
    }
    return result;
}

void* lso_stream_slot_weight(lso_stream_ctx* c, int slot)
{
    if (!c || slot < 0 || slot > 1) return nullptr;
    return c->slot_weight[slot];
}

lso_status lso_stream_destroy(lso_stream_ctx* c)
{
    lso::clear_error();
    release(c);
    return LSO_OK;
}

}  // extern "C"
