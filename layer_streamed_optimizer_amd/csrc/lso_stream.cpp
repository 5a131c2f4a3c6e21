// Layer streaming: authoritative state off the GPU (host memory or files),
// the GPU as a transient update engine.
//
// MegaTrain summary (blog.hotdry.top), section on streaming execution and
// the double-buffered pipeline: each layer's state is one contiguous,
// page-aligned block moved by one burst; staging buffers on the CPU side
// and slots on the GPU side alternate so the next layer loads while the
// current one computes; three streams (weight transfer H2D, compute,
// transfer back D2H) are tied only by events -- weights-ready,
// backward-done (here: step-done) and buffer-free -- with no host barrier
// in the GPU pipeline; the slot size is the largest layer (section on key
// engineering parameters).  The write-back of each layer is the
// frozen-incremental page's "stored W += delta" (section "The Math"): the
// device computes master + delta and the updated block overwrites the
// authoritative copy.  The same page's storage design (sections "Storage"
// and "Training Loop": per-layer W, M, V files on an SSD, loaded, updated
// and flushed one layer at a time) and its advice to preallocate the files
// (section "Limitations") give the file tier; the MegaTrain summary names
// NVMe tiering as the next step (section on limits and directions).
//
// Per layer i, device slot s = i % nslots:
//   H2D:     wait buffer-free[s]; copy src[i] -> slot[s]; record weights-ready[s]
//   compute: wait weights-ready[s]; gradient producer; fused update;
//            record step-done[s]
//   D2H:     wait step-done[s]; copy slot[s] -> dst[i]; record buffer-free[s]
// Every wait refers to an event recorded earlier in host order.  Each copy
// is one burst over a piece.  By default both directions run on two SDMA
// engines the library names (lso_sdma.h: H2D on one engine of a pair, D2H
// on its partner).  The buffer-free dependency is carried by the engines
// themselves: a piece's H2D is queued on the H2D engine as soon as the
// slot's previous D2H has been issued, with that D2H's completion signal as
// its dependency, so the engine starts it the moment the slot is copied
// back.  The host loop carries the other two: it enqueues a piece's update
// once the H2D has ended (the layer's gradient producer is queued ahead, at
// the H2D) and issues the D2H once the update has ended (HIP streams cannot
// wait on a ROCr signal, nor a ROCr copy on a HIP event).  No shader core
// moves a byte over the link.  LSO_STREAM_CHAIN=0 at context creation has
// the host carry buffer-free too (it issues the H2D once it has seen the
// slot's D2H end), as does the slot-poisoning debug mode below.  Where the engines
// cannot be named, H2D runs on a runtime-chosen DMA engine and D2H by a copy
// kernel, tied by the events above.  LSO_STREAM_COPY=kernel uses copy
// kernels both ways, LSO_STREAM_COPY=dma runtime-chosen DMA engines both
// ways, LSO_STREAM_COPY=dma-in the fallback.  LSO_STREAM_POISON=1 (a debug
// mode) fills each slot with NaN once its piece has been copied back and
// before the next piece may come in, so an update that ran ahead of its
// H2D, or a copy that overtook an update, shows up as NaN in the results.
//
// Three kinds of authoritative block:
//  - pinned host memory (page-locked, e.g. lso_host_alloc): src = dst = the
//    block itself; nothing for the host to do but issue;
//  - pageable host memory: the copy engines cannot reach it, so the block
//    passes through one of the context's pinned staging buffers (nslots + 1
//    unless LSO_STREAM_STAGING asks for more),
//    copied in and out by worker threads;
//  - a region of a file: read into a staging buffer with pread and written
//    back with pwrite, optionally followed by fdatasync.  O_DIRECT
//    descriptors work (offsets and sizes are 4 KB multiples), but the
//    kernel cannot pin the HIP-allocated staging memory for a direct
//    transfer (EFAULT), so their parts go through a small page-aligned
//    buffer per worker thread.
// The host thread runs an event loop over the layers: it starts the
// stage-in of a layer as soon as a staging buffer is free, issues the
// layer's GPU work as soon as its stage-in is complete, starts the
// write-out as soon as its D2H is complete, and frees the buffer when the
// write-out is complete.  Stage-ins and write-outs run on two separate
// worker pools, so reading layer i + 1, updating layer i and writing layer
// i - 1 overlap.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <string>
#include <new>
#include <thread>
#include <vector>

#include "lso_copy.h"
#include "lso_internal.h"
#include "lso_io.h"
#include "lso_runtime.h"
#include "lso_sdma.h"
#include "lso_shadow.h"

namespace {

using lso::IoPool;
using lso::IoRequest;
using lso::kIoCopy;
using lso::kIoRead;
using lso::kIoWrite;

constexpr uint64_t kShadowHeaderCopy = lso::kShadowCopy;

}  // namespace

constexpr int kMaxSlots = 4;
constexpr int kMaxStaging = 8;
// D2H completion signals, one per piece in flight: piece i uses
// i % (nslots + nstaging), so a signal is re-armed only after the host has
// seen the end of the piece that used it before (at most nstaging pieces
// are between their stage-in and their write-out's end)
constexpr int kMaxRing = kMaxSlots + kMaxStaging;

// Which engine moves each direction of a layer block.
// the LSO_COPY_* codes of lso.h
enum CopyMode { kCopyEngines = LSO_COPY_SDMA_PAIR, kCopyDmaIn = LSO_COPY_DMA_IN, kCopyKernels = LSO_COPY_KERNELS,
                kCopyDma = LSO_COPY_DMA };

struct lso_stream_ctx {
    int device = 0;
    uint64_t max_bytes = 0;
    uint64_t max_params = 0;
    lso_grad_fn fn = nullptr;
    void* user = nullptr;
    int nslots = 2;
    int nstaging = 3;   // CPU-side staging buffers, >= nslots + 1
    hipStream_t h2d = nullptr, compute = nullptr, d2h = nullptr;
    void* slot_state[kMaxSlots] = {};
    void* slot_grad[kMaxSlots] = {};
    uint64_t grad_elem_bytes = 2;       // slot_grad holds max_params of this size (2 or 4)
    void* slot_weight[kMaxSlots] = {};
    void* staging[kMaxStaging] = {};   // pinned, allocated on the first staged layer
    uint64_t staging_bytes = 0;         // size of each staging buffer
    hipEvent_t weights_ready[kMaxSlots] = {};
    hipEvent_t step_done[kMaxSlots] = {};
    hipEvent_t buffer_free[kMaxSlots] = {};
    hipEvent_t d2h_done[kMaxStaging] = {};   // per staging buffer: its layer's D2H ended
    IoPool* reader = nullptr;   // stage-ins
    IoPool* writer = nullptr;   // write-outs
    double* dev_norms = nullptr;   // per layer of a call: sum of g^2
    size_t norm_cap = 0;
    double* norm_ws = nullptr;     // chunk sums of the layer being updated
    uint64_t norm_ws_bytes = 0;
    // The host loop sleeps on note_cv until note_gen moves: worker pools
    // bump it when a stage-in or write-out completes and, with named
    // engines, ROCr's signal handlers when a copy ends and a host function
    // on the compute stream when an update ends.  `callbacks` counts those
    // handlers and host functions not yet run.
    std::mutex note_mu;
    std::condition_variable note_cv;
    std::atomic<uint64_t> note_gen{0};
    std::atomic<int> callbacks{0};
    int copy_mode = kCopyDmaIn;
    lso::SdmaLink sdma;                       // kCopyEngines: the two engines
    hsa_signal_t h2d_sig[kMaxSlots] = {};     // kCopyEngines: per slot, its H2D ended
    hsa_signal_t d2h_sig[kMaxRing] = {};      // kCopyEngines: per piece in flight, its D2H ended
    bool chain = true;                        // kCopyEngines: H2D waits for the slot's D2H on the engine
    uint64_t stat_pieces = 0;                 // the last call's pieces
    uint64_t stat_waits = 0;                  // the last call's host-loop sleeps
    hipEvent_t grad_ready[kMaxSlots] = {};    // kCopyEngines: a layer's producer ended (per parity)
    bool poison = false;                      // debug: NaN-fill each slot once copied back
    hipEvent_t poison_done[kMaxSlots] = {};   // kCopyEngines: the slot's fill ended
    unsigned copy_grid = lso::kCopyGrid;
    // largest piece of a tiled layer: on a 70B-shaped slice 512 MiB pieces
    // measured as fast as 256 MiB ones and 0.4% ahead of 1 GiB; 2 GiB pieces
    // were 1.5% slower on five pinned layers
    uint64_t piece_bytes = 512ull << 20;
};

namespace {

uint64_t round16(uint64_t x) { return (x + 15) & ~uint64_t(15); }

// Wake the host loop (see note_gen).
void notify(lso_stream_ctx* c)
{
    {
        std::lock_guard<std::mutex> l(c->note_mu);
        c->note_gen.fetch_add(1);
    }
    c->note_cv.notify_all();
}

// ROCr calls this on its own thread once a watched copy's signal drops
// below 1 (the copy ended, or failed); it runs once.
bool on_copy_end(hsa_signal_value_t, void* arg)
{
    auto* c = static_cast<lso_stream_ctx*>(arg);
    notify(c);
    c->callbacks.fetch_sub(1);
    return false;
}

// Host function on the compute stream after a piece's update.
void on_update_end(void* arg)
{
    auto* c = static_cast<lso_stream_ctx*>(arg);
    notify(c);
    c->callbacks.fetch_sub(1);
}

// Have the loop woken when the copy behind sig ends.  If ROCr refuses, the
// loop still sees the end at its next periodic look.
void watch_copy(lso_stream_ctx* c, hsa_signal_t sig)
{
    c->callbacks.fetch_add(1);
    if (hsa_amd_signal_async_handler(sig, HSA_SIGNAL_CONDITION_LT, 1, on_copy_end, c) != HSA_STATUS_SUCCESS)
        c->callbacks.fetch_sub(1);
}

void release(lso_stream_ctx* c)
{
    if (!c) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    for (hipStream_t s : {c->h2d, c->compute, c->d2h})
        if (s) (void)hipStreamSynchronize(s);
    // every copy and update has ended; their handlers may still be running
    for (int k = 0; k < 200000 && c->callbacks.load() > 0; ++k) std::this_thread::sleep_for(std::chrono::microseconds(50));
    const bool handlers_pending = c->callbacks.load() > 0;
    delete c->reader;   // joins its threads; no request is in flight between calls
    delete c->writer;
    if (c->dev_norms) (void)hipFree(c->dev_norms);
    if (c->norm_ws) (void)hipFree(c->norm_ws);
    for (int s = 0; s < kMaxStaging; ++s) {
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
        if (c->poison_done[s]) (void)hipEventDestroy(c->poison_done[s]);
        if (c->grad_ready[s]) (void)hipEventDestroy(c->grad_ready[s]);
    }
    for (hipStream_t s : {c->h2d, c->compute, c->d2h})
        if (s) (void)hipStreamDestroy(s);
    if (handlers_pending) {
        // a copy engine never signalled the end of a watched copy in 10 s:
        // its handler still holds the context and the signal, so both stay
        // (a leak, not a use after free)
        std::fprintf(stderr, "lso_stream_destroy: %d completion handler(s) never ran; keeping the context\n",
                     c->callbacks.load());
        (void)hipSetDevice(prev);
        return;
    }
    for (int s = 0; s < kMaxSlots; ++s)
        if (c->h2d_sig[s].handle) (void)hsa_signal_destroy(c->h2d_sig[s]);
    for (int s = 0; s < kMaxRing; ++s)
        if (c->d2h_sig[s].handle) (void)hsa_signal_destroy(c->d2h_sig[s]);
    lso::sdma_close(&c->sdma);
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

// True if the copy engines can reach the whole block (page-locked host
// memory known to HIP); false for ordinary pageable memory.
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

// One layer as the pipeline sees it, whatever holds its authoritative copy.
enum Kind { kPinned = 0, kPageable = 1, kFile = 2 };

struct Job {
    size_t index = 0;         // position in the caller's array
    double* sq_norm = nullptr;
    int kind = kPinned;
    char* host = nullptr;     // pinned or pageable block
    int fd = -1;              // file block
    uint64_t foff = 0;        // where it is read from
    uint64_t woff = 0;        // where it is written back (another slot if shadow)
    bool sync = false;
    bool direct = false;      // fd opened O_DIRECT
    bool shadow = false;      // commit header copy for new_epoch after the write
    uint64_t region = 0;      // start of the shadow region
    uint64_t new_epoch = 0;
    uint64_t bytes = 0, n = 0, off_master = 0, off_m = 0, off_v = 0;
    void* dev_weight = nullptr;
    uint32_t opt = 0, layout = 0;
    uint32_t grad_dtype = 0, reserved = 0;
    bool grad_f32 = false;    // the producer writes FP32 gradients
    uint64_t t = 0;
    double lr = 0, beta1 = 0, beta2 = 0, eps = 0;
};

// Checks shared by host and file layers: layout, optimizer, hyper-
// parameters, sizes and the state's place inside the block.
lso_status check_state(const lso_stream_ctx* c, const Job& L, size_t i)
{
    using lso::fail;
    if (L.layout != LSO_LAYOUT_PLANAR && L.layout != LSO_LAYOUT_TILED)
        return fail(LSO_E_INVALID, "layer %zu: unknown layout %u", i, L.layout);
    if (L.layout == LSO_LAYOUT_TILED && L.opt != LSO_OPT_ADAM)
        return fail(LSO_E_DTYPE, "layer %zu: the tiled state layout is for Adam only", i);
    lso_status s = lso::check_hyper(L.opt, L.t, L.lr, L.beta1, L.beta2, L.eps, i);
    if (s != LSO_OK) return s;
    if (L.grad_dtype != 0 && L.grad_dtype != LSO_DT_BF16 && L.grad_dtype != LSO_DT_F32)
        return fail(LSO_E_DTYPE, "layer %zu: gradients must be BF16 or FP32", i);
    if (L.reserved != 0) return fail(LSO_E_INVALID, "layer %zu: reserved field is not 0", i);
    if (L.bytes == 0 || L.bytes > c->max_bytes)
        return fail(LSO_E_INVALID, "layer %zu: bytes %llu outside (0, %llu]", i,
                    static_cast<unsigned long long>(L.bytes), static_cast<unsigned long long>(c->max_bytes));
    if (L.n > c->max_params)
        return fail(LSO_E_INVALID, "layer %zu: %llu params exceed the context's %llu", i,
                    static_cast<unsigned long long>(L.n), static_cast<unsigned long long>(c->max_params));
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

// Blocks of one call must not overlap: their stage-ins and write-outs run
// concurrently.  An extent is [lo, hi) in a space: (0, 0) for host memory,
// (device + 1, inode) of the file otherwise.
struct Extent {
    uint64_t dev, ino, lo, hi;
    size_t layer;
};

lso_status check_disjoint(std::vector<Extent>& ex)
{
    std::sort(ex.begin(), ex.end(), [](const Extent& a, const Extent& b) {
        if (a.dev != b.dev) return a.dev < b.dev;
        if (a.ino != b.ino) return a.ino < b.ino;
        return a.lo < b.lo;
    });
    for (size_t k = 1; k < ex.size(); ++k) {
        const Extent& a = ex[k - 1];
        const Extent& b = ex[k];
        if (a.dev == b.dev && a.ino == b.ino && b.lo < a.hi)
            return lso::fail(LSO_E_OVERLAP, "layers %zu and %zu share bytes of their blocks",
                             std::min(a.layer, b.layer), std::max(a.layer, b.layer));
    }
    return LSO_OK;
}

// Staging buffers: at least one more than device slots, so a layer can be
// read in while the layer before it is still being written out; more let
// stage-ins run further ahead of slow write-outs.
size_t staging_count(const lso_stream_ctx* c) { return static_cast<size_t>(c->nstaging); }

unsigned io_threads()
{
    if (const char* e = std::getenv("LSO_IO_THREADS")) {
        const int k = std::atoi(e);
        if (k >= 1 && k <= 64) return static_cast<unsigned>(k);
    }
    const unsigned hw = std::thread::hardware_concurrency();
    return std::max(2u, std::min(8u, (hw ? hw : 2u) / 2));
}

// Staging buffers hold one piece each: they are sized for the largest
// piece of the call (a whole layer unless it moves in pieces) and grown
// when a later call needs more.
lso_status ensure_staging(lso_stream_ctx* c, uint64_t need)
{
    need = (need + 4095) & ~uint64_t(4095);
    if (c->staging_bytes < need) {
        for (int s = 0; s < kMaxStaging; ++s) {
            if (c->staging[s]) (void)hipHostFree(c->staging[s]);
            c->staging[s] = nullptr;
        }
        c->staging_bytes = need;
    }
    for (size_t s = 0; s < staging_count(c); ++s) {
        if (c->staging[s]) continue;
        if (hipHostMalloc(&c->staging[s], c->staging_bytes, hipHostMallocDefault) != hipSuccess) {
            (void)hipGetLastError();
            c->staging[s] = nullptr;
            return lso::fail(LSO_E_NOMEM, "pinned staging buffer of %llu bytes",
                             static_cast<unsigned long long>(c->staging_bytes));
        }
    }
    if (!c->reader) c->reader = new (std::nothrow) IoPool(io_threads(), &c->note_mu, &c->note_cv, &c->note_gen);
    if (!c->writer) c->writer = new (std::nothrow) IoPool(io_threads(), &c->note_mu, &c->note_cv, &c->note_gen);
    if (!c->reader || !c->writer) return lso::fail(LSO_E_NOMEM, "worker pools");
    return LSO_OK;
}

// The fallback modes' block copy between a page-locked host buffer and a
// device slot: a copy kernel, or a runtime-chosen DMA engine, by direction.
hipError_t copy_block(const lso_stream_ctx* c, void* dst, const void* src, uint64_t bytes,
                      hipMemcpyKind kind, hipStream_t st)
{
    const bool dma = c->copy_mode == kCopyDma ||
                     (c->copy_mode == kCopyDmaIn && kind == hipMemcpyHostToDevice);
    if (dma) return hipMemcpyAsync(dst, src, bytes, kind, st);
    return static_cast<hipError_t>(lso::launch_block_copy(dst, src, bytes, c->copy_grid, st));
}

// One piece of a layer as it moves through the pipeline.  A tiled layer
// whose state starts the block is cut into pieces of whole tiles (about
// piece_bytes each), so a piece's state is a tiled region of its own; any
// other layer is one piece.  Moving pieces rather than whole layers keeps
// the pipeline's fill and drain (the first stage-in and H2D, the last D2H
// and write-out, which run with nothing beside them) to one piece.
struct Unit {
    const Job* job;
    size_t layer;        // position of the layer among the call's jobs
    uint64_t off;        // byte offset of the piece inside the block
    uint64_t bytes;      // bytes of the piece
    uint64_t e0, e1;     // the piece's elements of the layer
    bool first, last;    // first / last piece of its layer
};

std::vector<Unit> make_units(const lso_stream_ctx* c, const Job* J, size_t n)
{
    std::vector<Unit> u;
    constexpr uint64_t T = LSO_TILE_ELEMS;
    constexpr uint64_t tile_bytes = 12 * T;
    for (size_t L = 0; L < n; ++L) {
        const Job& j = J[L];
        const uint64_t per = std::max<uint64_t>(1, c->piece_bytes / tile_bytes);   // tiles per piece
        const uint64_t tiles = (j.n + T - 1) / T;
        if (j.layout != LSO_LAYOUT_TILED || j.off_master != 0 || tiles <= per) {
            u.push_back({&j, L, 0, j.bytes, 0, j.n, true, true});
            continue;
        }
        // as many pieces as pieces of at most `per` tiles take, with the
        // tiles spread evenly over them: a short last piece would leave the
        // D2H engine idle while the next layer's first piece comes in
        const uint64_t k_n = (tiles + per - 1) / per;
        const uint64_t q = tiles / k_n, r = tiles % k_n;   // the first r pieces take q + 1 <= per
        for (uint64_t k = 0; k < k_n; ++k) {
            const uint64_t t0 = k * q + std::min(k, r), t1 = t0 + q + (k < r ? 1 : 0);
            const bool last = k + 1 == k_n;
            const uint64_t off = t0 * tile_bytes;
            u.push_back({&j, L, off, last ? j.bytes - off : (t1 - t0) * tile_bytes, t0 * T,
                         std::min(j.n, t1 * T), k == 0, last});
        }
    }
    return u;
}

// (On a layer's first piece) the layer's gradients, into the buffer of its
// parity: the producer writes them on stream st.
lso_status enqueue_producer(lso_stream_ctx* c, const Unit& U, hipStream_t st)
{
    if (!U.first) return LSO_OK;
    const Job& h = *U.job;
    const int rc = c->fn(c->user, h.index, c->slot_grad[U.layer % c->nslots], h.n, st);
    if (rc != 0) return lso::fail(LSO_E_CALLBACK, "gradient producer returned %d at layer %zu", rc, h.index);
    return LSO_OK;
}

// The fused update of the piece at position i, resident in slot i % nslots,
// on the compute stream; records step_done for the slot.  wait_grads: on a
// layer's first piece, the compute stream first waits for the producer's
// grad_ready event (the producer ran on another stream).
lso_status enqueue_piece_update(lso_stream_ctx* c, const Unit& U, size_t i, bool wait_grads)
{
    const Job& h = *U.job;
    const int s = static_cast<int>(i % c->nslots);
    const int ls = static_cast<int>(U.layer % c->nslots);
    if (wait_grads && U.first) {
        const hipError_t err = hipStreamWaitEvent(c->compute, c->grad_ready[ls], 0);
        if (err != hipSuccess) return lso::hip_fail(err, "hipStreamWaitEvent(gradients ready)");
    }
    lso_block b{};
    // the piece's bytes [off, off + bytes) of the block sit at the slot's start
    const uintptr_t base = reinterpret_cast<uintptr_t>(c->slot_state[s]) - U.off;
    b.base = nullptr;   // absolute addresses below
    b.n = U.e1 - U.e0;
    if (h.layout == LSO_LAYOUT_TILED) {
        b.off_master = base + h.off_master + 12 * U.e0;   // e0 is a tile boundary
        b.off_m = b.off_v = b.off_master;
    } else {
        b.off_master = base + h.off_master;
        b.off_m = base + h.off_m;
        b.off_v = base + h.off_v;
    }
    b.off_grad = reinterpret_cast<uintptr_t>(c->slot_grad[ls]) + (h.grad_f32 ? 4 : 2) * U.e0;
    b.off_weight = reinterpret_cast<uintptr_t>(h.dev_weight ? h.dev_weight : c->slot_weight[ls]) + 2 * U.e0;
    b.grad_dtype = h.grad_f32 ? LSO_DT_F32 : LSO_DT_BF16;
    b.weight_dtype = LSO_DT_BF16;
    b.opt = h.opt;
    b.layout = h.layout;
    b.t = h.t;
    b.lr = h.lr;
    b.beta1 = h.beta1;
    b.beta2 = h.beta2;
    b.eps = h.eps;
    lso::NormOut o;
    o.sq_norms = c->dev_norms + i;
    o.workspace = c->norm_ws;
    o.workspace_bytes = c->norm_ws_bytes;
    if (h.sq_norm && lso::norm_workspace_bytes(&b, 1) > o.workspace_bytes)
        return lso::fail(LSO_E_INVALID, "layer %zu: norm workspace too small", h.index);
    lso_status st = lso::enqueue_update(&b, 1, c->compute, false, h.sq_norm ? &o : nullptr);
    if (st != LSO_OK) return st;
    hipError_t err = hipEventRecord(c->step_done[s], c->compute);
    if (err != hipSuccess) return lso::hip_fail(err, "hipEventRecord(step-done)");
    if (wait_grads && !c->poison) {
        // named engines: the host loop issues the D2H once it is woken here
        c->callbacks.fetch_add(1);
        err = hipLaunchHostFunc(c->compute, on_update_end, c);
        if (err != hipSuccess) {
            c->callbacks.fetch_sub(1);
            return lso::hip_fail(err, "hipLaunchHostFunc(step-done)");
        }
    }
    return LSO_OK;
}

// HIP-stream modes: enqueue H2D, (on a layer's first piece) the gradient
// producer, the update and D2H of the piece at position i of the pipeline
// (slot i % nslots), tied by events, and record d2h_done[i % nstaging]
// after its D2H.  buf: where the H2D reads and the D2H writes (inside the
// block itself when pinned, a staging buffer otherwise).  A layer's
// gradients and BF16 weights live in the buffers of its own parity
// (layer % nslots) for all its pieces.
lso_status issue_unit(lso_stream_ctx* c, const Unit& U, size_t i, void* buf)
{
    const int s = static_cast<int>(i % c->nslots);
    hipError_t err;
    // StreamIn: the device slot is free once the piece that used it last
    // (nslots pieces ago) has been copied back.
    if ((err = hipStreamWaitEvent(c->h2d, c->buffer_free[s], 0)) != hipSuccess ||
        (err = copy_block(c, c->slot_state[s], buf, U.bytes, hipMemcpyHostToDevice, c->h2d)) != hipSuccess ||
        (err = hipEventRecord(c->weights_ready[s], c->h2d)) != hipSuccess)
        return lso::hip_fail(err, "H2D stage");
    // Compute: the layer's gradients (once), then the fused update on the slot.
    if ((err = hipStreamWaitEvent(c->compute, c->weights_ready[s], 0)) != hipSuccess)
        return lso::hip_fail(err, "hipStreamWaitEvent(weights-ready)");
    lso_status st = enqueue_producer(c, U, c->compute);
    if (st != LSO_OK) return st;
    st = enqueue_piece_update(c, U, i, false);
    if (st != LSO_OK) return st;
    // Offload: the updated piece goes back over the authoritative copy.
    if ((err = hipStreamWaitEvent(c->d2h, c->step_done[s], 0)) != hipSuccess ||
        (err = copy_block(c, buf, c->slot_state[s], U.bytes, hipMemcpyDeviceToHost, c->d2h)) != hipSuccess ||
        (c->poison && (err = hipMemsetAsync(c->slot_state[s], 0xFF, U.bytes, c->d2h)) != hipSuccess) ||
        (err = hipEventRecord(c->buffer_free[s], c->d2h)) != hipSuccess ||
        (err = hipEventRecord(c->d2h_done[i % staging_count(c)], c->d2h)) != hipSuccess)
        return lso::hip_fail(err, "D2H stage");
    return LSO_OK;
}

// SDMA-pair mode, first stage of the piece at position i: (on a layer's
// first piece) the gradient producer, on the otherwise idle h2d stream with
// grad_ready recorded after it -- so the previous layer's updates on the
// compute stream never wait behind it -- then the H2D on the link's H2D
// engine.  The loop calls it once the piece that used the slot before
// (nslots pieces ago) has had its D2H issued -- which it does only after
// that piece's update has ended, and the updates end in order -- so the
// gradient buffer of the piece's parity (last read by layer - nslots, whose
// pieces all came earlier) and the slot's H2D signal are free; dep (that
// D2H's completion signal, or NULL once the host has seen it end) holds
// the copy on the engine until the slot has been copied back.
lso_status issue_h2d_engine(lso_stream_ctx* c, const Unit& U, size_t i, const void* buf, const hsa_signal_t* dep)
{
    const int s = static_cast<int>(i % c->nslots);
    lso_status st = enqueue_producer(c, U, c->h2d);
    if (st != LSO_OK) return st;
    if (U.first) {
        const hipError_t err = hipEventRecord(c->grad_ready[U.layer % c->nslots], c->h2d);
        if (err != hipSuccess) return lso::hip_fail(err, "hipEventRecord(gradients ready)");
    }
    const hsa_status_t hs = lso::sdma_copy(c->sdma, c->slot_state[s], buf, U.bytes, true, dep, c->h2d_sig[s]);
    if (hs != HSA_STATUS_SUCCESS) {
        hsa_signal_store_screlease(c->h2d_sig[s], 0);
        return lso::fail(LSO_E_HIP, "SDMA H2D copy of %llu bytes not accepted (status %d)",
                         static_cast<unsigned long long>(U.bytes), static_cast<int>(hs));
    }
    watch_copy(c, c->h2d_sig[s]);
    return LSO_OK;
}

// SDMA-pair mode, last stage: the piece's D2H on the link's D2H engine,
// once its update has completed; its completion is d2h_sig[sig].
lso_status issue_d2h_engine(lso_stream_ctx* c, const Unit& U, size_t i, void* buf, size_t sig)
{
    const int s = static_cast<int>(i % c->nslots);
    const hsa_status_t hs = lso::sdma_copy(c->sdma, buf, c->slot_state[s], U.bytes, false, nullptr, c->d2h_sig[sig]);
    if (hs != HSA_STATUS_SUCCESS) {
        hsa_signal_store_screlease(c->d2h_sig[sig], 0);
        return lso::fail(LSO_E_HIP, "SDMA D2H copy of %llu bytes not accepted (status %d)",
                         static_cast<unsigned long long>(U.bytes), static_cast<int>(hs));
    }
    watch_copy(c, c->d2h_sig[sig]);
    return LSO_OK;
}

const char* io_what(const Job& j) { return j.kind == kFile ? "file" : "host block"; }

// With LSO_STREAM_TRACE set, each call prints one line per piece to stderr:
// its layer and piece, when its stage-in started, when the loop saw it
// complete and issued the piece, when it saw the D2H complete (write-out
// start) and when it saw the write-out complete, in ms from the start of
// the call.
struct Trace {
    bool on = false;
    std::chrono::steady_clock::time_point t0;
    std::vector<double> read, issue, retire, done;

    explicit Trace(size_t n)
    {
        const char* e = std::getenv("LSO_STREAM_TRACE");
        on = e && *e && std::strcmp(e, "0") != 0;
        if (!on) return;
        t0 = std::chrono::steady_clock::now();
        read.assign(n, -1);
        issue.assign(n, -1);
        retire.assign(n, -1);
        done.assign(n, -1);
    }
    void mark(std::vector<double>& v, size_t i)
    {
        if (on) v[i] = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    }
    void print(const std::vector<Unit>& units) const
    {
        if (!on) return;
        std::fprintf(stderr, "[lso trace] layer.piece  read_start  issued  d2h_done  written   (ms)\n");
        size_t piece = 0;
        for (size_t i = 0; i < read.size(); ++i) {
            piece = units[i].first ? 0 : piece + 1;
            std::fprintf(stderr, "[lso trace] %5zu.%-5zu  %10.1f  %6.1f  %8.1f  %7.1f\n", units[i].job->index,
                         piece, read[i], issue[i], retire[i], done[i]);
        }
    }
};

// The event loop over all pieces of one call (see the top of this file).
// Piece i owns staging buffer i % K (K = nstaging) from the start of its
// stage-in until its write-out is complete.
lso_status run_pipeline(lso_stream_ctx* c, const Job* J, size_t nj)
{
    const std::vector<Unit> units = make_units(c, J, nj);
    const size_t n = units.size();
    bool any_staged = false, any_norm = false;
    uint64_t max_piece = 0;
    for (size_t i = 0; i < nj; ++i) {
        any_staged |= J[i].kind != kPinned;
        any_norm |= J[i].sq_norm != nullptr;
    }
    for (const Unit& u : units)
        if (u.job->kind != kPinned) max_piece = std::max(max_piece, u.bytes);
    if (any_staged) {
        lso_status s = ensure_staging(c, max_piece);
        if (s != LSO_OK) return s;
    }
    if (std::any_of(J, J + nj, [](const Job& j) { return j.grad_f32; }) && c->grad_elem_bytes < 4) {
        // FP32 gradients: the gradient buffers grow to 4 bytes per parameter,
        // all or none (no work of an earlier call is pending: every call
        // ends synchronised)
        const uint64_t gbytes = round16(4 * (c->max_params ? c->max_params : 1));
        void* grown[kMaxSlots] = {};
        for (int s = 0; s < c->nslots; ++s) {
            if (hipMalloc(&grown[s], gbytes) != hipSuccess) {
                (void)hipGetLastError();
                grown[s] = nullptr;
                for (int k = 0; k < s; ++k) (void)hipFree(grown[k]);
                return lso::fail(LSO_E_NOMEM, "FP32 gradient buffers of %llu bytes",
                                 static_cast<unsigned long long>(gbytes));
            }
        }
        for (int s = 0; s < c->nslots; ++s) {
            if (c->slot_grad[s]) (void)hipFree(c->slot_grad[s]);
            c->slot_grad[s] = grown[s];
        }
        c->grad_elem_bytes = 4;
    }
    if (any_norm && c->norm_cap < n) {
        if (c->dev_norms) (void)hipFree(c->dev_norms);
        c->dev_norms = nullptr;
        c->norm_cap = 0;
        if (hipMalloc(&c->dev_norms, n * sizeof(double)) != hipSuccess)
            return lso::fail(LSO_E_NOMEM, "device array of %zu piece norms", n);
        c->norm_cap = n;
    }
    const size_t K = staging_count(c);
    std::unique_ptr<IoRequest[]> rd(new IoRequest[K]), wr(new IoRequest[K]);
    // shadow commits: one page-aligned header copy per staging buffer
    std::unique_ptr<char, decltype(&std::free)> headers(nullptr, &std::free);
    {
        void* q = nullptr;
        if (posix_memalign(&q, 4096, K * kShadowHeaderCopy) != 0) return lso::fail(LSO_E_NOMEM, "header buffers");
        headers.reset(static_cast<char*>(q));
    }
    std::vector<char> wr_live(K, 0);   // a write-out was submitted for the buffer
    lso_status result = LSO_OK;
    auto record = [&](lso_status s) {
        if (result == LSO_OK) result = s;
    };
    const bool engines = c->copy_mode == kCopyEngines;
    const bool chain = engines && c->chain && !c->poison;
    const size_t S = static_cast<size_t>(c->nslots);
    const size_t R = S + K;   // D2H completion signals in the ring
    uint64_t waits = 0;
    size_t next_read = 0;     // next piece to stage in
    size_t next_issue = 0;    // next piece to enqueue on the GPU (SDMA-pair mode: its H2D)
    size_t next_update = 0;   // SDMA-pair mode: next piece whose H2D completion is awaited
    size_t next_offload = 0;  // SDMA-pair mode: next piece whose update completion is awaited
    size_t next_retire = 0;   // next piece whose D2H completion is awaited
    size_t next_done = 0;     // next piece whose write-out completion is awaited
    size_t stop_at = n;       // after an error no piece >= stop_at is read or issued
    bool gpu_ok = true;       // after a failed GPU stage no staged data is written out
    Trace trace(n);

    auto read_complete = [&](size_t i) {
        return units[i].job->kind == kPinned || rd[i % K].done.load();
    };
    auto buf_of = [&](size_t i) -> char* {
        const Unit& U = units[i];
        return U.job->kind == kPinned ? U.job->host + U.off : static_cast<char*>(c->staging[i % K]);
    };
    auto reads_in_flight = [&] {
        for (size_t i = next_issue; i < next_read; ++i)
            if (!read_complete(i)) return true;
        return false;
    };
    // with named engines (no slot poisoning) every completion the loop
    // waits for wakes it; otherwise it looks every 50 / 200 us
    const bool woken = engines && !c->poison;
    for (;;) {
        const uint64_t seen = c->note_gen.load();
        bool progress = false;
        // 1. stage in while a buffer is free
        while (next_read < stop_at && next_read < next_done + K) {
            const Unit& U = units[next_read];
            const Job& j = *U.job;
            if (j.kind != kPinned) {
                IoRequest& r = rd[next_read % K];
                r.reset();
                r.direct = false;
                r.bytes = U.bytes;
                r.dst = static_cast<char*>(c->staging[next_read % K]);
                if (j.kind == kFile) {
                    r.op = kIoRead;
                    r.fd = j.fd;
                    r.foff = j.foff + U.off;
                    r.direct = j.direct;
                } else {
                    r.op = kIoCopy;
                    r.src = j.host + U.off;
                }
                c->reader->submit(&r);
            }
            trace.mark(trace.read, next_read);
            ++next_read;
            progress = true;
        }
        // 2. issue staged pieces in order (SDMA-pair mode: once the piece
        //    that used the slot before has had its D2H issued -- the H2D
        //    engine then waits for that D2H itself -- or, unchained, once
        //    the host has seen that D2H end)
        while (next_issue < next_read && next_issue < stop_at && read_complete(next_issue) &&
               (!engines || next_issue < (chain ? next_offload : next_retire) + S)) {
            const Unit& U = units[next_issue];
            const Job& j = *U.job;
            if (engines && c->poison && next_issue >= S) {
                const hipError_t q = hipEventQuery(c->poison_done[next_issue % S]);
                if (q == hipErrorNotReady) break;
                if (q != hipSuccess) {
                    record(lso::hip_fail(q, "slot fill"));
                    gpu_ok = false;
                    stop_at = next_issue;
                    break;
                }
            }
            if (j.kind != kPinned) {
                if (const int e = rd[next_issue % K].err.load()) {
                    record(lso::fail(LSO_E_IO, "layer %zu: reading its %s failed: %s", j.index,
                                     io_what(j), std::strerror(e)));
                    stop_at = next_issue;
                    break;
                }
            }
            trace.mark(trace.issue, next_issue);
            // the slot's previous D2H, unless the host has already seen it end
            const hsa_signal_t* dep =
                chain && next_issue >= S && next_issue - S >= next_retire ? &c->d2h_sig[(next_issue - S) % R] : nullptr;
            const lso_status s = engines ? issue_h2d_engine(c, U, next_issue, buf_of(next_issue), dep)
                                         : issue_unit(c, U, next_issue, buf_of(next_issue));
            if (s != LSO_OK) {
                record(s);
                stop_at = next_issue;
                if (s == LSO_E_HIP) gpu_ok = false;
                break;
            }
            ++next_issue;
            progress = true;
        }
        // 2b. SDMA-pair mode: the update of each piece whose H2D is complete
        while (engines && next_update < next_issue) {
            const int64_t st = lso::sdma_state(c->h2d_sig[next_update % S]);
            if (st > 0) break;
            if (st < 0 && gpu_ok) {
                record(lso::fail(LSO_E_HIP, "SDMA H2D copy of layer %zu failed", units[next_update].job->index));
                gpu_ok = false;
                stop_at = std::min(stop_at, next_issue);
            }
            if (gpu_ok) {
                const lso_status s = enqueue_piece_update(c, units[next_update], next_update, true);
                if (s != LSO_OK) {
                    record(s);
                    gpu_ok = false;
                    stop_at = std::min(stop_at, next_issue);
                }
            }
            ++next_update;
            progress = true;
        }
        // 2c. SDMA-pair mode: the D2H of each piece whose update is complete
        while (engines && next_offload < next_update) {
            const size_t i = next_offload;
            if (gpu_ok) {
                const hipError_t q = hipEventQuery(c->step_done[i % S]);
                if (q == hipErrorNotReady) break;
                const lso_status s = q != hipSuccess ? lso::hip_fail(q, "update completion")
                                                     : issue_d2h_engine(c, units[i], i, buf_of(i), i % R);
                if (s != LSO_OK) {
                    record(s);
                    gpu_ok = false;
                    stop_at = std::min(stop_at, next_issue);
                }
            }
            ++next_offload;
            progress = true;
        }
        // 3. start the write-out of pieces whose D2H is complete, one at a
        //    time in order (so a failed write leaves every later piece
        //    untouched)
        while (next_retire < (engines ? next_offload : next_issue) && next_done == next_retire) {
            if (engines) {
                const int64_t st = gpu_ok ? lso::sdma_state(c->d2h_sig[next_retire % R]) : 0;
                if (st > 0) break;
                if (st < 0) {
                    record(lso::fail(LSO_E_HIP, "SDMA D2H copy of layer %zu failed", units[next_retire].job->index));
                    gpu_ok = false;
                    stop_at = std::min(stop_at, next_issue);
                    // an H2D chained to this copy waits for the signal to
                    // reach 0: release it (nothing of it is written back)
                    hsa_signal_store_screlease(c->d2h_sig[next_retire % R], 0);
                }
                if (gpu_ok && c->poison) {
                    const size_t s = next_retire % S;
                    hipError_t e = hipMemsetAsync(c->slot_state[s], 0xFF, units[next_retire].bytes, c->compute);
                    if (e == hipSuccess) e = hipEventRecord(c->poison_done[s], c->compute);
                    if (e != hipSuccess) {
                        record(lso::hip_fail(e, "slot fill"));
                        gpu_ok = false;
                        stop_at = std::min(stop_at, next_issue);
                    }
                }
            } else {
                const hipError_t q = gpu_ok ? hipEventQuery(c->d2h_done[next_retire % K]) : hipSuccess;
                if (q == hipErrorNotReady) break;
                if (q != hipSuccess) {
                    record(lso::hip_fail(q, "D2H completion"));
                    gpu_ok = false;
                    stop_at = std::min(stop_at, next_issue);
                }
            }
            const Unit& U = units[next_retire];
            const Job& j = *U.job;
            if (j.kind != kPinned && gpu_ok && next_retire < stop_at) {
                IoRequest& w = wr[next_retire % K];
                w.reset();
                w.direct = j.direct;
                w.sync = false;
                w.header = nullptr;
                w.bytes = U.bytes;
                w.src = static_cast<const char*>(c->staging[next_retire % K]);
                if (j.kind == kFile) {
                    w.op = kIoWrite;
                    w.fd = j.fd;
                    w.foff = j.woff + U.off;
                    w.sync = j.sync && U.last;
                    if (j.shadow && U.last) {
                        // every earlier piece of the layer is written (write-outs
                        // run one at a time): flush, then commit the new epoch
                        char* h = headers.get() + (next_retire % K) * kShadowHeaderCopy;
                        lso::shadow_encode(h, j.new_epoch, j.bytes, j.t);
                        w.header = h;
                        w.header_off = lso::shadow_header(j.region, j.new_epoch);
                    }
                } else {
                    w.op = kIoCopy;
                    w.dst = j.host + U.off;
                }
                wr_live[next_retire % K] = 1;
                c->writer->submit(&w);
            }
            trace.mark(trace.retire, next_retire);
            ++next_retire;
            progress = true;
        }
        // 4. free the buffers of pieces whose write-out is complete
        while (next_done < next_retire) {
            const size_t b = next_done % K;
            if (wr_live[b]) {
                if (!wr[b].done.load()) break;
                wr_live[b] = 0;
                if (const int e = wr[b].err.load()) {
                    // this region may be partly written; no later piece is
                    // written back
                    const Job& j = *units[next_done].job;
                    record(lso::fail(LSO_E_IO, "layer %zu: writing its %s back failed: %s", j.index,
                                     io_what(j), std::strerror(e)));
                    stop_at = std::min(stop_at, next_done + 1);
                }
            }
            trace.mark(trace.done, next_done);
            ++next_done;
            progress = true;
        }
        const size_t last = std::min(stop_at, n);
        if (next_done == next_issue && next_issue >= last && !reads_in_flight()) break;
        if (!progress) {
            ++waits;
            std::unique_lock<std::mutex> l(c->note_mu);
            if (woken) {
                // until something completes (the time limit only bounds a
                // missed notification)
                c->note_cv.wait_for(l, std::chrono::milliseconds(20), [&] { return c->note_gen.load() != seen; });
            } else {
                // SDMA-pair mode with poisoning: the loop itself moves each
                // piece from copy to update to copy, so it looks more often
                c->note_cv.wait_for(l, std::chrono::microseconds(engines ? 50 : 200));
            }
        }
    }
    // Every enqueued stage finishes before return (on error too, so no copy
    // into a block is still running when the caller looks at it).  A failed
    // D2H's signal is released, so an H2D chained to it can end too.
    if (engines) {
        for (size_t s = 0; s < R; ++s) {
            while (lso::sdma_state(c->d2h_sig[s]) > 0) std::this_thread::sleep_for(std::chrono::microseconds(50));
            if (lso::sdma_state(c->d2h_sig[s]) < 0) hsa_signal_store_screlease(c->d2h_sig[s], 0);
        }
        for (size_t s = 0; s < S; ++s)
            while (lso::sdma_state(c->h2d_sig[s]) > 0) std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
    c->stat_pieces = n;
    c->stat_waits = waits;
    for (hipStream_t st : {c->h2d, c->compute, c->d2h}) {
        const hipError_t err = hipStreamSynchronize(st);
        if (err != hipSuccess) record(lso::hip_fail(err, "hipStreamSynchronize"));
    }
    trace.print(units);
    if (result == LSO_OK && any_norm) {
        std::vector<double> sq(n);
        const hipError_t err = hipMemcpy(sq.data(), c->dev_norms, n * sizeof(double), hipMemcpyDeviceToHost);
        if (err != hipSuccess) return lso::hip_fail(err, "hipMemcpy (piece norms)");
        // a layer's norm: its pieces' sums added in piece order
        double acc = 0.0;
        for (size_t i = 0; i < n; ++i) {
            acc = units[i].first ? sq[i] : acc + sq[i];
            if (units[i].last && units[i].job->sq_norm) *units[i].job->sq_norm = acc;
        }
    }
    return result;
}

// Fields shared by lso_host_layer and lso_file_layer.
template <class T>
void copy_state_fields(Job& j, const T& L)
{
    j.bytes = L.bytes;
    j.n = L.n;
    j.off_master = L.off_master;
    j.off_m = L.off_m;
    j.off_v = L.off_v;
    j.dev_weight = L.dev_weight;
    j.opt = L.opt;
    j.layout = L.layout;
    j.t = L.t;
    j.lr = L.lr;
    j.beta1 = L.beta1;
    j.beta2 = L.beta2;
    j.eps = L.eps;
    j.sq_norm = L.sq_norm;
    j.grad_dtype = L.grad_dtype;
    j.reserved = L.reserved;
    j.grad_f32 = L.grad_dtype == LSO_DT_F32;
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
    // staging buffers serve file blocks too, whose sizes are 4 KB multiples
    c->max_bytes = (max_layer_bytes + 4095) & ~uint64_t(4095);
    c->max_params = max_layer_params;
    c->fn = fn;
    c->user = user;
    int want = kCopyEngines;
    if (const char* e = std::getenv("LSO_STREAM_COPY")) {
        if (!std::strcmp(e, "dma")) want = kCopyDma;
        else if (!std::strcmp(e, "dma-in")) want = kCopyDmaIn;
        else if (!std::strcmp(e, "kernel")) want = kCopyKernels;
    }
    if (const char* e = std::getenv("LSO_STREAM_SLOTS")) {
        const int k = std::atoi(e);
        if (k >= 2 && k <= kMaxSlots) c->nslots = k;
    }
    if (const char* e = std::getenv("LSO_STREAM_PIECE_BYTES")) {
        const long long k = std::atoll(e);
        if (k >= 12ll * LSO_TILE_ELEMS) c->piece_bytes = static_cast<uint64_t>(k);
    }
    c->nstaging = c->nslots + 1;
    if (const char* e = std::getenv("LSO_STREAM_STAGING")) {
        const int k = std::atoi(e);
        if (k >= c->nslots + 1 && k <= kMaxStaging) c->nstaging = k;
    }
    if (const char* e = std::getenv("LSO_STREAM_COPY_GRID")) {
        const int k = std::atoi(e);
        if (k >= 1 && k <= 4096) c->copy_grid = static_cast<unsigned>(k);
    }
    if (const char* e = std::getenv("LSO_STREAM_POISON")) c->poison = *e && std::strcmp(e, "0") != 0;
    // default priority on all three (different priorities are not used)
    for (hipStream_t* s : {&c->h2d, &c->compute, &c->d2h}) {
        err = hipStreamCreateWithFlags(s, hipStreamNonBlocking);
        if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipStreamCreateWithFlags"); }
    }
    const uint64_t pbytes = round16(2 * (max_layer_params ? max_layer_params : 1));
    for (int s = 0; s < c->nslots; ++s) {
        if (hipMalloc(&c->slot_state[s], c->max_bytes) != hipSuccess ||
            hipMalloc(&c->slot_grad[s], pbytes) != hipSuccess ||
            hipMalloc(&c->slot_weight[s], pbytes) != hipSuccess) {
            release(c);
            return lso::fail(LSO_E_NOMEM, "slot allocation (%llu + 2 x %llu bytes) failed",
                             static_cast<unsigned long long>(c->max_bytes),
                             static_cast<unsigned long long>(pbytes));
        }
        for (hipEvent_t* e : {&c->weights_ready[s], &c->step_done[s], &c->buffer_free[s], &c->poison_done[s],
                              &c->grad_ready[s]}) {
            err = hipEventCreateWithFlags(e, hipEventDisableTiming);
            if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipEventCreateWithFlags"); }
        }
    }
    for (size_t s = 0; s < staging_count(c); ++s) {
        err = hipEventCreateWithFlags(&c->d2h_done[s], hipEventDisableTiming);
        if (err != hipSuccess) { release(c); return lso::hip_fail(err, "hipEventCreateWithFlags"); }
    }
    // Named SDMA engines need ROCr's agents, engine masks and a completion
    // signal per slot and direction; without them the context copies H2D on
    // a runtime-chosen engine and D2H by kernel.
    c->copy_mode = want == kCopyEngines ? kCopyDmaIn : want;
    if (want == kCopyEngines && lso::sdma_open(device, &c->sdma)) {
        bool ok = true;
        auto make = [&ok](hsa_signal_t* sig) {
            if (ok && hsa_signal_create(0, 0, nullptr, sig) != HSA_STATUS_SUCCESS) {
                sig->handle = 0;
                ok = false;
            }
        };
        for (int s = 0; s < c->nslots; ++s) make(&c->h2d_sig[s]);
        for (int s = 0; s < c->nslots + c->nstaging; ++s) make(&c->d2h_sig[s]);
        if (ok) c->copy_mode = kCopyEngines;
    }
    if (const char* e = std::getenv("LSO_STREAM_CHAIN")) c->chain = std::strcmp(e, "0") != 0;
    // chunk sums of one layer at the smallest chunk size (any layout)
    const uint64_t min_chunk = lso::chunk_elems(lso::kUnrollSmall);
    const uint64_t max_chunks = ((max_layer_params ? max_layer_params : 1) + min_chunk - 1) / min_chunk;
    c->norm_ws_bytes = sizeof(double) * lso::kNormPartsPerChunk * max_chunks;
    if (hipMalloc(&c->norm_ws, c->norm_ws_bytes) != hipSuccess) {
        release(c);
        return lso::fail(LSO_E_NOMEM, "norm workspace of %llu bytes", static_cast<unsigned long long>(c->norm_ws_bytes));
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
    std::vector<Job> jobs;
    jobs.reserve(n_layers);
    std::vector<Extent> ex;
    ex.reserve(n_layers);
    for (size_t i = 0; i < n_layers; ++i) {
        if (L[i].n == 0) continue;   // skipped (a locked layer)
        jobs.emplace_back();
        Job& j = jobs.back();
        j.index = i;
        copy_state_fields(j, L[i]);
        j.host = static_cast<char*>(L[i].host_base);
        if (!j.host) return lso::fail(LSO_E_INVALID, "layer %zu: host_base is NULL", i);
        if (reinterpret_cast<uintptr_t>(j.host) % 16 != 0)
            return lso::fail(LSO_E_ALIGN, "layer %zu: host block is not 16-byte aligned", i);
        lso_status s = check_state(c, j, i);
        if (s != LSO_OK) return s;
        const uint64_t lo = reinterpret_cast<uintptr_t>(j.host);
        ex.push_back({0, 0, lo, lo + j.bytes, i});
    }
    lso_status s = check_disjoint(ex);
    if (s != LSO_OK) return s;
    DeviceGuard guard(c->device);
    for (Job& j : jobs) j.kind = is_pinned(j.host, j.bytes) ? kPinned : kPageable;
    return run_pipeline(c, jobs.data(), jobs.size());
}

lso_status lso_stream_files(lso_stream_ctx* c, const lso_file_layer* L, size_t n_layers)
{
    lso::clear_error();
    if (!c) return lso::fail(LSO_E_INVALID, "ctx is NULL");
    if (n_layers == 0) return LSO_OK;
    if (!L) return lso::fail(LSO_E_INVALID, "layers is NULL");
    std::vector<Job> jobs;
    jobs.reserve(n_layers);
    std::vector<Extent> ex;
    ex.reserve(n_layers);
    for (size_t i = 0; i < n_layers; ++i) {
        if (L[i].n == 0) continue;   // skipped (a locked layer)
        jobs.emplace_back();
        Job& j = jobs.back();
        j.index = i;
        copy_state_fields(j, L[i]);
        j.kind = kFile;
        j.fd = L[i].fd;
        j.foff = L[i].file_offset;
        if (L[i].flags & ~static_cast<uint32_t>(LSO_FILE_SYNC | LSO_FILE_SHADOW))
            return lso::fail(LSO_E_INVALID, "layer %zu: unknown flags %#x", i, L[i].flags);
        j.sync = (L[i].flags & LSO_FILE_SYNC) != 0;
        j.shadow = (L[i].flags & LSO_FILE_SHADOW) != 0;
        const uint64_t span = j.shadow ? LSO_SHADOW_HEADER_BYTES + 2 * j.bytes : j.bytes;
        if (j.foff % 4096 != 0 || j.bytes % 4096 != 0)
            return lso::fail(LSO_E_ALIGN, "layer %zu: file offset and bytes must be 4096-byte multiples", i);
        struct stat st {};
        if (j.fd < 0 || ::fstat(j.fd, &st) != 0)
            return lso::fail(LSO_E_INVALID, "layer %zu: fd %d is not an open file", i, j.fd);
        const int acc = ::fcntl(j.fd, F_GETFL);
        if (acc < 0 || (acc & O_ACCMODE) != O_RDWR)
            return lso::fail(LSO_E_INVALID, "layer %zu: fd %d is not open for reading and writing", i, j.fd);
        j.direct = (acc & O_DIRECT) != 0;
        if (S_ISREG(st.st_mode) && static_cast<uint64_t>(st.st_size) < j.foff + span)
            return lso::fail(LSO_E_INVALID, "layer %zu: the file ends before its block does", i);
        lso_status s = check_state(c, j, i);
        if (s != LSO_OK) return s;
        ex.push_back({static_cast<uint64_t>(st.st_dev) + 1, static_cast<uint64_t>(st.st_ino), j.foff,
                      j.foff + span, i});
        j.woff = j.foff;
        if (j.shadow) {
            // read the committed slot, write the other one, then commit it
            lso::ShadowState cur;
            s = lso::shadow_read(j.fd, j.foff, j.bytes, &cur);
            if (s != LSO_OK) {
                const std::string why = lso_last_error();
                return lso::fail(s, "layer %zu: %s", i, why.c_str());
            }
            j.region = j.foff;
            j.new_epoch = cur.epoch + 1;
            j.foff = lso::shadow_slot(j.region, j.bytes, cur.epoch);
            j.woff = lso::shadow_slot(j.region, j.bytes, j.new_epoch);
        }
    }
    lso_status s = check_disjoint(ex);
    if (s != LSO_OK) return s;
    DeviceGuard guard(c->device);
    return run_pipeline(c, jobs.data(), jobs.size());
}

int lso_stream_copy_mode(const lso_stream_ctx* c, uint32_t* h2d_engine, uint32_t* d2h_engine)
{
    if (!c) return -1;
    const bool eng = c->copy_mode == kCopyEngines;
    if (h2d_engine) *h2d_engine = eng ? c->sdma.h2d_engine : 0;
    if (d2h_engine) *d2h_engine = eng ? c->sdma.d2h_engine : 0;
    return c->copy_mode;
}

int lso_stream_stats(const lso_stream_ctx* c, uint64_t out[3])
{
    if (!c || !out) return -1;
    out[0] = c->stat_pieces;
    out[1] = c->stat_waits;
    out[2] = (c->copy_mode == kCopyEngines && c->chain && !c->poison) ? 1 : 0;
    return 0;
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
