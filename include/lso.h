/*
 * lso.h -- C ABI of the layer-streamed mixed-precision Adam library (gfx950).
 *
 * One operation, three ways of feeding it:
 *   lso_adam_step      updates blocks that already live in device memory
 *                      (HBM-resident state), one kernel launch per call
 *                      (lso_adam_step_norms: plus per-block gradient norms);
 *   lso_stream_layers  updates layers whose authoritative state lives in
 *                      host memory, streaming each layer in, updating it on
 *                      the GPU and writing it back, double-buffered;
 *   lso_stream_files   the same for layers held in files (the disk tier),
 *                      optionally crash-consistent (LSO_FILE_SHADOW).
 *
 * The update, per element i of a block (all arithmetic below is what the
 * library computes; the pages define it in exact arithmetic):
 *   g      = BF16 gradient widened to FP32 (exact), or an FP32 gradient
 *   m'     = beta1*m + (1-beta1)*g
 *   v'     = beta2*v + (1-beta2)*g^2
 *   delta  = -lr * (m'/(1-beta1^t)) / (sqrt(v'/(1-beta2^t)) + eps)
 *   master'= master + delta            (the additive write-back, W += delta)
 *   w      = BF16 round-to-nearest-even of master'
 * Sources: "Training 70B Models on Consumer Hardware (If You're Willing to
 * Wait)" (bombadil.systems), section "The Math" for the moments, the bias
 * correction with a global step t and the additive form of the update;
 * section "The Assumption Everyone Makes" for the SGD rewrite
 * W + (-lr*g) used by LSO_OPT_SGD; the Cloudera community training-memory
 * article, line item "Optimizer states", for the FP32 master copy that is
 * updated and cast back down; the MegaTrain summary on blog.hotdry.top for
 * BF16 weights/gradients with FP32 moments (section on the memory
 * bottleneck), layer-contiguous 4 KB-aligned host blocks, double buffering
 * and a weight-transfer, a compute and a write-back stage joined by
 * weights-ready / backward-done / buffer-free dependencies (section on
 * streaming execution and the double-buffered pipeline).
 * FP32 gradients (grad_dtype LSO_DT_F32) follow the LoRA memory accounting
 * of the Cloudera community article ("everything else": adapter gradients
 * in FP32, 4 bytes each).
 *
 * Precision: the per-block constants 1-beta, lr/(1-beta1^t),
 * 1/sqrt(1-beta2^t) are computed in FP64 on the host and rounded once to
 * FP32; the per-element arithmetic is FP32 with correctly rounded sqrt and
 * division.  Results match an FP64 evaluation to ~1e-6 relative after 10
 * steps; the BF16 weight is always exactly bf16_rne(master').
 *
 * Conventions for every call:
 *  - Return value: an lso_status.  Nothing throws across the ABI.  On an
 *    error, lso_last_error() returns a message for the calling thread.
 *  - Validation errors are detected before anything is enqueued; memory is
 *    then untouched.
 *  - Device faults from earlier asynchronous work surface as LSO_E_HIP from
 *    the next call that synchronises.
 *  - Streams are hipStream_t values passed as void* (NULL = the default
 *    stream of the current device).  All streams the library creates have
 *    the default priority.
 */
#ifndef LSO_H
#define LSO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lso_status {
    LSO_OK = 0,
    LSO_E_INVALID = 1,   /* bad argument: NULL, n, t, hyper-parameters, sizes */
    LSO_E_ALIGN = 2,     /* an array is not 16-byte aligned */
    LSO_E_DTYPE = 3,     /* unsupported dtype / optimizer combination */
    LSO_E_OVERLAP = 4,   /* a written array overlaps another array of the call */
    LSO_E_NOMEM = 5,     /* device or pinned host allocation failed */
    LSO_E_HIP = 6,       /* a HIP runtime call failed */
    LSO_E_CALLBACK = 7,  /* the gradient producer of the layer stream failed */
    LSO_E_IO = 8         /* reading or writing a layer's file failed */
} lso_status;

typedef enum lso_dtype { LSO_DT_NONE = 0, LSO_DT_F32 = 1, LSO_DT_BF16 = 2 } lso_dtype;
typedef enum lso_opt { LSO_OPT_ADAM = 0, LSO_OPT_SGD = 1 } lso_opt;

/* How a block's FP32 optimizer state (master, m, v) is laid out.
 *   PLANAR: three separate arrays at off_master, off_m, off_v.
 *   TILED:  one region at off_master holding master, m and v interleaved
 *           in tiles of LSO_TILE_ELEMS elements: tile k (elements
 *           [k*T, k*T + T), T = LSO_TILE_ELEMS) is 12*T bytes at region
 *           offset 12*T*k -- master of its elements at +0, m at +4*T, v at
 *           +8*T, element j of the tile at index j of each.  The region is
 *           lso_tiled_state_bytes(n) = 12*T*ceil(n/T) bytes; the padding
 *           after element n-1 is never read or written.  Adam only.
 * The state is private to the optimizer, so its layout is free; in the
 * tiled one a workgroup of the update reads and writes three runs a fixed
 * 32 KB apart inside one 96 KB tile, which the HBM serves markedly faster
 * than three arrays far apart.  The tile size is a measured optimum on
 * MI355X: tiles of 1,024 to 65,536 elements, powers of two and sizes
 * between them, were all slower.  Gradients and weights are planar in
 * both layouts (they are shared with the forward and backward passes).
 * lso_tiled_pack and lso_tiled_unpack convert between the two. */
typedef enum lso_layout { LSO_LAYOUT_PLANAR = 0, LSO_LAYOUT_TILED = 1 } lso_layout;
#define LSO_TILE_ELEMS 8192u

/*
 * One block: a layer, or any tensor, whose arrays are updated together.
 * The address of each array is (uintptr_t)base + off_*; base may be NULL
 * with absolute addresses in the offsets.  Element i of every array belongs
 * to parameter i.
 *   master  FP32, read and written           (always)
 *   m, v    FP32, read and written           (LSO_OPT_ADAM; ignored for SGD)
 *   grad    BF16 or FP32, read               (grad_dtype LSO_DT_BF16 or LSO_DT_F32)
 *   weight  BF16, written                    (weight_dtype BF16; NONE skips it)
 * layout (lso_layout): PLANAR, or TILED with master, m and v interleaved in
 * one region at off_master (off_m and off_v are then ignored).
 * Every used array (and a tiled region) must be 16-byte aligned.  No
 * written array may overlap any other array of the same call (across
 * blocks too); gradients may alias one another.  n == 0 makes the block a
 * no-op.
 * t is the step being applied (t >= 1; the first update is t = 1); the
 * caller owns it and increments it per step -- it is the resume point of a
 * checkpoint.  Per-block t lets blocks advance independently.
 * lr finite; 0 <= beta1 < 1; 0 <= beta2 < 1; eps finite and >= 0 (Adam).
 * For SGD only lr is used: master' = master + (-(fl32(lr) * g)), each
 * operation rounded once in FP32.
 */
typedef struct lso_block {
    void*    base;
    uint64_t n;
    uint64_t off_master;
    uint64_t off_m;
    uint64_t off_v;
    uint64_t off_grad;
    uint64_t off_weight;
    uint32_t grad_dtype;     /* lso_dtype */
    uint32_t weight_dtype;   /* lso_dtype */
    uint32_t opt;            /* lso_opt */
    uint32_t layout;         /* lso_layout of master, m, v */
    uint64_t t;
    double   lr, beta1, beta2, eps;
} lso_block;

/*
 * lso_adam_step: one update of n device-resident blocks, enqueued on
 * stream as ONE kernel launch (a ragged multi-tensor launch: hundreds of
 * small tensors cost one launch).
 * Defined by: "Training 70B Models on Consumer Hardware (If You're Willing
 * to Wait)", section "The Math" (the moments, the bias correction with the
 * step t, the update added to the stored weights); the Cloudera community
 * training-memory article, line item "Optimizer states" (the FP32 master is
 * updated and cast back down to the BF16 weight); the LoRA fine-tuning
 * memory article of the same site (adapters on seven projections of every
 * layer: the hundreds of small tensors one call takes).  More than 16 distinct
 * (opt, t, lr, beta1, beta2, eps) sets in one call, or blocks of different
 * layouts or gradient dtypes mixed in one call, split it into one launch
 * per (layout, gradient dtype) and per 16 sets.
 * blocks: host array, read before return; the caller may reuse it at once.
 * Arrays: device memory owned by the caller; they must stay untouched until
 * stream passes the step.  Asynchronous: returns after enqueueing.
 * Layout advice for calls that stream HBM (gigabytes per step): keep each
 * block's state, gradients and weights next to each other (one arena, block
 * after block).  Measured on MI355X, the update's rate then does not depend
 * on where the arena lands; with all states, all gradients and all weights
 * in three distant regions it varies by up to 3% with the placement.
 * n == 0 is a no-op.  Errors: INVALID, ALIGN, DTYPE, OVERLAP (nothing
 * enqueued), NOMEM, HIP.
 */
lso_status lso_adam_step(const lso_block* blocks, size_t n, void* stream);

/*
 * lso_adam_step_noalloc: lso_adam_step for callers that cannot allocate
 * device memory -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same update, bit for bit, with the
 * same arguments, validation and launches; it calls no hipMalloc, hipFree
 * or other allocating routine.  The block table of a launch with more
 * than 4 blocks goes into a fixed per-device scratch array of
 * LSO_NOALLOC_MAX_BLOCKS entries (256 KiB, held by each GPU the library
 * runs on until the process ends), written on `stream` by a small kernel
 * whose arguments carry it (so nothing is read from host memory after the
 * call returns); tables of up to 4 blocks travel in the kernel arguments as
 * with lso_adam_step.  The workgroups of the update then find their blocks
 * by a binary search over that table.  Limit: the launches of one call
 * hold at most LSO_NOALLOC_MAX_BLOCKS table entries in all (blocks with
 * n == 0 and launches of up to 4 blocks take none); a larger call returns
 * LSO_E_INVALID with nothing enqueued.  Every call on one GPU shares that
 * GPU's array and leaves its table there: calls that overlap on one GPU
 * (different streams, or unordered threads) race on it and must not be
 * issued.  The array's device address is looked up once per device, by
 * the first call that needs it (or by the first lso_adam_step on that
 * device); that first lookup must not happen under stream capture -- such
 * a call returns LSO_E_INVALID with nothing enqueued -- so make one call
 * before capturing.  Errors: as lso_adam_step (NOMEM cannot occur).
 */
#define LSO_NOALLOC_MAX_BLOCKS 4096u
lso_status lso_adam_step_noalloc(const lso_block* blocks, size_t n, void* stream);

/*
 * Gradient norms for progressive layer locking.  The frozen-incremental
 * page (section "Progressive Layer Locking") locks a layer once its
 * gradient magnitude is below a threshold: locked layers get no gradient,
 * no update and no I/O; its section "The Math" notes that per-layer steps t
 * keep Adam exact for layers that are locked and later resumed (lso_block
 * and the layer structs carry their own t).  The magnitude is taken as the
 * Euclidean norm of the layer's gradient; these calls return its square.
 *
 * lso_adam_step_norms: lso_adam_step plus, from the same pass over the
 * gradients, sq_norms[i] = sum over block i's elements of g^2, in FP64
 * (a fixed-order sum per wave of the kernel, the waves' sums added in a
 * fixed order, so results repeat bit for bit).  sq_norms: device array of n
 * doubles (entries of blocks with n == 0 are not written).  workspace:
 * device memory of at least lso_norm_workspace_bytes(blocks, n) bytes,
 * 8-byte aligned; it holds per-chunk sums while the call runs on stream, so
 * calls that run at the same time need separate workspaces.  Neither may
 * overlap the other or any array of the call.  Relative error of each
 * entry against the exact sum: below 2e-6 (FP32 sums of at most 1024
 * squares per wave: at most 16 per lane in sequence, then a 64-lane tree;
 * FP64 above that).  Errors: as lso_adam_step, and INVALID for a
 * NULL or too small buffer, ALIGN, OVERLAP.
 */
uint64_t lso_norm_workspace_bytes(const lso_block* blocks, size_t n);
lso_status lso_adam_step_norms(const lso_block* blocks, size_t n, double* sq_norms, void* workspace,
                               uint64_t workspace_bytes, void* stream);

/*
 * Host-only helpers (no device work, callable without a GPU).
 * lso_validate_blocks: the checks lso_adam_step runs, without enqueueing.
 * lso_block_constants: the FP32 constants the kernel uses for one block,
 *   out[0..7] = {beta1, 1-beta1, beta2, 1-beta2, lr/(1-beta1^t),
 *                1/sqrt(1-beta2^t), eps, 0}, each computed in FP64 and
 *   rounded once (SGD: {0,0,0,0, lr, 0, 0, 0}).
 */
lso_status lso_validate_blocks(const lso_block* blocks, size_t n);
lso_status lso_block_constants(const lso_block* block, float out[8]);

/* Fused-update kernel launches this process has enqueued so far (every
 * entry point, every device).  The update of a call is one launch per
 * (layout, gradient dtype) and per 16 hyper-parameter sets; this counter is
 * how a caller checks it.  Host-only, thread-safe. */
uint64_t lso_kernel_launches(void);

/* Bytes of the tiled state region of n parameters: 12 * T * ceil(n / T),
 * T = LSO_TILE_ELEMS (0 for n == 0). */
uint64_t lso_tiled_state_bytes(uint64_t n);

/* Convert n parameters between planar FP32 arrays and a tiled state region
 * (all device memory, 16-byte aligned, not overlapping), enqueued on
 * stream.  pack: m or v may be NULL, which writes zeros.  unpack: master,
 * m or v may be NULL, which skips that array.  Errors: INVALID, ALIGN,
 * HIP. */
lso_status lso_tiled_pack(void* state, const float* master, const float* m, const float* v,
                          uint64_t n, void* stream);
lso_status lso_tiled_unpack(const void* state, float* master, float* m, float* v, uint64_t n,
                            void* stream);

/* ---------------------------------------------------------------------
 * Layer streaming.  The authoritative state of each layer lives in host
 * memory as one contiguous block [master | m | v] (FP32, each sub-array
 * 4 KB aligned inside the block).  For each layer the library copies the
 * block into a device slot (one DMA burst), lets the caller's gradient
 * producer write that layer's BF16 gradients into the slot, runs the fused
 * update on the slot, and copies the block back over the host copy -- so
 * the host holds master + delta afterwards.  Two slots alternate (double
 * buffering): a slot's H2D waits until its previous block has been copied
 * back (buffer-free), the update waits for the H2D (weights-ready), the
 * D2H waits for the update (step-done).  By default the two copies run on
 * two SDMA engines the library names: each H2D is queued on its engine with
 * the slot's previous D2H as a dependency the engine waits for itself, and
 * the host loop carries weights-ready and step-done; in the fallback modes
 * (lso_stream_copy_mode) all three are events between three HIP streams.
 * Host blocks may be pinned (lso_host_alloc, or any page-locked HIP host
 * allocation): the copies then read and write them directly.  Or they may
 * be ordinary pageable memory (for state larger than the page-locked
 * budget): each then passes through one of the context's nslots + 1 pinned
 * staging buffers, copied in by worker threads before its H2D and out after
 * its D2H.  lso_stream_files does the same with blocks held in files (the
 * disk tier).  Stage-ins and write-outs run on two worker pools, so reading
 * layer i + 1, updating layer i and writing layer i - 1 overlap.  A tiled
 * layer whose state starts its block moves in equal pieces of whole tiles
 * (at most 512 MiB; LSO_STREAM_PIECE_BYTES at context creation sets another
 * size),
 * so the pipeline fills and drains in one piece rather than one layer; its
 * gradient producer still runs once, before the first piece's update.
 * ------------------------------------------------------------------- */

typedef struct lso_host_layer {
    void*    host_base;      /* host block, pinned or pageable, 16-byte aligned
                                (lso_host_alloc gives 4 KB-aligned pinned memory) */
    uint64_t bytes;          /* bytes copied each way: covers the state */
    uint64_t n;              /* parameters in the layer */
    uint64_t off_master;     /* byte offsets inside the block, 16-byte aligned;
                                TILED: offset of the tiled state region */
    uint64_t off_m;          /* PLANAR only */
    uint64_t off_v;          /* PLANAR only */
    void*    dev_weight;     /* device BF16 output for the re-cast weight, or
                                NULL: it then stays in the slot's own buffer
                                until the slot is reused */
    uint32_t opt;            /* lso_opt (SGD: m and v are not touched) */
    uint32_t layout;         /* lso_layout of the state inside the block */
    uint64_t t;
    double   lr, beta1, beta2, eps;
    double*  sq_norm;        /* host address that receives the sum of g^2 of
                                this layer's gradient (FP64) when the call
                                returns LSO_OK, or NULL */
    uint32_t grad_dtype;     /* the gradients the producer writes: LSO_DT_BF16
                                (or 0, the same) or LSO_DT_F32 (4 bytes each,
                                the FP32-gradient update of lso_adam_step) */
    uint32_t reserved;       /* must be 0 */
} lso_host_layer;

/* Gradient producer: enqueue (never synchronise) work on compute_stream
 * that writes the n gradients of layer `layer` into dev_grad, in the
 * layer's grad_dtype (BF16 unless it asks for LSO_DT_F32).  A nonzero
 * return stops the stream (lso_stream_layers returns LSO_E_CALLBACK). */
typedef int (*lso_grad_fn)(void* user, size_t layer, void* dev_grad, uint64_t n,
                           void* compute_stream);

typedef struct lso_stream_ctx lso_stream_ctx;

/* Defined by: the MegaTrain summary on blog.hotdry.top, section on
 * streaming execution and the double-buffered pipeline (two sets of
 * staging buffers, a weight-transfer, a compute and a write-back stream
 * tied by weights-ready / backward-done / buffer-free events) and section
 * on key engineering parameters (each buffer holds the largest layer).
 * Create a streaming context on `device`: its streams, two device slots
 * of max_layer_bytes (rounded up to 4 KB) of state plus max_layer_params
 * BF16 gradients and BF16 weights each, the events, and the copy mode (see
 * lso_stream_copy_mode; the three pinned staging buffers of that size and
 * the worker threads are added on the first staged layer, and the gradient
 * buffers grow to FP32 on the first call with an LSO_DT_F32 layer).
 * fn/user: the gradient producer.  Errors: INVALID, NOMEM, HIP.  *out is
 * NULL on error. */
lso_status lso_stream_create(uint64_t max_layer_bytes, uint64_t max_layer_params,
                             lso_grad_fn fn, void* user, int device, lso_stream_ctx** out);

/* Defined by: the MegaTrain summary, section on the system architecture
 * (host memory holds the authoritative parameters and optimizer state, the
 * GPU only computes on what is streamed in) and section on streaming
 * execution (one contiguous, page-aligned block per layer moved by one
 * burst; ping-pong buffers; the three events); "Training 70B Models on
 * Consumer Hardware", section "The Math" (the stored weights take
 * += delta) and section "Training Loop" (each layer loaded, updated and
 * written back in turn).
 * Stream n_layers layers through the pipeline, in order.  Synchronous with
 * respect to host memory: on LSO_OK every host block holds its updated
 * state, and each layer's sq_norm (if not NULL) its gradient's sum of g^2
 * (as lso_adam_step_norms).  A layer with n == 0 is skipped entirely -- no
 * transfer, no producer call, no update, no write-back, no checks of its
 * other fields -- which is how a locked layer is passed; the producer is
 * still called with the layer's position in host_blocks.  On
 * LSO_E_CALLBACK at layer k, layers < k are fully written back and layers
 * >= k are untouched on the host.  Validation (bytes, alignment,
 * hyper-parameters, blocks of different layers not overlapping) covers all
 * layers before anything is enqueued.  Calls on one context must not
 * overlap (one caller thread at a time). */
lso_status lso_stream_layers(lso_stream_ctx* ctx, const lso_host_layer* host_blocks,
                             size_t n_layers);

/* The disk tier.  The frozen-incremental page ("Training 70B Models on
 * Consumer Hardware", sections "Storage" and "Training Loop") keeps each
 * layer's W, M, V in files on an SSD and loads, updates and flushes one
 * layer at a time; its "Limitations" section asks for files preallocated
 * contiguously; the MegaTrain summary names NVMe tiering as the next step.
 * Here a layer's block (the same [master | m | v] or tiled bytes as a host
 * block) is a region of a file: read with pread into a pinned staging
 * buffer, streamed through the device like a pageable host block, and
 * written back over the same region with pwrite. */
#define LSO_FILE_SYNC 1u     /* fdatasync the file after the layer's write-back */
#define LSO_FILE_SHADOW 2u   /* crash-consistent shadow region, see below */

typedef struct lso_file_layer {
    int      fd;             /* open O_RDWR (O_DIRECT allowed); the caller owns it */
    uint32_t flags;          /* 0 or LSO_FILE_SYNC */
    uint64_t file_offset;    /* start of the block in the file, 4096-byte multiple */
    uint64_t bytes;          /* block size, 4096-byte multiple; the file must hold it */
    uint64_t n;              /* the rest as in lso_host_layer, offsets inside the block */
    uint64_t off_master;
    uint64_t off_m;
    uint64_t off_v;
    void*    dev_weight;
    uint32_t opt;
    uint32_t layout;
    uint64_t t;
    double   lr, beta1, beta2, eps;
    double*  sq_norm;
    uint32_t grad_dtype;
    uint32_t reserved;
} lso_file_layer;

/* Stream n_layers file blocks through the pipeline, in order.  On LSO_OK
 * every region holds its updated state (and is on stable storage if
 * LSO_FILE_SYNC was set).  Errors before anything runs: INVALID (bad fd,
 * not O_RDWR, file shorter than offset + bytes, flags), ALIGN, OVERLAP
 * (two regions of one call share bytes of the same file), DTYPE, NOMEM.
 * During the run: on LSO_E_CALLBACK at layer k, regions of layers < k
 * hold their new state and regions of layers >= k are untouched; on a
 * failed read or write (LSO_E_IO) at layer k, regions < k are new, region
 * k may be partly written (a failed write, or a failed read of a layer that
 * moves in several pieces; with LSO_FILE_SHADOW it is wholly at its old
 * epoch), regions > k are untouched.  The
 * step t is the caller's to persist beside the files (the page keeps the
 * global step with the model state so a resumed run continues from it). */
lso_status lso_stream_files(lso_stream_ctx* ctx, const lso_file_layer* layers, size_t n_layers);

/* ---------------------------------------------------------------------
 * Crash-consistent write-back (LSO_FILE_SHADOW).  The frozen-incremental
 * page (section "Verification", its safety note) warns that a crash
 * between the in-place update and the flush can corrupt the state, and
 * asks for atomic writes or shadow copies.  A shadow region keeps two
 * copies of the layer's block and commits each new one with a per-layer
 * epoch only once it is on stable storage:
 *
 *   file_offset + 0                : header copy 0 (4096 bytes)
 *   file_offset + 4096             : header copy 1
 *   file_offset + 8192             : data slot 0 (bytes)
 *   file_offset + 8192 + bytes     : data slot 1 (bytes)
 *
 * The committed state is the valid header copy (checksum, magic and bytes
 * match) with the highest epoch e; its data is slot e % 2 and it records
 * the step t that produced it.  With LSO_FILE_SHADOW, lso_stream_files
 * reads the committed slot, writes the updated block to the other slot,
 * flushes it (fdatasync), then writes header copy (e + 1) % 2 with epoch
 * e + 1 and the layer's t, and flushes again.  A crash or error at any
 * point leaves every layer either wholly at its old epoch or wholly at its
 * new one.  The region needs LSO_SHADOW_HEADER_BYTES + 2 * bytes bytes of
 * file; the file must have been formatted by lso_shadow_format.
 * ------------------------------------------------------------------- */
#define LSO_SHADOW_HEADER_BYTES 8192u

/* Host-only (no device work).  Format a shadow region: epoch 0 in header
 * copy 0 with step t0, header copy 1 cleared; data slot 0 is the caller's
 * to fill before the first update.  Flushes the headers.  Errors: INVALID
 * (bad fd, sizes), ALIGN (offset or bytes not a 4096 multiple), IO. */
lso_status lso_shadow_format(int fd, uint64_t file_offset, uint64_t bytes, uint64_t t0);

/* Host-only.  The committed state of a shadow region: its epoch, the step
 * t recorded with it, and the absolute file offset of its data slot.
 * Errors: INVALID, ALIGN, IO (no valid header: never formatted, or both
 * copies damaged). */
lso_status lso_shadow_state(int fd, uint64_t file_offset, uint64_t bytes, uint64_t* epoch,
                            uint64_t* t, uint64_t* data_offset);

/* Host-only.  Commit epoch `epoch` with step t by writing its header copy
 * (epoch % 2) and flushing it: the step lso_stream_files takes after the
 * data slot epoch % 2 is flushed.  For callers that write slots themselves
 * (initial state, tools).  Errors: INVALID, ALIGN, IO. */
lso_status lso_shadow_commit(int fd, uint64_t file_offset, uint64_t bytes, uint64_t epoch, uint64_t t);

/* Device address of slot s's BF16 weight buffer (s = layer index % 2 of
 * the most recent lso_stream_layers call), or NULL. */
void* lso_stream_slot_weight(lso_stream_ctx* ctx, int slot);

/* How a context moves blocks over the host link (each piece is one burst,
 * as the MegaTrain summary's section on streaming execution describes).
 * SDMA engines come in pairs sharing a path to the link: with both
 * directions busy, H2D on one engine of a pair and D2H on its partner is
 * the fastest split measured; two directions on one engine take turns.
 * The named engines are not reserved: other copies the process runs at the
 * same time (hipMemcpyAsync, another context's stream) may land on them
 * and share their time. */
#define LSO_COPY_SDMA_PAIR 0   /* both directions on DMA engines the library names (default) */
#define LSO_COPY_DMA_IN    1   /* H2D on a DMA engine the runtime picks, D2H by a copy kernel
                                  (default when the engines cannot be named) */
#define LSO_COPY_KERNELS   2   /* copy kernels both ways */
#define LSO_COPY_DMA       3   /* DMA engines the runtime picks, both ways */

/* The context's copy mode, an LSO_COPY_* code (LSO_STREAM_COPY=sdma-pair,
 * dma-in, kernel or dma at lso_stream_create asks for one; LSO_STREAM_SDMA
 * = "h,d" names the two engines by number), and with LSO_COPY_SDMA_PAIR
 * the engine of each direction as a one-bit mask (engine k = bit k), else
 * 0.  Either pointer may be NULL.  Returns -1 if ctx is NULL.
 * Debug: LSO_STREAM_POISON=1 at lso_stream_create makes the context fill
 * each device slot with NaN once its piece has been copied back, before
 * the next piece may come in (a slot-reuse race then shows as NaN). */
int lso_stream_copy_mode(const lso_stream_ctx* ctx, uint32_t* h2d_engine, uint32_t* d2h_engine);

/* Counters of the most recent lso_stream_layers / lso_stream_files call on
 * ctx: out[0] pieces moved, out[1] times the host loop slept waiting for a
 * completion (its wake-ups), out[2] 1 if each H2D was chained on the copy
 * engine to the slot's previous D2H (the default with named engines;
 * LSO_STREAM_CHAIN=0 or LSO_STREAM_POISON=1 at lso_stream_create turn it
 * off), else 0.  Returns 0, or -1 if ctx or out is NULL. */
int lso_stream_stats(const lso_stream_ctx* ctx, uint64_t out[3]);

/* The end of a context made by lso_stream_create (same sections of the
 * MegaTrain summary): waits for outstanding work, frees slots, events and
 * streams.  NULL is a no-op.  Always LSO_OK. */
lso_status lso_stream_destroy(lso_stream_ctx* ctx);

/* Defined by: the MegaTrain summary, section on streaming execution
 * (layer blocks aligned to 4 KB pages, for pinned staging) and section on
 * key engineering parameters (pinned buffers of the largest layer).
 * Pinned host memory for layer blocks (page aligned, so 4 KB aligned):
 * hipHostMalloc, owned by the caller until lso_host_free.  Errors: INVALID
 * (bytes == 0 or out NULL), NOMEM; *out is NULL on error.  lso_host_free:
 * NULL is a no-op; HIP on a pointer the runtime does not know. */
lso_status lso_host_alloc(uint64_t bytes, void** out);
lso_status lso_host_free(void* p);

/* Static text of a status, and the detail of the calling thread's last
 * error ("" if none). */
const char* lso_status_string(lso_status s);
const char* lso_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LSO_H */
