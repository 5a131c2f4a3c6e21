// Drives the host-side entry points of liblso (include/lso.h) that do no
// device work -- block validation, per-block constants, workspace sizes,
// the shadow-region headers on a scratch file, status strings and the
// argument checks that fail before any device call -- for a build of the
// whole library with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host side (device code is built as usual and never launched).  Exit
// status 0 when every call returned its documented status.  Test
// infrastructure only.
#include <fcntl.h>
#include <unistd.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "lso.h"

static int failures = 0;
#define EXPECT(cond)                                                                     \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::fprintf(stderr, "runtime driver: %s failed at line %d (%s)\n", #cond,  \
                         __LINE__, lso_last_error());                                    \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

static lso_block block(uint64_t addr, uint64_t n, uint32_t layout = LSO_LAYOUT_PLANAR)
{
    lso_block b{};
    b.base = nullptr;
    b.n = n;
    b.off_master = addr;
    b.off_m = addr + (16 << 20);
    b.off_v = addr + (32 << 20);
    b.off_grad = addr + (48 << 20);
    b.off_weight = addr + (56 << 20);
    b.grad_dtype = LSO_DT_BF16;
    b.weight_dtype = LSO_DT_BF16;
    b.opt = LSO_OPT_ADAM;
    b.layout = layout;
    if (layout == LSO_LAYOUT_TILED) b.off_m = b.off_v = b.off_master;
    b.t = 1;
    b.lr = 1e-3;
    b.beta1 = 0.9;
    b.beta2 = 0.999;
    b.eps = 1e-8;
    return b;
}

int main()
{
    // every value the enum can hold (0..15); the C test passes codes beyond
    for (int s = 0; s <= 15; ++s) EXPECT(lso_status_string(static_cast<lso_status>(s)) != nullptr);
    EXPECT(std::strcmp(lso_status_string(static_cast<lso_status>(15)), "unknown status") == 0);
    // validation: fake device addresses, never touched
    const uint64_t A = 1ull << 32;
    std::vector<lso_block> tab;
    for (int i = 0; i < 300; ++i) tab.push_back(block(A + (uint64_t(i) << 26), 1 + 37 * i));
    EXPECT(lso_validate_blocks(tab.data(), tab.size()) == LSO_OK);
    EXPECT(lso_validate_blocks(nullptr, 1) != LSO_OK);
    EXPECT(lso_validate_blocks(tab.data(), 0) == LSO_OK);
    std::vector<lso_block> bad = tab;
    bad[7].off_m += 4;   // misaligned
    EXPECT(lso_validate_blocks(bad.data(), bad.size()) == LSO_E_ALIGN);
    bad = tab;
    bad[9].off_v = bad[9].off_master;   // overlap inside a block
    EXPECT(lso_validate_blocks(bad.data(), bad.size()) == LSO_E_OVERLAP);
    bad = tab;
    bad[3].off_master = bad[4].off_master;   // overlap across blocks
    bad[3].off_m = bad[4].off_m + (1 << 12);
    EXPECT(lso_validate_blocks(bad.data(), bad.size()) != LSO_OK);
    bad = tab;
    bad[5].t = 0;
    EXPECT(lso_validate_blocks(bad.data(), bad.size()) == LSO_E_INVALID);
    bad = tab;
    bad[6].grad_dtype = 77;
    EXPECT(lso_validate_blocks(bad.data(), bad.size()) != LSO_OK);
    lso_block tb = block(A, 3 * 8192 + 5, LSO_LAYOUT_TILED);
    EXPECT(lso_validate_blocks(&tb, 1) == LSO_OK);
    // constants and sizes
    float c[8];
    EXPECT(lso_block_constants(&tab[0], c) == LSO_OK);
    EXPECT(lso_block_constants(nullptr, c) != LSO_OK);
    EXPECT(lso_norm_workspace_bytes(tab.data(), tab.size()) > 0);
    EXPECT(lso_norm_workspace_bytes(nullptr, 0) == 0);
    EXPECT(lso_tiled_state_bytes(0) == 0);
    EXPECT(lso_tiled_state_bytes(1) == 12ull * LSO_TILE_ELEMS);
    // argument checks ahead of any device call
    EXPECT(lso_adam_step(tab.data(), 0, nullptr) == LSO_OK);
    EXPECT(lso_adam_step(nullptr, 1, nullptr) != LSO_OK);
    // the allocation-free variant: its refusals come before any device call
    EXPECT(lso_adam_step_noalloc(tab.data(), 0, nullptr) == LSO_OK);
    EXPECT(lso_adam_step_noalloc(nullptr, 1, nullptr) != LSO_OK);
    std::vector<lso_block> many;
    for (uint64_t i = 0; i <= LSO_NOALLOC_MAX_BLOCKS; ++i) many.push_back(block(A + (i << 26), 16));
    EXPECT(lso_adam_step_noalloc(many.data(), many.size(), nullptr) == LSO_E_INVALID);
    EXPECT(lso_adam_step_noalloc(bad.data(), bad.size(), nullptr) != LSO_OK);
    const uint64_t launches = lso_kernel_launches();
    EXPECT(lso_kernel_launches() == launches);
    uint64_t stats[3] = {1, 1, 1};
    EXPECT(lso_stream_stats(nullptr, stats) == -1 && stats[0] == 1);
    lso_stream_ctx* ctx = reinterpret_cast<lso_stream_ctx*>(1);
    EXPECT(lso_stream_create(0, 1, nullptr, nullptr, 0, &ctx) == LSO_E_INVALID && ctx == nullptr);
    EXPECT(lso_stream_copy_mode(nullptr, nullptr, nullptr) == -1);
    EXPECT(lso_stream_layers(nullptr, nullptr, 1) == LSO_E_INVALID);
    EXPECT(lso_stream_files(nullptr, nullptr, 1) == LSO_E_INVALID);
    EXPECT(lso_host_alloc(0, nullptr) == LSO_E_INVALID);
    // shadow regions on a scratch file
    char path[] = "/tmp/lso_runtime_driver_XXXXXX";
    const int fd = mkstemp(path);
    EXPECT(fd >= 0);
    const uint64_t bytes = 8192, off = 4096;
    EXPECT(ftruncate(fd, off + LSO_SHADOW_HEADER_BYTES + 2 * bytes) == 0);
    EXPECT(lso_shadow_format(fd, off, bytes, 5) == LSO_OK);
    uint64_t epoch = 99, t = 99, data = 0;
    EXPECT(lso_shadow_state(fd, off, bytes, &epoch, &t, &data) == LSO_OK && epoch == 0 && t == 5);
    EXPECT(lso_shadow_commit(fd, off, bytes, 1, 6) == LSO_OK);
    EXPECT(lso_shadow_state(fd, off, bytes, &epoch, &t, &data) == LSO_OK && epoch == 1 && t == 6);
    // a torn newest copy: the older one wins
    const char junk[64] = "torn header torn header torn header torn header torn header";
    EXPECT(pwrite(fd, junk, sizeof junk, off + 4096) == static_cast<ssize_t>(sizeof junk));
    EXPECT(lso_shadow_state(fd, off, bytes, &epoch, &t, &data) == LSO_OK && epoch == 0 && t == 5);
    // both copies gone
    EXPECT(pwrite(fd, junk, sizeof junk, off) == static_cast<ssize_t>(sizeof junk));
    EXPECT(lso_shadow_state(fd, off, bytes, &epoch, &t, &data) == LSO_E_IO);
    EXPECT(lso_shadow_format(fd, off + 1, bytes, 0) == LSO_E_ALIGN);
    EXPECT(lso_shadow_format(-1, off, bytes, 0) != LSO_OK);
    EXPECT(lso_shadow_state(fd, off, bytes, nullptr, nullptr, nullptr) != LSO_OK);
    close(fd);
    unlink(path);
    if (failures) return 1;
    std::printf("runtime driver: every call returned its documented status\n");
    return 0;
}
