// Storage probe (not part of the update path): what one file reaches for
// large sequential pread / pwrite, alone and both at once, with the same
// part size and thread count the layer stream's worker pools use.  It is
// the peak the disk tier is measured against.
#include <fcntl.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// Move [off, off + bytes) of fd to/from buf with `threads` threads taking
// 4 KB-multiple parts in order.  Returns 0 or an errno.
int transfer(int fd, char* buf, uint64_t off, uint64_t bytes, unsigned threads, bool write)
{
    uint64_t part = (bytes / (4ull * threads) + 4095) & ~uint64_t(4095);
    part = std::min<uint64_t>(std::max<uint64_t>(part, 4ull << 20), 256ull << 20);
    const uint64_t parts = (bytes + part - 1) / part;
    std::atomic<uint64_t> next{0};
    std::atomic<int> err{0};
    auto work = [&] {
        for (;;) {
            const uint64_t k = next.fetch_add(1);
            if (k >= parts || err.load()) return;
            uint64_t lo = k * part;
            const uint64_t hi = std::min(bytes, lo + part);
            while (lo < hi) {
                const size_t len = static_cast<size_t>(std::min<uint64_t>(hi - lo, 1ull << 30));
                const ssize_t r = write ? ::pwrite(fd, buf + lo, len, static_cast<off_t>(off + lo))
                                        : ::pread(fd, buf + lo, len, static_cast<off_t>(off + lo));
                if (r < 0 && errno == EINTR) continue;
                if (r <= 0) {
                    int expected = 0;
                    err.compare_exchange_strong(expected, r < 0 ? errno : EIO);
                    return;
                }
                lo += static_cast<uint64_t>(r);
            }
        }
    };
    std::vector<std::thread> pool;
    for (unsigned t = 0; t < threads; ++t) pool.emplace_back(work);
    for (auto& t : pool) t.join();
    return err.load();
}

double seconds_since(std::chrono::steady_clock::time_point t0)
{
    return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

extern "C" {

// fd: open O_RDWR (O_DIRECT allowed), holding at least
// max(off_read, off_write) + bytes bytes; the two ranges must not overlap.
// Both ranges are overwritten.  offsets and bytes: 4096-byte multiples.
// out[0] read alone, out[1] write alone (with fdatasync), out[2] read and
// out[3] write while both run, in GB/s.  Returns 0 or an errno.
int lso_probe_file(int fd, uint64_t off_read, uint64_t off_write, uint64_t bytes, int threads,
                   double out[4])
{
    if (fd < 0 || bytes == 0 || threads < 1 || !out || (off_read | off_write | bytes) % 4096 != 0)
        return EINVAL;
    if (off_read < off_write + bytes && off_write < off_read + bytes) return EINVAL;
    void* a = nullptr;
    void* b = nullptr;
    if (posix_memalign(&a, 4096, bytes) != 0) return ENOMEM;
    if (posix_memalign(&b, 4096, bytes) != 0) {
        std::free(a);
        return ENOMEM;
    }
    std::memset(b, 0x5A, bytes);
    const unsigned T = static_cast<unsigned>(threads);
    std::memset(a, 0xA5, bytes);
    // Both ranges are written first, so every timed pass moves real data
    // (a read of a never-written, preallocated range returns zeros without
    // touching the device, and a first write converts extents).
    int rc = transfer(fd, static_cast<char*>(b), off_write, bytes, T, true);
    auto t0 = std::chrono::steady_clock::now();
    if (!rc) rc = transfer(fd, static_cast<char*>(a), off_read, bytes, T, true);
    if (!rc && ::fdatasync(fd) != 0) rc = errno;
    out[1] = bytes / seconds_since(t0) / 1e9;
    t0 = std::chrono::steady_clock::now();
    if (!rc) rc = transfer(fd, static_cast<char*>(a), off_read, bytes, T, false);
    out[0] = bytes / seconds_since(t0) / 1e9;
    double tr = 0, tw = 0;
    int rr = 0, rw = 0;
    t0 = std::chrono::steady_clock::now();
    std::thread reader([&] {
        rr = transfer(fd, static_cast<char*>(a), off_read, bytes, T, false);
        tr = seconds_since(t0);
    });
    std::thread writer([&] {
        rw = transfer(fd, static_cast<char*>(b), off_write, bytes, T, true);
        tw = seconds_since(t0);
    });
    reader.join();
    writer.join();
    if (!rc) rc = rr ? rr : rw;
    out[2] = bytes / tr / 1e9;
    out[3] = bytes / tw / 1e9;
    std::free(a);
    std::free(b);
    return rc;
}

}  // extern "C"
