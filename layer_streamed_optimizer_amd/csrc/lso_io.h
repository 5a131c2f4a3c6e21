// Worker pools for the layer stream's host side: each stage-in (memcpy
// from pageable memory, or pread from a file) and each write-out (memcpy or
// pwrite, with fdatasync and a shadow commit when asked) is one request,
// split into parts that the pool's threads take in order.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <deque>
#include <mutex>
#include <thread>
#include <vector>

namespace lso {

enum IoOp { kIoCopy = 0, kIoRead = 1, kIoWrite = 2 };

// One transfer between a staging buffer and the authoritative copy, split
// into parts that the pool's threads take in order.
struct IoRequest {
    IoOp op = kIoCopy;
    char* dst = nullptr;         // copy destination, or the pread buffer
    const char* src = nullptr;   // copy source, or the pwrite buffer
    int fd = -1;
    uint64_t foff = 0;           // file offset of byte 0
    uint64_t bytes = 0;
    bool sync = false;           // fdatasync(fd) after the last part
    bool direct = false;         // fd is O_DIRECT: transfer through a bounce buffer
    const char* header = nullptr;   // shadow commit: after the data is flushed,
    uint64_t header_off = 0;        // write this header copy here and flush
    std::atomic<uint32_t> parts_left{0};
    std::atomic<int> err{0};     // first errno seen; EIO for end of file
    std::atomic<bool> done{false};

    void reset()
    {
        parts_left.store(0);
        err.store(0);
        done.store(false);
    }
};

class IoPool {
public:
    // threads workers; whenever a request completes, *note_gen is
    // incremented under *note_mu and *note_cv notified.
    IoPool(unsigned threads, std::mutex* note_mu, std::condition_variable* note_cv,
           std::atomic<uint64_t>* note_gen);
    ~IoPool();   // joins the threads; no request may be in flight

    // Parts of 4 KB multiples, about 4 per thread, 4-256 MB each.  r must
    // stay alive (and untouched) until r->done.
    void submit(IoRequest* r);

private:
    struct Part {
        IoRequest* r;
        uint64_t lo, hi;
    };

    void run();

    unsigned n_;
    std::mutex* note_mu_;
    std::condition_variable* note_cv_;
    std::atomic<uint64_t>* note_gen_;
    std::vector<std::thread> workers_;
    std::mutex mu_;
    std::condition_variable cv_;
    std::deque<Part> q_;
    bool stop_ = false;
};

}  // namespace lso
