// Worker pools of the layer stream (see lso_io.h).
#include "lso_io.h"

#include <fcntl.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstdlib>
#include <cstring>
#include <memory>

#include "lso_shadow.h"

namespace lso {
namespace {

void note_error(IoRequest* r, int e)
{
    int expected = 0;
    r->err.compare_exchange_strong(expected, e ? e : EIO);
}

// pread / pwrite of [off, off + len) of the file to / from buf, whole.
bool file_io(IoRequest* r, char* buf, uint64_t off, uint64_t len, bool read)
{
    uint64_t done = 0;
    while (done < len) {
        const size_t step = static_cast<size_t>(std::min<uint64_t>(len - done, 1ull << 30));
        const off_t fo = static_cast<off_t>(r->foff + off + done);
        const ssize_t k = read ? ::pread(r->fd, buf + done, step, fo)
                               : ::pwrite(r->fd, buf + done, step, fo);
        if (k < 0) {
            if (errno == EINTR) continue;
            note_error(r, errno);
            return false;
        }
        if (k == 0) {   // end of file on a read, or a device that takes nothing
            note_error(r, EIO);
            return false;
        }
        done += static_cast<uint64_t>(k);
    }
    return true;
}

uint64_t bounce_bytes()
{
    static const uint64_t b = [] {
        const char* e = std::getenv("LSO_IO_BOUNCE_MB");
        const int mb = e ? std::atoi(e) : 0;
        return static_cast<uint64_t>(mb >= 1 && mb <= 256 ? mb : 64) << 20;
    }();
    return b;
}

void do_part(IoRequest* r, uint64_t lo, uint64_t hi)
{
    if (r->op == kIoCopy) {
        if (hi > lo) std::memcpy(r->dst + lo, r->src + lo, hi - lo);
        return;
    }
    const bool read = r->op == kIoRead;
    if (!r->direct) {
        if (read) file_io(r, r->dst + lo, lo, hi - lo, true);
        else file_io(r, const_cast<char*>(r->src) + lo, lo, hi - lo, false);
        return;
    }
    // O_DIRECT: through this thread's page-aligned bounce buffer
    thread_local std::unique_ptr<char, decltype(&std::free)> bounce(nullptr, &std::free);
    if (!bounce) {
        void* q = nullptr;
        if (posix_memalign(&q, 4096, bounce_bytes()) != 0) {
            note_error(r, ENOMEM);
            return;
        }
        bounce.reset(static_cast<char*>(q));
    }
    for (uint64_t off = lo; off < hi && r->err.load(std::memory_order_relaxed) == 0;) {
        const uint64_t len = std::min(bounce_bytes(), hi - off);
        if (read) {
            if (!file_io(r, bounce.get(), off, len, true)) return;
            std::memcpy(r->dst + off, bounce.get(), len);
        } else {
            std::memcpy(bounce.get(), r->src + off, len);
            if (!file_io(r, bounce.get(), off, len, false)) return;
        }
        off += len;
    }
}

}  // namespace

IoPool::IoPool(unsigned threads, std::mutex* note_mu, std::condition_variable* note_cv,
               std::atomic<uint64_t>* note_gen)
    : n_(threads ? threads : 1), note_mu_(note_mu), note_cv_(note_cv), note_gen_(note_gen)
{
    for (unsigned k = 0; k < n_; ++k) workers_.emplace_back([this] { run(); });
}

IoPool::~IoPool()
{
    {
        std::lock_guard<std::mutex> l(mu_);
        stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
}

void IoPool::submit(IoRequest* r)
{
    uint64_t part = (r->bytes / (4ull * n_) + 4095) & ~uint64_t(4095);
    part = std::min<uint64_t>(std::max<uint64_t>(part, 4ull << 20), 256ull << 20);
    const uint64_t parts = r->bytes == 0 ? 1 : (r->bytes + part - 1) / part;
    r->parts_left.store(static_cast<uint32_t>(parts));
    {
        std::lock_guard<std::mutex> l(mu_);
        for (uint64_t k = 0; k < parts; ++k)
            q_.push_back({r, k * part, std::min(r->bytes, (k + 1) * part)});
    }
    cv_.notify_all();
}

void IoPool::run()
{
    for (;;) {
        Part p{};
        {
            std::unique_lock<std::mutex> l(mu_);
            cv_.wait(l, [&] { return stop_ || !q_.empty(); });
            if (q_.empty()) return;   // stop_ with nothing left
            p = q_.front();
            q_.pop_front();
        }
        do_part(p.r, p.lo, p.hi);
        IoRequest* r = p.r;
        if (r->parts_left.fetch_sub(1) == 1) {
            if (r->op == kIoWrite && r->err.load() == 0) {
                if ((r->sync || r->header) && ::fdatasync(r->fd) != 0) {
                    note_error(r, errno);
                } else if (r->header) {
                    // the data slot is on stable storage: commit it
                    IoRequest h;
                    h.fd = r->fd;
                    h.foff = r->header_off;
                    if (!file_io(&h, const_cast<char*>(r->header), 0, kShadowCopy, false))
                        note_error(r, h.err.load());
                    else if (::fdatasync(r->fd) != 0)
                        note_error(r, errno);
                }
            }
            {
                std::lock_guard<std::mutex> l(*note_mu_);
                r->done.store(true);
                note_gen_->fetch_add(1);
            }
            note_cv_->notify_all();
        }
    }
}

}  // namespace lso
