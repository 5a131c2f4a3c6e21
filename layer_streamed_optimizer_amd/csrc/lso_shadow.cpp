// Shadow regions for crash-consistent write-back.
//
// The frozen-incremental page (section "Verification", its safety note)
// warns that a crash between the in-place update and the flush can corrupt
// the state and asks for atomic writes or shadow copies.  A shadow region
// holds two data slots and two header copies; epoch e lives in data slot
// e % 2 and is committed by header copy e % 2, written only after its data
// slot is on stable storage.  A header copy is valid when its magic, its
// size field and its checksum (CRC-32C, the Castagnoli polynomial, over
// the first 32 bytes) match; a torn or stale copy fails the check or loses
// on epoch, so the committed state is always a whole block.
//
// Header copy (little-endian): magic "LSOSHDW1" | epoch u64 | bytes u64 |
// t u64 | crc32c u32 | zeros to 4096 bytes.
#include "lso_shadow.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstdlib>
#include <cstring>
#include <memory>

#include "lso_runtime.h"

namespace lso {
namespace {

constexpr char kMagic[8] = {'L', 'S', 'O', 'S', 'H', 'D', 'W', '1'};
constexpr size_t kFields = 32;   // bytes the checksum covers

// CRC-32C, reflected polynomial 0x82F63B78, table built on first use.
uint32_t crc32c(const unsigned char* p, size_t n)
{
    static const auto table = [] {
        std::unique_ptr<uint32_t[]> t(new uint32_t[256]);
        for (uint32_t i = 0; i < 256; ++i) {
            uint32_t c = i;
            for (int k = 0; k < 8; ++k) c = (c & 1u) ? (c >> 1) ^ 0x82F63B78u : c >> 1;
            t[i] = c;
        }
        return t;
    }();
    uint32_t c = 0xFFFFFFFFu;
    for (size_t i = 0; i < n; ++i) c = table[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
    return c ^ 0xFFFFFFFFu;
}

void put64(unsigned char* p, uint64_t v)
{
    for (int k = 0; k < 8; ++k) p[k] = static_cast<unsigned char>(v >> (8 * k));
}

uint64_t get64(const unsigned char* p)
{
    uint64_t v = 0;
    for (int k = 7; k >= 0; --k) v = (v << 8) | p[k];
    return v;
}

// A page-aligned buffer (O_DIRECT descriptors need one).
struct Aligned {
    void* p = nullptr;
    explicit Aligned(size_t n)
    {
        if (posix_memalign(&p, 4096, n) != 0) p = nullptr;
        else std::memset(p, 0, n);
    }
    ~Aligned() { std::free(p); }
    char* get() const { return static_cast<char*>(p); }
};

bool full_io(int fd, char* buf, size_t n, uint64_t off, bool write)
{
    size_t done = 0;
    while (done < n) {
        const ssize_t k = write ? ::pwrite(fd, buf + done, n - done, static_cast<off_t>(off + done))
                                : ::pread(fd, buf + done, n - done, static_cast<off_t>(off + done));
        if (k < 0 && errno == EINTR) continue;
        if (k <= 0) {
            if (k == 0) errno = EIO;
            return false;
        }
        done += static_cast<size_t>(k);
    }
    return true;
}

// Decode one copy; false if it is not a valid header for `bytes`.
bool decode(const char* buf, uint64_t bytes, ShadowState* st)
{
    const auto* u = reinterpret_cast<const unsigned char*>(buf);
    if (std::memcmp(u, kMagic, 8) != 0) return false;
    const uint32_t crc = static_cast<uint32_t>(u[32]) | (static_cast<uint32_t>(u[33]) << 8) |
                         (static_cast<uint32_t>(u[34]) << 16) | (static_cast<uint32_t>(u[35]) << 24);
    if (crc != crc32c(u, kFields)) return false;
    if (get64(u + 16) != bytes) return false;
    st->epoch = get64(u + 8);
    st->t = get64(u + 24);
    return true;
}

lso_status check_region(int fd, uint64_t off, uint64_t bytes, bool need_size)
{
    if (off % 4096 != 0 || bytes % 4096 != 0)
        return fail(LSO_E_ALIGN, "shadow region offset and bytes must be 4096-byte multiples");
    if (bytes == 0) return fail(LSO_E_INVALID, "shadow region of 0 bytes");
    struct stat s {};
    if (fd < 0 || ::fstat(fd, &s) != 0) return fail(LSO_E_INVALID, "fd %d is not an open file", fd);
    if (need_size && S_ISREG(s.st_mode) &&
        static_cast<uint64_t>(s.st_size) < off + LSO_SHADOW_HEADER_BYTES + 2 * bytes)
        return fail(LSO_E_INVALID, "the file ends before the shadow region does");
    return LSO_OK;
}

lso_status write_header(int fd, uint64_t off, uint64_t bytes, uint64_t epoch, uint64_t t)
{
    Aligned buf(kShadowCopy);
    if (!buf.get()) return fail(LSO_E_NOMEM, "header buffer");
    shadow_encode(buf.get(), epoch, bytes, t);
    if (!full_io(fd, buf.get(), kShadowCopy, shadow_header(off, epoch), true) || ::fdatasync(fd) != 0)
        return fail(LSO_E_IO, "writing a shadow header failed: %s", std::strerror(errno));
    return LSO_OK;
}

}  // namespace

void shadow_encode(char* buf, uint64_t epoch, uint64_t bytes, uint64_t t)
{
    auto* u = reinterpret_cast<unsigned char*>(buf);
    std::memset(u, 0, kShadowCopy);
    std::memcpy(u, kMagic, 8);
    put64(u + 8, epoch);
    put64(u + 16, bytes);
    put64(u + 24, t);
    const uint32_t crc = crc32c(u, kFields);
    for (int k = 0; k < 4; ++k) u[32 + k] = static_cast<unsigned char>(crc >> (8 * k));
}

lso_status shadow_read(int fd, uint64_t off, uint64_t bytes, ShadowState* st)
{
    Aligned buf(2 * kShadowCopy);
    if (!buf.get()) return fail(LSO_E_NOMEM, "header buffer");
    if (!full_io(fd, buf.get(), 2 * kShadowCopy, off, false))
        return fail(LSO_E_IO, "reading the shadow headers failed: %s", std::strerror(errno));
    ShadowState a, b;
    const bool va = decode(buf.get(), bytes, &a);
    const bool vb = decode(buf.get() + kShadowCopy, bytes, &b);
    // a copy is only believed for the epochs it can hold (copy k: e % 2 == k)
    const bool ok_a = va && a.epoch % 2 == 0;
    const bool ok_b = vb && b.epoch % 2 == 1;
    if (!ok_a && !ok_b) return fail(LSO_E_IO, "no valid shadow header (never formatted, or both copies damaged)");
    *st = (ok_a && (!ok_b || a.epoch > b.epoch)) ? a : b;
    return LSO_OK;
}

}  // namespace lso

extern "C" {

lso_status lso_shadow_format(int fd, uint64_t file_offset, uint64_t bytes, uint64_t t0)
{
    lso::clear_error();
    lso_status s = lso::check_region(fd, file_offset, bytes, true);
    if (s != LSO_OK) return s;
    lso::Aligned zero(lso::kShadowCopy);
    if (!zero.get()) return lso::fail(LSO_E_NOMEM, "header buffer");
    // copy 1 cleared first, so a crash while formatting leaves no valid
    // header for a stale epoch
    if (!lso::full_io(fd, zero.get(), lso::kShadowCopy, file_offset + lso::kShadowCopy, true) ||
        ::fdatasync(fd) != 0)
        return lso::fail(LSO_E_IO, "clearing a shadow header failed: %s", std::strerror(errno));
    return lso::write_header(fd, file_offset, bytes, 0, t0);
}

lso_status lso_shadow_state(int fd, uint64_t file_offset, uint64_t bytes, uint64_t* epoch, uint64_t* t,
                            uint64_t* data_offset)
{
    lso::clear_error();
    lso_status s = lso::check_region(fd, file_offset, bytes, false);
    if (s != LSO_OK) return s;
    lso::ShadowState st;
    s = lso::shadow_read(fd, file_offset, bytes, &st);
    if (s != LSO_OK) return s;
    if (epoch) *epoch = st.epoch;
    if (t) *t = st.t;
    if (data_offset) *data_offset = lso::shadow_slot(file_offset, bytes, st.epoch);
    return LSO_OK;
}

lso_status lso_shadow_commit(int fd, uint64_t file_offset, uint64_t bytes, uint64_t epoch, uint64_t t)
{
    lso::clear_error();
    lso_status s = lso::check_region(fd, file_offset, bytes, true);
    if (s != LSO_OK) return s;
    return lso::write_header(fd, file_offset, bytes, epoch, t);
}

}  // extern "C"
