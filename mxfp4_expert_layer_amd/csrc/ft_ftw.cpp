// FTW expert files: the blob store on disk (lowalt.boxinlu2.cn article, section 三: every tensor
// 4096-aligned, so an expert moves from disk in a few large direct reads).  The file is a
// 4096-byte header page followed by the packed blobs at one stride; blobs are stored exactly
// as ft_pack_expert lays them out, so a read lands them ready for the slot pool and the host
// FFN with no conversion.
#include "ft_ftw.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

using namespace ft;

namespace {

constexpr uint32_t kFtwMagic = 0x31575446u;  // "FTW1"
constexpr uint32_t kFtwVersion = 1;

struct FtwHeader {
  uint32_t magic, version;
  int32_t fmt, H, I, E, n_shared, reserved0;
  uint64_t blob_bytes, blob_stride, data_offset, file_bytes;
  uint64_t reserved[8];
};
static_assert(sizeof(FtwHeader) <= kAlign, "header fits its page");

bool dims_valid(int fmt, int H, int I) {
  return (fmt == FT_MXFP4 || fmt == FT_NVFP4) && H > 0 && I > 0 && H % kTileK == 0 &&
         I % kTileK == 0;
}

int io_fail(const std::string& what, const char* path) {
  return fail(FT_EIO, what + " '" + path + "': " + std::strerror(errno));
}

// full write / read at an offset, retrying short transfers and EINTR
bool write_all(int fd, const uint8_t* p, uint64_t n, uint64_t off) {
  while (n > 0) {
    const ssize_t w = pwrite(fd, p, n, (off_t)off);
    if (w < 0 && errno == EINTR) continue;
    if (w <= 0) return false;
    p += w; n -= (uint64_t)w; off += (uint64_t)w;
  }
  return true;
}

bool read_all(int fd, uint8_t* p, uint64_t n, uint64_t off) {
  while (n > 0) {
    const ssize_t r = pread(fd, p, n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) {
      if (r == 0) errno = EIO;   // past the end: the file is shorter than its header says
      return false;
    }
    p += r; n -= (uint64_t)r; off += (uint64_t)r;
  }
  return true;
}

}  // namespace

struct ft_ftw {
  int fd = -1;
  int direct = 0;
  std::atomic<int> staged{0};   // direct reads go through aligned staging buffers
  std::string path;
  FtwHeader h{};
};

namespace ft {
uint64_t ftw_blob_stride(const ft_ftw* f) { return f->h.blob_stride; }
void ftw_dims(const ft_ftw* f, int* fmt, int* H, int* I, int* E, int* n_shared) {
  *fmt = f->h.fmt; *H = f->h.H; *I = f->h.I; *E = f->h.E; *n_shared = f->h.n_shared;
}
}  // namespace ft

extern "C" FT_API int ft_ftw_write(const char* path, int format, int H, int I, int E,
                                   int n_shared, const void* blobs, uint64_t src_stride) try {
  if (!path || !blobs || !dims_valid(format, H, I) || E < 1 || n_shared < 0)
    return fail(FT_EINVAL, "ft_ftw_write: bad argument");
  const BlobLayout L = blob_layout(format, H, I);
  if (src_stride < L.bytes) return fail(FT_EINVAL, "ft_ftw_write: src_stride below the blob size");
  const int nb = E + n_shared;
  for (int i = 0; i < nb; ++i) {
    BlobHeader bh;
    std::memcpy(&bh, (const uint8_t*)blobs + (uint64_t)i * src_stride, sizeof(bh));
    if (bh.magic != kBlobMagic || bh.fmt != format || bh.H != H || bh.I != I)
      return fail(FT_EINVAL, "ft_ftw_write: blob " + std::to_string(i) +
                                 " is not a packed blob of these dimensions");
  }
  std::vector<uint8_t> page(kAlign, 0);
  FtwHeader h{};
  h.magic = kFtwMagic;
  h.version = kFtwVersion;
  h.fmt = format; h.H = H; h.I = I; h.E = E; h.n_shared = n_shared;
  h.blob_bytes = L.bytes;
  h.blob_stride = L.bytes;
  h.data_offset = kAlign;
  h.file_bytes = kAlign + (uint64_t)nb * L.bytes;
  std::memcpy(page.data(), &h, sizeof(h));
  const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (fd < 0) return io_fail("ft_ftw_write: cannot create", path);
  bool ok = write_all(fd, page.data(), kAlign, 0);
  for (int i = 0; ok && i < nb; ++i)
    ok = write_all(fd, (const uint8_t*)blobs + (uint64_t)i * src_stride, L.bytes,
                   h.data_offset + (uint64_t)i * h.blob_stride);
  if (ok) ok = fsync(fd) == 0;
  const int saved = errno;
  if (close(fd) != 0 && ok) return io_fail("ft_ftw_write: close failed for", path);
  errno = saved;
  if (!ok) return io_fail("ft_ftw_write: write failed for", path);
  return FT_OK;
} FT_CATCH("ft_ftw_write")

extern "C" FT_API int ft_ftw_open(const char* path, int flags, ft_ftw** out) try {
  if (!path || !out || (flags & ~(FT_FTW_DIRECT | FT_FTW_STAGED)))
    return fail(FT_EINVAL, "ft_ftw_open: bad argument");
  int fd = -1, direct = 0;
  if (flags & FT_FTW_DIRECT) {
    fd = open(path, O_RDONLY | O_DIRECT);
    direct = fd >= 0;
  }
  if (fd < 0) fd = open(path, O_RDONLY);
  if (fd < 0) return io_fail("ft_ftw_open: cannot open", path);
  void* page = nullptr;
  if (posix_memalign(&page, kAlign, kAlign) != 0) {
    close(fd);
    return fail(FT_ENOMEM, "ft_ftw_open: out of host memory");
  }
  FtwHeader h{};
  const bool got = read_all(fd, (uint8_t*)page, kAlign, 0);
  std::memcpy(&h, page, sizeof(h));
  std::free(page);
  struct stat stt{};
  if (!got || fstat(fd, &stt) != 0) {
    const int rc = io_fail("ft_ftw_open: cannot read the header of", path);
    close(fd);
    return rc;
  }
  std::string why;
  if (h.magic != kFtwMagic) why = "not an FTW file";
  else if (h.version != kFtwVersion) why = "unknown version";
  else if (!dims_valid(h.fmt, h.H, h.I) || h.E < 1 || h.n_shared < 0) why = "bad dimensions";
  else if (h.blob_bytes != blob_layout(h.fmt, h.H, h.I).bytes) why = "blob size does not match";
  else if (h.blob_stride < h.blob_bytes || h.blob_stride % kAlign || h.data_offset % kAlign ||
           h.data_offset < kAlign)
    why = "misaligned layout";
  else if (h.file_bytes != h.data_offset + (uint64_t)(h.E + h.n_shared) * h.blob_stride ||
           (uint64_t)stt.st_size < h.file_bytes)
    why = "file shorter than its header says";
  if (!why.empty()) {
    close(fd);
    return fail(FT_EINVAL, std::string("ft_ftw_open: '") + path + "': " + why);
  }
  ft_ftw* f = new (std::nothrow) ft_ftw;
  if (!f) {
    close(fd);
    return fail(FT_ENOMEM, "ft_ftw_open: out of host memory");
  }
  f->fd = fd;
  f->direct = direct;
  f->staged = direct && (flags & FT_FTW_STAGED);
  f->path = path;
  f->h = h;
  *out = f;
  return FT_OK;
} FT_CATCH("ft_ftw_open")

extern "C" FT_API int ft_ftw_get_info(const ft_ftw* f, ft_ftw_info* info) try {
  if (!f || !info) return fail(FT_EINVAL, "ft_ftw_get_info: null argument");
  info->format = f->h.fmt;
  info->H = f->h.H;
  info->I = f->h.I;
  info->E = f->h.E;
  info->n_shared = f->h.n_shared;
  info->direct = f->direct;
  info->staged = f->staged.load();
  info->reserved = 0;
  info->blob_bytes = f->h.blob_bytes;
  info->file_bytes = f->h.file_bytes;
  return FT_OK;
} FT_CATCH("ft_ftw_get_info")

extern "C" FT_API int ft_ftw_close(ft_ftw* f) try {
  if (!f) return FT_OK;
  if (f->fd >= 0) close(f->fd);
  delete f;
  return FT_OK;
} FT_CATCH("ft_ftw_close")

namespace ft {
int ftw_read(ThreadPool* pool, ft_ftw* f, const int32_t* ids, int n, uint8_t* const* dst,
             uint64_t chunk) {
  const int nb = f->h.E + f->h.n_shared;
  const uint64_t bytes = f->h.blob_bytes;
  if (chunk == 0 || chunk > bytes) chunk = bytes;
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= nb) return fail(FT_EINVAL, "ft_ftw_read: blob id out of range");
    if (f->direct && ((uintptr_t)dst[i] % kAlign)) return fail(FT_EINVAL, "ft_ftw_read: O_DIRECT needs 4096-aligned destinations");
  }
  if (f->direct && chunk % kAlign) return fail(FT_EINVAL, "ft_ftw_read: O_DIRECT needs a chunk multiple of 4096");
  const uint64_t per = (bytes + chunk - 1) / chunk;
  const uint64_t total = (uint64_t)n * per;
  std::atomic<uint64_t> next{0};
  std::atomic<int> bad_errno{0};
  auto work = [&](int, int) {
    void* stage = nullptr;   // this thread's aligned staging buffer, made on first need
    constexpr uint64_t kStage = 4u << 20;
    auto staged_read = [&](uint8_t* p, uint64_t len, uint64_t off) {
      if (!stage && posix_memalign(&stage, kAlign, kStage) != 0) {
        stage = nullptr;
        errno = ENOMEM;
        return false;
      }
      while (len > 0) {
        const uint64_t l = std::min(len, kStage);
        if (!read_all(f->fd, (uint8_t*)stage, l, off)) return false;
        std::memcpy(p, stage, l);
        p += l; off += l; len -= l;
      }
      return true;
    };
    for (;;) {
      const uint64_t r = next.fetch_add(1);
      if (r >= total || bad_errno.load()) break;
      const int i = (int)(r / per);
      const uint64_t o = (r % per) * chunk;
      const uint64_t len = std::min(chunk, bytes - o);
      const uint64_t off = f->h.data_offset + (uint64_t)ids[i] * f->h.blob_stride + o;
      bool ok;
      if (f->staged.load()) {
        ok = staged_read(dst[i] + o, len, off);
      } else {
        ok = read_all(f->fd, dst[i] + o, len, off);
        if (!ok && f->direct && errno == EFAULT) {
          // the kernel cannot pin this destination for a direct read: stage from now on
          f->staged.store(1);
          ok = staged_read(dst[i] + o, len, off);
        }
      }
      if (!ok) {
        int expect = 0;
        bad_errno.compare_exchange_strong(expect, errno ? errno : EIO);
        break;
      }
    }
    std::free(stage);
  };
  if (pool && total > 1) pool->run(work);
  else work(0, 1);
  if (bad_errno.load()) {
    errno = bad_errno.load();
    return io_fail("ft_ftw_read: read failed for", f->path.c_str());
  }
  return FT_OK;
}
}  // namespace ft

extern "C" FT_API int ft_ftw_read(ft_ctx* ctx, ft_ftw* f, const int32_t* ids, int n, void* dst,
                                  uint64_t dst_stride, uint64_t chunk, double* seconds) try {
  if (!f || n < 0 || (n > 0 && (!ids || !dst))) return fail(FT_EINVAL, "ft_ftw_read: bad argument");
  if (dst_stride < f->h.blob_bytes && n > 1) return fail(FT_EINVAL, "ft_ftw_read: dst_stride below the blob size");
  if (f->direct && dst_stride % kAlign) return fail(FT_EINVAL, "ft_ftw_read: O_DIRECT needs a dst_stride multiple of 4096");
  std::vector<uint8_t*> d(n);
  for (int i = 0; i < n; ++i) d[i] = (uint8_t*)dst + (uint64_t)i * dst_stride;
  const auto t0 = std::chrono::steady_clock::now();
  const int rc = ftw_read(ctx_pool(ctx), f, ids, n, d.data(), chunk);
  if (seconds)
    *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  return rc;
} FT_CATCH("ft_ftw_read")
