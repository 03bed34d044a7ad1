// Expert pool files in the runtime layout (host code).
//
// FreeToken paper summary (agihunt.info, arXiv 2608.16157), execution-layer paragraph: the
// weights are merged ahead of time into the runtime layout, and loading puts them straight
// into their final place (no fill-then-overwrite pass).  Here the pool is pinned memory
// from hipHostMalloc (pinning memory that already exists is not available on this platform),
// and a pool file is read straight into it by several threads, each a contiguous range.
//
// File: a 64-byte header - magic "MOEPOOL1", then int32 layers, experts, hidden, inter,
// wfmt, int64 blob_bytes, int64 blob count (layers * experts) - followed by the blobs in key
// order (key = layer * experts + expert), each in the layout moe_blob_bytes describes.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstring>
#include <thread>
#include <vector>

#include "../../include/moe_offload.h"

namespace {

struct PoolHeader {
  char magic[8];
  int32_t layers, experts, hidden, inter, wfmt, pad;
  int64_t blob_bytes, blobs;
  char reserved[64 - 8 - 6 * 4 - 2 * 8];
};
static_assert(sizeof(PoolHeader) == 64, "pool file header");
constexpr char kMagic[8] = {'M', 'O', 'E', 'P', 'O', 'O', 'L', '1'};

bool shape_valid(const moe_shape* s) {
  return s && s->layers > 0 && s->experts > 0 && s->blob_bytes > 0 &&
         s->blob_bytes == moe_blob_bytes(s->wfmt, s->hidden, s->inter);
}

// every thread moves one contiguous range with pread / pwrite, retrying short transfers
bool parallel_io(int fd, unsigned char* buf, size_t bytes, off_t base, int threads, bool write) {
  if (threads < 1) threads = 1;
  std::vector<std::thread> th;
  std::vector<int> ok(threads, 1);
  for (int k = 0; k < threads; ++k) {
    th.emplace_back([&, k] {
      size_t a = bytes / threads * k, b = k + 1 == threads ? bytes : bytes / threads * (k + 1);
      while (a < b) {
        const size_t n = b - a < ((size_t)64 << 20) ? b - a : ((size_t)64 << 20);
        const ssize_t r = write ? pwrite(fd, buf + a, n, base + (off_t)a)
                                : pread(fd, buf + a, n, base + (off_t)a);
        if (r <= 0) {
          ok[k] = 0;
          return;
        }
        a += (size_t)r;
      }
    });
  }
  for (auto& t : th) t.join();
  for (int v : ok)
    if (!v) return false;
  return true;
}

}  // namespace

extern "C" {

moe_status moe_pool_write(const char* path, const moe_shape* shape, const void* pool,
                          int32_t threads) {
  if (!path || !pool || !shape_valid(shape) || threads < 1) return MOE_E_INVALID;
  PoolHeader h{};
  std::memcpy(h.magic, kMagic, 8);
  h.layers = shape->layers;
  h.experts = shape->experts;
  h.hidden = shape->hidden;
  h.inter = shape->inter;
  h.wfmt = shape->wfmt;
  h.blob_bytes = shape->blob_bytes;
  h.blobs = (int64_t)shape->layers * shape->experts;
  const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (fd < 0) return MOE_E_INVALID;
  bool good = pwrite(fd, &h, sizeof h, 0) == (ssize_t)sizeof h;
  const size_t bytes = (size_t)h.blobs * (size_t)h.blob_bytes;
  if (good) good = parallel_io(fd, (unsigned char*)pool, bytes, sizeof h, threads, true);
  good = (close(fd) == 0) && good;
  return good ? MOE_OK : MOE_E_INVALID;
}

moe_status moe_pool_read(const char* path, const moe_shape* shape, void* pool, int32_t threads) {
  if (!path || !pool || !shape_valid(shape) || threads < 1) return MOE_E_INVALID;
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return MOE_E_INVALID;
  PoolHeader h{};
  bool good = pread(fd, &h, sizeof h, 0) == (ssize_t)sizeof h;
  good = good && std::memcmp(h.magic, kMagic, 8) == 0 && h.layers == shape->layers &&
         h.experts == shape->experts && h.hidden == shape->hidden && h.inter == shape->inter &&
         h.wfmt == shape->wfmt && h.blob_bytes == shape->blob_bytes &&
         h.blobs == (int64_t)shape->layers * shape->experts;
  const size_t bytes = good ? (size_t)h.blobs * (size_t)h.blob_bytes : 0;
  struct stat st {};
  good = good && fstat(fd, &st) == 0 && (size_t)st.st_size == sizeof h + bytes;
  if (good) good = parallel_io(fd, (unsigned char*)pool, bytes, sizeof h, threads, false);
  close(fd);
  return good ? MOE_OK : MOE_E_INVALID;
}

}  // extern "C"
