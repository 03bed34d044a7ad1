// Measurement probes: the device-memory streaming-read ceiling the expert FFN is judged
// against, and the fixed cost of a launch.
//
// stream_read_kernel reads a buffer once, every byte exactly once, in the access pattern of the
// decode FFN's weight stream: a 256-thread workgroup owns a contiguous 96 KiB run, each thread
// issues all 24 of its 16-byte loads (lane-contiguous, 1 KiB per wave per instruction) before
// it uses any, and folds them into one word.  A launch over a buffer of the FFN launch's size
// is therefore the ceiling of such a launch (dispatch, ramp-up and drain included); a launch
// over gigabytes is the chip's sustained streaming rate.  The fold is stored only if it equals
// a fixed constant, which keeps the loads from being optimised away.
#include <vector>

#include "moe_dev.h"

namespace moe {

constexpr int PRB_T = 256;  // threads per workgroup
constexpr int PRB_L = 24;   // 16-byte loads per thread, all in flight
constexpr uint32_t kFoldMark = 0x9e3779b9u;

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(PRB_T) void stream_read_kernel(const u32x4p* p, long long n16,
                                                            uint32_t* sink) {
  const long long base = (long long)blockIdx.x * (PRB_T * PRB_L) + threadIdx.x;
  u32x4p r[PRB_L];
#pragma unroll
  for (int i = 0; i < PRB_L; ++i) {
    long long k = base + (long long)i * PRB_T;
    k = k < n16 ? k : n16 - 1;  // the tail re-reads the last chunk, in bounds
    if constexpr (NT)
      r[i] = __builtin_nontemporal_load(p + k);
    else
      r[i] = p[k];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < PRB_L; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
  if (acc == kFoldMark) sink[0] = acc;
}

__global__ __launch_bounds__(PRB_T) void empty_kernel() {}

// Plain device copy of n16 16-byte chunks: the reference kernel of known read and write bytes
// against which hardware byte counters are calibrated.
__global__ __launch_bounds__(PRB_T) void stream_copy_kernel(const u32x4p* src, u32x4p* dst,
                                                            long long n16) {
  const long long base = (long long)blockIdx.x * (PRB_T * 8) + threadIdx.x;
  u32x4p r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long long k = base + (long long)i * PRB_T;
    r[i] = src[k < n16 ? k : n16 - 1];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long long k = base + (long long)i * PRB_T;
    if (k < n16) dst[k] = r[i];
  }
}

// Average event-timed duration (us) of `reps` launches reading `bytes` each, launch r reading
// the r-th window of `bytes` (cyclically) inside the first `span` bytes of `buf`; one untimed
// launch first.  Synchronous.
hipError_t probe_stream_read(const void* buf, size_t span, size_t bytes, int nt, int reps,
                             uint32_t* sink, hipStream_t s, double* avg_us) {
  const size_t windows = span / bytes;
  const long long n16 = (long long)(bytes / 16);
  const int grid = (int)((n16 + PRB_T * PRB_L - 1) / (PRB_T * PRB_L));
  std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
  hipError_t e = hipSuccess;
  for (auto& x : ev)
    if (e == hipSuccess) e = hipEventCreate(&x);
  auto launch = [&](int r, hipEvent_t e0, hipEvent_t e1) {
    const u32x4p* p = (const u32x4p*)((const unsigned char*)buf + (size_t)(r % windows) * bytes);
    return nt ? launch_timed(stream_read_kernel<true>, dim3(grid), dim3(PRB_T), 0, s, e0, e1, p,
                             n16, sink)
              : launch_timed(stream_read_kernel<false>, dim3(grid), dim3(PRB_T), 0, s, e0, e1,
                             p, n16, sink);
  };
  if (e == hipSuccess) e = launch(reps, nullptr, nullptr);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch(r, ev[2 * r], ev[2 * r + 1]);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum = 0.0;
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
    sum += ms;
  }
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  if (e == hipSuccess) *avg_us = sum * 1e3 / reps;
  return e;
}

hipError_t probe_copy(const void* src, void* dst, size_t bytes, int reps, hipStream_t s,
                      double* avg_us) {
  const long long n16 = (long long)(bytes / 16);
  const int grid = (int)((n16 + PRB_T * 8 - 1) / (PRB_T * 8));
  std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
  hipError_t e = hipSuccess;
  for (auto& x : ev)
    if (e == hipSuccess) e = hipEventCreate(&x);
  for (int r = 0; r < reps && e == hipSuccess; ++r)
    e = launch_timed(stream_copy_kernel, dim3(grid), dim3(PRB_T), 0, s, ev[2 * r], ev[2 * r + 1],
                     (const u32x4p*)src, (u32x4p*)dst, n16);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum = 0.0;
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
    sum += ms;
  }
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  if (e == hipSuccess) *avg_us = sum * 1e3 / reps;
  return e;
}

hipError_t probe_empty_launch(int grid, int reps, hipStream_t s, double* avg_us) {
  std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
  hipError_t e = hipSuccess;
  for (auto& x : ev)
    if (e == hipSuccess) e = hipEventCreate(&x);
  if (e == hipSuccess)
    e = launch_timed(empty_kernel, dim3(grid), dim3(PRB_T), 0, s, nullptr, nullptr);
  for (int r = 0; r < reps && e == hipSuccess; ++r)
    e = launch_timed(empty_kernel, dim3(grid), dim3(PRB_T), 0, s, ev[2 * r], ev[2 * r + 1]);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum = 0.0;
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
    sum += ms;
  }
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  if (e == hipSuccess) *avg_us = sum * 1e3 / reps;
  return e;
}

}  // namespace moe
