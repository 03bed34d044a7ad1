// In-place CPU expert FFN (hybrid decode), AVX-512 BF16 when the host has it.
// Memory-bound like the GPU GEMV: every weight byte is read once per step for all of the
// expert's tokens; rows of I are split across the team so each member streams contiguous
// gate/up rows and the matching rows of WdT.
#include "cpu_expert.h"

#include <immintrin.h>

#include <chrono>
#include <cmath>
#include <cstring>

namespace moe {

CpuTeam::CpuTeam(int n) : n_(n < 1 ? 1 : n) {
  for (int k = 1; k < n_; ++k) th_.emplace_back([this, k] { member(k); });
}

CpuTeam::~CpuTeam() {
  stop_.store(true, std::memory_order_release);
  gen_.fetch_add(1, std::memory_order_acq_rel);
  for (auto& t : th_) t.join();
}

void CpuTeam::member(int k) {
  uint64_t seen = 0;
  unsigned spins = 0;
  auto idle_since = std::chrono::steady_clock::now();
  for (;;) {
    const uint64_t g = gen_.load(std::memory_order_acquire);
    if (g == seen) {
      // spin while jobs arrive; yield now and then; after 50 ms without a job, nap 50 us
      if (++spins & 1023u) {
        _mm_pause();
      } else if (std::chrono::steady_clock::now() - idle_since > std::chrono::milliseconds(50)) {
        std::this_thread::sleep_for(std::chrono::microseconds(50));
      } else {
        std::this_thread::yield();
      }
      continue;
    }
    idle_since = std::chrono::steady_clock::now();
    spins = 0;
    seen = g;
    if (stop_.load(std::memory_order_acquire)) return;
    (*job_)(k);
    left_.fetch_sub(1, std::memory_order_acq_rel);
  }
}

void CpuTeam::run(const std::function<void(int)>& job) {
  job_ = &job;
  left_.store(n_ - 1, std::memory_order_release);
  gen_.fetch_add(1, std::memory_order_acq_rel);
  job(0);
  // spin for the members; yield now and then so a member that lost its core (more runnable
  // threads than cores) gets it back instead of waiting out a scheduler slice
  unsigned spins = 0;
  while (left_.load(std::memory_order_acquire) != 0) {
    if (++spins & 1023u)
      _mm_pause();
    else
      std::this_thread::yield();
  }
}

static inline float bf16f(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---- dot products of one bf16 row with NT token rows ----
__attribute__((target("avx512f,avx512bf16,avx512bw,avx512vl"))) static void dots_avx512(
    const uint16_t* w, const uint16_t* const* xs, int nt, int H, float* out) {
  __m512 acc[8];
  for (int t = 0; t < nt; ++t) acc[t] = _mm512_setzero_ps();
  for (int h = 0; h < H; h += 32) {
    const __m512bh wv = (__m512bh)_mm512_loadu_si512(w + h);
    for (int t = 0; t < nt; ++t)
      acc[t] = _mm512_dpbf16_ps(acc[t], wv, (__m512bh)_mm512_loadu_si512(xs[t] + h));
  }
  for (int t = 0; t < nt; ++t) out[t] = _mm512_reduce_add_ps(acc[t]);
}

static void dots_scalar(const uint16_t* w, const uint16_t* const* xs, int nt, int H, float* out) {
  for (int t = 0; t < nt; ++t) {
    float s = 0.f;
    for (int h = 0; h < H; ++h) s += bf16f(w[h]) * bf16f(xs[t][h]);
    out[t] = s;
  }
}

// y_t[:] += a_t * row[:] for NT tokens (row bf16, y fp32)
__attribute__((target("avx512f,avx512bw,avx512vl"))) static void axpy_avx512(
    const uint16_t* row, const float* a, float* const* ys, int nt, int H) {
  for (int h = 0; h < H; h += 16) {
    const __m512 r = _mm512_castsi512_ps(
        _mm512_slli_epi32(_mm512_cvtepu16_epi32(_mm256_loadu_si256((const __m256i*)(row + h))), 16));
    for (int t = 0; t < nt; ++t)
      _mm512_storeu_ps(ys[t] + h, _mm512_fmadd_ps(_mm512_set1_ps(a[t]), r, _mm512_loadu_ps(ys[t] + h)));
  }
}

static void axpy_scalar(const uint16_t* row, const float* a, float* const* ys, int nt, int H) {
  for (int t = 0; t < nt; ++t)
    for (int h = 0; h < H; ++h) ys[t][h] += a[t] * bf16f(row[h]);
}

static bool host_has_avx512bf16() {
  static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                         __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512bf16");
  return ok;
}

void cpu_experts_ffn(CpuTeam& team, const uint16_t* const* blobs, int nexp, const int* row0,
                     const int* ntok, const int* row_tok, const float* row_w, int H, int I,
                     const uint16_t* x, int T, float* y, float* partial) {
  const int n = team.size();
  const bool fast = host_has_avx512bf16() && H % 32 == 0;
  team.run([&](int k) {
    // rows [i0, i1) of every expert: gate/up dots, SwiGLU, then the same rows of WdT into
    // this member's partial
    const int i0 = (int)((long long)I * k / n), i1 = (int)((long long)I * (k + 1) / n);
    float* part = partial + (size_t)k * T * H;
    std::memset(part, 0, sizeof(float) * (size_t)T * H);
    for (int e = 0; e < nexp; ++e) {
      const uint16_t* blob = blobs[e];
      const uint16_t* wdt = blob + (size_t)2 * I * H;
      for (int b = 0; b < ntok[e]; b += 8) {
        const int nt = ntok[e] - b < 8 ? ntok[e] - b : 8;
        const uint16_t* xs[8];
        float* ys[8];
        float w[8];
        for (int j = 0; j < nt; ++j) {
          const int r = row0[e] + b + j;
          xs[j] = x + (size_t)row_tok[r] * H;
          ys[j] = part + (size_t)row_tok[r] * H;
          w[j] = row_w[r];
        }
        for (int i = i0; i < i1; ++i) {
          float g[8], u[8], a[8];
          const uint16_t* gr = blob + (size_t)i * 2 * H;
          if (fast) {
            dots_avx512(gr, xs, nt, H, g);
            dots_avx512(gr + H, xs, nt, H, u);
          } else {
            dots_scalar(gr, xs, nt, H, g);
            dots_scalar(gr + H, xs, nt, H, u);
          }
          for (int j = 0; j < nt; ++j) a[j] = g[j] / (1.0f + std::exp(-g[j])) * u[j] * w[j];
          if (fast)
            axpy_avx512(wdt + (size_t)i * H, a, ys, nt, H);
          else
            axpy_scalar(wdt + (size_t)i * H, a, ys, nt, H);
        }
      }
    }
  });
  // y += partials in member order; columns split across the team
  team.run([&](int k) {
    const int c0 = (int)((long long)H * k / n), c1 = (int)((long long)H * (k + 1) / n);
    for (int t = 0; t < T; ++t) {
      float* yt = y + (size_t)t * H;
      for (int m = 0; m < n; ++m) {
        const float* p = partial + ((size_t)m * T + t) * H;
        for (int c = c0; c < c1; ++c) yt[c] += p[c];
      }
    }
  });
}

}  // namespace moe
