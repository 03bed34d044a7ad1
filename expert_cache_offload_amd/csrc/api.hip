// Host side of the C ABI declared in include/moe_offload.h: argument checks, workspace
// layout, step orchestration across the compute and fill streams, resize and snapshots.
#include <hip/hip_runtime.h>
#include <immintrin.h>

#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "../../include/moe_offload.h"
#include "cpu_expert.h"
#include "moe_dev.h"
#include "plan_core.h"

namespace moe {
hipError_t launch_route_plan(const Dims& d, const Dev& v, const void* x, const void* wr,
                             int* out_idx, float* out_w, int layer, int T, int split_bc,
                             int split_bp, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
size_t route_plan_lds_bytes(const Dims& d);
hipError_t launch_ffn_decode(const Dims& d, const Dev& v, const void* x, const void* arena,
                             const void* shared_blob, void* y, int sel, int group, int ngroups,
                             int T, int max_entries, int with_combine, int stage,
                             hipStream_t s, hipEvent_t e0, hipEvent_t e1);
int decode_ntok(int T);
int down_columns_per_block(int fmt);
int down_row_splits(int inter);
int fused_row_blocks(const Dims& d);
hipError_t launch_fill(const Dev& v, const void* pool_dev, void* arena, long long S, int group,
                       int ngroups, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                       int prefetch, int E);
hipError_t launch_init(const Dev& v, int max_capacity, int n_keys, int capacity, hipStream_t s);
hipError_t launch_resize(const Dev& v, int new_capacity, int max_capacity, int E,
                         const void* old_arena, void* new_arena, long long S, hipStream_t s);
size_t resize_lds_bytes(int max_capacity);
hipError_t launch_route_prefill(const Dims& d, const Dev& v, const void* x, const void* wr,
                                int* out_idx, float* out_w, int layer, int T, hipStream_t s,
                                hipEvent_t e0, hipEvent_t e1);
bool prefill_route_supported(const Dims& d);
hipError_t launch_ffn_prefill(const Dims& d, const Dev& v, const void* x, const void* arena,
                              const void* shared_blob, void* y, int sel, int group, int ngroups,
                              int T, int stage, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
bool prefill_ffn_supported(const Dims& d);
hipError_t launch_prefetch_plan(const Dims& d, const Dev& v, int layer, hipStream_t s);
hipError_t probe_stream_read(const void* buf, size_t span, size_t bytes, int nt, int reps,
                             uint32_t* sink, hipStream_t s, double* avg_us);
hipError_t probe_empty_launch(int grid, int reps, hipStream_t s, double* avg_us);
hipError_t probe_copy(const void* src, void* dst, size_t bytes, int reps, hipStream_t s,
                      double* avg_us);
}  // namespace moe

using namespace moe;

namespace {

constexpr int kMaxGroups = kMaxFillGroups;
// CPU expert rate over offload rate at which a format switches to hybrid decode ("FreeToken:
// az VRAM ile büyük MoE modelleri", "Tuzaklar": the start-up probe's 2.0x threshold).
constexpr double kHybridThreshold = 2.0;
constexpr int kMaxCapacity = kMaxSlots;  // LDS-resident LRU stamps and the resize sort
// Fill workgroups: 32 saturate the PCIe link (57 GB/s measured) while leaving HBM streaming
// of concurrent kernels untouched; 256 workgroups collapse a concurrent HBM stream to <2%.
constexpr int kFillGrid = 32;

enum class State { Idle, Planned, Filled };

struct Layout {
  size_t key_of, stamp, slot_of, ctrl, stats, hdr, U, u_slot, u_hit, hit_list, miss_list,
      miss_key, miss_slot, miss_victim, count, offset, perm, inv_pos, tk_idx, tk_w, logits,
      act, act_shared, yexp, yexp_shared, yfus, ent, row_tok, row_w, moves, blk_cnt, blk_off, brank,
      pact, pact_shared, pyexp, pyexp_shared, pf_hdr, pf_list, pf_ent, row_cpu, cpu_key, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }


Dims make_dims(const moe_shape& s, int max_capacity) {
  Dims d{};
  d.L = s.layers;
  d.E = s.experts;
  d.K = s.top_k;
  d.H = s.hidden;
  d.I = s.inter;
  d.fmt = s.wfmt;
  d.has_shared = s.has_shared;
  d.max_tokens = s.max_tokens;
  d.amax = s.max_tokens * s.top_k;
  d.umax = d.amax < s.experts ? d.amax : s.experts;
  d.pw = s.max_tokens > kDecodeMaxTokens ? s.experts : d.umax;
  d.tdec = s.max_tokens < kDecodeMaxTokens ? s.max_tokens : kDecodeMaxTokens;
  d.adec = d.tdec * s.top_k;
  d.nblk = s.max_tokens > kDecodeMaxTokens ? (s.max_tokens + 63) / 64 : 0;
  d.max_capacity = max_capacity;
  d.RS = down_row_splits(s.inter);
  d.S = s.blob_bytes;
  d.RSF = fused_row_blocks(d);
  return d;
}

Layout make_layout(const Dims& d) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t I4 = sizeof(int32_t);
  L.key_of = take(I4 * d.max_capacity);
  L.stamp = take(sizeof(int64_t) * d.max_capacity);
  L.slot_of = take(I4 * (size_t)d.L * d.E);
  L.ctrl = take(I4 * CTRL_WORDS);
  L.stats = take(sizeof(uint64_t) * STAT_WORDS);
  L.hdr = take(I4 * HDR_WORDS);
  L.U = take(I4 * d.umax);
  L.u_slot = take(I4 * d.umax);
  L.u_hit = take(I4 * d.umax);
  L.hit_list = take(I4 * d.umax);
  L.miss_list = take(I4 * d.umax);
  L.miss_key = take(I4 * d.umax);
  L.miss_slot = take(I4 * d.umax);
  L.miss_victim = take(I4 * d.umax);
  L.count = take(I4 * d.umax);
  L.offset = take(I4 * (d.umax + 1));
  L.perm = take(I4 * d.amax);
  L.inv_pos = take(I4 * d.amax);
  L.tk_idx = take(I4 * d.amax);
  L.tk_w = take(sizeof(float) * d.amax);
  L.logits = take(sizeof(double) * (size_t)d.tdec * d.E);
  L.act = take(sizeof(float) * (size_t)d.adec * d.I);
  L.act_shared = take(d.has_shared ? sizeof(float) * (size_t)d.tdec * d.I : 256);
  L.yexp = take(sizeof(float) * (size_t)d.adec * d.RS * d.H);
  L.yexp_shared = take(d.has_shared ? sizeof(float) * (size_t)d.tdec * d.RS * d.H : 256);
  L.yfus = take(d.RSF > 0 ? sizeof(float) * (size_t)d.K * d.RSF * d.H : 256);
  L.ent = take(sizeof(int) * 4 * (size_t)d.umax);
  L.row_tok = take(I4 * d.amax);
  L.row_w = take(sizeof(float) * d.amax);
  L.moves = take(I4 * 2 * (size_t)d.max_capacity);
  const bool many = d.nblk > 0;  // buffers of steps with more than eight tokens
  const size_t T = many ? (size_t)d.max_tokens : 0, A = many ? (size_t)d.amax : 0;
  L.blk_cnt = take(I4 * (size_t)d.nblk * d.E);
  L.blk_off = take(I4 * (size_t)d.nblk * d.E);
  L.brank = take(I4 * A);
  L.pact = take(sizeof(uint16_t) * A * d.I);
  L.pact_shared = take(d.has_shared ? sizeof(uint16_t) * T * d.I : 0);
  L.pyexp = take(sizeof(float) * A * d.H);
  L.pyexp_shared = take(d.has_shared ? sizeof(float) * T * d.H : 0);
  L.pf_hdr = take(I4 * HDR_WORDS);
  L.pf_list = take(I4 * (size_t)(11 * d.E + 1));
  L.pf_ent = take(sizeof(int) * 4 * (size_t)d.E);
  L.row_cpu = take(I4 * (size_t)d.adec);
  L.cpu_key = take(I4 * (size_t)d.umax);
  L.total = o;
  return L;
}

Dev make_dev(void* ws, const Layout& L) {
  char* b = (char*)ws;
  Dev v{};
  v.key_of = (int*)(b + L.key_of);
  v.stamp = (long long*)(b + L.stamp);
  v.slot_of = (int*)(b + L.slot_of);
  v.ctrl = (int*)(b + L.ctrl);
  v.stats = (unsigned long long*)(b + L.stats);
  v.hdr = (int*)(b + L.hdr);
  v.U = (int*)(b + L.U);
  v.u_slot = (int*)(b + L.u_slot);
  v.u_hit = (int*)(b + L.u_hit);
  v.hit_list = (int*)(b + L.hit_list);
  v.miss_list = (int*)(b + L.miss_list);
  v.miss_key = (int*)(b + L.miss_key);
  v.miss_slot = (int*)(b + L.miss_slot);
  v.miss_victim = (int*)(b + L.miss_victim);
  v.count = (int*)(b + L.count);
  v.offset = (int*)(b + L.offset);
  v.perm = (int*)(b + L.perm);
  v.inv_pos = (int*)(b + L.inv_pos);
  v.tk_idx = (int*)(b + L.tk_idx);
  v.tk_w = (float*)(b + L.tk_w);
  v.logits = (double*)(b + L.logits);
  v.act = (float*)(b + L.act);
  v.act_shared = (float*)(b + L.act_shared);
  v.yexp = (float*)(b + L.yexp);
  v.yexp_shared = (float*)(b + L.yexp_shared);
  v.yfus = (float*)(b + L.yfus);
  v.ent = (int4*)(b + L.ent);
  v.row_tok = (int*)(b + L.row_tok);
  v.row_w = (float*)(b + L.row_w);
  v.moves = (int*)(b + L.moves);
  v.blk_cnt = (int*)(b + L.blk_cnt);
  v.blk_off = (int*)(b + L.blk_off);
  v.brank = (int*)(b + L.brank);
  v.pact = (uint16_t*)(b + L.pact);
  v.pact_shared = (uint16_t*)(b + L.pact_shared);
  v.pyexp = (float*)(b + L.pyexp);
  v.pyexp_shared = (float*)(b + L.pyexp_shared);
  v.pf_hdr = (int*)(b + L.pf_hdr);
  v.pf_list = (int*)(b + L.pf_list);
  v.pf_ent = (int4*)(b + L.pf_ent);
  v.row_cpu = (int*)(b + L.row_cpu);
  v.cpu_key = (int*)(b + L.cpu_key);
  v.mail = nullptr;
  v.hyb_timeout_ticks = 200000000;  // 2 s
  return v;
}

bool shape_ok(const moe_shape* s) {
  if (!s) return false;
  if (s->layers < 1 || s->experts < 1 || s->experts > 1024) return false;
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > s->experts) return false;
  if (s->hidden < 256 || s->hidden % 256) return false;
  if (s->inter < 128 || s->inter % 128) return false;
  if (s->wfmt < 0 || s->wfmt > 2) return false;
  if (s->has_shared != 0 && s->has_shared != 1) return false;
  if (s->max_tokens < 1 || s->max_tokens > kMaxTokens) return false;
  if (s->blob_bytes != moe_blob_bytes(s->wfmt, s->hidden, s->inter)) return false;
  if (s->blob_bytes % 16) return false;
  if ((long long)s->layers * s->experts > (1ll << 30)) return false;
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Smallest capacity of a prefetching handle: a step's distinct keys plus a whole layer.
int prefetch_capacity_floor(const Dims& d) { return d.umax + d.E; }

}  // namespace

// Timing of the library's own launches with event pairs from a reusable ring; the events
// are handed to the kernel dispatch (start and end of the kernel, no marker packets).
struct Profiler {
  enum Kind { ROUTE = 0, FILL = 1, GATE_UP = 2, DOWN = 3, NKIND = 4 };
  static constexpr int kRing = 4096;
  int mask = 0;    // bit k: time launches of kind k
  int every = 1;   // time one launch in `every` of each selected kind
  int64_t seen[4] = {};
  std::vector<hipEvent_t> a, b;
  std::vector<int> kind;
  size_t head = 0, pending = 0;
  double ms[NKIND] = {};
  int64_t launches[NKIND] = {};
  unsigned long long stats0[STAT_WORDS] = {};

  hipError_t ensure() {
    if (!a.empty()) return hipSuccess;
    a.resize(kRing);
    b.resize(kRing);
    kind.resize(kRing);
    for (int i = 0; i < kRing; ++i) {
      hipError_t e = hipEventCreate(&a[i]);
      if (e == hipSuccess) e = hipEventCreate(&b[i]);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  hipError_t harvest_one() {
    const size_t i = (head + kRing - pending) % kRing;
    hipError_t e = hipEventSynchronize(b[i]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, a[i], b[i]);
    if (e != hipSuccess) return e;
    ms[kind[i]] += t;
    launches[kind[i]] += 1;
    --pending;
    return hipSuccess;
  }
  hipError_t harvest_all() {
    while (pending) {
      hipError_t e = harvest_one();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  template <class F>
  hipError_t timed(int k, hipStream_t s, F launch) {
    if (!(mask >> k & 1)) return launch(nullptr, nullptr);
    if (seen[k]++ % every != 0) return launch(nullptr, nullptr);
    if (pending == (size_t)kRing) {
      hipError_t e = harvest_one();
      if (e != hipSuccess) return e;
    }
    const size_t i = head;
    hipError_t e = launch(a[i], b[i]);  // the kernel dispatch itself takes both timestamps
    if (e != hipSuccess) return e;
    kind[i] = k;
    head = (head + 1) % kRing;
    ++pending;
    return hipSuccess;
  }
  void reset() {
    for (int k = 0; k < NKIND; ++k) {
      ms[k] = 0;
      launches[k] = 0;
      seen[k] = 0;
    }
  }
  void destroy() {
    for (auto e : a) (void)hipEventDestroy(e);
    for (auto e : b) (void)hipEventDestroy(e);
    a.clear();
    b.clear();
  }
};

// Host side of hybrid decode: a server thread polls the mailbox that the route kernel posts
// to, computes the step's CPU experts with its thread team straight from the host pool, and
// answers with the step value.  The GPU combine waits for the answer.
struct HybridServer {
  HybMail* mail = nullptr;   // host view (pinned, coherent)
  void* mail_dev = nullptr;  // device view
  const unsigned char* pool = nullptr;
  Dims d{};
  int threads = 1;
  std::thread th;
  std::atomic<bool> stop{false};
  std::atomic<bool> hold{false};      // leave requests unanswered (failure-path tests)
  std::atomic<long long> served{0};   // requests answered
  std::atomic<long long> experts{0};  // CPU experts computed
  std::atomic<long long> busy_ns{0};  // time spent computing them

  void serve(CpuTeam& team, std::vector<float>& partial) {
    HybMail* m = mail;
    const int T = m->T, q = m->q, layer = m->layer, H = d.H;
    float* y = (float*)((unsigned char*)m + mail_y_offset(H));
    const uint16_t* x = (const uint16_t*)((const unsigned char*)m + mail_x_offset());
    std::memset(y, 0, sizeof(float) * (size_t)T * H);
    const uint16_t* blobs[kMailRows];
    for (int j = 0; j < q; ++j)
      blobs[j] = (const uint16_t*)(pool + ((size_t)layer * d.E + m->exp[j]) * (size_t)d.S);
    cpu_experts_ffn(team, blobs, q, m->row0, m->ntok, m->row_tok, m->row_w, H, d.I, x, T, y,
                    partial.data());
  }
  void loop() {
    // the mailbox starts with req = -1; a request may already be posted by the time this
    // thread runs, so `last` is that initial value, never a fresh read
    long long last = -1;
    CpuTeam team(threads);
    std::vector<float> partial((size_t)threads * kDecodeMaxTokens * d.H);
    unsigned spins = 0;
    auto idle_since = std::chrono::steady_clock::now();
    while (!stop.load(std::memory_order_acquire)) {
      const long long r = __atomic_load_n(&mail->req, __ATOMIC_ACQUIRE);
      if (r == last || hold.load(std::memory_order_acquire)) {
        // poll hot while steps arrive; after 50 ms without one, every 50 us
        if (++spins < 4096) {
          _mm_pause();
          continue;
        }
        spins = 0;
        if (std::chrono::steady_clock::now() - idle_since > std::chrono::milliseconds(50))
          std::this_thread::sleep_for(std::chrono::microseconds(50));
        else
          std::this_thread::yield();
        continue;
      }
      const auto t0 = std::chrono::steady_clock::now();
      const int q = mail->q;
      serve(team, partial);
      last = r;
      __atomic_store_n(&mail->done, r, __ATOMIC_RELEASE);
      busy_ns.fetch_add(std::chrono::duration_cast<std::chrono::nanoseconds>(
                            std::chrono::steady_clock::now() - t0).count(),
                        std::memory_order_relaxed);
      experts.fetch_add(q, std::memory_order_relaxed);
      served.fetch_add(1, std::memory_order_relaxed);
      idle_since = std::chrono::steady_clock::now();
    }
  }
};

struct moe_cache_s {
  Profiler prof;
  HybridServer* hyb = nullptr;  // hybrid decode server, or null
  int split_bc = 0, split_bp = 0;
  moe_shape shape;
  Dims d;
  Layout L;
  Dev v;
  int capacity;
  int max_capacity;
  int arena_slots;  // slots the current arena holds
  void* arena;
  void* workspace;
  const void* host_pool;
  const void* pool_dev;
  int static_dev = -1;  // device whose static workspace this handle holds, or -1
  bool events = false;  // the events below exist (created on first multi-queue use)
  hipEvent_t ev_plan;
  hipEvent_t ev_fill[kMaxGroups];
  int prefetch;                    // prefetch the next layer in steps of many tokens
  int pf_layer[2] = {-1, -1};      // layer whose prefetch is in flight, by layer parity
  hipEvent_t ev_pfplan;
  hipEvent_t ev_pf[2];
  State state;
  int plan_T;
  int plan_layer;
  int fill_groups;
  int last_hip;
};

// The library's own workspace, for callers that cannot allocate device memory
// (moe_cache_create_static): one array per device, taken by at most one live handle at a
// time.  Host code never uses the array's name as an address: each device's address comes
// from hipGetSymbolAddress, asked once per device with that device current.
constexpr size_t kStaticWorkspaceBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_static_mu;
static void* g_static_ptr[kMaxDevices];  // device address of `scratch` on each device
static bool g_static_busy[kMaxDevices];  // a live handle holds that device's array

static moe_status static_workspace_acquire(int* dev_out, void** ptr_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOE_E_HIP;
  }
  std::lock_guard<std::mutex> g(g_static_mu);
  if (g_static_busy[dev]) return MOE_E_BUSY;
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_E_HIP;
    }
    g_static_ptr[dev] = p;
  }
  g_static_busy[dev] = true;
  *dev_out = dev;
  *ptr_out = g_static_ptr[dev];
  return MOE_OK;
}

static void static_workspace_release(int dev) {
  std::lock_guard<std::mutex> g(g_static_mu);
  g_static_busy[dev] = false;
}

static moe_status hip_fail(moe_cache c, hipError_t e) {
  if (c) c->last_hip = (int)e;
  return MOE_E_HIP;
}

extern "C" {

int64_t moe_blob_bytes(int32_t wfmt, int32_t hidden, int32_t inter) {
  const int64_t H = hidden, I = inter;
  if (H <= 0 || I <= 0) return -1;
  switch (wfmt) {
    case MOE_FMT_BF16: return 6 * I * H;
    case MOE_FMT_FP8_E4M3_K128:
      if (H % 128 || I % 128) return -1;
      return 3 * I * H + 4 * (2 * I * (H / 128)) + 4 * ((I / 128) * H);
    case MOE_FMT_MXFP4_K32:
      if (H % 64 || I % 32) return -1;
      return 3 * I * H / 2 + 2 * I * (H / 32) + (I / 32) * H;
    default: return -1;
  }
}

size_t moe_workspace_bytes(const moe_shape* shape, int32_t max_capacity) {
  if (!shape_ok(shape) || max_capacity < 1 || max_capacity > kMaxCapacity) return 0;
  return make_layout(make_dims(*shape, max_capacity)).total;
}

moe_status moe_auto_capacity(const moe_shape* shape, uint64_t free_bytes, uint64_t reserve_bytes,
                             double offload_ratio, int32_t* capacity) {
  if (!shape_ok(shape) || !capacity) return MOE_E_INVALID;
  if (offload_ratio >= 1.0) return MOE_E_INVALID;
  const int64_t n_keys = (int64_t)shape->layers * shape->experts;
  const int floor_c = shape->max_tokens * shape->top_k < shape->experts
                          ? shape->max_tokens * shape->top_k
                          : shape->experts;
  int64_t top = n_keys < kMaxCapacity ? n_keys : kMaxCapacity;
  if (offload_ratio >= 0.0) {
    const int64_t keep = (int64_t)((1.0 - offload_ratio) * (double)n_keys);
    top = keep < top ? keep : top;
  }
  if (free_bytes <= reserve_bytes) return MOE_E_CAPACITY;
  const uint64_t budget = free_bytes - reserve_bytes;
  // slots C and the workspace of a handle sized for C must fit the budget; the workspace
  // grows with C, so the admissible C form a prefix: bisect it
  auto fits = [&](int64_t c) {
    const size_t ws = make_layout(make_dims(*shape, (int)c)).total;
    return (uint64_t)c * (uint64_t)shape->blob_bytes + ws <= budget;
  };
  if (top < floor_c || !fits(floor_c)) return MOE_E_CAPACITY;
  int64_t lo = floor_c, hi = top;  // fits(lo), answer in [lo, hi]
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (fits(mid))
      lo = mid;
    else
      hi = mid - 1;
  }
  *capacity = (int32_t)lo;
  return MOE_OK;
}

moe_status moe_auto_capacity_device(const moe_shape* shape, uint64_t reserve_bytes,
                                    double offload_ratio, int32_t* capacity,
                                    uint64_t* free_bytes) {
  if (!shape_ok(shape) || !capacity) return MOE_E_INVALID;
  size_t fr = 0, total = 0;
  if (hipMemGetInfo(&fr, &total) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_HIP;
  }
  if (free_bytes) *free_bytes = (uint64_t)fr;
  return moe_auto_capacity(shape, (uint64_t)fr, reserve_bytes, offload_ratio, capacity);
}

moe_status moe_host_pool_alloc(size_t bytes, void** out) {
  if (!out || bytes == 0) return MOE_E_INVALID;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocNonCoherent);
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    *out = nullptr;
    return MOE_E_NOMEM;
  }
  *out = p;
  return MOE_OK;
}

moe_status moe_host_pool_free(void* p) {
  if (!p) return MOE_E_INVALID;
  return hipHostFree(p) == hipSuccess ? MOE_OK : MOE_E_HIP;
}

// Events joining the compute and fill queues (and the prefetch); created on first use, so a
// handle driven on one queue (moe_layer_step with groups == 0, no prefetch) creates none.
static hipError_t ensure_events(moe_cache c) {
  if (c->events) return hipSuccess;
  hipError_t e = hipEventCreateWithFlags(&c->ev_plan, hipEventDisableTiming);
  for (int g = 0; g < kMaxGroups && e == hipSuccess; ++g)
    e = hipEventCreateWithFlags(&c->ev_fill[g], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_pfplan, hipEventDisableTiming);
  for (int q = 0; q < 2 && e == hipSuccess; ++q)
    e = hipEventCreateWithFlags(&c->ev_pf[q], hipEventDisableTiming);
  c->events = true;  // (partially) created: destroy releases whatever exists
  return e;
}

static moe_status create_impl(const moe_shape* shape, int32_t capacity, int32_t max_capacity,
                              void* slot_arena, void* workspace, const void* host_pool,
                              void* stream, moe_cache* out) {
  if (!out) return MOE_E_INVALID;
  *out = nullptr;
  if (!shape_ok(shape) || !slot_arena || !workspace || !host_pool) return MOE_E_INVALID;
  if (!aligned16(slot_arena) || ((uintptr_t)workspace & 255)) return MOE_E_INVALID;
  if (max_capacity < 1 || max_capacity > kMaxCapacity) return MOE_E_CAPACITY;
  const int floor_c = shape->max_tokens * shape->top_k < shape->experts
                          ? shape->max_tokens * shape->top_k
                          : shape->experts;
  if (capacity < floor_c || capacity > max_capacity) return MOE_E_CAPACITY;
  void* pool_dev = nullptr;
  if (hipHostGetDevicePointer(&pool_dev, const_cast<void*>(host_pool), 0) != hipSuccess ||
      !pool_dev) {
    (void)hipGetLastError();
    return MOE_E_NOMEM;  // not pinned / not device-accessible
  }
  moe_cache c = new (std::nothrow) moe_cache_s();
  if (!c) return MOE_E_NOMEM;
  c->shape = *shape;
  c->d = make_dims(*shape, max_capacity);
  c->L = make_layout(c->d);
  c->v = make_dev(workspace, c->L);
  c->capacity = capacity;
  c->max_capacity = max_capacity;
  c->arena_slots = max_capacity;
  c->arena = slot_arena;
  c->workspace = workspace;
  c->host_pool = host_pool;
  c->pool_dev = pool_dev;
  c->state = State::Idle;
  hipError_t e = launch_init(c->v, max_capacity, shape->layers * shape->experts, capacity,
                             (hipStream_t)stream);
  if (e != hipSuccess) {
    moe_cache_destroy(c);
    return MOE_E_HIP;
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_cache_create(const moe_shape* shape, int32_t capacity, int32_t max_capacity,
                            void* slot_arena, void* workspace, const void* host_pool,
                            void* stream, moe_cache* out) {
  return create_impl(shape, capacity, max_capacity, slot_arena, workspace, host_pool, stream,
                     out);
}

moe_status moe_cache_create_static(const moe_shape* shape, int32_t capacity,
                                   int32_t max_capacity, void* slot_arena,
                                   const void* host_pool, void* stream, moe_cache* out) {
  if (!out) return MOE_E_INVALID;
  *out = nullptr;
  if (!shape_ok(shape)) return MOE_E_INVALID;
  if (max_capacity < 1 || max_capacity > kMaxCapacity) return MOE_E_CAPACITY;
  if (moe_workspace_bytes(shape, max_capacity) > kStaticWorkspaceBytes) return MOE_E_SCRATCH;
  int dev = -1;
  void* ws = nullptr;
  moe_status st = static_workspace_acquire(&dev, &ws);
  if (st != MOE_OK) return st;
  st = create_impl(shape, capacity, max_capacity, slot_arena, ws, host_pool, stream, out);
  if (st != MOE_OK) {
    static_workspace_release(dev);
    return st;
  }
  (*out)->static_dev = dev;
  return MOE_OK;
}

static void hybrid_stop(moe_cache c) {
  if (!c->hyb) return;
  (void)hipDeviceSynchronize();  // no combine may still be waiting for the server
  c->hyb->stop.store(true, std::memory_order_release);
  if (c->hyb->th.joinable()) c->hyb->th.join();
  if (c->hyb->mail) (void)hipHostFree(c->hyb->mail);
  delete c->hyb;
  c->hyb = nullptr;
  c->v.mail = nullptr;
  c->split_bc = c->split_bp = 0;
}

moe_status moe_cache_destroy(moe_cache c) {
  if (!c) return MOE_E_INVALID;
  hybrid_stop(c);
  (void)c->prof.harvest_all();
  c->prof.destroy();
  if (c->events) {
    if (c->ev_plan) (void)hipEventDestroy(c->ev_plan);
    for (int g = 0; g < kMaxGroups; ++g)
      if (c->ev_fill[g]) (void)hipEventDestroy(c->ev_fill[g]);
    if (c->ev_pfplan) (void)hipEventDestroy(c->ev_pfplan);
    for (int q = 0; q < 2; ++q)
      if (c->ev_pf[q]) (void)hipEventDestroy(c->ev_pf[q]);
  }
  if (c->static_dev >= 0) static_workspace_release(c->static_dev);
  delete c;
  return MOE_OK;
}

moe_status moe_cache_resize(moe_cache c, int32_t new_capacity, void* new_arena, void* stream) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_BUSY;
  if (c->pf_layer[0] >= 0 || c->pf_layer[1] >= 0) return MOE_E_BUSY;  // prefetch in flight
  const int floor_c = c->prefetch ? prefetch_capacity_floor(c->d) : c->d.umax;
  if (new_capacity < floor_c || new_capacity > c->max_capacity) return MOE_E_CAPACITY;
  if (new_arena && !aligned16(new_arena)) return MOE_E_INVALID;
  if (!new_arena && new_capacity > c->arena_slots) return MOE_E_CAPACITY;
  hipError_t e = launch_resize(c->v, new_capacity, c->max_capacity, c->d.E, c->arena, new_arena,
                               c->d.S, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(c, e);
  c->capacity = new_capacity;
  if (new_arena) {
    c->arena = new_arena;
    c->arena_slots = new_capacity;
  }
  return MOE_OK;
}

// Steps of more than eight tokens take the tiled router and the matrix-core FFN.
static bool many_tokens_ok(const Dims& d) {
  return d.nblk > 0 && prefill_route_supported(d) && prefill_ffn_supported(d);
}

static hipError_t route_launch(moe_cache c, int layer, const void* x, int T, const void* wr,
                               int* idx, float* w, hipStream_t s) {
  return c->prof.timed(Profiler::ROUTE, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (T > kDecodeMaxTokens)
      return launch_route_prefill(c->d, c->v, x, wr, idx, w, layer, T, s, e0, e1);
    const bool split = c->hyb != nullptr;
    return launch_route_plan(c->d, c->v, x, wr, idx, w, layer, T, split ? c->split_bc : 0,
                             split ? c->split_bp : 0, s, e0, e1);
  });
}

// One FFN launch group (gate/up, down, and the combine when with_combine) over the entries
// that sel / g / ngroups select.
static hipError_t ffn_launch(moe_cache c, const void* x, int T, const void* shared_blob, void* y,
                             int sel, int g, int ngroups, int max_entries, int with_combine,
                             hipStream_t s) {
  auto& P = c->prof;
  const bool many = T > kDecodeMaxTokens;
  hipError_t r = P.timed(Profiler::GATE_UP, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (many)
      return launch_ffn_prefill(c->d, c->v, x, c->arena, shared_blob, y, sel, g, ngroups, T, 0,
                                s, e0, e1);
    return launch_ffn_decode(c->d, c->v, x, c->arena, shared_blob, y, sel, g, ngroups, T,
                             max_entries, with_combine, 0, s, e0, e1);
  });
  if (r != hipSuccess) return r;
  return P.timed(Profiler::DOWN, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (many) {
      hipError_t q = launch_ffn_prefill(c->d, c->v, x, c->arena, shared_blob, y, sel, g, ngroups,
                                        T, 1, s, e0, with_combine ? nullptr : e1);
      if (q != hipSuccess || !with_combine) return q;
      return launch_ffn_prefill(c->d, c->v, x, c->arena, shared_blob, y, sel, g, ngroups, T, 2,
                                s, nullptr, e1);
    }
    return launch_ffn_decode(c->d, c->v, x, c->arena, shared_blob, y, sel, g, ngroups, T,
                             max_entries, with_combine, 1, s, e0, e1);
  });
}

// Prefetch of every expert of `layer` (steps of many tokens, prefetch mode): its plan on `cs`
// right after the step plan before it, its fills on `fs` (after the fills already queued
// there); the FFN of `layer` waits for them.
static hipError_t issue_prefetch(moe_cache c, int layer, hipStream_t cs, hipStream_t fs) {
  hipError_t e = ensure_events(c);
  if (e == hipSuccess) e = launch_prefetch_plan(c->d, c->v, layer, cs);
  if (e == hipSuccess && fs != cs) {
    e = hipEventRecord(c->ev_pfplan, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(fs, c->ev_pfplan, 0);
  }
  if (e == hipSuccess)
    e = c->prof.timed(Profiler::FILL, fs, [&](hipEvent_t e0, hipEvent_t e1) {
      return launch_fill(c->v, c->pool_dev, c->arena, c->d.S, 0, 1, kFillGrid, fs, e0, e1, 1,
                         c->d.E);
    });
  if (e == hipSuccess) e = hipEventRecord(c->ev_pf[layer & 1], fs);
  if (e == hipSuccess) c->pf_layer[layer & 1] = layer;
  return e;
}

static hipError_t wait_prefetch(moe_cache c, int layer, hipStream_t s) {
  if (c->pf_layer[layer & 1] != layer) return hipSuccess;
  c->pf_layer[layer & 1] = -1;
  return hipStreamWaitEvent(s, c->ev_pf[layer & 1], 0);
}

static bool prefetch_next(moe_cache c, int layer, int T) {
  return c->prefetch && T > kDecodeMaxTokens && layer + 1 < c->d.L;
}

moe_status moe_set_prefetch(moe_cache c, int32_t enable) {
  if (!c || (enable != 0 && enable != 1)) return MOE_E_INVALID;
  if (enable && c->d.nblk == 0) return MOE_E_INVALID;  // a handle for decode steps only
  if (c->state != State::Idle || c->pf_layer[0] >= 0 || c->pf_layer[1] >= 0) return MOE_E_BUSY;
  // a prefetch keeps the step's distinct keys (up to umax) and brings every expert of the
  // next layer: the cache must hold both, or the plan would run out of evictable slots
  if (enable && c->capacity < prefetch_capacity_floor(c->d)) return MOE_E_CAPACITY;
  c->prefetch = enable;
  return MOE_OK;
}

moe_status moe_set_hybrid(moe_cache c, int32_t b_cpu_mbps, int32_t b_pcie_mbps, int32_t threads) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_BUSY;
  if (b_cpu_mbps == 0) {
    hybrid_stop(c);
    return MOE_OK;
  }
  if (b_cpu_mbps < 0 || b_pcie_mbps < 0 || threads < 1 || threads > 256) return MOE_E_INVALID;
  if (c->d.fmt != FMT_BF16) return MOE_E_INVALID;  // the CPU path is bf16 only
  if (c->hyb && c->hyb->threads != threads) hybrid_stop(c);
  if (!c->hyb) {
    HybridServer* h = new (std::nothrow) HybridServer();
    if (!h) return MOE_E_NOMEM;
    void* p = nullptr;
    const size_t bytes = mail_bytes(c->d.H);
    if (hipHostMalloc(&p, bytes, hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess || !p) {
      (void)hipGetLastError();
      delete h;
      return MOE_E_NOMEM;
    }
    void* pd = nullptr;
    if (hipHostGetDevicePointer(&pd, p, 0) != hipSuccess || !pd) {
      (void)hipGetLastError();
      (void)hipHostFree(p);
      delete h;
      return MOE_E_NOMEM;
    }
    std::memset(p, 0, bytes);
    h->mail = (HybMail*)p;
    h->mail->req = -1;
    h->mail->done = -1;
    h->mail_dev = pd;
    h->pool = (const unsigned char*)c->host_pool;
    h->d = c->d;
    h->threads = threads;
    h->th = std::thread([h] { h->loop(); });
    c->hyb = h;
    c->v.mail = (HybMail*)pd;
  }
  c->split_bc = b_cpu_mbps;
  c->split_bp = b_pcie_mbps;
  return MOE_OK;
}

int32_t moe_choose_mode(int32_t wfmt, double cpu_gbps, double fill_gbps) {
  if (wfmt < MOE_FMT_BF16 || wfmt > MOE_FMT_MXFP4_K32) return -1;
  if (!(cpu_gbps >= 0.0) || !(fill_gbps >= 0.0)) return -1;  // negative or NaN
  if (wfmt != MOE_FMT_BF16) return 0;  // no CPU expert path for block-scaled formats
  return cpu_gbps > 0.0 && fill_gbps > 0.0 && cpu_gbps >= kHybridThreshold * fill_gbps ? 1 : 0;
}

moe_status moe_probe_stream_read(const void* buf, uint64_t span_bytes, uint64_t bytes_per_launch,
                                 int32_t nontemporal, int32_t reps, void* sink, void* stream,
                                 double* avg_us) {
  if (!buf || !sink || !avg_us || reps < 1 || reps > 100000) return MOE_E_INVALID;
  if (!aligned16(buf) || ((uintptr_t)sink & 3)) return MOE_E_INVALID;
  if (bytes_per_launch < 16 || bytes_per_launch % 16 || bytes_per_launch > span_bytes)
    return MOE_E_INVALID;
  if (nontemporal != 0 && nontemporal != 1) return MOE_E_INVALID;
  const hipError_t e = probe_stream_read(buf, span_bytes, bytes_per_launch, nontemporal, reps,
                                         (uint32_t*)sink, (hipStream_t)stream, avg_us);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_HIP;
  }
  return MOE_OK;
}

moe_status moe_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t reps, void* stream,
                          double* avg_us) {
  if (!src || !dst || !avg_us || reps < 1 || reps > 100000) return MOE_E_INVALID;
  if (!aligned16(src) || !aligned16(dst) || bytes < 16 || bytes % 16) return MOE_E_INVALID;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_E_INVALID;  // overlapping
  const hipError_t e = probe_copy(src, dst, bytes, reps, (hipStream_t)stream, avg_us);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_HIP;
  }
  return MOE_OK;
}

moe_status moe_probe_empty_launch(int32_t grid, int32_t reps, void* stream, double* avg_us) {
  if (!avg_us || grid < 1 || grid > (1 << 20) || reps < 1 || reps > 100000)
    return MOE_E_INVALID;
  const hipError_t e = probe_empty_launch(grid, reps, (hipStream_t)stream, avg_us);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_HIP;
  }
  return MOE_OK;
}

int32_t moe_miss_split(int32_t misses, int32_t b_cpu_mbps, int32_t b_pcie_mbps) {
  if (misses < 0 || b_cpu_mbps < 0 || b_pcie_mbps < 0) return -1;
  return miss_split(misses, b_cpu_mbps, b_pcie_mbps);
}

moe_status moe_set_hybrid_timeout(moe_cache c, int64_t microseconds) {
  if (!c || microseconds < 1) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_BUSY;
  c->v.hyb_timeout_ticks = microseconds * 100;  // the GPU's constant clock runs at 100 MHz
  return MOE_OK;
}

moe_status moe_hybrid_hold(moe_cache c, int32_t hold) {
  if (!c || !c->hyb || (hold != 0 && hold != 1)) return MOE_E_INVALID;
  c->hyb->hold.store(hold != 0, std::memory_order_release);
  return MOE_OK;
}

moe_status moe_hybrid_read(moe_cache c, int64_t* requests, int64_t* experts, double* busy_s) {
  if (!c) return MOE_E_INVALID;
  const HybridServer* h = c->hyb;
  if (requests) *requests = h ? h->served.load() : 0;
  if (experts) *experts = h ? h->experts.load() : 0;
  if (busy_s) *busy_s = h ? 1e-9 * (double)h->busy_ns.load() : 0.0;
  return MOE_OK;
}

moe_status moe_cpu_expert_ffn(const moe_shape* shape, const void* blob, const void* x, int32_t T,
                              const float* w, float* y, int32_t threads) {
  if (!shape_ok(shape) || shape->wfmt != MOE_FMT_BF16) return MOE_E_INVALID;
  if (!blob || !x || !w || !y || T < 1 || T > kDecodeMaxTokens) return MOE_E_INVALID;
  if (threads < 1 || threads > 256) return MOE_E_INVALID;
  CpuTeam team(threads);
  std::vector<float> partial((size_t)threads * T * shape->hidden);
  int row_tok[kDecodeMaxTokens];
  for (int t = 0; t < T; ++t) row_tok[t] = t;
  const int row0 = 0, ntok = T;
  const uint16_t* b = (const uint16_t*)blob;
  cpu_experts_ffn(team, &b, 1, &row0, &ntok, row_tok, w, shape->hidden, shape->inter,
                  (const uint16_t*)x, T, y, partial.data());
  return MOE_OK;
}

moe_status moe_cpu_expert_rate(const moe_shape* shape, const void* pool, int32_t n_blobs,
                               int32_t threads, int32_t reps, double* gbps) {
  if (!shape_ok(shape) || shape->wfmt != MOE_FMT_BF16 || !pool || !gbps) return MOE_E_INVALID;
  if (n_blobs < 1 || threads < 1 || threads > 256 || reps < 1) return MOE_E_INVALID;
  const int H = shape->hidden, I = shape->inter;
  CpuTeam team(threads);
  std::vector<float> partial((size_t)threads * H), y(H);
  std::vector<uint16_t> x(H, (uint16_t)0x3c00);  // 2^-7 in bf16
  const int row_tok = 0, row0 = 0, ntok = 1;
  const float w = 1.0f;
  auto one = [&](int b) {
    const uint16_t* blob = (const uint16_t*)((const unsigned char*)pool + (size_t)b * shape->blob_bytes);
    cpu_experts_ffn(team, &blob, 1, &row0, &ntok, &row_tok, &w, H, I, x.data(), 1, y.data(),
                    partial.data());
  };
  one(0);
  const auto t0 = std::chrono::steady_clock::now();
  for (int r = 0; r < reps; ++r)
    for (int b = 0; b < n_blobs; ++b) one(b);
  const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  *gbps = (double)reps * n_blobs * (double)shape->blob_bytes / dt / 1e9;
  return MOE_OK;
}

moe_status moe_route_classify(moe_cache c, int32_t layer, const void* x, int32_t T,
                              const void* w_router, int32_t* topk_idx, float* topk_w,
                              void* stream) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_INVALID;
  if (layer < 0 || layer >= c->d.L || T < 0 || T > c->d.max_tokens) return MOE_E_INVALID;
  if (T > 0 && (!x || !w_router || !aligned16(x) || !aligned16(w_router))) return MOE_E_INVALID;
  if (T > kDecodeMaxTokens && !many_tokens_ok(c->d)) return MOE_E_INVALID;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = ensure_events(c);
  if (e == hipSuccess) e = route_launch(c, layer, x, T, w_router, topk_idx, topk_w, s);
  if (e == hipSuccess) e = hipEventRecord(c->ev_plan, s);
  if (e != hipSuccess) return hip_fail(c, e);
  c->state = State::Planned;
  c->plan_T = T;
  c->plan_layer = layer;
  return MOE_OK;
}

moe_status moe_fill_misses(moe_cache c, int32_t groups, void* fill_stream) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Planned) return MOE_E_INVALID;
  if (groups < 1 || groups > kMaxGroups) return MOE_E_INVALID;
  hipStream_t s = (hipStream_t)fill_stream;
  // The plan is ready, and (same compute stream) the previous step's FFN has finished reading
  // the victim slots.
  hipError_t e = hipStreamWaitEvent(s, c->ev_plan, 0);
  for (int g = 0; g < groups && e == hipSuccess; ++g) {
    e = c->prof.timed(Profiler::FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      return launch_fill(c->v, c->pool_dev, c->arena, c->d.S, g, groups, kFillGrid, s, e0, e1, 0, c->d.E);
    });
    if (e == hipSuccess) e = hipEventRecord(c->ev_fill[g], s);
  }
  if (e != hipSuccess) return hip_fail(c, e);
  c->fill_groups = groups;
  c->state = State::Filled;
  return MOE_OK;
}

moe_status moe_expert_ffn(moe_cache c, int32_t layer, const void* x, int32_t T,
                          const void* shared_blob, void* y, void* stream) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Filled) return MOE_E_INVALID;
  if (layer != c->plan_layer || T != c->plan_T) return MOE_E_INVALID;
  if (T > 0 && (!x || !y || !aligned16(x) || ((uintptr_t)y & 3))) return MOE_E_INVALID;
  if (c->d.has_shared && T > 0 && (!shared_blob || !aligned16(shared_blob))) return MOE_E_INVALID;
  hipStream_t s = (hipStream_t)stream;
  auto& P = c->prof;
  const int nu = T * c->d.K < c->d.E ? T * c->d.K : c->d.E;
  const int G = c->fill_groups;
  hipError_t e = wait_prefetch(c, layer, s);  // hits may have been prefetched
  (void)P;
  if (e == hipSuccess && T > 0)  // hit experts and the shared expert: no fill to wait for
    e = ffn_launch(c, x, T, shared_blob, y, 0, 0, 1, nu + c->d.has_shared, 0, s);
  for (int g = 0; g < G && e == hipSuccess; ++g) {
    e = hipStreamWaitEvent(s, c->ev_fill[g], 0);
    if (e == hipSuccess && T > 0)
      e = ffn_launch(c, x, T, shared_blob, y, 1, g, G, (nu + G - 1) / G, g == G - 1, s);
  }
  if (e != hipSuccess) return hip_fail(c, e);
  c->state = State::Idle;
  return MOE_OK;
}

// The whole step in stream order on one queue: route/plan, the fill of every miss, then
// one FFN over all the step's experts (hits, shared, misses) and the combine.  No event
// joins two queues, so consecutive kernels start back to back.
static moe_status layer_step_serial(moe_cache c, int32_t layer, const void* x, int32_t T,
                                    const void* w_router, const void* shared_blob,
                                    int32_t* topk_idx, float* topk_w, void* y, hipStream_t s,
                                    hipStream_t fs) {
  if (T > 0 && (!aligned16(x) || !aligned16(w_router) || ((uintptr_t)y & 3)))
    return MOE_E_INVALID;
  if (c->d.has_shared && T > 0 && !aligned16(shared_blob)) return MOE_E_INVALID;
  auto& P = c->prof;
  hipError_t e = route_launch(c, layer, x, T, w_router, topk_idx, topk_w, s);
  if (e == hipSuccess)
    e = P.timed(Profiler::FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      return launch_fill(c->v, c->pool_dev, c->arena, c->d.S, 0, 1, kFillGrid, s, e0, e1, 0, c->d.E);
    });
  const int nu = T * c->d.K < c->d.E ? T * c->d.K : c->d.E;
  if (e == hipSuccess && prefetch_next(c, layer, T)) e = issue_prefetch(c, layer + 1, s, fs);
  if (e == hipSuccess) e = wait_prefetch(c, layer, s);
  if (e == hipSuccess && T > 0)
    e = ffn_launch(c, x, T, shared_blob, y, 2, 0, 1, nu + c->d.has_shared, 1, s);
  if (e != hipSuccess) return hip_fail(c, e);
  c->plan_T = T;
  c->plan_layer = layer;
  c->fill_groups = 1;
  return MOE_OK;
}

moe_status moe_layer_step(moe_cache c, int32_t layer, const void* x, int32_t T,
                          const void* w_router, const void* shared_blob, int32_t* topk_idx,
                          float* topk_w, void* y, int32_t groups, void* compute_stream,
                          void* fill_stream) {
  if (!c) return MOE_E_INVALID;
  if (groups < 0 || groups > kMaxGroups) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_INVALID;
  if (layer < 0 || layer >= c->d.L || T < 0 || T > c->d.max_tokens) return MOE_E_INVALID;
  if (T > 0 && (!x || !y || !w_router)) return MOE_E_INVALID;
  if (c->d.has_shared && T > 0 && !shared_blob) return MOE_E_INVALID;
  if (T > kDecodeMaxTokens && !many_tokens_ok(c->d)) return MOE_E_INVALID;
  if (groups == 0)
    return layer_step_serial(c, layer, x, T, w_router, shared_blob, topk_idx, topk_w, y,
                             (hipStream_t)compute_stream,
                             fill_stream ? (hipStream_t)fill_stream : (hipStream_t)compute_stream);
  moe_status st = moe_route_classify(c, layer, x, T, w_router, topk_idx, topk_w, compute_stream);
  if (st != MOE_OK) return st;
  st = moe_fill_misses(c, groups, fill_stream);
  if (st != MOE_OK) return st;
  if (prefetch_next(c, layer, T)) {
    hipError_t e = issue_prefetch(c, layer + 1, (hipStream_t)compute_stream,
                                  (hipStream_t)fill_stream);
    if (e != hipSuccess) return hip_fail(c, e);
  }
  return moe_expert_ffn(c, layer, x, T, shared_blob, y, compute_stream);
}

moe_status moe_cache_snapshot(moe_cache c, int32_t* key_of, int64_t* stamp, int32_t* slot_of,
                              int32_t* n_occupied, int64_t* step, int32_t* capacity) {
  if (!c) return MOE_E_INVALID;
  if (c->state != State::Idle) return MOE_E_BUSY;
  hipError_t e = hipDeviceSynchronize();
  const size_t cap = (size_t)c->capacity;
  if (e == hipSuccess && key_of) e = hipMemcpy(key_of, c->v.key_of, 4 * cap, hipMemcpyDeviceToHost);
  if (e == hipSuccess && stamp) e = hipMemcpy(stamp, c->v.stamp, 8 * cap, hipMemcpyDeviceToHost);
  if (e == hipSuccess && slot_of)
    e = hipMemcpy(slot_of, c->v.slot_of, 4 * (size_t)c->d.L * c->d.E, hipMemcpyDeviceToHost);
  int ctrl[CTRL_WORDS];
  if (e == hipSuccess) e = hipMemcpy(ctrl, c->v.ctrl, sizeof(ctrl), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  if (n_occupied) *n_occupied = ctrl[CTRL_N];
  if (step) *step = (int64_t)(uint32_t)ctrl[CTRL_STEP_LO] | ((int64_t)ctrl[CTRL_STEP_HI] << 32);
  if (capacity) *capacity = ctrl[CTRL_C];
  if (ctrl[CTRL_ERR] & ERR_CAPACITY) return MOE_E_CAPACITY;
  if (ctrl[CTRL_ERR] & ERR_HYBRID) return MOE_E_HYBRID;
  return MOE_OK;
}

moe_status moe_cache_set_step(moe_cache c, int64_t step) {
  if (!c || step < 0) return MOE_E_INVALID;
  if (c->state != State::Idle || c->pf_layer[0] >= 0 || c->pf_layer[1] >= 0) return MOE_E_BUSY;
  hipError_t e = hipDeviceSynchronize();
  int ctrl[CTRL_WORDS];
  if (e == hipSuccess) e = hipMemcpy(ctrl, c->v.ctrl, sizeof(ctrl), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  if (ctrl[CTRL_N] != 0) return MOE_E_INVALID;  // cached stamps would no longer precede it
  const int w[2] = {(int)(step & 0xffffffff), (int)(step >> 32)};
  e = hipMemcpy(c->v.ctrl + CTRL_STEP_LO, w, sizeof(w), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(c, e);
  return MOE_OK;
}

moe_status moe_plan_read(moe_cache c, moe_plan_host* o) {
  if (!c || !o) return MOE_E_INVALID;
  hipError_t e = hipDeviceSynchronize();
  int hdr[HDR_WORDS];
  if (e == hipSuccess) e = hipMemcpy(hdr, c->v.hdr, sizeof(hdr), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  const int nu = hdr[HDR_NU], nm = hdr[HDR_NMISS], T = hdr[HDR_T];
  o->n_unique = nu;
  o->n_hit = hdr[HDR_NHIT];
  o->n_miss = nm;
  o->n_cpu = hdr[HDR_NCPU];
  o->layer = hdr[HDR_LAYER];
  o->step = (int64_t)(uint32_t)hdr[HDR_STEP_LO] | ((int64_t)hdr[HDR_STEP_HI] << 32);
  std::vector<int> hit(nu > 0 ? nu : 1);
  auto cp = [&](void* dst, const void* src, size_t n) {
    if (e == hipSuccess && dst && n) e = hipMemcpy(dst, src, n, hipMemcpyDeviceToHost);
  };
  cp(o->unique, c->v.U, 4 * (size_t)nu);
  cp(o->slot, c->v.u_slot, 4 * (size_t)nu);
  cp(hit.data(), c->v.u_hit, 4 * (size_t)nu);
  cp(o->miss_key, c->v.miss_key, 4 * (size_t)nm);
  cp(o->miss_slot, c->v.miss_slot, 4 * (size_t)nm);
  cp(o->miss_victim, c->v.miss_victim, 4 * (size_t)nm);
  cp(o->count, c->v.count, 4 * (size_t)nu);
  cp(o->perm, c->v.perm, 4 * (size_t)T * c->d.K);
  cp(o->cpu_key, c->v.cpu_key, 4 * (size_t)o->n_cpu);
  if (e != hipSuccess) return hip_fail(c, e);
  if (o->hit)
    for (int i = 0; i < nu; ++i) o->hit[i] = (uint8_t)hit[i];
  return MOE_OK;
}

moe_status moe_stats(moe_cache c, moe_counters* out) {
  if (!c || !out) return MOE_E_INVALID;
  unsigned long long s[STAT_WORDS];
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(s, c->v.stats, sizeof(s), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  out->steps = (int64_t)s[STAT_STEPS];
  out->hits = (int64_t)s[STAT_HITS];
  out->misses = (int64_t)s[STAT_MISSES];
  out->bytes_filled = (int64_t)s[STAT_BYTES];
  out->cpu_misses = (int64_t)s[STAT_CPU];
  int ctrl[CTRL_WORDS];
  e = hipMemcpy(ctrl, c->v.ctrl, sizeof(ctrl), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  if (ctrl[CTRL_ERR] & ERR_HYBRID) return MOE_E_HYBRID;
  return MOE_OK;
}

moe_status moe_profile_enable(moe_cache c, int32_t mask, int32_t every) {
  if (!c) return MOE_E_INVALID;
  hipError_t e = c->prof.harvest_all();
  if (mask < 0 || mask > MOE_PROF_ALL || every < 1) return MOE_E_INVALID;
  if (e == hipSuccess && mask) e = c->prof.ensure();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess)
    e = hipMemcpy(c->prof.stats0, c->v.stats, sizeof(c->prof.stats0), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  c->prof.reset();
  c->prof.mask = mask;
  c->prof.every = every;
  return MOE_OK;
}

moe_status moe_profile_read(moe_cache c, moe_profile* out) {
  if (!c || !out) return MOE_E_INVALID;
  hipError_t e = c->prof.harvest_all();
  unsigned long long st[STAT_WORDS];
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(st, c->v.stats, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  const auto& P = c->prof;
  for (int k = 0; k < Profiler::NKIND; ++k) {
    out->launches[k] = P.launches[k];
    out->ms[k] = P.ms[k];
  }
  out->fill_bytes = (int64_t)(st[STAT_BYTES] - P.stats0[STAT_BYTES]);
  out->ffn_weight_bytes = (int64_t)(st[STAT_FFN_BYTES] - P.stats0[STAT_FFN_BYTES]);
  // the gate/up rows and their scales are exactly two thirds of a blob in every format; a
  // fused one-token launch reads the whole blob
  out->fused_timed_bytes =
      (int64_t)(st[STAT_TIMED_FUSED_BYTES] - P.stats0[STAT_TIMED_FUSED_BYTES]);
  out->gate_up_timed_bytes =
      (int64_t)((st[STAT_TIMED_BLOB_BYTES] - P.stats0[STAT_TIMED_BLOB_BYTES]) / 3 * 2) +
      out->fused_timed_bytes;
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_INVALID: return "invalid argument or call order";
    case MOE_E_CAPACITY: return "capacity out of range";
    case MOE_E_BUSY: return "a step is in flight";
    case MOE_E_HIP: return "HIP runtime error";
    case MOE_E_NOMEM: return "pinned host memory unavailable";
    case MOE_E_HYBRID: return "hybrid decode: the host did not answer a step in time";
    case MOE_E_SCRATCH:
      return "workspace larger than the library's static workspace (16 MiB per device)";
    default: return "unknown status";
  }
}

int32_t moe_last_hip_error(moe_cache c) { return c ? c->last_hip : 0; }

}  // extern "C"
