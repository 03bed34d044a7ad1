// Miss fills from the pinned host pool, cache state initialisation, and elastic resize.
//
// Fills: only missed experts cross PCIe, on demand ("FreeToken vs vLLM on one RTX 3090",
// Summary and "FreeToken exploits MoE sparsity"); the pool is pinned and DMA-visible (FreeToken
// paper summary, last paragraph); each blob lands directly in its final slot (execution-layer
// paragraph: runtime layout, load straight to the final place).  The misses of a step are
// split into groups copied one after another so the FFN of group g overlaps the copy of group
// g+1 ("FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理", "FreeToken 解决的问题").
//
// Gfx950 design: the copy is a kernel that reads the pinned pool through its device mapping
// (zero-copy over PCIe) and writes the slot in HBM.  Its source and destination come from the
// plan in device memory (the step plan, or the prefetch plan of the next layer), so no host
// round trip is needed and the whole step can be captured in a hipGraph; 32 workgroups move
// 9 MiB blobs at the link's full rate (55-57 GB/s against 53-54 GB/s for pinned
// hipMemcpyAsync of the same blobs) and leave the rest of the GPU to concurrent kernels.
//
// Resize: FreeToken paper summary, execution-layer paragraph (cache rebuilt at a scheduler
// safe point when the VRAM budget changes, without restarting) and problem paragraph (budgets
// change during a session).  Reading used: keep the new_capacity most recently used keys;
// survivors in slots >= new_capacity move into the freed slots below it, in ascending slot
// order; stamps are kept.
#include "moe_dev.h"

namespace moe {

// ---------------------------------------------------------------- fills
struct FillArgs {
  const int* hdr;        // plan header (HDR_NMISS misses)
  const int* miss_key;   // [misses] pool key of each miss
  const int* miss_slot;  // [misses] destination slot
  const uint4* pool;     // device mapping of the pinned pool
  uint4* arena;
  long long S16;         // blob bytes / 16
  int group;
  int ngroups;
};

constexpr int FILL_THREADS = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(FILL_THREADS) void fill_kernel(FillArgs a) {
  const int m = a.hdr[HDR_NMISS];
  const int n0 = (int)((long long)a.group * m / a.ngroups);
  const int n1 = (int)((long long)(a.group + 1) * m / a.ngroups);
  const size_t tid = (size_t)blockIdx.x * FILL_THREADS + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * FILL_THREADS;
  const size_t S16 = (size_t)a.S16;
  for (int b = n0; b < n1; ++b) {
    const uint4* src = a.pool + (size_t)a.miss_key[b] * S16;
    uint4* dst = a.arena + (size_t)a.miss_slot[b] * S16;
    for (size_t i = tid; i < S16; i += 4 * nthr) {
      uint4 r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t k = i + q * nthr;
        if (k < S16) r[q] = src[k];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t k = i + q * nthr;
        // plain stores: the step's FFN reads the blob right after this kernel, and a blob
        // stored through the caches reaches it sooner than a streaming store (measured:
        // the fused FFN launch that follows runs 0.6 us shorter, the link rate is unchanged)
        if (k < S16) *(u32x4*)(dst + k) = *(const u32x4*)&r[q];
      }
    }
  }
}

// Copies the misses of a plan (`prefetch`: the prefetch plan, else the step plan).
hipError_t launch_fill(const Dev& v, const void* pool_dev, void* arena, long long S, int group,
                       int ngroups, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                       int prefetch, int E) {
  const PlanOut o = prefetch ? prefetch_plan_out(v, E) : step_plan_out(v);
  FillArgs a{o.hdr, o.miss_key, o.miss_slot, (const uint4*)pool_dev, (uint4*)arena, S / 16,
             group, ngroups};
  return launch_timed(fill_kernel, dim3(grid), dim3(FILL_THREADS), 0, s, e0, e1, a);
}

// ---------------------------------------------------------------- state init
struct InitArgs {
  Dev v;
  int max_capacity;
  int n_keys;
  int capacity;
};

__global__ void init_kernel(InitArgs a) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int nthr = gridDim.x * blockDim.x;
  for (int i = tid; i < a.max_capacity; i += nthr) {
    a.v.key_of[i] = -1;
    a.v.stamp[i] = -1;
  }
  for (int i = tid; i < a.n_keys; i += nthr) a.v.slot_of[i] = -1;
  if (tid < CTRL_WORDS) a.v.ctrl[tid] = (tid == CTRL_C) ? a.capacity : 0;
  if (tid < HDR_WORDS) a.v.hdr[tid] = 0;
  if (tid < STAT_WORDS) a.v.stats[tid] = 0;
}

hipError_t launch_init(const Dev& v, int max_capacity, int n_keys, int capacity, hipStream_t s) {
  InitArgs a{v, max_capacity, n_keys, capacity};
  hipLaunchKernelGGL(init_kernel, dim3(64), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- resize
constexpr int RZ = 256;
enum : int { CTRL_NMOVES = 6, CTRL_NCOPY = 7 };

struct ResizeArgs {
  Dev v;
  int new_capacity;
  int max_capacity;
  int E;
  int relocate;  // 1: survivors are copied to a new arena, slot by slot
};

// Single workgroup.  Output: v.moves[2*k] = source slot, v.moves[2*k+1] = destination slot of
// the k-th blob copy; ctrl[CTRL_NCOPY] copies.  In place only the compaction moves are copied;
// with relocate every surviving slot is copied (source slot -> its new slot).
__global__ __launch_bounds__(RZ) void resize_plan_kernel(ResizeArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dev& v = a.v;
  const int n = v.ctrl[CTRL_N];
  const int C = v.ctrl[CTRL_C];
  const int Cn = a.new_capacity;
  __shared__ int s_nh, s_nm;
  if (Cn >= C || n <= Cn) {
    // nothing is evicted; slots beyond Cn are empty (occupied slots form [0, n))
    for (int i = threadIdx.x; i < n; i += RZ) {
      if (a.relocate) {
        v.moves[2 * i] = i;
        v.moves[2 * i + 1] = i;
      }
    }
    if (threadIdx.x == 0) {
      v.ctrl[CTRL_C] = Cn;
      v.ctrl[CTRL_NCOPY] = a.relocate ? n : 0;
    }
    return;
  }
  // Sort the n occupied slots by (stamp, key) ascending: bitonic sort in LDS.
  int P = 1;
  while (P < n) P <<= 1;
  uint64_t* s_st = (uint64_t*)smem;       // [P] 64-bit stamps
  uint32_t* s_key = (uint32_t*)(s_st + P);  // [P] keys
  int* s_slot = (int*)(s_key + P);        // [P]
  int* s_evict = s_slot + P;              // [max_capacity] 1 = evicted
  for (int i = threadIdx.x; i < P; i += RZ) {
    if (i < n) {
      s_st[i] = (uint64_t)v.stamp[i];
      s_key[i] = (uint32_t)v.key_of[i];
      s_slot[i] = i;
    } else {
      s_st[i] = ~0ull;
      s_key[i] = ~0u;
      s_slot[i] = -1;
    }
  }
  for (int i = threadIdx.x; i < a.max_capacity; i += RZ) s_evict[i] = 0;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < P; i += RZ) {
        const int l = i ^ jj;
        if (l > i) {
          const bool up = (i & k) == 0;
          const uint64_t si = s_st[i], sl = s_st[l];
          const uint32_t ki = s_key[i], kl = s_key[l];
          const bool gt = si > sl || (si == sl && ki > kl);
          if (gt == up) {
            s_st[i] = sl;
            s_st[l] = si;
            s_key[i] = kl;
            s_key[l] = ki;
            const int t = s_slot[i];
            s_slot[i] = s_slot[l];
            s_slot[l] = t;
          }
        }
      }
      __syncthreads();
    }
  }
  const int nev = n - Cn;
  for (int q = threadIdx.x; q < nev; q += RZ) {
    const int sl = s_slot[q];
    s_evict[sl] = 1;
    v.slot_of[v.key_of[sl]] = -1;
  }
  __syncthreads();
  // holes: evicted slots < Cn ascending; movers: surviving slots >= Cn ascending
  int* s_holes = (int*)(s_evict + a.max_capacity);  // [Cn]
  int* s_movers = s_holes + Cn;                     // [n - Cn]
  if (threadIdx.x == 0) {
    int nh = 0, nm = 0;
    for (int i = 0; i < Cn; ++i)
      if (s_evict[i]) s_holes[nh++] = i;
    for (int i = Cn; i < n; ++i)
      if (!s_evict[i]) s_movers[nm++] = i;
    s_nh = nh;
    s_nm = nm;
  }
  __syncthreads();
  const int nmv = s_nm;  // == s_nh
  for (int q = threadIdx.x; q < nmv; q += RZ) {
    const int src = s_movers[q], dst = s_holes[q];
    const int key = v.key_of[src];
    v.key_of[dst] = key;
    v.stamp[dst] = v.stamp[src];
    v.slot_of[key] = dst;
    if (!a.relocate) {
      v.moves[2 * q] = src;
      v.moves[2 * q + 1] = dst;
    }
  }
  __syncthreads();
  if (a.relocate) {
    // every surviving slot i < Cn: source = its mover if i was a hole, else i
    for (int i = threadIdx.x; i < Cn; i += RZ) {
      v.moves[2 * i] = i;
      v.moves[2 * i + 1] = i;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < nmv; q += RZ) v.moves[2 * s_holes[q]] = s_movers[q];
  }
  for (int i = Cn + threadIdx.x; i < C; i += RZ) {
    v.key_of[i] = -1;
    v.stamp[i] = -1;
  }
  if (threadIdx.x == 0) {
    v.ctrl[CTRL_N] = Cn;
    v.ctrl[CTRL_C] = Cn;
    v.ctrl[CTRL_NCOPY] = a.relocate ? Cn : nmv;
  }
}

size_t resize_lds_bytes(int max_capacity) {
  int P = 1;
  while (P < max_capacity) P <<= 1;
  return (size_t)P * (sizeof(uint64_t) + 2 * sizeof(int)) +
         sizeof(int) * (size_t)max_capacity * 2 + 64;
}

struct CopyArgs {
  Dev v;
  const uint4* src_arena;
  uint4* dst_arena;
  long long S16;
};

__global__ __launch_bounds__(256) void slot_copy_kernel(CopyArgs a) {
  const int nc = a.v.ctrl[CTRL_NCOPY];
  const size_t S16 = (size_t)a.S16;
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * 256;
  for (int c = 0; c < nc; ++c) {
    const int src = a.v.moves[2 * c], dst = a.v.moves[2 * c + 1];
    if (src == dst && a.src_arena == a.dst_arena) continue;
    const uint4* s = a.src_arena + (size_t)src * S16;
    uint4* d = a.dst_arena + (size_t)dst * S16;
    for (size_t i = tid; i < S16; i += nthr) d[i] = s[i];
  }
}

hipError_t launch_resize(const Dev& v, int new_capacity, int max_capacity, int E,
                         const void* old_arena, void* new_arena, long long S, hipStream_t s) {
  const int relocate = (new_arena != nullptr && new_arena != old_arena) ? 1 : 0;
  ResizeArgs ra{v, new_capacity, max_capacity, E, relocate};
  const size_t lds = resize_lds_bytes(max_capacity);
  if (lds > 65536) {
    hipError_t e0 = hipFuncSetAttribute((const void*)resize_plan_kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(resize_plan_kernel, dim3(1), dim3(RZ), lds, s, ra);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CopyArgs ca{v, (const uint4*)old_arena, (uint4*)(relocate ? new_arena : const_cast<void*>(old_arena)),
              S / 16};
  hipLaunchKernelGGL(slot_copy_kernel, dim3(1024), dim3(256), 0, s, ca);
  return hipGetLastError();
}

}  // namespace moe
