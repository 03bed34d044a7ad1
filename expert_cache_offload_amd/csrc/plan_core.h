// The single-workgroup part of a layer step's plan, shared by the decode route kernel and
// the prefill plan kernel: per-step dedup of the selected experts, hit/miss classification
// against the (layer, expert)-keyed slot table, LRU victim selection and the slot-table
// update, the FFN entry table, the plan header and the counters.
//
// FreeToken paper summary (agihunt.info, arXiv 2608.16157), execution-layer paragraph:
// routing dedup, hit classification and LRU victim selection run on the GPU with no host
// round trip; the cache is one slot pool shared by all MoE layers (memory-architecture
// paragraph) with a global LRU (attribution paragraph).  The rule reproduced: U is the
// ascending set of selected experts; misses are taken in ascending expert id; free slots
// [n, C) go first in ascending order, then the `need` smallest (stamp, key) among occupied
// slots not used by this step; every key of U is stamped with the step counter.
#pragma once
#include "moe_dev.h"

namespace moe {

constexpr int RT = 256;  // threads of a plan workgroup (4 waves)
constexpr int kSlotsPerThread = kMaxSlots / RT;

// Ordered compaction over [0, n): emit(i, pos) for every i with pred(i); pos ascends with i.
template <class P, class F>
__device__ int block_compact(int n, P pred, F emit, int* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  for (int base = 0; base < n; base += RT) {
    int i = base + (int)threadIdx.x;
    bool p = i < n && pred(i);
    uint64_t b = __ballot(p);
    if (lane == 0) s_tmp[wave] = __popcll(b);
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += s_tmp[w];
    int tot = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    if (p) emit(i, off + (int)__popcll(b & lanemask_lt()));
    running += tot;
    __syncthreads();
  }
  return running;
}

__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t* s_tmp) {
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  uint64_t m = s_tmp[0];
  for (int w = 1; w < RT / 64; ++w) m = s_tmp[w] < m ? s_tmp[w] : m;
  __syncthreads();
  return m;
}

// LDS arrays of the plan (dynamic shared memory).
struct PlanLds {
  uint64_t* comp;  // [max_capacity] 64-bit stamp per occupied slot (~0: not evictable)
  int* cnt;        // [E] assignments per expert this step
  int* uidx;       // [E] position of an expert in U, -1 if unused
  int* srow;       // [E] this layer's row of slot_of
  int* U;          // [pw] + the arrays below, per position in U unless noted
  int* off;        // [pw + 1]
  int* uslot;
  int* hit;
  int* miss;       // [pw] miss list (positions in U)
  int* vict;       // [pw] victim slots in eviction order
  int* vkey;       // [pw] their keys
  int* grp;
  int* sorted;
  int* aslot;      // [pw] per miss: assigned slot
  int* avkey;      // [pw] per miss: evicted key or -1
  int* hitl;       // [pw] hit list (positions in U)
};

// The arrays indexed by a position in U (and the victim group buffers) hold d.pw entries:
// the step's distinct experts (at most umax), or every expert of a layer for a prefetch plan.
inline __host__ __device__ size_t plan_lds_bytes(const Dims& d) {
  size_t b = sizeof(uint64_t) * (size_t)d.max_capacity;
  b += sizeof(int) * 3 * (size_t)d.E;
  b += sizeof(int) * (size_t)(12 * d.pw + 1);
  return (b + 15) & ~(size_t)15;
}

__device__ inline unsigned char* plan_carve(const Dims& d, unsigned char* p, PlanLds& s) {
  const int pw = d.pw;
  s.comp = (uint64_t*)p;  p += sizeof(uint64_t) * d.max_capacity;
  s.cnt = (int*)p;        p += sizeof(int) * d.E;
  s.uidx = (int*)p;       p += sizeof(int) * d.E;
  s.srow = (int*)p;       p += sizeof(int) * d.E;
  s.U = (int*)p;          p += sizeof(int) * pw;
  s.off = (int*)p;        p += sizeof(int) * (pw + 1);
  s.uslot = (int*)p;      p += sizeof(int) * pw;
  s.hit = (int*)p;        p += sizeof(int) * pw;
  s.miss = (int*)p;       p += sizeof(int) * pw;
  s.vict = (int*)p;       p += sizeof(int) * pw;
  s.vkey = (int*)p;       p += sizeof(int) * pw;
  s.grp = (int*)p;        p += sizeof(int) * pw;
  s.sorted = (int*)p;     p += sizeof(int) * pw;
  s.aslot = (int*)p;      p += sizeof(int) * pw;
  s.avkey = (int*)p;      p += sizeof(int) * pw;
  s.hitl = (int*)p;       p += sizeof(int) * pw;
  // align by adding an offset: a round trip through an integer would lose the pointer's
  // LDS address space, and every access through it would become a flat access
  return p + ((16 - ((uintptr_t)p & 15)) & 15);
}

// Static shared scratch of the plan.
struct PlanTmp {
  int tmp[8];
  uint64_t tmp64[8];
  int g;
  int err;
  int nfill, ncpu;  // misses filled / computed by the CPU (set by plan_cache)
};

// Hybrid decode: how many of m misses the CPU computes in place.  Serving q misses on the
// CPU (expert-weight rate bc) and m - q by fills (PCIe rate bp, both MB/s) finishes at
// max((m - q) / bp, q / bc); q minimises it, the smaller q on a tie.  The makespan falls
// while q is below the equal-finish point m*bc/(bc+bp) and rises after it, so the
// minimiser is that point's floor or the next integer; exact in integers.
// (FreeToken paper summary: q is a closed-form split by measured bandwidth, derived in the
// fused routing kernel.)
__host__ __device__ inline int miss_split(int m, int bc, int bp) {
  if (m <= 0 || bc <= 0) return 0;
  const long long q0 = (long long)m * bc / ((long long)bc + (long long)bp);
  if (q0 >= m) return m;
  const long long a0 = (m - q0) * (long long)bc, b0 = q0 * (long long)bp;
  const long long a1 = (m - q0 - 1) * (long long)bc, b1 = (q0 + 1) * (long long)bp;
  const long long t0 = a0 > b0 ? a0 : b0, t1 = a1 > b1 ? a1 : b1;
  return (int)(t1 < t0 ? q0 + 1 : q0);
}

// Cache state the plan reads, loaded once at its start.
constexpr int kRowsPerThread = 1024 / RT;  // slot_of row entries per thread (E <= 1024)
struct PlanState {
  int n, C;
  long long step;
  uint64_t st[kSlotsPerThread];   // this thread's slots: stamps (~0: empty) and keys
  uint32_t key[kSlotsPerThread];
  int srow[kRowsPerThread];                            // this thread's slot_of row entries
};

// All threads: issue every load of the plan's start - this layer's slot_of row, the control
// words and the (stamp, key) of every slot the handle can hold (unconditionally: a bound on
// the occupancy would make these loads wait for the control words) - into registers.
__device__ inline void plan_begin_load(const Dims& d, const Dev& v, int layer, PlanState& ps) {
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int e = (int)threadIdx.x + j * RT;
    ps.srow[j] = e < d.E ? v.slot_of[layer * d.E + e] : -1;
  }
  ps.n = v.ctrl[CTRL_N];
  ps.C = v.ctrl[CTRL_C];
  ps.step = (long long)(unsigned)v.ctrl[CTRL_STEP_LO] | ((long long)v.ctrl[CTRL_STEP_HI] << 32);
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int i = (int)threadIdx.x + j * RT;
    const bool in = i < d.max_capacity;
    ps.st[j] = in ? (uint64_t)v.stamp[i] : ~0ull;
    ps.key[j] = in ? (uint32_t)v.key_of[i] : 0xffffffffu;
  }
}

// All threads, after plan_begin_load: the per-expert LDS arrays, and the slots beyond the
// occupancy marked empty.  The caller syncs before reading the LDS arrays.
__device__ inline void plan_begin_store(const Dims& d, PlanLds& s, PlanState& ps) {
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int e = (int)threadIdx.x + j * RT;
    if (e < d.E) {
      s.cnt[e] = 0;
      s.uidx[e] = -1;
      s.srow[e] = ps.srow[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int i = (int)threadIdx.x + j * RT;
    if (i >= ps.n) {
      ps.st[j] = ~0ull;
      ps.key[j] = 0xffffffffu;
    }
  }
}

// Both parts at once (plans whose start has no other loads to overlap).
__device__ inline void plan_begin(const Dims& d, const Dev& v, int layer, PlanLds& s,
                                  PlanState& ps) {
  plan_begin_load(d, v, layer, ps);
  plan_begin_store(d, s, ps);
}

// After s.cnt holds the step's assignments per expert (synced): U ascending (ballot /
// popcount compaction), count/offset per position in U; returns nU.  Ends synced.
__device__ inline int plan_dedup(const Dims& d, const PlanOut& o, PlanLds& s, PlanTmp& pt) {
  const int nU = block_compact(
      d.E, [&](int e) { return s.cnt[e] > 0; },
      [&](int e, int pos) {
        s.U[pos] = e;
        s.uidx[e] = pos;
        o.U[pos] = e;
      },
      pt.tmp);
  if (threadIdx.x == 0) {
    int run = 0;
    for (int u = 0; u < nU; ++u) {
      s.off[u] = run;
      o.offset[u] = run;
      const int c = s.cnt[s.U[u]];
      o.count[u] = c;
      run += c;
    }
    s.off[nU] = run;
    o.offset[nU] = run;
  }
  __syncthreads();
  return nU;
}

// Classification, LRU victims, slot-table update, entry table, header and counters, written
// to `o`.  The slots prot[0 .. n_prot) are never victims (a prefetch protects the slots of the
// step before it).  With split rates (bc > 0, decode only) the last q = miss_split(m) misses
// in ascending expert id are computed by the CPU: no slot, no eviction, no stamp; the
// header's miss count is then the filled misses only.  Returns false (after recording the
// error and an empty plan) when fewer slots can be evicted than there are misses to fill.
struct NoSplitPost {
  __device__ void operator()(int, int) const {}
};

template <class SplitPost = NoSplitPost>
__device__ inline bool plan_cache(const Dims& d, const Dev& v, const PlanOut& o, int layer,
                                  int T, int nU, PlanLds& s, const PlanState& ps, PlanTmp& pt,
                                  const int* prot = nullptr, int n_prot = 0, int split_bc = 0,
                                  int split_bp = 0, SplitPost split_post = SplitPost{}) {
  const int E = d.E, pw = d.pw;
  for (int u = threadIdx.x; u < nU; u += RT) {
    const int sl = s.srow[s.U[u]];
    s.uslot[u] = sl;
    s.hit[u] = sl >= 0 ? 1 : 0;
  }
  __syncthreads();
  const int nHit = block_compact(
      nU, [&](int u) { return s.hit[u] != 0; },
      [&](int u, int pos) {
        o.hit_list[pos] = u;
        s.hitl[pos] = u;
      },
      pt.tmp);
  const int nAllMiss = block_compact(
      nU, [&](int u) { return s.hit[u] == 0; },
      [&](int u, int pos) {
        s.miss[pos] = u;
        o.miss_list[pos] = u;
      },
      pt.tmp);
  const int nCpu = miss_split(nAllMiss, split_bc, split_bp);
  const int nMiss = nAllMiss - nCpu;  // misses filled into slots: the first nMiss of the list
  // the CPU misses are known here (the last nCpu of the list): the caller may hand them to the
  // host before the victims are chosen (all threads call it; s.miss, s.U and s.off are synced)
  split_post(nMiss, nCpu);

  // LRU victims: the `need` smallest (stamp, key) among occupied slots not used this step,
  // found in rounds of "oldest remaining stamp" (one round per distinct stamp taken: a
  // step stamps all of its experts alike, so a group never exceeds pw - at most umax keys
  // for a routed step, E for a prefetch step)
  const int n = ps.n, C = ps.C;
  const int nfree = C - n;
  const int need = nMiss > nfree ? nMiss - nfree : 0;
  if (threadIdx.x == 0) pt.err = 0;
  if (need > 0) {
    const uint64_t NONE = ~0ull;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {  // the keys stay in this thread's registers
      const int i = (int)threadIdx.x + j * RT;
      if (i < n) s.comp[i] = ps.st[j];
    }
    __syncthreads();
    for (int u = threadIdx.x; u < nU; u += RT)  // keys of this step are never victims
      if (s.hit[u]) s.comp[s.uslot[u]] = NONE;
    for (int i = threadIdx.x; i < n_prot; i += RT) {  // nor are protected slots
      const int sl = prot[i];
      if (sl >= 0 && sl < n) s.comp[sl] = NONE;
    }
    __syncthreads();
    // group keys in collection order and in key order: the slot assignment's arrays, which
    // are free until the victims are known
    int* gkey = s.aslot;
    int* skey = s.avkey;
    int got = 0;
    for (int round = 0; round < need && got < need; ++round) {
      uint64_t m = NONE;
      for (int i = threadIdx.x; i < n; i += RT) m = s.comp[i] < m ? s.comp[i] : m;
      m = block_min_u64(m, pt.tmp64);
      if (m == NONE) {  // fewer evictable slots than misses: capacity floor violated
        if (threadIdx.x == 0) pt.err = 1;
        break;
      }
      if (threadIdx.x == 0) pt.g = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kSlotsPerThread; ++j) {
        const int i = (int)threadIdx.x + j * RT;
        if (i < n && s.comp[i] == m) {
          const int q = atomicAdd(&pt.g, 1);
          if (q < pw) {
            s.grp[q] = i;
            gkey[q] = (int)ps.key[j];
          }
        }
      }
      __syncthreads();
      const int g = pt.g < pw ? pt.g : pw;
      for (int q = threadIdx.x; q < g; q += RT) {  // order the group by key
        const int kq = gkey[q];
        int rank = 0;
        for (int r = 0; r < g; ++r) rank += (gkey[r] < kq);
        s.sorted[rank] = s.grp[q];
        skey[rank] = kq;
      }
      __syncthreads();
      const int take = g < need - got ? g : need - got;
      for (int q = threadIdx.x; q < take; q += RT) {
        s.vict[got + q] = s.sorted[q];
        s.vkey[got + q] = skey[q];
        s.comp[s.sorted[q]] = NONE;
      }
      got += take;
      __syncthreads();
    }
  }
  __syncthreads();
  if (pt.err) {
    if (threadIdx.x == 0) {
      atomicOr(&v.ctrl[CTRL_ERR], ERR_CAPACITY);
      o.hdr[HDR_NU] = 0;
      o.hdr[HDR_NHIT] = 0;
      o.hdr[HDR_NMISS] = 0;
      o.hdr[HDR_NCPU] = 0;
      pt.nfill = 0;
      pt.ncpu = 0;
    }
    return false;
  }

  // slot assignment: free slots n, n+1, ... first, then victims in LRU order
  for (int i = threadIdx.x; i < nMiss; i += RT) {
    const int slot = i < nfree ? n + i : s.vict[i - nfree];
    s.aslot[i] = slot;
    s.avkey[i] = i < nfree ? -1 : s.vkey[i - nfree];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nMiss; i += RT)
    if (s.avkey[i] >= 0) v.slot_of[s.avkey[i]] = -1;
  __syncthreads();
  for (int i = threadIdx.x; i < nMiss; i += RT) {
    const int u = s.miss[i];
    const int key = layer * E + s.U[u];
    const int slot = s.aslot[i];
    v.key_of[slot] = key;
    v.slot_of[key] = slot;
    s.uslot[u] = slot;
    o.miss_key[i] = key;
    o.miss_slot[i] = slot;
    o.miss_victim[i] = s.avkey[i];
  }
  __syncthreads();
  for (int u = threadIdx.x; u < nU; u += RT) {
    if (s.uslot[u] >= 0) v.stamp[s.uslot[u]] = ps.step;  // CPU misses hold no slot
    o.u_slot[u] = s.uslot[u];
    o.u_hit[u] = s.hit[u];
  }
  if (o.cpu_key)
    for (int j = threadIdx.x; j < nCpu; j += RT) o.cpu_key[j] = layer * E + s.U[s.miss[nMiss + j]];
  // FFN entry table: hits first, then filled misses in ascending expert id (the fill order)
  for (int g = threadIdx.x; g < nHit + nMiss; g += RT) {
    const int miss = g < nHit ? -1 : g - nHit;
    const int u = miss < 0 ? s.hitl[g] : s.miss[miss];
    o.ent[g] = make_int4(s.uslot[u], s.cnt[s.U[u]], s.off[u], miss);
  }
  if (threadIdx.x == 0) {
    const int nn = n + nMiss;
    v.ctrl[CTRL_N] = nn < C ? nn : C;
    o.hdr[HDR_NU] = nU;
    o.hdr[HDR_NHIT] = nHit;
    o.hdr[HDR_NMISS] = nMiss;
    o.hdr[HDR_NCPU] = nCpu;
    o.hdr[HDR_LAYER] = layer;
    o.hdr[HDR_T] = T;
    o.hdr[HDR_STEP_LO] = (int)(ps.step & 0xffffffff);
    o.hdr[HDR_STEP_HI] = (int)(ps.step >> 32);
    const long long ns = ps.step + 1;
    v.ctrl[CTRL_STEP_LO] = (int)(ns & 0xffffffff);
    v.ctrl[CTRL_STEP_HI] = (int)(ns >> 32);
    v.stats[STAT_STEPS] += 1;
    v.stats[STAT_HITS] += (unsigned long long)nHit;
    v.stats[STAT_MISSES] += (unsigned long long)nAllMiss;
    v.stats[STAT_CPU] += (unsigned long long)nCpu;
    v.stats[STAT_BYTES] += (unsigned long long)nMiss * (unsigned long long)d.S;
    pt.nfill = nMiss;
    pt.ncpu = nCpu;
  }
  return true;
}

}  // namespace moe
