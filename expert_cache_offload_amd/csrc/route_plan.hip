// Fused route / top-k / dedup / classify / LRU kernel for one MoE layer step.
//
// Follows the FreeToken paper summary (agihunt.info, arXiv 2608.16157), execution-layer
// paragraph: one GPU kernel per layer does routing dedup, hit classification and LRU
// victim selection, with no host round trip.  The cache is the one of the
// memory-architecture paragraph: a single slot cache shared by all MoE layers, keyed by
// (layer, expert).  Replacement is a global LRU (same page, attribution paragraph;
// "FreeToken vs vLLM on one RTX 3090", "FreeToken exploits MoE sparsity").
//
// Gfx950 design: every workgroup computes router logits for a slice of the experts
// (one expert row per wave, fp64 accumulation of exact bf16 x bf16 products so near
// ties are ordered as in exact arithmetic); the last workgroup to arrive (an
// agent-scope ticket) then runs the whole plan in LDS:
//   top-k per token by rank counting over the LDS-resident logits (ties to the lower
//   expert id; every (token, expert) pair ranked in parallel) and renormalised softmax;
//   dedup by an LDS histogram and a wave-ballot / popcount prefix that yields the
//   distinct experts U already ascending;
//   hit/miss classification against slot_of;
//   LRU victims as the `need` smallest (stamp, key) among occupied slots not in U, found
//   in rounds of "oldest remaining stamp" over the LDS-resident stamps (one round per
//   distinct stamp taken: a step stamps all its experts alike);
//   slot-table update and the per-expert token lists consumed by the FFN.
// The rule reproduced (free slots [n, C) first in ascending order, then victims in
// (stamp, key) order; misses taken in ascending expert id; all of U stamped with the
// step counter) is the LRU reading documented with the header.
#include "moe_dev.h"

namespace moe {

constexpr int RT = 256;  // threads per route workgroup (4 waves)
constexpr int kSlotsPerThread = kMaxSlots / RT;

struct RouteArgs {
  Dims d;
  Dev v;
  const uint16_t* x;   // [T][H] bf16
  const uint16_t* wr;  // [E][H] bf16
  int* out_idx;        // [T][K] or null
  float* out_w;        // [T][K] or null
  int layer;
  int T;
};

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

__device__ uint64_t block_min_u64(uint64_t v, uint64_t* s_tmp) {
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

__global__ __launch_bounds__(RT) void route_plan_kernel(RouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, E = d.E, K = d.K, H = d.H;

  // ---------------- phase A: router logits, fp64 accumulation ----------------
  const int waves_total = gridDim.x * (RT / 64);
  for (int e = blockIdx.x * (RT / 64) + wave; e < E; e += waves_total) {
    double acc[kDecodeMaxTokens];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] = 0.0;
    const uint16_t* wrow = a.wr + (size_t)e * H;
    // chunks of 8 elements per lane, RCH chunks' loads (weights and activations) in flight
    // before any arithmetic
    constexpr int RCH = 4;
    const int nch = (H + 511) / 512;  // H is a multiple of 256: the last chunk may be half
    for (int base = 0; base < nch; base += RCH) {
      uint4 w[RCH], xv[RCH][kDecodeMaxTokens];
#pragma unroll
      for (int k = 0; k < RCH; ++k) {
        const int h = (base + k) * 512 + lane * 8;
        if (base + k < nch && h < H) {
          w[k] = *(const uint4*)(wrow + h);
#pragma unroll
          for (int t = 0; t < kDecodeMaxTokens; ++t)
            if (t < T) xv[k][t] = *(const uint4*)(a.x + (size_t)t * H + h);
        }
      }
#pragma unroll
      for (int k = 0; k < RCH; ++k) {
        if (base + k < nch && (base + k) * 512 + lane * 8 < H) {
          const float wf[8] = {bf16_lo(w[k].x), bf16_hi(w[k].x), bf16_lo(w[k].y),
                               bf16_hi(w[k].y), bf16_lo(w[k].z), bf16_hi(w[k].z),
                               bf16_lo(w[k].w), bf16_hi(w[k].w)};
#pragma unroll
          for (int t = 0; t < kDecodeMaxTokens; ++t) {
            if (t < T) {
              const uint4 q = xv[k][t];
              const float xf[8] = {bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y),
                                   bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w)};
              double s = 0.0;
#pragma unroll
              for (int c = 0; c < 8; ++c) s += (double)(wf[c] * xf[c]);  // exact fp32 product
              acc[t] += s;
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) {
      if (t < T) {
        double s = acc[t];
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) v.logits[(size_t)t * E + e] = s;
      }
    }
  }

  // ---------------- ticket: the last workgroup plans ----------------
  // Each wave's logit stores complete (workgroup-scope release: a wait, no cache action);
  // one agent-scope release per workgroup publishes them before its ticket, and the last
  // workgroup's single acquire makes every workgroup's logits visible to it.
  __shared__ int s_last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = __hip_atomic_fetch_add(&v.ctrl[CTRL_TICKET], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // ---------------- phase B (one workgroup) ----------------
  const int A = T * K;
  const int umax = d.umax;
  const int layer = a.layer;
  // LDS carve-up
  unsigned char* p = smem;
  uint64_t* s_comp = (uint64_t*)p;  p += sizeof(uint64_t) * d.max_capacity;
  double* s_z = (double*)p;         p += sizeof(double) * (size_t)d.max_tokens * E;
  int* s_cnt = (int*)p;             p += sizeof(int) * E;
  int* s_uidx = (int*)p;            p += sizeof(int) * E;
  int* s_srow = (int*)p;            p += sizeof(int) * E;
  int* s_tk_idx = (int*)p;          p += sizeof(int) * d.amax;
  float* s_tk_w = (float*)p;        p += sizeof(float) * d.amax;
  double* s_tk_z = (double*)p;      p += sizeof(double) * d.amax;
  int* s_U = (int*)p;               p += sizeof(int) * umax;
  int* s_off = (int*)p;             p += sizeof(int) * (umax + 1);
  int* s_uslot = (int*)p;           p += sizeof(int) * umax;
  int* s_hit = (int*)p;             p += sizeof(int) * umax;
  int* s_miss = (int*)p;            p += sizeof(int) * umax;
  int* s_vict = (int*)p;            p += sizeof(int) * umax;
  int* s_vkey = (int*)p;            p += sizeof(int) * umax;
  int* s_grp = (int*)p;             p += sizeof(int) * umax;
  int* s_sorted = (int*)p;          p += sizeof(int) * umax;
  int* s_aslot = (int*)p;           p += sizeof(int) * umax;
  int* s_avkey = (int*)p;           p += sizeof(int) * umax;
  int* s_hitl = (int*)p;            p += sizeof(int) * umax;
  __shared__ int s_tmp[8];
  __shared__ uint64_t s_tmp64[8];
  __shared__ int s_g;

  // Every global read of the plan goes out together: the logits, this layer's row of
  // slot_of and the control words; the occupied slots' (stamp, key) follow as soon as the
  // occupancy is known and stay in registers until the victim search.
  for (int i = threadIdx.x; i < T * E; i += RT) {
    const double z = v.logits[i];
    s_z[i] = (z == z) ? z : -__builtin_huge_val();  // NaN ranks as -inf
  }
  for (int e = threadIdx.x; e < E; e += RT) {
    s_cnt[e] = 0;
    s_uidx[e] = -1;
    s_srow[e] = v.slot_of[layer * E + e];
  }
  const int n = v.ctrl[CTRL_N];
  const int C = v.ctrl[CTRL_C];
  const long long step = (long long)(unsigned)v.ctrl[CTRL_STEP_LO] |
                         ((long long)v.ctrl[CTRL_STEP_HI] << 32);
  uint32_t r_st[kSlotsPerThread], r_key[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int i = (int)threadIdx.x + j * RT;
    r_st[j] = 0xffffffffu;
    r_key[j] = 0xffffffffu;
    if (i < n) {
      r_st[j] = (uint32_t)v.stamp[i];
      r_key[j] = (uint32_t)v.key_of[i];
    }
  }
  __syncthreads();

  // top-k per token by rank: rank(e) = #{e' : z_e' > z_e or (z_e' == z_e and e' < e)};
  // the experts of rank < K are the selection, in order.
  for (int i = threadIdx.x; i < T * E; i += RT) {
    const int t = i / E, e = i - t * E;
    const double z = s_z[i];
    const double* zt = s_z + (size_t)t * E;
    int rank = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const double z2 = zt[e2];
      rank += (z2 > z) || (z2 == z && e2 < e);
    }
    if (rank < K) {
      s_tk_idx[t * K + rank] = e;
      s_tk_z[t * K + rank] = z;
    }
  }
  __syncthreads();
  // renormalised softmax over the selected logits (differences in fp64, exp in fp32)
  for (int i = threadIdx.x; i < A; i += RT) {
    const int t = i / K;
    const double z0 = s_tk_z[t * K];
    float sum = 0.f;
    for (int jj = 0; jj < K; ++jj) sum += expf((float)(s_tk_z[t * K + jj] - z0));
    s_tk_w[i] = expf((float)(s_tk_z[i] - z0)) / sum;
  }
  __syncthreads();

  for (int i = threadIdx.x; i < A; i += RT) {
    int e = s_tk_idx[i];
    atomicAdd(&s_cnt[e], 1);
    v.tk_idx[i] = e;
    v.tk_w[i] = s_tk_w[i];
    if (a.out_idx) a.out_idx[i] = e;
    if (a.out_w) a.out_w[i] = s_tk_w[i];
  }
  __syncthreads();

  // dedup: distinct experts ascending via ballot / popcount prefix
  const int nU = block_compact(
      E, [&](int e) { return s_cnt[e] > 0; },
      [&](int e, int pos) {
        s_U[pos] = e;
        s_uidx[e] = pos;
        v.U[pos] = e;
      },
      s_tmp);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int u = 0; u < nU; ++u) {
      s_off[u] = run;
      v.offset[u] = run;
      int c = s_cnt[s_U[u]];
      v.count[u] = c;
      run += c;
    }
    s_off[nU] = run;
    v.offset[nU] = run;
  }
  // classification against the layer's slot_of row (in LDS)
  for (int u = threadIdx.x; u < nU; u += RT) {
    int sl = s_srow[s_U[u]];
    s_uslot[u] = sl;
    s_hit[u] = sl >= 0 ? 1 : 0;
  }
  __syncthreads();
  // per-expert assignment lists, ascending token inside an expert
  for (int i = threadIdx.x; i < A; i += RT) {
    int e = s_tk_idx[i];
    int rank = 0;
    for (int q = 0; q < i; ++q) rank += (s_tk_idx[q] == e);
    int pos = s_off[s_uidx[e]] + rank;
    v.perm[pos] = i;
    v.inv_pos[i] = pos;
    v.row_tok[pos] = i / K;
    v.row_w[pos] = s_tk_w[i];
  }
  const int nHit = block_compact(
      nU, [&](int u) { return s_hit[u] != 0; },
      [&](int u, int pos) {
        v.hit_list[pos] = u;
        s_hitl[pos] = u;
      },
      s_tmp);
  const int nMiss = block_compact(
      nU, [&](int u) { return s_hit[u] == 0; },
      [&](int u, int pos) {
        s_miss[pos] = u;
        v.miss_list[pos] = u;
      },
      s_tmp);

  // LRU victims: the `need` smallest (stamp, key) among occupied slots not used this step
  const int nfree = C - n;
  const int need = nMiss > nfree ? nMiss - nfree : 0;
  __shared__ int s_err;
  if (threadIdx.x == 0) s_err = 0;
  if (need > 0) {
    const uint64_t NONE = ~0ull;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int i = (int)threadIdx.x + j * RT;
      if (i < n) s_comp[i] = ((uint64_t)r_st[j] << 32) | r_key[j];
    }
    __syncthreads();
    for (int u = threadIdx.x; u < nU; u += RT)  // keys of this step are never victims
      if (s_hit[u]) s_comp[s_uslot[u]] = NONE;
    __syncthreads();
    int got = 0;
    for (int round = 0; round < need && got < need; ++round) {
      uint64_t m = NONE;
      for (int i = threadIdx.x; i < n; i += RT) m = s_comp[i] < m ? s_comp[i] : m;
      m = block_min_u64(m, s_tmp64);
      if (m == NONE) {  // fewer evictable slots than misses: capacity floor violated
        if (threadIdx.x == 0) s_err = 1;
        break;
      }
      const uint32_t st = (uint32_t)(m >> 32);
      if (threadIdx.x == 0) s_g = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += RT) {
        uint64_t c = s_comp[i];
        if (c != NONE && (uint32_t)(c >> 32) == st) {
          int q = atomicAdd(&s_g, 1);
          if (q < umax) s_grp[q] = i;
        }
      }
      __syncthreads();
      const int g = s_g < umax ? s_g : umax;
      for (int q = threadIdx.x; q < g; q += RT) {  // order the group by key
        uint32_t kq = (uint32_t)s_comp[s_grp[q]];
        int rank = 0;
        for (int r = 0; r < g; ++r) rank += ((uint32_t)s_comp[s_grp[r]] < kq);
        s_sorted[rank] = s_grp[q];
      }
      __syncthreads();
      const int take = g < need - got ? g : need - got;
      for (int q = threadIdx.x; q < take; q += RT) {
        s_vict[got + q] = s_sorted[q];
        s_vkey[got + q] = (int)(uint32_t)s_comp[s_sorted[q]];
        s_comp[s_sorted[q]] = NONE;
      }
      got += take;
      __syncthreads();
    }
  }
  __syncthreads();
  if (s_err) {
    if (threadIdx.x == 0) {
      atomicOr(&v.ctrl[CTRL_ERR], ERR_CAPACITY);
      v.hdr[HDR_NU] = 0;
      v.hdr[HDR_NHIT] = 0;
      v.hdr[HDR_NMISS] = 0;
      __hip_atomic_store(&v.ctrl[CTRL_TICKET], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // slot assignment: free slots n, n+1, ... first, then victims in LRU order
  for (int i = threadIdx.x; i < nMiss; i += RT) {
    int slot = i < nfree ? n + i : s_vict[i - nfree];
    s_aslot[i] = slot;
    s_avkey[i] = i < nfree ? -1 : s_vkey[i - nfree];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nMiss; i += RT)
    if (s_avkey[i] >= 0) v.slot_of[s_avkey[i]] = -1;
  __syncthreads();
  for (int i = threadIdx.x; i < nMiss; i += RT) {
    int u = s_miss[i];
    int key = layer * E + s_U[u];
    int slot = s_aslot[i];
    v.key_of[slot] = key;
    v.slot_of[key] = slot;
    s_uslot[u] = slot;
    v.miss_key[i] = key;
    v.miss_slot[i] = slot;
    v.miss_victim[i] = s_avkey[i];
  }
  __syncthreads();
  for (int u = threadIdx.x; u < nU; u += RT) {
    v.stamp[s_uslot[u]] = (int)step;
    v.u_slot[u] = s_uslot[u];
    v.u_hit[u] = s_hit[u];
  }
  // FFN entry table: hits first, then misses in ascending expert id (the fill order)
  for (int g = threadIdx.x; g < nU; g += RT) {
    const int miss = g < nHit ? -1 : g - nHit;
    const int u = miss < 0 ? s_hitl[g] : s_miss[miss];
    v.ent[g] = make_int4(s_uslot[u], s_cnt[s_U[u]], s_off[u], miss);
  }
  if (threadIdx.x == 0) {
    int nn = n + nMiss;
    v.ctrl[CTRL_N] = nn < C ? nn : C;
    v.hdr[HDR_NU] = nU;
    v.hdr[HDR_NHIT] = nHit;
    v.hdr[HDR_NMISS] = nMiss;
    v.hdr[HDR_LAYER] = layer;
    v.hdr[HDR_T] = T;
    v.hdr[HDR_STEP_LO] = (int)(step & 0xffffffff);
    v.hdr[HDR_STEP_HI] = (int)(step >> 32);
    long long ns = step + 1;
    v.ctrl[CTRL_STEP_LO] = (int)(ns & 0xffffffff);
    v.ctrl[CTRL_STEP_HI] = (int)(ns >> 32);
    v.stats[STAT_STEPS] += 1;
    v.stats[STAT_HITS] += (unsigned long long)nHit;
    v.stats[STAT_MISSES] += (unsigned long long)nMiss;
    v.stats[STAT_BYTES] += (unsigned long long)nMiss * (unsigned long long)d.S;
    __hip_atomic_store(&v.ctrl[CTRL_TICKET], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

size_t route_plan_lds_bytes(const Dims& d) {
  size_t b = sizeof(uint64_t) * (size_t)d.max_capacity;
  b += sizeof(double) * (size_t)d.max_tokens * d.E;
  b += sizeof(int) * 3 * (size_t)d.E;
  b += (sizeof(int) + sizeof(float) + sizeof(double)) * (size_t)d.amax;
  b += sizeof(int) * (size_t)(12 * d.umax + 1);
  return (b + 15) & ~(size_t)15;
}

hipError_t launch_route_plan(const Dims& d, const Dev& v, const void* x, const void* wr,
                             int* out_idx, float* out_w, int layer, int T, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  RouteArgs a{d, v, (const uint16_t*)x, (const uint16_t*)wr, out_idx, out_w, layer, T};
  int grid = (d.E + (RT / 64) - 1) / (RT / 64);
  return launch_timed(route_plan_kernel, dim3(grid), dim3(RT), route_plan_lds_bytes(d), s, e0, e1,
                      a);
}

}  // namespace moe
