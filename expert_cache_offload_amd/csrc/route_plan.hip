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
#include "plan_core.h"

namespace moe {

struct RouteArgs {
  Dims d;
  Dev v;
  const uint16_t* x;   // [T][H] bf16
  const uint16_t* wr;  // [E][H] bf16
  int* out_idx;        // [T][K] or null
  float* out_w;        // [T][K] or null
  int layer;
  int T;
  int split_bc, split_bp;  // hybrid decode: CPU expert rate and PCIe fill rate (MB/s), 0: off
};

// NTOK: token bound of the step (1, 2, 4 or 8): the router loops are unrolled for it only,
// which keeps the kernel's code (fetched by every workgroup) small at one token.
template <int NTOK>
__global__ __launch_bounds__(RT) void route_plan_kernel(RouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, E = d.E, K = d.K, H = d.H;

  // ---------------- phase A: router logits, fp64 accumulation ----------------
  const int waves_total = gridDim.x * (RT / 64);
  for (int e = blockIdx.x * (RT / 64) + wave; e < E; e += waves_total) {
    double acc[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = 0.0;
    const uint16_t* wrow = a.wr + (size_t)e * H;
    // chunks of 8 elements per lane, RCH chunks' loads (weights and activations) in flight
    // before any arithmetic
    constexpr int RCH = 4;
    const int nch = (H + 511) / 512;  // H is a multiple of 256: the last chunk may be half
    for (int base = 0; base < nch; base += RCH) {
      uint4 w[RCH], xv[RCH][NTOK];
#pragma unroll
      for (int k = 0; k < RCH; ++k) {
        const int h = (base + k) * 512 + lane * 8;
        if (base + k < nch && h < H) {
          w[k] = *(const uint4*)(wrow + h);
#pragma unroll
          for (int t = 0; t < NTOK; ++t)
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
          for (int t = 0; t < NTOK; ++t) {
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
    for (int t = 0; t < NTOK; ++t) {
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
  const int layer = a.layer;
  unsigned char* p = smem;
  PlanLds s;
  p = plan_carve(d, p, s);
  double* s_z = (double*)p;     p += sizeof(double) * (size_t)kDecodeMaxTokens * E;
  int* s_tk_idx = (int*)p;      p += sizeof(int) * d.adec;
  float* s_tk_w = (float*)p;    p += sizeof(float) * d.adec;
  double* s_tk_z = (double*)p; p += sizeof(double) * d.adec;
  int* s_rt = (int*)p;          p += sizeof(int) * d.adec;   // token of each sorted row
  float* s_rw = (float*)p;                                   // routing weight of each row
  __shared__ PlanTmp pt;
  PlanState ps;

  // Every global read of the plan goes out together: the logits (the first RT of them into
  // registers), this layer's row of slot_of, the control words and the slots' (stamp, key);
  // the LDS stores follow.
  const double z0 = (int)threadIdx.x < T * E ? v.logits[threadIdx.x] : 0.0;
  plan_begin_load(d, v, layer, ps);
  if ((int)threadIdx.x < T * E) s_z[threadIdx.x] = (z0 == z0) ? z0 : -__builtin_huge_val();
  for (int i = threadIdx.x + RT; i < T * E; i += RT) {
    const double z = v.logits[i];
    s_z[i] = (z == z) ? z : -__builtin_huge_val();  // NaN ranks as -inf
  }
  plan_begin_store(d, s, ps);
  __syncthreads();

  // Top-k per token, ties to the lower expert id.  Counting ranks costs T * E^2 / RT compares
  // per thread; the wave argmax costs K rounds of a six-step shuffle chain per token a wave
  // holds.  Measured crossover: counting ranks is faster up to about T * E^2 = 8192 * K * (tokens
  // per wave) (one token of 128 or 256 experts: 16.7 / 24.4 against 23.4 / 25.6 us per launch),
  // the argmax beyond (four tokens of 256 experts: 42.6 against 64.5 us).
  if ((long long)T * E * E <= 8192ll * K * ((T + 3) / 4)) {
    // top-k per token by rank: rank(e) = #{e' : z_e' > z_e or (z_e' == z_e and e' < e)};
    // the experts of rank < K are the selection, in order.  P adjacent lanes count one
    // (token, expert) pair, each over 1/P of the experts, and add their counts (P = 2 measured
    // best at E = 128: one pair per thread of the workgroup at one token).
    {
      constexpr int P = 2;
      const int part = (E + P - 1) / P;
      for (int idx = threadIdx.x; idx < P * T * E; idx += RT) {
        const int i = idx / P, h = idx % P;
        const int t = i / E, e = i - t * E;
        const double z = s_z[i];
        const double* zt = s_z + (size_t)t * E;
        const int e_beg = h * part, e_end = e_beg + part < E ? e_beg + part : E;
        int rank = 0;
#pragma unroll 8
        for (int e2 = e_beg; e2 < e_end; ++e2) {  // 8 LDS reads in flight per step
          const double z2 = zt[e2];
          rank += (z2 > z) || (z2 == z && e2 < e);
        }
#pragma unroll
        for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o);  // the P lanes are adjacent
                                                                       // and all active
        if (h == 0 && rank < K) {
          s_tk_idx[t * K + rank] = e;
          s_tk_z[t * K + rank] = z;
        }
      }
    }
  } else {
    // one wave per token (tokens w, w + 4): K rounds of a wave-wide argmax over the token's
    // logits held in registers (lane l holds experts l, l + 64, ...), largest logit first, ties
    // to the lower expert id - the order of the ranks above.
    {
      constexpr int MAXC = 16;  // candidates per lane: E <= 1024
      const int C = (E + 63) / 64;
      for (int t = wave; t < T; t += RT / 64) {
        const double* zt = s_z + (size_t)t * E;
        double cz[MAXC];
        unsigned taken = 0;  // bit j: candidate j is selected or does not exist
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
          const int e = lane + 64 * j;
          const bool ok = j < C && e < E;
          cz[j] = ok ? zt[e] : 0.0;
          taken |= ok ? 0u : 1u << j;
        }
        for (int r = 0; r < K; ++r) {
          double bz = -__builtin_huge_val();
          int be = 0x7fffffff;  // no candidate: loses to any candidate, also to -inf logits
#pragma unroll
          for (int j = 0; j < MAXC; ++j) {
            const int e = lane + 64 * j;
            if (!((taken >> j) & 1u) && (cz[j] > bz || (cz[j] == bz && e < be))) {
              bz = cz[j];
              be = e;
            }
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) {
            const double oz = __shfl_xor(bz, off);
            const int oe = __shfl_xor(be, off);
            if (oz > bz || (oz == bz && oe < be)) {
              bz = oz;
              be = oe;
            }
          }
          // every lane holds the winner; its owner marks it taken
          if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);  // K <= E: be < E
          if (lane == 0) {
            s_tk_idx[t * K + r] = be;
            s_tk_z[t * K + r] = bz;
          }
        }
      }
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
    const int e = s_tk_idx[i];
    atomicAdd(&s.cnt[e], 1);
    v.tk_idx[i] = e;
    v.tk_w[i] = s_tk_w[i];
    if (a.out_idx) a.out_idx[i] = e;
    if (a.out_w) a.out_w[i] = s_tk_w[i];
  }
  __syncthreads();

  const PlanOut o = step_plan_out(v);
  const int nU = plan_dedup(d, o, s, pt);
  // per-expert assignment lists, ascending token inside an expert
  for (int i = threadIdx.x; i < A; i += RT) {
    const int e = s_tk_idx[i];
    int rank = 0;
    for (int q = 0; q < i; ++q) rank += (s_tk_idx[q] == e);
    const int pos = s.off[s.uidx[e]] + rank;
    v.perm[pos] = i;
    v.inv_pos[i] = pos;
    v.row_tok[pos] = i / K;
    v.row_w[pos] = s_tk_w[i];
    s_rt[pos] = i / K;
    s_rw[pos] = s_tk_w[i];
  }
  // hybrid decode: as soon as the split is known (before the victims are chosen), flag the
  // rows of the CPU experts (the combine skips them) and post the request to the host: CPU
  // experts, the step's rows, the activations, then the step value.  Posting ahead of the
  // victim search and the slot-table update lets the host start that much earlier.
  auto post = [&](int nfill, int q) {
    if (a.split_bc <= 0) return;
    __syncthreads();
    for (int r = threadIdx.x; r < A; r += RT) v.row_cpu[r] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < q; j += RT) {
      const int u = s.miss[nfill + j];
      for (int r = s.off[u]; r < s.off[u + 1]; ++r) v.row_cpu[r] = 1;
    }
    if (q > 0 && wave == 0) {
      HybMail* m = v.mail;
      for (int j = lane; j < q; j += 64) {
        const int u = s.miss[nfill + j];
        m->exp[j] = s.U[u];
        m->ntok[j] = s.off[u + 1] - s.off[u];
        m->row0[j] = s.off[u];
      }
      for (int r = lane; r < A; r += 64) {
        m->row_tok[r] = s_rt[r];
        m->row_w[r] = s_rw[r];
      }
      if (lane == 0) {
        m->layer = layer;
        m->T = T;
        m->q = q;
        m->K = K;
      }
      uint4* mx = (uint4*)((unsigned char*)m + mail_x_offset());
      const uint4* xs = (const uint4*)a.x;
      for (int i = lane; i < T * H / 8; i += 64) mx[i] = xs[i];
      __threadfence_system();
      if (lane == 0)
        __hip_atomic_store(&m->req, ps.step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __syncthreads();
  };
  plan_cache(d, v, o, layer, T, nU, s, ps, pt, nullptr, 0, a.split_bc, a.split_bp, post);
  if (threadIdx.x == 0)
    __hip_atomic_store(&v.ctrl[CTRL_TICKET], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t route_plan_lds_bytes(const Dims& d) {
  size_t b = plan_lds_bytes(d);
  b += sizeof(double) * (size_t)kDecodeMaxTokens * d.E;
  b += (sizeof(int) + sizeof(float) + sizeof(double)) * (size_t)d.adec;
  b += (sizeof(int) + sizeof(float)) * (size_t)d.adec;
  return (b + 15) & ~(size_t)15;
}

hipError_t launch_route_plan(const Dims& d, const Dev& v, const void* x, const void* wr,
                             int* out_idx, float* out_w, int layer, int T, int split_bc,
                             int split_bp, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  RouteArgs a{d, v, (const uint16_t*)x, (const uint16_t*)wr, out_idx, out_w, layer, T,
              split_bc, split_bp};
  int grid = (d.E + (RT / 64) - 1) / (RT / 64);
  const size_t lds = route_plan_lds_bytes(d);
  auto go = [&](auto kernel) -> hipError_t {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    return launch_timed(kernel, dim3(grid), dim3(RT), lds, s, e0, e1, a);
  };
  if (T <= 1) return go(route_plan_kernel<1>);
  if (T <= 2) return go(route_plan_kernel<2>);
  if (T <= 4) return go(route_plan_kernel<4>);
  return go(route_plan_kernel<kDecodeMaxTokens>);
}

}  // namespace moe
