// Route / top-k / dedup / classify / LRU for a layer step of many tokens (prefill chunks).
//
// The same plan as at decode (FreeToken paper summary, execution-layer paragraph: routing
// dedup, hit classification and LRU victim selection on the GPU with no host round trip),
// over a chunk whose routing union covers nearly every expert (same page, problem
// paragraph).  A fourth kernel plans the prefetch of the next layer (every expert of it, the
// step before protected from eviction), whose fills then overlap this layer's FFN
// ("FreeToken：在消费级 NVIDIA GPU 上进行 MoE 推理", "FreeToken 解决的问题": experts are
// streamed ahead so that transfers overlap compute).
//
// Gfx950 design, three launches:
//   router/top-k  - a workgroup owns 64 tokens: their router logits (fp64 accumulation of
//                   exact bf16 x bf16 products, operands staged through LDS in 64-wide
//                   contraction chunks, the next chunk's loads in flight) stay in LDS; one
//                   lane per token keeps its top-k list (ties to the lower expert id) and the
//                   renormalised softmax
//                   weights; an LDS bitmask per expert gives each (token, choice) its rank
//                   among the block's tokens routed to the same expert, and the block's
//                   per-expert counts;
//   plan          - one workgroup: per-expert totals, dedup, per-block row offsets (the
//                   expert-sorted order keeps tokens ascending inside an expert), then the
//                   shared classification / LRU / slot-table / entry-table code;
//   scatter       - every (token, choice) writes its expert-sorted row.
#include "plan_core.h"

namespace moe {

constexpr int PTOK = 64;        // tokens per router workgroup (one wave of top-k lanes)
constexpr int PKC = 64;         // contraction chunk staged in LDS
constexpr int PKP = PKC + 2;    // padded LDS row, bf16 elements (33 words: no bank conflicts)
constexpr int kMaxTopK = 16;

struct PrefRouteArgs {
  Dims d;
  Dev v;
  const uint16_t* x;   // [T][H] bf16
  const uint16_t* wr;  // [E][H] bf16
  int* out_idx;        // [T][K] or null
  float* out_w;        // [T][K] or null
  int layer;
  int T;
};

size_t prefill_router_lds_bytes(const Dims& d) {
  const int ept = (d.E + 15) / 16;
  const size_t stage = sizeof(uint16_t) * (size_t)(PTOK + 16 * ept) * PKP;
  const size_t logits = sizeof(double) * (size_t)PTOK * (d.E + 1);
  return stage > logits ? stage : logits;
}

// EPT experts per thread: experts tx, tx + 16, ... (E <= 16 * EPT); two tokens per thread, so
// eight waves share a 64-token block (two per SIMD).
constexpr int PRT = 512;  // threads of the router workgroup

template <int EPT>
__global__ __launch_bounds__(PRT) void prefill_router_topk_kernel(PrefRouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int E = d.E, H = d.H, K = d.K, T = a.T;
  const int t0 = blockIdx.x * PTOK;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // ty: tokens 2 ty, 2 ty + 1
  __shared__ unsigned long long s_mask[16 * EPT];  // bit t: token t0 + t chose the expert
  for (int e = threadIdx.x; e < 16 * EPT; e += PRT) s_mask[e] = 0ull;

  uint16_t* xs = (uint16_t*)smem;   // [PTOK][PKP]
  uint16_t* ws = xs + PTOK * PKP;   // [16 * EPT][PKP]
  double acc[2][EPT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0;

  // this thread's 16-byte chunks of a stage: activation row xr (a row past T reads row 0
  // and is zeroed when stored) and router rows xr + 64 q (q < WQ)
  constexpr int WQ = (16 * EPT * 8 + PRT - 1) / PRT;  // router chunks per thread
  const int xr = threadIdx.x >> 3, xc = (threadIdx.x & 7) * 8;
  const bool xval = t0 + xr < T;
  const uint16_t* xrow = a.x + (size_t)(xval ? t0 + xr : 0) * H + xc;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  u32x4 rx, rw[WQ];
  auto load_stage = [&](int k0) {
    rx = *(const u32x4*)(xrow + k0);
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int r = xr + 64 * q;
      rw[q] = r < E ? *(const u32x4*)(a.wr + (size_t)r * H + k0 + xc) : z4;
    }
  };
  load_stage(0);
  for (int k0 = 0; k0 < H; k0 += PKC) {
    __syncthreads();  // the previous stage's reads of the LDS tiles are done
    {
      const u32x4 q = xval ? rx : z4;
      uint32_t* dst = (uint32_t*)(xs + xr * PKP + xc);
      dst[0] = q[0]; dst[1] = q[1]; dst[2] = q[2]; dst[3] = q[3];
    }
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int r = xr + 64 * q;
      if (r < 16 * EPT) {
        uint32_t* dst = (uint32_t*)(ws + r * PKP + xc);
        dst[0] = rw[q][0]; dst[1] = rw[q][1]; dst[2] = rw[q][2]; dst[3] = rw[q][3];
      }
    }
    __syncthreads();
    load_stage(k0 + PKC < H ? k0 + PKC : k0);  // the next stage's loads overlap the FMAs
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 4
    for (int kk = 0; kk < PKC; kk += 2) {
      double xa[2], xb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t w2 = *(const uint32_t*)(xs + (ty * 2 + i) * PKP + kk);
        xa[i] = (double)bf16_lo(w2);
        xb[i] = (double)bf16_hi(w2);
      }
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int e = tx + 16 * j;
        if (e < E) {
          const uint32_t w2 = *(const uint32_t*)(ws + e * PKP + kk);
          const double wa = (double)bf16_lo(w2), wb = (double)bf16_hi(w2);
#pragma unroll
          for (int i = 0; i < 2; ++i) {  // the product is exact in fp64: one rounding per add
            acc[i][j] = __builtin_fma(xa[i], wa, acc[i][j]);
            acc[i][j] = __builtin_fma(xb[i], wb, acc[i][j]);
          }
        }
      }
    }
  }
  __syncthreads();

  // logits tile in LDS (the staging area is free after the last barrier); NaN ranks as -inf
  double* sz = (double*)smem;  // [PTOK][E + 1]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tx + 16 * j;
      if (e < E) {
        const double z = acc[i][j];
        sz[(ty * 2 + i) * (E + 1) + e] = (z == z) ? z : -__builtin_huge_val();
      }
    }
  __syncthreads();

  // top-k: lane t of wave 0 scans its token's logits in ascending expert order and keeps
  // a list sorted by (logit desc, expert asc)
  double bz[kMaxTopK];
  int bi[kMaxTopK];
  const int t = threadIdx.x;
  const bool live = t < PTOK && t0 + t < T;
  if (live) {
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) {
      bz[q] = 0.0;
      bi[q] = -1;
    }
    const double* zt = sz + t * (E + 1);
    for (int e = 0; e < E; ++e) {
      double zc = zt[e];
      int ic = e;
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q) {
        if (q < K) {
          const bool better = bi[q] < 0 || zc > bz[q] || (zc == bz[q] && ic < bi[q]);
          if (better) {
            const double tz = bz[q];
            const int ti = bi[q];
            bz[q] = zc;
            bi[q] = ic;
            zc = tz;
            ic = ti;
          }
        }
      }
    }
    // renormalised softmax over the selected logits (differences in fp64, exp in fp32)
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q)
      if (q < K) sum += expf((float)(bz[q] - bz[0]));
    const size_t base = (size_t)(t0 + t) * K;
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) {
      if (q < K) {
        const float w = expf((float)(bz[q] - bz[0])) / sum;
        v.tk_idx[base + q] = bi[q];
        v.tk_w[base + q] = w;
        if (a.out_idx) a.out_idx[base + q] = bi[q];
        if (a.out_w) a.out_w[base + q] = w;
        atomicOr(&s_mask[bi[q]], 1ull << t);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PRT)
    v.blk_cnt[(size_t)blockIdx.x * E + e] = __popcll(s_mask[e]);
  if (live) {
    const unsigned long long below = t == 0 ? 0ull : (~0ull >> (64 - t));
    const size_t base = (size_t)(t0 + t) * K;
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q)
      if (q < K) v.brank[base + q] = __popcll(s_mask[bi[q]] & below);
  }
}

__global__ __launch_bounds__(RT) void prefill_plan_kernel(PrefRouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int E = d.E;
  const int nblk = (a.T + PTOK - 1) / PTOK;
  PlanLds s;
  plan_carve(d, smem, s);
  __shared__ PlanTmp pt;
  PlanState ps;
  plan_begin(d, v, a.layer, s, ps);
  __syncthreads();
  constexpr int BB = 16;  // block counts loaded per batch
  for (int e = threadIdx.x; e < E; e += RT) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += BB) {
      int c[BB];
#pragma unroll
      for (int q = 0; q < BB; ++q) c[q] = b0 + q < nblk ? v.blk_cnt[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < BB; ++q) run += c[q];
    }
    s.cnt[e] = run;
  }
  __syncthreads();
  const PlanOut o = step_plan_out(v);
  const int nU = plan_dedup(d, o, s, pt);
  // first expert-sorted row of each (block, expert): tokens stay ascending inside an expert
  for (int e = threadIdx.x; e < E; e += RT) {
    if (s.uidx[e] < 0) continue;
    int run = s.off[s.uidx[e]];
    for (int b0 = 0; b0 < nblk; b0 += BB) {
      int c[BB];
#pragma unroll
      for (int q = 0; q < BB; ++q) c[q] = b0 + q < nblk ? v.blk_cnt[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < BB; ++q) {
        if (b0 + q < nblk) v.blk_off[(size_t)(b0 + q) * E + e] = run;
        run += c[q];
      }
    }
  }
  plan_cache(d, v, o, a.layer, a.T, nU, s, ps, pt);
}

// Prefetch plan of layer a.layer: a plan step whose distinct set is every expert of the layer
// (one workgroup), written to the prefetch plan area; the slots of the step plan just before
// it (whose FFN may still be reading them) are protected from eviction.
__global__ __launch_bounds__(RT) void prefetch_plan_kernel(PrefRouteArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  PlanLds s;
  plan_carve(d, smem, s);
  __shared__ PlanTmp pt;
  PlanState ps;
  plan_begin(d, v, a.layer, s, ps);
  __syncthreads();
  for (int e = threadIdx.x; e < d.E; e += RT) s.cnt[e] = 1;
  __syncthreads();
  const PlanOut o = prefetch_plan_out(v, d.E);
  const int nU = plan_dedup(d, o, s, pt);
  plan_cache(d, v, o, a.layer, 0, nU, s, ps, pt, v.u_slot, v.hdr[HDR_NU]);
}

__global__ __launch_bounds__(RT) void prefill_scatter_kernel(PrefRouteArgs a) {
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int i = blockIdx.x * RT + threadIdx.x;
  if (i >= a.T * d.K) return;
  const int t = i / d.K;
  const int e = v.tk_idx[i];
  const int pos = v.blk_off[(size_t)(t / PTOK) * d.E + e] + v.brank[i];
  v.perm[pos] = i;
  v.inv_pos[i] = pos;
  v.row_tok[pos] = t;
  v.row_w[pos] = v.tk_w[i];
}

template <class Kern>
static hipError_t set_lds(Kern k, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <int EPT>
static hipError_t launch_router(const PrefRouteArgs& a, hipStream_t s, hipEvent_t e0) {
  const size_t lds = prefill_router_lds_bytes(a.d);
  hipError_t e = set_lds(prefill_router_topk_kernel<EPT>, lds);
  if (e != hipSuccess) return e;
  return launch_timed(prefill_router_topk_kernel<EPT>, dim3((a.T + PTOK - 1) / PTOK), dim3(PRT),
                      lds, s, e0, nullptr, a);
}

bool prefill_route_supported(const Dims& d) { return d.E <= 256 && d.K <= kMaxTopK; }

hipError_t launch_prefetch_plan(const Dims& d, const Dev& v, int layer, hipStream_t s) {
  PrefRouteArgs a{d, v, nullptr, nullptr, nullptr, nullptr, layer, 0};
  const size_t lds = plan_lds_bytes(d);
  hipError_t e = set_lds(prefetch_plan_kernel, lds);
  if (e != hipSuccess) return e;
  return launch_timed(prefetch_plan_kernel, dim3(1), dim3(RT), lds, s, nullptr, nullptr, a);
}

hipError_t launch_route_prefill(const Dims& d, const Dev& v, const void* x, const void* wr,
                                int* out_idx, float* out_w, int layer, int T, hipStream_t s,
                                hipEvent_t e0, hipEvent_t e1) {
  PrefRouteArgs a{d, v, (const uint16_t*)x, (const uint16_t*)wr, out_idx, out_w, layer, T};
  const int ept = (d.E + 15) / 16;
  hipError_t e = ept <= 1 ? launch_router<1>(a, s, e0)
               : ept <= 2 ? launch_router<2>(a, s, e0)
               : ept <= 4 ? launch_router<4>(a, s, e0)
               : ept <= 8 ? launch_router<8>(a, s, e0)
                          : launch_router<16>(a, s, e0);
  if (e != hipSuccess) return e;
  const size_t lds = plan_lds_bytes(d);
  e = set_lds(prefill_plan_kernel, lds);
  if (e != hipSuccess) return e;
  e = launch_timed(prefill_plan_kernel, dim3(1), dim3(RT), lds, s, nullptr, nullptr, a);
  if (e != hipSuccess) return e;
  return launch_timed(prefill_scatter_kernel, dim3((T * d.K + RT - 1) / RT), dim3(RT), 0, s,
                      nullptr, e1, a);
}

}  // namespace moe
