// SwiGLU expert FFN at decode: a weight-streaming GEMV over the cached expert blobs.
//
// The pages give no expert form; the SwiGLU expert (FFN_e(x) = Wd (silu(Wg x) * (Wu x)))
// is the one this library computes, summed over the top-k experts with the renormalised
// routing weights (plus a GPU-resident shared expert with weight 1 when the model has
// one).  Selected experts run on the GPU once fetched ("FreeToken vs vLLM on one RTX
// 3090", "FreeToken exploits MoE sparsity"); hit experts run first and each group of
// misses runs as soon as its fill has landed ("FreeToken：在消费级 NVIDIA GPU 上进行 MoE
// 推理", "FreeToken 解决的问题": one group computes while the next transfers).
//
// Gfx950 design: decode is HBM-bound (about one FLOP per weight byte), so every weight
// byte is read once, coalesced, 16 bytes per lane.  A workgroup owns R consecutive
// intermediate rows of one expert: it streams the gate|up rows (contiguous 2H elements
// per row in the blob), forms a = silu(g) * u * w_token for each token routed to the
// expert, then streams the same R rows of the stored down-projection transpose WdT and
// writes an fp32 partial output row per (token, row block).  Every expert is read once
// per step whatever number of tokens use it (cross-request sharing at batch > 1).
// A combine kernel adds the partial rows of each token in a fixed order (deterministic)
// and rounds to bf16.  Weight formats: bf16, fp8 e4m3fn with fp32 scale per 1x128 block,
// MXFP4 (e2m1 with e8m0 scale per 32), decoded with gfx950's packed conversions.
#include "moe_dev.h"

namespace moe {

constexpr int FT = 256;  // threads per FFN workgroup (4 waves)

struct FfnArgs {
  Dims d;
  Dev v;
  const uint16_t* x;  // [T][H] bf16
  const unsigned char* arena;
  const unsigned char* shared_blob;
  int mode;  // 0: hit experts, 1: miss group `group` of `ngroups`, 2: shared expert
  int group;
  int ngroups;
  int T;
};

// ---- format helpers -------------------------------------------------------------
template <int FMT>
struct Fmt;

template <>
struct Fmt<FMT_BF16> {
  static constexpr int EPL = 8;    // elements per 16 bytes
  static constexpr int DCOLS = 8;  // down-projection columns per thread load
  __device__ static size_t gu_row_bytes(int H) { return (size_t)2 * H * 2; }
  __device__ static size_t d_row_bytes(int H) { return (size_t)H * 2; }
  __device__ static size_t d_base(int H, int I) { return (size_t)4 * I * H; }
  __device__ static void unpack(uint4 w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
  __device__ static void load_d(const unsigned char* p, float* f) { unpack(*(const uint4*)p, f); }
};

__device__ __forceinline__ void fp8x4(uint32_t v, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

template <>
struct Fmt<FMT_FP8> {
  static constexpr int EPL = 16;
  static constexpr int DCOLS = 16;
  __device__ static size_t gu_row_bytes(int H) { return (size_t)2 * H; }
  __device__ static size_t d_row_bytes(int H) { return (size_t)H; }
  __device__ static size_t d_base(int H, int I) { return (size_t)2 * I * H; }
  __device__ static void unpack(uint4 w, float* f) {
    fp8x4(w.x, f); fp8x4(w.y, f + 4); fp8x4(w.z, f + 8); fp8x4(w.w, f + 12);
  }
  __device__ static void load_d(const unsigned char* p, float* f) { unpack(*(const uint4*)p, f); }
};

__device__ __forceinline__ void fp4x8(uint32_t v, float* f) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

template <>
struct Fmt<FMT_MXFP4> {
  static constexpr int EPL = 32;
  static constexpr int DCOLS = 16;  // 8-byte loads keep the accumulators in registers
  __device__ static size_t gu_row_bytes(int H) { return (size_t)H; }
  __device__ static size_t d_row_bytes(int H) { return (size_t)H / 2; }
  __device__ static size_t d_base(int H, int I) { return (size_t)I * H; }
  __device__ static void unpack(uint4 w, float* f) {
    fp4x8(w.x, f); fp4x8(w.y, f + 8); fp4x8(w.z, f + 16); fp4x8(w.w, f + 24);
  }
  __device__ static void load_d(const unsigned char* p, float* f) {
    const uint2 w = *(const uint2*)p;
    fp4x8(w.x, f);
    fp4x8(w.y, f + 8);
  }
};

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) { return __uint_as_float(c << 23); }

// Scale of the gate (g=0) or up (g=1) row i at contraction position xp.
template <int FMT>
__device__ __forceinline__ float gu_scale(const unsigned char* blob, int H, int I, int i, int g,
                                          int xp) {
  if constexpr (FMT == FMT_FP8) {
    const float* s = (const float*)(blob + (size_t)3 * I * H);
    return s[(size_t)(2 * i + g) * (H / 128) + xp / 128];
  } else if constexpr (FMT == FMT_MXFP4) {
    const unsigned char* s = blob + (size_t)3 * I * H / 2;
    return e8m0_to_f32(s[(size_t)(2 * i + g) * (H / 32) + xp / 32]);
  } else {
    return 1.0f;
  }
}

// Scale of the down-projection block holding row i at column h.
template <int FMT>
__device__ __forceinline__ float d_scale(const unsigned char* blob, int H, int I, int i, int h) {
  if constexpr (FMT == FMT_FP8) {
    const float* s = (const float*)(blob + (size_t)3 * I * H + (size_t)4 * 2 * I * (H / 128));
    return s[(size_t)(i / 128) * H + h];
  } else if constexpr (FMT == FMT_MXFP4) {
    const unsigned char* s = blob + (size_t)3 * I * H / 2 + (size_t)2 * I * (H / 32);
    return e8m0_to_f32(s[(size_t)(i / 32) * H + h]);
  } else {
    return 1.0f;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int FMT, int NTOK>
__global__ __launch_bounds__(FT) void ffn_decode_kernel(FfnArgs a) {
  using F = Fmt<FMT>;
  constexpr int EPL = F::EPL;
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int H = d.H, I = d.I, R = d.R;
  const int j = blockIdx.x / d.nR, rb = blockIdx.x % d.nR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ int s_tok[NTOK];
  __shared__ float s_w[NTOK];
  __shared__ int s_prow[NTOK];
  int u = -1, ntok;
  const unsigned char* blob;
  if (a.mode == 2) {
    if (j > 0) return;
    blob = a.shared_blob;
    ntok = a.T;
  } else {
    int n0, n1;
    const int* list;
    if (a.mode == 0) {
      list = v.hit_list;
      n0 = 0;
      n1 = v.hdr[HDR_NHIT];
    } else {
      const int m = v.hdr[HDR_NMISS];
      list = v.miss_list;
      n0 = (int)((long long)a.group * m / a.ngroups);
      n1 = (int)((long long)(a.group + 1) * m / a.ngroups);
    }
    if (j >= n1 - n0) return;
    u = list[n0 + j];
    blob = a.arena + (size_t)v.u_slot[u] * (size_t)d.S;
    ntok = v.count[u];
  }
  if (ntok > NTOK) ntok = NTOK;  // host picks NTOK >= T
  if ((int)threadIdx.x < ntok) {
    const int q = threadIdx.x;
    if (u >= 0) {
      const int pos = v.offset[u] + q;
      const int asg = v.perm[pos];
      s_tok[q] = asg / d.K;
      s_w[q] = v.tk_w[asg];
      s_prow[q] = pos;
    } else {
      s_tok[q] = q;
      s_w[q] = 1.0f;
      s_prow[q] = q;
    }
  }
  __syncthreads();

  // token activations -> LDS (bf16)
  uint16_t* xs = (uint16_t*)smem;  // [NTOK][H]
  float* as = (float*)(smem + (size_t)NTOK * H * 2);  // [NTOK][R]
  for (int q = 0; q < ntok; ++q) {
    const uint4* src = (const uint4*)(a.x + (size_t)s_tok[q] * H);
    uint4* dst = (uint4*)(xs + (size_t)q * H);
    for (int c = threadIdx.x; c < H / 8; c += FT) dst[c] = src[c];
  }
  __syncthreads();

  const int r0 = rb * R;
  // ---- gate / up: one wave per row, the row's 2H elements spread over the lanes ----
  const int nq = 2 * H / EPL;
  for (int rl = wave; rl < R; rl += FT / 64) {
    const int i = r0 + rl;
    const uint4* row = (const uint4*)(blob + (size_t)i * F::gu_row_bytes(H));
    float accg[NTOK], accu[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) accg[t] = accu[t] = 0.f;
#pragma unroll 4
    for (int q = lane; q < nq; q += 64) {
      const uint4 w = row[q];
      const int p = q * EPL;
      const bool isg = p < H;
      const int xp = isg ? p : p - H;
      float wf[EPL];
      F::unpack(w, wf);
      const float sc = gu_scale<FMT>(blob, H, I, i, isg ? 0 : 1, xp);
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        if (t < ntok) {
          const uint4* xv = (const uint4*)(xs + (size_t)t * H + xp);
          float dsum = 0.f;
#pragma unroll
          for (int c8 = 0; c8 < EPL / 8; ++c8) {
            uint4 xx = xv[c8];
            dsum += wf[c8 * 8 + 0] * bf16_lo(xx.x) + wf[c8 * 8 + 1] * bf16_hi(xx.x) +
                    wf[c8 * 8 + 2] * bf16_lo(xx.y) + wf[c8 * 8 + 3] * bf16_hi(xx.y) +
                    wf[c8 * 8 + 4] * bf16_lo(xx.z) + wf[c8 * 8 + 5] * bf16_hi(xx.z) +
                    wf[c8 * 8 + 6] * bf16_lo(xx.w) + wf[c8 * 8 + 7] * bf16_hi(xx.w);
          }
          dsum *= sc;
          accg[t] += isg ? dsum : 0.f;
          accu[t] += isg ? 0.f : dsum;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      if (t < ntok) {
        float g = accg[t], uu = accu[t];
        for (int off = 32; off > 0; off >>= 1) {
          g += __shfl_xor(g, off);
          uu += __shfl_xor(uu, off);
        }
        if (lane == 0) as[t * R + rl] = silu(g) * uu * s_w[t];
      }
    }
  }
  __syncthreads();

  // ---- down projection: each thread owns DCOLS consecutive output columns ----
  constexpr int DC = F::DCOLS;
  const unsigned char* dbase = blob + F::d_base(H, I);
  const size_t drow = F::d_row_bytes(H);
  for (int c0 = threadIdx.x * DC; c0 < H; c0 += FT * DC) {
    float acc[NTOK][DC];
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
#pragma unroll
      for (int c = 0; c < DC; ++c) acc[t][c] = 0.f;
    const size_t col_byte = (size_t)c0 * drow / H;
#pragma unroll 4
    for (int rl = 0; rl < R; ++rl) {
      float wf[DC];
      F::load_d(dbase + (size_t)(r0 + rl) * drow + col_byte, wf);
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        if (t < ntok) {
          const float at = as[t * R + rl];
#pragma unroll
          for (int c = 0; c < DC; ++c) acc[t][c] += at * wf[c];
        }
      }
    }
    if constexpr (FMT != FMT_BF16) {
      // R divides the scale block (128 for fp8, 32 for MXFP4): one scale per column
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const float sc = d_scale<FMT>(blob, H, I, r0, c0 + c);
#pragma unroll
        for (int t = 0; t < NTOK; ++t) acc[t][c] *= sc;
      }
    }
    float* outbase = (u >= 0) ? v.partial : v.shared_partial;
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      if (t < ntok) {
        float4* o = (float4*)(outbase + ((size_t)s_prow[t] * d.nR + rb) * H + c0);
#pragma unroll
        for (int c = 0; c < DC; c += 4)
          o[c / 4] = make_float4(acc[t][c], acc[t][c + 1], acc[t][c + 2], acc[t][c + 3]);
      }
    }
  }
}

// ---- combine: y[t] = bf16( sum_j sum_r partial[pos(t,j)][r] + sum_r shared[t][r] ) ----
constexpr int CT = 256;

struct CombArgs {
  Dims d;
  Dev v;
  uint16_t* y;
  int T;
  int with_shared;
};

__global__ __launch_bounds__(CT) void combine_kernel(CombArgs a) {
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.y * 64 + lane;
  const int nrow = d.K * d.nR + (a.with_shared ? d.nR : 0);
  float s = 0.f;
  for (int rho = wave; rho < nrow; rho += CT / 64) {
    const float* src;
    if (rho < d.K * d.nR) {
      const int jj = rho / d.nR, r = rho % d.nR;
      const int pos = v.inv_pos[t * d.K + jj];
      src = v.partial + ((size_t)pos * d.nR + r) * d.H;
    } else {
      const int r = rho - d.K * d.nR;
      src = v.shared_partial + ((size_t)t * d.nR + r) * d.H;
    }
    s += src[c];
  }
  __shared__ float red[CT / 64][64];
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0) {
    float tot = red[0][lane];
    for (int w = 1; w < CT / 64; ++w) tot += red[w][lane];
    a.y[(size_t)t * d.H + c] = f32_to_bf16_rne(tot);
  }
}

size_t ffn_decode_lds_bytes(const Dims& d, int ntok) {
  return (size_t)ntok * d.H * 2 + sizeof(float) * (size_t)ntok * d.R;
}

template <int FMT, int NTOK>
static hipError_t launch_one(const FfnArgs& a, int grid, hipStream_t s) {
  const size_t lds = ffn_decode_lds_bytes(a.d, NTOK);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)ffn_decode_kernel<FMT, NTOK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ffn_decode_kernel<FMT, NTOK>), dim3(grid), dim3(FT), lds, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const FfnArgs& a, int ntok, int grid, hipStream_t s) {
  switch (ntok) {
    case 1: return launch_one<FMT, 1>(a, grid, s);
    case 2: return launch_one<FMT, 2>(a, grid, s);
    case 4: return launch_one<FMT, 4>(a, grid, s);
    default: return launch_one<FMT, 8>(a, grid, s);
  }
}

int decode_ntok(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

// mode 0: hits, 1: miss group, 2: shared.  max_entries bounds the workgroups launched.
hipError_t launch_ffn_decode(const Dims& d, const Dev& v, const void* x, const void* arena,
                             const void* shared_blob, int mode, int group, int ngroups, int T,
                             int max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  FfnArgs a{d, v, (const uint16_t*)x, (const unsigned char*)arena,
            (const unsigned char*)shared_blob, mode, group, ngroups, T};
  const int ntok = decode_ntok(T);
  const int grid = max_entries * d.nR;
  switch (d.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16>(a, ntok, grid, s);
    case FMT_FP8: return launch_fmt<FMT_FP8>(a, ntok, grid, s);
    default: return launch_fmt<FMT_MXFP4>(a, ntok, grid, s);
  }
}

hipError_t launch_combine(const Dims& d, const Dev& v, void* y, int T, int with_shared,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  CombArgs a{d, v, (uint16_t*)y, T, with_shared};
  hipLaunchKernelGGL(combine_kernel, dim3(T, d.H / 64), dim3(CT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
