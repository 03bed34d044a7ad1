// SwiGLU expert FFN at decode: weight-streaming GEMVs over the cached expert blobs.
//
// The pages give no expert form; the SwiGLU expert (FFN_e(x) = Wd (silu(Wg x) * (Wu x)))
// is the one this library computes, summed over the top-k experts with the renormalised
// routing weights (plus a GPU-resident shared expert with weight 1 when the model has
// one).  Selected experts run on the GPU once fetched ("FreeToken vs vLLM on one RTX
// 3090", "FreeToken exploits MoE sparsity"); hit experts run first and each group of
// misses runs as soon as its fill has landed ("FreeToken：在消费级 NVIDIA GPU 上进行 MoE
// 推理", "FreeToken 解决的问题": one group computes while the next transfers).
//
// Gfx950 design.  Decode is HBM-bound (about one FLOP per weight byte): every weight byte
// is read once, in coalesced 16-byte lanes, with many loads in flight per wave.  Per group
// of experts two streaming kernels run back to back, and the step ends with a combine:
//   gate/up  - a workgroup owns 8 intermediate rows of one expert; each wave streams two
//              gate|up rows (contiguous 2H elements each) with both rows' loads in flight,
//              reduces across the wave, and writes a = silu(g) * u * w_token (fp32) for
//              every token routed to the expert;
//   down     - a workgroup owns a 128-byte-wide column block of the stored transpose WdT
//              (64 bytes for MXFP4) and half or all of its rows; each thread streams a
//              contiguous run of rows for 16 (8) bytes of columns, so no partial sums over
//              the intermediate dimension leave the workgroup; it writes the expert's
//              output columns (fp32);
//   combine  - y[t] = bf16(sum over the token's k experts (+ shared) in a fixed order).
// Kernel boundaries carry the dependencies: on gfx950 an agent-scope fence is an L2
// write-back plus invalidate, far too costly per workgroup while fills stream into HBM.
// The route kernel publishes a packed entry table (slot, token count, first row, miss
// index) so a workgroup reaches its weights after two dependent loads.
// Every expert is read once per step whatever number of tokens use it (cross-request
// sharing at batch > 1).  fp8 e4m3fn and e2m1 are decoded with gfx950's packed conversions;
// block scales are applied once per block of rows (down) or per 16-byte chunk (gate/up).
#include "moe_dev.h"

namespace moe {

constexpr int FT = 256;  // threads per FFN workgroup (4 waves)
constexpr int RA = 8;    // intermediate rows per gate/up workgroup (2 per wave)

struct FfnArgs {
  Dims d;
  Dev v;
  const uint16_t* x;  // [T][H] bf16
  const unsigned char* arena;
  const unsigned char* shared_blob;
  uint16_t* y;  // [T][H] bf16, written by the combine
  int sel;      // 0: hit experts + shared expert, 1: miss group `group` of `ngroups`, 2: all
  int group;
  int ngroups;
  int T;
  int NE;  // entry slots of this launch
  int NC;     // combine workgroups (0 unless this is the step's last launch)
  int timed;  // this launch is bracketed by timing events: count its blob bytes
};

// ---- format helpers -------------------------------------------------------------
__device__ __forceinline__ void fp8x4(uint32_t v, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

__device__ __forceinline__ void fp4x8(uint32_t v, float* f) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) { return __uint_as_float(c << 23); }

template <int FMT>
struct Fmt;

template <>
struct Fmt<FMT_BF16> {
  static constexpr int EPL = 8;  // elements per 16 bytes
  static constexpr int DC = 8;   // down-projection columns per thread load (16 bytes)
  static constexpr int SB = 0;   // no scale blocks
  __device__ static size_t row_bytes(int n) { return (size_t)n * 2; }
  __device__ static void unpack(uint4 w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
  __device__ static void load_d(const unsigned char* p, float* f) { unpack(*(const uint4*)p, f); }
};

template <>
struct Fmt<FMT_FP8> {
  static constexpr int EPL = 16;
  static constexpr int DC = 16;  // 16 bytes
  static constexpr int SB = 128;
  __device__ static size_t row_bytes(int n) { return (size_t)n; }
  __device__ static void unpack(uint4 w, float* f) {
    fp8x4(w.x, f); fp8x4(w.y, f + 4); fp8x4(w.z, f + 8); fp8x4(w.w, f + 12);
  }
  __device__ static void load_d(const unsigned char* p, float* f) { unpack(*(const uint4*)p, f); }
};

template <>
struct Fmt<FMT_MXFP4> {
  static constexpr int EPL = 32;
  static constexpr int DC = 16;  // 8 bytes: keeps the down accumulators in registers
  static constexpr int SB = 32;
  __device__ static size_t row_bytes(int n) { return (size_t)n / 2; }
  __device__ static void unpack(uint4 w, float* f) {
    fp4x8(w.x, f); fp4x8(w.y, f + 8); fp4x8(w.z, f + 16); fp4x8(w.w, f + 24);
  }
  __device__ static void load_d(const unsigned char* p, float* f) {
    const uint2 w = *(const uint2*)p;
    fp4x8(w.x, f);
    fp4x8(w.y, f + 8);
  }
};

// Scale of gate (g=0) / up (g=1) row i at contraction position xp.
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

// Scales of the down-projection block `blk` for DC consecutive columns starting at c.
template <int FMT>
__device__ __forceinline__ void d_scales(const unsigned char* blob, int H, int I, int blk, int c,
                                         float* sc) {
  if constexpr (FMT == FMT_FP8) {
    const float4* s = (const float4*)(blob + (size_t)3 * I * H + (size_t)4 * 2 * I * (H / 128) +
                                      ((size_t)blk * H + c) * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = s[q];
      sc[4 * q] = v.x; sc[4 * q + 1] = v.y; sc[4 * q + 2] = v.z; sc[4 * q + 3] = v.w;
    }
  } else if constexpr (FMT == FMT_MXFP4) {
    const uint4 a = *(const uint4*)(blob + (size_t)3 * I * H / 2 + (size_t)2 * I * (H / 32) +
                                    (size_t)blk * H + c);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 16; ++q) sc[q] = e8m0_to_f32((w[q / 4] >> (8 * (q % 4))) & 0xffu);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Launch selection -> entry index g in the step's order [hits, shared, misses].
struct Entry {
  int g;       // entry index
  int ntok;
  int row0;    // first act/yexp row (routed) or 0 (shared)
  bool shared;
  const unsigned char* blob;
};

__device__ __forceinline__ int n_entries_in_launch(const FfnArgs& a, int nHit, int nMiss,
                                                   int& first) {
  const int nHS = nHit + a.d.has_shared;
  if (a.sel == 0) {  // hits and shared expert
    first = 0;
    return nHS;
  }
  if (a.sel == 2) {  // every entry of the step
    first = 0;
    return nHS + nMiss;
  }
  const int m0 = (int)((long long)a.group * nMiss / a.ngroups);
  const int m1 = (int)((long long)(a.group + 1) * nMiss / a.ngroups);
  first = nHS + m0;
  return m1 - m0;
}

__device__ __forceinline__ bool resolve(const FfnArgs& a, int j, Entry& en) {
  const Dev& v = a.v;
  if (a.sel == 2 && !a.d.has_shared) {
    // every entry of the step, no shared expert: entry j is table row j, so its load goes
    // out together with the header's (rows past the step's count are never used)
    const int4 e = v.ent[j < a.d.umax ? j : 0];
    if (j >= v.hdr[HDR_NHIT] + v.hdr[HDR_NMISS]) return false;
    en.g = j;
    en.shared = false;
    en.ntok = e.y;
    en.row0 = e.z;
    en.blob = a.arena + (size_t)e.x * (size_t)a.d.S;
    return true;
  }
  const int nHit = v.hdr[HDR_NHIT], nMiss = v.hdr[HDR_NMISS];
  int first;
  const int n = n_entries_in_launch(a, nHit, nMiss, first);
  if (j >= n) return false;
  const int g = first + j;
  en.g = g;
  if (a.d.has_shared && g == nHit) {
    en.shared = true;
    en.ntok = a.T;
    en.row0 = 0;
    en.blob = a.shared_blob;
    return true;
  }
  const int4 e = v.ent[g < nHit ? g : g - a.d.has_shared];
  en.shared = false;
  en.ntok = e.y;
  en.row0 = e.z;
  en.blob = a.arena + (size_t)e.x * (size_t)a.d.S;
  return true;
}

// ---------------------------------------------------------------- gate / up role
// No LDS and no barrier: every wave owns two rows, puts all of its weight loads in flight
// first (the chain hdr -> entry -> slot is the only dependency), then reads the token
// activations (a few KiB, shared by all waves through the L1) and reduces across the wave.
constexpr int GPF = 8;  // 16-byte chunks per lane per row kept in flight

template <int FMT, int NTOK>
__device__ void gate_up_role(const FfnArgs& a, const Entry& en, int rb) {
  using F = Fmt<FMT>;
  constexpr int EPL = F::EPL;
  const Dims& d = a.d;
  const int H = d.H, I = d.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntok = en.ntok < NTOK ? en.ntok : NTOK;
  if (rb == 0 && threadIdx.x == 0) {
    atomicAdd(&a.v.stats[STAT_FFN_BYTES], (unsigned long long)d.S);
    if (a.timed) atomicAdd(&a.v.stats[STAT_TIMED_BLOB_BYTES], (unsigned long long)d.S);
  }
  const int i0 = rb * RA + wave, i1 = i0 + 4;
  const size_t rbytes = F::row_bytes(2 * H);
  const uint4* row0 = (const uint4*)(en.blob + (size_t)i0 * rbytes);
  const uint4* row1 = (const uint4*)(en.blob + (size_t)i1 * rbytes);
  const int nq = 2 * H / EPL;          // 16-byte chunks per row
  const int nper = (nq + 63) / 64;     // per lane
  int tok[NTOK];
  float wt[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    tok[t] = 0;
    wt[t] = 0.f;
  }
  float g0[NTOK], u0[NTOK], g1[NTOK], u1[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) g0[t] = u0[t] = g1[t] = u1[t] = 0.f;
  for (int base = 0; base < nper; base += GPF) {
    uint4 w0[GPF], w1[GPF];
#pragma unroll
    for (int k = 0; k < GPF; ++k) {
      if ((base + k) * 64 + lane < nq) {
        w0[k] = row0[(base + k) * 64 + lane];
        w1[k] = row1[(base + k) * 64 + lane];
      }
    }
    if (base == 0) {
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        if (t < ntok) {
          tok[t] = en.shared ? t : a.v.row_tok[en.row0 + t];
          wt[t] = en.shared ? 1.0f : a.v.row_w[en.row0 + t];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < GPF; ++k) {
      if ((base + k) * 64 + lane < nq) {
        const int p = ((base + k) * 64 + lane) * EPL;
        const bool isg = p < H;
        const int xp = isg ? p : p - H;
        float f0[EPL], f1[EPL];
        F::unpack(w0[k], f0);
        F::unpack(w1[k], f1);
        const float s0 = gu_scale<FMT>(en.blob, H, I, i0, isg ? 0 : 1, xp);
        const float s1 = gu_scale<FMT>(en.blob, H, I, i1, isg ? 0 : 1, xp);
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
          if (t < ntok) {
            const uint4* xv = (const uint4*)(a.x + (size_t)tok[t] * H + xp);
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < EPL / 8; ++c8) {
              const uint4 xx = xv[c8];
              const float xf[8] = {bf16_lo(xx.x), bf16_hi(xx.x), bf16_lo(xx.y), bf16_hi(xx.y),
                                   bf16_lo(xx.z), bf16_hi(xx.z), bf16_lo(xx.w), bf16_hi(xx.w)};
#pragma unroll
              for (int c = 0; c < 8; ++c) {
                d0 += f0[c8 * 8 + c] * xf[c];
                d1 += f1[c8 * 8 + c] * xf[c];
              }
            }
            d0 *= s0;
            d1 *= s1;
            if (isg) {
              g0[t] += d0;
              g1[t] += d1;
            } else {
              u0[t] += d0;
              u1[t] += d1;
            }
          }
        }
      }
    }
  }
  float* act = en.shared ? a.v.act_shared : a.v.act;
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    if (t < ntok) {
      float a0 = g0[t], b0 = u0[t], a1 = g1[t], b1 = u1[t];
      for (int off = 32; off > 0; off >>= 1) {
        a0 += __shfl_xor(a0, off);
        b0 += __shfl_xor(b0, off);
        a1 += __shfl_xor(a1, off);
        b1 += __shfl_xor(b1, off);
      }
      if (lane == 0) {
        float* out = act + (size_t)(en.row0 + t) * I;
        out[i0] = silu(a0) * b0 * wt[t];
        out[i1] = silu(a1) * b1 * wt[t];
      }
    }
  }
}

// ---------------------------------------------------------------- down role
// A workgroup owns a column block of DTC*DC columns of the stored transpose WdT and I/RS of
// its rows; thread (row lane rl, column lane cl) owns DC columns of a contiguous run of at
// most DMAXR rows.  All of a thread's weight loads go out first; the activations (fp32,
// L1-shared) follow, then row lanes reduce by shuffles and through LDS across waves.  The
// workgroup writes one partial sum per row split; the combine adds the splits.
constexpr int DTC = 16;            // column lanes
constexpr int DTR = FT / DTC;      // row lanes
constexpr int DMAXR = 16;          // rows per thread, at most

template <int FMT>
struct DVec {
  using T = uint4;
};
template <>
struct DVec<FMT_MXFP4> {
  using T = uint2;
};

template <int FMT>
__device__ __forceinline__ void unpack_d(const typename DVec<FMT>::T& w, float* f);
template <>
__device__ __forceinline__ void unpack_d<FMT_BF16>(const uint4& w, float* f) {
  Fmt<FMT_BF16>::unpack(w, f);
}
template <>
__device__ __forceinline__ void unpack_d<FMT_FP8>(const uint4& w, float* f) {
  Fmt<FMT_FP8>::unpack(w, f);
}
template <>
__device__ __forceinline__ void unpack_d<FMT_MXFP4>(const uint2& w, float* f) {
  fp4x8(w.x, f);
  fp4x8(w.y, f + 8);
}

template <int FMT, int NTOK>
__device__ void down_role(const FfnArgs& a, const Entry& en, int cb, int rs, unsigned char* smem) {
  using F = Fmt<FMT>;
  using W = typename DVec<FMT>::T;
  constexpr int DC = F::DC;
  constexpr int HC = DTC * DC;
  const Dims& d = a.d;
  const int H = d.H, I = d.I, RS = d.RS;
  const int ntok = en.ntok < NTOK ? en.ntok : NTOK;
  const int IR = I / RS;
  const int nrw = IR / DTR;  // <= DMAXR (host-chosen RS)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = threadIdx.x % DTC, rl = threadIdx.x / DTC;
  const int c0 = cb * HC + cl * DC;
  const int ra = rs * IR + rl * nrw;
  const unsigned char* wdt = en.blob + F::row_bytes(2 * H) * (size_t)I;  // WdT after Wgu
  const size_t drow = F::row_bytes(H);
  const unsigned char* wp = wdt + (size_t)ra * drow + F::row_bytes(c0);
  W w[DMAXR];
#pragma unroll
  for (int r = 0; r < DMAXR; ++r)
    if (r < nrw) w[r] = *(const W*)(wp + (size_t)r * drow);
  float sc0[DC], sc1[DC];
  int bsplit = DMAXR;  // first r that uses sc1
  if constexpr (F::SB > 0) {
    const int blk0 = ra / F::SB, blk1 = (ra + nrw - 1) / F::SB;
    d_scales<FMT>(en.blob, H, I, blk0, c0, sc0);
    d_scales<FMT>(en.blob, H, I, blk1, c0, sc1);
    bsplit = (blk0 + 1) * F::SB - ra;
  }
  const float* act = (en.shared ? a.v.act_shared : a.v.act) + (size_t)en.row0 * I + ra;
  float acc[NTOK][DC];
#pragma unroll
  for (int t = 0; t < NTOK; ++t)
#pragma unroll
    for (int c = 0; c < DC; ++c) acc[t][c] = 0.f;
#pragma unroll
  for (int r = 0; r < DMAXR; ++r) {
    if (r < nrw) {
      float f[DC];
      unpack_d<FMT>(w[r], f);
      if constexpr (F::SB > 0) {
#pragma unroll
        for (int c = 0; c < DC; ++c) f[c] *= (r < bsplit ? sc0[c] : sc1[c]);
      }
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        if (t < ntok) {
          const float at = act[(size_t)t * I + r];
#pragma unroll
          for (int c = 0; c < DC; ++c) acc[t][c] += at * f[c];
        }
      }
    }
  }
  // reduce over the DTR row lanes: those inside a wave by shuffles, the 4 waves through LDS
  float* s_red = (float*)smem;  // [4][NTOK][HC]
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    if (t < ntok) {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        float v = acc[t][c];
        for (int off = DTC; off < 64; off <<= 1) v += __shfl_xor(v, off);
        acc[t][c] = v;
      }
    }
  }
  if (lane < DTC) {
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
      if (t < ntok)
#pragma unroll
        for (int c = 0; c < DC; ++c)
          s_red[((size_t)wave * NTOK + t) * HC + lane * DC + c] = acc[t][c];
  }
  __syncthreads();
  float* yexp = en.shared ? a.v.yexp_shared : a.v.yexp;
  for (int idx = threadIdx.x; idx < ntok * HC; idx += FT) {
    const int t = idx / HC, c = idx % HC;
    float sum = 0.f;
#pragma unroll
    for (int wv = 0; wv < FT / 64; ++wv) sum += s_red[((size_t)wv * NTOK + t) * HC + c];
    yexp[((size_t)(en.row0 + t) * RS + rs) * H + cb * HC + c] = sum;
  }
}

// ---------------------------------------------------------------- combine role
// y[t] = bf16( sum_j sum_rs yexp[pos(t,j)][rs] + sum_rs yexp_shared[t][rs] ), in that fixed
// order.
__device__ void combine_role(const FfnArgs& a, int cblk) {
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int per_tok = (d.H + FT - 1) / FT;
  const int t = cblk / per_tok;
  const int c = (cblk % per_tok) * FT + threadIdx.x;
  __shared__ int s_pos[32];
  if ((int)threadIdx.x < d.K) s_pos[threadIdx.x] = v.inv_pos[t * d.K + threadIdx.x];
  __syncthreads();
  if (c >= d.H) return;
  // all partials of a chunk are loaded before any is added: one memory latency per chunk
  constexpr int CH = 16;
  const int RS = d.RS, nrouted = d.K * RS, nall = nrouted + (d.has_shared ? RS : 0);
  float s = 0.f;
  for (int base = 0; base < nall; base += CH) {
    float pv[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int i = base + q;
      pv[q] = 0.f;
      if (i < nrouted)
        pv[q] = v.yexp[((size_t)s_pos[i / RS] * RS + i % RS) * d.H + c];
      else if (i < nall)
        pv[q] = v.yexp_shared[((size_t)t * RS + (i - nrouted)) * d.H + c];
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) s += pv[q];
  }
  a.y[(size_t)t * d.H + c] = f32_to_bf16_rne(s);
}

template <int FMT>
static constexpr int down_hc() {
  return DTC * Fmt<FMT>::DC;
}

template <int FMT, int NTOK>
__global__ __launch_bounds__(FT) void ffn_gate_up_kernel(FfnArgs a) {
  const int nra = a.d.I / RA;
  Entry en;
  if (!resolve(a, blockIdx.x / nra, en)) return;
  gate_up_role<FMT, NTOK>(a, en, blockIdx.x % nra);
}

template <int FMT, int NTOK>
__global__ __launch_bounds__(FT) void ffn_down_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& d = a.d;
  const int ndn = (d.H / down_hc<FMT>()) * d.RS;
  Entry en;
  if (!resolve(a, blockIdx.x / ndn, en)) return;
  const int r = blockIdx.x % ndn;
  down_role<FMT, NTOK>(a, en, r / d.RS, r % d.RS, smem);
}

__global__ __launch_bounds__(FT) void combine_kernel(FfnArgs a) { combine_role(a, blockIdx.x); }

int decode_ntok(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

template <class Kern>
static hipError_t launch_with_lds(Kern kernel, int grid, size_t lds, const FfnArgs& a,
                                  hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (grid <= 0) {  // nothing to run; keep the timing events valid
    hipError_t e = e0 ? hipEventRecord(e0, s) : hipSuccess;
    if (e == hipSuccess && e1) e = hipEventRecord(e1, s);
    return e;
  }
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  return launch_timed(kernel, dim3(grid), dim3(FT), lds, s, e0, e1, a);
}

// stage 0: the gate/up kernel; stage 1: the down kernel (+ combine when a.NC > 0)
template <int FMT, int NTOK>
static hipError_t launch_ffn(const FfnArgs& a, int stage, hipStream_t s, hipEvent_t e0,
                             hipEvent_t e1) {
  const Dims& d = a.d;
  constexpr int HC = down_hc<FMT>();
  if (stage == 0)
    return launch_with_lds(ffn_gate_up_kernel<FMT, NTOK>, a.NE * (d.I / RA), 0, a, s, e0, e1);
  hipError_t e = launch_with_lds(ffn_down_kernel<FMT, NTOK>, a.NE * (d.H / HC) * d.RS,
                                 sizeof(float) * (size_t)4 * NTOK * HC, a, s, e0,
                                 a.NC > 0 ? nullptr : e1);
  if (e != hipSuccess || a.NC <= 0) return e;
  return launch_timed(combine_kernel, dim3(a.NC), dim3(FT), 0, s, nullptr, e1, a);
}

template <int FMT>
static hipError_t launch_fmt(const FfnArgs& a, int ntok, int stage, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  switch (ntok) {
    case 1: return launch_ffn<FMT, 1>(a, stage, s, e0, e1);
    case 2: return launch_ffn<FMT, 2>(a, stage, s, e0, e1);
    case 4: return launch_ffn<FMT, 4>(a, stage, s, e0, e1);
    default: return launch_ffn<FMT, 8>(a, stage, s, e0, e1);
  }
}

int down_columns_per_block(int fmt) {
  return fmt == FMT_BF16 ? down_hc<FMT_BF16>()
                         : fmt == FMT_FP8 ? down_hc<FMT_FP8>() : down_hc<FMT_MXFP4>();
}

// Row splits of the down projection: the fewest (a power of two) that keep a thread's rows
// within DMAXR.  I is a multiple of 128, so I / (RS * DTR) is whole for every RS it picks.
int down_row_splits(int inter) {
  int rs = 1;
  while (inter / (rs * DTR) > DMAXR) rs *= 2;
  return rs;
}

// sel 0: hit experts and the shared expert; sel 1: miss group `group` of `ngroups`;
// sel 2: every entry of the step (hits, shared, misses).  max_entries bounds the entries of
// the launch; with_combine adds the combine kernel after the down kernel (only on the step's
// last launch); stage 0 launches the gate/up kernel, stage 1 the down kernel (and the
// combine).  e0/e1 (nullable) take the start of the first and the end of the last kernel.
hipError_t launch_ffn_decode(const Dims& d, const Dev& v, const void* x, const void* arena,
                             const void* shared_blob, void* y, int sel, int group, int ngroups,
                             int T, int max_entries, int with_combine, int stage,
                             hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nc = with_combine ? T * ((d.H + FT - 1) / FT) : 0;
  FfnArgs a{d, v, (const uint16_t*)x, (const unsigned char*)arena,
            (const unsigned char*)shared_blob, (uint16_t*)y, sel, group, ngroups, T,
            max_entries > 0 ? max_entries : 0, nc, e0 != nullptr};
  const int ntok = decode_ntok(T);
  switch (d.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16>(a, ntok, stage, s, e0, e1);
    case FMT_FP8: return launch_fmt<FMT_FP8>(a, ntok, stage, s, e0, e1);
    default: return launch_fmt<FMT_MXFP4>(a, ntok, stage, s, e0, e1);
  }
}

}  // namespace moe
