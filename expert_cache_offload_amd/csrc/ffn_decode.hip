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
//              gate|up rows (contiguous 2H elements each) with every weight load in flight
//              before any is used, reduces across the wave, and writes
//              a = silu(g) * u * w_token (fp32) for every token routed to the expert;
//   down     - a workgroup owns a 128-column block of the stored transpose WdT (256 columns
//              for fp8 / MXFP4) and 1/RS of its rows; each thread streams a contiguous run of
//              rows for 16 (8) bytes of columns, so no partial sums over the intermediate
//              dimension leave the workgroup except one per row split; it writes the
//              expert's output columns (fp32);
//   combine  - y[t] = bf16(sum over the token's k experts' row splits, + the CPU experts'
//              sum in hybrid decode, + the shared expert) in a fixed order.
// At one token with bf16 weights and no shared expert (the batch-1 decode of the bf16
// models) one fused kernel replaces gate/up and down: a workgroup owns 8 intermediate rows
// of an expert, computes their activations and multiplies them straight into its 8 rows of
// WdT, writing one fp32 partial of the output per row block; a wider combine adds them.  One
// launch then streams every blob of the step, which halves the fixed launch and dependency
// cost per byte; the partials cost 8% more HBM traffic than the activations they replace.
// Kernel boundaries carry the dependencies: on gfx950 an agent-scope release / acquire per
// workgroup is an L2 write-back / invalidate, far costlier than a second launch.
// The route kernel publishes a packed entry table (slot, token count, first row, miss
// index) so a workgroup reaches its weights after two dependent loads.
// Every expert is read once per step whatever number of tokens use it (cross-request
// sharing at batch > 1).  fp8 e4m3fn and e2m1 codes are widened to bf16 exactly with gfx950's
// scaled conversions and multiplied with two-wide bf16 dot products (gate/up) or widened to
// fp32 (down); block scales are applied per 16-byte chunk (gate/up) or per block of rows
// (down).
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
};

template <>
struct Fmt<FMT_FP8> {
  static constexpr int EPL = 16;
  static constexpr int DC = 16;  // 16 bytes
  static constexpr int SB = 128;
  __device__ static size_t row_bytes(int n) { return (size_t)n; }
};

template <>
struct Fmt<FMT_MXFP4> {
  static constexpr int EPL = 32;
  static constexpr int DC = 16;  // 8 bytes: keeps the down accumulators in registers
  static constexpr int SB = 32;
  __device__ static size_t row_bytes(int n) { return (size_t)n / 2; }
};

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
// No barrier at one token: every wave owns two rows (i0 and i0 + 4 of the workgroup's
// eight).  Lane l takes the gate chunks l, l + 64, ... of both rows and the up chunks at the
// same contraction positions, so one set of activations serves four weight chunks.  The
// lane's activations go out first (at one token they do not depend on the plan), then every
// weight chunk and scale of the pass; loads complete in issue order, so nothing waits on a
// later load.  Products use gfx950's two-wide bf16 dot (fp8 and e2m1 codes are widened to
// bf16 first, exactly); per-chunk block scales multiply the chunk's sum.  At more tokens the
// routed tokens' activations are staged in LDS once per workgroup.
constexpr int GN = 4;  // gate chunks per lane per pass (4 * GN weight loads in flight)

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Expert weights are read once per step: streaming (non-temporal) loads, so they do not
// displace the activations, partials and plan tables from the caches.
template <class V>
__device__ __forceinline__ V ld_stream(const unsigned char* p) {
  return __builtin_nontemporal_load((const V*)p);
}

// Workgroup barrier that orders LDS accesses only: global loads still in flight (the weight
// stream) stay in flight across it, where __syncthreads would wait for every one of them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w),
                                         __builtin_bit_cast(bf16x2v, x), acc, false);
}
__device__ __forceinline__ float dot2(bf16x2v w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2v, x), acc, false);
}

// One 16-byte weight chunk widened to EPL/2 words of bf16 pairs (fp8 and e2m1 codes are
// exact in bf16; unscaled), once per chunk whatever the number of tokens.
template <int FMT>
__device__ __forceinline__ void widen(const u32x4v& w, uint32_t* o);
template <>
__device__ __forceinline__ void widen<FMT_BF16>(const u32x4v& w, uint32_t* o) {
  o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
}
template <>
__device__ __forceinline__ void widen<FMT_FP8>(const u32x4v& w, uint32_t* o) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, false));
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, true));
  }
}
template <>
__device__ __forceinline__ void widen<FMT_MXFP4>(const u32x4v& w, uint32_t* o) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[4 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 0));
    o[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 1));
    o[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 2));
    o[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 3));
  }
}

// acc + sum over N words of bf16 pairs: weights (widened) times activations
template <int N>
__device__ __forceinline__ float wdot(const uint32_t* ww, const uint32_t* xw, float acc) {
#pragma unroll
  for (int j = 0; j < N; ++j) acc = dot2(ww[j], xw[j], acc);
  return acc;
}

// scale of gate (g = 0) or up (g = 1) row i for the 16-byte chunk c of that half-row
template <int FMT>
__device__ __forceinline__ float gu_chunk_scale(const unsigned char* blob, int H, int I, int i,
                                                int g, int c) {
  if constexpr (FMT == FMT_FP8) {
    const float* s = (const float*)(blob + (size_t)3 * I * H);
    return s[(size_t)(2 * i + g) * (H / 128) + c / 8];  // 8 chunks of 16 codes per block
  } else if constexpr (FMT == FMT_MXFP4) {
    const unsigned char* s = blob + (size_t)3 * I * H / 2;
    return e8m0_to_f32(s[(size_t)(2 * i + g) * (H / 32) + c]);  // one 32-code block per chunk
  } else {
    return 1.0f;
  }
}

// Butterfly reduce-scatter over the wave of M = 2 * NTOK units (gate, up): afterwards lane l
// holds the wave total of unit gu_unit<NTOK>(l) (every lane sharing that unit holds it).
// Read-only views of plan arrays for uniform indices: loads through the constant address
// space become scalar loads (the arrays are written by an earlier launch, never by this one).
typedef __attribute__((address_space(4))) const int kconst_i32;
typedef __attribute__((address_space(4))) const float kconst_f32;

template <int NTOK>
__device__ __forceinline__ void wave_reduce_units(float* gv, float* uv, int lane) {
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int o = 32 >> st, n = (2 * NTOK) >> st;
    if (n > 1) {
      const int half = n / 2;
      const bool hi = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        // opaque copies: keeps the lane-dependent choice a register select (a select of two
        // array loads would otherwise become a dynamically indexed private array)
        float ga = gv[i], gb = gv[half + i], ua = uv[i], ub = uv[half + i];
        asm volatile("" : "+v"(ga), "+v"(gb), "+v"(ua), "+v"(ub));
        const float sg = hi ? ga : gb, kg = hi ? gb : ga;
        const float su = hi ? ua : ub, ku = hi ? ub : ua;
        gv[i] = kg + __shfl_xor(sg, o);
        uv[i] = ku + __shfl_xor(su, o);
      }
    } else {
      gv[0] += __shfl_xor(gv[0], o);
      uv[0] += __shfl_xor(uv[0], o);
    }
  }
}
template <int NTOK>
__device__ __forceinline__ int gu_unit(int lane) {
  int m = 0;
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int o = 32 >> st, n = (2 * NTOK) >> st;
    if (n > 1 && (lane & o)) m += n / 2;
  }
  return m;
}

template <int FMT>
struct GuX {
  static constexpr int XV = Fmt<FMT>::EPL / 8;  // 16-byte activation vectors per weight chunk
  // gate chunk groups of 64 per lane per pass: three for e2m1 (a 6144-wide row is 192 chunks
  // of 32 codes, so a fourth group would only reload the last chunk), else GN
  static constexpr int GNF = FMT == FMT_MXFP4 ? 3 : GN;
};

// At one token: the lane's activations of pass kb (gate chunks c = (kb + k) * 64 + lane).
// xrow: the token's activation row ([H] bf16).
template <int FMT>
__device__ __forceinline__ void load_x1(const FfnArgs& a, int kb, int lane,
                                        u32x4v (&xr)[GuX<FMT>::GNF][GuX<FMT>::XV], const uint16_t* xrow) {
  constexpr int EPL = Fmt<FMT>::EPL, XV = GuX<FMT>::XV;
  const int ngq = a.d.H / EPL;
#pragma unroll
  for (int k = 0; k < GuX<FMT>::GNF; ++k) {
    int c = (kb + k) * 64 + lane;
    c = c < ngq ? c : ngq - 1;
    const u32x4v* p = (const u32x4v*)(xrow + (size_t)c * EPL);
#pragma unroll
    for (int q = 0; q < XV; ++q) xr[k][q] = p[q];
  }
}

// Chunks per token of the staged activations of a gate/up pass at more than one token: a
// pass covers GNF * 64 chunks, trimmed for rows shorter than that to the staging loads' own
// granularity (FT / XV chunks), so no LDS is reserved for chunks that are never loaded.
template <int FMT>
__host__ __device__ inline int gate_up_stage_chunks(int ngq) {
  constexpr int CPI = FT / GuX<FMT>::XV, PC = GuX<FMT>::GNF * 64;
  const int rounded = (ngq + CPI - 1) / CPI * CPI;
  return rounded < PC ? rounded : PC;
}

// xrow (NTOK == 1): the activation row of the entry's one token, for passes after the first.
template <int FMT, int NTOK>
__device__ void gate_up_role(const FfnArgs& a, const Entry& en, int rb,
                             u32x4v (&xr)[GuX<FMT>::GNF][GuX<FMT>::XV], uint16_t* s_x,
                             const uint16_t* xrow) {
  using F = Fmt<FMT>;
  constexpr int EPL = F::EPL, XV = GuX<FMT>::XV, GN = GuX<FMT>::GNF;
  const Dims& d = a.d;
  const int H = d.H, I = d.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntok = en.ntok < NTOK ? en.ntok : NTOK;
  if (rb == 0 && threadIdx.x == 0) {
    atomicAdd(&a.v.stats[STAT_FFN_BYTES], (unsigned long long)d.S);
    if (a.timed) atomicAdd(&a.v.stats[STAT_TIMED_BLOB_BYTES], (unsigned long long)d.S);
  }
  // routed tokens and their weights: scalar loads issued together behind the first pass's
  // weight stream (the plan wrote them before this launch; per-token vector loads each waited
  // before the next, and in front of the weight loads); the staged activations' addresses then
  // wait on them alone.  For the shared expert (row0 0) the loaded values are valid, unused.
  int tok[NTOK];
  float wt[NTOK];
  auto load_tokens = [&]() {
    const kconst_i32* rt = (const kconst_i32*)(a.v.row_tok + en.row0);
    const kconst_f32* rw = (const kconst_f32*)(a.v.row_w + en.row0);
    int lt[NTOK];
    float lw[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      const int tc = t < ntok ? t : 0;
      lt[t] = rt[tc];
      lw[t] = rw[tc];
    }
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      const int tc = t < ntok ? t : 0;
      tok[t] = en.shared ? tc : lt[t];
      wt[t] = en.shared ? 1.0f : lw[t];
    }
  };
  const int i0 = rb * RA + wave, i1 = i0 + 4;
  const size_t rbytes = F::row_bytes(2 * H), hbytes = F::row_bytes(H);
  const unsigned char* r0 = en.blob + (size_t)i0 * rbytes;
  const unsigned char* r1 = en.blob + (size_t)i1 * rbytes;
  const int ngq = H / EPL;  // 16-byte chunks per half-row (gate or up)
  float g0[NTOK], u0[NTOK], g1[NTOK], u1[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) g0[t] = u0[t] = g1[t] = u1[t] = 0.f;
  constexpr int PC = GN * 64;                           // chunk slots per token per pass
  constexpr int CPI = FT / XV;  // chunks one staging load of the workgroup covers
  const int pce = gate_up_stage_chunks<FMT>(ngq);  // staged chunks per token
  for (int kb = 0; kb * 64 < ngq; kb += GN) {
    u32x4v wg0[GN], wu0[GN], wg1[GN], wu1[GN];
    float sg0[GN], su0[GN], sg1[GN], su1[GN];  // block scales (fp8, MXFP4)
#pragma unroll
    for (int k = 0; k < GN; ++k) {
      int c = (kb + k) * 64 + lane;
      c = c < ngq ? c : ngq - 1;  // in-row address; masked below
      wg0[k] = ld_stream<u32x4v>(r0 + (size_t)c * 16);
      wu0[k] = ld_stream<u32x4v>(r0 + hbytes + (size_t)c * 16);
      wg1[k] = ld_stream<u32x4v>(r1 + (size_t)c * 16);
      wu1[k] = ld_stream<u32x4v>(r1 + hbytes + (size_t)c * 16);
    }
    if constexpr (F::SB > 0) {
#pragma unroll
      for (int k = 0; k < GN; ++k) {
        int c = (kb + k) * 64 + lane;
        c = c < ngq ? c : ngq - 1;
        sg0[k] = gu_chunk_scale<FMT>(en.blob, H, I, i0, 0, c);
        su0[k] = gu_chunk_scale<FMT>(en.blob, H, I, i0, 1, c);
        sg1[k] = gu_chunk_scale<FMT>(en.blob, H, I, i1, 0, c);
        su1[k] = gu_chunk_scale<FMT>(en.blob, H, I, i1, 1, c);
      }
    }
    if (kb == 0) load_tokens();
    if constexpr (NTOK > 1) {
      // the pass's activations of every routed token, staged in LDS as [t][pce chunks of EPL]
      // (rows past the entry's tokens repeat its first token) by 16-byte global-to-LDS loads
      // behind the weight stream: no registers held for them.  Load q2 of token t covers the
      // pass's chunks q2 * CPI .. + CPI - 1; loads outside the pass or wholly past the row are
      // skipped, and lanes past the row load its last chunk into slots no product reads.
      if (kb > 0) lds_barrier();  // the previous pass is done with s_x
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        const int tk = tok[t < ntok ? t : 0];
#pragma unroll
        for (int q2 = 0; q2 < XV; ++q2) {
          // uniform: outside the pass (an e2m1 pass is 3 of the 4 groups a token's XV loads
          // could cover) or wholly past the row
          if (q2 * CPI >= PC || kb * 64 + q2 * CPI >= ngq) continue;
          const int r = q2 * FT + (int)threadIdx.x;
          const int c = kb * 64 + r / XV;
          const int cc = c < ngq ? c : ngq - 1;
          __builtin_amdgcn_global_load_lds(a.x + (size_t)tk * H + (size_t)cc * EPL + (r % XV) * 8,
                                           s_x + ((size_t)t * pce * XV + q2 * FT + wave * 64) * 8,
                                           16, 0, 0);
        }
      }
    }
    if constexpr (NTOK == 1) {
      if (kb > 0) load_x1<FMT>(a, kb, lane, xr, xrow);
    } else {
      lds_barrier();  // waits for the staging loads (and the weight loads issued before them)
    }
#pragma unroll
    for (int k = 0; k < GN; ++k) {
      const int c = (kb + k) * 64 + lane;
      if (c < ngq) {
        constexpr int NW = EPL / 2;
        uint32_t ag0[NW], au0[NW], ag1[NW], au1[NW];
        widen<FMT>(wg0[k], ag0);
        widen<FMT>(wu0[k], au0);
        widen<FMT>(wg1[k], ag1);
        widen<FMT>(wu1[k], au1);
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
          if (t < ntok) {
            uint32_t xw[EPL / 2];
            if constexpr (NTOK == 1) {
#pragma unroll
              for (int q = 0; q < XV; ++q) {
                xw[4 * q] = xr[k][q].x; xw[4 * q + 1] = xr[k][q].y;
                xw[4 * q + 2] = xr[k][q].z; xw[4 * q + 3] = xr[k][q].w;
              }
            } else {
              const u32x4v* sp =
                  (const u32x4v*)(s_x + ((size_t)t * pce * XV + (size_t)(k * 64 + lane) * XV) * 8);
#pragma unroll
              for (int q = 0; q < XV; ++q) {
                const u32x4v v = sp[q];
                xw[4 * q] = v.x; xw[4 * q + 1] = v.y; xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
              }
            }
            if constexpr (F::SB > 0) {
              g0[t] += sg0[k] * wdot<NW>(ag0, xw, 0.f);
              u0[t] += su0[k] * wdot<NW>(au0, xw, 0.f);
              g1[t] += sg1[k] * wdot<NW>(ag1, xw, 0.f);
              u1[t] += su1[k] * wdot<NW>(au1, xw, 0.f);
            } else {
              g0[t] = wdot<NW>(ag0, xw, g0[t]);
              u0[t] = wdot<NW>(au0, xw, u0[t]);
              g1[t] = wdot<NW>(ag1, xw, g1[t]);
              u1[t] = wdot<NW>(au1, xw, u1[t]);
            }
          }
        }
      }
    }
  }
  // units m = r * NTOK + t: (gate, up) of row r (i0 or i1) for token t
  float gv[2 * NTOK], uv[2 * NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    gv[t] = g0[t]; uv[t] = u0[t];
    gv[NTOK + t] = g1[t]; uv[NTOK + t] = u1[t];
  }
  wave_reduce_units<NTOK>(gv, uv, lane);
  const int m = gu_unit<NTOK>(lane);
  const int t = m % NTOK;
  if ((lane & (64 / (2 * NTOK) - 1)) == 0 && t < ntok) {
    float w = wt[0];
#pragma unroll
    for (int q = 1; q < NTOK; ++q) w = t == q ? wt[q] : w;
    float* act = en.shared ? a.v.act_shared : a.v.act;
    act[(size_t)(en.row0 + t) * I + (m < NTOK ? i0 : i1)] = silu(gv[0]) * uv[0] * w;
  }
}

// ---------------------------------------------------------------- down role
// A workgroup owns a column block of DTC*DC columns of the stored transpose WdT and I/RS of
// its rows; thread (row lane rl, column lane cl) owns DC columns of a contiguous run of at
// most DMAXR rows.  The thread's activations go out first (fp32 rows written by the gate/up
// kernel; at more than one token they are staged in LDS for the workgroup), then all of its
// weight loads, so no load waits behind another; row lanes reduce by shuffles and through
// LDS across waves.  The workgroup writes one partial sum per row split; the combine adds
// the splits.
constexpr int DTC = 16;            // column lanes
constexpr int DTR = FT / DTC;      // row lanes
constexpr int DMAXR = 16;          // rows per thread, at most

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

template <int FMT>
struct DVec {
  using T = u32x4v;
};
template <>
struct DVec<FMT_MXFP4> {
  using T = u32x2v;
};

template <int FMT>
__device__ __forceinline__ void unpack_d(const typename DVec<FMT>::T& w, float* f);
template <>
__device__ __forceinline__ void unpack_d<FMT_BF16>(const u32x4v& w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack_d<FMT_FP8>(const u32x4v& w, float* f) {
  fp8x4(w.x, f); fp8x4(w.y, f + 4); fp8x4(w.z, f + 8); fp8x4(w.w, f + 12);
}
template <>
__device__ __forceinline__ void unpack_d<FMT_MXFP4>(const u32x2v& w, float* f) {
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
  const float* act = (en.shared ? a.v.act_shared : a.v.act) + (size_t)en.row0 * I;
  float* s_red = (float*)smem;                  // [4][NTOK][HC]
  float* s_act = s_red + (size_t)4 * NTOK * HC;  // [NTOK][IR] (NTOK > 1)
  // activations first
  float av[DMAXR];
  constexpr int SA = (NTOK * 256 + FT - 1) / FT;  // staged values per thread (IR <= 256)
  float sv[NTOK > 1 ? SA : 1];
  if constexpr (NTOK == 1) {
#pragma unroll
    for (int r = 0; r < DMAXR; ++r) av[r] = act[ra + (r < nrw ? r : nrw - 1)];
  } else {
#pragma unroll
    for (int q = 0; q < SA; ++q) {
      int idx = threadIdx.x + q * FT;
      const int t = idx / IR, r = idx % IR;
      const int tc = t < ntok ? t : 0;
      sv[q] = act[(size_t)tc * I + rs * IR + r];
    }
  }
  // then every weight row of the thread (clamped to its run; extra rows are not used)
  const unsigned char* wdt = en.blob + F::row_bytes(2 * H) * (size_t)I;  // WdT after Wgu
  const size_t drow = F::row_bytes(H);
  const unsigned char* wp = wdt + (size_t)ra * drow + F::row_bytes(c0);
  W w[DMAXR];
#pragma unroll
  for (int r = 0; r < DMAXR; ++r) w[r] = ld_stream<W>(wp + (size_t)(r < nrw ? r : nrw - 1) * drow);
  float sc0[DC], sc1[DC];
  int bsplit = DMAXR;  // first r that uses sc1
  if constexpr (F::SB > 0) {
    const int blk0 = ra / F::SB, blk1 = (ra + nrw - 1) / F::SB;
    d_scales<FMT>(en.blob, H, I, blk0, c0, sc0);
    d_scales<FMT>(en.blob, H, I, blk1, c0, sc1);
    bsplit = (blk0 + 1) * F::SB - ra;
  }
  if constexpr (NTOK > 1) {
#pragma unroll
    for (int q = 0; q < SA; ++q) {
      const int idx = threadIdx.x + q * FT;
      if (idx < NTOK * IR) s_act[idx] = sv[q];
    }
    lds_barrier();  // the weight rows stay in flight
  }
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
          const float at = NTOK == 1 ? av[r] : s_act[t * IR + rl * nrw + r];
#pragma unroll
          for (int c = 0; c < DC; ++c) acc[t][c] += at * f[c];
        }
      }
    }
  }
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


// Wait for the host's answer to this step (hybrid decode), bounded by the handle's timeout on
// the GPU's constant 100 MHz clock; no answer in time sets ERR_HYBRID and returns false (the
// step then goes on without the CPU experts' sum).  One thread per workgroup calls it.
__device__ bool wait_host_answer(const Dev& v) {
  const long long step =
      (long long)(unsigned)v.hdr[HDR_STEP_LO] | ((long long)v.hdr[HDR_STEP_HI] << 32);
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
#pragma nounroll
  while (__hip_atomic_load(&v.mail->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != step) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > (unsigned long long)v.hyb_timeout_ticks) {
      atomicOr(&v.ctrl[CTRL_ERR], ERR_HYBRID);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  return true;
}

// ---------------------------------------------------------------- combine role
// y[t] = bf16( sum_j sum_rs yexp[pos(t,j)][rs] + y_cpu[t] + sum_rs yexp_shared[t][rs] ), in
// that fixed order; the routed sum skips the rows whose expert the CPU computed (hybrid
// decode), and y_cpu[t] (their weighted sum, from the host mailbox) is added once the host
// has answered this step.  Every partial of a chunk is loaded before any is added (one
// memory latency per chunk of CH partials).
constexpr int kMaxPartials = 640;             // top_k * row splits, checked at launch

__device__ void combine_role(const FfnArgs& a, int cblk) {
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int per_tok = (d.H + FT - 1) / FT;
  const int t = cblk / per_tok;
  const int c = (cblk % per_tok) * FT + threadIdx.x;
  const int RS = d.RS, nrouted = d.K * RS;
  __shared__ int s_row[kMaxPartials];  // yexp row of each routed partial, -1: the CPU's expert
  __shared__ int s_ok;
  // one routed partial per thread: the row of the token's j-th expert, split r; the header
  // word is a vector load so that it goes out with the position loads (a scalar load would
  // be waited for first)
  const int ncpu = __hip_atomic_load(&v.hdr[HDR_NCPU], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < nrouted; i += FT) {
    const int j = i / RS, r = i - j * RS;
    const int pos = v.inv_pos[t * d.K + j];
    s_row[i] = ncpu > 0 && v.row_cpu[pos] ? -1 : pos * RS + r;
  }
  if (ncpu > 0 && threadIdx.x == 0) s_ok = wait_host_answer(v);
  __syncthreads();
  if (c >= d.H) return;
  constexpr int CH = 32;
  float s = 0.f;
  for (int base = 0; base < nrouted; base += CH) {
    int row[CH];
    float pv[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) row[q] = s_row[base + q < nrouted ? base + q : nrouted - 1];
#pragma unroll
    for (int q = 0; q < CH; ++q) pv[q] = v.yexp[(size_t)(row[q] < 0 ? 0 : row[q]) * d.H + c];
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (base + q < nrouted && row[q] >= 0) s += pv[q];
  }
  if (ncpu > 0 && s_ok) {
    const float* yc = (const float*)((const unsigned char*)v.mail + mail_y_offset(d.H));
    s += __hip_atomic_load(yc + (size_t)t * d.H + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (d.has_shared) {
    for (int r0 = 0; r0 < RS; r0 += 8) {  // the shared expert's row splits, 8 loads at a time
      float sh[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        sh[q] = v.yexp_shared[((size_t)t * RS + (r0 + q < RS ? r0 + q : RS - 1)) * d.H + c];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (r0 + q < RS) s += sh[q];
    }
  }
  a.y[(size_t)t * d.H + c] = f32_to_bf16_rne(s);
}

// ---------------------------------------------------------------- fused one-token role
// At one token (bf16 weights, no shared expert) the gate/up and down rows of an expert's
// intermediate block run in one workgroup, so a single launch streams every blob of the step
// and no activation row leaves the chip.  The workgroup owns FR = 8 intermediate rows: each
// of its 4 waves computes the gate and up sums of two rows as in the gate/up role, the 8
// activations meet in LDS, and the workgroup multiplies them into its 8 rows of WdT for every
// output column.  Thread (column chunk cc, row group rg) holds NR rows of 8 columns; the
// FR / NR row groups are added in LDS in a fixed order and the workgroup writes one fp32
// partial per (expert row, row block).  Every weight load of the workgroup - its gate/up
// chunks and its WdT rows - is issued before the first product.  The combine adds the
// I / FR partials of each of the token's experts.
constexpr int FR = 8;            // intermediate rows per fused workgroup (two per wave)
constexpr int FFT = FR / 2 * 64;  // threads per fused workgroup
constexpr int FWPE = 1;           // lower bound of waves per SIMD asked of the compiler
constexpr int kMaxPartialsF = 1024;  // top_k * I / FR, checked on the host

template <int NR>
__device__ void fused_role(const FfnArgs& a, const Entry& en, int rb, u32x4v (&xr)[GN][1],
                           float* s_a, float* s_red) {
  const Dims& d = a.d;
  const int H = d.H, I = d.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (rb == 0 && tid == 0) {
    atomicAdd(&a.v.stats[STAT_FFN_BYTES], (unsigned long long)d.S);
    if (a.timed) atomicAdd(&a.v.stats[STAT_TIMED_FUSED_BYTES], (unsigned long long)d.S);
  }
  const float wt = en.shared ? 1.0f : a.v.row_w[en.row0];
  const int i0 = rb * FR + wave, i1 = i0 + FR / 2;
  const size_t hbytes = 2 * (size_t)H, rbytes = 2 * hbytes;  // bf16 half-row, gate|up row
  const unsigned char* r0 = en.blob + (size_t)i0 * rbytes;
  const unsigned char* r1 = en.blob + (size_t)i1 * rbytes;
  const int ngq = H / 8;  // 16-byte chunks per half-row and per WdT row
  const int cc = tid % ngq, rg = tid / ngq;
  const unsigned char* wdt =
      en.blob + (size_t)I * rbytes + (size_t)(rb * FR + rg * NR) * hbytes + (size_t)cc * 16;
  float g0 = 0.f, u0 = 0.f, g1 = 0.f, u1 = 0.f;
  u32x4v wd[NR];
  for (int kb = 0; kb * 64 < ngq; kb += GN) {
    u32x4v wg0[GN], wu0[GN], wg1[GN], wu1[GN];
#pragma unroll
    for (int k = 0; k < GN; ++k) {
      int c = (kb + k) * 64 + lane;
      c = c < ngq ? c : ngq - 1;  // in-row address; masked below
      wg0[k] = ld_stream<u32x4v>(r0 + (size_t)c * 16);
      wu0[k] = ld_stream<u32x4v>(r0 + hbytes + (size_t)c * 16);
      wg1[k] = ld_stream<u32x4v>(r1 + (size_t)c * 16);
      wu1[k] = ld_stream<u32x4v>(r1 + hbytes + (size_t)c * 16);
    }
    if (kb == 0) {  // the WdT rows go out behind the first pass, before any product
#pragma unroll
      for (int r = 0; r < NR; ++r) wd[r] = ld_stream<u32x4v>(wdt + (size_t)r * hbytes);
    } else {
      load_x1<FMT_BF16>(a, kb, lane, xr, a.x);
    }
#pragma unroll
    for (int k = 0; k < GN; ++k) {
      if ((kb + k) * 64 + lane < ngq) {
        const uint32_t xw[4] = {xr[k][0].x, xr[k][0].y, xr[k][0].z, xr[k][0].w};
        const uint32_t ag0[4] = {wg0[k].x, wg0[k].y, wg0[k].z, wg0[k].w};
        const uint32_t au0[4] = {wu0[k].x, wu0[k].y, wu0[k].z, wu0[k].w};
        const uint32_t ag1[4] = {wg1[k].x, wg1[k].y, wg1[k].z, wg1[k].w};
        const uint32_t au1[4] = {wu1[k].x, wu1[k].y, wu1[k].z, wu1[k].w};
        g0 = wdot<4>(ag0, xw, g0);
        u0 = wdot<4>(au0, xw, u0);
        g1 = wdot<4>(ag1, xw, g1);
        u1 = wdot<4>(au1, xw, u1);
      }
    }
  }
  float gv[2] = {g0, g1}, uv[2] = {u0, u1};
  wave_reduce_units<1>(gv, uv, lane);
  if ((lane & 31) == 0)  // lane 0 holds row i0, lane 32 row i1
    s_a[lane == 0 ? wave : wave + FR / 2] = silu(gv[0]) * uv[0] * wt;
  lds_barrier();  // the WdT rows may still be arriving
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float ar = s_a[rg * NR + r];
    float f[8];
    unpack_d<FMT_BF16>(wd[r], f);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += ar * f[c];
  }
  float* out = a.v.yfus + ((size_t)en.row0 * d.RSF + rb) * H;
  constexpr int RG = FR / NR;  // row groups (FFT / ngq)
  if constexpr (RG == 1) {
    *(float4*)(out + cc * 8) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(out + cc * 8 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    *(float4*)(s_red + (size_t)rg * H + cc * 8) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(s_red + (size_t)rg * H + cc * 8 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    __syncthreads();
    for (int c = tid; c < H; c += FFT) {
      float s = 0.f;
#pragma unroll
      for (int g = 0; g < RG; ++g) s += s_red[(size_t)g * H + c];
      out[c] = s;
    }
  }
}

// Combine of the fused partials: y[t] = bf16( sum over the token's experts and row blocks
// + y_cpu[t] ).  A workgroup owns 32 columns of one token; thread (partial lane pl, column
// quad cq) adds every 32nd partial with 16-byte loads, CFP of them in flight at once; the 32
// partial lanes are added in LDS in a fixed order.
constexpr int CFC = 32;         // output columns per combine workgroup
constexpr int CFL = FT / (CFC / 4);  // partial lanes
constexpr int CFP = 24;         // partials per thread per round

__device__ void combine_fused_role(const FfnArgs& a, int cblk) {
  const Dims& d = a.d;
  const Dev& v = a.v;
  const int per_tok = d.H / CFC;
  const int t = cblk / per_tok, c0 = (cblk % per_tok) * CFC;
  const int RSF = d.RSF, nrouted = d.K * RSF;
  __shared__ int s_row[kMaxPartialsF];
  __shared__ __align__(16) float s_sum[CFL * CFC];
  __shared__ int s_ok;
  const int ncpu = __hip_atomic_load(&v.hdr[HDR_NCPU], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < nrouted; i += FT) {
    const int j = i / RSF, r = i - j * RSF;
    const int pos = v.inv_pos[t * d.K + j];
    s_row[i] = ncpu > 0 && v.row_cpu[pos] ? -1 : pos * RSF + r;
  }
  if (ncpu > 0 && threadIdx.x == 0) s_ok = wait_host_answer(v);
  __syncthreads();
  const int cq = threadIdx.x % (CFC / 4), pl = threadIdx.x / (CFC / 4);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int base = pl; base < nrouted; base += CFL * CFP) {
    int row[CFP];
    float4 pv[CFP];
#pragma unroll
    for (int q = 0; q < CFP; ++q)
      row[q] = base + CFL * q < nrouted ? s_row[base + CFL * q] : -1;
#pragma unroll
    for (int q = 0; q < CFP; ++q)
      pv[q] = *(const float4*)(v.yfus + (size_t)(row[q] < 0 ? 0 : row[q]) * d.H + c0 + cq * 4);
#pragma unroll
    for (int q = 0; q < CFP; ++q)
      if (row[q] >= 0) {
        s.x += pv[q].x; s.y += pv[q].y; s.z += pv[q].z; s.w += pv[q].w;
      }
  }
  *(float4*)(s_sum + pl * CFC + cq * 4) = s;
  __syncthreads();
  if (threadIdx.x >= CFC) return;
  const int c = c0 + threadIdx.x;
  float y = 0.f;
#pragma unroll
  for (int p = 0; p < CFL; ++p) y += s_sum[p * CFC + threadIdx.x];
  if (ncpu > 0 && s_ok) {
    const float* yc = (const float*)((const unsigned char*)v.mail + mail_y_offset(d.H));
    y += __hip_atomic_load(yc + (size_t)t * d.H + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  a.y[(size_t)t * d.H + c] = f32_to_bf16_rne(y);
}

template <int FMT>
static constexpr int down_hc() {
  return DTC * Fmt<FMT>::DC;
}

template <int FMT, int NTOK>
__global__ __launch_bounds__(FT) void ffn_gate_up_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nra = a.d.I / RA;
  u32x4v xr[GuX<FMT>::GNF][GuX<FMT>::XV];
  if constexpr (NTOK == 1) {
    // at one token the activations do not depend on the plan: they go out before the entry
    load_x1<FMT>(a, 0, threadIdx.x & 63, xr, a.x);
    Entry en;
    if (!resolve(a, blockIdx.x / nra, en)) return;
    gate_up_role<FMT, 1>(a, en, blockIdx.x % nra, xr, nullptr, a.x);
  } else {
    Entry en;
    if (!resolve(a, blockIdx.x / nra, en)) return;
    if (FMT != FMT_MXFP4 && en.ntok == 1 && !en.shared) {
      // an expert that one token of the step uses (the common case across streams): that
      // token's activations in registers, as at one token, with no staging in LDS (not for
      // e2m1 weights, whose 16-byte chunk needs 64 bytes of activations: there the four waves
      // share one staged copy)
      const uint16_t* xrow = a.x + (size_t)a.v.row_tok[en.row0] * a.d.H;
      load_x1<FMT>(a, 0, threadIdx.x & 63, xr, xrow);
      gate_up_role<FMT, 1>(a, en, blockIdx.x % nra, xr, nullptr, xrow);
    } else {
      gate_up_role<FMT, NTOK>(a, en, blockIdx.x % nra, xr, (uint16_t*)smem, nullptr);
    }
  }
}

template <int FMT, int NTOK>
static size_t gate_up_lds_bytes(const Dims& d) {
  return NTOK > 1 ? (size_t)NTOK * gate_up_stage_chunks<FMT>(d.H / Fmt<FMT>::EPL) *
                        Fmt<FMT>::EPL * 2
                  : 0;
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

template <int NR>
__global__ __launch_bounds__(FFT, FWPE) void ffn_fused_kernel(FfnArgs a) {
  __shared__ float s_a[FR];
  extern __shared__ __align__(16) unsigned char smem[];  // row-group sums: (FR / NR) * H fp32
  const int nrb = a.d.I / FR;
  u32x4v xr[GN][1];
  // the activations do not depend on the plan: they go out before the entry
  load_x1<FMT_BF16>(a, 0, threadIdx.x & 63, xr, a.x);
  Entry en;
  if (!resolve(a, blockIdx.x / nrb, en)) return;  // uniform per workgroup
  fused_role<NR>(a, en, blockIdx.x % nrb, xr, s_a, (float*)smem);
}

__global__ __launch_bounds__(FT) void combine_fused_kernel(FfnArgs a) {
  combine_fused_role(a, blockIdx.x);
}

// Row blocks of the fused one-token FFN for this shape, or 0 when the shape takes the
// gate/up + down kernels: bf16 weights without a shared expert, H / 8 chunks per row that
// divide the FFT threads with FR * (H / 8) / FFT in {1, 2, 4, 8} rows per thread (at most FR),
// and at most kMaxPartialsF partials per output.
int fused_row_blocks(const Dims& d) {
  if (d.fmt != FMT_BF16 || d.has_shared || d.I % FR != 0 || d.H % 64 != 0) return 0;
  const int ngq = d.H / 8;
  if (ngq > FFT || FFT % ngq != 0) return 0;
  const int nr = FR * ngq / FFT;
  if (nr < 1 || (nr & (nr - 1)) != 0 || nr > 8 || nr > FR) return 0;
  if (d.K * (d.I / FR) > kMaxPartialsF) return 0;
  return d.I / FR;
}

template <int NR>
static hipError_t launch_fused_nr(const FfnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                  hipEvent_t e1) {
  return launch_timed(ffn_fused_kernel<NR>, dim3(grid), dim3(FFT), sizeof(float) * FFT * 8, s,
                      e0, e1, a);
}

// stage 0: the fused kernel over the launch's entries; stage 1: the combine (when a.NC > 0)
static hipError_t launch_fused(const FfnArgs& a, int stage, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
  const Dims& d = a.d;
  const int grid = stage == 0 ? a.NE * d.RSF : (a.NC > 0 ? a.T * (d.H / CFC) : 0);
  if (grid <= 0) {  // nothing to run; keep the timing events valid
    hipError_t e = e0 ? hipEventRecord(e0, s) : hipSuccess;
    if (e == hipSuccess && e1) e = hipEventRecord(e1, s);
    return e;
  }
  if (stage == 1)
    return launch_timed(combine_fused_kernel, dim3(grid), dim3(FT), 0, s, e0, e1, a);
  switch (FR * (d.H / 8) / FFT) {
    case 1: return launch_fused_nr<1>(a, grid, s, e0, e1);
    case 2: return launch_fused_nr<2>(a, grid, s, e0, e1);
    case 4: return launch_fused_nr<4>(a, grid, s, e0, e1);
    default: return launch_fused_nr<8>(a, grid, s, e0, e1);
  }
}

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
    return launch_with_lds(ffn_gate_up_kernel<FMT, NTOK>, a.NE * (d.I / RA),
                           gate_up_lds_bytes<FMT, NTOK>(d), a, s, e0, e1);
  const size_t dlds =
      sizeof(float) * ((size_t)4 * NTOK * HC + (NTOK > 1 ? (size_t)NTOK * (d.I / d.RS) : 0));
  hipError_t e = launch_with_lds(ffn_down_kernel<FMT, NTOK>, a.NE * (d.H / HC) * d.RS, dlds, a,
                                 s, e0, a.NC > 0 ? nullptr : e1);
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
  if (d.K * d.RS > kMaxPartials) return hipErrorInvalidValue;
  const int nc = with_combine ? T * ((d.H + FT - 1) / FT) : 0;
  FfnArgs a{d, v, (const uint16_t*)x, (const unsigned char*)arena,
            (const unsigned char*)shared_blob, (uint16_t*)y, sel, group, ngroups, T,
            max_entries > 0 ? max_entries : 0, nc, e0 != nullptr};
  const int ntok = decode_ntok(T);
  if (ntok == 1 && d.RSF > 0) return launch_fused(a, stage, s, e0, e1);
  switch (d.fmt) {
    case FMT_BF16: return launch_fmt<FMT_BF16>(a, ntok, stage, s, e0, e1);
    case FMT_FP8: return launch_fmt<FMT_FP8>(a, ntok, stage, s, e0, e1);
    default: return launch_fmt<FMT_MXFP4>(a, ntok, stage, s, e0, e1);
  }
}

}  // namespace moe
