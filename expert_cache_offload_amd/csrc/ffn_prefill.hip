// SwiGLU expert FFN for a step of many tokens: grouped GEMMs on the bf16 matrix cores.
//
// Same computation as at decode (y_t = sum_j w_tj * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)) over
// the token's top-k experts, plus a shared expert with weight 1 when the model has one),
// with every expert's rows gathered in the expert-sorted order of the plan.  Hit experts
// run first and each fill group as soon as its copy has landed ("FreeToken：在消费级
// NVIDIA GPU 上进行 MoE 推理", section on the problems FreeToken solves: the next group
// transfers while this group computes; the same page's measurements put the cost of
// turning this overlap off at about a quarter of prefill speed).
//
// Gfx950 design.  Dense contractions on v_mfma_f32_32x32x16_bf16 (fp32 accumulation):
//   gate/up  - tile = 256 rows x 128 intermediate rows; the 256 GEMM columns are the 128
//              gate rows and the 128 up rows, so each wave holds gate and up of the same
//              (row, i) in the same lane and the epilogue a = silu(g) * u * w is per lane;
//              eight waves, each 64 rows x 64 intermediate rows (eight 32 x 32 MFMA tiles:
//              six 16-byte LDS reads feed eight MFMAs, the next step's reads issued in the
//              same asm block as this step's MFMAs); rows are gathered from x by the plan's
//              row -> token map; a is stored bf16;
//   down     - tile = 256 rows x 256 output columns over the stored transpose WdT
//              ([contraction][column]), loaded into LDS as stored and read with gfx950's
//              transposing LDS reads; eight waves, 64 x 128 each; fp32 partial rows per
//              (token, choice);
//   combine  - y[t] = bf16(sum over the token's k rows (+ shared) in a fixed order).
// A 64-wide contraction stage in LDS with the next stage's global loads in flight during the
// MFMAs.  Workgroups are persistent over the launch's tiles, whose count depends on the plan
// (read on the device): a prefix over the launch's entries maps a tile to its expert, row
// tile and column tile.
#include "moe_dev.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int PFT = 256;        // threads of the combine kernel
constexpr int BK = 64;          // contraction per LDS stage (128-byte row segments)
constexpr int GBI = 128;        // intermediate rows per gate/up tile (256 GEMM columns)
constexpr int kMaxEntriesPf = 1040;

struct PfArgs {
  Dims d;
  Dev v;
  const uint16_t* x;  // [T][H] bf16
  const unsigned char* arena;
  const unsigned char* shared_blob;
  uint16_t* y;        // [T][H] bf16
  int sel;            // 0: hits + shared, 1: miss group `group` of `ngroups`, 2: all
  int group;
  int ngroups;
  int T;
  int timed;
};

struct PfEntry {
  const unsigned char* blob;
  int rows;    // routed: tokens of the expert; shared: T
  int row0;    // first expert-sorted row (routed) or 0 (shared)
  bool shared;
};

__device__ __forceinline__ int pf_launch_entries(const PfArgs& a, int& first) {
  const int nHit = a.v.hdr[HDR_NHIT], nMiss = a.v.hdr[HDR_NMISS];
  const int nHS = nHit + a.d.has_shared;
  if (a.sel == 0) {
    first = 0;
    return nHS;
  }
  if (a.sel == 2) {
    first = 0;
    return nHS + nMiss;
  }
  const int m0 = (int)((long long)a.group * nMiss / a.ngroups);
  const int m1 = (int)((long long)(a.group + 1) * nMiss / a.ngroups);
  first = nHS + m0;
  return m1 - m0;
}

__device__ __forceinline__ PfEntry pf_entry(const PfArgs& a, int g) {
  const int nHit = a.v.hdr[HDR_NHIT];
  PfEntry en;
  if (a.d.has_shared && g == nHit) {
    en.blob = a.shared_blob;
    en.rows = a.T;
    en.row0 = 0;
    en.shared = true;
    return en;
  }
  const int4 e = a.v.ent[g < nHit ? g : g - a.d.has_shared];
  en.blob = a.arena + (size_t)e.x * (size_t)a.d.S;
  en.rows = e.y;
  en.row0 = e.z;
  en.shared = false;
  return en;
}

// Row tiles of TBM rows of the launch's entries: s_mt[j] = first row tile of entry j
// (exclusive prefix), s_mt[n] = total.  Returns n.
template <int TBM>
__device__ int pf_tile_prefix(const PfArgs& a, int* s_mt, int& first) {
  const int n = pf_launch_entries(a, first);
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const PfEntry en = pf_entry(a, first + j);
    s_mt[j + 1] = (en.rows + TBM - 1) / TBM;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_mt[0] = 0;
    for (int j = 1; j <= n; ++j) s_mt[j] += s_mt[j - 1];
  }
  __syncthreads();
  return n;
}

__device__ __forceinline__ int pf_find(const int* s_mt, int n, int mt) {
  int lo = 0, hi = n - 1;  // last j with s_mt[j] <= mt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mt[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float pf_silu(float z) { return z / (1.0f + __expf(-z)); }

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that consecutive tiles
// (the column tiles of one row tile, the row tiles of one expert) run on the same XCD and
// meet their shared rows in that XCD's L2.  The grid is a multiple of 8.
__device__ __forceinline__ int xcd_order() {
  return (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8);
}

__device__ __forceinline__ uint16_t pf_bf16(float f) { return f32_to_bf16_rne(f); }

typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {  // byte address in LDS
  return (uint32_t)(uintptr_t)(const lds_u16_t*)p;
}

// One 16-deep step of the gate/up tile in one asm block: the next step's six fragment reads
// (two row tiles of x at byte offsets 0 and 4096 from `aa`; gate and up of two column tiles at
// 0, 4096, 16384 and 20480 from `ba`) go out first, then this step's eight MFMAs
// (c[rr * 4 + g * 2 + cc] += a[rr] x b[g * 2 + cc]), and the block ends waiting for its reads,
// which land under the MFMAs.  Written as asm because the compiler, with global-to-LDS loads in
// the kernel, waits for every outstanding LDS read before each MFMA group.  The block's MFMAs
// are invisible to the compiler's hazard tracking: their accumulators are read by compiled
// code only after gu_drain().
__device__ __forceinline__ void gu_step(f32x16_t& c0, f32x16_t& c1, f32x16_t& c2, f32x16_t& c3,
                                        f32x16_t& c4, f32x16_t& c5, f32x16_t& c6, f32x16_t& c7,
                                        const bf16x8_t (&a)[2], const bf16x8_t (&b)[4],
                                        bf16x8_t (&na)[2], bf16x8_t (&nb)[4], uint32_t aa,
                                        uint32_t ba) {
  asm volatile(
      "ds_read_b128 %0, %20\n\t"
      "ds_read_b128 %1, %20 offset:4096\n\t"
      "ds_read_b128 %2, %21\n\t"
      "ds_read_b128 %3, %21 offset:4096\n\t"
      "ds_read_b128 %4, %21 offset:16384\n\t"
      "ds_read_b128 %5, %21 offset:20480\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %14, %16, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %14, %17, %7\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %14, %18, %8\n\t"
      "v_mfma_f32_32x32x16_bf16 %9, %14, %19, %9\n\t"
      "v_mfma_f32_32x32x16_bf16 %10, %15, %16, %10\n\t"
      "v_mfma_f32_32x32x16_bf16 %11, %15, %17, %11\n\t"
      "v_mfma_f32_32x32x16_bf16 %12, %15, %18, %12\n\t"
      "v_mfma_f32_32x32x16_bf16 %13, %15, %19, %13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(na[0]), "=&v"(na[1]), "=&v"(nb[0]), "=&v"(nb[1]), "=&v"(nb[2]), "=&v"(nb[3]),
        "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
      : "v"(a[0]), "v"(a[1]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(aa), "v"(ba)
      : "memory");
}

// The last step of a stage: its eight MFMAs only.
__device__ __forceinline__ void gu_step_last(f32x16_t& c0, f32x16_t& c1, f32x16_t& c2,
                                             f32x16_t& c3, f32x16_t& c4, f32x16_t& c5,
                                             f32x16_t& c6, f32x16_t& c7, const bf16x8_t (&a)[2],
                                             const bf16x8_t (&b)[4]) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %8, %10, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %8, %11, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %12, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %8, %13, %3\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %9, %10, %4\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %9, %11, %5\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %9, %12, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %9, %13, %7"
      : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
      : "v"(a[0]), "v"(a[1]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3])
      : "memory");
}

// Wait states after asm MFMAs before compiled code reads their results (the 16-pass
// 32 x 32 MFMA needs up to 18 before a VALU read of its destination).
__device__ __forceinline__ void gu_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// ---------------------------------------------------------------- gate / up
// Tile = 256 rows x 128 intermediate rows (256 GEMM columns: 128 gate rows, then the 128 up
// rows of the same i), one workgroup of eight waves per CU in a 4 x 2 arrangement; a wave owns
// 64 rows x 64 i: eight 32 x 32 MFMA tiles (two row tiles times gate and up times two column
// tiles) fed by six 16-byte LDS reads per 16-deep step (written ahead of the previous step's
// MFMAs; the compiler interleaves them).  Operands go from global memory straight into LDS
// (gfx950's 16-byte global-to-LDS loads: no registers, no LDS store instructions) in two
// stages of 64 contraction elements (32 KiB of rows + 32 KiB of weights each) with one barrier
// per stage: a stage's loads are issued right after the barrier that frees its buffer and land
// while the other stage computes.  Rows are 128 bytes without padding; 16-byte chunk c of row r
// sits at chunk c ^ ((r / 2) % 8): gfx950's LDS serves a 16-byte read 16 lanes (256 bytes, all
// 64 banks) at a time, and the 16 consecutive rows such a group reads at one chunk then fill
// distinct 16-byte bank slots (row parity times the XOR).  Rows past the expert's count load a
// valid row: they only reach output rows that are never stored.
constexpr int GU_T = 512;                         // threads (8 waves)
constexpr int GU_BM = 256;                        // rows per gate/up tile
constexpr int GU_STAGE = (GU_BM + 2 * GBI) * BK;  // bf16 elements per LDS stage
constexpr int GU_LPW = GU_STAGE * 2 / (16 * 64) / (GU_T / 64);  // 1 KiB loads per wave per stage (8)

__device__ __forceinline__ int gu_sx(int row) { return (row >> 1) & 7; }  // chunk XOR of a row
__device__ __forceinline__ int gu_swz(int row, int chunk) {  // element offset of (row, chunk)
  return row * BK + ((chunk ^ gu_sx(row)) << 3);
}

__global__ __launch_bounds__(GU_T, 1) void ffn_prefill_gate_up_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint16_t pf_smem[];  // 2 stages: [rows][BK] then [cols][BK]
  __shared__ int s_mt[kMaxEntriesPf + 1];
  __shared__ float s_w[GU_BM];  // routing weight of each row of the tile
  const Dims& d = a.d;
  const int H = d.H, I = d.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int first;
  const int n = pf_tile_prefix<GU_BM>(a, s_mt, first);
  const int NT = I / GBI;
  const int ntiles = s_mt[n] * NT;
  const int nst = H / BK;  // contraction stages
  // global-to-LDS loads: load i of wave w fills LDS rows 8 (w * GU_LPW + i) .. + 7 of the
  // stage (rows 0..255: x rows, 256..511: weight rows); lane l brings row ... + l / 8,
  // physical chunk l % 8, which holds logical chunk (l % 8) ^ gu_sx(row)
  const int lrow = lane >> 3;
  for (int tile = xcd_order(); tile < ntiles; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile - mt * NT;
    const int j = pf_find(s_mt, n, mt);
    const PfEntry en = pf_entry(a, first + j);
    if (threadIdx.x == 0 && mt == s_mt[j] && nt == 0) {
      atomicAdd(&a.v.stats[STAT_FFN_BYTES], (unsigned long long)d.S);
      if (a.timed) atomicAdd(&a.v.stats[STAT_TIMED_BLOB_BYTES], (unsigned long long)d.S);
    }
    const int m0 = (mt - s_mt[j]) * GU_BM;
    const int i0 = nt * GBI;
    if ((int)threadIdx.x < GU_BM) {  // read by the epilogue, after the k loop's barriers
      const int r = m0 + threadIdx.x;
      s_w[threadIdx.x] = r >= en.rows ? 0.f : en.shared ? 1.0f : a.v.row_w[en.row0 + r];
    }
    // this lane's GU_LPW source rows: x rows gathered by token (T * H < 2^31), weight rows
    // (tile column c < GBI: gate row i0 + c, else up row i0 + c - GBI)
    const uint16_t* src[GU_LPW];
#pragma unroll
    for (int i = 0; i < GU_LPW; ++i) {
      const int row = (wave * GU_LPW + i) * 8 + lrow;  // stage row 0 .. 511
      const int lc = (lane & 7) ^ gu_sx(row);
      if (row < GU_BM) {
        const int r = m0 + row;
        const int tok = r >= en.rows ? (en.shared ? 0 : a.v.row_tok[en.row0]) :
                        en.shared ? r : a.v.row_tok[en.row0 + r];
        src[i] = a.x + (size_t)tok * H + lc * 8;
      } else {
        const int col = row - GU_BM, g = col >> 7, c = col & (GBI - 1);
        src[i] = (const uint16_t*)en.blob + (size_t)(2 * (i0 + c) + g) * H + lc * 8;
      }
    }
    f32x16_t acc[2][2][2];  // [row tile][gate, up][column tile]
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[rr][g][cc][q] = 0.f;
    auto load_stage = [&](int st, int buf) {
      uint16_t* dst = pf_smem + buf * GU_STAGE + wave * GU_LPW * 8 * BK;
      const int k0 = st * BK;
#pragma unroll
      for (int i = 0; i < GU_LPW; ++i)
        __builtin_amdgcn_global_load_lds(src[i] + k0, dst + i * 8 * BK, 16, 0, 0);
    };
    load_stage(0, 0);
    load_stage(1, 1);  // H >= 256: at least 4 stages
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt <= 8: stage 0 has landed
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const uint16_t* As = pf_smem + (st & 1) * GU_STAGE;
      const uint16_t* Bs = As + GU_BM * BK;
      // this lane's fragment addresses of step kk: x rows wm * 64 + (lane % 32) (+ 32 for the
      // second row tile) and weight rows wn * 64 + (lane % 32) (+ 32 per column tile, + GBI
      // for up), all at the lane's 16-byte chunk 2 kk + lane / 32
      auto aaddr = [&](int kk) {
        return lds_addr(As + gu_swz(wm * 64 + (lane & 31), 2 * kk + (lane >> 5)));
      };
      auto baddr = [&](int kk) {
        return lds_addr(Bs + gu_swz(wn * 64 + (lane & 31), 2 * kk + (lane >> 5)));
      };
      bf16x8_t f0a[2], f0b[4], f1a[2], f1b[4];
      {  // step 0: plain loads (the compiler waits for them before the first block)
        const int ch = lane >> 5;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          f0a[rr] = *(const bf16x8_t*)(As + gu_swz(wm * 64 + rr * 32 + (lane & 31), ch));
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
            f0b[g * 2 + cc] =
                *(const bf16x8_t*)(Bs + gu_swz(g * GBI + wn * 64 + cc * 32 + (lane & 31), ch));
      }
      static_assert(BK / 16 == 4, "four steps per stage");
      gu_step(acc[0][0][0], acc[0][0][1], acc[0][1][0], acc[0][1][1], acc[1][0][0], acc[1][0][1],
              acc[1][1][0], acc[1][1][1], f0a, f0b, f1a, f1b, aaddr(1), baddr(1));
      gu_step(acc[0][0][0], acc[0][0][1], acc[0][1][0], acc[0][1][1], acc[1][0][0], acc[1][0][1],
              acc[1][1][0], acc[1][1][1], f1a, f1b, f0a, f0b, aaddr(2), baddr(2));
      gu_step(acc[0][0][0], acc[0][0][1], acc[0][1][0], acc[0][1][1], acc[1][0][0], acc[1][0][1],
              acc[1][1][0], acc[1][1][1], f0a, f0b, f1a, f1b, aaddr(3), baddr(3));
      gu_step_last(acc[0][0][0], acc[0][0][1], acc[0][1][0], acc[0][1][1], acc[1][0][0],
                   acc[1][0][1], acc[1][1][0], acc[1][1][1], f1a, f1b);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's loads of stage st + 1 landed
      __syncthreads();  // every wave is done with buffer st & 1; stage st + 1 is visible
      if (st + 2 < nst) load_stage(st + 2, st & 1);
    }
    gu_drain();
    // epilogue: lane holds column i = i0 + wn*64 + cc*32 + lane%32 for 16 rows of each row tile
    uint16_t* act = en.shared ? a.v.pact_shared : a.v.pact;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int i = i0 + wn * 64 + cc * 32 + (lane & 31);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = m0 + wm * 64 + rr * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
          if (r < en.rows) {
            const float val = pf_silu(acc[rr][0][cc][q]) * acc[rr][1][cc][q] * s_w[r - m0];
            act[(size_t)(en.row0 + r) * I + i] = pf_bf16(val);
          }
        }
      }
    }
    __syncthreads();  // s_w and the LDS stages are rewritten by the next tile
  }
}

// ---------------------------------------------------------------- down
// Tile = 256 rows x 256 output columns, one workgroup of eight waves per CU in a 4 x 2
// arrangement; a wave owns 64 rows x 128 columns (eight 32 x 32 MFMA tiles).  Both operands go
// from global memory straight into LDS in two stages of 64 contraction elements: the a rows
// (32 KiB, 128-byte rows, chunk c of row r at c ^ ((r / 2) % 8), as in gate/up) and 64 rows of the
// stored transpose WdT as they lie in memory (32 KiB, [contraction][column], 512-byte rows).
// The MFMA's B operand needs eight consecutive contraction values of one column per lane; the
// gfx950 transposing LDS read (ds_read_b64_tr_b16) gives four: within each group of 16 lanes,
// lane j receives element j % 4 of the 8-byte reads of lanes 4m + j / 4 (m = 0..3), so lane
// 4m + q of group g points at contraction row 8 (g / 2) + 4 h + m and columns
// 16 (g % 2) + 4 q .. + 3 of a 32-column MFMA tile, and two reads (h = 0, 1) make a fragment.
// One such read covers 4 contraction rows x 32 bytes per 16 lanes and 4 rows x 64 bytes per
// 32 lanes; WdT's 16-byte chunk c of contraction row k sits at c ^ x(k % 4) with
// x = {0, 6, 10, 12}, which puts both footprints on distinct banks.
constexpr int DN_T = 512;   // threads (8 waves)
constexpr int DN_BM = 256;  // rows per down tile
constexpr int DN_BN = 256;  // output columns per down tile
constexpr int DN_ASTAGE = DN_BM * BK;  // bf16 elements of a rows per stage
constexpr int DN_STAGE = DN_ASTAGE + BK * DN_BN;
constexpr int DN_ALPW = DN_ASTAGE * 2 / 1024 / (DN_T / 64);     // 1 KiB a loads per wave (4)
constexpr int DN_BLPW = BK * DN_BN * 2 / 1024 / (DN_T / 64);    // 1 KiB WdT loads per wave (4)

__device__ __forceinline__ int dn_bx(int k) {  // chunk XOR of WdT contraction row k
  return (0xCA60 >> (4 * (k & 3))) & 15;         // nibbles 0, 6, 10, 12
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// The eight transposing reads of one 16-deep step: two (byte offsets OFF and OFF + 2048, four
// contraction rows apart) from each of this lane's four column-tile addresses, with the wait
// for them in the same block.  Written as one asm block because the compiler's wait insertion
// treats its transposing-read builtin as aliasing the global-to-LDS loads in flight and waits
// for those first, which would serialise every stage's loads with its MFMAs; the stages are
// ordered by the explicit wait and barrier at the end of each stage instead.
template <int OFF>
__device__ __forceinline__ void dn_read_b(s16x4_t (&r)[8], uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%c13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%c13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%c13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%c13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(OFF), "n"(OFF + 4 * DN_BN * 2)
      : "memory");
}

__global__ __launch_bounds__(DN_T, 1) void ffn_prefill_down_kernel(PfArgs a) {
  extern __shared__ __align__(16) uint16_t pf_smem[];  // 2 stages: a [rows][BK], WdT [BK][cols]
  __shared__ int s_mt[kMaxEntriesPf + 1];
  const Dims& d = a.d;
  const int H = d.H, I = d.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int first;
  const int n = pf_tile_prefix<DN_BM>(a, s_mt, first);
  const int NT = H / DN_BN;
  const int ntiles = s_mt[n] * NT;
  const int nst = I / BK;  // contraction stages (I is a multiple of 128)
  // a loads: load i of wave w fills rows 8 (w * DN_ALPW + i) + lane / 8, physical chunk lane % 8
  const int arow = lane >> 3;
  // WdT loads: load i of wave w fills contraction rows 2 (w * DN_BLPW + i) + lane / 32, physical
  // chunk lane % 32 (the row's parity is lane / 32; its residue mod 4 is set per load below)
  const int brow = lane >> 5, bpc = lane & 31;
  // transposing reads: this lane's contraction row and column within a 32 x 32 MFMA B tile
  const int tg = lane >> 4, tm = (lane >> 2) & 3, tq = lane & 3;
  const int tk = 8 * (tg >> 1) + tm;        // + 16 kk + 4 h: always tm modulo 4
  const int tcol = 16 * (tg & 1) + 4 * tq;  // + 32 cc + 128 wn
  int toff[4];  // element offset of this lane's read of column tile cc at kk = h = 0
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int col = wn * 128 + cc * 32 + tcol;
    toff[cc] = tk * DN_BN + (((col >> 3) ^ dn_bx(tm)) << 3) + (col & 7);
  }
  for (int tile = xcd_order(); tile < ntiles; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile - mt * NT;
    const int j = pf_find(s_mt, n, mt);
    const PfEntry en = pf_entry(a, first + j);
    const int m0 = (mt - s_mt[j]) * DN_BM;
    const int n0 = nt * DN_BN;
    const uint16_t* act = (en.shared ? a.v.pact_shared : a.v.pact) + (size_t)en.row0 * I;
    const uint16_t* wdt = (const uint16_t*)en.blob + (size_t)2 * I * H;  // WdT [I][H]
    const uint16_t* asrc[DN_ALPW];
    const uint16_t* bsrc[DN_BLPW];
#pragma unroll
    for (int i = 0; i < DN_ALPW; ++i) {
      const int tr = (wave * DN_ALPW + i) * 8 + arow;  // tile row
      const int r = m0 + tr;                             // rows past the count read row 0
      asrc[i] = act + (size_t)(r < en.rows ? r : 0) * I + (((lane & 7) ^ gu_sx(tr)) << 3);
    }
#pragma unroll
    for (int i = 0; i < DN_BLPW; ++i) {
      const int k = (wave * DN_BLPW + i) * 2 + brow;  // contraction row within the stage
      bsrc[i] = wdt + (size_t)k * H + n0 + ((bpc ^ dn_bx(k)) << 3);
    }
    f32x16_t acc[2][4];  // [row tile][column tile]
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[rr][cc][q] = 0.f;
    auto load_stage = [&](int st, int buf) {
      uint16_t* da = pf_smem + buf * DN_STAGE + wave * DN_ALPW * 8 * BK;
      uint16_t* db = pf_smem + buf * DN_STAGE + DN_ASTAGE + wave * DN_BLPW * 2 * DN_BN;
      const int k0 = st * BK;
#pragma unroll
      for (int i = 0; i < DN_ALPW; ++i)
        __builtin_amdgcn_global_load_lds(asrc[i] + k0, da + i * 8 * BK, 16, 0, 0);
#pragma unroll
      for (int i = 0; i < DN_BLPW; ++i)
        __builtin_amdgcn_global_load_lds(bsrc[i] + (size_t)k0 * H, db + i * 2 * DN_BN, 16, 0, 0);
    };
    load_stage(0, 0);
    load_stage(1, 1);  // I >= 128: at least 2 stages
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt <= 8: stage 0 has landed
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const uint16_t* As = pf_smem + (st & 1) * DN_STAGE;
      const uint32_t b0 = lds_addr(As + toff[0]), b1 = lds_addr(As + toff[1]);
      const uint32_t b2 = lds_addr(As + toff[2]), b3 = lds_addr(As + toff[3]);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        bf16x8_t af[2], bf[4];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          af[rr] = *(const bf16x8_t*)(As + gu_swz(wm * 64 + rr * 32 + (lane & 31), ch));
        s16x4_t h8[8];  // [cc][h]
        constexpr int kBOff = DN_ASTAGE * 2;  // bytes from a stage's start to its WdT rows
        if (kk == 0) dn_read_b<kBOff>(h8, b0, b1, b2, b3);
        if (kk == 1) dn_read_b<kBOff + 16 * DN_BN * 2>(h8, b0, b1, b2, b3);
        if (kk == 2) dn_read_b<kBOff + 32 * DN_BN * 2>(h8, b0, b1, b2, b3);
        if (kk == 3) dn_read_b<kBOff + 48 * DN_BN * 2>(h8, b0, b1, b2, b3);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          bf[cc] = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(h8[2 * cc], h8[2 * cc + 1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            acc[rr][cc] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rr], bf[cc], acc[rr][cc], 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's loads of stage st + 1 landed
      __syncthreads();  // every wave is done with buffer st & 1; stage st + 1 is visible
      if (st + 2 < nst) load_stage(st + 2, st & 1);
    }
    float* yrow = en.shared ? a.v.pyexp_shared : a.v.pyexp;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = m0 + wm * 64 + rr * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (r < en.rows) {
          float* out = yrow + (size_t)(en.row0 + r) * H + n0 + wn * 128 + (lane & 31);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) out[32 * cc] = acc[rr][cc][q];
        }
      }
    }
    __syncthreads();  // the LDS stages are rewritten by the next tile
  }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(PFT) void ffn_prefill_combine_kernel(PfArgs a) {
  const Dims& d = a.d;
  const int H = d.H, K = d.K;
  const int per_tok = H / PFT;  // H is a multiple of 256
  const int t = blockIdx.x / per_tok;
  const int c = (blockIdx.x % per_tok) * PFT + threadIdx.x;
  __shared__ int s_pos[16];
  if ((int)threadIdx.x < K) s_pos[threadIdx.x] = a.v.inv_pos[t * K + threadIdx.x];
  __syncthreads();
  float pv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) pv[j] = j < K ? a.v.pyexp[(size_t)s_pos[j] * H + c] : 0.f;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += pv[j];
  if (d.has_shared) s += a.v.pyexp_shared[(size_t)t * H + c];
  a.y[(size_t)t * H + c] = f32_to_bf16_rne(s);
}

constexpr int kPfGridDn = 256;  // persistent workgroups of the down GEMM (one per CU)
constexpr size_t kPfDownLds = sizeof(uint16_t) * 2 * (size_t)DN_STAGE;
constexpr int kPfGridGu = 256;  // persistent workgroups of the gate/up GEMM (one per CU)
constexpr size_t kPfGateUpLds = sizeof(uint16_t) * 2 * (size_t)GU_STAGE;

// stage 0: gate/up; stage 1: down; stage 2: combine.  e0/e1 (nullable) time the launch.
hipError_t launch_ffn_prefill(const Dims& d, const Dev& v, const void* x, const void* arena,
                              const void* shared_blob, void* y, int sel, int group, int ngroups,
                              int T, int stage, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  PfArgs a{d, v, (const uint16_t*)x, (const unsigned char*)arena,
           (const unsigned char*)shared_blob, (uint16_t*)y, sel, group, ngroups, T,
           e0 != nullptr};
  if (stage == 0) {
    const hipError_t e = hipFuncSetAttribute((const void*)ffn_prefill_gate_up_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kPfGateUpLds);
    if (e != hipSuccess) return e;
    return launch_timed(ffn_prefill_gate_up_kernel, dim3(kPfGridGu), dim3(GU_T), kPfGateUpLds, s,
                        e0, e1, a);
  }
  if (stage == 1) {
    const hipError_t e = hipFuncSetAttribute((const void*)ffn_prefill_down_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kPfDownLds);
    if (e != hipSuccess) return e;
    return launch_timed(ffn_prefill_down_kernel, dim3(kPfGridDn), dim3(DN_T), kPfDownLds, s, e0,
                        e1, a);
  }
  return launch_timed(ffn_prefill_combine_kernel, dim3(T * (d.H / PFT)), dim3(PFT), 0, s, e0, e1,
                      a);
}

bool prefill_ffn_supported(const Dims& d) {
  return d.fmt == FMT_BF16 && d.I % GBI == 0 && d.H % DN_BN == 0 && d.K <= 16 &&
         d.umax + d.has_shared <= kMaxEntriesPf;
}

}  // namespace moe
