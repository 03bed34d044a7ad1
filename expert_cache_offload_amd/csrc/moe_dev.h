// Device-side definitions shared by the expert-offload kernels and their host driver.
//
// Workspace state (persistent across steps, device memory owned by the caller):
//   key_of[max_capacity]  key held by each slot (key = layer*E + expert), -1 empty
//   stamp[max_capacity]   global step of the slot's last use, -1 empty
//   slot_of[L*E]          slot of each key, -1 when not cached
//   ctrl[16]              occupancy n, capacity C, step counter, error bits, tickets
//   stats[4]              steps, hits, misses, bytes filled
// Per-step plan (rewritten by every route launch):
//   hdr[16], U/u_slot/u_hit/hit_list/miss_list/miss_key/miss_slot/miss_victim[umax],
//   count[umax], offset[umax+1], perm/inv_pos/tk_idx/tk_w[amax], logits[max_tokens*E],
//   FFN intermediates (act) and per-expert outputs (yexp).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum : int {
  CTRL_N = 0,
  CTRL_C = 1,
  CTRL_STEP_LO = 2,
  CTRL_STEP_HI = 3,
  CTRL_ERR = 4,
  CTRL_TICKET = 5,
  CTRL_WORDS = 16
};
enum : int {
  HDR_NU = 0,
  HDR_NHIT = 1,
  HDR_NMISS = 2,
  HDR_LAYER = 3,
  HDR_T = 4,
  HDR_STEP_LO = 5,
  HDR_STEP_HI = 6,
  HDR_WORDS = 16
};
enum : int { ERR_CAPACITY = 1 };
constexpr int kMaxSlots = 4096;  // most cache slots a handle supports (LDS-resident LRU)

// Launch with optional timing events taken by the dispatch itself (start/end of the kernel,
// no extra packets in the queue); plain launch when both are null.
template <class K, class... Args>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                               hipEvent_t e0, hipEvent_t e1, Args... args) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}
enum : int {
  STAT_STEPS = 0,
  STAT_HITS = 1,
  STAT_MISSES = 2,
  STAT_BYTES = 3,
  STAT_FFN_BYTES = 4,
  STAT_TIMED_BLOB_BYTES = 5,  // blobs read by gate/up launches bracketed by timing events
  STAT_WORDS = 8
};

constexpr int FMT_BF16 = 0, FMT_FP8 = 1, FMT_MXFP4 = 2;
constexpr int kDecodeMaxTokens = 8;  // T handled by the GEMV decode path

struct Dims {
  int L, E, K, H, I, fmt, has_shared, max_tokens;
  int umax;          // min(max_tokens*K, E): distinct experts per step
  int amax;          // max_tokens*K: (token, choice) assignments per step
  int max_capacity;  // slots the arena holds
  int RS;            // row splits of the down projection (1 or 2)
  long long S;       // blob bytes
};

struct Dev {
  int* key_of;
  int* stamp;
  int* slot_of;
  int* ctrl;
  unsigned long long* stats;
  int* hdr;
  int* U;
  int* u_slot;
  int* u_hit;
  int* hit_list;
  int* miss_list;
  int* miss_key;
  int* miss_slot;
  int* miss_victim;
  int* count;
  int* offset;
  int* perm;
  int* inv_pos;
  int* tk_idx;
  float* tk_w;
  double* logits;
  float* act;          // [amax][I] silu(g)*u*w per (expert, token) row
  float* act_shared;   // [max_tokens][I] shared expert
  float* yexp;         // [amax][RS][H] per (expert, token) output
  float* yexp_shared;  // [max_tokens][RS][H] shared expert
  int4* ent;           // [umax] FFN entries in order hits, misses: {slot, ntok, row0, miss idx}
  int* row_tok;        // [amax] token of each expert-sorted assignment row
  float* row_w;        // [amax] routing weight of each row
  int* moves;          // [max_capacity * 2] resize moves (src, dst)
};

constexpr int kMaxFillGroups = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
