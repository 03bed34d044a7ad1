// Device-side definitions shared by the expert-offload kernels and their host driver.
//
// Workspace state (persistent across steps, device memory owned by the caller):
//   key_of[max_capacity]  key held by each slot (key = layer*E + expert), -1 empty
//   stamp[max_capacity]   global step of the slot's last use (64-bit), -1 empty
//   slot_of[L*E]          slot of each key, -1 when not cached
//   ctrl[16]              occupancy n, capacity C, step counter, error bits, tickets
//   stats[8]              steps, hits, misses, bytes filled, FFN bytes, CPU misses, ...
// Per-step plan (rewritten by every route launch):
//   hdr[16], U/u_slot/u_hit/hit_list/miss_list/miss_key/miss_slot/miss_victim[umax],
//   count[umax], offset[umax+1], perm/inv_pos/tk_idx/tk_w[amax], logits[tdec*E],
//   FFN intermediates (act) and per-expert outputs (yexp), the hybrid decode's CPU rows and
//   keys; for steps of more than eight tokens the block counts and offsets of the router,
//   bf16 / fp32 row buffers and the prefetch plan.
// Host memory of a hybrid handle: the mailbox (HybMail, below) the route kernel posts to.
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
  HDR_NCPU = 7,  // misses computed in place by the CPU (hybrid decode)
  HDR_WORDS = 16
};
enum : int { ERR_CAPACITY = 1, ERR_HYBRID = 2 };
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
  STAT_CPU = 6,               // misses computed in place by the CPU
  STAT_TIMED_FUSED_BYTES = 7, // blobs read by fused one-token FFN launches bracketed by events
  STAT_WORDS = 8
};

constexpr int FMT_BF16 = 0, FMT_FP8 = 1, FMT_MXFP4 = 2;
constexpr int kDecodeMaxTokens = 8;  // T handled by the GEMV decode path
constexpr int kMaxTokens = 65536;    // most tokens of one layer step

struct Dims {
  int L, E, K, H, I, fmt, has_shared, max_tokens;
  int umax;          // min(max_tokens*K, E): distinct experts per step
  int pw;            // entries of the plan's per-expert LDS arrays: umax, or E when the
                     // handle has the many-token path (a prefetch plans all E experts)
  int amax;          // max_tokens*K: (token, choice) assignments per step
  int tdec;          // min(max_tokens, kDecodeMaxTokens): tokens of the decode path
  int adec;          // tdec*K
  int nblk;          // 64-token blocks of the many-token path (0 when max_tokens <= 8)
  int max_capacity;  // slots the arena holds
  int RS;            // row splits of the decode down projection
  int RSF;           // row blocks of the fused one-token FFN (0: the shape takes two kernels)
  long long S;       // blob bytes
};

// Hybrid decode mailbox in pinned, coherent host memory (one request in flight at a time).
// The route kernel posts a request when it sends q > 0 misses of a step to the CPU: the CPU
// experts, their rows (token, routing weight) and the step's activations, then `req` = the
// step counter value.  The host server computes y_cpu[t] = sum over the CPU experts of
// w * FFN_e(x_t), then sets `done` = req; the combine kernel waits for it.
constexpr int kMailRows = 128;  // kDecodeMaxTokens * the largest top_k (16)
struct HybMail {
  long long req;
  int layer, T, q, K;
  int pad0[26];
  int exp[kMailRows];    // CPU experts, ascending
  int ntok[kMailRows];   // rows of each
  int row0[kMailRows];   // first expert-sorted row of each
  int row_tok[kMailRows];
  float row_w[kMailRows];
  long long done;        // own 128-byte line
  int pad1[30];
};
static_assert(sizeof(HybMail) % 128 == 0, "mailbox lines");
static_assert(__builtin_offsetof(HybMail, done) % 128 == 0, "done on its own line");
__host__ __device__ inline size_t mail_x_offset() { return (sizeof(HybMail) + 127) & ~(size_t)127; }
__host__ __device__ inline size_t mail_y_offset(int H) {
  return mail_x_offset() + (((size_t)kDecodeMaxTokens * H * 2 + 127) & ~(size_t)127);
}
__host__ __device__ inline size_t mail_bytes(int H) {
  return mail_y_offset(H) + (size_t)kDecodeMaxTokens * H * 4;
}

struct Dev {
  int* key_of;
  long long* stamp;
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
  float* act;          // [adec][I] silu(g)*u*w per (expert, token) row (decode)
  float* act_shared;   // [tdec][I] shared expert (decode)
  float* yexp;         // [adec][RS][H] per (expert, token) output (decode)
  float* yexp_shared;  // [tdec][RS][H] shared expert (decode)
  float* yfus;         // [K][RSF][H] fused one-token FFN partials per (expert row, row block)
  int* blk_cnt;        // [nblk][E] assignments per (64-token block, expert)
  int* blk_off;        // [nblk][E] first expert-sorted row of each (block, expert)
  int* brank;          // [amax] rank of a (token, choice) among its block's rows
  uint16_t* pact;      // [amax][I] bf16 silu(g)*u*w per expert-sorted row (many tokens)
  uint16_t* pact_shared;  // [max_tokens][I] shared expert
  float* pyexp;        // [amax][H] fp32 expert output per row
  float* pyexp_shared; // [max_tokens][H] shared expert output
  int4* ent;           // [umax] FFN entries in order hits, misses: {slot, ntok, row0, miss idx}
  int* row_tok;        // [amax] token of each expert-sorted assignment row
  float* row_w;        // [amax] routing weight of each row
  int* moves;          // [max_capacity * 2] resize moves (src, dst)
  // plan of a prefetch step (every expert of the next layer; steps of many tokens only),
  // kept apart from the step plan that the FFN may still be reading
  int* pf_hdr;         // [HDR_WORDS]
  int* pf_list;        // [11 * E + 1]: U, u_slot, u_hit, hit_list, miss_list, miss_key,
                       //   miss_slot, miss_victim, count, offset[E + 1]
  int4* pf_ent;        // [E]
  int* row_cpu;        // [adec] 1: the row's expert is computed by the CPU (hybrid decode)
  int* cpu_key;        // [umax] keys of the step's CPU misses, ascending expert
  HybMail* mail;       // device view of the hybrid mailbox, or null
  long long hyb_timeout_ticks;  // longest wait for the host's answer, 100 MHz clock ticks
};

// Where a plan writes its outputs: the step plan or a prefetch plan.
struct PlanOut {
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
  int4* ent;
  int* hdr;
  int* cpu_key;  // keys of CPU misses (null: the plan never splits)
};

__host__ __device__ inline PlanOut step_plan_out(const Dev& v) {
  return PlanOut{v.U,         v.u_slot,      v.u_hit, v.hit_list, v.miss_list, v.miss_key,
                 v.miss_slot, v.miss_victim, v.count, v.offset,   v.ent,       v.hdr,
                 v.cpu_key};
}

__host__ __device__ inline PlanOut prefetch_plan_out(const Dev& v, int E) {
  int* b = v.pf_list;
  return PlanOut{b,         b + E,     b + 2 * E, b + 3 * E, b + 4 * E, b + 5 * E,
                 b + 6 * E, b + 7 * E, b + 8 * E, b + 9 * E, v.pf_ent,  v.pf_hdr, nullptr};
}

constexpr int kMaxFillGroups = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16, round to nearest even.  A NaN stays a NaN of the same sign (quieted): the
// rounding bias must not carry its payload into the exponent or the sign.
__host__ __device__ __forceinline__ uint16_t bf16_bits_rne(uint32_t u) {
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return bf16_bits_rne(__float_as_uint(f));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
