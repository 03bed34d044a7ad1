// In-place CPU expert FFN of the hybrid decode path (host code).
//
// FreeToken paper summary (agihunt.info, arXiv 2608.16157): a decode miss may be computed by
// the CPU straight from the host expert pool instead of being moved over PCIe; the CPU path
// exists for bf16 weights only ("FreeToken: az VRAM ile büyük MoE modelleri", "Tuzaklar").
// The expert is the same SwiGLU FFN as on the GPU, over the same blob layout:
// Wgu [I][2][H] (gate row i then up row i) followed by WdT [I][H], bf16.
#pragma once
#include <atomic>
#include <cstdint>
#include <functional>
#include <thread>
#include <vector>

namespace moe {

// A team of n threads (the caller is member 0) that runs one job at a time; members spin
// between jobs, so a job starts within microseconds.  run() returns when every member is done.
class CpuTeam {
 public:
  explicit CpuTeam(int n);
  ~CpuTeam();
  int size() const { return n_; }
  void run(const std::function<void(int)>& job);

 private:
  void member(int k);
  int n_;
  std::vector<std::thread> th_;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> left_{0};
  std::atomic<bool> stop_{false};
  const std::function<void(int)>* job_ = nullptr;
};

// y[t][:] += sum over the experts e < nexp and their rows r in [row0[e], row0[e] + ntok[e])
// with row_tok[r] = t, row_w[r] = w:  w * WdT_e^T (silu(Wg_e x_t) * (Wu_e x_t)).
// x: [T][H] bf16; y: [T][H] fp32; partial: team.size() * T * H floats of scratch.  Rows of I
// are split across the team; each member accumulates its rows of every expert into its own
// partial (experts in order), and the partials are added in member order: deterministic.
void cpu_experts_ffn(CpuTeam& team, const uint16_t* const* blobs, int nexp, const int* row0,
                     const int* ntok, const int* row_tok, const float* row_w, int H, int I,
                     const uint16_t* x, int T, float* y, float* partial);

}  // namespace moe
