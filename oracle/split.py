"""Split of a decode step's cache misses between PCIe fills and in-place CPU compute, and the
per-dtype mode choice (test oracle only).

Pages:
* FreeToken paper summary (agihunt.info, arXiv 2608.16157), problem paragraph: at decode a
  missed expert is either moved over PCIe or computed by the CPU, and no principled rule for
  the division existed; execution-layer paragraph: the number q is derived inside the fused
  routing kernel; last paragraph: q is a closed-form split by measured bandwidth.  No formula
  is printed.
* "FreeToken: az VRAM ile büyük MoE modelleri" (kptndocs), section "Tuzaklar": a start-up
  probe prints per-dtype CPU and offload rates against a 2.0x threshold (bf16 52.4 vs
  51.5 GB/s -> 1.02x -> offload; fp8 has no CPU path -> offload).

Reading (the plainest the pages support):
* Both ways of serving a missed expert stream its whole blob of S bytes: a fill over PCIe
  at b_pcie, an in-place CPU FFN at b_cpu (its expert-weight rate).  Serving q misses on the
  CPU and m - q by fills finishes at max((m - q) S / b_pcie, q S / b_cpu).  q is the integer
  that minimises this makespan, the smaller q on a tie.  Rates are integers (MB/s), so the
  comparison is exact: scaled by b_cpu * b_pcie / S it is max((m - q) b_cpu, q b_pcie).
* Hybrid execution (q > 0 possible) is chosen for a dtype iff its CPU expert rate is at least
  `threshold` times the offload rate; otherwise q = 0.
"""
from __future__ import annotations


def makespan(m: int, q: int, b_cpu: int, b_pcie: int) -> int:
    """max((m - q) / b_pcie, q / b_cpu), scaled by b_cpu * b_pcie (integers)."""
    return max((m - q) * b_cpu, q * b_pcie)


def miss_split(m: int, b_cpu: int, b_pcie: int) -> int:
    """Misses (of m) computed on the CPU: the makespan minimiser, the smallest on a tie."""
    if m <= 0 or b_cpu <= 0:
        return 0
    best_q, best = 0, makespan(m, 0, b_cpu, b_pcie)
    for q in range(1, m + 1):
        t = makespan(m, q, b_cpu, b_pcie)
        if t < best:
            best_q, best = q, t
    return best_q


def hybrid_mode(cpu_rate: float, offload_rate: float, threshold: float = 2.0) -> bool:
    """True: split misses between the CPU and PCIe; False: fill every miss ("offload").
    A dtype without a CPU expert path has cpu_rate 0."""
    return cpu_rate > 0 and offload_rate > 0 and cpu_rate >= threshold * offload_rate
