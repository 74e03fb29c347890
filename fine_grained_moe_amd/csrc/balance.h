// The aux-loss-free balancing step of one wave and the batch's balance
// figures, shared by the kernels that take the step (route.hip, decode.hip).
#pragma once

#include "common.h"

namespace fgmoe {

// The bias step of one wave, lane e holding expert e's load c (0 for e >= E):
// bias[e] <- fl32(bias[e] + gamma * sign(total - E * c)), and with stats the
// batch's balance figures, stats = [experts with zero load / E, max load * E /
// total, load entropy -sum p ln p (p = load / total, 0 ln 0 = 0), entropy /
// ln E (1 for E = 1)]; an empty batch reads (1, 0, 0, 0).  ("Relay training"
// section: a low dead-expert fraction under aux-loss-free balancing, expert
// balance on the dashboard.)  The sums and the maximum are butterfly
// reductions in a fixed order.  Used by the bias kernel and by the dispatch
// kernel's fused step, so both give the same bits.
__device__ __forceinline__ void bias_step_wave(int e, int E, long long total, int c, float gamma,
                                               float* __restrict__ bias, float* __restrict__ stats) {
  if (e < E) {
    const long long diff = total - (long long)E * (long long)c;
    const float sg = (float)((diff > 0) - (diff < 0));
    bias[e] = __fadd_rn(bias[e], gamma * sg);
  }
  if (!stats) return;
  int dead = (e < E && c == 0) ? 1 : 0;
  int mx = c;
  float h = 0.f;
  if (c > 0 && total > 0) {
    const float pr = (float)c / (float)total;
    h = -pr * logf(pr);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    dead += __shfl_xor(dead, off);
    mx = max(mx, __shfl_xor(mx, off));
    h += __shfl_xor(h, off);
  }
  if (e == 0) {
    if (total <= 0) {
      stats[0] = 1.f;
      stats[1] = stats[2] = stats[3] = 0.f;
    } else {
      stats[0] = (float)dead / (float)E;
      stats[1] = (float)((double)mx * E / (double)total);
      stats[2] = h;
      stats[3] = E > 1 ? h / logf((float)E) : 1.f;
    }
  }
}

}  // namespace fgmoe
