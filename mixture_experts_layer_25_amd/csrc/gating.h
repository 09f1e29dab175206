// Combine weight of one selected expert, shared by the exact router and the
// screened many-expert router so that both write the same bits.
//
// "FFN, SwiGLU and MoE" sec. 3: p = softmax(r) over all experts, then the
// k largest, optionally divided by their sum (the module's top-k
// renormalisation). With renormalisation the softmax denominator cancels,
// so the weight of slot s is exp(key_s - m) / sum_j exp(key_j - m) over the
// selected j only (m = the largest key): no sum over all experts is needed.
// "MoE routing: Top-K, Expert-Choice and Sigmoid Gating": w = sigmoid(s).
// "DeepSeek-V4.1-Flash fine-grained MoE (5A)" sec. 1, 3 and 4: w =
// sqrt(softplus(s)) of the raw score, softplus in the form that cannot
// overflow.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/moe.h"

namespace moe {

// Weight of a selected expert before renormalisation: `key` = logit + bias
// (softmax), `logit` = the raw score (sigmoid, sqrt-softplus); m = the
// largest key of the token, Z = sum over all experts of exp(key - m) (read
// only by softmax without renormalisation).
__device__ __forceinline__ float gate_weight(int gating, int renorm, float key, float logit,
                                             float m, float Z) {
  if (gating == MOE_GATE_SOFTMAX) return renorm ? expf(key - m) : expf(key - m) / Z;
  if (gating == MOE_GATE_SIGMOID) return 1.0f / (1.0f + expf(-logit));
  const float sp = fmaxf(logit, 0.0f) + log1pf(expf(-fabsf(logit)));
  return sqrtf(sp);
}

}  // namespace moe
