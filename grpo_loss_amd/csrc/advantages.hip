// Group-relative advantages [Train your own R1 reasoning model with Unsloth, §3;
// Long-context GRPO, §4].  Compiled with -ffp-contract=off; every operation below is an
// explicitly rounded fp32 intrinsic as well, so no step can be fused or reordered and the
// result is reproducible bit for bit.  The square root is sqrtf, which this unit's
// -fhip-fp32-correctly-rounded-divide-sqrt lowers to the correctly rounded sequence
// (__fsqrt_rn would be the approximate native instruction here).
#include "common.h"

namespace grpo {
namespace {

constexpr int kAdvThreads = 256;
constexpr int kAdvLds = 8192;  // floats of rewards staged per block

// One thread per prompt group.  The block first copies its groups' contiguous span of
// rewards [b0*G*K, (b0+nb)*G*K) into LDS with coalesced loads, then each thread walks
// its own group in the fixed order: scores summed over k ascending, the group sum over g
// ascending, mean = sum / G, squared deviations summed over g ascending (product rounded
// before the add), var = ss / (G - 1) (or / G), std = sqrt(var) correctly rounded,
// A = (r - mean) / (std + eps).
__global__ void __launch_bounds__(kAdvThreads)
advantage_kernel(const float* __restrict__ rewards, int64_t B, int G, int K, float eps,
                 int unbiased, int groups_per_block, float* __restrict__ adv) {
  __shared__ float stage[kAdvLds];
  const int64_t b0 = (int64_t)blockIdx.x * groups_per_block;
  const int64_t nb = (B - b0) < groups_per_block ? (B - b0) : groups_per_block;
  const int64_t per = (int64_t)G * K;
  const bool staged = nb * per <= kAdvLds;
  if (staged) {
    const float* src = rewards + b0 * per;
    for (int64_t i = threadIdx.x; i < nb * per; i += blockDim.x) stage[i] = src[i];
    __syncthreads();
  }
  const int64_t local = threadIdx.x;
  if (local >= nb) return;
  const float* r = staged ? stage + local * per : rewards + (b0 + local) * per;
  float total = 0.0f;
  for (int g = 0; g < G; ++g) {
    float s = r[(int64_t)g * K];
    for (int k = 1; k < K; ++k) s = __fadd_rn(s, r[(int64_t)g * K + k]);
    total = __fadd_rn(total, s);
  }
  const float mean = __fdiv_rn(total, (float)G);
  float ss = 0.0f;
  for (int g = 0; g < G; ++g) {
    float s = r[(int64_t)g * K];
    for (int k = 1; k < K; ++k) s = __fadd_rn(s, r[(int64_t)g * K + k]);
    const float d = __fsub_rn(s, mean);
    ss = __fadd_rn(ss, __fmul_rn(d, d));
  }
  const float var = __fdiv_rn(ss, (float)(unbiased ? G - 1 : G));
  const float den = __fadd_rn(sqrtf(var), eps);
  float* out = adv + (b0 + local) * G;
  for (int g = 0; g < G; ++g) {
    float s = r[(int64_t)g * K];
    for (int k = 1; k < K; ++k) s = __fadd_rn(s, r[(int64_t)g * K + k]);
    out[g] = __fdiv_rn(__fsub_rn(s, mean), den);
  }
}

}  // namespace

hipError_t launch_advantages(const float* rewards, int64_t B, int64_t G, int64_t K, float eps,
                             int unbiased, float* adv, hipStream_t st) {
  const int64_t per = G * K;
  int64_t gpb = per > 0 ? kAdvLds / per : 1;
  if (gpb < 1) gpb = 1;
  if (gpb > kAdvThreads) gpb = kAdvThreads;
  const int64_t blocks = (B + gpb - 1) / gpb;
  hipLaunchKernelGGL(advantage_kernel, dim3((unsigned)blocks), dim3(kAdvThreads), 0, st,
                     rewards, B, (int)G, (int)K, eps, unbiased, (int)gpb, adv);
  return hipGetLastError();
}

}  // namespace grpo
