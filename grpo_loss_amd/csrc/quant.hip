// Per-row fp8 (e4m3, "fn": no infinities, maximum 448) quantisation of X and W rows for
// the fp8-logits option.  Built with correctly rounded fp32 division and no contraction,
// so every code and scale is a fixed function of the row.
#include "common.h"

namespace grpo {
namespace {

constexpr int kQThreads = 256;

// e4m3 byte of |a| <= 448 (a >= 0, an fp32 value), round to nearest even: 3 fraction
// bits from 2^-6 up, steps of 2^-9 below (codes 0..8, 8 being 2^-6 itself).
__device__ inline uint32_t e4m3_code(float a) {
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t u = __float_as_uint(a);
  int e = (int)(u >> 23) - 127;                 // -6 .. 8
  const uint32_t m = u & 0x7FFFFFu;
  uint32_t f = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;   // 3 bits, ties to even
  if (f == 8u) {
    f = 0u;
    ++e;
  }
  return (uint32_t)((e + 7) << 3) | f;
}

template <class E>
__global__ void __launch_bounds__(kQThreads)
quant_rows_kernel(const typename E::T* __restrict__ src, int64_t H,
                  const int32_t* __restrict__ idx, const int32_t* __restrict__ ntok,
                  uint8_t* __restrict__ dst, float* __restrict__ scale) {
  __shared__ float red[kQThreads];
  const int64_t r = blockIdx.x;
  if (ntok && r >= *ntok) return;
  const typename E::T* x = src + (idx ? (int64_t)idx[r] : r) * H;
  // a non-finite element makes the row's scale NaN, so its logits (and the status word)
  // show it instead of the element being clamped away
  float amax = 0.f;
  for (int64_t h = threadIdx.x; h < H; h += kQThreads) {
    const float v = fabsf(E::to_f32(x[h]));
    amax = (v <= 3.402823466e38f) ? fmaxf(amax, v) : __builtin_inff();
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int off = kQThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  amax = red[0];
  const bool finite = amax <= 3.402823466e38f;
  const float inv = (amax > 0.f && finite) ? 448.0f / amax : 1.0f;
  if (threadIdx.x == 0) scale[r] = !finite ? __builtin_nanf("") : (amax > 0.f ? amax / 448.0f : 1.0f);
  uint8_t* d = dst + r * H;
  for (int64_t h = threadIdx.x * 4; h < H; h += kQThreads * 4) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = E::to_f32(x[h + j]) * inv;
      const float a = fminf(fabsf(y), 448.0f);
      const uint32_t code = e4m3_code(a) | ((__float_as_uint(y) >> 24) & 0x80u);
      word |= code << (8 * j);
    }
    *reinterpret_cast<uint32_t*>(d + h) = word;
  }
}

}  // namespace

hipError_t launch_quant_rows(int dtype, const void* src, int64_t H, const int32_t* idx,
                             const int32_t* ntok, int64_t nmax, uint8_t* dst, float* scale,
                             hipStream_t st) {
  if (nmax <= 0) return hipSuccess;
  if (dtype == GRPO_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<BF16T>, dim3((unsigned)nmax), dim3(kQThreads), 0, st,
                       reinterpret_cast<const u16*>(src), H, idx, ntok, dst, scale);
  else if (dtype == GRPO_F16)
    hipLaunchKernelGGL(quant_rows_kernel<F16T>, dim3((unsigned)nmax), dim3(kQThreads), 0, st,
                       reinterpret_cast<const u16*>(src), H, idx, ntok, dst, scale);
  else
    hipLaunchKernelGGL(quant_rows_kernel<F32T>, dim3((unsigned)nmax), dim3(kQThreads), 0, st,
                       reinterpret_cast<const float*>(src), H, idx, ntok, dst, scale);
  return hipGetLastError();
}

}  // namespace grpo
