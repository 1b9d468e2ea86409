// Row compaction, the KL / advantage epilogue with the loss reduction, and the zero fill
// of masked gradient rows.  These kernels move tens of bytes per row and are bound by
// latency and HBM bandwidth, not arithmetic.
#include "common.h"

namespace grpo {
namespace {

constexpr int kCompactThreads = 1024;

// Loss rows in ascending order: idx[r] = row of the r-th loss token, rank[t] = r or -1.
// One workgroup; each thread owns a contiguous segment of the mask, counts its ones, the
// block scans the counts, then each thread writes its segment's indices in order.  The
// result does not depend on scheduling.  Also clears the forward's status word.
__global__ void __launch_bounds__(kCompactThreads)
compact_kernel(const uint8_t* __restrict__ mask, int64_t N, int32_t* __restrict__ ntok,
               int32_t* __restrict__ idx, int32_t* __restrict__ rank,
               int32_t* __restrict__ status) {
  __shared__ int32_t scan[kCompactThreads];
  const int64_t seg = (N + kCompactThreads - 1) / kCompactThreads;
  const int64_t lo = (int64_t)threadIdx.x * seg;
  const int64_t hi = lo + seg < N ? lo + seg : N;
  int32_t c = 0;
  for (int64_t t = lo; t < hi; ++t) c += mask[t] ? 1 : 0;
  scan[threadIdx.x] = c;
  __syncthreads();
  // Hillis-Steele inclusive scan over the block
  for (int off = 1; off < kCompactThreads; off <<= 1) {
    int32_t v = threadIdx.x >= (unsigned)off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t pos = scan[threadIdx.x] - c;
  for (int64_t t = lo; t < hi; ++t) {
    if (mask[t]) {
      idx[pos] = (int32_t)t;
      rank[t] = pos;
      ++pos;
    } else {
      rank[t] = -1;
    }
  }
  if (threadIdx.x == kCompactThreads - 1) {
    *ntok = scan[kCompactThreads - 1];
    if (status) *status = 0;
  }
}

// Merge of the per-phase partials of one side (policy or reference) for compact row r:
// log-sum-exp in natural units and the target logit.  Partial maxima are kept in log2
// units (logit * log2 e); sums are of exp2(logit*log2e - max).
__device__ inline void merge_side(const float* __restrict__ pm, const float* __restrict__ ps,
                                  const float* __restrict__ pz, int used, int64_t N,
                                  int64_t r, float* lse, float* zt) {
  float M = -INFINITY;
  for (int p = 0; p < used; ++p) M = fmaxf(M, pm[p * N + r]);
  float s = 0.0f, z = 0.0f;
  for (int p = 0; p < used; ++p) {
    const float sp = ps[p * N + r];
    if (sp != 0.0f) s += sp * exp2f(pm[p * N + r] - M);
    z += pz[p * N + r];
  }
  *lse = (M + log2f(s)) * kLn2;
  *zt = z;
}

// Per row t (grid over all rows, masked rows included so their outputs are zeroed):
//   q = z_q[y] - lse_q, ref = z_p[y] - lse_p, d = ref - q,
//   KL = expm1(d) - d                                  (reverse-KL estimator)
//   l  = beta * KL - A_s                               (loss value; ratio = 1)
//   g  = (-A_s - beta * expm1(d)) / N_tok             (dloss/dq; ratio gradient is A*dq)
// [Long-context GRPO, §4].  Each block reduces m_t * l_t in fp64 by a fixed tree into
// lsum[block]; the final kernel adds the block sums in index order.
__global__ void __launch_bounds__(kMergeBlock)
merge_kernel(int64_t N, int64_t L, int64_t V, int phases, int adaptive,
             const int32_t* __restrict__ ntok_p,
             const int32_t* __restrict__ rank, const float* __restrict__ part,
             const int64_t* __restrict__ targets, const uint8_t* __restrict__ mask,
             const float* __restrict__ adv, float beta, float* __restrict__ saved,
             float* __restrict__ logp, float* __restrict__ ref_logp, float* __restrict__ kl_out,
             int32_t* __restrict__ status, double* __restrict__ lsum) {
  __shared__ double red[kMergeBlock];
  const int64_t t = (int64_t)blockIdx.x * kMergeBlock + threadIdx.x;
  const int32_t ntok = *ntok_p;
  const float denom = (float)(ntok > 1 ? ntok : 1);
  // partial slots written by the forward: all of them, or the adaptive phase count
  const int used = adaptive ? fwd_phases(2 * (((int64_t)ntok + 255) / 256), (V + 255) / 256)
                            : phases;
  double ell_d = 0.0;
  int flags = 0;
  if (t < N) {
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
    float q = 0.f, ref = 0.f, klv = 0.f;
    if (mask[t]) {
      const int64_t r = rank[t];
      const int64_t PN = (int64_t)phases * N;
      const float* pm = part;
      const float* ps = part + 2 * PN;
      const float* pz = part + 4 * PN;
      float lse_q, zq, lse_p, zp;
      merge_side(pm, ps, pz, used, N, r, &lse_q, &zq);
      merge_side(pm + PN, ps + PN, pz + PN, used, N, r, &lse_p, &zp);
      const int64_t y = targets[t];
      if (y < 0 || y >= V) flags |= GRPO_FLAG_BAD_TARGET;
      q = zq - lse_q;
      ref = zp - lse_p;
      const float d = ref - q;
      const float em1 = expm1f(d);
      klv = em1 - d;
      const float a = adv[t / L];
      const float g = (-a - beta * em1) / denom;
      ell_d = (double)beta * (double)klv - (double)a;
      sv = make_float4(lse_q, q, ref, g);
      if (!isfinite(lse_q) || !isfinite(q) || !isfinite(ref) || !isfinite(klv) ||
          !isfinite(g))
        flags |= GRPO_FLAG_NONFINITE;
    }
    reinterpret_cast<float4*>(saved)[t] = sv;
    if (logp) logp[t] = q;
    if (ref_logp) ref_logp[t] = ref;
    if (kl_out) kl_out[t] = klv;
  }
  if (flags) atomicOr(status, flags);
  red[threadIdx.x] = ell_d;
  __syncthreads();
  for (int off = kMergeBlock / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) lsum[blockIdx.x] = red[0];
}

constexpr int kFinalThreads = 256;

__global__ void __launch_bounds__(kFinalThreads)
loss_final_kernel(const double* __restrict__ lsum, int64_t nblocks,
                  const int32_t* __restrict__ ntok_p, float* __restrict__ loss,
                  int32_t* __restrict__ status) {
  __shared__ double red[kFinalThreads];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < nblocks; i += kFinalThreads) s += lsum[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = kFinalThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t n = *ntok_p;
    const float l = (float)(red[0] / (double)(n > 1 ? n : 1));
    *loss = l;
    if (!isfinite(l)) atomicOr(status, GRPO_FLAG_NONFINITE);
  }
}

// dX rows of masked positions are zero.  One block per 4 rows, 16-byte stores.
__global__ void __launch_bounds__(256)
zero_rows_kernel(const uint8_t* __restrict__ mask, int64_t N, int64_t row_bytes,
                 char* __restrict__ dX) {
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= N || mask[t]) return;
  uint4* row = reinterpret_cast<uint4*>(dX + t * row_bytes);
  const int64_t n16 = row_bytes / 16;
  for (int64_t i = threadIdx.x % 64; i < n16; i += 64) row[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_compact(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                          int32_t* rank, hipStream_t st) {
  return launch_compact_status(mask, N, ntok, idx, rank, nullptr, st);
}

hipError_t launch_compact_status(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                                 int32_t* rank, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kCompactThreads), 0, st, mask, N, ntok, idx,
                     rank, status);
  return hipGetLastError();
}

hipError_t launch_merge(const Plan& p, const void* ws, const int64_t* targets,
                        const uint8_t* mask, const float* adv, float beta, float* saved,
                        float* logp, float* ref_logp, float* kl, int32_t* status, float* loss,
                        hipStream_t st) {
  void* w = const_cast<void*>(ws);
  const int64_t nblocks = (p.N + kMergeBlock - 1) / kMergeBlock;
  double* lsum = ws_ptr<double>(w, p.off_lsum);
  const int32_t* ntok = ws_ptr<int32_t>(w, p.off_ntok);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nblocks), dim3(kMergeBlock), 0, st, p.N, p.L,
                     p.V, p.phases, p.mfma, ntok, ws_ptr<int32_t>(w, p.off_rank),
                     ws_ptr<float>(w, p.off_part), targets, mask, adv, beta, saved, logp,
                     ref_logp, kl, status, lsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, lsum, nblocks, ntok,
                     loss, status);
  return hipGetLastError();
}

hipError_t launch_zero_masked_rows(const Plan& p, const uint8_t* mask, void* dX,
                                   hipStream_t st) {
  const int64_t blocks = (p.N + 3) / 4;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, mask, p.N,
                     p.H * p.esize, reinterpret_cast<char*>(dX));
  return hipGetLastError();
}

}  // namespace grpo
