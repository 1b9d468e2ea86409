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

struct MergeArgs {
  int64_t N, L, V;
  int phases, adaptive;
  int kl, detach, norm;
  float beta, inv_tau;
  const int32_t* ntok;
  const int32_t* rank;
  const float* part;
  const int32_t* seq;   // [S] loss rows per sequence, then the count of non-empty sequences
  int64_t S;
  const int64_t* targets;
  const uint8_t* mask;
  const float* adv;
  float* saved;
  float* logp;
  float* ref_logp;
  float* kl_out;
  int32_t* status;
  double* lsum;
};

// Per row t (grid over all rows, masked rows included so their outputs are zeroed):
//   q = z_q[y] / tau - lse_q, ref = z_p[y] / tau - lse_p, d = ref - q,
//   KL and dKL/dq of the chosen estimator:
//     reverse    expm1(d) - d               -expm1(d)
//     forward    expm1(-d) + d              expm1(-d)
//     reverse_q  exp(q) (expm1(d) - d)      -d exp(q)
//   l = beta * KL - A_s                      (loss value; the ratio is 1 at q = sg(q))
//   g = w_t (-A_s [if detached] + beta dKL/dq)   (dloss/dq)
// with w_t = 1 / N_tok (token mean) or 1 / (n_s S') (sequence mean: n_s loss rows of the
// row's sequence, S' sequences with any) [Long-context GRPO, §4].  Each block reduces
// m_t * l_t (token mean) or m_t * l_t / n_s (sequence mean) in fp64 by a fixed tree into
// lsum[block]; the final kernel adds the block sums in index order.
__global__ void __launch_bounds__(kMergeBlock) merge_kernel(MergeArgs a) {
  __shared__ double red[kMergeBlock];
  const int64_t t = (int64_t)blockIdx.x * kMergeBlock + threadIdx.x;
  const int64_t N = a.N;
  const int32_t ntok = *a.ntok;
  const float denom = (float)(ntok > 1 ? ntok : 1);
  // partial slots written by the forward: all of them, or the adaptive phase count
  const int used = a.adaptive ? fwd_phases(2 * (((int64_t)ntok + 255) / 256), (a.V + 255) / 256)
                              : a.phases;
  double ell_d = 0.0;
  int flags = 0;
  if (t < N) {
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
    float q = 0.f, ref = 0.f, klv = 0.f;
    if (a.mask[t]) {
      const int64_t r = a.rank[t];
      const int64_t PN = (int64_t)a.phases * N;
      const float* pm = a.part;
      const float* ps = a.part + 2 * PN;
      const float* pz = a.part + 4 * PN;
      float lse_q, zq, lse_p, zp;
      merge_side(pm, ps, pz, used, N, r, &lse_q, &zq);
      merge_side(pm + PN, ps + PN, pz + PN, used, N, r, &lse_p, &zp);
      const int64_t y = a.targets[t];
      if (y < 0 || y >= a.V) flags |= GRPO_FLAG_BAD_TARGET;
      q = zq * a.inv_tau - lse_q;
      ref = zp * a.inv_tau - lse_p;
      const float d = ref - q;
      float dkl;
      if (a.kl == GRPO_KL_FORWARD) {
        const float em1 = expm1f(-d);
        klv = em1 + d;
        dkl = em1;
      } else {
        const float em1 = expm1f(d);
        klv = em1 - d;
        dkl = -em1;
        if (a.kl == GRPO_KL_REVERSE_Q) {
          const float eq = expf(q);
          klv = eq * klv;
          dkl = -d * eq;
        }
      }
      const float av = a.adv[t / a.L];
      const float num = (a.detach ? -av : 0.f) + a.beta * dkl;
      float g;
      ell_d = (double)a.beta * (double)klv - (double)av;
      if (a.norm == GRPO_NORM_SEQUENCES) {
        const int32_t ns = a.seq[t / a.L], nseq = a.seq[a.S];
        g = num / (float)((double)ns * (double)nseq);
        ell_d /= (double)ns;
      } else {
        g = num / denom;
      }
      sv = make_float4(lse_q, q, ref, g);
      if (!isfinite(lse_q) || !isfinite(q) || !isfinite(ref) || !isfinite(klv) ||
          !isfinite(g))
        flags |= GRPO_FLAG_NONFINITE;
    }
    reinterpret_cast<float4*>(a.saved)[t] = sv;
    if (a.logp) a.logp[t] = q;
    if (a.ref_logp) a.ref_logp[t] = ref;
    if (a.kl_out) a.kl_out[t] = klv;
  }
  if (flags) atomicOr(a.status, flags);
  red[threadIdx.x] = ell_d;
  __syncthreads();
  for (int off = kMergeBlock / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.lsum[blockIdx.x] = red[0];
}

// Loss rows of each sequence: one block per sequence.
__global__ void __launch_bounds__(256)
seq_count_kernel(const uint8_t* __restrict__ mask, int64_t L, int32_t* __restrict__ seq) {
  __shared__ int32_t red[256];
  const uint8_t* m = mask + (int64_t)blockIdx.x * L;
  int32_t c = 0;
  for (int64_t i = threadIdx.x; i < L; i += 256) c += m[i] ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq[blockIdx.x] = red[0];
}

// seq[S] = number of sequences with at least one loss row.
__global__ void __launch_bounds__(1024) seq_nonempty_kernel(int64_t S, int32_t* __restrict__ seq) {
  __shared__ int32_t red[1024];
  int32_t c = 0;
  for (int64_t s = threadIdx.x; s < S; s += 1024) c += seq[s] > 0 ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq[S] = red[0];
}

constexpr int kFinalThreads = 256;

__global__ void __launch_bounds__(kFinalThreads)
loss_final_kernel(const double* __restrict__ lsum, int64_t nblocks,
                  const int32_t* __restrict__ count_p, float* __restrict__ loss,
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
    const int32_t n = *count_p;  // N_tok, or S' for the sequence mean
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
  MergeArgs a;
  a.N = p.N;
  a.L = p.L;
  a.V = p.V;
  a.phases = p.phases;
  a.adaptive = p.mfma;
  a.kl = p.kl;
  a.detach = p.detach;
  a.norm = p.norm;
  a.beta = beta;
  a.inv_tau = p.inv_tau;
  a.ntok = ws_ptr<int32_t>(w, p.off_ntok);
  a.rank = ws_ptr<int32_t>(w, p.off_rank);
  a.part = ws_ptr<float>(w, p.off_part);
  a.seq = ws_ptr<int32_t>(w, p.off_seq);
  a.S = p.N / p.L;
  a.targets = targets;
  a.mask = mask;
  a.adv = adv;
  a.saved = saved;
  a.logp = logp;
  a.ref_logp = ref_logp;
  a.kl_out = kl;
  a.status = status;
  a.lsum = ws_ptr<double>(w, p.off_lsum);
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nblocks), dim3(kMergeBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t* count = p.norm == GRPO_NORM_SEQUENCES ? a.seq + a.S : a.ntok;
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, a.lsum, nblocks,
                     count, loss, status);
  return hipGetLastError();
}

hipError_t launch_seq_counts(const Plan& p, const uint8_t* mask, void* ws, hipStream_t st) {
  const int64_t S = p.N / p.L;
  int32_t* seq = ws_ptr<int32_t>(ws, p.off_seq);
  hipLaunchKernelGGL(seq_count_kernel, dim3((unsigned)S), dim3(256), 0, st, mask, p.L, seq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_nonempty_kernel, dim3(1), dim3(1024), 0, st, S, seq);
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
