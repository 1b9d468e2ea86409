// Row compaction, the KL / advantage epilogue with the loss reduction, and the zero fill
// of masked gradient rows.  These kernels move tens of bytes per row and are bound by
// latency and HBM bandwidth, not arithmetic.
#include "common.h"

namespace grpo {
namespace {

constexpr int kScanThreads = 1024;

// Loss rows in ascending order, idx[r] = row of the r-th loss token and rank[t] = r or -1,
// in three launches whose results do not depend on scheduling (no atomics, no waits
// between workgroups).  Blocks of kCompactRows rows, read as 16 rounds of 256 consecutive
// mask bytes (one byte per thread and round):
//   1. compact_count_kernel: loss rows per block -> bsum[b];
//   2. compact_scan_kernel (one workgroup): bsum[b] <- rows before block b, in block order;
//      *ntok = the total; the forward's status word cleared;
//   3. compact_scatter_kernel: each block numbers its loss rows from bsum[b] in row order
//      (per round: a ballot within each wave, the waves' counts through LDS).
__global__ void __launch_bounds__(256)
compact_count_kernel(const uint8_t* __restrict__ mask, int64_t N, int32_t* __restrict__ bsum) {
  __shared__ int32_t red[4];
  const int64_t base = (int64_t)blockIdx.x * kCompactRows;
  int32_t c = 0;
  for (int j = 0; j < kCompactRows / 256; ++j) {
    const int64_t t = base + j * 256 + threadIdx.x;
    c += (t < N && mask[t]) ? 1 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ void __launch_bounds__(kScanThreads)
compact_scan_kernel(int64_t nblocks, int32_t* __restrict__ bsum, int32_t* __restrict__ ntok,
                    int32_t* __restrict__ status) {
  __shared__ int32_t s[kScanThreads];
  int32_t carry = 0;
  for (int64_t b0 = 0; b0 < nblocks; b0 += kScanThreads) {
    const int64_t b = b0 + threadIdx.x;
    const int32_t v = b < nblocks ? bsum[b] : 0;
    s[threadIdx.x] = v;
    __syncthreads();
    // Hillis-Steele inclusive scan over the workgroup
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int32_t u = threadIdx.x >= (unsigned)off ? s[threadIdx.x - off] : 0;
      __syncthreads();
      s[threadIdx.x] += u;
      __syncthreads();
    }
    if (b < nblocks) bsum[b] = carry + s[threadIdx.x] - v;
    carry += s[kScanThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *ntok = carry;
    if (status) *status = 0;
  }
}

__global__ void __launch_bounds__(256)
compact_scatter_kernel(const uint8_t* __restrict__ mask, int64_t N,
                       const int32_t* __restrict__ bsum, int32_t* __restrict__ idx,
                       int32_t* __restrict__ rank) {
  __shared__ int32_t wsum[4];
  const int64_t base = (int64_t)blockIdx.x * kCompactRows;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t pos = bsum[blockIdx.x];
  for (int j = 0; j < kCompactRows / 256; ++j) {
    const int64_t t = base + j * 256 + threadIdx.x;
    const bool f = t < N && mask[t];
    const uint64_t bal = __ballot(f);
    const int32_t below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int32_t woff = 0;
    for (int k = 0; k < w; ++k) woff += wsum[k];
    const int32_t round = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (t < N) {
      if (f) {
        idx[pos + woff + below] = (int32_t)t;
        rank[t] = pos + woff + below;
      } else {
        rank[t] = -1;
      }
    }
    pos += round;
    __syncthreads();  // wsum is rewritten by the next round
  }
}

// Merge of the per-phase partials of one side (policy or reference) of one row, held at
// l.at(., sd, ., r) of `part`: log-sum-exp in natural units and the target logit.
// Partial maxima are kept in log2 units (logit * log2 e); sums are of
// exp2(logit*log2e - max).
__device__ inline void merge_side(const float* __restrict__ part, const PartLayout& l, int sd,
                                  int64_t r, float* lse, float* zt) {
  // (unrolled so that a wave has several phases' loads in flight: the single pass's chunk
  // merge reads 64 phases per row on only R / 256 workgroups; the sums keep their order)
  float M = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < l.P; ++p) M = fmaxf(M, part[l.at(0, sd, p, r)]);
  float s = 0.0f, z = 0.0f;
#pragma unroll 8
  for (int p = 0; p < l.P; ++p) {
    // all three loads unconditional and the empty partial's factor a select, so the
    // unrolled loads are issued together (a branch around one of them kept them one at a
    // time); the fused multiply-add rounds as the branch's contracted form did, and adds
    // exactly 0 for an empty partial
    const float sp = part[l.at(1, sd, p, r)], mp = part[l.at(0, sd, p, r)];
    s = fmaf(sp, sp != 0.0f ? exp2f(mp - M) : 0.0f, s);
    z += part[l.at(2, sd, p, r)];
  }
  *lse = (M + log2f(s)) * kLn2;
  *zt = z;
}

// Where the two sides' partials of one row are.
struct PartRefs {
  const float* q;  // policy
  PartLayout lq;
  int sdq;
  int64_t rq;
  const float* p;  // reference
  PartLayout lp;
  int sdp;
  int64_t rp;
};

struct MergeArgs {
  int64_t N, L, V;
  int phases, adaptive;
  int kl, detach, norm;
  float beta, inv_tau;
  const int32_t* ntok;
  const int32_t* rank;
  const int32_t* idx;
  const float* part;     // the forward's partials over all loss rows
  const float* cpart;    // single pass: the policy partials of the chunk, in the
                         // split_layout of cp_pieces launches of cp_tiles tiles each
  int64_t cp_tiles;
  int cp_pieces;
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
  int64_t c0, R;        // chunked merge: compact rows [c0, c0 + R)
  // Single-pass mode 3 (non-null): the policy partials share the row's reference mr as
  // their maximum; a row whose sum of terms 2^(lse2_q - mr) lies outside the window
  // [2^win_lo, 2^win_hi] sets *redo, and its outputs, left for the fallback to rewrite,
  // raise no status flag.  bf16: [2^-60, 2^60] (beyond it the fp32 sum overflows, or terms
  // below 2^-126 drop out of it).  fp16: [2^-4, 2^14]: a stored term p 2^(lse2_q - mr) must
  // stay below 65504, and when lse2_q < mr the terms that turn subnormal carry a rounding
  // error that dX multiplies by f = 2^(mr - lse2_q), which the window keeps below 16.  With
  // dW, fp16 takes [2^-4, 2^4]: the dW operand carries f per row, and a chunk whose f span
  // 2^18 would push its smallest rows into fp16's subnormals.  Every other row
  // gets its target entry of the chunk buffer (row r - c0, patch_ld entries per row, in
  // the storage type patch_dtype) replaced by expm1(q) / f, f = 2^(mr - lse2_q), which
  // makes the buffer row -T / f with the target entry 1 - p_y = -expm1(q) kept to the
  // precision of the storage type.
  int32_t* redo;
  float win_lo, win_hi;
  char* patch;
  int64_t patch_ld;
  int patch_dtype;
  const int32_t* gate;  // merge only when *gate != 0 (null: always)
};

// Per loss row t (compact index r):
//   q = z_q[y] / tau - lse_q, ref = z_p[y] / tau - lse_p, d = ref - q,
//   KL and dKL/dq of the chosen estimator:
//     reverse    expm1(d) - d               -expm1(d)
//     forward    expm1(-d) + d              expm1(-d)
//     reverse_q  exp(q) (expm1(d) - d)      -d exp(q)
//   l = beta * KL - A_s                      (loss value; the ratio is 1 at q = sg(q))
//   g = w_t (-A_s [if detached] + beta dKL/dq)   (dloss/dq)
// with w_t = 1 / N_tok (token mean) or 1 / (n_s S') (sequence mean: n_s loss rows of the
// row's sequence, S' sequences with any) [Long-context GRPO, §4].  pr: where the row's
// partials are (r: its compact index).  Returns the row's contribution to the loss sum
// (l, or l / n_s for the sequence mean) and ORs status bits into *flags.
// (merge_row_q: the same with the policy side's lse_q and target logit zq merged already.)
__device__ inline double merge_row_q(const MergeArgs& a, int64_t t, int64_t r,
                                     const PartRefs& pr, int32_t ntok, int* flags, float lse_q,
                                     float zq) {
  float lse_p, zp;
  merge_side(pr.p, pr.lp, pr.sdp, pr.rp, &lse_p, &zp);
  bool quiet = false;
  float l2s = 0.f;
  if (a.redo) {
    // every policy partial of a mode-3 chunk carries the row's reference as its maximum
    l2s = lse_q * kLog2e - pr.q[pr.lq.at(0, pr.sdq, 0, pr.rq)];
    if (!(l2s >= a.win_lo && l2s <= a.win_hi)) {
      atomicOr(a.redo, 1);
      quiet = true;
    }
  }
  const int64_t y = a.targets[t];
  if ((y < 0 || y >= a.V) && !quiet) *flags |= GRPO_FLAG_BAD_TARGET;
  const float q = zq * a.inv_tau - lse_q;
  const float ref = zp * a.inv_tau - lse_p;
  if (a.redo && a.patch && !quiet && y >= 0 && y < a.V) {
    const float ey = expm1f(q) * exp2f(l2s);
    u16* e = reinterpret_cast<u16*>(a.patch) + (r - a.c0) * a.patch_ld + y;
    *e = a.patch_dtype == GRPO_BF16 ? BF16T::from_f32(ey) : F16T::from_f32(ey);
  }
  const float d = ref - q;
  float klv, dkl;
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
  double ell_d = (double)a.beta * (double)klv - (double)av;
  if (a.norm == GRPO_NORM_SEQUENCES) {
    const int32_t ns = a.seq[t / a.L], nseq = a.seq[a.S];
    g = num / (float)((double)ns * (double)nseq);
    ell_d /= (double)ns;
  } else {
    g = num / (float)(ntok > 1 ? ntok : 1);
  }
  reinterpret_cast<float4*>(a.saved)[t] = make_float4(lse_q, q, ref, g);
  if (a.logp) a.logp[t] = q;
  if (a.ref_logp) a.ref_logp[t] = ref;
  if (a.kl_out) a.kl_out[t] = klv;
  if (!quiet &&
      (!isfinite(lse_q) || !isfinite(q) || !isfinite(ref) || !isfinite(klv) || !isfinite(g)))
    *flags |= GRPO_FLAG_NONFINITE;
  return ell_d;
}

__device__ inline double merge_row(const MergeArgs& a, int64_t t, int64_t r, const PartRefs& pr,
                                   int32_t ntok, int* flags) {
  float lse_q, zq;
  merge_side(pr.q, pr.lq, pr.sdq, pr.rq, &lse_q, &zq);
  return merge_row_q(a, t, r, pr, ntok, flags, lse_q, zq);
}

// merge_side by a group of kMergeLanes consecutive lanes, lane q taking the phases
// p = q (mod kMergeLanes) and the group combining them with shuffles; every lane of the
// group returns the row's results.  The whole group must be active.
__device__ inline void merge_side_group(const float* __restrict__ part, const PartLayout& l,
                                        int sd, int64_t r, int q, float* lse, float* zt) {
  // (unrolled like merge_side, so that each lane has several phases' loads in flight; the
  // sums keep their order)
  float M = -INFINITY;
#pragma unroll 8
  for (int p = q; p < l.P; p += kMergeLanes) M = fmaxf(M, part[l.at(0, sd, p, r)]);
#pragma unroll
  for (int off = 1; off < kMergeLanes; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, kMergeLanes));
  float s = 0.0f, z = 0.0f;
#pragma unroll 8
  for (int p = q; p < l.P; p += kMergeLanes) {
    const float sp = part[l.at(1, sd, p, r)], mp = part[l.at(0, sd, p, r)];
    s = fmaf(sp, sp != 0.0f ? exp2f(mp - M) : 0.0f, s);   // as in merge_side
    z += part[l.at(2, sd, p, r)];
  }
#pragma unroll
  for (int off = 1; off < kMergeLanes; off <<= 1) {
    s += __shfl_xor(s, off, kMergeLanes);
    z += __shfl_xor(z, off, kMergeLanes);
  }
  *lse = (M + log2f(s)) * kLn2;
  *zt = z;
}

__device__ inline void block_sum_store(double v, double* out) {
  __shared__ double red[kMergeBlock];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = kMergeBlock / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// Two-pass forward: grid over all rows (masked rows included so their outputs are
// zeroed), both sides' partials from one launch.  Each block reduces its rows' loss terms
// in fp64 by a fixed tree into lsum[block]; the final kernel adds the block sums in index
// order.
__global__ void __launch_bounds__(kMergeBlock) merge_kernel(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * kMergeBlock + threadIdx.x;
  const int32_t ntok = *a.ntok;
  // the layout the forward wrote: the MFMA kernels' adaptive one (both sides in one
  // launch), or the FMA kernels' fixed phases with row stride N
  PartLayout l;
  if (a.adaptive) {
    l = part_layout(ntok, 2, (a.V + 255) / 256);
  } else {
    l.P = a.phases;
    l.nsides = 2;
    l.stride = a.N;
  }
  double ell_d = 0.0;
  int flags = 0;
  if (t < a.N) {
    if (a.mask[t]) {
      const int64_t r = a.rank[t];
      const PartRefs pr{a.part, l, 0, r, a.part, l, 1, r};
      ell_d = merge_row(a, t, r, pr, ntok, &flags);
    } else {
      reinterpret_cast<float4*>(a.saved)[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.logp) a.logp[t] = 0.f;
      if (a.ref_logp) a.ref_logp[t] = 0.f;
      if (a.kl_out) a.kl_out[t] = 0.f;
    }
  }
  if (flags) atomicOr(a.status, flags);
  block_sum_store(ell_d, a.lsum + blockIdx.x);
}

// Single-pass forward: compact rows [c0, min(c0 + R, ntok)) after the chunk's policy
// partials; the reference partials come from one launch over all rows.  Blocks are
// aligned to 256 compact rows, so lsum[r / 256] sums the same rows in the same order
// whatever the chunking.
// kMergeLanes lanes per row: the chunk's policy partials (pieces x phases of them) are
// merged by the row's group of lanes, the rest of the row by its first lane; the block's
// loss sum is the same 256-row tree as merge_kernel's.
__global__ void __launch_bounds__(kMergeBlock * kMergeLanes) merge_rows_kernel(MergeArgs a) {
  __shared__ double red[kMergeBlock];
  if (a.gate && *a.gate == 0) return;
  const int32_t ntok = *a.ntok;
  const int row = threadIdx.x / kMergeLanes, q = threadIdx.x % kMergeLanes;
  const int64_t r = a.c0 + (int64_t)blockIdx.x * kMergeBlock + row;
  const int64_t blk0 = a.c0 / kMergeBlock + blockIdx.x;
  if ((int64_t)blk0 * kMergeBlock >= ntok) return;   // whole block past the last row
  const int64_t nvt = (a.V + 255) / 256;
  const int64_t crow = (ntok - a.c0 < a.R ? ntok - a.c0 : a.R);
  // policy: the chunk's own launch over its rows; reference: one launch over all rows
  const PartRefs pr{a.cpart, split_layout(crow, a.cp_tiles, a.cp_pieces), 0, r - a.c0,
                    a.part, part_layout(ntok, 1, nvt), 0, r};
  double ell_d = 0.0;
  int flags = 0;
  if (r < ntok && r < a.c0 + a.R) {   // the same for the row's whole group
    float lse_q, zq;
    merge_side_group(pr.q, pr.lq, pr.sdq, pr.rq, q, &lse_q, &zq);
    if (q == 0) ell_d = merge_row_q(a, a.idx[r], r, pr, ntok, &flags, lse_q, zq);
  }
  if (flags) atomicOr(a.status, flags);
  if (q == 0) red[row] = ell_d;
  __syncthreads();
  for (int off = kMergeBlock / 2; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.lsum[blk0] = red[0];
}

// Outputs of masked rows for the single-pass forward (its merge visits loss rows only).
__global__ void __launch_bounds__(256)
zero_masked_outputs_kernel(int64_t N, const uint8_t* __restrict__ mask, float* __restrict__ saved,
                           float* __restrict__ logp, float* __restrict__ ref_logp,
                           float* __restrict__ kl) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N || mask[t]) return;
  reinterpret_cast<float4*>(saved)[t] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (logp) logp[t] = 0.f;
  if (ref_logp) ref_logp[t] = 0.f;
  if (kl) kl[t] = 0.f;
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
loss_final_kernel(const double* __restrict__ lsum, int64_t nblocks, int compact,
                  const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ count_p,
                  float* __restrict__ loss, int32_t* __restrict__ status) {
  __shared__ double red[kFinalThreads];
  // compact: the block sums are over 256 loss rows each (single-pass forward)
  if (compact) nblocks = ((int64_t)*ntok_p + kMergeBlock - 1) / kMergeBlock;
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

// dX rows of masked positions are zero.  A wave per row, grid-stride over the rows (a
// launch of one block per 4 rows spent 0.25 ms scheduling 41k blocks for 2k masked rows),
// 16-byte stores.
__global__ void __launch_bounds__(256)
zero_rows_kernel(const uint8_t* __restrict__ mask, int64_t N, int64_t row_bytes,
                 char* __restrict__ dX) {
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t n16 = row_bytes / 16;
  for (int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / 64; t < N; t += waves) {
    if (mask[t]) continue;
    uint4* row = reinterpret_cast<uint4*>(dX + t * row_bytes);
    for (int64_t i = threadIdx.x % 64; i < n16; i += 64) row[i] = make_uint4(0, 0, 0, 0);
  }
}

// x * c rounded to fp32, then to the storage type.  The product is pinned in a register
// first, so that the compiler cannot fold the multiply and the narrowing into one
// mixed-precision instruction (one rounding instead of two) in some kernels and not in
// others: every kernel that scales a gradient gets the same bits.
template <class E>
__device__ inline typename E::T scaled(typename E::T x, float c) {
  float p = E::to_f32(x) * c;
  asm volatile("" : "+v"(p));
  return E::from_f32(p);
}

// In-place scaling of a gradient by grad_loss / loss_scale, 8 elements per thread
// (16 bytes of 16-bit data, or two 16-byte fp32 vectors), grid-stride.
template <class E>
__global__ void __launch_bounds__(256)
scale_kernel(typename E::T* __restrict__ x, int64_t n, const float* __restrict__ grad_loss,
             float loss_scale, int32_t* __restrict__ found_inf) {
  const float c = (grad_loss ? *grad_loss : 1.0f) / loss_scale;
  if (c == 1.0f) return;
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += stride) {
    if (i + 8 <= n) {
      typename E::T h[8];
      __builtin_memcpy(h, x + i, sizeof(h));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = scaled<E>(h[j], c);
        bad |= !isfinite(E::to_f32(h[j]));
      }
      __builtin_memcpy(x + i, h, sizeof(h));
    } else {
      for (int64_t k = i; k < n; ++k) {
        x[k] = scaled<E>(x[k], c);
        bad |= !isfinite(E::to_f32(x[k]));
      }
    }
  }
  if (bad) atomicOr(found_inf, 1);
}

// Gradient offload, the way back: dst[idx[r]] = src[r] * grad_loss / loss_scale for the
// rows r < *ntok (idx, ntok null: all n rows, dst[r]), with the arithmetic of scale_kernel
// (the product skipped when the factor is exactly 1), so the result equals a device-held
// gradient scaled by grpo_scale_grad bit for bit.  src is pinned host memory, read over
// PCIe: no staging copy, and nothing else to overlap with in a backward.  One row per
// block, 16 bytes per thread and step.
template <class E>
__global__ void __launch_bounds__(256)
restore_rows_kernel(const typename E::T* __restrict__ src, int64_t n, int64_t H,
                    const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                    const float* __restrict__ grad_loss, float loss_scale,
                    typename E::T* __restrict__ dst, int32_t* __restrict__ found_inf) {
  typedef typename E::T T;
  constexpr int kPer = 16 / sizeof(T);
  const int64_t r = blockIdx.x;
  if (r >= n || (ntok_p && r >= *ntok_p)) return;
  const float c = (grad_loss ? *grad_loss : 1.0f) / loss_scale;
  const T* in = src + r * H;
  T* out = dst + (idx ? (int64_t)idx[r] : r) * H;
  bool bad = false;
  for (int64_t h = (int64_t)threadIdx.x * kPer; h < H; h += 256 * kPer) {
    T v[kPer];
    __builtin_memcpy(v, in + h, 16);
    if (c != 1.0f) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        v[j] = scaled<E>(v[j], c);
        bad |= !isfinite(E::to_f32(v[j]));
      }
    }
    __builtin_memcpy(out + h, v, 16);
  }
  if (bad) atomicOr(found_inf, 1);
}

template <class E>
hipError_t scale_one(void* x, int64_t n, const float* grad_loss, float loss_scale,
                     int32_t* found_inf, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 2047) / 2048;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(scale_kernel<E>, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<typename E::T*>(x), n, grad_loss, loss_scale, found_inf);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_grad(void* dX, int dtype, int64_t nX, float* dW, int64_t nW,
                             const float* grad_loss, float loss_scale, int32_t* found_inf,
                             hipStream_t st) {
  hipError_t e;
  switch (dtype) {
    case GRPO_F32: e = scale_one<F32T>(dX, nX, grad_loss, loss_scale, found_inf, st); break;
    case GRPO_BF16: e = scale_one<BF16T>(dX, nX, grad_loss, loss_scale, found_inf, st); break;
    default: e = scale_one<F16T>(dX, nX, grad_loss, loss_scale, found_inf, st); break;
  }
  if (e != hipSuccess || !dW) return e;
  return scale_one<F32T>(dW, nW, grad_loss, loss_scale, found_inf, st);
}

hipError_t launch_restore_rows(int dtype, const void* src, int64_t n, int64_t H,
                               const int32_t* ntok, const int32_t* idx, const float* grad_loss,
                               float loss_scale, void* dst, int32_t* found_inf, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(256);
  switch (dtype) {
    case GRPO_F32:
      hipLaunchKernelGGL(restore_rows_kernel<F32T>, grid, block, 0, st, (const float*)src, n, H,
                         ntok, idx, grad_loss, loss_scale, (float*)dst, found_inf);
      break;
    case GRPO_BF16:
      hipLaunchKernelGGL(restore_rows_kernel<BF16T>, grid, block, 0, st, (const u16*)src, n, H,
                         ntok, idx, grad_loss, loss_scale, (u16*)dst, found_inf);
      break;
    default:
      hipLaunchKernelGGL(restore_rows_kernel<F16T>, grid, block, 0, st, (const u16*)src, n, H,
                         ntok, idx, grad_loss, loss_scale, (u16*)dst, found_inf);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                          int32_t* rank, hipStream_t st) {
  return launch_compact_status(mask, N, ntok, idx, rank, nullptr, st);
}

hipError_t launch_compact_status(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                                 int32_t* rank, int32_t* status, hipStream_t st) {
  int32_t* bsum = ntok + 4;  // the block counts follow the count (compact_bytes)
  const int64_t nb = (N + kCompactRows - 1) / kCompactRows;
  hipLaunchKernelGGL(compact_count_kernel, dim3((unsigned)nb), dim3(256), 0, st, mask, N, bsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, nb, bsum, ntok,
                     status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3((unsigned)nb), dim3(256), 0, st, mask, N,
                     (const int32_t*)bsum, idx, rank);
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
  a.idx = ws_ptr<int32_t>(w, p.off_idx);
  a.part = ws_ptr<float>(w, p.off_part);
  a.cpart = nullptr;
  a.cp_tiles = 0;
  a.cp_pieces = 1;
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
  a.c0 = 0;
  a.R = p.N;
  a.redo = nullptr;
  a.win_lo = a.win_hi = 0.f;
  a.patch = nullptr;
  a.patch_ld = 0;
  a.patch_dtype = 0;
  a.gate = nullptr;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nblocks), dim3(kMergeBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_loss_final(p, ws, 0, status, loss, st);
}

hipError_t launch_loss_final(const Plan& p, const void* ws, int compact, int32_t* status,
                             float* loss, hipStream_t st) {
  void* w = const_cast<void*>(ws);
  const int64_t nblocks = (p.N + kMergeBlock - 1) / kMergeBlock;
  const int32_t* ntok = ws_ptr<int32_t>(w, p.off_ntok);
  const int32_t* seq = ws_ptr<int32_t>(w, p.off_seq);
  const int32_t* count = p.norm == GRPO_NORM_SEQUENCES ? seq + p.N / p.L : ntok;
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kFinalThreads), 0, st,
                     ws_ptr<double>(w, p.off_lsum), nblocks, compact, ntok, count, loss, status);
  return hipGetLastError();
}

hipError_t launch_merge_rows(const Plan& p, const void* ws, int64_t c0, const int64_t* targets,
                             const uint8_t* mask, const float* adv, float beta, float* saved,
                             float* logp, float* ref_logp, float* kl, int32_t* status,
                             hipStream_t st, int32_t* redo, void* patch,
                             const int32_t* gate, int64_t cp_tiles, int cp_pieces) {
  void* w = const_cast<void*>(ws);
  MergeArgs a;
  a.N = p.N;
  a.L = p.L;
  a.V = p.V;
  a.phases = p.phases;
  a.adaptive = 1;
  a.kl = p.kl;
  a.detach = p.detach;
  a.norm = p.norm;
  a.beta = beta;
  a.inv_tau = p.inv_tau;
  a.ntok = ws_ptr<int32_t>(w, p.off_ntok);
  a.rank = ws_ptr<int32_t>(w, p.off_rank);
  a.idx = ws_ptr<int32_t>(w, p.off_idx);
  a.part = ws_ptr<float>(w, p.off_part);
  a.cpart = ws_ptr<float>(w, p.off_cpart);
  a.cp_tiles = cp_tiles > 0 ? cp_tiles : p.Vpad / kVocTile;
  a.cp_pieces = cp_pieces;
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
  a.c0 = c0;
  a.R = p.R;
  a.redo = redo;
  a.win_lo = p.dtype == GRPO_F16 ? -4.f : -60.f;
  a.win_hi = p.dtype == GRPO_F16 ? (p.need_dW ? 4.f : 14.f) : 60.f;
  a.patch = reinterpret_cast<char*>(patch);
  a.patch_ld = p.Vpad;
  a.patch_dtype = p.dtype;
  a.gate = gate;
  hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)(p.R / kMergeBlock)),
                     dim3(kMergeBlock * kMergeLanes),
                     0, st, a);
  return hipGetLastError();
}

hipError_t launch_zero_masked_outputs(const Plan& p, const uint8_t* mask, float* saved,
                                      float* logp, float* ref_logp, float* kl, hipStream_t st) {
  hipLaunchKernelGGL(zero_masked_outputs_kernel, dim3((unsigned)((p.N + 255) / 256)), dim3(256),
                     0, st, p.N, mask, saved, logp, ref_logp, kl);
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
  const int64_t blocks = (p.N + 3) / 4 < 1024 ? (p.N + 3) / 4 : 1024;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, mask, p.N,
                     p.H * p.esize, reinterpret_cast<char*>(dX));
  return hipGetLastError();
}

}  // namespace grpo
