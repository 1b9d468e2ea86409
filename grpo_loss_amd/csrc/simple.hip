// The fp32 path: LDS-tiled FMA kernels, 64 x 64 output tiles, 256 threads with a 4 x 4
// register tile each.  Same algorithm and workspace layout as the MFMA path:
//   forward   per (token tile, vocabulary phase, side): online max / sum-exp / target
//             logit over the phase's vocabulary tiles -> partials
//   backward  per chunk of R loss rows: T = onehot - softmax staged in the workspace,
//             dX = diag(g) T W, dW += T^T diag(g) X.
#include "common.h"

namespace grpo {
namespace {

constexpr int kT = 64;   // tile edge
constexpr int kBK = 16;  // reduction step
constexpr int kPadLds = kT + 4;

// acc[i][j] += sum_k As[k][ty*4+i] * Bs[k][tx*4+j]
__device__ inline void fma_tile(const float (*As)[kPadLds], const float (*Bs)[kPadLds], int ty,
                                int tx, float acc[4][4]) {
#pragma unroll
  for (int k = 0; k < kBK; ++k) {
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
  }
}

// z = X[idx[r]] . W[v] for a 64-token x 64-vocabulary tile, K = H (any multiple of 8: the
// last reduction step's entries past H load as 0).
template <class E>
__device__ inline void logits_tile(const typename E::T* __restrict__ xrow,
                                   const typename E::T* __restrict__ wrow, bool vok, int64_t H,
                                   float (*As)[kPadLds], float (*Bs)[kPadLds], int lrow, int lk,
                                   int ty, int tx, float acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int64_t k0 = 0; k0 < H; k0 += kBK) {
    const bool kok = k0 + lk < H;  // H % 4 == 0: a thread's 4 entries are all in or all out
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      As[lk + j][lrow] = kok ? E::to_f32(xrow[k0 + lk + j]) : 0.0f;
      Bs[lk + j][lrow] = vok && kok ? E::to_f32(wrow[k0 + lk + j]) : 0.0f;
    }
    __syncthreads();
    fma_tile(As, Bs, ty, tx, acc);
    __syncthreads();
  }
}

template <class E>
__global__ void __launch_bounds__(256)
simple_fwd_kernel(int64_t N, int64_t H, int64_t V, int phases, float scale2,
                  const int32_t* __restrict__ ntok_p,
                  const int32_t* __restrict__ idx, const typename E::T* __restrict__ Xq,
                  const typename E::T* __restrict__ Xp, const typename E::T* __restrict__ W,
                  const int64_t* __restrict__ targets, float* __restrict__ part) {
  __shared__ float As[kBK][kPadLds];
  __shared__ float Bs[kBK][kPadLds];
  const int ntok = *ntok_p;
  const int64_t r0 = (int64_t)blockIdx.x * kT;
  if (r0 >= ntok) return;
  const int phase = blockIdx.y, side = blockIdx.z;
  const typename E::T* X = side ? Xp : Xq;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  int64_t rl = r0 + lrow;
  if (rl >= ntok) rl = ntok - 1;
  const typename E::T* xrow = X + (int64_t)idx[rl] * H;
  int64_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + ty * 4 + i;
    y[i] = r < ntok ? targets[idx[r]] : -1;
  }
  float rm[4], rs[4], rz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rm[i] = -INFINITY;
    rs[i] = 0.0f;
    rz[i] = 0.0f;
  }
  const int64_t nvt = (V + kT - 1) / kT;
  for (int64_t vt = phase; vt < nvt; vt += phases) {
    const int64_t vl = vt * kT + lrow;
    const bool vok = vl < V;
    float acc[4][4];
    logits_tile<E>(xrow, W + (vok ? vl : 0) * H, vok, H, As, Bs, lrow, lk, ty, tx, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (vt * kT + tx * 4 + j < V) tmax = fmaxf(tmax, acc[i][j]);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 16));
      const float nm = fmaxf(rm[i], tmax * scale2);
      float s = rs[i] * exp2f(rm[i] - nm);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t v = vt * kT + tx * 4 + j;
        if (v < V) {
          s += exp2f(acc[i][j] * scale2 - nm);
          if (v == y[i]) rz[i] += acc[i][j];
        }
      }
      rm[i] = nm;
      rs[i] = s;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      rs[i] += __shfl_xor(rs[i], off, 16);
      rz[i] += __shfl_xor(rz[i], off, 16);
    }
    const int64_t r = r0 + ty * 4 + i;
    if (tx == 0 && r < ntok) {
      const int64_t PN = (int64_t)phases * N;
      const int64_t o = (int64_t)(side * phases + phase) * N + r;
      part[o] = rm[i];
      part[2 * PN + o] = rs[i];
      part[4 * PN + o] = rz[i];
    }
  }
}

// T[r - c0][v] = onehot(y_r)[v] - exp(z_rv / tau - lse_r) (scale2 = log2(e) / tau);
// zero for v >= V.
template <class E>
__global__ void __launch_bounds__(256)
simple_recompute_kernel(int64_t H, int64_t V, int64_t Vpad, int64_t c0, float scale2,
                        const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                        const typename E::T* __restrict__ Xq, const typename E::T* __restrict__ W,
                        const int64_t* __restrict__ targets, const float* __restrict__ saved,
                        typename E::T* __restrict__ T) {
  __shared__ float As[kBK][kPadLds];
  __shared__ float Bs[kBK][kPadLds];
  const int ntok = *ntok_p;
  const int64_t r0 = c0 + (int64_t)blockIdx.x * kT;
  if (r0 >= ntok) return;
  const int64_t v0 = (int64_t)blockIdx.y * kT;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  int64_t rl = r0 + lrow;
  if (rl >= ntok) rl = ntok - 1;
  const int64_t vl = v0 + lrow;
  const bool vok = vl < V;
  float acc[4][4];
  logits_tile<E>(Xq + (int64_t)idx[rl] * H, W + (vok ? vl : 0) * H, vok, H, As, Bs, lrow, lk, ty,
                 tx, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + ty * 4 + i;
    if (r >= ntok) continue;
    const int64_t t = idx[r];
    const int64_t y = targets[t];
    const float lse2 = saved[t * 4] * kLog2e;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t v = v0 + tx * 4 + j;
      float val = 0.0f;
      if (v < V) val = (v == y ? 1.0f : 0.0f) - exp2f(acc[i][j] * scale2 - lse2);
      T[(r - c0) * Vpad + v] = E::from_f32(val);
    }
  }
}

// dX[idx[r]] = c * g_r * sum_v T[r][v] W[v]   (c = grad_loss / loss_scale; row r - srow0
// instead of idx[r] when srow0 >= 0: a staging slot of the gradient offload)
template <class E>
__global__ void __launch_bounds__(256)
simple_dx_kernel(int64_t H, int64_t V, int64_t Vpad, int64_t c0,
                 const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                 const typename E::T* __restrict__ T, const typename E::T* __restrict__ W,
                 const float* __restrict__ saved, const float* __restrict__ grad_loss,
                 float loss_scale, typename E::T* __restrict__ dX, int64_t srow0,
                 int32_t* __restrict__ found_inf) {
  __shared__ float As[kBK][kPadLds];
  __shared__ float Bs[kBK][kPadLds];
  const int ntok = *ntok_p;
  const int64_t rt = (int64_t)blockIdx.x * kT;  // row offset within the chunk
  if (c0 + rt >= ntok) return;
  const int64_t h0 = (int64_t)blockIdx.y * kT;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;      // T loader: row, 4 consecutive v
  const int kr = tid / 16, hc = (tid % 16) * 4;       // W loader: v row, 4 consecutive h
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  const typename E::T* trow = T + (rt + lrow) * Vpad;
  for (int64_t v0 = 0; v0 < Vpad; v0 += kBK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      As[lk + j][lrow] = E::to_f32(trow[v0 + lk + j]);
      const int64_t v = v0 + kr;
      Bs[kr][hc + j] = v < V && h0 + hc < H ? E::to_f32(W[v * H + h0 + hc + j]) : 0.0f;
    }
    __syncthreads();
    fma_tile(As, Bs, ty, tx, acc);
    __syncthreads();
  }
  const float c = (grad_loss ? *grad_loss : 1.0f) / loss_scale;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = c0 + rt + ty * 4 + i;
    if (r >= ntok) continue;
    const int64_t t = idx[r];
    const float gs = saved[t * 4 + 3] * c;
    if (h0 + tx * 4 >= H) continue;  // the last H tile's columns past H (H % 4 == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float val = acc[i][j] * gs;
      const typename E::T o = E::from_f32(val);
      bad |= !isfinite(E::to_f32(o));
      dX[(srow0 < 0 ? t : r - srow0) * H + h0 + tx * 4 + j] = o;
    }
  }
  if (bad) atomicOr(found_inf, 1);
}

// dW[v] (+)= sum_r T[r][v] * c * g_r * X[idx[r]]  over this chunk's rows.
template <class E>
__global__ void __launch_bounds__(256)
simple_dw_kernel(int64_t H, int64_t V, int64_t Vpad, int64_t R, int64_t c0, int accumulate,
                 const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                 const typename E::T* __restrict__ T, const typename E::T* __restrict__ Xq,
                 const float* __restrict__ saved, const float* __restrict__ grad_loss,
                 float loss_scale, float* __restrict__ dW, int32_t* __restrict__ found_inf) {
  __shared__ float As[kBK][kPadLds];
  __shared__ float Bs[kBK][kPadLds];
  const int ntok = *ntok_p;
  int64_t nrows = (int64_t)ntok - c0;
  if (nrows > R) nrows = R;
  if (nrows <= 0 && accumulate) return;
  const int64_t v0 = (int64_t)blockIdx.x * kT;
  const int64_t h0 = (int64_t)blockIdx.y * kT;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int kr = tid / 16, cc = (tid % 16) * 4;
  const float c = (grad_loss ? *grad_loss : 1.0f) / loss_scale;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int64_t k0 = 0; k0 < nrows; k0 += kBK) {
    const int64_t r = k0 + kr;
    const bool ok = r < nrows;
    const int64_t t = ok ? idx[c0 + r] : 0;
    const float gs = ok ? saved[t * 4 + 3] * c : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      As[kr][cc + j] = ok ? E::to_f32(T[r * Vpad + v0 + cc + j]) : 0.0f;
      Bs[kr][cc + j] = ok && h0 + cc < H ? gs * E::to_f32(Xq[t * H + h0 + cc + j]) : 0.0f;
    }
    __syncthreads();
    fma_tile(As, Bs, ty, tx, acc);
    __syncthreads();
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = v0 + ty * 4 + i;
    if (v >= V || h0 + tx * 4 >= H) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* o = dW + v * H + h0 + tx * 4 + j;
      const float val = (accumulate ? *o : 0.0f) + acc[i][j];
      bad |= !isfinite(val);
      *o = val;
    }
  }
  if (bad) atomicOr(found_inf, 1);
}

template <class E>
hipError_t simple_fwd(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                      const int64_t* targets, hipStream_t st) {
  typedef typename E::T T;
  const int64_t tiles = (p.N + kT - 1) / kT;
  hipLaunchKernelGGL(simple_fwd_kernel<E>, dim3((unsigned)tiles, p.phases, 2), dim3(256), 0, st,
                     p.N, p.H, p.V, p.phases, p.scale2, ws_ptr<int32_t>(ws, p.off_ntok),
                     ws_ptr<int32_t>(ws, p.off_idx), (const T*)Xq, (const T*)Xp, (const T*)W,
                     targets, ws_ptr<float>(ws, p.off_part));
  return hipGetLastError();
}

template <class E>
hipError_t simple_bwd(const Plan& p, void* ws, const void* Xq, const void* W,
                      const int64_t* targets, const float* saved, const float* grad_loss,
                      float loss_scale, void* dX, float* dW, int accumulate_dW,
                      int32_t* found_inf, hipStream_t st) {
  typedef typename E::T T;
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  T* Tbuf = ws_ptr<T>(ws, p.off_T);
  for (int64_t c0 = 0; c0 < p.N; c0 += p.R) {
    hipLaunchKernelGGL(simple_recompute_kernel<E>, dim3((unsigned)(p.R / kT), (unsigned)(p.Vpad / kT)),
                       dim3(256), 0, st, p.H, p.V, p.Vpad, c0, p.scale2, ntok, idx, (const T*)Xq,
                       (const T*)W, targets, saved, Tbuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.ring && (e = p.ring->acquire(c0)) != hipSuccess) return e;
    const unsigned htiles = (unsigned)((p.H + kT - 1) / kT);
    hipLaunchKernelGGL(simple_dx_kernel<E>, dim3((unsigned)(p.R / kT), htiles),
                       dim3(256), 0, st, p.H, p.V, p.Vpad, c0, ntok, idx, (const T*)Tbuf,
                       (const T*)W, saved, grad_loss, loss_scale, (T*)dx_out(p, dX, c0),
                       stage_row0(p, c0), found_inf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.ring && (e = p.ring->transfer(c0)) != hipSuccess) return e;
    if (dW) {
      hipLaunchKernelGGL(simple_dw_kernel<E>, dim3((unsigned)(p.Vpad / kT), htiles),
                         dim3(256), 0, st, p.H, p.V, p.Vpad, p.R, c0,
                         c0 == 0 ? accumulate_dW : 1, ntok, idx, (const T*)Tbuf, (const T*)Xq,
                         saved, grad_loss, loss_scale, dW, found_inf);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t simple_fwd_partials(const Plan& p, void* ws, const void* Xq, const void* Xp,
                               const void* W, const int64_t* targets, hipStream_t st) {
  switch (p.dtype) {
    case GRPO_F32: return simple_fwd<F32T>(p, ws, Xq, Xp, W, targets, st);
    case GRPO_BF16: return simple_fwd<BF16T>(p, ws, Xq, Xp, W, targets, st);
    default: return simple_fwd<F16T>(p, ws, Xq, Xp, W, targets, st);
  }
}

hipError_t simple_backward(const Plan& p, void* ws, const void* Xq, const void* W,
                           const int64_t* targets, const float* saved, const float* grad_loss,
                           float loss_scale, void* dX, float* dW, int accumulate_dW,
                           int32_t* found_inf, hipStream_t st) {
  switch (p.dtype) {
    case GRPO_F32:
      return simple_bwd<F32T>(p, ws, Xq, W, targets, saved, grad_loss, loss_scale, dX, dW,
                              accumulate_dW, found_inf, st);
    case GRPO_BF16:
      return simple_bwd<BF16T>(p, ws, Xq, W, targets, saved, grad_loss, loss_scale, dX, dW,
                               accumulate_dW, found_inf, st);
    default:
      return simple_bwd<F16T>(p, ws, Xq, W, targets, saved, grad_loss, loss_scale, dX, dW,
                              accumulate_dW, found_inf, st);
  }
}

}  // namespace grpo
