// Internal declarations shared by the HIP translation units of libgrpo.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "grpo.h"

namespace grpo {

typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------------ element types
// Storage types of X, W, dX and of the staged (onehot - softmax) chunk.  Values are
// widened to fp32 for arithmetic; narrowing rounds to nearest-even.
struct F32T {
  typedef float T;
  static constexpr int kBytes = 4;
  __device__ static inline float to_f32(T v) { return v; }
  __device__ static inline T from_f32(float f) { return f; }
};

struct BF16T {
  typedef u16 T;
  static constexpr int kBytes = 2;
  __device__ static inline float to_f32(T v) { return __uint_as_float((uint32_t)v << 16); }
  __device__ static inline T from_f32(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (T)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (T)(u >> 16);
  }
  // a and b narrowed together by v_cvt_pk_bf16_f32 (nearest even, NaN stays NaN), a in
  // the low half: one instruction for what from_f32 does in several
  __device__ static inline uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
  }
  // either half of a pack2 result is inf or NaN (all exponent bits set)
  __device__ static inline bool nonfinite2(uint32_t p) {
    return (p & 0x7f80u) == 0x7f80u || (p & 0x7f800000u) == 0x7f800000u;
  }
};

struct F16T {
  typedef u16 T;
  static constexpr int kBytes = 2;
  __device__ static inline float to_f32(T v) {
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
  }
  __device__ static inline T from_f32(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
    T v;
    __builtin_memcpy(&v, &h, 2);
    return v;
  }
  // a and b narrowed together by v_cvt_pk_f16_f32 (nearest even), a in the low half
  __device__ static inline uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
  }
  // either half of a pack2 result is inf or NaN (all exponent bits set)
  __device__ static inline bool nonfinite2(uint32_t p) {
    return (p & 0x7c00u) == 0x7c00u || (p & 0x7c000000u) == 0x7c000000u;
  }
};

// fp8 e4m3 GEMM operand (per-row scaled copies of X and W); no arithmetic of its own.
struct FP8T {
  typedef uint8_t T;
  static constexpr int kBytes = 1;
};

// ------------------------------------------------------------------------ gradient offload
// rows x row_bytes from device to (pinned) host memory on stream st, on the copy engines:
// this runtime runs the one-dimensional device-to-host copy as a kernel on the compute
// units, which cannot start while a persistent GEMM holds every CU (measured: 1.25 GiB of
// such copies added 29 ms to a 411 ms step), while the two-dimensional form goes to the
// SDMA engines and runs beside the kernels.
inline hipError_t copy_to_host(void* dst, const void* src, size_t row_bytes, size_t rows,
                               hipStream_t st) {
  return hipMemcpy2DAsync(dst, row_bytes, src, row_bytes, row_bytes, rows,
                          hipMemcpyDeviceToHost, st);
}

// Two staging slots of a chunk's rows between the call's stream (st), whose kernels fill a
// slot, and a copy stream (cs), which copies it to pinned host memory; a slot is refilled
// only after its previous copy is done.  grpo_loss_fwd_bwd's gradient offload writes
// dX rows through it.  Event handles are created and destroyed by the entry point; nothing
// here allocates memory.
struct CopyRing {
  char* slots = nullptr;   // 2 x rows x row_bytes of device memory (the workspace)
  char* host = nullptr;    // pinned host rows, row r at host + r row_bytes
  size_t row_bytes = 0;
  int64_t rows = 0;        // rows per slot
  int64_t total = 0;       // rows of the host buffer
  hipStream_t st = nullptr, cs = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  int used[2] = {0, 0};

  int slot_of(int64_t r0) const { return (int)((r0 / rows) & 1); }
  char* slot(int64_t r0) const { return slots + (size_t)slot_of(r0) * rows * row_bytes; }
  // st waits until slot(r0)'s previous copy is done
  hipError_t acquire(int64_t r0) {
    const int s = slot_of(r0);
    return used[s] ? hipStreamWaitEvent(st, freed[s], 0) : hipSuccess;
  }
  // rows [r0, r0 + rows) to the host once the kernels enqueued on st so far are done
  hipError_t transfer(int64_t r0) {
    const int s = slot_of(r0);
    const int64_t n = total - r0 < rows ? total - r0 : rows;
    hipError_t e;
    if ((e = hipEventRecord(ready[s], st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(cs, ready[s], 0)) != hipSuccess) return e;
    e = copy_to_host(host + (size_t)r0 * row_bytes, slot(r0), row_bytes, (size_t)n, cs);
    if (e != hipSuccess) return e;
    used[s] = 1;
    return hipEventRecord(freed[s], cs);
  }
};

// ------------------------------------------------------------------------ workspace plan
// One plan describes every buffer carved out of the caller's workspace.  The host fills
// it from the sizes alone (the number of loss tokens lives on the device).
struct Plan {
  int64_t N;        // rows = S * L
  int64_t L, H, V;
  int64_t Vpad;     // V rounded up to the vocabulary tile (256)
  int dtype;        // grpo_dtype
  int esize;        // bytes per element of X / W / T
  int need_dW;
  int phases;       // fp32 FMA forward: vocabulary phases (fixed; partial stride N)
  int64_t R;        // backward: rows per recompute chunk (multiple of 256)
  int chunk_rows;   // grpo_options::chunk_rows (0: the default chunk)
  int vocab_piece;  // grpo_options::vocab_piece (0: the default piece)
  int ksplit;       // backward: split of the dX reduction over the vocabulary
  int mfma;         // 1: 16-bit MFMA kernels, 0: fp32 FMA kernels
  // Vocabulary split of the backward (MFMA, no dW): a chunk's terms are produced and
  // consumed one piece of ptiles vocabulary tiles at a time (npieces per chunk), so the
  // chunk buffer holds R x (ptiles * 256) entries, and dX accumulates in fp32 [ksplit][R][H]
  int vsplit;
  int npieces;
  int64_t ptiles;
  int64_t pt_ld;    // entries per row of the chunk buffer: ptiles * 256, or Vpad
  // loss variant (grpo_options)
  int kl;           // grpo_kl_estimator
  int detach;       // 1: ratio exp(q - sg(q)), 0: exp(q - q)
  int norm;         // grpo_normalization
  float inv_tau;    // 1 / temperature
  float scale2;     // log2(e) / temperature: logits -> log2 units of the softmax argument
  int fp8;          // logits from per-row e4m3 copies of X and W
  // event brackets around one kernel's launches (grpo_options.trace_*); trace_n counts the
  // launches of this call (a counter owned by the entry point, may be null)
  int trace_kernel, trace_cap;
  void* const* trace_ev;
  int* trace_n;
  // byte offsets into the workspace
  size_t off_ntok, off_idx, off_rank, off_part, off_lsum, off_seq, off_T, off_pm, off_Xg,
      off_redo, off_dxp, off_xq8, off_xp8, off_w8, off_sxq, off_sxp, off_sw, total;
  size_t off_cpart;  // forward partials of one chunk of policy rows (single pass)
  size_t off_xgs;    // dW operand's chunk scale (2^k, 2^-k)
  size_t fwd_total;  // bytes the forward alone (grpo_loss_fwd) uses: a prefix of the plan
  size_t off_ring;   // gradient offload: two staging slots of R rows x H (grpo_options.dx_host)
  int offload;       // grpo_options.dx_host is set
  // gradient offload of this call (null: dX rows go to dX[idx[r]]).  A chunk's dX writer
  // then takes dx_out(p, dX, c0) as its base and stage_row0(p, c0) as the row of c0.
  CopyRing* ring;
};

// Base pointer and the loss-row origin of the chunk at c0's dX writes: with the offload,
// the chunk's staging slot, loss row r landing in its row r - c0; without, dX itself with
// rows idx[r] (origin -1).
inline void* dx_out(const Plan& p, void* dX, int64_t c0) {
  return p.ring ? (void*)p.ring->slot(c0) : dX;
}
inline int64_t stage_row0(const Plan& p, int64_t c0) { return p.ring ? c0 : -1; }

constexpr int kTokTile = 256;    // rows per token tile of the MFMA kernels
constexpr int kVocTile = 256;    // vocabulary entries per tile
constexpr int kMergeBlock = 256; // rows per block of the merge kernel
constexpr int kMergeLanes = 4;   // lanes per row merging a chunk's policy partials
constexpr int kMaxPhases = 32;   // vocabulary phases of the FMA forward
constexpr int kMaxFwdPhases = 256; // most vocabulary phases of one MFMA forward launch
constexpr int kPieceTiles = 128; // vocabulary tiles per piece of the split backward (32768)
constexpr int kCompactRows = 4096; // rows per workgroup of the row compaction

// Bytes of the loss-row count's slot in a workspace: the count (16 bytes), then the row
// compaction's per-block counts.
inline size_t compact_bytes(int64_t N) {
  return 16 + (size_t)((N + kCompactRows - 1) / kCompactRows) * 4;
}

// Vocabulary phases of the MFMA forward.  Its persistent grid (8 XCDs x 32 workgroups)
// covers 256 / P token blocks x P phases per round (32 / P per XCD for P <= 32; a token
// block's phases spread over P / 32 XCDs above that); pick P in {4, .., 256} that
// minimises the tiles per workgroup, ceil(blocks / (256 / P)) * ceil(tiles / P),
// preferring fewer phases (each W tile then feeds more workgroups of an XCD; W tiles are
// also shared across XCDs, X blocks are not).  Phases past 32 serve short launches, whose
// last round 32 phases would leave on few XCDs (a last chunk of 3 token blocks: P = 64,
// all 8 XCDs, instead of 3; 19 token blocks: rounds of 4 instead of 8, 8 and 3); they are
// considered only while P x blocks <= kWidePhaseBlocks, which bounds the partials (P per
// row) of the launches that pick them below those of the largest launches.
constexpr int64_t kWidePhaseBlocks = 2048;
__host__ __device__ inline int fwd_phases(int64_t token_blocks, int64_t vocab_tiles) {
  int best = 4;
  int64_t best_cost = -1;
  for (int P = 4; P <= kMaxFwdPhases; P *= 2) {
    if (P > 32 && P * token_blocks > kWidePhaseBlocks) break;
    const int64_t per_round = 256 / P;
    const int64_t cost = ((token_blocks + per_round - 1) / per_round) * ((vocab_tiles + P - 1) / P);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = P;
    }
  }
  return best;
}

// Where a forward launch keeps its partials: for `rows` loss rows of `nsides` sides it
// runs P = fwd_phases(nsides * ntbs, nvt) phases (ntbs = ceil(rows / 256)) and holds, per
// (side, phase, row), the running maximum in log2 units (q = 0), the sum of exp2 (q = 1)
// and the target logit (q = 2) at at(q, sd, ph, r), rows padded to whole token blocks.
// The device derives the layout from the number of loss rows it counted; the host sizes
// the buffer for the largest layout any count up to the rows it knows of can produce.
struct PartLayout {
  int P;
  int nsides;
  int64_t stride;  // rows per (quantity, side, phase) slot
  __host__ __device__ inline int64_t at(int q, int sd, int ph, int64_t r) const {
    return ((int64_t)(q * nsides + sd) * P + ph) * stride + r;
  }
};
__host__ __device__ inline PartLayout part_layout(int64_t rows, int nsides, int64_t nvt) {
  const int64_t ntbs = (rows + 255) / 256;
  PartLayout l;
  l.P = fwd_phases(nsides * ntbs, nvt);
  l.nsides = nsides;
  l.stride = ntbs * 256;
  return l;
}
// Several launches over the same rows of one side, one per vocabulary piece of ptiles
// tiles: each runs P = fwd_phases(ntbs, ptiles) phases (the last piece's empty phases
// write empty partials) and piece j's phase ph lands in slot j P + ph.  With one piece of
// every tile this is part_layout(rows, 1, nvt).
__host__ __device__ inline PartLayout split_layout(int64_t rows, int64_t ptiles, int npieces) {
  const int64_t ntbs = (rows + 255) / 256;
  PartLayout l;
  l.P = npieces * fwd_phases(ntbs, ptiles);
  l.nsides = 1;
  l.stride = ntbs * 256;
  return l;
}
// Floats of the largest layout over 0 <= rows <= max_rows: part_layout(rows, nsides, tiles)
// (npieces = 1), or split_layout(rows, tiles, npieces) (nsides = 1).
size_t part_floats_max(int64_t max_rows, int nsides, int64_t tiles, int npieces = 1);

bool make_plan(int64_t S, int64_t L, int64_t H, int64_t V, int dtype, int need_dW, Plan* p,
               const grpo_options* opts = nullptr);
// Copies a validated grpo_options (NULL = defaults) into the plan.
void plan_options(const grpo_options* o, Plan* p);

// Event brackets around the launches of the kernel the caller asked to time (no-ops for
// any other kernel).  Recording is a stream operation: nothing synchronises.
inline void trace_begin(const Plan& p, int kernel, hipStream_t st) {
  if (p.trace_kernel != kernel || !p.trace_n || !p.trace_ev || *p.trace_n >= p.trace_cap) return;
  (void)hipEventRecord((hipEvent_t)p.trace_ev[2 * *p.trace_n], st);
}
inline void trace_end(const Plan& p, int kernel, hipStream_t st) {
  if (p.trace_kernel != kernel || !p.trace_n) return;
  if (p.trace_ev && *p.trace_n < p.trace_cap)
    (void)hipEventRecord((hipEvent_t)p.trace_ev[2 * *p.trace_n + 1], st);
  ++*p.trace_n;
}

template <typename P>
inline P* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off);
}

// ------------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  All run on `st` and read the number of
// loss tokens from device memory (ntok), so no host synchronisation is needed.
hipError_t launch_advantages(const float* rewards, int64_t B, int64_t G, int64_t K, float eps,
                             int unbiased, float* adv, hipStream_t st);
// ntok: compact_bytes(N) bytes (the count, then scratch of the compaction).
hipError_t launch_compact(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                          int32_t* rank, hipStream_t st);
// Same, and clears the forward's status word first.
hipError_t launch_compact_status(const uint8_t* mask, int64_t N, int32_t* ntok, int32_t* idx,
                                 int32_t* rank, int32_t* status, hipStream_t st);
hipError_t launch_merge(const Plan& p, const void* ws, const int64_t* targets,
                        const uint8_t* mask, const float* adv, float beta, float* saved,
                        float* logp, float* ref_logp, float* kl, int32_t* status, float* loss,
                        hipStream_t st);
// Single-pass forward: merge of compact rows [c0, c0 + R) (R = Plan::R), the zeroing of
// masked rows' outputs, and the loss reduction (compact = 1: block sums over loss rows).
// redo (non-null): the policy partials are fixed-reference ones, a row out of their range
// sets *redo, and (patch non-null) the other rows' target entries of the chunk buffer
// `patch` (Plan::Vpad entries per row) are rewritten; gate (non-null): merge only when
// *gate != 0.  The chunk's policy partials follow split_layout(rows, cp_tiles, cp_pieces)
// (cp_tiles 0: every tile, one piece).
hipError_t launch_merge_rows(const Plan& p, const void* ws, int64_t c0, const int64_t* targets,
                             const uint8_t* mask, const float* adv, float beta, float* saved,
                             float* logp, float* ref_logp, float* kl, int32_t* status,
                             hipStream_t st, int32_t* redo = nullptr, void* patch = nullptr,
                             const int32_t* gate = nullptr, int64_t cp_tiles = 0,
                             int cp_pieces = 1);
hipError_t launch_zero_masked_outputs(const Plan& p, const uint8_t* mask, float* saved,
                                      float* logp, float* ref_logp, float* kl, hipStream_t st);
hipError_t launch_loss_final(const Plan& p, const void* ws, int compact, int32_t* status,
                             float* loss, hipStream_t st);
// Per-row e4m3 quantisation of rows src[idx ? idx[r] : r] for r < (ntok ? *ntok : nmax):
// scale[r] = amax / 448, dst[r][:] = e4m3(x * (448 / amax)), round to nearest even.
hipError_t launch_quant_rows(int dtype, const void* src, int64_t H, const int32_t* idx,
                             const int32_t* ntok, int64_t nmax, uint8_t* dst, float* scale,
                             hipStream_t st);
// x *= grad_loss / loss_scale over n16 elements of the storage type and nW fp32 elements;
// found_inf on a non-finite result.  Nothing happens when the factor is exactly 1.
// grad_loss null: 1.
hipError_t launch_scale_grad(void* dX, int dtype, int64_t nX, float* dW, int64_t nW,
                             const float* grad_loss, float loss_scale, int32_t* found_inf,
                             hipStream_t st);
// Gradient offload, the way back: dst[idx[r]] = src[r] * grad_loss / loss_scale
// (grad_loss null: 1) for r < *ntok (idx and ntok null: every one of the n rows, in place
// order), with the arithmetic of launch_scale_grad.  src may be pinned host memory, which
// the kernel reads over PCIe.
hipError_t launch_restore_rows(int dtype, const void* src, int64_t n, int64_t H,
                               const int32_t* ntok, const int32_t* idx, const float* grad_loss,
                               float loss_scale, void* dst, int32_t* found_inf, hipStream_t st);
// Loss rows per sequence and the number of sequences that have any (sequence-mean
// normalisation only).
hipError_t launch_seq_counts(const Plan& p, const uint8_t* mask, void* ws, hipStream_t st);
hipError_t launch_zero_masked_rows(const Plan& p, const uint8_t* mask, void* dX,
                                   hipStream_t st);

// Forward partials (online max / sum-exp / target logit per row and vocabulary phase).
hipError_t launch_fwd_partials(const Plan& p, void* ws, const void* Xq, const void* Xp,
                               const void* W, const int64_t* targets, hipStream_t st);
// Backward over all row chunks: recompute, dX (and dW).
hipError_t launch_bwd(const Plan& p, void* ws, const void* Xq, const void* W,
                      const int64_t* targets, const float* saved, const float* grad_loss,
                      float loss_scale, void* dX, float* dW, int accumulate_dW,
                      int32_t* found_inf, hipStream_t st);

}  // namespace grpo
