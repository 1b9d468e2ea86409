// The 16-bit path: MFMA kernels for gfx950 (v_mfma_f32_16x16x32_{bf16,f16}).
//
// Every GEMM here is C[m][n] = sum_k A[m][k] * B[n][k], each operand stored either with k
// contiguous (X and W in the forward, T in dX) or with k as its row index (W in dX, T and
// g X in dW), both read in place.  Block tile 256 (m) x 256 (n) x 64 (k), 512 threads =
// 8 waves in a 2 (m) x 4 (n) grid, each wave owning a 128 x 64 sub-tile as 8 x 4 MFMA
// blocks of 16 x 16 (128 fp32 accumulators per lane).  Two waves share each SIMD, so the
// accumulators fit in the architectural VGPRs with room to spare (a 128 x 128 wave tile
// needs all 256 AGPRs and the register allocator then shuffles accumulators between
// MFMAs), and one wave's LDS and barrier latency is covered by its neighbour's MFMAs.
// Operand tiles go straight from global memory
// into a double-buffered LDS ring (2 x 64 KB) with buffer_load_dwordx4 ... lds, so no
// registers are spent on staging; the 16-byte chunks of a tile row are XOR-swizzled so
// fragment reads are free of bank conflicts.
//
// In the 16 x 16 accumulator layout, lane l holds C[4*(l/16) + j][l % 16], j = 0..3.
// All kernels put the vocabulary (or the hidden dimension) on m and tokens on n, so a
// lane owns whole token columns: the forward's online max / sum-exp runs per lane with
// no cross-lane traffic until a token block is finished.
#include "common.h"

namespace grpo {

hipError_t mfma_fwd_partials(const Plan& p, void* ws, const void* Xq, const void* Xp,
                             const void* W, const int64_t* targets, hipStream_t st);
hipError_t mfma_backward(const Plan& p, void* ws, const void* Xq, const void* W,
                         const int64_t* targets, const float* saved, const float* grad_loss,
                         float loss_scale, void* dX, float* dW, int accumulate_dW,
                         int32_t* found_inf, hipStream_t st);
hipError_t mfma_fused(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                      const int64_t* targets, const uint8_t* mask, const float* adv, float beta,
                      float* saved, float* logp, float* ref_logp, float* kl, int32_t* status,
                      float* loss, const float* grad_loss, float loss_scale, void* dX, float* dW,
                      int accumulate_dW, int32_t* found_inf, hipStream_t st);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class E>
struct Mma;
template <>
struct Mma<BF16T> {
  __device__ static inline f32x4 op(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mma<F16T> {
  __device__ static inline f32x4 op(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

typedef int v8i __attribute__((ext_vector_type(8)));
template <>
struct Mma<FP8T> {
  // v_mfma_f32_16x16x128_f8f6f4 with both operands e4m3 and unit block scales: 32 bytes
  // of k per lane and row.  Any k order shared by A and B gives the same dot product, so
  // lane group g simply takes bytes 32 g .. 32 g + 31 of the 128-byte k-step.
  __device__ static inline f32x4 op(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
    const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                   (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                   (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

constexpr int kThreads = 512;
constexpr int kWN = 4;                        // waves along n
constexpr int kMB = 8, kNB = 4;               // 16 x 16 blocks per wave along m, n
constexpr int kWaveN = 16 * kNB;              // 64 columns per wave
constexpr int kTileBytes = 256 * 64 * 2;      // one operand, one stage: 256 rows x 128 B
constexpr int kNumWG = 256;                   // persistent grid: one workgroup per CU
constexpr int kXcds = 8;

// LDS layout of one operand tile: 256 rows x 128 B; the 16-byte chunk c of row r sits at
// position c ^ f(r) of its row, f(r) = (r & 7) ^ ((r >> 3) & 1).  A fragment read has 16
// consecutive rows at one chunk: rows 0-7 and 8-15 each land on 8 distinct positions
// (conflict free when the LDS serves 8 lanes x 16 B per pass over 32 banks), and the 16
// (row parity, position) pairs are distinct (conflict free for 16 lanes over 64 banks).
//
// Tiles are filled with buffer_load_dwordx4 ... lds: one wave instruction writes 1 KB of LDS
// (8 rows) with lane l landing at byte 16 l.  Wave w's instruction i covers rows
// 32 w + 8 i .. + 7, so lane l lands in row r = 32 w + 8 i + l / 8 at position l % 8 and
// therefore loads chunk (l % 8) ^ f(r) of that row: the swizzle is applied to the source
// address.  Every thread stages the same 8 rows of each operand for every k, addressed as
// a wave-uniform base plus a 32-bit per-row offset.
//
// The two ring stages are four distinct LDS arrays and the k loop is unrolled by two,
// so every LDS read names the array it reads and the compiler can see that the loads in
// flight target the other stage: it then waits for them only at the barrier that hands
// the stage over, and the loads overlap the MFMAs of the current stage.
__shared__ __attribute__((aligned(16))) char g_sA0[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_sB0[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_sA1[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_sB1[kTileBytes];

__device__ inline int stage_row(int i) {
  return 32 * (int)(threadIdx.x >> 6) + 8 * i + (int)((threadIdx.x & 63) >> 3);
}
__device__ inline int swz_f(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ inline uint32_t stage_chunk_bytes(int r) {
  return (uint32_t)((((int)threadIdx.x & 7) ^ swz_f(r)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void_t;
// An operand as a buffer resource: base, extent in bytes (loads past it return 0), and the
// raw-buffer format word of this GPU family.  The tile loads then take one 32-bit VGPR
// offset per lane and the k-step offset in an SGPR, instead of 64-bit per-lane addresses.
typedef __amdgpu_buffer_rsrc_t Src;
__device__ inline Src make_src(const char* base, const char* end) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0,
                                           (int)(uint32_t)(end - base), 0x00020000);
}

typedef f32x4 Acc[kMB][kNB];
typedef uint32_t Offs[4];

// A second tile layout, for an operand stored with m (or n) contiguous and k as the row
// index, such as W [V][H] as the A operand of dX = T W or a row block of T as the B operand
// of dW = T^T X: 64 k-rows of 256 entries (512 B).  The 32-byte unit u of k-row r sits at
// unit u ^ F(r) of its row, F(r) = (r & 3) | ((r >> 3) & 1) << 2.
//
// Fragments come from ds_read_b64_tr_b16: in each 16-lane group, source lane s addresses
// 4 consecutive entries of one k-row, and lane j receives entry j % 4 of the rows read by
// source lanes 4 i + j / 4, i = 0..3.  With source lane s pointing at k-row k0 + s / 4,
// entries m0 + 4 (s % 4) .. + 3, lane j therefore holds k0 .. k0 + 3 of entry m0 + j, the
// layout of half an MFMA operand.  Lane group g reads k-rows 8 g + 4 t + (0..3) for the
// two halves t, so the 8 k-rows of a two-group read pass have 8 distinct F and their
// 32-byte units fall on 8 distinct bank windows.
//
// Staging: wave w's instruction i writes k-rows 8 w + 2 i and 8 w + 2 i + 1 (1 KB); lane l
// lands at 16-byte position l % 32 of k-row 8 w + 2 i + l / 32 and loads chunk
// (l % 32) ^ 2 F(row) of that row.
__device__ inline int nat_f(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// Staging offsets of a natural-layout operand with ld bytes per k-row, for instructions
// i = 0 and 1.  Instruction i + 2 writes the k-rows 4 further on, whose F is the same
// (r & 3 repeats with period 4 in i, and (r >> 3) & 1 = w & 1 for all four), so it reuses
// the offset of i from a resource based 4 k-rows further (Op<true>::at_hi): two VGPRs per
// operand instead of four, and loads past the operand's end still return 0.
__device__ inline void nat_offsets(int64_t ld, Offs& o) {
  const int l = (int)threadIdx.x & 63, w = (int)(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * w + 2 * i + (l >> 5);
    o[i] = (uint32_t)(r * ld) + (uint32_t)(((l & 31) ^ (2 * nat_f(r))) << 4);
  }
  o[2] = o[3] = 0;
}

// An operand of the k loop.  kNat = false: rows are m (n) with k contiguous; k-step kt is
// the byte offset 128 kt of every row.  kNat = true: rows are k; k-step kt starts kstep
// bytes further, and the resource is rebuilt from there with the bytes left to the
// operand's end, so that k-rows past it (a vocabulary padded past V) load as 0.
template <bool kNat>
struct Op;
template <>
struct Op<false> {
  Src r;
  __device__ inline Src at(int kt, int& so) const {
    so = kt * 128;
    return r;
  }
};
template <>
struct Op<true> {
  const char* base;
  int64_t left;   // bytes from base to the end of the operand
  int64_t kstep;
  __device__ inline Src at(int kt, int& so) const {
    so = 0;
    return from((int64_t)kt * kstep);
  }
  // k-step kt's second half of staged k-rows: 4 k-rows (kstep / 16 bytes) further on
  __device__ inline Src at_hi(int kt) const { return from((int64_t)kt * kstep + (kstep >> 4)); }
  __device__ inline Src from(int64_t o) const {
    const int64_t n = left - o;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + o), (short)0,
                                             n > 0 ? (int)(uint32_t)n : 0, 0x00020000);
  }
};

typedef short v4s __attribute__((ext_vector_type(4)));
// Half an MFMA operand (4 k of one m) from a natural-layout tile: see above.
__device__ inline uint2 tr_read(const char* p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<char*>(p)));
  return __builtin_bit_cast(uint2, v);
}
// The 8-k operand of fragment unit x (already XORed with F) for k half hf: rows
// 32 hf + 8 g + 0..7 of this lane's entry.  lb is the lane's base: k-row 8 g + s / 4,
// byte 8 (s % 4).
__device__ inline uint4 nat_frag(const char* tile, int lb, int x, int hf) {
  const char* q = tile + lb + (x << 5) + hf * (32 * 512);
  const uint2 lo = tr_read(q), hi = tr_read(q + 4 * 512);
  return uint4{lo.x, lo.y, hi.x, hi.y};
}

__device__ inline void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Enqueue the direct-to-LDS loads of k-step kt into stage S.
template <int S, bool kNatA, bool kNatB>
__device__ inline void stage_tiles(const Op<kNatA>& A, const Op<kNatB>& B, const Offs& ao,
                                   const Offs& bo, int kt, int w) {
  char* sa = (S ? g_sA1 : g_sA0) + w * 4 * 1024;
  char* sb = (S ? g_sB1 : g_sB0) + w * 4 * 1024;
  int soa, sob;
  const Src ra = A.at(kt, soa), rb = B.at(kt, sob);
  Src ra2 = ra, rb2 = rb;
  if constexpr (kNatA) ra2 = A.at_hi(kt);
  if constexpr (kNatB) rb2 = B.at_hi(kt);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kNatA && i >= 2 ? ra2 : ra,
                                             (lds_void_t*)(sa + i * 1024), 16,
                                             (int)ao[kNatA ? (i & 1) : i], soa, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kNatB && i >= 2 ? rb2 : rb,
                                             (lds_void_t*)(sb + i * 1024), 16,
                                             (int)bo[kNatB ? (i & 1) : i], sob, 0, 0);
  }
}

// fp8 operands: acc += (128-wide k slab of stage S), one 16 x 16 x 128 MFMA per block.
// Fragment rows wm*128 + mb*16 + (lane & 15) of A and wn*64 + nb*16 + (lane & 15) of B,
// chunks 2 g and 2 g + 1 of each row (g = lane / 16); all fragments are requested up front.
// (The 16-bit operands go through the pipelined kstep_pipe below.)
template <int S>
__device__ inline void mma_stage_fp8(Acc& acc, int fa, int fb, int fs, int lane) {
  const char* As = S ? g_sA1 : g_sA0;
  const char* Bs = S ? g_sB1 : g_sB0;
  // Raised wave priority while this wave feeds the matrix unit: the arbiter then prefers
  // the MFMA-issuing wave over its SIMD neighbour that is between bursts (+10% measured
  // with this stage-at-a-time schedule).
  __builtin_amdgcn_s_setprio(1);
  {
    // fp8: one 16 x 16 x 128 MFMA per block and k-step, chunks 2 g and 2 g + 1 per lane
    const int g2 = 2 * (lane >> 4);
    const int c0 = (g2 ^ fs) << 4;
    const int c1 = ((g2 + 1) ^ fs) << 4;
    uint4 a0[kMB], a1[kMB], b0[kNB], b1[kNB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      a0[mb] = *reinterpret_cast<const uint4*>(As + fa + mb * 2048 + c0);
      a1[mb] = *reinterpret_cast<const uint4*>(As + fa + mb * 2048 + c1);
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      b0[nb] = *reinterpret_cast<const uint4*>(Bs + fb + nb * 2048 + c0);
      b1[nb] = *reinterpret_cast<const uint4*>(Bs + fb + nb * 2048 + c1);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[mb][nb] = Mma<FP8T>::op(a0[mb], a1[mb], b0[nb], b1[nb], acc[mb][nb]);
  }
  __builtin_amdgcn_s_setprio(0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for data exchanged through ds_write / ds_read only: it waits for this
// wave's LDS instructions but not for its vector memory operations in flight, which
// __syncthreads (and an LDS fence, because of the direct-to-LDS loads) would drain as well:
// the next tile's prefetch and the stored softmax terms.  Callers must not read LDS that a
// direct-to-LDS load in flight writes.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 2^x with the bare v_exp_f32: results below 2^-126 come back as 0 instead of a
// subnormal.  Used only for softmax terms exp2(z - m) with m at least the running
// maximum, where a term that small cannot change an fp32 sum that already holds a
// term of 1.
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// First half of the k-loop prologue: enqueue k-step 0 into stage 0.  Stage 0 is free
// once the previous gemm_main on this workgroup has returned, so a persistent kernel
// issues its next tile's loads before working on the previous tile's accumulators.
// rot: the k loop visits k-steps rot, rot + 1, .., nk - 1, 0, .., rot - 1 (0 <= rot < nk),
// the same rot given to gemm_main for the tile.
template <bool kNatA = false, bool kNatB = false>
__device__ inline void gemm_pre_op(const Op<kNatA>& A, const Op<kNatB>& B, const Offs& ao,
                                   const Offs& bo, int rot = 0) {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  stage_tiles<0>(A, B, ao, bo, rot, w);
}
__device__ inline void gemm_pre(Src ra, Src rb, const Offs& ao, const Offs& bo, int rot = 0) {
  gemm_pre_op(Op<false>{ra}, Op<false>{rb}, ao, bo, rot);
}

// Fragment reads of one k-step for the pipelined core below.  A fragment (A row block mb,
// k half hf) and B fragment (B row block nb, k half hf) of stage S, in either tile layout.
struct FragBase {
  int fa, fb, c0, c1, F, wn4;
};
template <int S, bool kNat>
__device__ inline uint4 frag_a(const FragBase& q, int mb, int hf) {
  const char* As = S ? g_sA1 : g_sA0;
  if constexpr (kNat) return nat_frag(As, q.fa, mb ^ q.F, hf);
  else return *reinterpret_cast<const uint4*>(As + q.fa + mb * 2048 + (hf ? q.c1 : q.c0));
}
template <int S, bool kNat>
__device__ inline uint4 frag_b(const FragBase& q, int nb, int hf) {
  const char* Bs = S ? g_sB1 : g_sB0;
  if constexpr (kNat) return nat_frag(Bs, q.fb, (q.wn4 + nb) ^ q.F, hf);
  else return *reinterpret_cast<const uint4*>(Bs + q.fb + nb * 2048 + (hf ? q.c1 : q.c0));
}
// One k-step of the pipelined 16-bit core, stage S.  A k-step is eight groups of 8 MFMAs
// (k half 0, A row blocks 0-1, 2-3, 4-5, 6-7 against the four B row blocks; then k half
// 1), and each group's fragments are requested while the group before it runs, so the
// matrix unit does not wait on an LDS read that could have been issued earlier.  On entry
// a and b hold (or are receiving) the first group's fragments; on exit the next k-step's.
// The hand-over barrier comes before the last group: this wave's reads of stage S have
// all been issued by then (the barrier waits for them), stage S ^ 1 is complete for every
// wave, so the next k-step's first fragments are requested from it while the last 8 MFMAs
// run, and the stage just read is refilled with k-step kt + 2.  Peak fragment registers:
// the current group's and the next one's, 48 at a k-half boundary.
template <class G, int S, bool kNatA, bool kNatB>
__device__ inline void kstep_pipe(const Op<kNatA>& A, const Op<kNatB>& B, const Offs& ao,
                                  const Offs& bo, int kt, int nk, int rot, int w, FragBase q,
                                  Acc& acc, uint4 (&a)[2], uint4 (&b)[kNB]) {
  // keep the natural-layout fragment addresses from being hoisted out of the k loop and
  // held in registers (they are one v_xad each at the read)
  if constexpr (kNatA || kNatB) asm("" : "+v"(q.F) : "s"(kt));
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 na[2], nb[kNB];
      const bool last = h == 1 && j == 3;
      if (last) {
        __builtin_amdgcn_s_setprio(0);
        wait_vmem();
        __syncthreads();  // stage S ^ 1 holds k-step kt + 1; every wave is done reading stage S
        // After the last k-step these read stage 0, which nothing is filling then; the
        // values are dead.  Reading unconditionally keeps selects out of the hand-over.
        // The reads go before the refill of stage S: issued after it, the compiler's
        // wait insertion put an s_waitcnt vmcnt on reads inside the k loop (a full memory
        // round trip for the loads just issued), although no read touches the stage
        // being filled.
        na[0] = frag_a<S ^ 1, kNatA>(q, 0, 0);
        na[1] = frag_a<S ^ 1, kNatA>(q, 1, 0);
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) nb[jj] = frag_b<S ^ 1, kNatB>(q, jj, 0);
        __builtin_amdgcn_s_setprio(1);
      } else if (j < 3) {
        na[0] = frag_a<S, kNatA>(q, 2 * j + 2, h);
        na[1] = frag_a<S, kNatA>(q, 2 * j + 3, h);
      } else {
        na[0] = frag_a<S, kNatA>(q, 0, 1);
        na[1] = frag_a<S, kNatA>(q, 1, 1);
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) nb[jj] = frag_b<S, kNatB>(q, jj, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int n = 0; n < kNB; ++n)
          acc[2 * j + i][n] = Mma<G>::op(a[i], b[n], acc[2 * j + i][n]);
        // the refill of the stage just read is issued after the last group's first 4
        // MFMAs, so the matrix unit restarts right after the barrier
        if (last && i == 0) {
          __builtin_amdgcn_sched_barrier(0);
          if (kt + 2 < nk) {
            const int k = kt + 2 + rot;
            stage_tiles<S>(A, B, ao, bo, k < nk ? k : k - nk, w);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      a[0] = na[0];
      a[1] = na[1];
      if (j == 3) {
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) b[jj] = nb[jj];
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// acc += A . B^T over nk k-steps of 64 (nk even and > 0), k-step 0 already enqueued by
// gemm_pre.  Row i of this thread's staging set is at byte ao[i] of A's buffer and bo[i]
// of B's for k-step 0.  On return every wave has finished reading stage 0 (a barrier
// follows its last reads), so stage 0 may be refilled at once; stage 1 is refilled only
// after the first barrier of the next call.
// threadIdx.x, opaque to the optimiser: values derived from it after this point are
// recomputed where they are used (a few VALU operations) instead of being hoisted out of
// a persistent kernel's tile loop and held, or spilled, across the epilogue.  A spill
// reload there costs far more than the arithmetic: its s_waitcnt vmcnt also waits for
// every direct-to-LDS load issued before it.
__device__ inline int tid_opaque() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <class E, bool kNatA = false, bool kNatB = false>
__device__ inline void gemm_main_op(const Op<kNatA>& A, const Op<kNatB>& B, const Offs& ao,
                                    const Offs& bo, int nk, Acc& acc, int rot = 0) {
  const int lane = tid_opaque() & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = w / kWN, wn = w % kWN;
  const int fr = lane & 15;
  const int fs = swz_f(fr);
  // natural-layout fragments: lane base (k-row 8 g + s / 4, byte 8 (s % 4)) and F of it
  const int g = lane >> 4;
  const int nlb = (8 * g + (fr >> 2)) * 512 + 8 * (fr & 3);
  const int F = nat_f(8 * g + (fr >> 2));
  const int fa = kNatA ? nlb + wm * 256 : (wm * 128 + fr) * 128;
  const int fb = kNatB ? nlb : (wn * kWaveN + fr) * 128;
  if constexpr (E::kBytes == 1) {
    static_assert(!kNatA && !kNatB, "fp8 operands are k-contiguous copies");
    for (int kt = 0; kt < nk; kt += 2) {
      wait_vmem();
      __syncthreads();  // stage 0 holds k-step kt; every wave is done reading stage 1
      const int k1 = kt + 1 + rot, k2 = kt + 2 + rot;
      stage_tiles<1>(A, B, ao, bo, k1 < nk ? k1 : k1 - nk, w);
      mma_stage_fp8<0>(acc, fa, fb, fs, lane);
      wait_vmem();
      __syncthreads();  // stage 1 holds k-step kt + 1; every wave is done reading stage 0
      if (kt + 2 < nk) stage_tiles<0>(A, B, ao, bo, k2 < nk ? k2 : k2 - nk, w);
      mma_stage_fp8<1>(acc, fa, fb, fs, lane);
    }
  } else {
    const FragBase q{fa, fb, (g ^ fs) << 4, ((4 + g) ^ fs) << 4, F, wn * 4};
    uint4 a[2], b[kNB];
    wait_vmem();
    __syncthreads();  // stage 0 holds k-step 0; every wave is done reading stage 1
    stage_tiles<1>(A, B, ao, bo, rot + 1 < nk ? rot + 1 : rot + 1 - nk, w);
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = frag_a<0, kNatA>(q, i, 0);
#pragma unroll
    for (int j = 0; j < kNB; ++j) b[j] = frag_b<0, kNatB>(q, j, 0);
    for (int kt = 0; kt < nk; kt += 2) {
      kstep_pipe<E, 0>(A, B, ao, bo, kt, nk, rot, w, q, acc, a, b);
      kstep_pipe<E, 1>(A, B, ao, bo, kt + 1, nk, rot, w, q, acc, a, b);
    }
  }
}
template <class E>
__device__ inline void gemm_main(Src ra, Src rb, const Offs& ao, const Offs& bo, int nk,
                                 Acc& acc, int rot = 0) {
  gemm_main_op<E, false, false>(Op<false>{ra}, Op<false>{rb}, ao, bo, nk, acc, rot);
}

template <class E, bool kNatA = false, bool kNatB = false>
__device__ inline void gemm_core_op(const Op<kNatA>& A, const Op<kNatB>& B, const Offs& ao,
                                    const Offs& bo, int nk, Acc& acc) {
  gemm_pre_op(A, B, ao, bo);
  gemm_main_op<E>(A, B, ao, bo, nk, acc);
}
template <class E>
__device__ inline void gemm_core(Src ra, Src rb, const Offs& ao, const Offs& bo, int nk,
                                 Acc& acc) {
  gemm_core_op<E>(Op<false>{ra}, Op<false>{rb}, ao, bo, nk, acc);
}

// ------------------------------------------------------------------------------ forward
// First k-step of a tile of rows tok0 .. tok0 + 255 (the k loop wraps around).  With all
// workgroups starting at k-step 0, the concurrent loads of a k-step fall at one offset of
// rows rowb bytes apart, and where rowb is a multiple of 4 KB that offset is a hot spot.
// The forward that keeps softmax terms (an XCD holds 2 token blocks x 16 vocabulary
// phases of a chunk) starts each token block one k-step further on (2.4% of that kernel
// measured, on any row size); the forwards over all rows (8 token blocks x 4 phases per
// XCD) start every second token block half of K further on when rowb is a multiple of
// 4 KB (1.5-5% measured; one k-step apart gained nothing, and with 10 KB rows half of K
// lost 1.5%).  A function of the row block alone, so each logit's k-steps are summed in
// the same order whichever workgroup computes it.
__device__ inline int tile_rot(int64_t tok0, int nk, bool keep_terms, int64_t rowb) {
  if (keep_terms) return (int)((uint32_t)(int)(tok0 >> 8) % (uint32_t)nk);
  if (rowb % 4096 == 0) return (int)((tok0 >> 8) & 1) * (nk >> 1);
  return 0;
}

struct FwdArgs {
  int64_t N, H, V;
  const int32_t* ntok;
  const int32_t* idx;
  const char* Xq;
  const char* Xp;
  const char* W;
  const int64_t* targets;
  // Partials of this launch (PartLayout over its rows, row index r - row_lo): the running
  // maximum (log2 units), sum of exp2 and target logit per side, phase and row.
  float* part;
  // Mode 3: the reference side's partials written by the mode-1 launch over all loss rows.
  const float* ref_part;
  float scale2; // log2(e) / temperature
  // This launch covers the loss rows [row_lo, min(row_hi, ntok)) of sides side0 ..
  // side0 + nsides - 1 (side 0: policy X_q, side 1: reference X_p).
  int64_t row_lo, row_hi;
  int side0, nsides;
  // Single-pass modes (policy rows of one chunk): every softmax term is also stored, in
  // the storage type, at pt[(r - row_lo) Vpad + v] (0 for v >= V and for rows past the
  // last loss row).  Mode 2: the term is exp2(z s2 - m_vt) with m_vt the running maximum
  // of row r after vocabulary tile vt, identical for all lanes of the row, stored at
  // pm[(r - row_lo) nvt + vt]; the backward's logit gradient is then
  // onehot - pt * exp2(m_vt - lse2) without recomputing the logits.  Mode 3: the term is
  // exp2(z s2 - mr) with mr the row's reference-side log-sum-exp, stored at pm[r - row_lo].
  char* pt;
  float* pm;
  int64_t pt_ld;  // entries per pt row (the chunk buffer's width: a piece, or Vpad)
  // Vocabulary piece `piece` of `npieces`, each of ptiles tiles: the launch sweeps tiles
  // [piece ptiles, min((piece + 1) ptiles, nvt)) with P = fwd_phases(blocks, ptiles)
  // phases, writes its partials at slots piece P + phase of split_layout (one side) or
  // part_layout (npieces 1), and its terms at pt column v - piece ptiles 256.
  int piece, npieces;
  int64_t ptiles;
  // Mode 3: store 0 at each row's target entry (the vocabulary split leaves the target
  // to the final dX kernel), and take the fixed reference from saved[idx[r] * 4] (the row's
  // own policy log-sum-exp: the split's fallback) instead of ref_part.
  int zero_target, ref_from_saved;
  const float* saved;
  // Launch only when *gate != 0 (null: always); the single-pass fallback of a chunk.
  const int32_t* gate;
  // fp8 logits: per-row e4m3 copies of W [V][H] and of the loss rows of X_q and X_p
  // [compact row][H], with their fp32 scales; the logit is scale_w * scale_x * (W8 . X8)
  const char* W8;
  const char* Xq8;
  const char* Xp8;
  const float* sw;
  const float* sxq;
  const float* sxp;
};

// Rows and token blocks of one launch.
struct FwdRange {
  int64_t rhi;  // one past the last row
  int ntbs;     // token blocks per side
  int TB;       // token blocks in all
};
__device__ inline FwdRange fwd_range(const FwdArgs& a, int ntok) {
  FwdRange f;
  f.rhi = a.row_hi < ntok ? a.row_hi : ntok;
  const int64_t nrows = f.rhi > a.row_lo ? f.rhi - a.row_lo : 0;
  f.ntbs = (int)((nrows + 255) / 256);
  f.TB = a.nsides * f.ntbs;
  return f;
}

// Staging offsets of vocabulary tile v0 < V (rows from V on clamped to V - 1), in 32-bit
// row arithmetic on a lane index recomputed here: 64-bit rows derived from threadIdx.x
// are hoisted out of a persistent tile loop and spilled, and each reload then waits for
// every vector memory operation in flight.
__device__ inline void w_offsets(int64_t v0, int64_t V, int64_t rowb, Offs& ao) {
  const int64_t left = V - 1 - v0;
  const int lim = left < 255 ? (int)left : 255;
  const int t = tid_opaque();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sr = 32 * (t >> 6) + 8 * i + ((t & 63) >> 3);
    const int d = sr < lim ? sr : lim;
    ao[i] = (uint32_t)d * (uint32_t)rowb + (uint32_t)(((t & 7) ^ swz_f(sr)) << 4);
  }
}

// Staging offsets of the loss rows tok0 .. tok0 + 255 (rows from rhi on clamped to the
// last valid one).
__device__ inline void x_offsets(int64_t tok0, int64_t rhi, const int32_t* __restrict__ idx,
                                 int64_t rowb, Offs& bo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sr = stage_row(i);
    int r = (int)tok0 + sr;  // 32-bit rows and byte offsets: the operand is below 4 GiB
    if (r >= rhi) r = (int)rhi - 1;
    bo[i] = (uint32_t)idx[r] * (uint32_t)rowb + stage_chunk_bytes(sr);
  }
}

// Staging offsets of compact rows tok0 .. tok0 + 255 of a buffer holding one row per loss
// row (the fp8 copies), rows from rhi on clamped to the last valid one.
__device__ inline void xc_offsets(int64_t tok0, int64_t rhi, int64_t rowb, Offs& bo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sr = stage_row(i);
    int r = (int)tok0 + sr;
    if (r >= rhi) r = (int)rhi - 1;
    bo[i] = (uint32_t)r * (uint32_t)rowb + stage_chunk_bytes(sr);
  }
}

// fp8 logits: acc[mb][nb][j] (vocabulary row vb + 16 mb + j, compact token row
// tok0 + column) times the two rows' scales.  Rows past V or rhi take a valid row's scale;
// their values are masked later.
__device__ inline void scale_acc(Acc& acc, const float* __restrict__ sw,
                                 const float* __restrict__ sx, int vb, int64_t V, int64_t tok0,
                                 int64_t rhi, int wn, int lane) {
  float cs[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    int64_t r = tok0 + wn * kWaveN + nb * 16 + (lane & 15);
    if (r >= rhi) r = rhi - 1;
    cs[nb] = sx[r];
  }
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t v = vb + mb * 16 + j;
      if (v >= V) v = V - 1;
      const float rs = sw[v];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb][j] *= rs * cs[nb];
    }
}

// Where a fold stores the softmax terms of its tile (single-pass mode).  The stores are
// buffer stores addressed by one 32-bit per-lane offset plus a wave-uniform offset, so no
// per-column 64-bit addresses are held across the GEMM loop.
struct FoldOut {
  Src pt;            // this block's 256 pt rows (Vpad elements each)
  Src pm;            // this block's 256 pm rows (nvt floats each)
  uint32_t lane_t;   // byte offset in pt of column wn*64 + lane%16, vocabulary wm*128 + 4(lane/16)
  uint32_t lane_m;   // byte offset in pm of column wn*64 + lane%16
  uint32_t col16_t;  // bytes of 16 pt rows
  uint32_t col16_m;  // bytes of 16 pm rows
  uint32_t v0_t;     // byte offset of the tile's first vocabulary entry in a pt row
  uint32_t vt_m;     // byte offset of the tile's entry in a pm row
  int nvalid;        // token columns of this block that are loss rows
};

// Kept terms of two vocabulary blocks (mb, mb + 1) of one token column, packed (4 terms
// per lane and block: p for mb, q for mb + 1), written with one 16-byte store per lane
// instead of two 8-byte ones.  A lane of an even 16-lane row (lane group g = 0, 2) holds
// entries 4g .. 4g + 3 of each block and its partner lane ^ 16 in the odd row the next
// four: the even lane trades its q for the odd lane's p (ds_swizzle, xor 16), so the even
// lane stores entries 4g .. 4g + 7 of block mb and the odd lane entries 4(g - 1) .. 4g + 3
// of block mb + 1, 24 bytes past its own 8-byte slot (term_lane_off).  Same bytes, same
// addresses, half the store instructions.  Every lane of the wave must be active.
__device__ inline uint32_t term_lane_off(int lane) { return ((lane >> 4) & 1) ? 24u : 0u; }
__device__ inline uint32_t from_lane_xor16(uint32_t v) {
  // ds_swizzle bit mode: and mask 0x1f, or mask 0, xor mask 0x10
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
__device__ inline void store_term_pair(u32x2 p, u32x2 q, bool odd, Src pt, uint32_t lane_off,
                                       uint32_t off) {
  const uint32_t r0 = from_lane_xor16(odd ? p[0] : q[0]);
  const uint32_t r1 = from_lane_xor16(odd ? p[1] : q[1]);
  const u32x4 v = odd ? u32x4{r0, r1, q[0], q[1]} : u32x4{p[0], p[1], r0, r1};
  __builtin_amdgcn_raw_buffer_store_b128(v, pt, lane_off, off, 0);
  // A vector store of more than 8 bytes still reads its data registers after it issues:
  // a VALU write of them in the next instruction slot changed what some lanes stored
  // (the terms of the next block's fma), and the compiler puts no gap there by itself.
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

// Fold one 256 x 256 logit tile into this lane's running (max, sum of exp2) per token
// column, kept in LDS, and catch the target logit.  kFull: every vocabulary row of the
// tile is below V, so no row masks are evaluated.  kStore: single-pass mode; the running
// maximum is first made common to the eight lanes (four lane groups, two m-waves) that
// hold a token column, so the stored terms of a row share one reference per tile.
template <class E, bool kFull, bool kStore>
__device__ inline void fwd_fold(const Acc& acc, float s2, int vlim, int vb, int wm, int wn,
                                int lane, int tid, float (*s_run)[kNB][kThreads],
                                const int* s_y, float* s_zt, float (*s_cm)[256],
                                const FoldOut& fo) {
  float cmax[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    float t = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (kFull || mb * 16 + j < vlim) t = fmaxf(t, acc[mb][nb][j]);
    cmax[nb] = t;
  }
  if (kStore) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      float t = fmaxf(cmax[nb], __shfl_xor(cmax[nb], 16));
      t = fmaxf(t, __shfl_xor(t, 32));
      cmax[nb] = t;
      if (lane < 16) s_cm[wm][wn * kWaveN + nb * 16 + lane] = t;
    }
    lds_barrier();
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int n = wn * kWaveN + nb * 16 + (lane & 15);
      cmax[nb] = fmaxf(s_cm[0][n], s_cm[1][n]);
    }
  }
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int n = wn * kWaveN + nb * 16 + (lane & 15);
    const float rm = s_run[0][nb][tid];
    const float nm = fmaxf(rm, cmax[nb] * s2);
    float sum = rm == -INFINITY ? 0.f : s_run[1][nb][tid] * exp2_fast(rm - nm);
    if (kStore) {
      const bool ok = n < fo.nvalid;
      // a column past the last loss row takes +inf as its reference, so its terms are
      // stored as 0 (its sum is never read)
      const float ns = ok ? nm : INFINITY;
      const uint32_t so = (uint32_t)nb * fo.col16_t + fo.v0_t;
      const bool odd = (lane >> 4) & 1;
      const uint32_t lt = fo.lane_t + term_lane_off(lane);
#pragma unroll
      for (int mb = 0; mb < kMB; mb += 2) {
        u32x2 pk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            e[j] = (kFull || (mb + h) * 16 + j < vlim)
                       ? exp2_fast(fmaf(acc[mb + h][nb][j], s2, -ns)) : 0.f;
            sum += e[j];
          }
          pk[h] = u32x2{E::pack2(e[0], e[1]), E::pack2(e[2], e[3])};
        }
        store_term_pair(pk[0], pk[1], odd, fo.pt, lt, so + mb * 32);
      }
      if (wm == 0 && lane < 16 && ok)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nm), fo.pm, fo.lane_m,
                                              nb * fo.col16_m + fo.vt_m, 0);
    } else {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kFull || mb * 16 + j < vlim) sum += exp2_fast(fmaf(acc[mb][nb][j], s2, -nm));
    }
    s_run[0][nb][tid] = nm;
    s_run[1][nb][tid] = sum;
    const int loc = s_y[n] - vb;
    if ((unsigned)loc < 128u && (loc & 12) == 0) {  // this lane holds the target logit
      float z = 0.f;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) z = (loc == mb * 16 + j) ? acc[mb][nb][j] : z;
      s_zt[n] = z;
    }
  }
}

// Fixed-reference fold (single-pass mode 3): the terms of token column n are
// exp2(z s2 - mr_n), mr_n the reference side's log-sum-exp of the row (log2 units), so no
// running maximum is kept and the tiles of a row need no common reference.  The terms are
// summed per lane and stored; mr_n = +inf (past the last loss row) stores zeros.
template <class E, bool kFull>
__device__ inline void fwd_fold_fixed(const Acc& acc, float s2, int vlim, int vb, int wn,
                                      int lane, int tid, float (*s_run)[kNB][kThreads],
                                      const int* s_y, float* s_zt, const float* s_mr,
                                      const FoldOut& fo, int zero_target) {
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int n = wn * kWaveN + nb * 16 + (lane & 15);
    const float mr = s_mr[n];
    float sum = s_run[1][nb][tid];
    const uint32_t so = (uint32_t)nb * fo.col16_t + fo.v0_t;
    const bool odd = (lane >> 4) & 1;
    const uint32_t lt = fo.lane_t + term_lane_off(lane);
#pragma unroll
    for (int mb = 0; mb < kMB; mb += 2) {
      u32x2 pk[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          e[j] = (kFull || (mb + h) * 16 + j < vlim)
                     ? exp2_fast(fmaf(acc[mb + h][nb][j], s2, -mr)) : 0.f;
          sum += e[j];
        }
        pk[h] = u32x2{E::pack2(e[0], e[1]), E::pack2(e[2], e[3])};
      }
      store_term_pair(pk[0], pk[1], odd, fo.pt, lt, so + mb * 32);
    }
    s_run[1][nb][tid] = sum;
    const int loc = s_y[n] - vb;
    if (zero_target) {
      // The kept term of the target is replaced by 0 (its term is still in the row's sum)
      // by the lane whose 16-byte store above wrote it, at the same address and after
      // it, so it lands last.  That store's 8 entries start at vocabulary vb + 16 mb (even
      // lane group) or vb + 16 mb + 12 (odd), mb = 0, 2, 4, 6.
      const int d = loc - (odd ? 12 : 0);
      if ((unsigned)d < 128u && (d & 31) < 8)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, fo.pt,
                                              lt + (d >> 5) * 64 + (d & 31) * 2, so, 0);
    }
    if ((unsigned)loc < 128u && (loc & 12) == 0) {  // this lane holds the target logit
      float z = 0.f;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) z = (loc == mb * 16 + j) ? acc[mb][nb][j] : z;
      s_zt[n] = z;
    }
  }
}

// Persistent.  Workgroup w runs on XCD w % 8; its slot s = w / 8 picks a token block of
// the current round and a vocabulary phase: the 32 workgroups of one XCD cover 32 / P
// token blocks x P phases (P = fwd_phases(...), 4 for the long-context shape), so each W
// tile in flight on an XCD is shared by 32 / P workgroups and each X block by P, and all
// XCDs sweep the same W tiles together.  With few token blocks (a short last chunk) P
// can exceed 32: the phases of one token block then span P / 32 XCDs, and the round
// holds 256 / P token blocks.  A workgroup keeps its token block for a whole
// round and walks the vocabulary tiles of its phase (vt = phase, phase + P, ...), folding
// each 256 x 256 logit tile into per-lane running (max, sum of exp2, target logit)
// without storing it (or, in single-pass mode, storing its softmax terms).  The loads of
// each next tile are issued before the previous tile is folded, so the fold overlaps the
// first k-step's memory latency.
// kMode 0: both sides over all rows (two-pass forward); 1: one side over all rows
// (single-pass reference); 2: policy rows of one chunk, softmax terms kept relative to a
// running maximum (single-pass); 3: as 2 with the reference side's log-sum-exp of each
// row as the fixed reference of its terms, which mode 1 must have produced: the first
// piece's launch merges its partials per row at the start of each token block, and its
// workgroups of phase 0 store the result at pm[r - row_lo], which the later pieces read
// back (the merge costs the reference launch's phase count in loads per row and
// workgroup).  The partials of mode 3 carry that reference as their
// maximum.  Modes 0 and 1 run the same code; distinct instances keep their profiles apart.
template <class E, class G, int kMode>
__global__ void __launch_bounds__(kThreads, 1) fwd_kernel(FwdArgs a) {
  constexpr bool kFixed = kMode == 3;
  constexpr bool kStore = kMode == 2 || kFixed;
  constexpr bool kF8 = G::kBytes == 1;   // operands are the fp8 copies
  __shared__ float mrg[2][2][256];
  __shared__ float s_run[2][kNB][kThreads];
  __shared__ int s_y[256];
  __shared__ float s_zt[256];
  __shared__ float s_cm[kMode == 2 ? 2 : 1][256];
  __shared__ float s_mr[kFixed ? 256 : 1];
  if (a.gate && *a.gate == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / kWN, wn = w % kWN;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;           // workgroups per XCD
  const int ntok = *a.ntok;
  const FwdRange fr = fwd_range(a, ntok);
  const int TB = fr.TB;
  const int64_t nvt_all = (a.V + 255) / 256;
  const int64_t vt_lo = a.piece * a.ptiles;                      // this launch's tiles
  const int64_t nvt = vt_lo + a.ptiles < nvt_all ? vt_lo + a.ptiles : nvt_all;  // end
  const int P = fwd_phases(TB, a.ptiles);
  PartLayout pl;  // part_layout(rows, nsides, nvt) for one piece, else split_layout
  pl.P = a.npieces * P;
  pl.nsides = a.nsides;
  pl.stride = (int64_t)fr.ntbs * 256;
  // P <= 32: each XCD holds 32 / P token blocks x P phases; P > 32 (fewer token blocks
  // than XCDs x 32 / P... in the rounds): a token block's phases span P / 32 XCDs
  const int xpb = P > slots ? P / slots : 1;     // XCDs per token block
  const int tb_per_xcd = P > slots ? 0 : slots / P;
  const int phase = P > slots ? (xcd % xpb) * slots + slot : slot % P;
  const int tbg = P > slots ? kXcds / xpb : kXcds * tb_per_xcd;  // token blocks per round
  const int64_t rowb = a.H * G::kBytes;          // bytes per row
  const int nk = (int)(rowb / 128);              // k-steps of 128 bytes
  const float s2 = a.scale2;
  const char* Wop = kF8 ? a.W8 : a.W;
  const char* wend = Wop + a.V * rowb;           // operand extents for the buffer loads
  const int64_t xbytes = a.N * rowb;
  auto xop = [&](int side) { return kF8 ? (side ? a.Xp8 : a.Xq8) : (side ? a.Xp : a.Xq); };
  auto xoffs = [&](int64_t tok0, Offs& bo) {
    if (kF8)
      xc_offsets(tok0, fr.rhi, rowb, bo);
    else
      x_offsets(tok0, fr.rhi, a.idx, rowb, bo);
  };

  const int slot_ph = a.piece * P + phase;      // this phase's partial slot
  int tb = P > slots ? xcd / xpb : xcd * tb_per_xcd + slot / P;
  if (tb >= TB) return;
  // loads of the first tile.  A phase with no vocabulary tile (the piece has fewer than P
  // tiles) still writes its empty partials (max -inf, sum 0) for every token block.
  Offs ao, bo;
  if (vt_lo + phase < nvt) {
    const int sd = (int)(tb / fr.ntbs);
    xoffs(a.row_lo + (tb - sd * fr.ntbs) * 256, bo);
    const int64_t f0 = (vt_lo + phase) * 256;
    w_offsets(f0, a.V, rowb, ao);
    const char* X0 = xop(a.side0 + sd);
    gemm_pre(make_src(Wop + f0 * rowb, wend), make_src(X0, X0 + xbytes), ao, bo,
             tile_rot(a.row_lo + (tb - sd * fr.ntbs) * 256, nk, kStore, rowb));
  }
  for (; tb < TB; tb += tbg) {
    const int sd = (int)(tb / fr.ntbs);
    const int side = a.side0 + sd;
    const int64_t tok0 = a.row_lo + (tb - sd * fr.ntbs) * 256;
    const char* X = xop(side);
    // per-block state lives in LDS so the GEMM loop keeps its registers: target id and
    // target logit per token column, running (max, sum) per lane and column block
    if (tid < 256) {
      const int r = (int)tok0 + tid;  // row indices fit int32 (checked at the boundary)
      int yy = -1;
      if (r < fr.rhi) {
        const int64_t t = a.targets[a.idx[r]];
        yy = (t >= 0 && t < a.V) ? (int)t : -1;
      }
      s_y[tid] = yy;
      s_zt[tid] = 0.f;
      if (kFixed) {
        // the reference side's log-sum-exp of row r from the partials of the mode-1 launch
        float mr = INFINITY;
        if (r < fr.rhi) {
          if (a.ref_from_saved) {
            mr = a.saved[(int64_t)a.idx[r] * 4] * kLog2e;
          } else if (a.piece > 0) {
            // the chunk's first piece stored it (below); nothing writes pm between the
            // pieces' forward launches
            mr = a.pm[r - a.row_lo];
          } else {
            const PartLayout rl = part_layout(ntok, 1, nvt_all);
            float M = -INFINITY;
            for (int ph = 0; ph < rl.P; ++ph) M = fmaxf(M, a.ref_part[rl.at(0, 0, ph, r)]);
            float sm = 0.f;
            for (int ph = 0; ph < rl.P; ++ph) {
              const float sp = a.ref_part[rl.at(1, 0, ph, r)];
              if (sp != 0.f) sm += sp * exp2f(a.ref_part[rl.at(0, 0, ph, r)] - M);
            }
            mr = M + log2f(sm);
          }
          if (phase == 0 && (a.piece == 0 || a.ref_from_saved)) a.pm[r - a.row_lo] = mr;
        }
        s_mr[tid] = mr;
      }
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      s_run[0][nb][tid] = -INFINITY;
      s_run[1][nb][tid] = 0.f;
    }
    // The block state written above is read by other waves: in the folds (after the k
    // loop's barriers) and in the final merge of the token block, which a phase with no
    // vocabulary tile reaches without any barrier in between.  LDS only, so the next
    // tile's loads in flight are not waited for.
    lds_barrier();
    FoldOut fo;
    if (kStore) {
      const int64_t rt = a.pt_ld * E::kBytes, rm = nvt_all * 4;  // bytes per pt, pm row
      const char* pt0 = a.pt + (tok0 - a.row_lo) * rt;
      const char* pm0 = reinterpret_cast<const char*>(a.pm + (tok0 - a.row_lo) * nvt);
      fo.pt = make_src(pt0, pt0 + 256 * rt);
      fo.pm = make_src(pm0, pm0 + 256 * rm);
      const int col = wn * kWaveN + (lane & 15);
      fo.lane_t = (uint32_t)(col * rt + (wm * 128 + 4 * (lane >> 4)) * E::kBytes);
      fo.lane_m = (uint32_t)(col * rm);
      fo.col16_t = (uint32_t)(16 * rt);
      fo.col16_m = (uint32_t)(16 * rm);
      fo.nvalid = (int)(fr.rhi - tok0 < 256 ? fr.rhi - tok0 : 256);
    }
    for (int64_t vt = vt_lo + phase; vt < nvt; vt += P) {
      const int64_t v0 = vt * 256;
      Acc acc;
      zero_acc(acc);
      gemm_main<G>(make_src(Wop + v0 * rowb, wend), make_src(X, X + xbytes), ao, bo, nk, acc,
                   tile_rot(tok0, nk, kStore, rowb));
      // enqueue the next tile: the next vocabulary tile of this block, else the first
      // tile of this workgroup's next token block
      {
        int64_t nv = vt + P;
        int ntb = tb;
        if (nv >= nvt) {
          nv = vt_lo + phase;
          ntb = tb + tbg;
        }
        if (ntb < TB) {
          const int nsd = (int)(ntb / fr.ntbs);
          const int64_t ntok0 = a.row_lo + (ntb - nsd * fr.ntbs) * 256;
          if (ntb != tb) xoffs(ntok0, bo);
          w_offsets(nv * 256, a.V, rowb, ao);
          const char* Xn = xop(a.side0 + nsd);
          gemm_pre(make_src(Wop + nv * 256 * rowb, wend), make_src(Xn, Xn + xbytes), ao, bo,
                   tile_rot(ntok0, nk, kStore, rowb));
        }
      }
      // vocab of acc[mb][.][j] = vb + 16 mb + j (the lane part recomputed here, not held
      // across the k loop)
      const int vb = (int)(v0 + wm * 128 + 4 * ((tid_opaque() & 63) >> 4));
      if (kF8) scale_acc(acc, a.sw, side ? a.sxp : a.sxq, vb, a.V, tok0, fr.rhi, wn, lane);
      FoldOut ft = fo;
      if (kStore) {
        ft.v0_t = (uint32_t)((v0 - vt_lo * 256) * E::kBytes);
        ft.vt_m = (uint32_t)(vt * 4);
      }
      if constexpr (kFixed) {
        if (v0 + 256 <= a.V)
          fwd_fold_fixed<E, true>(acc, s2, 0, vb, wn, lane, tid, s_run, s_y, s_zt, s_mr, ft,
                                  a.zero_target);
        else
          fwd_fold_fixed<E, false>(acc, s2, (int)(a.V - vb), vb, wn, lane, tid, s_run, s_y,
                                   s_zt, s_mr, ft, a.zero_target);
      } else {
        if (v0 + 256 <= a.V)
          fwd_fold<E, true, kStore>(acc, s2, 0, vb, wm, wn, lane, tid, s_run, s_y, s_zt, s_cm,
                                    ft);
        else
          fwd_fold<E, false, kStore>(acc, s2, (int)(a.V - vb), vb, wm, wn, lane, tid, s_run,
                                     s_y, s_zt, s_cm, ft);
      }
    }
    // merge the four lane groups holding each token column, then the two m-waves
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      float m = kFixed ? s_mr[wn * kWaveN + nb * 16 + (lane & 15)] : s_run[0][nb][tid];
      float sum = s_run[1][nb][tid];
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2x = __shfl_xor(sum, off);
        const float M = fmaxf(m, m2);
        sum = M == -INFINITY ? 0.f
                             : (m == -INFINITY ? 0.f : sum * exp2f(m - M)) +
                                   (m2 == -INFINITY ? 0.f : s2x * exp2f(m2 - M));
        m = M;
      }
      if (lane < 16) {
        const int n = wn * kWaveN + nb * 16 + lane;
        mrg[wm][0][n] = m;
        mrg[wm][1][n] = sum;
      }
    }
    __syncthreads();
    if (tid < 256) {  // one thread per token column of the block
      const int n = tid;
      const int r = (int)tok0 + n;
      if (r < fr.rhi) {
        const float m0 = mrg[0][0][n], m1 = mrg[1][0][n];
        const float M = fmaxf(m0, m1);
        const float sum = M == -INFINITY
                              ? 0.f
                              : (m0 == -INFINITY ? 0.f : mrg[0][1][n] * exp2f(m0 - M)) +
                                    (m1 == -INFINITY ? 0.f : mrg[1][1][n] * exp2f(m1 - M));
        a.part[pl.at(0, sd, slot_ph, r - a.row_lo)] = M;
        a.part[pl.at(1, sd, slot_ph, r - a.row_lo)] = sum;
        a.part[pl.at(2, sd, slot_ph, r - a.row_lo)] = s_zt[n];
      }
    }
    __syncthreads();
  }
}

template <class E>
__device__ inline void fixup_row(int64_t Vpad, int64_t nvt, int64_t row, int64_t v, int64_t t,
                                 const int64_t* __restrict__ targets,
                                 const float* __restrict__ saved, const float* __restrict__ pm,
                                 typename E::T* __restrict__ T) {
  const float lse2 = saved[t * 4] * kLog2e;
  const int64_t y = targets[t];
  const float f = exp2f(pm[row * nvt + v / 256] - lse2);
  // the target entry 1 - p_y = -expm1(q) from the row's log-probability, exact even
  // where p_y is close to 1 (its kept term carries the 16-bit rounding of p_y)
  const float ty = -expm1f(saved[t * 4 + 1]);
  uint4* p = reinterpret_cast<uint4*>(T + row * Vpad + v);
  uint4 q = *p;
  uint16_t h[8];
  __builtin_memcpy(h, &q, 16);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    h[j] = E::from_f32(v + j == y ? ty : -E::to_f32(h[j]) * f);
  __builtin_memcpy(&q, h, 16);
  *p = q;
}

// Single-pass mode 2, after the merge of a chunk: T = onehot(y) - pt * exp2(m_vt - lse2) in
// place, 8 elements (16 bytes) per thread and step, the target entry as -expm1(log p_y).
// Rows past the last loss row stay 0.  A fixed grid strides over the chunk (row = y block
// index + k gridDim.y), so a launch that *gate turns off (null: always on) costs little.
template <class E>
__global__ void __launch_bounds__(256)
fixup_kernel(int64_t Vpad, int64_t nvt, int64_t c0, int64_t R, const int32_t* __restrict__ ntok_p,
             const int32_t* __restrict__ idx, const int64_t* __restrict__ targets,
             const float* __restrict__ saved, const float* __restrict__ pm,
             typename E::T* __restrict__ T, const int32_t* __restrict__ gate) {
  if (gate && *gate == 0) return;
  const int64_t v = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (v >= Vpad) return;
  const int ntok = *ntok_p;
  for (int64_t row = blockIdx.y; c0 + row < ntok && row < R; row += gridDim.y)
    fixup_row<E>(Vpad, nvt, row, v, idx[c0 + row], targets, saved, pm, T);
}

// ---------------------------------------------------------------------------- recompute
// T[r - c0][v - vt0 256] = onehot(y_r)[v] - exp(z_rv / tau - lse_r) for one 256-token x
// 256-vocabulary tile of the chunk (scale2 = log2(e) / tau); zero for v >= V and for rows
// past the last loss token.  The grid covers the vocabulary tiles vt0 .. of one piece and
// T rows hold ld entries.  kept = 1 (the vocabulary split): the plain softmax terms
// exp(z_rv / tau - lse_r), with 0 at the target entry, which the final dX kernel adds
// back as 1 - p_y = -expm1(q).  G = FP8T: Xq and W are the fp8 copies (Xq by compact
// row) with scales sxq and sw.
template <class E, class G>
__global__ void __launch_bounds__(kThreads, 1)
recompute_kernel(int64_t N, int64_t H, int64_t V, int64_t ld, int64_t vt0, int64_t c0, int ntt,
                 float scale2, int kept, const int32_t* __restrict__ ntok_p,
                 const int32_t* __restrict__ idx, const char* __restrict__ Xq,
                 const char* __restrict__ W, const int64_t* __restrict__ targets,
                 const float* __restrict__ saved, typename E::T* __restrict__ T,
                 const float* __restrict__ sw, const float* __restrict__ sxq) {
  constexpr bool kF8 = G::kBytes == 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / kWN, wn = w % kWN;
  // token tiles vary fastest so consecutive workgroups share a W tile
  const int64_t tt = blockIdx.x % ntt, vt = vt0 + blockIdx.x / ntt;
  const int ntok = *ntok_p;
  const int64_t tok0 = c0 + tt * 256;
  if (tok0 >= ntok) return;
  const int64_t v0 = vt * 256;
  const int64_t rowb = H * G::kBytes;
  Offs ao, bo;
  w_offsets(v0, V, rowb, ao);
  if (kF8)
    xc_offsets(tok0, ntok, rowb, bo);
  else
    x_offsets(tok0, ntok, idx, rowb, bo);
  Acc acc;
  zero_acc(acc);
  gemm_core<G>(make_src(W + v0 * rowb, W + V * rowb), make_src(Xq, Xq + N * rowb), ao, bo,
               (int)(rowb / 128), acc);
  const int64_t vb = v0 + wm * 128 + 4 * (lane >> 4);
  if (kF8) scale_acc(acc, sw, sxq, (int)vb, V, tok0, ntok, wn, lane);
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int64_t r = tok0 + wn * kWaveN + nb * 16 + (lane & 15);
    const bool ok = r < ntok;
    float lse2 = 0.f;
    int64_t y = -1;
    if (ok) {
      const int64_t t = idx[r];
      lse2 = saved[t * 4] * kLog2e;
      y = targets[t];
    }
    typename E::T* trow = T + (r - c0) * ld - vt0 * 256;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int64_t v = vb + mb * 16;
      uint16_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float val = 0.f;
        if (ok && v + j < V) {
          const float pv = exp2_fast(fmaf(acc[mb][nb][j], scale2, -lse2));
          val = kept ? (v + j == y ? 0.f : pv) : (v + j == y ? 1.f : 0.f) - pv;
        }
        o[j] = E::from_f32(val);
      }
      uint2 pk;
      pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
      pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
      *reinterpret_cast<uint2*>(trow + v) = pk;
    }
  }
}

// Row factor of a mode-3 chunk (see dx_kernel): -f_r, f_r = exp2(mr_r - lse2_r).
__device__ inline float fixed_row_factor(int64_t rl, int64_t t, const float* __restrict__ saved,
                                         const float* __restrict__ mr) {
  return -exp2f(mr[rl] - saved[t * 4] * kLog2e);
}

// Float offset of accumulator block (mb, nb) of lane `lane` of wave w in tile `tile` of the
// vocabulary split's dX sums: each tile takes 65536 floats, wave-major, then block
// q = nb 8 + mb (1 KB), then lane (16 bytes).
__host__ __device__ inline int64_t dx_sum_offset(int64_t tile, int w, int nb, int mb, int lane) {
  return tile * 65536 + w * 8192 + (nb * 8 + mb) * 256 + lane * 4;
}

// dX with its reduction split ksplit ways over the vocabulary: a launch's n_items (output
// tile, split) parts go out as runs when they divide evenly over its nwg workgroups, q =
// n_items / nwg >= 2 each: workgroup L takes parts L q .. L q + q - 1 of the tile-major
// order (part = tile ksplit + ks, tile = token tile nht + H tile), the consecutive parts of
// one tile as one k loop whose sum goes to the slot of the run's first part.  Slot ks of a
// tile then holds a partial only where a run starts: ks == 0 or part % q == 0.  Otherwise
// (a ragged last chunk, no split) every item is one part and every slot holds one.
__host__ __device__ inline bool dx_runs(int64_t n_items, int ksplit, int nwg) {
  return ksplit > 1 && n_items > nwg && n_items % nwg == 0;
}
__host__ __device__ inline bool dx_slot_used(bool runs, int64_t tile, int ks, int ksplit,
                                             int64_t q) {
  return !runs || ks == 0 || (tile * ksplit + ks) % q == 0;
}

// ------------------------------------------------------------------------------- dX
// C[h][r] = sum_v W[v][h] T[r][v] over the chunk buffer's vocabulary columns (the padded
// vocabulary, or one piece of it: columns 0 .. kcols - 1 of rows of ld entries hold
// vocabulary rows v_base ..), or one split of them, with W read in its own [V][H] layout
// (natural-layout A tiles; rows past V load as 0).
// acc_mode 0, ksplit == 1: dX[idx[r]][h] = c * g_r * s_r * C, in the storage type (row
// r - srow0 instead of idx[r] when srow0 >= 0: a staging slot of the gradient offload).
// acc_mode 0, ksplit > 1: fp32 partials of C to dxp[ks][r - c0][h], reduced by
// dx_reduce_kernel, which scales the same.  acc_mode 1: fp32 partials for every ksplit
// (the first piece of a vocabulary-split chunk); acc_mode 2: added to them (the later
// pieces: the k loop starts from the stored sums), scaled by dx_final_kernel.  acc_mode 3
// (ksplit == 1, the last piece once the chunk's merge has run): starts from the sums like
// 2 (from 0 when it is also the first piece) and writes dX itself with dx_final_kernel's arithmetic (targets; mr the per-row
// reference, pm there), or nothing when the chunk's flag (redo) sends it to the fallback.
// s_r = 1 where the chunk buffer holds T = onehot - softmax (two-pass, single-pass mode 2,
// or a mode-3 chunk whose fallback ran: redo null or *redo != 0).  Otherwise it holds the
// mode-3 row E = -T / f_r: the kept terms e_v = p_v / f_r, f_r = exp2(mr_r - lse2_r) (mr:
// the reference log-sum-exp the terms were taken against), with the target entry
// replaced by expm1(q_r) / f_r in the merge; then s_r = -f_r.
//
// Persistent over a work list of (k split, token tile, H tile) items, H tile fastest,
// holding only the token tiles of this chunk that have loss rows, so every workgroup gets
// the same number of items up to one; with the reduction split and items that divide
// evenly over the workgroups, as runs of one tile's consecutive parts instead (dx_runs),
// so that a workgroup stores about 2 partials rather than one per part.  Workgroups are numbered XCD-major (workgroup b
// runs on XCD b % 8), so the items that share a T tile and k range run on one XCD.  Each
// item's first k-step is enqueued before the previous item's epilogue, so its memory
// latency overlaps the epilogue's instead of following it.
template <class E>
__global__ void __launch_bounds__(kThreads, 1)
dx_kernel(int64_t H, int64_t V, int64_t ld, int64_t kcols, int64_t v_base, int64_t R,
          int64_t c0, int nht, int ksplit, int acc_mode, const int32_t* __restrict__ ntok_p,
          const int32_t* __restrict__ idx, const char* __restrict__ W,
          const char* __restrict__ T, const float* __restrict__ saved,
          const float* __restrict__ grad_loss, float loss_scale,
          typename E::T* __restrict__ dX, int64_t srow0, float* __restrict__ dxp,
          int32_t* __restrict__ found_inf, const int32_t* __restrict__ redo,
          const float* __restrict__ mr, const int32_t* __restrict__ gate,
          const int64_t* __restrict__ targets) {
  if (gate && *gate == 0) return;   // the vocabulary split's fallback
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / kWN, wn = w % kWN;
  const int ntok = *ntok_p;
  int64_t rows = (int64_t)ntok - c0;
  if (rows <= 0) return;
  if (rows > R) rows = R;
  const int64_t ntt = (rows + 255) / 256;
  const int64_t n_items = ntt * nht * ksplit;
  const int nwg = gridDim.x;                       // a multiple of 8
  const int64_t first = (int64_t)(blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
  // k-steps of 64 over the kcols columns written for this launch (a multiple of 256; the
  // last piece of a split chunk leaves the buffer's later columns as the previous piece
  // wrote them), split into ksplit ranges with even boundaries
  const int64_t npair = kcols / 128;
  const int64_t rowb = ld * 2;    // bytes per T row
  const int64_t ldw = H * 2;      // bytes per W row
  Offs ao, bo;
  nat_offsets(ldw, ao);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sr = stage_row(i);
    bo[i] = (uint32_t)(sr * rowb) + stage_chunk_bytes(sr);
  }
  const float c = (grad_loss ? *grad_loss : 1.f) / loss_scale;
  const bool fixed = redo && *redo == 0;
  const bool final_dx = acc_mode == 3;
  const bool skip = final_dx && redo && *redo != 0;   // the fallback writes this chunk
  const bool to_slots = acc_mode == 1 || acc_mode == 2 || (acc_mode == 0 && ksplit > 1);
  bool bad = false;
  // item -> (token tile, H tile, k range) and its two operands
  struct Item {
    int64_t tt, ks, h0, kbeg, kend;
  };
  auto decode = [&](int64_t item) {
    Item d;
    const int64_t rest = item / nht;
    d.h0 = (item % nht) * 256;
    d.tt = rest % ntt;
    d.ks = rest / ntt;
    d.kbeg = 2 * (npair * d.ks / ksplit);
    d.kend = 2 * (npair * (d.ks + 1) / ksplit);
    return d;
  };
  auto opA = [&](const Item& d) {
    const int64_t v = v_base + d.kbeg * 64;
    return Op<true>{W + v * ldw + d.h0 * 2, (V - v) * ldw - d.h0 * 2, 64 * ldw};
  };
  auto opB = [&](const Item& d) {
    return Op<false>{make_src(T + d.tt * 256 * rowb + d.kbeg * 128, T + R * rowb)};
  };
  // The fp32 sums of an item's tile.  ksplit > 1 with acc_mode 0: row-major partials
  // dxp[ks][r - c0][h] for dx_reduce_kernel.  acc_mode 1 and 2: the tile's own 256 KB in
  // the accumulator layout (dx_sum_offset), so that each of the 32 stores (and, for the
  // later pieces, loads) of a wave covers 1 KB of consecutive bytes.
  auto slot_ptr = [&](const Item& d, int nb, int mb) {
    const int lq = tid_opaque() & 63;
    if (acc_mode != 0)
      return reinterpret_cast<f32x4*>(
          dxp + dx_sum_offset((d.ks * (R / 256) + d.tt) * nht + d.h0 / 256, w, nb, mb, lq));
    const int rl = (int)d.tt * 256 + wn * kWaveN + nb * 16 + (lq & 15);
    const int hb = (int)d.h0 + wm * 128 + 4 * (lq >> 4);
    return reinterpret_cast<f32x4*>(dxp + (d.ks * R + rl) * H + hb + mb * 16);
  };
  // the sums of the pieces before this one (acc_mode 3 on the first piece: none)
  const bool from_sums = acc_mode == 2 || (acc_mode == 3 && v_base > 0);
  auto init_acc = [&](Acc& acc, const Item& d) {
    if (!from_sums) {
      zero_acc(acc);
      return;
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = *slot_ptr(d, nb, mb);
  };
  // this workgroup's work units: items first, first + nwg, .. or, with runs (dx_runs), the
  // runs of one tile's consecutive parts within parts first q .. first q + q - 1
  const bool runs = dx_runs(n_items, ksplit, nwg);
  const int64_t q = n_items / nwg;
  auto unit = [&](int64_t u, Item& d) -> bool {
    if (!runs) {
      const int64_t item = first + u * nwg;
      if (item >= n_items) return false;
      d = decode(item);
      return true;
    }
    int64_t part = first * q;
    const int64_t pend = part + q;
    for (int64_t i = 0; part < pend; ++i) {
      const int64_t tile = part / ksplit, ks0 = part % ksplit;
      const int64_t len = ksplit - ks0 < pend - part ? ksplit - ks0 : pend - part;
      if (i == u) {
        d.tt = tile / nht;
        d.h0 = (tile % nht) * 256;
        d.ks = ks0;
        d.kbeg = 2 * (npair * ks0 / ksplit);
        d.kend = 2 * (npair * (ks0 + len) / ksplit);
        return true;
      }
      part += len;
    }
    return false;
  };
  Acc acc;
  Item d;
  bool have = unit(0, d);
  if (have) {
    if (d.kend > d.kbeg) gemm_pre_op(opA(d), opB(d), ao, bo);
    init_acc(acc, d);
  }
  for (int64_t u = 0; have; ++u) {
    const int64_t tok0 = c0 + d.tt * 256;
    if (d.kend > d.kbeg)
      gemm_main_op<E, true, false>(opA(d), opB(d), ao, bo, (int)(d.kend - d.kbeg), acc);
    Item dn;
    const bool more = unit(u + 1, dn);
    if (more && dn.kend > dn.kbeg) gemm_pre_op(opA(dn), opB(dn), ao, bo);
    if (final_dx) {
      if (!skip) {
        // dX = c g_r ((1 - p_y) W[y_r] - f_r C), as dx_final_kernel
        const int lq = tid_opaque() & 63;
        const int hb = (int)d.h0 + wm * 128 + 4 * (lq >> 4);
        const typename E::T* Wt = reinterpret_cast<const typename E::T*>(W);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int r = (int)tok0 + wn * kWaveN + nb * 16 + (lq & 15);
          if (r >= ntok) continue;
          const int64_t t = idx[r];
          const int64_t y = targets[t];
          const float lse2 = saved[t * 4] * kLog2e;
          const float gs = saved[t * 4 + 3] * c;
          const float f = mr ? exp2f(mr[r - c0] - lse2) : 1.f;
          const bool yok = y >= 0 && y < V;
          const float ty = yok ? -expm1f(saved[t * 4 + 1]) : 0.f;
          const typename E::T* wy = Wt + (yok ? y : 0) * H + hb;
          typename E::T* drow = dX + (srow0 < 0 ? t : r - srow0) * H + hb;
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            const f32x4 sm = acc[mb][nb];
            const uint2 wv = *reinterpret_cast<const uint2*>(wy + mb * 16);
            const float w0 = E::to_f32((typename E::T)(wv.x & 0xffffu));
            const float w1 = E::to_f32((typename E::T)(wv.x >> 16));
            const float w2 = E::to_f32((typename E::T)(wv.y & 0xffffu));
            const float w3 = E::to_f32((typename E::T)(wv.y >> 16));
            uint2 pk;
            pk.x = E::pack2(gs * (ty * w0 - f * sm[0]), gs * (ty * w1 - f * sm[1]));
            pk.y = E::pack2(gs * (ty * w2 - f * sm[2]), gs * (ty * w3 - f * sm[3]));
            bad |= E::nonfinite2(pk.x) || E::nonfinite2(pk.y);
            *reinterpret_cast<uint2*>(drow + mb * 16) = pk;
          }
        }
      }
    } else if (!to_slots) {
      // lane-derived indices recomputed here (32-bit: rows and H fit), not held across
      // the k loop
      const int lq = tid_opaque() & 63;
      const int hb = (int)d.h0 + wm * 128 + 4 * (lq >> 4);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int r = (int)tok0 + wn * kWaveN + nb * 16 + (lq & 15);
        if (r >= ntok) continue;
        const int64_t t = idx[r];
        float gs = saved[t * 4 + 3] * c;
        if (fixed) gs *= fixed_row_factor(r - c0, t, saved, mr);
        typename E::T* drow = dX + (srow0 < 0 ? t : r - srow0) * H;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const f32x4 v = acc[mb][nb] * gs;
          uint2 pk;
          pk.x = E::pack2(v[0], v[1]);
          pk.y = E::pack2(v[2], v[3]);
          bad |= E::nonfinite2(pk.x) || E::nonfinite2(pk.y);
          *reinterpret_cast<uint2*>(drow + hb + mb * 16) = pk;
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) *slot_ptr(d, nb, mb) = acc[mb][nb];
    }
    if (more) init_acc(acc, dn);
    d = dn;
    have = more;
  }
  if (bad) atomicOr(found_inf, 1);
}

// dX[idx[r]][h] = c * g_r * sum_ks dxp[ks][r - c0][h], ks ascending (row r - srow0 when
// srow0 >= 0).
template <class E>
__global__ void __launch_bounds__(256)
dx_reduce_kernel(int64_t H, int64_t R, int64_t c0, int ksplit, const int32_t* __restrict__ ntok_p,
                 const int32_t* __restrict__ idx, const float* __restrict__ dxp,
                 const float* __restrict__ saved, const float* __restrict__ grad_loss,
                 float loss_scale, typename E::T* __restrict__ dX, int64_t srow0,
                 int32_t* __restrict__ found_inf, const int32_t* __restrict__ redo,
                 const float* __restrict__ mr) {
  const int64_t rl = blockIdx.x;
  const int ntok = *ntok_p;
  const int64_t r = c0 + rl;
  if (r >= ntok) return;
  const int64_t t = idx[r];
  float gs = saved[t * 4 + 3] * ((grad_loss ? *grad_loss : 1.f) / loss_scale);
  if (redo && *redo == 0) gs *= fixed_row_factor(rl, t, saved, mr);
  // the slots dx_kernel wrote: with runs, only those where a run starts
  const int64_t rows = ntok - c0 < R ? ntok - c0 : R;
  const int64_t nht = H / 256, n_items = (rows + 255) / 256 * nht * ksplit;
  const bool runs = dx_runs(n_items, ksplit, kNumWG);
  const int64_t q = n_items / kNumWG;
  bool bad = false;
  for (int64_t h = threadIdx.x * 4; h < H; h += 256 * 4) {
    const int64_t tile = rl / 256 * nht + h / 256;
    f32x4 s = *reinterpret_cast<const f32x4*>(dxp + rl * H + h);
    for (int k = 1; k < ksplit; ++k)
      if (dx_slot_used(runs, tile, k, ksplit, q))
        s += *reinterpret_cast<const f32x4*>(dxp + (k * R + rl) * H + h);
    uint16_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = E::from_f32(s[j] * gs);
      bad |= !isfinite(E::to_f32(o[j]));
    }
    uint2 pk;
    pk.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
    pk.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
    *reinterpret_cast<uint2*>(dX + (srow0 < 0 ? t : r - srow0) * H + h) = pk;
  }
  if (bad) atomicOr(found_inf, 1);
}

// dX of a vocabulary-split chunk from the fp32 sums of its pieces (dx_kernel, acc_mode 1 and
// 2): each piece's buffer held p_v / f_r for v != y_r and 0 at the target, so
//   dX[idx[r]][h] = c g_r ((1 - p_y) W[y_r][h] - f_r sum_ks C_ks[r][h])
// with 1 - p_y = -expm1(q_r) from the row's log-probability (exact even for p_y near 1),
// f_r = exp2(pm[r - c0] - lse2_r) (pm: the reference the single pass's terms were taken
// against; null: 1, the two-pass recompute's plain softmax terms).  One workgroup per
// (token tile, H tile) of the chunk, its threads in the accumulator layout of dx_kernel,
// so the sums are read as they were written; a target outside [0, V) (flagged by the
// forward) adds no W row.  srow0 >= 0: row r goes to row r - srow0 of dX (a staging slot).
template <class E>
__global__ void __launch_bounds__(kThreads)
dx_final_kernel(int64_t H, int64_t V, int64_t R, int64_t c0, int nht, int ksplit,
                const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                const int64_t* __restrict__ targets, const float* __restrict__ dxp,
                const float* __restrict__ saved, const float* __restrict__ grad_loss,
                float loss_scale, const float* __restrict__ pm,
                const typename E::T* __restrict__ W, typename E::T* __restrict__ dX,
                int64_t srow0, int32_t* __restrict__ found_inf, const int32_t* __restrict__ gate) {
  if (gate && *gate == 0) return;   // the fallback's final dX, when the last piece did not write it
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / kWN, wn = w % kWN;
  const int64_t tt = blockIdx.x / nht, ht = blockIdx.x % nht;
  const int ntok = *ntok_p;
  const int64_t tok0 = c0 + tt * 256;
  if (tok0 >= ntok) return;
  const float c = (grad_loss ? *grad_loss : 1.f) / loss_scale;
  const int64_t hb = ht * 256 + wm * 128 + 4 * (lane >> 4);
  // the slots dx_kernel wrote: with runs, only those where a run starts
  const int64_t rows = ntok - c0 < R ? ntok - c0 : R;
  const int64_t n_items = (rows + 255) / 256 * nht * ksplit;
  const bool runs = dx_runs(n_items, ksplit, kNumWG);
  const int64_t q = n_items / kNumWG, tile = tt * nht + ht;
  bool bad = false;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int64_t rl = tt * 256 + wn * kWaveN + nb * 16 + (lane & 15);
    const int64_t r = c0 + rl;
    if (r >= ntok) continue;
    const int64_t t = idx[r];
    const int64_t y = targets[t];
    const float lse2 = saved[t * 4] * kLog2e;
    const float gs = saved[t * 4 + 3] * c;
    const float f = pm ? exp2f(pm[rl] - lse2) : 1.f;
    const bool yok = y >= 0 && y < V;
    const float ty = yok ? -expm1f(saved[t * 4 + 1]) : 0.f;
    const typename E::T* wy = W + (yok ? y : 0) * H + hb;
    typename E::T* drow = dX + (srow0 < 0 ? t : r - srow0) * H + hb;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      f32x4 sm = *reinterpret_cast<const f32x4*>(dxp + dx_sum_offset(tt * nht + ht, w, nb, mb, lane));
      for (int k = 1; k < ksplit; ++k)
        if (dx_slot_used(runs, tile, k, ksplit, q))
          sm += *reinterpret_cast<const f32x4*>(
              dxp + dx_sum_offset((k * (R / 256) + tt) * nht + ht, w, nb, mb, lane));
      const uint2 wv = *reinterpret_cast<const uint2*>(wy + mb * 16);
      const float w0 = E::to_f32((typename E::T)(wv.x & 0xffffu));
      const float w1 = E::to_f32((typename E::T)(wv.x >> 16));
      const float w2 = E::to_f32((typename E::T)(wv.y & 0xffffu));
      const float w3 = E::to_f32((typename E::T)(wv.y >> 16));
      uint2 pk;
      pk.x = E::pack2(gs * (ty * w0 - f * sm[0]), gs * (ty * w1 - f * sm[1]));
      pk.y = E::pack2(gs * (ty * w2 - f * sm[2]), gs * (ty * w3 - f * sm[3]));
      bad |= E::nonfinite2(pk.x) || E::nonfinite2(pk.y);
      *reinterpret_cast<uint2*>(drow + mb * 16) = pk;
    }
  }
  if (bad) atomicOr(found_inf, 1);
}

// ------------------------------------------------------------------------------- dW
// C[h][v] = sum_r XgT[h][r] T[r][v] over the chunk's rows; dW[v][h] = 2^-k C (+ dW[v][h]),
// 2^k the chunk's scale of the operand (xg_scale).  A is XgT [H][R] (gather_cols_kernel),
// rows contiguous, staged like the forward's operands; B is a natural-layout tile of the
// chunk's T [R][Vpad] read in place.
//
// Persistent over the (vocabulary tile, H tile) items, H tile fastest, numbered so that
// workgroup b (on XCD b % 8) takes item 256 r + 32 (b % 8) + b / 8 in round r: the items
// sharing a T slice run on one XCD.  Each item's first k-step is enqueued before the
// previous item's epilogue, so the epilogue's read of the old dW tile and that k-step's
// loads are in flight together.  (The old tile is added after the GEMM, not used as the
// k loop's starting value: that would round every step at the scale of the accumulated
// dW instead of the chunk's own contribution.)
template <class E>
__global__ void __launch_bounds__(kThreads, 1)
dw_kernel(int64_t H, int64_t V, int64_t Vpad, int64_t R, int64_t c0, int nht, int accumulate,
          const int32_t* __restrict__ ntok_p, const char* __restrict__ XgT,
          const char* __restrict__ T, float* __restrict__ dW, int32_t* __restrict__ found_inf,
          const float* __restrict__ xg_scale) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / kWN, wn = w % kWN;
  const int ntok = *ntok_p;
  int64_t nrows = (int64_t)ntok - c0;
  if (nrows > R) nrows = R;
  if (nrows <= 0 && accumulate) return;
  if (nrows < 0) nrows = 0;
  // rows padded to a multiple of 128 (an even number of k-steps); the padding rows of
  // T and XgT are zero
  const int nk = (int)(2 * ((nrows + 127) / 128));
  const int64_t ldx = R * 2, ldt = Vpad * 2;   // bytes per row of XgT and of T
  const int64_t n_items = (int64_t)nht * (Vpad / 256);
  const int nwg = gridDim.x;  // a multiple of 8
  const int64_t first = (int64_t)(blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
  Offs ao, bo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sr = stage_row(i);
    ao[i] = (uint32_t)(sr * ldx) + stage_chunk_bytes(sr);
  }
  nat_offsets(ldt, bo);
  auto opA = [&](int64_t it) {
    const int64_t h0 = (it % nht) * 256;
    return Op<false>{make_src(XgT + h0 * ldx, XgT + H * ldx)};
  };
  auto opB = [&](int64_t it) {
    const int64_t v0 = (it / nht) * 256;
    return Op<true>{T + v0 * 2, R * ldt - v0 * 2, 64 * ldt};
  };
  const float inv = xg_scale[1];
  bool bad = false;
  // first k-step of an item: the workgroups of an XCD that read different H tiles of XgT
  // start one k-step apart instead of all at the same offset of rows 2 R bytes apart
  // (2.4-3.3% of dW measured; rotating by vocabulary tile was 1.5% slower).  A function
  // of the item alone, so each dW entry sums its k-steps in one fixed order.
  auto rot = [&](int64_t it) { return (int)((uint32_t)(it % nht) % (uint32_t)nk); };
  if (first < n_items && nk > 0) gemm_pre_op(opA(first), opB(first), ao, bo, rot(first));
  for (int64_t it = first; it < n_items; it += nwg) {
    Acc acc;
    zero_acc(acc);
    if (nk > 0) gemm_main_op<E, false, true>(opA(it), opB(it), ao, bo, nk, acc, rot(it));
    const int64_t next = it + nwg;
    if (next < n_items && nk > 0) gemm_pre_op(opA(next), opB(next), ao, bo, rot(next));
    const int lq = tid_opaque() & 63;
    const int hb = (int)((it % nht) * 256) + wm * 128 + 4 * (lq >> 4);
    const int64_t v0 = (it / nht) * 256;
    // the tile's rows below V as a buffer resource: rows from V on read 0 and their stores
    // are dropped by the resource's extent, with no per-lane branch
    const int64_t vrows = V - v0 < 256 ? V - v0 : 256;
    const Src dws = make_src(reinterpret_cast<const char*>(dW + v0 * H),
                             reinterpret_cast<const char*>(dW + (v0 + vrows) * H));
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] *= inv;  // undo the chunk's 2^k (exact)
    if (accumulate) {
      // every old value of the lane's columns in flight at once (with the next item's
      // first loads): one memory round trip per item
      f32x4 old[kNB][kMB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const uint32_t o = (uint32_t)((wn * kWaveN + nb * 16 + (lq & 15)) * H + hb) * 4u;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          old[nb][mb] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(dws, o + mb * 64, 0, 0));
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] += old[nb][mb];
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int vr = wn * kWaveN + nb * 16 + (lq & 15);
      const uint32_t o = (uint32_t)(vr * H + hb) * 4u;
      const bool ok = vr < vrows;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const f32x4 val = acc[mb][nb];
#pragma unroll
        for (int j = 0; j < 4; ++j) bad |= ok && !isfinite(val[j]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), dws,
                                               o + mb * 64, 0, 0);
      }
    }
  }
  if (bad) atomicOr(found_inf, 1);
}

// --------------------------------------------------------------------------- dW operand
// The chunk's row factors c g_r s_r (s_r as in dx_kernel) of the dW operand.
__device__ inline float xg_row_factor(int64_t rl, int64_t t, const float* __restrict__ saved,
                                      float c, bool fixed, const float* __restrict__ mr) {
  float sc = saved[t * 4 + 3] * c;
  if (fixed) sc *= fixed_row_factor(rl, t, saved, mr);
  return sc;
}

// xg_scale = (2^k, 2^-k) with 2^k max_r |c g_r s_r| in [1/2, 1) over the chunk's loss rows
// (k = 0 when the maximum is 0 or not finite), one block.  The dW operand is stored in
// the 16-bit type as 2^k c g s X: with g about 1 / N_tok and s down to 2^-14 (fp16
// single-pass window), c g s X alone falls into fp16's subnormals and loses its bits;
// scaled, the largest row sits just below |X| (never above it, so no overflow), and
// dw_kernel multiplies its fp32 tile by 2^-k, exactly.
__global__ void __launch_bounds__(256)
xg_scale_kernel(int64_t R, int64_t c0, const int32_t* __restrict__ ntok_p,
                const int32_t* __restrict__ idx, const float* __restrict__ saved,
                const float* __restrict__ grad_loss, float loss_scale,
                const int32_t* __restrict__ redo, const float* __restrict__ mr,
                float* __restrict__ xg_scale) {
  __shared__ float red[256];
  int64_t nrows = (int64_t)(*ntok_p) - c0;
  if (nrows > R) nrows = R;
  const float c = (grad_loss ? *grad_loss : 1.f) / loss_scale;
  const bool fixed = redo && *redo == 0;
  float m = 0.f;
  for (int64_t rl = threadIdx.x; rl < nrows; rl += 256)
    m = fmaxf(m, fabsf(xg_row_factor(rl, idx[c0 + rl], saved, c, fixed, mr)));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < (unsigned)off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int e = 0;
    const float M = red[0];
    if (M > 0.f && isfinite(M)) {
      frexpf(M, &e);                 // M = f 2^e, f in [1/2, 1)
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
    }
    xg_scale[0] = ldexpf(1.f, -e);
    xg_scale[1] = ldexpf(1.f, e);
  }
}

// XgT[h][rl] = 2^k c g_r s_r X_q[idx[c0 + rl]][h] in the storage type (2^k = xg_scale[0])
// for the chunk's loss rows rl < nrows, and 0 for rl from nrows up to the next multiple of
// 128 (the k range of dw_kernel): the dW operand with the chunk's rows, the reduction index,
// contiguous (R entries per h), so dw_kernel stages it like the forward's operands.  One
// 64-row x 64-column tile per workgroup, transposed through LDS: a thread reads 16
// consecutive h of one row (two 16-byte loads) and writes 16 consecutive rows of one h
// (two 16-byte stores).
template <class E>
__global__ void __launch_bounds__(256)
gather_cols_kernel(const typename E::T* __restrict__ X, int64_t H, int64_t R, int64_t c0,
                   const int32_t* __restrict__ ntok_p, const int32_t* __restrict__ idx,
                   const float* __restrict__ saved, const float* __restrict__ grad_loss,
                   float loss_scale, typename E::T* __restrict__ XgT,
                   const int32_t* __restrict__ redo, const float* __restrict__ mr,
                   const float* __restrict__ xg_scale) {
  typedef typename E::T T;
  __shared__ __attribute__((aligned(16))) T tile[64][72];  // [h][row], 144-byte rows
  int64_t nrows = (int64_t)(*ntok_p) - c0;
  if (nrows > R) nrows = R;
  const int64_t r0 = (int64_t)blockIdx.x * 64, h0 = (int64_t)blockIdx.y * 64;
  if (nrows <= 0 || r0 >= (nrows + 127) / 128 * 128) return;
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, hs = (tid & 3) * 16;
    const int64_t rl = r0 + rr;
    uint32_t out[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (rl < nrows) {
      const int64_t t = idx[c0 + rl];
      const float sc = xg_row_factor(rl, t, saved, (grad_loss ? *grad_loss : 1.f) / loss_scale,
                                     redo && *redo == 0, mr) * xg_scale[0];
      const uint4* src = reinterpret_cast<const uint4*>(X + t * H + h0 + hs);
      const uint4 q0 = src[0], q1 = src[1];
      const uint32_t in[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k)
        out[k] = E::pack2(sc * E::to_f32((T)(in[k] & 0xffffu)), sc * E::to_f32((T)(in[k] >> 16)));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      tile[hs + 2 * k][rr] = (T)(out[k] & 0xffffu);
      tile[hs + 2 * k + 1][rr] = (T)(out[k] >> 16);
    }
  }
  __syncthreads();
  const int hh = tid >> 2, rs = (tid & 3) * 16;
  const uint4 v0 = *reinterpret_cast<const uint4*>(&tile[hh][rs]);
  const uint4 v1 = *reinterpret_cast<const uint4*>(&tile[hh][rs + 8]);
  uint4* dst = reinterpret_cast<uint4*>(XgT + (h0 + hh) * R + r0 + rs);
  dst[0] = v0;
  dst[1] = v1;
}

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

FwdArgs fwd_args(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                 const int64_t* targets) {
  FwdArgs a;
  a.N = p.N;
  a.H = p.H;
  a.V = p.V;
  a.ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  a.idx = ws_ptr<int32_t>(ws, p.off_idx);
  a.Xq = (const char*)Xq;
  a.Xp = (const char*)Xp;
  a.W = (const char*)W;
  a.targets = targets;
  a.part = ws_ptr<float>(ws, p.off_part);
  a.ref_part = ws_ptr<float>(ws, p.off_part);
  a.scale2 = p.scale2;
  a.row_lo = 0;
  a.row_hi = p.N;
  a.side0 = 0;
  a.nsides = 2;
  a.pt = nullptr;
  a.pm = nullptr;
  a.gate = nullptr;
  a.pt_ld = p.pt_ld;
  a.piece = 0;
  a.npieces = 1;
  a.ptiles = p.Vpad / kVocTile;
  a.zero_target = 0;
  a.ref_from_saved = 0;
  a.saved = nullptr;
  a.W8 = ws_ptr<char>(ws, p.off_w8);
  a.Xq8 = ws_ptr<char>(ws, p.off_xq8);
  a.Xp8 = ws_ptr<char>(ws, p.off_xp8);
  a.sw = ws_ptr<float>(ws, p.off_sw);
  a.sxq = ws_ptr<float>(ws, p.off_sxq);
  a.sxp = ws_ptr<float>(ws, p.off_sxp);
  return a;
}

// fp8 logits: e4m3 copies of W and of the loss rows of X_q (and X_p), by compact row.
hipError_t quantize_operands(const Plan& p, void* ws, const void* Xq, const void* Xp,
                             const void* W, hipStream_t st) {
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  hipError_t e = launch_quant_rows(p.dtype, W, p.H, nullptr, nullptr, p.V,
                                   ws_ptr<uint8_t>(ws, p.off_w8), ws_ptr<float>(ws, p.off_sw), st);
  if (e != hipSuccess) return e;
  e = launch_quant_rows(p.dtype, Xq, p.H, idx, ntok, p.N, ws_ptr<uint8_t>(ws, p.off_xq8),
                        ws_ptr<float>(ws, p.off_sxq), st);
  if (e != hipSuccess || !Xp) return e;
  return launch_quant_rows(p.dtype, Xp, p.H, idx, ntok, p.N, ws_ptr<uint8_t>(ws, p.off_xp8),
                           ws_ptr<float>(ws, p.off_sxp), st);
}

template <class E, class G>
hipError_t fwd_impl(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                    const int64_t* targets, hipStream_t st) {
  if (G::kBytes == 1) {
    const hipError_t e = quantize_operands(p, ws, Xq, Xp, W, st);
    if (e != hipSuccess) return e;
  }
  FwdArgs a = fwd_args(p, ws, Xq, Xp, W, targets);
  trace_begin(p, GRPO_TRACE_FWD_ALL, st);
  hipLaunchKernelGGL((fwd_kernel<E, G, 0>), dim3(kNumWG), dim3(kThreads), 0, st, a);
  trace_end(p, GRPO_TRACE_FWD_ALL, st);
  return hipGetLastError();
}

// dX (and dW) of the loss rows of chunk c0 from the chunk's T = onehot - softmax.
template <class E>
// redo (non-null): the chunk buffer holds mode-3 rows -T / f unless *redo != 0 (see
// dx_kernel); mr: their per-row reference.
hipError_t chunk_grads(const Plan& p, void* ws, int64_t c0, const void* Xq, const void* W,
                       const float* saved, const float* grad_loss, float loss_scale, void* dX,
                       float* dW, int accumulate_dW, int32_t* found_inf, hipStream_t st,
                       const int32_t* redo = nullptr, const float* mr = nullptr) {
  typedef typename E::T T;
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  T* Tb = ws_ptr<T>(ws, p.off_T);
  const int nvt = (int)(p.Vpad / 256), nht = (int)(p.H / 256);
  hipError_t e;
  trace_begin(p, GRPO_TRACE_DX, st);
  hipLaunchKernelGGL(dx_kernel<E>, dim3(kNumWG), dim3(kThreads), 0, st,
                     p.H, p.V, p.Vpad, p.Vpad, (int64_t)0, p.R, c0, nht, p.ksplit, 0, ntok, idx,
                     (const char*)W, (const char*)Tb, saved, grad_loss, loss_scale,
                     (T*)dx_out(p, dX, c0), stage_row0(p, c0), ws_ptr<float>(ws, p.off_dxp),
                     found_inf, redo, mr, (const int32_t*)nullptr, (const int64_t*)nullptr);
  trace_end(p, GRPO_TRACE_DX, st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.ksplit > 1) {
    hipLaunchKernelGGL(dx_reduce_kernel<E>, dim3((unsigned)p.R), dim3(256), 0, st, p.H, p.R, c0,
                       p.ksplit, ntok, idx, (const float*)ws_ptr<float>(ws, p.off_dxp), saved,
                       grad_loss, loss_scale, (T*)dx_out(p, dX, c0), stage_row0(p, c0),
                       found_inf, redo, mr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dW) {
    T* Xg = ws_ptr<T>(ws, p.off_Xg);
    float* xs = ws_ptr<float>(ws, p.off_xgs);
    hipLaunchKernelGGL(xg_scale_kernel, dim3(1), dim3(256), 0, st, p.R, c0, ntok, idx, saved,
                       grad_loss, loss_scale, redo, mr, xs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gather_cols_kernel<E>, dim3((unsigned)(p.R / 64), (unsigned)(p.H / 64)),
                       dim3(256), 0, st, (const T*)Xq, p.H, p.R, c0, ntok, idx, saved, grad_loss,
                       loss_scale, Xg, redo, mr, (const float*)xs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    trace_begin(p, GRPO_TRACE_DW, st);
    hipLaunchKernelGGL(dw_kernel<E>, dim3(kNumWG), dim3(kThreads), 0, st, p.H,
                       p.V, p.Vpad, p.R, c0, nht, c0 == 0 ? accumulate_dW : 1, ntok,
                       (const char*)Xg, (const char*)Tb, dW, found_inf, (const float*)xs);
    trace_end(p, GRPO_TRACE_DW, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class E, class G>
hipError_t bwd_impl(const Plan& p, void* ws, const void* Xq, const void* W,
                    const int64_t* targets, const float* saved, const float* grad_loss,
                    float loss_scale, void* dX, float* dW, int accumulate_dW, int32_t* found_inf,
                    hipStream_t st) {
  typedef typename E::T T;
  constexpr bool kF8 = G::kBytes == 1;
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  T* Tb = ws_ptr<T>(ws, p.off_T);
  hipError_t e = hipSuccess;
  if (kF8 && (e = quantize_operands(p, ws, Xq, nullptr, W, st)) != hipSuccess) return e;
  const char* Xop = kF8 ? ws_ptr<char>(ws, p.off_xq8) : (const char*)Xq;
  const char* Wop = kF8 ? ws_ptr<char>(ws, p.off_w8) : (const char*)W;
  const int ntt = (int)(p.R / 256), nvt = (int)(p.Vpad / 256);
  for (int64_t c0 = 0; c0 < p.N; c0 += p.R) {
    trace_begin(p, GRPO_TRACE_RECOMPUTE, st);
    hipLaunchKernelGGL((recompute_kernel<E, G>), dim3((unsigned)(ntt * nvt)), dim3(kThreads), 0,
                       st, p.N, p.H, p.V, p.Vpad, (int64_t)0, c0, ntt, p.scale2, 0, ntok, idx,
                       Xop, Wop, targets, saved, Tb, (const float*)ws_ptr<float>(ws, p.off_sw),
                       (const float*)ws_ptr<float>(ws, p.off_sxq));
    trace_end(p, GRPO_TRACE_RECOMPUTE, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = chunk_grads<E>(p, ws, c0, Xq, W, saved, grad_loss, loss_scale, dX, dW, accumulate_dW,
                       found_inf, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Single pass: reference forward over all rows, then per chunk of R loss rows the policy
// forward that also keeps its softmax terms, the chunk's merge, and dX (and dW) from the
// kept terms.  The logits of each row are computed once per side instead of twice for
// the policy.  The terms are taken against the row's reference-side log-sum-exp (mode 3)
// and the merge rewrites each row's target entry, so the chunk buffer holds -T / f per row
// and dX, dW scale their rows by -f (dx_kernel).  A chunk with a row whose policy and
// reference log-sum-exp lie too far apart (outside [-60, 60] in log2 units for bf16,
// [-4, 14] for fp16, whose stored terms must fit fp16) sets its flag in the merge,
// and then the mode-2 forward, merge and fixup below, which exit at once otherwise, redo
// the chunk with running maxima into T = onehot - softmax.
template <class E, class G>
hipError_t fused_impl(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                      const int64_t* targets, const uint8_t* mask, const float* adv, float beta,
                      float* saved, float* logp, float* ref_logp, float* kl, int32_t* status,
                      float* loss, const float* grad_loss, float loss_scale, void* dX, float* dW,
                      int accumulate_dW, int32_t* found_inf, hipStream_t st) {
  typedef typename E::T T;
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  T* Tb = ws_ptr<T>(ws, p.off_T);
  float* pm = ws_ptr<float>(ws, p.off_pm);
  int32_t* redo = ws_ptr<int32_t>(ws, p.off_redo);
  const int64_t nvt = (p.V + 255) / 256;
  const int nchunks = (int)((p.N + p.R - 1) / p.R);
  hipError_t e = launch_zero_masked_outputs(p, mask, saved, logp, ref_logp, kl, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st,
                     redo, nchunks, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (G::kBytes == 1 && (e = quantize_operands(p, ws, Xq, Xp, W, st)) != hipSuccess) return e;
  FwdArgs a = fwd_args(p, ws, Xq, Xp, W, targets);
  a.side0 = 1;
  a.nsides = 1;
  trace_begin(p, GRPO_TRACE_FWD_ALL, st);
  hipLaunchKernelGGL((fwd_kernel<E, G, 1>), dim3(kNumWG), dim3(kThreads), 0, st, a);
  trace_end(p, GRPO_TRACE_FWD_ALL, st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t c0 = 0, ci = 0; c0 < p.N; c0 += p.R, ++ci) {
    int32_t* rd = redo + ci;
    a.row_lo = c0;
    a.row_hi = c0 + p.R;
    a.side0 = 0;
    a.part = ws_ptr<float>(ws, p.off_cpart);
    a.pt = reinterpret_cast<char*>(Tb);
    a.pm = pm;
    a.gate = nullptr;
    trace_begin(p, GRPO_TRACE_FWD_CHUNK, st);
    hipLaunchKernelGGL((fwd_kernel<E, G, 3>), dim3(kNumWG), dim3(kThreads), 0, st, a);
    trace_end(p, GRPO_TRACE_FWD_CHUNK, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_merge_rows(p, ws, c0, targets, mask, adv, beta, saved, logp, ref_logp, kl,
                          status, st, rd, Tb, nullptr);
    if (e != hipSuccess) return e;
    // fallback, gated on the chunk's flag
    a.gate = rd;
    hipLaunchKernelGGL((fwd_kernel<E, G, 2>), dim3(kNumWG), dim3(kThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_merge_rows(p, ws, c0, targets, mask, adv, beta, saved, logp, ref_logp, kl, status,
                          st, nullptr, nullptr, rd);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fixup_kernel<E>,
                       dim3((unsigned)((p.Vpad + 2047) / 2048), (unsigned)(p.R < 64 ? p.R : 64)),
                       dim3(256), 0, st, p.Vpad, nvt, c0, p.R, ntok, idx, targets, saved,
                       (const float*)pm, Tb, (const int32_t*)rd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.ring && (e = p.ring->acquire(c0)) != hipSuccess) return e;
    e = chunk_grads<E>(p, ws, c0, Xq, W, saved, grad_loss, loss_scale, dX, dW, accumulate_dW,
                       found_inf, st, rd, pm);
    if (e != hipSuccess) return e;
    if (p.ring && (e = p.ring->transfer(c0)) != hipSuccess) return e;
  }
  return launch_loss_final(p, ws, 1, status, loss, st);
}

// Vocabulary split: dX of chunk c0 from one piece of its buffer (columns 0 .. pt_ld - 1
// hold vocabulary rows piece ptiles 256 ..), into the chunk's fp32 sums: the first piece
// writes them, the later ones add to them.  gate: the fallback's launches.  fin (non-null,
// ksplit == 1, the last piece after the chunk's merge): dX itself (dx_kernel's acc_mode 3)
// with the row factors of the merged chunk, skipped when the chunk's flag fin->redo is set.
struct FinalDx {
  const int64_t* targets;
  const float* saved;
  const float* grad_loss;
  float loss_scale;
  void* dX;
  const int32_t* redo;
  const float* pm;
};
template <class E>
hipError_t piece_dx(const Plan& p, void* ws, int64_t c0, int piece, const void* W,
                    int32_t* found_inf, hipStream_t st, const int32_t* gate, bool traced,
                    const FinalDx* fin = nullptr) {
  typedef typename E::T T;
  const int nht = (int)(p.H / 256);
  const int64_t nvt = p.Vpad / kVocTile, vt0 = (int64_t)piece * p.ptiles;
  const int64_t tiles = nvt - vt0 < p.ptiles ? nvt - vt0 : p.ptiles;
  const int mode = fin ? 3 : (piece == 0 ? 1 : 2);
  if (traced) trace_begin(p, GRPO_TRACE_DX, st);
  hipLaunchKernelGGL(dx_kernel<E>, dim3(kNumWG), dim3(kThreads), 0, st, p.H, p.V, p.pt_ld,
                     tiles * kVocTile, vt0 * kVocTile, p.R, c0, nht, p.ksplit, mode,
                     ws_ptr<int32_t>(ws, p.off_ntok), ws_ptr<int32_t>(ws, p.off_idx),
                     (const char*)W, (const char*)ws_ptr<T>(ws, p.off_T),
                     fin ? fin->saved : (const float*)nullptr,
                     fin ? fin->grad_loss : (const float*)nullptr,
                     fin ? fin->loss_scale : 1.f,
                     fin ? (T*)dx_out(p, fin->dX, c0) : (T*)nullptr,
                     fin ? stage_row0(p, c0) : (int64_t)-1, ws_ptr<float>(ws, p.off_dxp),
                     found_inf, fin ? fin->redo : (const int32_t*)nullptr,
                     fin ? fin->pm : (const float*)nullptr, gate,
                     fin ? fin->targets : (const int64_t*)nullptr);
  if (traced) trace_end(p, GRPO_TRACE_DX, st);
  return hipGetLastError();
}

// dX of a vocabulary-split chunk from its pieces' sums (dx_final_kernel).
template <class E>
hipError_t split_dx_final(const Plan& p, void* ws, int64_t c0, const void* W,
                          const int64_t* targets, const float* saved, const float* grad_loss,
                          float loss_scale, const float* pm, void* dX, int32_t* found_inf,
                          hipStream_t st, const int32_t* gate = nullptr) {
  typedef typename E::T T;
  const int nht = (int)(p.H / 256);
  hipLaunchKernelGGL(dx_final_kernel<E>, dim3((unsigned)(p.R / 256 * nht)), dim3(kThreads), 0,
                     st, p.H, p.V, p.R, c0, nht, p.ksplit, ws_ptr<int32_t>(ws, p.off_ntok),
                     ws_ptr<int32_t>(ws, p.off_idx), targets,
                     (const float*)ws_ptr<float>(ws, p.off_dxp), saved, grad_loss, loss_scale, pm,
                     (const T*)W, (T*)dx_out(p, dX, c0), stage_row0(p, c0), found_inf, gate);
  return hipGetLastError();
}

// Two-pass backward with the vocabulary split: per chunk and piece, the softmax terms of
// the piece (target entry 0) recomputed from the forward's log-sum-exp, and their dX sums;
// then the chunk's dX.
template <class E, class G>
hipError_t bwd_split_impl(const Plan& p, void* ws, const void* Xq, const void* W,
                          const int64_t* targets, const float* saved, const float* grad_loss,
                          float loss_scale, void* dX, int32_t* found_inf, hipStream_t st) {
  typedef typename E::T T;
  constexpr bool kF8 = G::kBytes == 1;
  const int32_t* ntok = ws_ptr<int32_t>(ws, p.off_ntok);
  const int32_t* idx = ws_ptr<int32_t>(ws, p.off_idx);
  T* Tb = ws_ptr<T>(ws, p.off_T);
  hipError_t e = hipSuccess;
  if (kF8 && (e = quantize_operands(p, ws, Xq, nullptr, W, st)) != hipSuccess) return e;
  const char* Xop = kF8 ? ws_ptr<char>(ws, p.off_xq8) : (const char*)Xq;
  const char* Wop = kF8 ? ws_ptr<char>(ws, p.off_w8) : (const char*)W;
  const int ntt = (int)(p.R / 256);
  const int64_t nvt = p.Vpad / 256;
  for (int64_t c0 = 0; c0 < p.N; c0 += p.R) {
    for (int j = 0; j < p.npieces; ++j) {
      const int64_t vt0 = (int64_t)j * p.ptiles;
      const int64_t tiles = nvt - vt0 < p.ptiles ? nvt - vt0 : p.ptiles;
      trace_begin(p, GRPO_TRACE_RECOMPUTE, st);
      hipLaunchKernelGGL((recompute_kernel<E, G>), dim3((unsigned)(ntt * tiles)),
                         dim3(kThreads), 0, st, p.N, p.H, p.V, p.pt_ld, vt0, c0, ntt, p.scale2,
                         1, ntok, idx, Xop, Wop, targets, saved, Tb,
                         (const float*)ws_ptr<float>(ws, p.off_sw),
                         (const float*)ws_ptr<float>(ws, p.off_sxq));
      trace_end(p, GRPO_TRACE_RECOMPUTE, st);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      // the last piece writes dX itself when the reduction is not split (the row
      // factors are the forward's, already in `saved`)
      const bool last = j == p.npieces - 1 && p.ksplit == 1;
      const FinalDx fin{targets, saved, grad_loss, loss_scale, dX, nullptr, nullptr};
      if ((e = piece_dx<E>(p, ws, c0, j, W, found_inf, st, nullptr, true,
                           last ? &fin : nullptr)) != hipSuccess)
        return e;
    }
    if (p.ksplit > 1) {
      e = split_dx_final<E>(p, ws, c0, W, targets, saved, grad_loss, loss_scale, nullptr, dX,
                            found_inf, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Single pass with the vocabulary split (no dW).  The reference side runs over all rows;
// then per chunk, piece by piece, the policy forward keeps the piece's terms against the
// row's reference log-sum-exp (target entry 0) and dX sums them; the chunk's merge then
// knows each row's log-sum-exp, and dx_final_kernel applies the row factor and adds the
// target's term.  A chunk whose merge finds a row outside the window redoes it: the
// policy forward over the chunk's rows without kept terms (a robust log-sum-exp), the
// merge again, and the pieces once more against that log-sum-exp, whose terms are then
// the softmax itself (these launches exit at once when the chunk's flag is clear).
template <class E, class G>
hipError_t fused_split_impl(const Plan& p, void* ws, const void* Xq, const void* Xp,
                            const void* W, const int64_t* targets, const uint8_t* mask,
                            const float* adv, float beta, float* saved, float* logp,
                            float* ref_logp, float* kl, int32_t* status, float* loss,
                            const float* grad_loss, float loss_scale, void* dX,
                            int32_t* found_inf, hipStream_t st) {
  typedef typename E::T T;
  T* Tb = ws_ptr<T>(ws, p.off_T);
  float* pm = ws_ptr<float>(ws, p.off_pm);
  int32_t* redo = ws_ptr<int32_t>(ws, p.off_redo);
  const int64_t nvt = p.Vpad / 256;
  const int nchunks = (int)((p.N + p.R - 1) / p.R);
  hipError_t e = launch_zero_masked_outputs(p, mask, saved, logp, ref_logp, kl, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st,
                     redo, nchunks, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (G::kBytes == 1 && (e = quantize_operands(p, ws, Xq, Xp, W, st)) != hipSuccess) return e;
  FwdArgs a = fwd_args(p, ws, Xq, Xp, W, targets);
  a.side0 = 1;
  a.nsides = 1;
  trace_begin(p, GRPO_TRACE_FWD_ALL, st);
  hipLaunchKernelGGL((fwd_kernel<E, G, 1>), dim3(kNumWG), dim3(kThreads), 0, st, a);
  trace_end(p, GRPO_TRACE_FWD_ALL, st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // chunks last to first: they are independent here (no dW to accumulate), and the
  // chunks past the loss-row count, which exit at once, then come first, so that the
  // gradient offload's copies of their (unused) rows run beside real work instead of
  // after it
  for (int64_t ci = nchunks - 1; ci >= 0; --ci) {
    const int64_t c0 = ci * p.R;
    int32_t* rd = redo + ci;
    FwdArgs c = a;
    c.row_lo = c0;
    c.row_hi = c0 + p.R;
    c.side0 = 0;
    c.part = ws_ptr<float>(ws, p.off_cpart);
    c.pt = reinterpret_cast<char*>(Tb);
    c.pm = pm;
    c.npieces = p.npieces;
    c.ptiles = p.ptiles;
    c.zero_target = 1;
    // With the reduction not split, the last piece's dX waits for the chunk's merge and
    // writes dX itself (no fp32 sums round trip, no final launch), unless the merge sends
    // the chunk to the fallback, which then ends with dx_final_kernel.
    const bool fuse = p.ksplit == 1;
    for (int j = 0; j < p.npieces; ++j) {
      c.piece = j;
      trace_begin(p, GRPO_TRACE_FWD_CHUNK, st);
      hipLaunchKernelGGL((fwd_kernel<E, G, 3>), dim3(kNumWG), dim3(kThreads), 0, st, c);
      trace_end(p, GRPO_TRACE_FWD_CHUNK, st);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (fuse && j == p.npieces - 1) break;
      if ((e = piece_dx<E>(p, ws, c0, j, W, found_inf, st, nullptr, true)) != hipSuccess)
        return e;
    }
    e = launch_merge_rows(p, ws, c0, targets, mask, adv, beta, saved, logp, ref_logp, kl,
                          status, st, rd, nullptr, nullptr, p.ptiles, p.npieces);
    if (e != hipSuccess) return e;
    if (p.ring && (e = p.ring->acquire(c0)) != hipSuccess) return e;
    if (fuse) {
      const FinalDx fin{targets, saved, grad_loss, loss_scale, dX, rd, pm};
      e = piece_dx<E>(p, ws, c0, p.npieces - 1, W, found_inf, st, nullptr, true, &fin);
      if (e != hipSuccess) return e;
    }
    // fallback, gated on the chunk's flag: a robust policy sweep, its merge, the pieces
    FwdArgs f = c;
    f.gate = rd;
    f.piece = 0;
    f.npieces = 1;
    f.ptiles = nvt;
    f.pt = nullptr;
    f.zero_target = 0;
    hipLaunchKernelGGL((fwd_kernel<E, G, 1>), dim3(kNumWG), dim3(kThreads), 0, st, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_merge_rows(p, ws, c0, targets, mask, adv, beta, saved, logp, ref_logp, kl,
                          status, st, nullptr, nullptr, rd, nvt, 1);
    if (e != hipSuccess) return e;
    c.gate = rd;
    c.ref_from_saved = 1;
    c.saved = saved;
    for (int j = 0; j < p.npieces; ++j) {
      c.piece = j;
      hipLaunchKernelGGL((fwd_kernel<E, G, 3>), dim3(kNumWG), dim3(kThreads), 0, st, c);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = piece_dx<E>(p, ws, c0, j, W, found_inf, st, rd, false)) != hipSuccess) return e;
    }
    e = split_dx_final<E>(p, ws, c0, W, targets, saved, grad_loss, loss_scale, pm, dX,
                          found_inf, st, fuse ? rd : nullptr);
    if (e != hipSuccess) return e;
    if (p.ring && (e = p.ring->transfer(c0)) != hipSuccess) return e;
  }
  return launch_loss_final(p, ws, 1, status, loss, st);
}

}  // namespace

hipError_t mfma_fwd_partials(const Plan& p, void* ws, const void* Xq, const void* Xp,
                             const void* W, const int64_t* targets, hipStream_t st) {
  if (p.dtype == GRPO_BF16)
    return p.fp8 ? fwd_impl<BF16T, FP8T>(p, ws, Xq, Xp, W, targets, st)
                 : fwd_impl<BF16T, BF16T>(p, ws, Xq, Xp, W, targets, st);
  return p.fp8 ? fwd_impl<F16T, FP8T>(p, ws, Xq, Xp, W, targets, st)
               : fwd_impl<F16T, F16T>(p, ws, Xq, Xp, W, targets, st);
}

hipError_t mfma_fused(const Plan& p, void* ws, const void* Xq, const void* Xp, const void* W,
                      const int64_t* targets, const uint8_t* mask, const float* adv, float beta,
                      float* saved, float* logp, float* ref_logp, float* kl, int32_t* status,
                      float* loss, const float* grad_loss, float loss_scale, void* dX, float* dW,
                      int accumulate_dW, int32_t* found_inf, hipStream_t st) {
#define GRPO_FUSED(E, G)                                                                       \
  (p.vsplit ? fused_split_impl<E, G>(p, ws, Xq, Xp, W, targets, mask, adv, beta, saved, logp, \
                                     ref_logp, kl, status, loss, grad_loss, loss_scale, dX,    \
                                     found_inf, st)                                            \
            : fused_impl<E, G>(p, ws, Xq, Xp, W, targets, mask, adv, beta, saved, logp,        \
                               ref_logp, kl, status, loss, grad_loss, loss_scale, dX, dW,       \
                               accumulate_dW, found_inf, st))
  if (p.dtype == GRPO_BF16) return p.fp8 ? GRPO_FUSED(BF16T, FP8T) : GRPO_FUSED(BF16T, BF16T);
  return p.fp8 ? GRPO_FUSED(F16T, FP8T) : GRPO_FUSED(F16T, F16T);
#undef GRPO_FUSED
}

hipError_t mfma_backward(const Plan& p, void* ws, const void* Xq, const void* W,
                         const int64_t* targets, const float* saved, const float* grad_loss,
                         float loss_scale, void* dX, float* dW, int accumulate_dW,
                         int32_t* found_inf, hipStream_t st) {
#define GRPO_BWD(E, G)                                                                         \
  (p.vsplit ? bwd_split_impl<E, G>(p, ws, Xq, W, targets, saved, grad_loss, loss_scale, dX,   \
                                   found_inf, st)                                              \
            : bwd_impl<E, G>(p, ws, Xq, W, targets, saved, grad_loss, loss_scale, dX, dW,      \
                             accumulate_dW, found_inf, st))
  if (p.dtype == GRPO_BF16) return p.fp8 ? GRPO_BWD(BF16T, FP8T) : GRPO_BWD(BF16T, BF16T);
  return p.fp8 ? GRPO_BWD(F16T, FP8T) : GRPO_BWD(F16T, F16T);
#undef GRPO_BWD
}

}  // namespace grpo
