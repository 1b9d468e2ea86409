// Host side of the C ABI declared in include/grpo.h: argument validation, the workspace
// plan and the launch sequence.  Nothing here allocates, synchronises or prints.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "common.h"

namespace grpo {

hipError_t simple_fwd_partials(const Plan& p, void* ws, const void* Xq, const void* Xp,
                               const void* W, const int64_t* targets, hipStream_t st);
hipError_t simple_backward(const Plan& p, void* ws, const void* Xq, const void* W,
                           const int64_t* targets, const float* saved, const float* grad_loss,
                           float loss_scale, void* dX, float* dW, int accumulate_dW,
                           int32_t* found_inf, hipStream_t st);
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

constexpr size_t kAlign = 256;
// Rows per backward chunk (a multiple of 256): the workspace holds one chunk of
// onehot - softmax, chunk rows x V in the storage type.
#ifndef GRPO_CHUNK_ROWS
#define GRPO_CHUNK_ROWS 4096
#endif
constexpr int64_t kChunkRows = GRPO_CHUNK_ROWS;
constexpr int kMaxDevices = 64;
constexpr int kXcdsHost = 8;  // XCDs of the persistent grids (8 x 32 workgroups)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device memory of grpo_loss_fwd_noalloc, for callers that cannot allocate: a fixed array
// in place of a workspace.  Each GPU the library runs on holds its own copy until the
// process ends; every call on one GPU uses the same copy.
constexpr size_t kScratchBytes = GRPO_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

// This device's address of `scratch`, looked up once per device.  On the host the symbol
// names a stand-in, not device memory, so only this address may reach a kernel.
void* scratch_address() {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

bool valid_dtype(int dt) { return dt == GRPO_F32 || dt == GRPO_BF16 || dt == GRPO_F16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 1 = gfx950, 0 = another device, cached per device ordinal.
int device_ok() {
  static int cache[kMaxDevices] = {0};  // 0 unknown, 1 ok, 2 not ok
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices && cache[dev]) return cache[dev] == 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) cache[dev] = ok ? 1 : 2;
  return ok;
}

bool options_ok(const grpo_options* o) {
  if (!o) return true;
  if (o->kl_estimator < GRPO_KL_REVERSE || o->kl_estimator > GRPO_KL_REVERSE_Q) return false;
  if (o->detach_ratio != 0 && o->detach_ratio != 1) return false;
  if (o->normalization != GRPO_NORM_TOKENS && o->normalization != GRPO_NORM_SEQUENCES)
    return false;
  if (o->fp8_logits != 0 && o->fp8_logits != 1) return false;
  if (o->chunk_rows != 0 &&
      (o->chunk_rows % 256 != 0 || o->chunk_rows < 256 || o->chunk_rows > 65536))
    return false;
  if (o->vocab_piece != 0 && (o->vocab_piece % 256 != 0 || o->vocab_piece < 256)) return false;
  if (o->trace_kernel < GRPO_TRACE_NONE || o->trace_kernel > GRPO_TRACE_DW ||
      o->trace_capacity < 0 || (o->trace_capacity > 0 && !o->trace_events))
    return false;
  if ((o->dx_host || o->dw_host) && !o->copy_stream) return false;
  if ((o->dx_host && !aligned16(o->dx_host)) || (o->dw_host && !aligned16(o->dw_host)))
    return false;
  // the softmax argument z / tau must stay finite for finite logits
  return isfinite(o->temperature) && o->temperature >= 1e-3f && o->temperature <= 1e3f;
}

// Pieces of the vocabulary split when the caller names no size: at least enough that no
// piece has more than kPieceTiles tiles (the workspace bound), at most twice that, chosen
// for the fewest rounds of the chunk forward's persistent grid on a full chunk (ntb token
// blocks): a piece of pt tiles takes ceil(ntb / (256 / P)) ceil(pt / P) rounds with P
// phases (fwd_phases), plus about one round's worth per piece for its launches and the dX
// sums it writes and reads (measured at the 20K-context shape: 87 us per extra piece
// against 112 us per round).  Phi-4's 392 tiles: 5 pieces of 79 tiles, 25 rounds, instead
// of 4 of 98, 28 rounds.
int default_pieces(int64_t nvt, int64_t ntb) {
  const int64_t lo = (nvt + kPieceTiles - 1) / kPieceTiles;
  int64_t best = lo, best_cost = -1;
  for (int64_t np = lo; np <= 2 * lo; ++np) {
    const int64_t pt = (nvt + np - 1) / np;
    const int P = fwd_phases(ntb, pt);
    const int64_t per_round = (int64_t)kXcdsHost * 32 / P;   // P <= 256
    const int64_t rounds = ((ntb + per_round - 1) / per_round) * ((pt + P - 1) / P);
    const int64_t cost = np * (rounds + 1);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = np;
    }
  }
  return (int)best;
}

bool sizes_ok(int64_t S, int64_t L, int64_t H, int64_t V) {
  if (S < 1 || L < 1 || H < 8 || V < 1) return false;
  if (H % 8 != 0) return false;                   // 16-byte rows of 16-bit data
  if (S > INT32_MAX / L) return false;            // row indices are int32
  if (V > (int64_t)1 << 30 || H > (int64_t)1 << 20) return false;
  return true;
}

}  // namespace

bool make_plan(int64_t S, int64_t L, int64_t H, int64_t V, int dtype, int need_dW, Plan* p,
               const grpo_options* opts) {
  if (!sizes_ok(S, L, H, V) || !valid_dtype(dtype)) return false;
  memset(p, 0, sizeof(*p));
  p->N = S * L;
  p->L = L;
  p->H = H;
  p->V = V;
  p->Vpad = (V + kVocTile - 1) / kVocTile * kVocTile;
  p->dtype = dtype;
  p->esize = dtype == GRPO_F32 ? 4 : 2;
  p->need_dW = need_dW ? 1 : 0;
  p->phases = kMaxPhases;
  plan_options(opts, p);
  // 16-bit operands with H a multiple of 256 take the MFMA kernels (256-wide tiles over H);
  // everything else takes the fp32-accumulating FMA kernels.
  const int64_t Npad = (p->N + kTokTile - 1) / kTokTile * kTokTile;
  const int64_t chunk = p->chunk_rows > 0 ? p->chunk_rows : kChunkRows;
  p->R = Npad < chunk ? Npad : chunk;
  // (the MFMA kernels address each operand with 32-bit byte offsets from a buffer base:
  // X, W and one chunk of onehot - softmax must each stay below 4 GiB)
  const uint64_t k4G = (uint64_t)1 << 32;
  p->mfma = dtype != GRPO_F32 && H % 256 == 0 && (uint64_t)p->N * H * 2 < k4G &&
            (uint64_t)p->Vpad * H * 2 < k4G && (uint64_t)p->R * p->Vpad * 2 < k4G;
  p->ksplit = 1;
  if (p->mfma) {
    // Split the dX reduction over the vocabulary so that a full chunk's (tile, split)
    // items fill whole rounds of the 256 persistent workgroups: time goes as
    // ceil(tiles k / 256) / k, minimised over k <= 8 (the smallest k on ties).
    const int64_t tiles = (H / 256) * (p->R / 256);
    double best = 1e30;
    for (int k = 1; k <= 8; ++k) {
      const double cost = (double)((tiles * k + 255) / 256) / k;
      if (cost < best - 1e-9) {
        best = cost;
        p->ksplit = k;
      }
    }
  }
  const int64_t nvt = p->Vpad / kVocTile;
  // Vocabulary split of the backward (everything on the MFMA kernels but the single pass
  // with dW, whose row factor is known only once the chunk's whole vocabulary has been
  // swept): pieces of at most kPieceTiles tiles (vocab_piece entries if given), balanced.
  p->vsplit = p->mfma && !need_dW;
  p->npieces = 1;
  p->ptiles = nvt;
  if (p->vsplit) {
    if (p->vocab_piece > 0) {
      const int64_t want = p->vocab_piece / kVocTile;
      p->npieces = (int)((nvt + want - 1) / want);
    } else {
      p->npieces = default_pieces(nvt, p->R / kTokTile);
    }
    p->ptiles = (nvt + p->npieces - 1) / p->npieces;
  }
  p->pt_ld = p->ptiles * kVocTile;
  // what the forward uses comes first, so that its size is a prefix of the plan
  size_t o = 0;
  p->off_ntok = o;
  o = align_up(o + compact_bytes(p->N));
  p->off_idx = o;
  o = align_up(o + (size_t)p->N * 4);
  p->off_rank = o;
  o = align_up(o + (size_t)p->N * 4);
  p->off_part = o;
  // MFMA: the larger of the two-pass forward's (both sides in one launch) and the single
  // pass's reference-side layouts; FMA: a fixed phase count with row stride N
  const size_t part_floats =
      p->mfma ? std::max(part_floats_max(p->N, 2, nvt), part_floats_max(p->N, 1, nvt))
              : (size_t)6 * p->phases * p->N;
  o = align_up(o + part_floats * 4);
  p->off_lsum = o;
  o = align_up(o + (size_t)((p->N + kMergeBlock - 1) / kMergeBlock) * 8);
  p->off_seq = o;
  o = align_up(o + (size_t)(S + 1) * 4);
  if (p->fp8 && !p->mfma) return false;   // fp8 logits run on the MFMA kernels only
  p->off_xq8 = p->off_xp8 = p->off_w8 = p->off_sxq = p->off_sxp = p->off_sw = o;
  if (p->fp8) {
    p->off_xq8 = o;
    o = align_up(o + (size_t)p->N * H);
    p->off_xp8 = o;
    o = align_up(o + (size_t)p->N * H);
    p->off_w8 = o;
    o = align_up(o + (size_t)V * H);
    p->off_sxq = o;
    o = align_up(o + (size_t)p->N * 4);
    p->off_sxp = o;
    o = align_up(o + (size_t)p->N * 4);
    p->off_sw = o;
    o = align_up(o + (size_t)V * 4);
  }
  p->fwd_total = o;
  p->off_cpart = o;  // single pass: the policy partials of one chunk (pieces, or one sweep)
  if (p->mfma)
    o = align_up(o + std::max(part_floats_max(p->R, 1, p->ptiles, p->npieces),
                              part_floats_max(p->R, 1, nvt)) * 4);
  p->off_T = o;      // the chunk buffer: R rows of one piece (or of the whole vocabulary)
  o = align_up(o + (size_t)p->R * p->pt_ld * p->esize);
  p->off_pm = o;     // per row (vocabulary split) or per row and tile (running maxima)
  if (p->mfma) o = align_up(o + (size_t)p->R * (p->vsplit ? 1 : nvt) * 4);
  p->off_Xg = o;
  if (p->mfma && need_dW) o = align_up(o + (size_t)p->R * H * p->esize);
  p->off_xgs = o;
  if (p->mfma && need_dW) o = align_up(o + 16);
  p->off_redo = o;  // single-pass fallback flags, one per chunk
  if (p->mfma) o = align_up(o + (size_t)((p->N + p->R - 1) / p->R) * 4);
  p->off_dxp = o;    // fp32 dX partials [ksplit][R][H]: split reductions, or the pieces' sums
  if (p->mfma && (p->ksplit > 1 || p->vsplit))
    o = align_up(o + (size_t)p->ksplit * p->R * H * 4);
  p->off_ring = o;   // gradient offload: two staging slots of a chunk's dX rows
  if (p->offload) o = align_up(o + (size_t)2 * p->R * H * p->esize);
  p->total = o;
  return true;
}

// The traced launches of a call, for its caller (grpo_options.trace_count).
static int traced(const grpo_options* opts, int launches) {
  if (opts && opts->trace_count) *opts->trace_count = launches;
  return GRPO_OK;
}

size_t part_floats_max(int64_t max_rows, int nsides, int64_t tiles, int npieces) {
  // the phase count depends on the token blocks through a ceiling, so the product is not
  // monotone in the rows: take the maximum over every block count (P <= kMaxFwdPhases
  // bounds the blocks past a million, which no workload reaches)
  const int64_t nb = (max_rows + 255) / 256;
  const int64_t lim = nb < ((int64_t)1 << 20) ? nb : ((int64_t)1 << 20);
  size_t best = 0;
  for (int64_t b = 1; b <= lim; ++b) {
    const size_t f = (size_t)3 * nsides * npieces * fwd_phases(nsides * b, tiles) * b * 256;
    best = std::max(best, f);
  }
  if (nb > lim) best = std::max(best, (size_t)3 * nsides * npieces * kMaxFwdPhases * nb * 256);
  return best;
}

void plan_options(const grpo_options* o, Plan* p) {
  grpo_options d;
  grpo_default_options(&d);
  if (!o) o = &d;
  p->kl = o->kl_estimator;
  p->detach = o->detach_ratio;
  p->norm = o->normalization;
  p->inv_tau = 1.0f / o->temperature;
  p->scale2 = kLog2e / o->temperature;
  p->fp8 = o->fp8_logits;
  p->chunk_rows = o->chunk_rows;
  p->vocab_piece = o->vocab_piece;
  p->trace_kernel = o->trace_kernel;
  p->trace_cap = o->trace_capacity;
  p->trace_ev = o->trace_events;
  p->trace_n = nullptr;  // set by the entry point that launches
  p->offload = o->dx_host != nullptr;
  p->ring = nullptr;     // set by grpo_loss_fwd_bwd for the call
}

// Events of a CopyRing (and two more for the call's own hand-overs), created for one call
// and destroyed at its end (a destroyed event still pending completes normally).
struct RingEvents {
  hipEvent_t ev[6] = {};
  hipError_t create(CopyRing* r) {
    for (hipEvent_t& e : ev) {
      const hipError_t rc = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (rc != hipSuccess) return rc;
    }
    if (r) {
      r->ready[0] = ev[0];
      r->ready[1] = ev[1];
      r->freed[0] = ev[2];
      r->freed[1] = ev[3];
    }
    return hipSuccess;
  }
  ~RingEvents() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

// `to` waits for everything enqueued on `from` so far.
hipError_t stream_after(hipStream_t to, hipStream_t from, hipEvent_t ev) {
  hipError_t e = hipEventRecord(ev, from);
  return e != hipSuccess ? e : hipStreamWaitEvent(to, ev, 0);
}

// Workspace of grpo_grad_restore: the loss-row list of S*L rows.
struct RestorePlan {
  size_t off_ntok, off_idx, off_rank, total;
};
RestorePlan restore_plan(int64_t S, int64_t L) {
  RestorePlan r;
  const int64_t N = S * L;
  size_t o = 0;
  r.off_ntok = o;
  o = align_up(o + compact_bytes(N));
  r.off_idx = o;
  o = align_up(o + (size_t)N * 4);
  r.off_rank = o;
  o = align_up(o + (size_t)N * 4);
  r.total = o;
  return r;
}

// [p, p + bytes) lies inside one allocation of pinned host memory (hipHostMalloc), which
// kernels and the copy engines reach over PCIe.  Pageable memory, or a range that runs past
// its allocation, would fault a kernel that reads it.
bool pinned_host(const void* p, size_t bytes) {
  if (!p || bytes == 0) return false;
  hipPointerAttribute_t a;
  void* start = nullptr;
  size_t size = 0;
  hipDeviceptr_t dp = const_cast<void*>(p);
  const bool ok =
      hipPointerGetAttributes(&a, p) == hipSuccess && a.type == hipMemoryTypeHost &&
      hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, dp) == hipSuccess &&
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, dp) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();  // leave no error behind for the launches' checks
    return false;
  }
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(start), q = reinterpret_cast<uintptr_t>(p);
  return q >= s0 && q - s0 <= size && bytes <= size - (q - s0);
}

}  // namespace grpo

using namespace grpo;

extern "C" {

const char* grpo_status_string(int status) {
  switch (status) {
    case GRPO_OK: return "ok";
    case GRPO_ERR_NULL: return "a required pointer is NULL";
    case GRPO_ERR_SHAPE: return "a size is out of range";
    case GRPO_ERR_DTYPE: return "unknown dtype";
    case GRPO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case GRPO_ERR_WORKSPACE: return "workspace too small";
    case GRPO_ERR_HIP: return "HIP runtime error while enqueuing";
    case GRPO_ERR_DEVICE: return "current device is not gfx950";
    case GRPO_ERR_OPTIONS: return "a loss option is out of range";
    case GRPO_ERR_SCRATCH: return "the forward needs more than the fixed scratch array holds";
    case GRPO_ERR_HOST: return "a host buffer is not pinned host memory";
    default: return "unknown status";
  }
}

void grpo_default_options(grpo_options* opts) {
  if (!opts) return;
  opts->kl_estimator = GRPO_KL_REVERSE;
  opts->detach_ratio = 1;
  opts->normalization = GRPO_NORM_TOKENS;
  opts->temperature = 1.0f;
  opts->fp8_logits = 0;
  opts->chunk_rows = 0;
  opts->vocab_piece = 0;
  opts->trace_kernel = GRPO_TRACE_NONE;
  opts->trace_capacity = 0;
  opts->trace_events = nullptr;
  opts->trace_count = nullptr;
  opts->dx_host = nullptr;
  opts->dw_host = nullptr;
  opts->copy_stream = nullptr;
}

size_t grpo_workspace_bytes(int64_t S, int64_t L, int64_t H, int64_t V, grpo_dtype dtype,
                            int need_dW) {
  return grpo_workspace_bytes_opts(S, L, H, V, dtype, need_dW, nullptr);
}

size_t grpo_workspace_bytes_opts(int64_t S, int64_t L, int64_t H, int64_t V, grpo_dtype dtype,
                                 int need_dW, const grpo_options* opts) {
  if (!options_ok(opts)) return 0;
  Plan p;
  if (!make_plan(S, L, H, V, dtype, need_dW, &p, opts)) return 0;
  return p.total;
}

int grpo_quantize_e4m3(const void* src, grpo_dtype dtype, int64_t rows, int64_t H,
                       uint8_t* dst, float* scales, grpo_stream_t stream) {
  if (!src || !dst || !scales) return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (rows < 0 || rows > INT32_MAX || H < 4 || H % 4 != 0) return GRPO_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(dst) & 3u) != 0) return GRPO_ERR_ALIGN;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  if (launch_quant_rows(dtype, src, H, nullptr, nullptr, rows, dst, scales,
                        (hipStream_t)stream) != hipSuccess)
    return GRPO_ERR_HIP;
  return GRPO_OK;
}

int grpo_advantages(const float* rewards, int64_t B, int64_t G, int64_t K, float eps,
                    int unbiased, float* adv, grpo_stream_t stream) {
  if (!rewards || !adv) return GRPO_ERR_NULL;
  if (B < 1 || G < 1 || K < 1 || (unbiased && G < 2)) return GRPO_ERR_SHAPE;
  if (G > INT32_MAX / K || B > INT64_MAX / (G * K)) return GRPO_ERR_SHAPE;
  if (!(eps >= 0.0f) || !isfinite(eps)) return GRPO_ERR_SHAPE;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  if (launch_advantages(rewards, B, G, K, eps, unbiased, adv, (hipStream_t)stream) !=
      hipSuccess)
    return GRPO_ERR_HIP;
  return GRPO_OK;
}

// The forward shared by grpo_loss_fwd and grpo_loss_fwd_noalloc.  workspace NULL: use
// this device's scratch array, which must hold the forward's part of the plan.
static int loss_fwd(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                    const int64_t* targets, const uint8_t* mask, const float* adv, int64_t S,
                    int64_t L, int64_t H, int64_t V, float beta, float* loss, float* saved,
                    float* logp_out, float* ref_logp_out, float* kl_out, int32_t* status,
                    const grpo_options* opts, void* workspace, size_t workspace_bytes,
                    grpo_stream_t stream) {
  const bool own = workspace == nullptr;
  if (!Xq || !Xp || !W || !targets || !mask || !adv || !loss || !saved || !status)
    return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (!sizes_ok(S, L, H, V) || !isfinite(beta)) return GRPO_ERR_SHAPE;
  if (!aligned16(Xq) || !aligned16(Xp) || !aligned16(W) || !aligned16(saved) ||
      !aligned16(workspace))
    return GRPO_ERR_ALIGN;
  Plan p;
  if (!options_ok(opts)) return GRPO_ERR_OPTIONS;
  if (!make_plan(S, L, H, V, dtype, 0, &p)) return GRPO_ERR_SHAPE;
  if (!make_plan(S, L, H, V, dtype, 0, &p, opts)) return GRPO_ERR_OPTIONS;
  if (own ? p.fwd_total > kScratchBytes : workspace_bytes < p.total)
    return own ? GRPO_ERR_SCRATCH : GRPO_ERR_WORKSPACE;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  hipStream_t st = (hipStream_t)stream;
  int launches = 0;  // launches of the traced kernel
  p.trace_n = &launches;
  void* ws = own ? scratch_address() : workspace;
  if (!ws) return GRPO_ERR_HIP;
  if (launch_compact_status(mask, p.N, ws_ptr<int32_t>(ws, p.off_ntok),
                            ws_ptr<int32_t>(ws, p.off_idx), ws_ptr<int32_t>(ws, p.off_rank),
                            status, st) != hipSuccess)
    return GRPO_ERR_HIP;
  if (p.norm == GRPO_NORM_SEQUENCES && launch_seq_counts(p, mask, ws, st) != hipSuccess)
    return GRPO_ERR_HIP;
  const hipError_t fe = p.mfma ? mfma_fwd_partials(p, ws, Xq, Xp, W, targets, st)
                               : simple_fwd_partials(p, ws, Xq, Xp, W, targets, st);
  if (fe != hipSuccess) return GRPO_ERR_HIP;
  if (launch_merge(p, ws, targets, mask, adv, beta, saved, logp_out, ref_logp_out, kl_out,
                   status, loss, st) != hipSuccess)
    return GRPO_ERR_HIP;
  return traced(opts, launches);
}

int grpo_loss_fwd(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                  const int64_t* targets, const uint8_t* mask, const float* adv, int64_t S,
                  int64_t L, int64_t H, int64_t V, float beta, float* loss, float* saved,
                  float* logp_out, float* ref_logp_out, float* kl_out, int32_t* status,
                  const grpo_options* opts, void* workspace, size_t workspace_bytes,
                  grpo_stream_t stream) {
  if (!workspace) return GRPO_ERR_NULL;
  return loss_fwd(Xq, Xp, W, dtype, targets, mask, adv, S, L, H, V, beta, loss, saved,
                  logp_out, ref_logp_out, kl_out, status, opts, workspace, workspace_bytes,
                  stream);
}

int grpo_loss_fwd_noalloc(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                          const int64_t* targets, const uint8_t* mask, const float* adv,
                          int64_t S, int64_t L, int64_t H, int64_t V, float beta, float* loss,
                          float* saved, float* logp_out, float* ref_logp_out, float* kl_out,
                          int32_t* status, const grpo_options* opts, grpo_stream_t stream) {
  return loss_fwd(Xq, Xp, W, dtype, targets, mask, adv, S, L, H, V, beta, loss, saved,
                  logp_out, ref_logp_out, kl_out, status, opts, nullptr, 0, stream);
}

int grpo_loss_bwd(const void* Xq, const void* W, grpo_dtype dtype, const int64_t* targets,
                  const uint8_t* mask, const float* saved, int64_t S, int64_t L, int64_t H,
                  int64_t V, const float* grad_loss, float loss_scale, void* dXq, float* dW,
                  int accumulate_dW, int32_t* found_inf, const grpo_options* opts,
                  void* workspace, size_t workspace_bytes, grpo_stream_t stream) {
  if (!Xq || !W || !targets || !mask || !saved || !dXq || !found_inf || !workspace)
    return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (!sizes_ok(S, L, H, V) || !(loss_scale > 0.0f) || !isfinite(loss_scale))
    return GRPO_ERR_SHAPE;
  if (!aligned16(Xq) || !aligned16(W) || !aligned16(saved) || !aligned16(dXq) ||
      (dW && !aligned16(dW)) || !aligned16(workspace))
    return GRPO_ERR_ALIGN;
  if (!options_ok(opts)) return GRPO_ERR_OPTIONS;
  Plan p;
  if (!make_plan(S, L, H, V, dtype, dW != nullptr, &p)) return GRPO_ERR_SHAPE;
  if (!make_plan(S, L, H, V, dtype, dW != nullptr, &p, opts)) return GRPO_ERR_OPTIONS;
  // dq/dz = (onehot - softmax(z / tau)) / tau: the 1 / tau joins the per-row factor
  // grad_loss / loss_scale as a larger divisor (exactly loss_scale at tau = 1)
  const float ls_eff = opts ? loss_scale * opts->temperature : loss_scale;
  if (!(ls_eff > 0.0f) || !isfinite(ls_eff)) return GRPO_ERR_SHAPE;
  if (workspace_bytes < p.total) return GRPO_ERR_WORKSPACE;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  hipStream_t st = (hipStream_t)stream;
  int launches = 0;  // launches of the traced kernel
  p.trace_n = &launches;
  void* ws = workspace;
  if (launch_compact(mask, p.N, ws_ptr<int32_t>(ws, p.off_ntok), ws_ptr<int32_t>(ws, p.off_idx),
                     ws_ptr<int32_t>(ws, p.off_rank), st) != hipSuccess)
    return GRPO_ERR_HIP;
  if (launch_zero_masked_rows(p, mask, dXq, st) != hipSuccess) return GRPO_ERR_HIP;
  const hipError_t be =
      p.mfma ? mfma_backward(p, ws, Xq, W, targets, saved, grad_loss, ls_eff, dXq, dW,
                             accumulate_dW, found_inf, st)
             : simple_backward(p, ws, Xq, W, targets, saved, grad_loss, ls_eff, dXq, dW,
                               accumulate_dW, found_inf, st);
  if (be != hipSuccess) return GRPO_ERR_HIP;
  return traced(opts, launches);
}

int grpo_loss_fwd_bwd(const void* Xq, const void* Xp, const void* W, grpo_dtype dtype,
                      const int64_t* targets, const uint8_t* mask, const float* adv, int64_t S,
                      int64_t L, int64_t H, int64_t V, float beta, const float* grad_loss,
                      float loss_scale, float* loss, float* saved, float* logp_out,
                      float* ref_logp_out, float* kl_out, int32_t* status, void* dXq, float* dW,
                      int accumulate_dW, int32_t* found_inf, const grpo_options* opts,
                      void* workspace, size_t workspace_bytes, grpo_stream_t stream) {
  const bool offload = opts && opts->dx_host;
  if (!Xq || !Xp || !W || !targets || !mask || !adv || !loss || !saved || !status ||
      (!dXq && !offload) || !found_inf || !workspace)
    return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (!sizes_ok(S, L, H, V) || !isfinite(beta) || !(loss_scale > 0.0f) || !isfinite(loss_scale))
    return GRPO_ERR_SHAPE;
  if (!aligned16(Xq) || !aligned16(Xp) || !aligned16(W) || !aligned16(saved) ||
      !aligned16(dXq) || (dW && !aligned16(dW)) || !aligned16(workspace))
    return GRPO_ERR_ALIGN;
  if (!options_ok(opts)) return GRPO_ERR_OPTIONS;
  // the offload writes no device dX, and dW goes to the host only from a device dW
  if ((offload && dXq) || (opts && opts->dw_host && !dW) ||
      (opts && (opts->dx_host || opts->dw_host) && opts->copy_stream == stream))
    return GRPO_ERR_OPTIONS;
  Plan p;
  if (!make_plan(S, L, H, V, dtype, dW != nullptr, &p)) return GRPO_ERR_SHAPE;
  if (!make_plan(S, L, H, V, dtype, dW != nullptr, &p, opts)) return GRPO_ERR_OPTIONS;
  const float ls_eff = opts ? loss_scale * opts->temperature : loss_scale;
  if (!(ls_eff > 0.0f) || !isfinite(ls_eff)) return GRPO_ERR_SHAPE;
  if (workspace_bytes < p.total) return GRPO_ERR_WORKSPACE;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  if ((offload && !pinned_host(opts->dx_host, (size_t)p.N * H * p.esize)) ||
      (opts && opts->dw_host && !pinned_host(opts->dw_host, (size_t)V * H * 4)))
    return GRPO_ERR_HOST;
  hipStream_t st = (hipStream_t)stream;
  int launches = 0;  // launches of the traced kernel
  p.trace_n = &launches;
  void* ws = workspace;
  // gradient offload: the staging ring and its events
  const bool host_copies = opts && (opts->dx_host || opts->dw_host);
  hipStream_t cs = host_copies ? (hipStream_t)opts->copy_stream : nullptr;
  CopyRing ring;
  RingEvents evs;
  if (host_copies) {
    if (evs.create(&ring) != hipSuccess) return GRPO_ERR_HIP;
    if (offload) {
      ring.slots = ws_ptr<char>(ws, p.off_ring);
      ring.host = reinterpret_cast<char*>(opts->dx_host);
      ring.row_bytes = (size_t)H * p.esize;
      ring.rows = p.R;
      ring.total = p.N;
      ring.st = st;
      ring.cs = cs;
      p.ring = &ring;
    }
  }
  if (launch_compact_status(mask, p.N, ws_ptr<int32_t>(ws, p.off_ntok),
                            ws_ptr<int32_t>(ws, p.off_idx), ws_ptr<int32_t>(ws, p.off_rank),
                            status, st) != hipSuccess)
    return GRPO_ERR_HIP;
  if (p.norm == GRPO_NORM_SEQUENCES && launch_seq_counts(p, mask, ws, st) != hipSuccess)
    return GRPO_ERR_HIP;
  if (!offload && launch_zero_masked_rows(p, mask, dXq, st) != hipSuccess) return GRPO_ERR_HIP;
  if (p.mfma) {
    if (mfma_fused(p, ws, Xq, Xp, W, targets, mask, adv, beta, saved, logp_out, ref_logp_out,
                   kl_out, status, loss, grad_loss, ls_eff, dXq, dW, accumulate_dW, found_inf,
                   st) != hipSuccess)
      return GRPO_ERR_HIP;
  } else {
    // fp32 (or H not a multiple of 256): the two passes back to back
    if (simple_fwd_partials(p, ws, Xq, Xp, W, targets, st) != hipSuccess) return GRPO_ERR_HIP;
    if (launch_merge(p, ws, targets, mask, adv, beta, saved, logp_out, ref_logp_out, kl_out,
                     status, loss, st) != hipSuccess)
      return GRPO_ERR_HIP;
    if (simple_backward(p, ws, Xq, W, targets, saved, grad_loss, ls_eff, dXq, dW, accumulate_dW,
                        found_inf, st) != hipSuccess)
      return GRPO_ERR_HIP;
  }
  if (host_copies) {
    if (opts->dw_host) {
      if (stream_after(cs, st, evs.ev[4]) != hipSuccess ||
          copy_to_host(opts->dw_host, dW, (size_t)H * 4, (size_t)V, cs) != hipSuccess)
        return GRPO_ERR_HIP;
    }
    if (stream_after(st, cs, evs.ev[5]) != hipSuccess) return GRPO_ERR_HIP;
  }
  return traced(opts, launches);
}

int grpo_scale_grad(void* dXq, grpo_dtype dtype, int64_t rows, int64_t H, float* dW, int64_t V,
                    const float* grad_loss, float loss_scale, int32_t* found_inf,
                    grpo_stream_t stream) {
  if (!dXq || !grad_loss || !found_inf) return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (rows < 0 || H < 1 || H % 8 != 0 || (dW && V < 1) || !(loss_scale > 0.0f) ||
      !isfinite(loss_scale))
    return GRPO_ERR_SHAPE;
  if (!aligned16(dXq) || (dW && !aligned16(dW))) return GRPO_ERR_ALIGN;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  if (launch_scale_grad(dXq, dtype, rows * H, dW, dW ? V * H : 0, grad_loss, loss_scale,
                        found_inf, (hipStream_t)stream) != hipSuccess)
    return GRPO_ERR_HIP;
  return GRPO_OK;
}

size_t grpo_restore_workspace_bytes(int64_t S, int64_t L) {
  if (S < 1 || L < 1 || S > INT32_MAX / L) return 0;
  return restore_plan(S, L).total;
}

int grpo_grad_restore(const void* dx_host, const float* dw_host, grpo_dtype dtype,
                      const uint8_t* mask, int64_t S, int64_t L, int64_t H, int64_t V,
                      const float* grad_loss, float loss_scale, void* dXq, float* dW,
                      int32_t* found_inf, void* workspace, size_t workspace_bytes,
                      grpo_stream_t stream) {
  if (!found_inf || (!dx_host != !dXq) || (!dw_host != !dW) || (!dx_host && !dw_host) ||
      (dx_host && (!mask || !workspace)))
    return GRPO_ERR_NULL;
  if (!valid_dtype(dtype)) return GRPO_ERR_DTYPE;
  if (!sizes_ok(S, L, H, dW ? V : 1) || !(loss_scale > 0.0f) || !isfinite(loss_scale))
    return GRPO_ERR_SHAPE;
  if (!aligned16(dx_host) || !aligned16(dw_host) || !aligned16(dXq) || !aligned16(dW) ||
      !aligned16(workspace))
    return GRPO_ERR_ALIGN;
  const RestorePlan rp = restore_plan(S, L);
  if (dx_host && workspace_bytes < rp.total) return GRPO_ERR_WORKSPACE;
  if (!device_ok()) return GRPO_ERR_DEVICE;
  const int64_t N = S * L;
  const size_t esize = dtype == GRPO_F32 ? 4 : 2;
  if ((dx_host && !pinned_host(dx_host, (size_t)N * H * esize)) ||
      (dw_host && !pinned_host(dw_host, (size_t)V * H * 4)))
    return GRPO_ERR_HOST;
  hipStream_t st = (hipStream_t)stream;
  if (dx_host) {
    int32_t* ntok = ws_ptr<int32_t>(workspace, rp.off_ntok);
    int32_t* idx = ws_ptr<int32_t>(workspace, rp.off_idx);
    Plan p;
    memset(&p, 0, sizeof(p));
    p.N = N;
    p.H = H;
    p.esize = (int)esize;
    if (launch_compact(mask, N, ntok, idx, ws_ptr<int32_t>(workspace, rp.off_rank), st) !=
            hipSuccess ||
        launch_zero_masked_rows(p, mask, dXq, st) != hipSuccess ||
        launch_restore_rows(dtype, dx_host, N, H, ntok, idx, grad_loss, loss_scale, dXq,
                            found_inf, st) != hipSuccess)
      return GRPO_ERR_HIP;
  }
  if (dw_host && launch_restore_rows(GRPO_F32, dw_host, V, H, nullptr, nullptr, grad_loss,
                                     loss_scale, dW, found_inf, st) != hipSuccess)
    return GRPO_ERR_HIP;
  return GRPO_OK;
}

}  // extern "C"
