// Host layer of the C ABI declared in include/lla.h: argument validation
// (before anything is enqueued), the context-split plan, workspace layout,
// and dispatch of the gfx950 kernels on the caller's stream.
#include "lla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "lla_internal.h"

namespace {

using namespace lla;

constexpr int kMaxHeadDim = 256;
constexpr int kMaxLatent = 16384;     // r_k + r_v limit of the general kernels
constexpr int kMaxWindow = 8192;
constexpr int kTargetWorkgroups = 256;  // one per compute unit on MI355X (256 CUs)
constexpr int kLongSplit = 768;         // tokens per split above which the absorbed scan fills every CU

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const lla_set_desc& d) { return d.dtype == LLA_BF16 ? 2 : 4; }

lla_status check_desc(const lla_set_desc* d) {
  if (!d) return LLA_ERR_INVALID_ARGUMENT;
  if (d->n_heads <= 0 || d->head_dim <= 0 || (d->head_dim & 1)) return LLA_ERR_INVALID_ARGUMENT;
  if (d->groups <= 0 || d->n_heads % d->groups) return LLA_ERR_INVALID_ARGUMENT;
  if (d->r_k <= 0 || d->r_v <= 0 || d->r_k % kTile || d->r_v % kTile) return LLA_ERR_INVALID_ARGUMENT;
  if (d->loop_first < 1 || d->loop_last < d->loop_first) return LLA_ERR_INVALID_ARGUMENT;
  if (d->page_size <= 0 || d->page_size % kTile) return LLA_ERR_INVALID_ARGUMENT;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16) return LLA_ERR_INVALID_ARGUMENT;
  if (!(d->rope_base >= 0.f) || !std::isfinite(d->rope_base)) return LLA_ERR_INVALID_ARGUMENT;
  if (d->rope_baked != 0 && d->rope_baked != 1) return LLA_ERR_INVALID_ARGUMENT;
  if (d->rope_baked && d->rope_base == 0.f) return LLA_ERR_INVALID_ARGUMENT;
  if (d->rope_baked && d->r_k % d->head_dim) return LLA_ERR_UNSUPPORTED;
  if (d->head_dim > kMaxHeadDim) return LLA_ERR_UNSUPPORTED;
  if (d->r_k + d->r_v > kMaxLatent) return LLA_ERR_UNSUPPORTED;
  if (d->latent_fp8 != 0 && d->latent_fp8 != 1) return LLA_ERR_INVALID_ARGUMENT;
  if (d->latent_fp8 && d->dtype != LLA_BF16) return LLA_ERR_INVALID_ARGUMENT;
  if (d->latent_fp8 && (d->r_k % 64 || d->r_v % 64)) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

lla_status check_store(const lla_store* s) {
  if (!s || !s->pages || !s->block_table || s->max_pages_per_seq <= 0) return LLA_ERR_INVALID_ARGUMENT;
  if (!aligned16(s->pages)) return LLA_ERR_INVALID_ARGUMENT;
  return LLA_OK;
}

// ---------------------------------------------------------------- split plan
struct Plan {
  int S;
  int chunk;
};

// Latent tokens of the longest sequence are cut into S contiguous ranges of
// `chunk` tokens (a multiple of 64); `wgs` workgroups work on each
// (sequence, range).  S aims at kTargetWorkgroups in flight.
Plan make_plan(int batch, int max_pos, int window, int splits, int wgs, int target = kTargetWorkgroups,
               int gran = kChunk, int cap = 1 << 30) {
  const int64_t n_lat = std::max<int64_t>(0, (int64_t)max_pos - window);
  const int64_t tiles = std::max<int64_t>(1, (n_lat + gran - 1) / gran);
  int64_t S = splits > 0 ? splits
                         : std::min<int64_t>(cap, (target + (int64_t)batch * wgs - 1) / ((int64_t)batch * wgs));
  S = std::min<int64_t>(std::max<int64_t>(S, 1), tiles);
  const int64_t per = (tiles + S - 1) / S;
  S = (tiles + per - 1) / per;
  return Plan{(int)S, (int)(per * gran)};
}

// max_pages: columns of the store's block table, or 0 for the store-free
// queries (workspace size, split plan, kernel name), which assume a table
// within every matrix-core kernel's LDS page table
bool use_mfma_scan(const lla_set_desc& d, int flags, int max_pages = 0) {
  if (flags & LLA_FLAG_GENERIC) return false;
  if (d.dtype != LLA_BF16) return false;
  DecodeParams p{};
  p.hpg = d.n_heads / d.groups;
  p.rk = d.r_k;
  p.rv = d.r_v;
  p.dh = d.head_dim;
  p.bf16 = 1;
  p.fp8 = d.latent_fp8;
  p.max_pages = max_pages;
  return scan_absorbed_mfma_supports(p);
}

// the two-pass scan of one wide latent shared by all heads, for the bf16
// shapes the one-pass matrix-core scan does not cover
bool use_wide_scan(const lla_set_desc& d, int flags) {
  if (flags & (LLA_FLAG_GENERIC | LLA_FLAG_FUSED)) return false;
  if (d.dtype != LLA_BF16 || use_mfma_scan(d, flags)) return false;
  DecodeParams p{};
  p.B = 1; p.H = d.n_heads; p.G = d.groups; p.hpg = d.n_heads / d.groups;
  p.rk = d.r_k; p.rv = d.r_v; p.dh = d.head_dim;
  p.bf16 = 1;
  p.fp8 = d.latent_fp8;
  return scan_absorbed_wide_supports(p);
}

bool use_mfma_reconstruct(const lla_set_desc& d, int flags, int max_pages = 0) {
  if (flags & LLA_FLAG_GENERIC) return false;
  DecodeParams p{};
  p.hpg = d.n_heads / d.groups;
  p.rk = d.r_k;
  p.rv = d.r_v;
  p.dh = d.head_dim;
  p.bf16 = d.dtype == LLA_BF16;
  p.max_pages = max_pages;
  return scan_reconstruct_mfma_supports(p);
}

bool use_gemm_reconstruct(const lla_set_desc& d, int flags) {
  if (flags & LLA_FLAG_GENERIC) return false;
  DecodeParams p{};
  p.G = d.groups;
  p.rk = d.r_k;
  p.rv = d.r_v;
  p.dh = d.head_dim;
  p.bf16 = d.dtype == LLA_BF16;
  return scan_reconstruct_gemm_supports(p);
}

bool fused_shape(const lla_set_desc& d) {
  DecodeParams p{};
  p.bf16 = d.dtype == LLA_BF16;
  p.fp8 = d.latent_fp8;
  p.rk = d.r_k;
  p.rv = d.r_v;
  p.dh = d.head_dim;
  return fused_decode_supports(p);
}

constexpr int kValidFlags = LLA_FLAG_GENERIC | LLA_FLAG_FUSED;

bool flags_ok(int flags) {
  return !(flags & ~kValidFlags) && (flags & kValidFlags) != kValidFlags;
}

// The latent-scan kernel family of one decode call.  Every decision that
// depends on it (split plan, workspace layout, launches, the name reported to
// profilers) goes through this one choice.
enum class Scan {
  kFused, kAbsorbedMfma, kAbsorbedWide, kAbsorbedGeneric, kReconstructMfma, kReconstructGemm,
  kReconstructGeneric
};

// max_pages > 0: the call's store has a block table of that many columns
// (and max_pos_hint is the call's): a table longer than a matrix-core scan's
// LDS page table, or covering more tokens than the wide scan's score rows,
// takes the general scan.  max_pages == 0: the store-free queries.
Scan choose_scan(const lla_set_desc& d, bool absorbed, int flags, int max_pages = 0, int max_pos_hint = 0) {
  if (absorbed) {
    if (flags & LLA_FLAG_FUSED) return Scan::kFused;
    if (use_mfma_scan(d, flags)) return use_mfma_scan(d, flags, max_pages) ? Scan::kAbsorbedMfma
                                                                             : Scan::kAbsorbedGeneric;
    if (use_wide_scan(d, flags)) {
      if (max_pages <= 0) return Scan::kAbsorbedWide;
      const int lcap = scan_absorbed_wide_lcap(max_pos_hint);
      const bool rows_cover = (int64_t)max_pages * d.page_size <= lcap && max_pages <= kWideMaxPages;
      return rows_cover ? Scan::kAbsorbedWide : Scan::kAbsorbedGeneric;
    }
    return Scan::kAbsorbedGeneric;
  }
  if (use_mfma_reconstruct(d, flags))
    return use_mfma_reconstruct(d, flags, max_pages) ? Scan::kReconstructMfma : Scan::kReconstructGeneric;
  if (use_gemm_reconstruct(d, flags)) return Scan::kReconstructGemm;
  return Scan::kReconstructGeneric;
}

const char* scan_kernel_name(Scan k) {
  switch (k) {
    case Scan::kFused: return "k_fused_decode";
    case Scan::kAbsorbedMfma: return "k_scan_absorbed_mfma";
    case Scan::kAbsorbedWide: return "k_scan_absorbed_wide";
    case Scan::kAbsorbedGeneric: return "k_scan_absorbed_generic";
    case Scan::kReconstructMfma: return "k_scan_reconstruct_mfma";
    case Scan::kReconstructGemm: return "k_scan_reconstruct_gemm";
    case Scan::kReconstructGeneric: return "k_scan_reconstruct_generic";
  }
  return "k_scan_absorbed_generic";
}

Plan plan_for(const lla_set_desc& d, int batch, int max_pos, int window, int splits, Scan k) {
  int wgs = d.n_heads;                                  // general kernels: one per head
  int target = kTargetWorkgroups;
  int gran = kChunk;
  switch (k) {
    case Scan::kFused: {
      target = 2 * kTargetWorkgroups;   // small workgroups: a few resident per CU
      const Plan pl = make_plan(batch, max_pos, window, splits, wgs, target, kChunk);
      if (pl.S <= kMaxFusedSplits) return pl;
      return make_plan(batch, max_pos, window, kMaxFusedSplits, wgs, target, kChunk);
    }
    case Scan::kAbsorbedMfma: {
      // One workgroup per CU when that still leaves a split at least
      // kLongSplit tokens (the launch then keeps every CU busy and loads its
      // tiles as streaming), else three quarters of one per CU with cached
      // loads.  Measured per call at the HLA shapes, 192 against 256
      // workgroups: batch 32 at 16k 198.7 / 189.1 us, batch 64 at 4k 120.6 /
      // 111.5 us, batch 32 at 4k 68.7 / 68.1 us, batch 16 at 4k 45.6 / 47.1 us;
      // batch 128 at 4k takes 2 splits either way.  The matrix-core combine
      // merges at most kCombineMaxParts splits + window slices (one window
      // slice per split when the scan takes the window along).
      const Plan full = make_plan(batch, max_pos, window, splits, d.groups, kTargetWorkgroups, kChunk,
                                  kCombineMaxParts / 2);
      if (splits > 0 || full.chunk >= kLongSplit) return full;
      return make_plan(batch, max_pos, window, splits, d.groups, 3 * kTargetWorkgroups / 4, kChunk,
                       kCombineMaxParts / 2);
    }
    case Scan::kAbsorbedWide:
      // the value pass runs one workgroup per (256-dim slab, split, sequence)
      return make_plan(batch, max_pos, window, splits, scan_absorbed_wide_slabs(d.r_v), target, kChunk,
                       kCombineMaxParts / 2);
    case Scan::kReconstructMfma:
      wgs = d.n_heads;                    // one head per workgroup
      target = 2 * kTargetWorkgroups;   // small workgroups: two resident per CU
      break;
    case Scan::kReconstructGemm:
      wgs = (d.n_heads + 1) / 2;          // two heads per workgroup
      gran = scan_reconstruct_gemm_tile(d.head_dim);
      break;
    default:
      break;
  }
  return make_plan(batch, max_pos, window, splits, wgs, target, gran);
}

struct WsLayout {
  size_t qlat, qhead, part_ml, part_o, win_ml, win_o, dect, wscore, wprob, tickets, fpart, total;
  bool has_dect;
};

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kWindowSlice = 32;   // exact tokens per window slice (fast window kernel)

int window_slices(int window) { return (window + 1 + kWindowSlice - 1) / kWindowSlice; }

// lcap > 0: the two-pass wide scan's score and probability rows of lcap tokens
WsLayout ws_layout(const lla_set_desc& d, int B, int S, int WS, int Dp, bool fused = false, int lcap = 0) {
  WsLayout w{};
  const size_t H = d.n_heads, dh = d.head_dim;
  size_t off = 0;
  if (fused) {   // tickets and the splits' partials only
    w.tickets = off; off = up256(off + (size_t)B * H * 4);
    w.fpart = off;   off = up256(off + (size_t)B * H * S * fused_partial_floats(d.r_k, d.head_dim) * 4);
    w.total = off;
    return w;
  }
  // (the two-pass scan of a wide latent keeps q~ as bf16 hi and lo parts)
  w.qlat = off;    off = up256(off + (size_t)B * H * d.r_k * elem_bytes(d) * (lcap > 0 ? 2 : 1));
  w.qhead = off;   off = up256(off + (size_t)B * H * dh * 4);
  w.part_ml = off; off = up256(off + (size_t)B * S * H * 2 * 4);
  w.part_o = off;  off = up256(off + (size_t)B * S * H * Dp * 4);
  w.win_ml = off;  off = up256(off + (size_t)B * WS * H * 2 * 4);
  w.win_o = off;   off = up256(off + (size_t)B * WS * H * dh * 4);
  // head-folded reconstruct: A_t and B_t^T regrouped per K step
  w.has_dect = scan_reconstruct_gemm_tiles_decoders(d.head_dim, d.groups, d.r_k, d.r_v, d.dtype == LLA_BF16);
  if (w.has_dect) {
    w.dect = off;  off = up256(off + (size_t)2 * H * dh * d.r_k * 2);
  }
  if (lcap > 0) {
    w.wscore = off; off = up256(off + (size_t)scan_absorbed_wide_ksplit(B, lcap, d.r_k) * B * H * lcap * 4);
    w.wprob = off;  off = up256(off + (size_t)B * H * lcap * 2);
  }
  w.total = off;
  return w;
}

// width of a latent-scan partial row: latent space (r_v) for the absorbed
// read, head space (d_h) when keys and values are rebuilt
int partial_width(const lla_set_desc& d, int entry) { return entry ? d.r_v : d.head_dim; }

size_t decode_ws_bytes(const lla_set_desc& d, int batch, int max_pos, int window, int splits) {
  // enough for every entry point and kernel family at these sizes
  // (the general kernels, which a store too long for a matrix-core kernel
  // falls back to, are the LLA_FLAG_GENERIC choices)
  size_t best = 0;
  for (int entry = 0; entry < 2; ++entry)
    for (int flags = 0; flags < 2; ++flags) {
      const Scan k = choose_scan(d, entry != 0, flags);
      const int S = plan_for(d, batch, max_pos, window, splits, k).S;
      const int lcap = k == Scan::kAbsorbedWide ? scan_absorbed_wide_lcap(max_pos) : 0;
      best = std::max(best, ws_layout(d, batch, S, std::max(S, window_slices(window)),
                                      partial_width(d, entry), false, lcap).total);
    }
  if (fused_shape(d)) {
    const int S = plan_for(d, batch, max_pos, window, splits, Scan::kFused).S;
    best = std::max(best, ws_layout(d, batch, S, S, d.r_v, true).total);
  }
  return best;
}

lla_status hip_status(hipError_t e) { return e == hipSuccess ? LLA_OK : LLA_ERR_HIP; }

// ---------------------------------------------------------------- full cache
lla_status check_kv_desc(const lla_kv_desc* d) {
  if (!d) return LLA_ERR_INVALID_ARGUMENT;
  if (d->n_heads <= 0 || d->head_dim <= 0 || (d->head_dim & 1)) return LLA_ERR_INVALID_ARGUMENT;
  if (d->page_size <= 0 || d->page_size % 8) return LLA_ERR_INVALID_ARGUMENT;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16) return LLA_ERR_INVALID_ARGUMENT;
  if (!(d->rope_base >= 0.f) || !std::isfinite(d->rope_base)) return LLA_ERR_INVALID_ARGUMENT;
  if (d->head_dim != 64 && d->head_dim != 128) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

Plan full_plan(const lla_kv_desc& d, int batch, int max_pos, int splits) {
  const int hpb = full_scan_heads_per_block(d.head_dim);
  return make_plan(batch, max_pos, 0, splits, (d.n_heads + hpb - 1) / hpb);
}

struct FullWs {
  size_t part_ml, part_o, total;
};

FullWs full_ws_layout(const lla_kv_desc& d, int B, int S) {
  FullWs w{};
  const size_t H = d.n_heads;
  w.part_ml = 0;
  w.part_o = up256((size_t)B * S * H * 2 * 4);
  w.total = up256(w.part_o + (size_t)B * S * H * d.head_dim * 4);
  return w;
}


// ---------------------------------------------------------------- parallel pass
lla_status check_parallel_desc(const lla_set_desc* d) {
  lla_status r = check_desc(d);
  if (r != LLA_OK) return r;
  if (d->dtype != LLA_BF16 || d->latent_fp8) return LLA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return LLA_ERR_UNSUPPORTED;
  if (d->r_k % 32 || d->r_v % 32) return LLA_ERR_UNSUPPORTED;
  if (d->rope_base > 0.f && !d->rope_baked) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

int parallel_pad(int n_max) { return (n_max + kParQueryTile - 1) / kParQueryTile * kParQueryTile; }

struct ParWs {
  size_t sk, sv, rtab, kh, vh, total;
};

ParWs parallel_ws_layout(const lla_set_desc& d, int B, int n_max) {
  ParWs w{};
  const size_t np = parallel_pad(n_max), H = d.n_heads, dh = d.head_dim, G = d.groups;
  const size_t head_rows = (size_t)B * np * H * dh * 2;
  size_t off = 0;
  w.sk = off;  off = up256(off + (size_t)B * np * G * d.r_k * 2);
  w.sv = off;  off = up256(off + (size_t)B * np * G * d.r_v * 2);
  w.rtab = off;  off = up256(off + np * (dh / 2) * 8);
  w.kh = off;  off = up256(off + head_rows);
  w.vh = off;  off = up256(off + head_rows);
  w.total = off;
  return w;
}

lla_status decode(const lla_set_desc* d, const lla_store* st, int32_t batch,
                  const lla_decode_args* a, lla_stream_t stream, int entry) {
  // entry: 0 reconstruct, 1 absorbed (LLA-D), 2 HLA windowed
  lla_status r = check_desc(d);
  if (r != LLA_OK) return r;
  if ((r = check_store(st)) != LLA_OK) return r;
  if (batch <= 0 || !a) return LLA_ERR_INVALID_ARGUMENT;
  if (a->loop < d->loop_first || a->loop > d->loop_last) return LLA_ERR_INVALID_ARGUMENT;
  if (a->window < 0 || a->max_pos_hint < 0 || a->splits < 0) return LLA_ERR_INVALID_ARGUMENT;
  if (!flags_ok(a->flags)) return LLA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a->pos, a->q, a->k_cur, a->v_cur, a->ring_k, a->ring_v, a->A, a->B, a->out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LLA_ERR_INVALID_ARGUMENT;
  if (entry == 2 && d->groups != 1) return LLA_ERR_INVALID_ARGUMENT;
  if (entry == 0 && d->latent_fp8) return LLA_ERR_UNSUPPORTED;   // fp8 latents: absorbed read only
  const bool fused = (a->flags & LLA_FLAG_FUSED) != 0;
  if (fused && (entry == 0 || !fused_shape(*d))) return LLA_ERR_UNSUPPORTED;
  if (a->window > kMaxWindow) return LLA_ERR_UNSUPPORTED;
  if (d->rope_base > 0.f && !d->rope_baked) return LLA_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(*d, batch, a->max_pos_hint, a->window, a->splits);
  if (!a->workspace || a->workspace_bytes < need) return LLA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(a->workspace)) return LLA_ERR_INVALID_ARGUMENT;

  const bool absorbed = entry != 0;
  const bool generic = (a->flags & LLA_FLAG_GENERIC) != 0;
  // the wide scan keeps a score row per (sequence, head) covering every
  // latent token the store can hold, and the matrix-core scans stage the
  // split's page ids in LDS: a store beyond either takes the general scan
  const Scan kind = choose_scan(*d, absorbed, a->flags, st->max_pages_per_seq, a->max_pos_hint);
  const Plan plan = plan_for(*d, batch, a->max_pos_hint, a->window, a->splits, kind);
  const int Dp = partial_width(*d, absorbed ? 1 : 0);
  const int WSmax = window_slices(a->window);
  const bool wide_scan = kind == Scan::kAbsorbedWide;
  const int lcap = wide_scan ? scan_absorbed_wide_lcap(a->max_pos_hint) : 0;
  const WsLayout w = ws_layout(*d, batch, plan.S, std::max(plan.S, WSmax), Dp, fused, lcap);
  char* ws = static_cast<char*>(a->workspace);

  DecodeParams p{};
  p.B = batch; p.H = d->n_heads; p.dh = d->head_dim; p.G = d->groups; p.hpg = d->n_heads / d->groups;
  p.rk = d->r_k; p.rv = d->r_v; p.P = d->page_size; p.W = a->window;
  p.S = plan.S; p.chunk = plan.chunk; p.Dp = Dp; p.max_pages = st->max_pages_per_seq;
  p.mode = absorbed ? kAbsorbed : kReconstruct;
  p.bf16 = d->dtype == LLA_BF16;
  p.fp8 = d->latent_fp8;
  p.rope_base = d->rope_base;
  p.scale = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
  p.pos = a->pos; p.bt = st->block_table; p.pages = st->pages;
  p.q = a->q; p.k_cur = a->k_cur; p.v_cur = a->v_cur; p.ring_k = a->ring_k; p.ring_v = a->ring_v;
  p.A = a->A; p.Bm = a->B; p.out = a->out;
  p.qlat = ws + w.qlat;
  p.qhead = reinterpret_cast<float*>(ws + w.qhead);
  p.part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  p.part_o = reinterpret_cast<float*>(ws + w.part_o);
  p.win_ml = reinterpret_cast<float*>(ws + w.win_ml);
  p.win_o = reinterpret_cast<float*>(ws + w.win_o);
  p.dect = w.has_dect ? ws + w.dect : nullptr;
  if (wide_scan) {
    p.lcap = lcap;
    p.wsplit = scan_absorbed_wide_ksplit(batch, lcap, d->r_k);
    p.wscore = reinterpret_cast<float*>(ws + w.wscore);
    p.wprob = ws + w.wprob;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(a->scan_events);
  if (fused) {
    p.tickets = reinterpret_cast<int32_t*>(ws + w.tickets);
    p.fpart = reinterpret_cast<float*>(ws + w.fpart);
    p.tw = (a->window + 1 + plan.S - 1) / plan.S;
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e == hipSuccess) e = launch_fused_decode(p, s);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
    return hip_status(e);
  }
  if (kind == Scan::kReconstructMfma) {
    // one kernel does the query rotation, the latent scan and the exact
    // window (split s takes window slice s); then the split merge
    p.fuse_window = 1;
    p.WS = 0;
    p.tw = (a->window + 1 + plan.S - 1) / plan.S;
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e == hipSuccess) e = launch_scan_reconstruct_mfma(p, s);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
    if (e == hipSuccess) e = launch_combine(p, s);
    return hip_status(e);
  }
  const bool mfma_scan = kind == Scan::kAbsorbedMfma;
  const bool fast_window = !generic && window_fast_supports(p);
  // the matrix-core scan takes the window along when its group's heads fit
  // one workgroup (thread per 8 dims of a head)
  p.fuse_window = (mfma_scan && fast_window && p.hpg * (p.dh / 8) <= 256) ? 1 : 0;
  if (p.fuse_window) {
    p.WS = plan.S;
    p.tw = (a->window + 1 + plan.S - 1) / plan.S;
  } else {
    p.tw = fast_window ? kWindowSlice : a->window + 1;
    p.WS = fast_window ? WSmax : 1;
  }
  p.need_qhead = (!fast_window || !absorbed) ? 1 : 0;
  const bool wide_maps = wide_scan && maps_wide_supports(p);
  p.part_bf16 = wide_maps ? 1 : 0;
  hipError_t e = wide_maps                                ? launch_qmap_wide(p, s)
                 : (!generic && qmap_mfma_supports(p)) ? launch_qmap_mfma(p, absorbed, s)
                                                       : launch_qmap(p, absorbed, s);
  if (e == hipSuccess && !p.fuse_window) e = fast_window ? launch_window_fast(p, s) : launch_window(p, s);
  if (e == hipSuccess && kind == Scan::kReconstructGemm) e = launch_scan_reconstruct_gemm_prep(p, s);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[0], s);
  if (e == hipSuccess) {
    switch (kind) {
      case Scan::kReconstructMfma: e = launch_scan_reconstruct_mfma(p, s); break;
      case Scan::kReconstructGemm: e = launch_scan_reconstruct_gemm(p, s); break;
      case Scan::kReconstructGeneric: e = launch_scan_reconstruct_generic(p, s); break;
      case Scan::kAbsorbedMfma: e = launch_scan_absorbed_mfma(p, s); break;
      case Scan::kAbsorbedWide: e = launch_scan_absorbed_wide(p, s); break;
      default: e = launch_scan_absorbed_generic(p, s); break;
    }
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
  if (e == hipSuccess)
    e = wide_maps                                  ? launch_combine_wide(p, s)
        : (!generic && combine_mfma_supports(p)) ? launch_combine_mfma(p, s)
                                                 : launch_combine(p, s);
  return hip_status(e);
}

}  // namespace

extern "C" {

lla_status lla_write_latents(const lla_set_desc* desc, const lla_store* store, int32_t batch,
                             int32_t n_tok, const int32_t* pos, const void* x, int32_t d_in,
                             const void* enc, void* workspace, size_t workspace_bytes,
                             lla_stream_t stream) {
  lla_status r = check_desc(desc);
  if (r != LLA_OK) return r;
  if ((r = check_store(store)) != LLA_OK) return r;
  if (batch <= 0 || n_tok <= 0 || d_in <= 0) return LLA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {pos, x, enc};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LLA_ERR_INVALID_ARGUMENT;
  const size_t need = lla_write_workspace_bytes(desc, batch, n_tok, d_in);
  if (need > 0 && (!workspace || workspace_bytes < need)) return LLA_ERR_WORKSPACE_TOO_SMALL;
  if (workspace && !aligned16(workspace)) return LLA_ERR_INVALID_ARGUMENT;

  WriterParams p{};
  p.B = batch; p.n_tok = n_tok; p.n_loops = desc->loop_last - desc->loop_first + 1;
  p.G = desc->groups; p.rk = desc->r_k; p.rv = desc->r_v; p.R = desc->r_k + desc->r_v;
  p.d_in = d_in; p.P = desc->page_size; p.dh = desc->head_dim;
  p.max_pages = store->max_pages_per_seq;
  p.rope_baked = desc->rope_baked; p.bf16 = desc->dtype == LLA_BF16; p.rope_base = desc->rope_base;
  p.fp8 = desc->latent_fp8;
  p.pos = pos; p.bt = store->block_table; p.pages = store->pages; p.x = x; p.enc = enc;
  p.acc = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (writer_mfma_supports(p)) {
    p.ksplit = writer_mfma_ksplit(batch * n_tok, p.G, p.R, p.n_loops, d_in);
    return hip_status(launch_writer_mfma(p, s));
  }
  p.ksplit = 1;
  return hip_status(launch_writer_generic(p, s));
}

size_t lla_write_workspace_bytes(const lla_set_desc* desc, int32_t batch, int32_t n_tok, int32_t d_in) {
  if (check_desc(desc) != LLA_OK || batch <= 0 || n_tok <= 0 || d_in <= 0) return 0;
  WriterParams p{};
  p.bf16 = desc->dtype == LLA_BF16;
  p.d_in = d_in;
  if (!writer_mfma_supports(p)) return 0;
  const int R = desc->r_k + desc->r_v, n_loops = desc->loop_last - desc->loop_first + 1;
  const int ks = writer_mfma_ksplit(batch * n_tok, desc->groups, R, n_loops, d_in);
  return (size_t)ks * batch * n_tok * desc->groups * R * sizeof(float);
}

lla_status lla_decode_reconstruct(const lla_set_desc* desc, const lla_store* store, int32_t batch,
                                  const lla_decode_args* args, lla_stream_t stream) {
  return decode(desc, store, batch, args, stream, 0);
}

lla_status lla_decode_absorbed(const lla_set_desc* desc, const lla_store* store, int32_t batch,
                               const lla_decode_args* args, lla_stream_t stream) {
  return decode(desc, store, batch, args, stream, 1);
}

lla_status hla_decode_windowed(const lla_set_desc* desc, const lla_store* store, int32_t batch,
                               const lla_decode_args* args, lla_stream_t stream) {
  return decode(desc, store, batch, args, stream, 2);
}

size_t lla_decode_workspace_bytes(const lla_set_desc* desc, int32_t batch, int32_t max_pos,
                                  int32_t window, int32_t splits) {
  if (check_desc(desc) != LLA_OK || batch <= 0 || max_pos < 0 || window < 0 || splits < 0) return 0;
  return decode_ws_bytes(*desc, batch, max_pos, window, splits);
}

int32_t lla_decode_plan_splits(const lla_set_desc* desc, int32_t batch, int32_t max_pos,
                               int32_t window, int32_t splits, int32_t entry) {
  if (check_desc(desc) != LLA_OK || batch <= 0 || max_pos < 0 || window < 0 || splits < 0) return 0;
  return plan_for(*desc, batch, max_pos, window, splits, choose_scan(*desc, entry != 0, 0)).S;
}

const char* lla_decode_scan_kernel(const lla_set_desc* desc, int32_t entry, int32_t flags) {
  if (check_desc(desc) != LLA_OK || entry < 0 || entry > 2 || !flags_ok(flags)) return nullptr;
  if ((flags & LLA_FLAG_FUSED) && (entry == 0 || !fused_shape(*desc))) return nullptr;
  return scan_kernel_name(choose_scan(*desc, entry != 0, flags));
}

const char* lla_decode_scan_kernel_for_store(const lla_set_desc* desc, int32_t entry, int32_t flags,
                                             int32_t max_pos_hint, int32_t max_pages_per_seq) {
  if (check_desc(desc) != LLA_OK || entry < 0 || entry > 2 || !flags_ok(flags)) return nullptr;
  if ((flags & LLA_FLAG_FUSED) && (entry == 0 || !fused_shape(*desc))) return nullptr;
  if (max_pos_hint < 0 || max_pages_per_seq <= 0) return nullptr;
  return scan_kernel_name(choose_scan(*desc, entry != 0, flags, max_pages_per_seq, max_pos_hint));
}

size_t lla_parallel_workspace_bytes(const lla_set_desc* desc, int32_t batch, int32_t n_max) {
  if (check_parallel_desc(desc) != LLA_OK || batch <= 0 || n_max <= 0) return 0;
  return parallel_ws_layout(*desc, batch, n_max).total;
}

lla_status hla_attention_parallel(const lla_set_desc* d, const lla_store* st, int32_t batch,
                                  const lla_parallel_args* a, lla_stream_t stream) {
  lla_status r = check_parallel_desc(d);
  if (r != LLA_OK) return r;
  if ((r = check_store(st)) != LLA_OK) return r;
  if (batch <= 0 || !a) return LLA_ERR_INVALID_ARGUMENT;
  if (a->loop < d->loop_first || a->loop > d->loop_last) return LLA_ERR_INVALID_ARGUMENT;
  if (a->window < 0 || a->n_max <= 0 || a->flags != 0) return LLA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a->n_tok, a->q, a->k, a->v, a->A, a->B, a->out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LLA_ERR_INVALID_ARGUMENT;
  // the latents some position reads: tokens below n_max - 1 - W
  const int64_t n_lat = std::max<int64_t>(0, (int64_t)a->n_max - 1 - a->window);
  if ((int64_t)st->max_pages_per_seq * d->page_size < n_lat) return LLA_ERR_INVALID_ARGUMENT;
  const ParWs w = parallel_ws_layout(*d, batch, a->n_max);
  if (!a->workspace || a->workspace_bytes < w.total) return LLA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(a->workspace)) return LLA_ERR_INVALID_ARGUMENT;
  char* ws = static_cast<char*>(a->workspace);

  ParParams p{};
  p.B = batch; p.H = d->n_heads; p.dh = d->head_dim; p.G = d->groups; p.hpg = d->n_heads / d->groups;
  p.rk = d->r_k; p.rv = d->r_v; p.P = d->page_size; p.max_pages = st->max_pages_per_seq;
  p.W = a->window; p.n_max = a->n_max; p.n_pad = parallel_pad(a->n_max);
  p.rope_base = d->rope_base;
  p.scale = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
  p.n_tok = a->n_tok; p.bt = st->block_table; p.pages = st->pages;
  p.q = a->q; p.k = a->k; p.v = a->v; p.A = a->A; p.Bm = a->B; p.out = a->out;
  p.sk = ws + w.sk; p.sv = ws + w.sv; p.rtab = ws + w.rtab;
  p.kh = ws + w.kh; p.vh = ws + w.vh;
  return hip_status(launch_parallel(p, static_cast<hipStream_t>(stream), static_cast<hipEvent_t*>(a->attn_events)));
}

size_t lla_full_decode_workspace_bytes(const lla_kv_desc* desc, int32_t batch, int32_t max_pos,
                                       int32_t splits) {
  if (check_kv_desc(desc) != LLA_OK || batch <= 0 || max_pos < 0 || splits < 0) return 0;
  return full_ws_layout(*desc, batch, full_plan(*desc, batch, max_pos, splits).S).total;
}

int32_t lla_full_decode_plan_splits(const lla_kv_desc* desc, int32_t batch, int32_t max_pos,
                                    int32_t splits) {
  if (check_kv_desc(desc) != LLA_OK || batch <= 0 || max_pos < 0 || splits < 0) return 0;
  return full_plan(*desc, batch, max_pos, splits).S;
}

lla_status lla_decode_full_cache(const lla_kv_desc* d, const lla_kv_cache* c, int32_t batch,
                                 const lla_full_decode_args* a, lla_stream_t stream) {
  lla_status r = check_kv_desc(d);
  if (r != LLA_OK) return r;
  if (!c || !c->k_pages || !c->v_pages || !c->block_table || c->max_pages_per_seq <= 0)
    return LLA_ERR_INVALID_ARGUMENT;
  if (!aligned16(c->k_pages) || !aligned16(c->v_pages)) return LLA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || !a) return LLA_ERR_INVALID_ARGUMENT;
  if (a->max_pos_hint < 0 || a->splits < 0 || a->flags != 0) return LLA_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a->pos, a->q, a->k_cur, a->v_cur, a->out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LLA_ERR_INVALID_ARGUMENT;
  const Plan plan = full_plan(*d, batch, a->max_pos_hint, a->splits);
  const FullWs w = full_ws_layout(*d, batch, plan.S);
  if (!a->workspace || a->workspace_bytes < w.total) return LLA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(a->workspace)) return LLA_ERR_INVALID_ARGUMENT;
  char* ws = static_cast<char*>(a->workspace);

  FullParams f{};
  f.B = batch; f.H = d->n_heads; f.dh = d->head_dim; f.P = d->page_size; f.S = plan.S;
  f.chunk = plan.chunk; f.max_pages = c->max_pages_per_seq; f.bf16 = d->dtype == LLA_BF16;
  f.rope_base = d->rope_base;
  f.scale = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
  f.pos = a->pos; f.bt = c->block_table; f.k_pages = c->k_pages; f.v_pages = c->v_pages;
  f.q = a->q; f.k_cur = a->k_cur; f.v_cur = a->v_cur;
  f.part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  f.part_o = reinterpret_cast<float*>(ws + w.part_o);

  // the merge: head-space partials, no window part
  DecodeParams p{};
  p.B = batch; p.H = d->n_heads; p.dh = d->head_dim; p.S = plan.S; p.WS = 0; p.Dp = d->head_dim;
  p.mode = kReconstruct; p.bf16 = f.bf16;
  p.part_ml = f.part_ml; p.part_o = f.part_o; p.out = a->out;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(a->scan_events);
  hipError_t e = hipSuccess;
  if (ev) e = hipEventRecord(ev[0], s);
  if (e == hipSuccess) e = launch_full_scan(f, s);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
  if (e == hipSuccess) e = launch_combine(p, s);
  return hip_status(e);
}

lla_status lla_check_indices(const int32_t* pos_host, int32_t batch, const int32_t* block_table_host,
                             int32_t max_pages_per_seq, int32_t page_size, int32_t n_pages) {
  if (!pos_host || !block_table_host || batch <= 0 || max_pages_per_seq <= 0 || page_size <= 0 || n_pages <= 0)
    return LLA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t i = pos_host[b];
    if (i < 0 || (int64_t)i >= (int64_t)max_pages_per_seq * page_size) return LLA_ERR_INVALID_ARGUMENT;
    const int32_t* row = block_table_host + (int64_t)b * max_pages_per_seq;
    for (int32_t pg = 0; pg <= i / page_size; ++pg)
      if (row[pg] < 0 || row[pg] >= n_pages) return LLA_ERR_INVALID_ARGUMENT;
  }
  return LLA_OK;
}

size_t lla_bytes_per_token(const lla_set_desc* desc) {
  if (check_desc(desc) != LLA_OK) return 0;
  if (desc->latent_fp8) return (size_t)desc->groups * (desc->r_k + desc->r_v + 8);   // codes + 2 fp32 scales
  return (size_t)desc->groups * (desc->r_k + desc->r_v) * elem_bytes(*desc);
}

const char* lla_status_string(lla_status status) {
  switch (status) {
    case LLA_OK: return "ok";
    case LLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LLA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t lla_abi_version(void) { return LLA_ABI_VERSION; }

}  // extern "C"
