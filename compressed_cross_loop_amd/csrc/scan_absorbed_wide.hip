// Absorbed latent scan for one very wide latent shared by all heads (the
// head-folded LLA-D read: "Looped Latent Attention" abstract, LLA-D reading
// latents without reconstruction; "Hybrid Latent Attention" summary, "Latent
// Reader", Eqs. 3-4 first term).  With r in the thousands and dozens of heads
// the running output O~[heads][r_v] of one sequence no longer fits a
// workgroup, so the scan takes two passes over the store, each a batched
// contraction on the matrix cores:
//
//   scores   S[b][h][j] = q~_h . c^K_j for every latent token j
//            (M = 16-token blocks, N = heads, K = r_k; keys straight from the
//            store's token-major rows, q~ from the query map's output)
//   softmax  per (sequence, head): m = max_j S, P_j = 2^(S_j - m) in bf16,
//            and per context split l_s = sum of 2^(S_j - m) over its tokens
//            (exp2 domain: q~ carries log2(e)/sqrt(d_h))
//   values   O~^T[r_v x heads] = C^V^T . P^T per context split and 256-dim
//            slab of r_v (value blocks straight from the store's
//            dimension-major 16 x 16 blocks)
//
// The partials (m, l_s, O~_s) have the layout of the one-pass scans, so the
// combine kernel merges them and applies the value map as usual.  Both long
// passes read every latent byte once: the extra traffic is S (fp32, one row
// per part of r_k when small batches split the score pass) and P (bf16), 6
// bytes per (head, token) at one part, against 2 (r_k + r_v) bytes of latents.
#include <algorithm>
#include <utility>

#include "device_common.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTokPerWave = 64;                   // scores: 4 row blocks of 16 tokens
constexpr int kScoreWaves = 8;                    // scores workgroup: 8 waves share each staged q~ chunk
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kTokPerBlock = kScoreWaves * kTokPerWave;   // scores workgroup
constexpr int kSlab = 256;                        // values: r_v dims per workgroup
constexpr int kWidePageTab = kWideMaxPages;       // page ids of one split, in LDS
constexpr int kSoftmaxLdsTokens = 16384;          // longest score row the softmax pass keeps in LDS (64 KiB)
constexpr int kScoreWorkgroups = 512;             // score-pass workgroups aimed at (two rounds of one per CU)
constexpr int kXcds = 8;                          // XCDs of the GPU; workgroups are dealt to them round-robin

template <typename F, int... U>
__device__ __forceinline__ void wide_static_for_impl(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void wide_static_for(F&& f) {
  wide_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int latent_tokens(const DecodeParams& p, int b) {
  return min(max(0, p.pos[b] - p.W), p.lcap);
}

// ---------------------------------------------------------------- scores
// One workgroup = 512 consecutive tokens x all heads (padded to 64) x one part
// of r_k (the whole of it unless the batch is small); wave w (of 8) owns tokens
// 64 w .. 64 w + 63 (4 row blocks of 16), K in steps of 32
// (v_mfma_f32_16x16x32_bf16, 16 per step).  Key fragments come straight from
// the store (one 16-byte load per lane, token = lane % 16 of the row block),
// kKeyAhead steps ahead.  q~ is shared by the eight waves: it is staged in LDS
// in chunks of 128 latent dims (64 head rows of 256 contiguous bytes, loaded
// once per workgroup, double-buffered) and its fragments are read from there;
// the 16-byte pieces of a row are XOR-swizzled by the row so that the 16
// heads of a fragment read spread over the banks.
constexpr int kKeyAhead = 4;      // = steps per q~ chunk (the key ring index is the step in the chunk)
constexpr int kQChunk = 128;      // latent dims per staged q~ chunk

__global__ __launch_bounds__(kScoreThreads) void k_scan_absorbed_wide_scores(DecodeParams p, int by_xcd) {
  __shared__ __attribute__((aligned(16))) bf16 qs[2][64 * kQChunk];   // q~ hi part, double-buffered
  __shared__ __attribute__((aligned(16))) bf16 ql[2][64 * kQChunk];   // q~ lo part
  // workgroup -> (token block, sequence, part of r_k); with `by_xcd` the grid
  // is one-dimensional and the ids of one sequence's workgroups are
  // congruent mod 8, so the round-robin dealing puts them on one XCD and
  // its L2 serves their q~ re-reads
  int wx = blockIdx.x, wb = blockIdx.y, wz = blockIdx.z;
  if (by_xcd) {
    const int nx = p.lcap / kTokPerBlock, per = nx * p.wsplit;
    const int L = blockIdx.x, xcd = L % kXcds, k = L / kXcds;
    wb = (k / per) * kXcds + xcd;
    wx = (k % per) % nx;
    wz = (k % per) / nx;
  }
  const int b = wb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int n_lat = latent_tokens(p, b);
  const int tb = wx * kTokPerBlock;
  if (tb >= n_lat) return;                       // workgroup-uniform
  // waves past the last latent token compute on clamped tokens and store nothing
  const int tw = tb + wave * kTokPerWave;
  const int H = p.H, rk = p.rk, P = p.P, R = p.rk + p.rv;
  const bf16* pages = static_cast<const bf16*>(p.pages);
  // a lane's 8 key dims of K step ks: row (t % 16) of the tile, dims 32 ks +
  // 8 grp; wide rows are chunk-major, so a step is one contiguous KiB per tile
  const bool wide = wide_keys(rk);
  const int kstep = wide ? 16 * kKeyChunk : 32;
  const bf16* krow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // tokens past the end read the last latent token (always written); their
    // scores land in S but nothing reads them
    const int t = min(tw + 16 * i + col, n_lat - 1);
    const int64_t page = p.bt[(int64_t)b * p.max_pages + t / P];
    krow[i] = pages + tile_base(page, 0, t % P, 1, P, R) + (t % 16) * (wide ? kKeyChunk : rk) + 8 * grp;
  }
  // q~ staging: piece x = tid + kScoreThreads k of a chunk is head row x / 16,
  // dims 8 (x % 16) .. + 7, kept at slot (x % 16) ^ (row % 16) of its LDS row
  constexpr int QP = 64 * 16 / kScoreThreads;   // pieces per thread
  // the query map leaves q~ as bf16 hi and lo parts (lo at qlat + B H r_k);
  // each K step multiplies both, which keeps the scores at fp32-level accuracy
  const bf16* qsrc[QP];
  int qoff[QP], qdst[QP];
  const int64_t qlo = (int64_t)p.B * H * rk;
#pragma unroll
  for (int k = 0; k < QP; ++k) {
    const int x = tid + kScoreThreads * k, row = x >> 4, c = x & 15;
    qsrc[k] = static_cast<const bf16*>(p.qlat) + ((int64_t)b * H + min(row, H - 1)) * rk;
    qoff[k] = 8 * c;
    qdst[k] = row * kQChunk + 8 * (c ^ (row & 15));
  }
  u32x4 qreg[QP], qreg_lo[QP];
  auto q_load = [&](int kc0) {   // pieces past r_k feed no step (r_k % 32 == 0): clamp their address
#pragma unroll
    for (int k = 0; k < QP; ++k) {
      const bf16* src = qsrc[k] + min(kc0 + qoff[k], rk - 8);
      qreg[k] = *reinterpret_cast<const u32x4*>(src);
      qreg_lo[k] = *reinterpret_cast<const u32x4*>(src + qlo);
    }
  };
  auto q_store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < QP; ++k) {
      *reinterpret_cast<u32x4*>(&qs[buf][qdst[k]]) = qreg[k];
      *reinterpret_cast<u32x4*>(&ql[buf][qdst[k]]) = qreg_lo[k];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc[i][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ka[kKeyAhead][4];
  const int nk = rk / 32;
  auto issue = [&](auto U, int ks) {
    constexpr int u = decltype(U)::value;
    const int k0 = kstep * min(ks, nk - 1);    // clamped: always a valid step
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[u][i] = *reinterpret_cast<const bf16x8*>(krow[i] + k0);
  };
  // step U of the chunk in LDS buffer buf: B fragment of head block hb =
  // q~[16 hb + col][32 U + 8 grp ..], piece 4 U + grp of the row
  auto step = [&](auto U, int buf) {
    constexpr int u = decltype(U)::value;
    bf16x8 qa[4], qb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int o = (16 * hb + col) * kQChunk + 8 * ((4 * u + grp) ^ col);
      qa[hb] = *reinterpret_cast<const bf16x8*>(&qs[buf][o]);
      qb[hb] = *reinterpret_cast<const bf16x8*>(&ql[buf][o]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        acc[i][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][i], qa[hb], acc[i][hb], 0, 0, 0);
        acc[i][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][i], qb[hb], acc[i][hb], 0, 0, 0);
      }
  };
  // q~ chunks of this workgroup's part of r_k (part wz of wsplit parts,
  // none empty); every chunk but the last of r_k is whole
  const int nch = (nk + kKeyAhead - 1) / kKeyAhead;
  const int cpz = (nch + p.wsplit - 1) / p.wsplit;
  const int c0 = wz * cpz, c1 = min(nch, c0 + cpz);
  wide_static_for<kKeyAhead>([&](auto U) { issue(U, kKeyAhead * c0 + decltype(U)::value); });
  q_load(kQChunk * c0);
  q_store(0);
  __syncthreads();
  int c = c0;
  for (; c + 1 < c1; ++c) {
    q_load(kQChunk * (c + 1));
    wide_static_for<kKeyAhead>([&](auto U) {
      step(U, (c - c0) & 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(U, kKeyAhead * (c + 1) + decltype(U)::value);
      __builtin_amdgcn_sched_barrier(0);
    });
    q_store((c + 1 - c0) & 1);
    __syncthreads();
  }
  wide_static_for<kKeyAhead>([&](auto U) {
    if (kKeyAhead * c + decltype(U)::value < nk) step(U, (c - c0) & 1);
  });
  if (tw >= n_lat) return;
  // lane holds S[head 16 hb + col][tokens 16 i + 4 grp .. + 3] (this part's sum)
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 16 * hb + col;
    if (h >= H) continue;
    float* srow = p.wscore + (((int64_t)wz * p.B + b) * H + h) * p.lcap + tw + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(srow + 16 * i) = acc[i][hb];
  }
}

// ---------------------------------------------------------------- softmax
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();                               // red is reused
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// one workgroup per (head, sequence).  With LDS the summed score row is kept
// there after the first read (rows up to kSoftmaxLdsTokens tokens), so the
// probability and split-sum passes do not read it from memory again.
template <bool LDS>
__global__ __launch_bounds__(kThreads) void k_scan_absorbed_wide_softmax(DecodeParams p) {
  __shared__ float red[4];
  extern __shared__ __attribute__((aligned(16))) float srow[];   // [lcap] when LDS
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n_lat = latent_tokens(p, b);
  const int64_t row = ((int64_t)b * p.H + h) * p.lcap;
  f32x4* s4 = reinterpret_cast<f32x4*>(p.wscore + row);
  f32x4* r4 = LDS ? reinterpret_cast<f32x4*>(srow) : s4;   // where the summed row is read back
  // probabilities for every token the value pass reads: up to the 16-token
  // tile holding the last latent token (zero past n_lat)
  const int n16 = (n_lat + 15) / 16 * 16;
  // scores split along r_k are summed (fixed order)
  const int64_t part = (int64_t)p.B * p.H * p.lcap / 4;
  float m = -INFINITY;
  for (int x = tid; x < n16 / 4; x += kThreads) {
    f32x4 v = s4[x];
    for (int z = 1; z < p.wsplit; ++z) v += s4[z * part + x];
    if (LDS || p.wsplit > 1) r4[x] = v;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * x + r < n_lat) m = fmaxf(m, v[r]);
  }
  m = block_max(m, red);   // its barriers also publish the summed row
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4* p4 = reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.wprob) + row);
  for (int x = tid; x < n16 / 4; x += kThreads) {
    const f32x4 v = r4[x];
    bf16x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(4 * x + r < n_lat ? fast_exp2(v[r] - m) : 0.f);
    p4[x] = o;
  }
  // l per context split (the splits of the value pass and the combine)
  const float* rs = reinterpret_cast<const float*>(r4);
  for (int s = 0; s < p.S; ++s) {
    int t0 = s * p.chunk;
    const int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
    if (t0 > n_lat) t0 = n_lat;
    float l = 0.f;
    for (int j = t0 + tid; j < t1; j += kThreads) l += fast_exp2(rs[j] - m);
    l = block_sum(l, red);
    if (tid == 0) {
      const int64_t pr = ((int64_t)b * p.S + s) * p.H + h;
      p.part_ml[pr * 2 + 0] = m;
      p.part_ml[pr * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- values
// One workgroup = (256-dim slab of r_v, context split, sequence); wave w owns
// dims 64 w .. 64 w + 63 of the slab (4 value blocks) for all heads and walks
// every 16-token tile of the split: per tile 4 value fragments (8 bytes per
// lane, 512 contiguous bytes per block) straight from the store, prefetched
// kTileAhead tiles ahead, and 16 v_mfma_f32_16x16x16_bf16.  The
// probabilities are shared by the four waves: they are staged in LDS in
// chunks of 128 tokens (64 head rows of 256 contiguous bytes, loaded once per
// workgroup, double-buffered; rows padded by 16 bytes so that the 16 heads
// of a fragment read fall in different banks).  The split's page ids are
// staged in LDS too.
constexpr int kTileAhead = 4;                 // value tiles in flight per wave
constexpr int kPChunk = 128;                  // tokens per staged probability chunk (8 tiles)
constexpr int kPRow = kPChunk + 8;            // its LDS row (bf16)

__global__ __launch_bounds__(kThreads, 2) void k_scan_absorbed_wide_values(DecodeParams p, int by_xcd) {
  __shared__ int32_t ptab[kWidePageTab];
  __shared__ __attribute__((aligned(16))) bf16 ps[2][64 * kPRow];
  // workgroup -> (slab, split, sequence); with `by_xcd` the grid is
  // one-dimensional and the ids of one sequence's workgroups are congruent
  // mod 8, so they share one XCD and its L2 serves their re-reads of the
  // sequence's probabilities
  int ws_ = blockIdx.x, ss = blockIdx.y, sb = blockIdx.z;
  if (by_xcd) {
    const int nsl = (p.rv + kSlab - 1) / kSlab, per = nsl * p.S;
    const int L = blockIdx.x, xcd = L % kXcds, k = L / kXcds;
    sb = (k / per) * kXcds + xcd;
    ws_ = (k % per) % nsl;
    ss = (k % per) / nsl;
  }
  const int s = ss, b = sb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int H = p.H, rk = p.rk, rv = p.rv, P = p.P, R = p.rk + p.rv;
  const int n_lat = latent_tokens(p, b);
  int t0 = s * p.chunk;
  const int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;
  const int pfirst = t0 / P;
  {
    const int npg = t1 > t0 ? (t1 - 1) / P - pfirst + 1 : 0;   // <= max_pages <= kWidePageTab
    for (int x = tid; x < npg; x += kThreads) ptab[x] = p.bt[(int64_t)b * p.max_pages + pfirst + x];
  }
  __syncthreads();
  const int nblk = rv / 16;
  // waves past the last value block load clamped blocks and store nothing
  const int db0 = ws_ * (kSlab / 16) + 4 * wave;
  int voff[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) voff[jb] = 16 * rk + min(db0 + jb, nblk - 1) * 256 + col * 16 + 4 * grp;
  // probability staging: piece x = tid + 256 k of a chunk is head row x / 16,
  // tokens 8 (x % 16) .. + 7
  const bf16* psrc[4];
  int poff[4], pdst[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int x = tid + kThreads * k, row = x >> 4, c = x & 15;
    psrc[k] = static_cast<const bf16*>(p.wprob) + ((int64_t)b * H + min(row, H - 1)) * p.lcap;
    poff[k] = 8 * c;
    pdst[k] = row * kPRow + 8 * c;
  }
  u32x4 preg[4];
  auto p_load = [&](int j0c) {   // tokens past the row feed no tile: clamp their address
#pragma unroll
    for (int k = 0; k < 4; ++k) preg[k] = *reinterpret_cast<const u32x4*>(psrc[k] + min(j0c + poff[k], p.lcap - 8));
  };
  auto p_store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(&ps[buf][pdst[k]]) = preg[k];
  };
  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int ntiles = (t1 - t0 + 15) / 16;

  f32x4 acc[4][4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc[jb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  s16x4 va[kTileAhead][4];
  auto issue = [&](auto U, int ti) {
    constexpr int u = decltype(U)::value;
    const int j0 = t0 + 16 * min(ti, ntiles - 1);              // clamped: always a valid tile
    const int64_t page = ptab[j0 / P - pfirst];
    const bf16* tp = pages + tile_base(page, 0, j0 % P, 1, P, R);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) va[u][jb] = *reinterpret_cast<const s16x4*>(tp + voff[jb]);
  };
  // tile tl (0..7) of the chunk in LDS buffer buf; B fragment of head block hb
  // = probabilities of head 16 hb + col, tokens 16 tl + 4 grp .. + 3
  auto step = [&](auto U, int buf, int tl, int nvalid) {
    constexpr int u = decltype(U)::value;
    if (nvalid < 16) {
      // tokens past the end of the split: their value slots may hold anything
      // (even NaN), and their probabilities are zero or belong to no split
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * grp + r >= nvalid) va[u][jb][r] = 0;
    }
    s16x4 pa[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      pa[hb] = *reinterpret_cast<const s16x4*>(&ps[buf][(16 * hb + col) * kPRow + 16 * tl + 4 * grp]);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        acc[jb][hb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[u][jb], pa[hb], acc[jb][hb], 0, 0, 0);
  };
  constexpr int kTilesPerChunk = kPChunk / 16;
  if (ntiles > 0) {                              // workgroup-uniform
    const int nch = (ntiles + kTilesPerChunk - 1) / kTilesPerChunk;   // every chunk but the last is whole
    wide_static_for<kTileAhead>([&](auto U) { issue(U, decltype(U)::value); });
    p_load(t0);
    p_store(0);
    __syncthreads();
    int c = 0;
    for (; c + 1 < nch; ++c) {
      p_load(t0 + kPChunk * (c + 1));
#pragma unroll
      for (int half = 0; half < kTilesPerChunk / kTileAhead; ++half) {
        wide_static_for<kTileAhead>([&](auto U) {
          const int tl = kTileAhead * half + decltype(U)::value;
          step(U, c & 1, tl, 16);
          __builtin_amdgcn_sched_barrier(0);
          issue(U, kTilesPerChunk * c + tl + kTileAhead);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      p_store((c + 1) & 1);
      __syncthreads();
    }
#pragma unroll
    for (int half = 0; half < kTilesPerChunk / kTileAhead; ++half) {
      wide_static_for<kTileAhead>([&](auto U) {
        const int tl = kTileAhead * half + decltype(U)::value, ti = kTilesPerChunk * c + tl;
        if (ti < ntiles) {
          step(U, c & 1, tl, min(16, t1 - (t0 + 16 * ti)));
          if (half + 1 < kTilesPerChunk / kTileAhead) issue(U, ti + kTileAhead);
        }
      });
    }
  }
  // lane holds O~[dims 16 db + 4 grp .. + 3][head 16 hb + col]
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 16 * hb + col;
    if (h >= H) continue;
    const int64_t orow = (((int64_t)b * p.S + s) * H + h) * p.Dp;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (db0 + jb >= nblk) continue;
      const int d = 16 * (db0 + jb) + 4 * grp;
      if (p.part_bf16) {   // the wide combine reads them in bf16, as it feeds them to its products
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<bf16>(acc[jb][hb][r]);
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.part_o) + orow + d) = v;
      } else {
        *reinterpret_cast<f32x4*>(p.part_o + orow + d) = acc[jb][hb];
      }
    }
  }
}

}  // namespace

bool scan_absorbed_wide_supports(const DecodeParams& p) {
  return p.bf16 && !p.fp8 && p.G == 1 && p.H <= 64 && p.rk % 32 == 0 && p.rv % 16 == 0 && p.rk >= 32 &&
         p.rv >= 16 && p.max_pages <= kWidePageTab;
}

int scan_absorbed_wide_slabs(int rv) { return (rv + kSlab - 1) / kSlab; }

int scan_absorbed_wide_lcap(int max_pos) {
  return (max(max_pos, 0) + 1 + kTokPerBlock - 1) / kTokPerBlock * kTokPerBlock;
}

// Parts of r_k the score pass is split into: enough workgroups to fill the
// chip at small batches (a part is a whole number of 128-dim q~ chunks, and
// no part is empty).
int scan_absorbed_wide_ksplit(int B, int lcap, int rk) {
  const int64_t base = (int64_t)(lcap / kTokPerBlock) * B;
  const int nch = (rk / 32 + kKeyAhead - 1) / kKeyAhead;
  int kz = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (kScoreWorkgroups + base - 1) / base));
  const int cpz = (nch + kz - 1) / kz;
  return (nch + cpz - 1) / cpz;
}

hipError_t launch_scan_absorbed_wide(const DecodeParams& p, hipStream_t s) {
  if (!scan_absorbed_wide_supports(p) || p.lcap % kTokPerBlock || !p.wscore || !p.wprob ||
      p.wsplit != scan_absorbed_wide_ksplit(p.B, p.lcap, p.rk))
    return hipErrorNotSupported;
  // a sequence's score workgroups on one XCD when every XCD still gets
  // sequences (batch a multiple of 8), else the plain three-dimensional grid
  const int nx = p.lcap / kTokPerBlock;
  if (p.B % kXcds == 0)
    hipLaunchKernelGGL(k_scan_absorbed_wide_scores, dim3(nx * p.B * p.wsplit), dim3(kScoreThreads), 0, s, p, 1);
  else
    hipLaunchKernelGGL(k_scan_absorbed_wide_scores, dim3(nx, p.B, p.wsplit), dim3(kScoreThreads), 0, s, p, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.lcap <= kSoftmaxLdsTokens)
    hipLaunchKernelGGL(k_scan_absorbed_wide_softmax<true>, dim3(p.H, p.B), dim3(kThreads), (size_t)p.lcap * 4, s, p);
  else
    hipLaunchKernelGGL(k_scan_absorbed_wide_softmax<false>, dim3(p.H, p.B), dim3(kThreads), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.B % kXcds == 0)
    hipLaunchKernelGGL(k_scan_absorbed_wide_values, dim3(scan_absorbed_wide_slabs(p.rv) * p.S * p.B), dim3(kThreads),
                       0, s, p, 1);
  else
    hipLaunchKernelGGL(k_scan_absorbed_wide_values, dim3(scan_absorbed_wide_slabs(p.rv), p.S, p.B), dim3(kThreads),
                       0, s, p, 0);
  return hipGetLastError();
}

}  // namespace lla
