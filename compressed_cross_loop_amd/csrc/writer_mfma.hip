// Latent writer on the gfx950 matrix cores ("Hybrid Latent Attention"
// summary, "Latent Writer", Eq. 2).  Per group, the writer is one GEMM
//     c[tokens x (r_k+r_v)] = sum_t X_t[tokens x d_in] . E_t^T[d_in x (r_k+r_v)]
// with the loops concatenated along K.  For a decode step the matrices are
// short and wide (one token per sequence), so the GEMM is split along K
// across workgroups: each writes an fp32 partial tile to the workspace, and
// a second kernel sums the partials in a fixed order, rotates the key part
// by R~_p when the set bakes rotary embedding, rounds to bf16 and scatters
// into the paged store.  A bulk write (a whole prompt or training sequence:
// kBulkTokens tokens or more) runs the tiled GEMM of gemm_nt.h instead, one
// K segment per loop, into a single fp32 partial for the same second kernel.
//   v_mfma_f32_16x16x32_bf16: A = 8 consecutive inputs of one token (16-B
//   load from x), B = 8 consecutive inputs of one encoder row (16-B load
//   from E_t), both in their natural row-major layouts.
#include <algorithm>

#include "device_common.h"
#include "gemm_nt.h"
#include "lla_internal.h"
#include "writer_common.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileM = 16 * kWaves;   // tokens per workgroup (16 per wave)
constexpr int kTileN = 64;            // latent outputs per workgroup
constexpr int kRound = 12;            // 32-wide K steps staged per round
constexpr int kPieces = kTileN * kRound * 4;            // 16-byte pieces of an E round
constexpr int kPiecesPerThread = kPieces / kThreads;    // 6
constexpr int kReduceThreads = 256;
constexpr int kBulkTokens = 1024;   // tokens per call from which the tiled GEMM writes

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<bf16>(0.f);
  return z;
}

// grid (ceil(R / 64), ceil(M / 128), G * ksplit).  Each workgroup owns a
// 128-token x 64-output tile and one contiguous K range of the concatenated
// loops; per round of up to 12 K steps the 64 encoder rows' slice is staged
// in LDS (shared by the eight waves) and each wave keeps its 16 tokens'
// inputs for the whole round in registers.  All loads of a round are issued
// before its first product.
__global__ __launch_bounds__(kThreads) void k_writer_mfma(WriterParams p) {
  __shared__ __attribute__((aligned(16))) bf16 es[kTileN][kRound * 32 + 8];
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int g = blockIdx.z / p.ksplit, ks = blockIdx.z % p.ksplit;
  const int M = p.B * p.n_tok, R = p.R, d_in = p.d_in, G = p.G;
  const int ksteps = p.n_loops * d_in / 32;
  const int per = (ksteps + p.ksplit - 1) / p.ksplit;
  const int s0 = min(ksteps, ks * per), s1 = min(ksteps, s0 + per);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int m = mt * kTileM + wave * 16 + col;       // A-operand row (token)
  const bool m_ok = m < M;
  const bf16* x = static_cast<const bf16*>(p.x);
  const bf16* enc = static_cast<const bf16*>(p.enc);
  f32x4 acc[kTileN / 16];
#pragma unroll
  for (int j = 0; j < kTileN / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int r0 = s0; r0 < s1; r0 += kRound) {
    const int ns = min(kRound, s1 - r0);
    // this thread's pieces of the E slice: (row, step, 8-wide sub-block)
    bf16x8 ev[kPiecesPerThread];
#pragma unroll
    for (int u = 0; u < kPiecesPerThread; ++u) {
      const int xq = tid + u * kThreads;
      const int row = xq / (kRound * 4), st = (xq % (kRound * 4)) / 4, sub = xq % 4;
      const int n = nt * kTileN + row;
      const int k0 = (r0 + st) * 32;
      const int t = k0 / d_in, kk = k0 % d_in + sub * 8;
      ev[u] = (st < ns && n < R)
                  ? *reinterpret_cast<const bf16x8*>(enc + (((int64_t)t * G + g) * R + n) * d_in + kk)
                  : zero8();
    }
    bf16x8 a[kRound];
#pragma unroll
    for (int st = 0; st < kRound; ++st) {
      const int k0 = (r0 + st) * 32;
      const int t = k0 / d_in, kk = k0 % d_in + grp * 8;
      a[st] = (st < ns && m_ok) ? *reinterpret_cast<const bf16x8*>(
                                      x + (((int64_t)m * p.n_loops + t) * G + g) * d_in + kk)
                                : zero8();
    }
    __syncthreads();   // the previous round's reads of es are done
#pragma unroll
    for (int u = 0; u < kPiecesPerThread; ++u) {
      const int xq = tid + u * kThreads;
      const int row = xq / (kRound * 4), st = (xq % (kRound * 4)) / 4, sub = xq % 4;
      *reinterpret_cast<bf16x8*>(&es[row][st * 32 + sub * 8]) = ev[u];
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < kRound; ++st) {
      if (st < ns) {
#pragma unroll
        for (int j = 0; j < kTileN / 16; ++j) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&es[16 * j + col][st * 32 + grp * 8]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[st], bv, acc[j], 0, 0, 0);
        }
      }
    }
  }
  // lane holds C[row 4*grp + r][col] of each 16x16 tile
#pragma unroll
  for (int j = 0; j < kTileN / 16; ++j) {
    const int n = nt * kTileN + 16 * j + col;
    if (n >= R) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = mt * kTileM + wave * 16 + 4 * grp + r;
      if (mm < M) p.acc[(((int64_t)ks * M + mm) * G + g) * R + n] = acc[j][r];
    }
  }
}

// Sum the K-split partials of one (token, group) in split order, then
// rotate the key part by R~_p (baked sets) and store (bf16, or e4m3 codes
// with per-token scales).  The partial sums are read as float4 rows, eight splits'
// loads in flight at a time; the rotation angles come from a per-token table.
__global__ __launch_bounds__(kReduceThreads) void k_writer_reduce(WriterParams p) {
  extern __shared__ float c[];
  __shared__ float csn[128][2];     // d_h / 2 <= 128
  const int m = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int M = p.B * p.n_tok, R = p.R, G = p.G, KS = p.ksplit;
  const int b = m / p.n_tok, n = m % p.n_tok;
  const int pos = p.pos[(int64_t)b * p.n_tok + n];
  if (p.rope_baked && tid < p.dh / 2) {
    float cs, sn;
    rope_cs(p.rope_base, p.dh, tid, pos, cs, sn);
    csn[tid][0] = cs;
    csn[tid][1] = sn;
  }
  const float* src = p.acc + ((int64_t)m * G + g) * R;
  const int64_t kstride = (int64_t)M * G * R;
  for (int u = tid; u < R / 4; u += kReduceThreads) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KS; k0 += 8) {
      float4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = reinterpret_cast<const float4*>(src + min(k0 + q, KS - 1) * kstride)[u];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (k0 + q < KS) sum += f32x4{v[q].x, v[q].y, v[q].z, v[q].w};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * u + e] = sum[e];
  }
  __syncthreads();
  const int64_t page = p.bt[(int64_t)b * p.max_pages + pos / p.P];
  finish_latent<bf16, kReduceThreads>(p, c, csn, pos, page, pos % p.P, g);
}

// Bulk bf16 writes (prompts, the training pass): one workgroup per 16
// consecutive tokens.  When they are one sequence's positions 16 j .. 16 j +
// 15 (the usual case) they fill one 16-token tile of the store, which the
// workgroup assembles in LDS and writes as 16-byte pieces: key rows, and per
// value dimension the 16 tokens that lie next to each other in the
// dimension-major value sub-blocks.  Written token by token, every value
// element is a 2-byte store of its own and the 16 tokens sharing 32 bytes
// come from 16 workgroups.  Other groups take the per-token epilogue.  The
// partial is a single fp32 row per token (no K split for bulk writes);
// rotation and rounding are the per-token path's, in the same order.
constexpr int kTileTok = 16;

__global__ __launch_bounds__(kReduceThreads) void k_writer_reduce_tile(WriterParams p) {
  extern __shared__ float c[];                 // [16][R]
  __shared__ float csn[kTileTok][64][2];       // per token (cos, sin), d_h <= 128 (two workgroups per CU at R = 1024)
  __shared__ double theta[64];                 // frequencies, shared by the 16 tokens
  __shared__ int tpos[kTileTok];
  __shared__ int tile_ok;
  const int m0 = blockIdx.x * kTileTok, g = blockIdx.y, tid = threadIdx.x;
  const int M = p.B * p.n_tok, R = p.R, G = p.G, rk = p.rk, rv = p.rv, dh = p.dh, half = dh / 2;
  const int nt = min(kTileTok, M - m0);
  if (tid < kTileTok) tpos[tid] = tid < nt ? p.pos[m0 + tid] : -1;
  if (p.rope_baked && tid < half) theta[tid] = rope_theta(p.rope_base, dh, tid);
  const float* src = p.acc + ((int64_t)m0 * G + g) * R;
  for (int x = tid; x < nt * (R / 4); x += kReduceThreads) {
    const int t = x / (R / 4), u = x % (R / 4);
    reinterpret_cast<float4*>(c + t * R)[u] = reinterpret_cast<const float4*>(src + (int64_t)t * G * R)[u];
  }
  __syncthreads();
  if (tid == 0) {
    int ok = nt == kTileTok && m0 / p.n_tok == (m0 + kTileTok - 1) / p.n_tok && tpos[0] % kTileTok == 0;
    for (int t = 1; t < kTileTok && ok; ++t) ok = tpos[t] == tpos[0] + t;
    tile_ok = ok;
  }
  if (p.rope_baked) {
    for (int x = tid; x < nt * half; x += kReduceThreads) {
      const int t = x / half, f = x % half;
      float cs, sn;
      rope_cs_theta(theta[f], tpos[t], cs, sn);
      csn[t][f][0] = cs;
      csn[t][f][1] = sn;
    }
    __syncthreads();
    for (int x = tid; x < nt * (rk / 2); x += kReduceThreads) {
      const int t = x / (rk / 2), y = x % (rk / 2), blk = y / half, f = y % half;
      const int lo = blk * dh + f, hi = lo + half;
      float* ct = c + t * R;
      const float cs = csn[t][f][0], sn = csn[t][f][1];
      const float a = ct[lo], b = ct[hi];
      ct[lo] = a * cs - b * sn;
      ct[hi] = a * sn + b * cs;
    }
  }
  __syncthreads();
  if (tile_ok) {
    const int b = m0 / p.n_tok, pos0 = tpos[0];
    const int64_t page = p.bt[(int64_t)b * p.max_pages + pos0 / p.P];
    bf16* tile = static_cast<bf16*>(p.pages) + tile_base(page, g, pos0 % p.P, G, p.P, R);
    for (int x = tid; x < kTileTok * (rk / 8); x += kReduceThreads) {   // key rows, 8 dims a piece
      const int t = x / (rk / 8), d = 8 * (x % (rk / 8));
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = from_f<bf16>(c[t * R + d + e]);
      *reinterpret_cast<bf16x8*>(tile + key_in_tile(t, d, rk)) = o;
    }
    for (int x = tid; x < rv * 2; x += kReduceThreads) {   // value dim d, tokens t8 .. t8 + 7
      const int d = x / 2, t8 = 8 * (x % 2);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = from_f<bf16>(c[(t8 + e) * R + rk + d]);
      *reinterpret_cast<bf16x8*>(tile + 16 * rk + (d >> 4) * 256 + (d & 15) * 16 + t8) = o;
    }
  } else {
    WriterParams q = p;
    q.rope_baked = 0;   // rotated above
    for (int t = 0; t < nt; ++t) {
      const int m = m0 + t, pos = tpos[t];
      const int64_t page = p.bt[(int64_t)(m / p.n_tok) * p.max_pages + pos / p.P];
      finish_latent<bf16, kReduceThreads>(q, c + t * R, nullptr, pos, page, pos % p.P, g);
    }
  }
}

// the tile epilogue's shapes: bf16 store, 16-byte pieces, the 16 rows in 64 KiB of LDS
bool reduce_tile_supports(const WriterParams& p) {
  return p.bf16 && !p.fp8 && p.rk % 8 == 0 && p.rv % 16 == 0 && p.R % 4 == 0 &&
         (size_t)kTileTok * p.R * sizeof(float) <= 65536 && p.dh <= 128;
}

}  // namespace

bool writer_mfma_supports(const WriterParams& p) { return p.bf16 && p.d_in % 32 == 0; }

int writer_mfma_ksplit(int M, int G, int R, int n_loops, int d_in) {
  if (M >= kBulkTokens) return 1;   // tiled GEMM, no K split
  const int64_t tiles = (int64_t)((R + kTileN - 1) / kTileN) * ((M + kTileM - 1) / kTileM) * G;
  const int ksteps = n_loops * d_in / 32;
  int64_t ks = (256 + tiles - 1) / tiles;                       // about one workgroup per CU
  ks = std::min<int64_t>(ks, std::max(1, ksteps / 8));          // at least 8 K steps each
  ks = std::max<int64_t>(ks, (ksteps + 32 * kRound - 1) / (32 * kRound));   // at most 32 rounds each
  return (int)std::max<int64_t>(ks, 1);
}

hipError_t launch_writer_mfma(const WriterParams& p, hipStream_t s) {
  if (!writer_mfma_supports(p)) return hipErrorNotSupported;
  const int M = p.B * p.n_tok;
  hipError_t e;
  if (M >= kBulkTokens) {
    // c[m][g][r] = sum_t sum_d x[m][t][g][d] E[t][g][r][d]: K segment t per loop
    GemmParams<float> q{};
    q.X = static_cast<const bf16*>(p.x);
    q.Y = static_cast<const bf16*>(p.enc);
    q.C = p.acc;
    q.M = M; q.N = p.R; q.K = p.n_loops * p.d_in; q.kseg = p.d_in; q.G = p.G;
    q.ldx = p.n_loops * p.G * p.d_in; q.sxg = p.d_in; q.sxk = (int64_t)p.G * p.d_in;
    q.ldy = p.d_in; q.syg = (int64_t)p.R * p.d_in; q.syk = (int64_t)p.G * p.R * p.d_in;
    q.ldc = p.G * p.R; q.scg = p.R;
    // one latent group: x's K range is contiguous per token and each loop's
    // encoder a plain [R][d_in] matrix, so the vendor GEMM takes it (one
    // product per loop, summed), else the tiled GEMM
    const bool lib = p.G == 1 && lt_gemm_nt(q.X, q.Y, q.C, true, q.M, q.N, q.kseg, q.K / q.kseg, q.ldx, q.ldy,
                                            q.ldc, q.sxk, q.syk, s);
    e = lib ? hipSuccess : launch_gemm(q, 1, s);
  } else {
    const dim3 grid((p.R + kTileN - 1) / kTileN, (M + kTileM - 1) / kTileM, p.G * p.ksplit);
    hipLaunchKernelGGL(k_writer_mfma, grid, dim3(kThreads), 0, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (M >= kBulkTokens && reduce_tile_supports(p))
    hipLaunchKernelGGL(k_writer_reduce_tile, dim3((M + kTileTok - 1) / kTileTok, p.G), dim3(kReduceThreads),
                       (size_t)kTileTok * p.R * sizeof(float), s, p);
  else
    hipLaunchKernelGGL(k_writer_reduce, dim3(M, p.G), dim3(kReduceThreads), (size_t)p.R * sizeof(float), s, p);
  return hipGetLastError();
}

}  // namespace lla
