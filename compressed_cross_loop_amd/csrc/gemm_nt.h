// A plain "NT" GEMM on the gfx950 matrix cores, shared by the kernels that
// need one: C[m][n] = sum_k X[m][k] Y[n][k] (bf16 operands, fp32
// accumulation, C in bf16 or fp32), one (batch, group) per blockIdx.z.
//
// 128 x BN tiles, 4 waves of 64 x BN/2 (v_mfma_f32_16x16x32_bf16: A = 8
// consecutive k of one X row, B = 8 consecutive k of one Y row, both 16-byte
// loads in the natural row-major layouts).  BN = 256 (waves of 64 x 128)
// reads a quarter fewer LDS bytes per product than BN = 128 and each Y row
// half as often; it serves the wide rebuilds of the parallel pass (N a
// multiple of 256, K of 512 up to 1023).  K steps of BK staged in LDS and
// double-buffered (the next step's loads in flight during the products): BK =
// 64 for long reductions whose K segments allow it (one barrier per 32
// products of a wave), else 32.  K may be made of segments of kseg elements that lie apart in
// memory (the loops of the latent writer: one segment per loop); every K step
// lies in one segment.  Rows past M and N are clamped on load and skipped on
// store.  With a bf16 C the products are taken transposed (Y fragment as the A
// operand), so a lane holds four consecutive columns of one row; the tile is
// written through LDS (8-byte writes) and leaves as whole 16-byte row chunks.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace lla {
namespace {

template <typename TC>
struct GemmParams {
  const bf16* X;
  const bf16* Y;
  TC* C;
  int32_t M, N, K, ldx, ldy, ldc, G;
  int32_t kseg;                     // K segment length (K % kseg == 0, kseg % 32 == 0)
  int64_t sxk, syk;                 // element strides between K segments of X and Y
  int64_t sxb, sxg, syb, syg, scb, scg;
};

template <typename TC, int BK, int BN = 128>
__global__ __launch_bounds__(256, BN == 256 ? 2 : 1) void k_gemm_nt(GemmParams<TC> q) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  // LDS rows of BK + 8 bf16: the 16 rows a fragment read touches start in
  // distinct 4-bank groups
  constexpr int BM = 128, LD = BK + 8, NT = 256;
  constexpr int WN = BN / 2;             // wave tile: 64 x WN
  constexpr int NJ = WN / 16;            // column fragments per wave
  constexpr int CH = BM * BK / 8 / NT;   // 16-byte chunks per thread per K step: X
  constexpr int CHY = BN * BK / 8 / NT;  // .. and Y
  constexpr int KS = BK / 32;            // products per fragment pair and K step
  const int z = blockIdx.z, zb = z / q.G, zg = z % q.G;
  const bf16* X = q.X + zb * q.sxb + zg * q.sxg;
  const bf16* Y = q.Y + zb * q.syb + zg * q.syg;
  TC* C = q.C + zb * q.scb + zg * q.scg;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool kBf16C = std::is_same<TC, bf16>::value;
  constexpr int LC = BN + 8;        // LDS row of the output tile (bf16)
  constexpr int kOps = 2 * (BM + BN) * LD, kOut = kBf16C ? BM * LC : 0;
  __shared__ __attribute__((aligned(16))) bf16 smem[kOps > kOut ? kOps : kOut];
  bf16 (*xs)[BM][LD] = reinterpret_cast<bf16 (*)[BM][LD]>(smem);
  bf16 (*ys)[BN][LD] = reinterpret_cast<bf16 (*)[BN][LD]>(smem + 2 * BM * LD);
  // loader: CH chunks of 16 B per thread per operand and K step
  // chunk c of a K step: row (tid + NT c) / (BK / 8), k offset kc (the same
  // for every c, since NT is a multiple of BK / 8)
  const int kc = 8 * (tid % (BK / 8));
  int xr[CH], yr[CHY];
#pragma unroll
  for (int c = 0; c < CH; ++c) xr[c] = min(m0 + (tid + NT * c) / (BK / 8), q.M - 1);
#pragma unroll
  for (int c = 0; c < CHY; ++c) yr[c] = min(n0 + (tid + NT * c) / (BK / 8), q.N - 1);
  u32x4_t rx[CH], ry[CHY];
  auto load = [&](int k0) {
    const int seg = k0 / q.kseg, kk = k0 - seg * q.kseg;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      rx[c] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)xr[c] * q.ldx + seg * q.sxk + kk + kc);
#pragma unroll
    for (int c = 0; c < CHY; ++c)
      ry[c] = *reinterpret_cast<const u32x4_t*>(Y + (int64_t)yr[c] * q.ldy + seg * q.syk + kk + kc);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      *reinterpret_cast<u32x4_t*>(&xs[buf][(tid + NT * c) / (BK / 8)][kc]) = rx[c];
#pragma unroll
    for (int c = 0; c < CHY; ++c)
      *reinterpret_cast<u32x4_t*>(&ys[buf][(tid + NT * c) / (BK / 8)][kc]) = ry[c];
  };
  f32x4_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = q.K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < nk) load((kk + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t a[4], bb[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&xs[cur][64 * wm + 16 * i + col][32 * ks + 8 * grp]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bb[j] = *reinterpret_cast<const bf16x8_t*>(&ys[cur][WN * wn + 16 * j + col][32 * ks + 8 * grp]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = kBf16C ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(bb[j], a[i], acc[i][j], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    if (kk + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  if constexpr (kBf16C) {
    // lane holds C[row col][columns 4 grp .. + 3] of each 16 x 16 block; the
    // loop's last barrier has released the operand buffers
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bf16x4_t v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<bf16>(acc[i][j][r]);
        *reinterpret_cast<bf16x4_t*>(&smem[(64 * wm + 16 * i + col) * LC + WN * wn + 16 * j + 4 * grp]) = v;
      }
    __syncthreads();
    const bool vec = (q.ldc % 8 == 0) && (reinterpret_cast<uintptr_t>(C) % 16 == 0);
#pragma unroll
    for (int c = 0; c < BM * BN / 8 / NT; ++c) {
      const int idx = tid + NT * c, row = idx / (BN / 8), c8 = 8 * (idx % (BN / 8));
      const int m = m0 + row, n = n0 + c8;
      if (m >= q.M) continue;
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(&smem[row * LC + c8]);
      TC* dst = C + (int64_t)m * q.ldc + n;
      if (vec && n + 7 < q.N) {
        *reinterpret_cast<bf16x8_t*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < q.N) dst[e] = v[e];
      }
    }
    return;
  }
  // lane holds C[4 grp + r][col] of each 16 x 16 block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + WN * wn + 16 * j + col;
      if (n >= q.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * i + 4 * grp + r;
        if (m < q.M) C[(int64_t)m * q.ldc + n] = static_cast<TC>(acc[i][j][r]);
      }
    }
}

template <typename TC>
hipError_t launch_gemm(const GemmParams<TC>& g, int batches, hipStream_t s) {
  if (std::is_same<TC, bf16>::value && g.N % 256 == 0 && g.K >= 512 && g.K < 1024) {
    // wide bf16 outputs (the parallel pass's rebuild, N = heads x d_h):
    // median 51.3 -> 49.1 us at K = 512; at K = 256 the 128 x 128 tiles are
    // faster (31.1 against 32.6 us)
    const dim3 grid(g.N / 256, (g.M + 127) / 128, batches * g.G);
    hipLaunchKernelGGL((k_gemm_nt<TC, 32, 256>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
  }
  const dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, batches * g.G);
  // K steps of 64 for long reductions (the bulk writer's K = loops x d_in:
  // 188.6 -> 167 us at 16384 x 1024 x 6144); at K = 512 (the parallel pass's
  // rebuild) the shorter loop did not pay for the lower occupancy (44.8 ->
  // 46.0 us)
  if (g.K >= 1024 && g.K % 64 == 0 && g.kseg % 64 == 0)
    hipLaunchKernelGGL((k_gemm_nt<TC, 64>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm_nt<TC, 32>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace
}  // namespace lla
