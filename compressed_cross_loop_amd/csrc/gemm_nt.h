// A plain "NT" GEMM on the gfx950 matrix cores, shared by the kernels that
// need one: C[m][n] = sum_k X[m][k] Y[n][k] (bf16 operands, fp32
// accumulation, C in bf16 or fp32), one (batch, group) per blockIdx.z.
//
// 128 x 128 tiles, 4 waves of 64 x 64 (v_mfma_f32_16x16x32_bf16: A = 8
// consecutive k of one X row, B = 8 consecutive k of one Y row, both 16-byte
// loads in the natural row-major layouts), K steps of 32 staged in LDS and
// double-buffered (the next step's loads in flight during the products).
// K may be made of segments of kseg elements that lie apart in memory (the
// loops of the latent writer: one segment per loop); every 32-wide K step
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

template <typename TC>
__global__ __launch_bounds__(256) void k_gemm_nt(GemmParams<TC> q) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int BM = 128, BN = 128, BK = 32, LD = BK + 8, NT = 256;
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
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * LD];
  static_assert(BM * LC <= 2 * (BM + BN) * LD, "output tile must fit the operand buffers");
  bf16 (*xs)[BM][LD] = reinterpret_cast<bf16 (*)[BM][LD]>(smem);
  bf16 (*ys)[BN][LD] = reinterpret_cast<bf16 (*)[BN][LD]>(smem + 2 * BM * LD);
  // loader: 2 chunks of 16 B per thread per operand and K step
  int xr[2], yr[2], kc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int idx = tid + NT * c;
    kc[c] = 8 * (idx % 4);
    xr[c] = min(m0 + idx / 4, q.M - 1);
    yr[c] = min(n0 + idx / 4, q.N - 1);
  }
  u32x4_t rx[2], ry[2];
  auto load = [&](int k0) {
    const int seg = k0 / q.kseg, kk = k0 - seg * q.kseg;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      rx[c] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)xr[c] * q.ldx + seg * q.sxk + kk + kc[c]);
      ry[c] = *reinterpret_cast<const u32x4_t*>(Y + (int64_t)yr[c] * q.ldy + seg * q.syk + kk + kc[c]);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = tid + NT * c;
      *reinterpret_cast<u32x4_t*>(&xs[buf][idx / 4][kc[c]]) = rx[c];
      *reinterpret_cast<u32x4_t*>(&ys[buf][idx / 4][kc[c]]) = ry[c];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = q.K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < nk) load((kk + 1) * BK);
    bf16x8_t a[4], bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(&xs[cur][64 * wm + 16 * i + col][8 * grp]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bb[j] = *reinterpret_cast<const bf16x8_t*>(&ys[cur][64 * wn + 16 * j + col][8 * grp]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = kBf16C ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(bb[j], a[i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
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
      for (int j = 0; j < 4; ++j) {
        bf16x4_t v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = static_cast<bf16>(acc[i][j][r]);
        *reinterpret_cast<bf16x4_t*>(&smem[(64 * wm + 16 * i + col) * LC + 64 * wn + 16 * j + 4 * grp]) = v;
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
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + col;
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
  const dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, batches * g.G);
  hipLaunchKernelGGL(k_gemm_nt<TC>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace
}  // namespace lla
