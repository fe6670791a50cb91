// Query map and combine for the absorbed read of one wide latent shared by
// all heads ("Hybrid Latent Attention" summary, "Latent Reader": q~ = A_t^T q
// before the scan, o = B_t^T O~ / l after it; LLA-D of the Looped Latent
// Attention abstract).  With r in the thousands each head's A_t and B_t^T are
// about a MiB, so these kernels take every sequence of a head together and
// read each map once per workgroup, instead of once per (sequence, head).
//
//   k_qmap_wide     workgroup = (slab of latent dims, head); a thread holds
//                   its latent dim's column of A_t in registers (bf16 pairs)
//                   and takes every sequence in turn: q is the same for the
//                   whole workgroup, staged in LDS and read as broadcasts,
//                   and each pair of products is one v_dot2_f32_bf16.  RoPE on the
//                   latent (frequency-paired decoders) rotates dim pairs
//                   (f, f + d_h/2) inside each d_h block, exchanged in LDS.
//   k_combine_wide  workgroup = (head, 16 sequences): merge weights of the
//                   context splits and window slices per sequence, then
//                   O~ B_t on the matrix cores (M = 16 sequences, N = d_h,
//                   K = r_v; O~ rounded to bf16 as the scans round their
//                   probabilities), K split over the four waves and summed
//                   in LDS, plus the window's head-space sums, over l.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSeqChunk = 16;   // sequences per LDS round of the query map / per combine workgroup

// ---------------------------------------------------------------- query map
template <int DH>
__global__ __launch_bounds__(kThreads) void k_qmap_wide(DecodeParams p) {
  constexpr int HALF = DH / 2;
  __shared__ float ub[kSeqChunk][kThreads];
  __shared__ float cs[kSeqChunk][HALF][2];
  __shared__ __attribute__((aligned(16))) unsigned qs[kSeqChunk][HALF];   // q of the chunk, bf16 pairs
  const int h = blockIdx.y, tid = threadIdx.x;
  const int H = p.H, rk = p.rk, B = p.B;
  const bool rope = p.rope_base != 0.f;
  const int slab = rope ? (kThreads / DH) * DH : kThreads;   // whole d_h blocks when rotating
  const int n0 = blockIdx.x * slab;
  const int n = n0 + tid;
  const bool act = tid < slab && n < rk;
  const unsigned short* Ah = static_cast<const unsigned short*>(p.A) + (int64_t)h * DH * rk;
  const int nc = min(n, rk - 1);
  unsigned acol[HALF];   // A_t[e][n], A_t[e+1][n] packed
#pragma unroll
  for (int e2 = 0; e2 < HALF; ++e2)
    acol[e2] = (unsigned)Ah[(int64_t)(2 * e2) * rk + nc] | ((unsigned)Ah[(int64_t)(2 * e2 + 1) * rk + nc] << 16);
  bf16* ql = static_cast<bf16*>(p.qlat);
  for (int b0 = 0; b0 < B; b0 += kSeqChunk) {
    const int nb = min(kSeqChunk, B - b0);
    for (int x = tid; x < nb * HALF; x += kThreads) {
      const int bb = x / HALF, e2 = x % HALF;
      qs[bb][e2] = reinterpret_cast<const unsigned*>(static_cast<const bf16*>(p.q) + ((int64_t)(b0 + bb) * H + h) * DH)[e2];
    }
    if (rope) {
      for (int x = tid; x < nb * HALF; x += kThreads) {
        const int bb = x / HALF, f = x % HALF;
        float c, s;
        rope_cs(p.rope_base, DH, f, p.pos[b0 + bb], c, s);
        cs[bb][f][0] = c;
        cs[bb][f][1] = s;
      }
    }
    __syncthreads();
    for (int bb = 0; bb < nb; ++bb) {
      const unsigned* qp = qs[bb];   // same address in every lane: LDS broadcast
      float acc = 0.f;
#pragma unroll
      for (int e2 = 0; e2 < HALF; ++e2)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, acol[e2]),
                                              __builtin_bit_cast(bf16x2, qp[e2]), acc, false);
      if (rope)
        ub[bb][tid] = acc;
      else if (act)
        ql[((int64_t)(b0 + bb) * H + h) * rk + n] = static_cast<bf16>(acc * p.scale);
    }
    if (rope) {
      __syncthreads();
      if (act) {
        const int f = n % DH;   // n0 is a multiple of d_h, so the partner is in this slab
        const int fp = f < HALF ? f : f - HALF;
        for (int bb = 0; bb < nb; ++bb) {
          const float c = cs[bb][fp][0], s = cs[bb][fp][1];
          const float u = ub[bb][tid];
          const float v = f < HALF ? u * c - ub[bb][tid + HALF] * s : ub[bb][tid - HALF] * s + u * c;
          ql[((int64_t)(b0 + bb) * H + h) * rk + n] = static_cast<bf16>(v * p.scale);
        }
      }
    }
    __syncthreads();   // qs, ub and cs are refilled next round
  }
  // q rotated to its position (head space), for the exact-window kernel
  if (p.need_qhead && blockIdx.x == 0) {
    for (int x = tid; x < B * HALF; x += kThreads) {
      const int b = x / HALF, f = x % HALF;
      const bf16* q = static_cast<const bf16*>(p.q) + ((int64_t)b * H + h) * DH;
      float c = 1.f, s = 0.f;
      if (rope) rope_cs(p.rope_base, DH, f, p.pos[b], c, s);
      const float x1 = static_cast<float>(q[f]), x2 = static_cast<float>(q[f + HALF]);
      float* qh = p.qhead + ((int64_t)b * H + h) * DH;
      qh[f] = p.scale * (x1 * c - x2 * s);
      qh[f + HALF] = p.scale * (x1 * s + x2 * c);
    }
  }
}

// ---------------------------------------------------------------- combine
template <int DH>
__global__ __launch_bounds__(kThreads) void k_combine_wide(DecodeParams p) {
  constexpr int NB = DH / 16;
  constexpr int KB = 4;   // K steps whose loads are issued together
  extern __shared__ float wsm[];                           // [16][S + WS] merge weights
  __shared__ float red[4][kSeqChunk][DH + 4];
  __shared__ float inv[kSeqChunk];
  const int h = blockIdx.x, b0 = blockIdx.y * kSeqChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = p.H, S = p.S, WS = p.WS, NP = S + WS, B = p.B, rv = p.rv;
  // ---- merge weights: wave w takes sequences 4w .. 4w+3 of the chunk
  for (int q = 0; q < 4; ++q) {
    const int bl = 4 * wave + q, b = b0 + bl;
    float* wrow = wsm + bl * NP;
    if (b >= B) {
      for (int j = lane; j < NP; j += 64) wrow[j] = 0.f;
      if (lane == 0) inv[bl] = 0.f;
      continue;
    }
    auto pm = [&](int j) {
      return j < S ? p.part_ml[(((int64_t)b * S + j) * H + h) * 2] : p.win_ml[(((int64_t)b * WS + (j - S)) * H + h) * 2];
    };
    auto pl = [&](int j) {
      return j < S ? p.part_ml[(((int64_t)b * S + j) * H + h) * 2 + 1]
                   : p.win_ml[(((int64_t)b * WS + (j - S)) * H + h) * 2 + 1];
    };
    float mx = -INFINITY;
    for (int j = lane; j < NP; j += 64) mx = fmaxf(mx, pm(j));
    const float M = wave_max(mx);
    float ls = 0.f;
    for (int j = lane; j < NP; j += 64) {
      const float w = exp2_diff(pm(j), M);
      wrow[j] = w;
      ls += w * pl(j);
    }
    const float l = wave_sum(ls);
    if (lane == 0) inv[bl] = 1.f / l;
  }
  __syncthreads();
  // ---- O~ B_t: lane (row = sequence lane % 16, k group lane / 16)
  const int row = lane & 15, grp = lane >> 4;
  const int bA = min(b0 + row, B - 1);
  const float* wrow = wsm + row * NP;
  const float* po = p.part_o + ((int64_t)bA * S * H + h) * p.Dp;   // split s at + s H Dp
  const int64_t split_stride = (int64_t)H * p.Dp;
  const bf16* bt[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) bt[nb] = static_cast<const bf16*>(p.Bm) + ((int64_t)h * DH + 16 * nb + row) * rv;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = (rv + 31) / 32;
  const float w0 = wrow[0];
  for (int ks0 = wave; ks0 < nk; ks0 += 4 * KB) {
    f32x4 oa[KB][2];
    bf16x8 ba[KB][NB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int ks = min(ks0 + 4 * u, nk - 1);
      const int k = min(32 * ks + 8 * grp, rv - 8);   // clamped; zeroed below when past r_v
      oa[u][0] = *reinterpret_cast<const f32x4*>(po + k);
      oa[u][1] = *reinterpret_cast<const f32x4*>(po + k + 4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ba[u][nb] = *reinterpret_cast<const bf16x8*>(bt[nb] + k);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int ks = ks0 + 4 * u;
      if (ks >= nk) break;                           // wave-uniform
      const int k = 32 * ks + 8 * grp;
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = w0 * oa[u][0][e];
        o[e + 4] = w0 * oa[u][1][e];
      }
      for (int s = 1; s < S; ++s) {                  // further context splits (forced or long contexts)
        const float ws = wrow[s];
        const float* ps = po + s * split_stride + min(k, rv - 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += ws * ps[e];
      }
      bf16x8 a;
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = static_cast<bf16>(k < rv ? o[e] : 0.f);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba[u][nb], a, acc[nb], 0, 0, 0);
    }
  }
  // B_t^T rows are the A operand, so lane holds out[sequence row][e = 16 nb + 4 grp + r]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][row][16 * nb + 4 * grp + r] = acc[nb][r];
  __syncthreads();
  for (int x = tid; x < kSeqChunk * DH; x += kThreads) {
    const int bl = x / DH, e = x % DH, b = b0 + bl;
    if (b >= B) continue;
    float v = (red[0][bl][e] + red[1][bl][e]) + (red[2][bl][e] + red[3][bl][e]);
    const float* ww = wsm + bl * NP + S;
    for (int s = 0; s < WS; ++s) v += ww[s] * p.win_o[(((int64_t)b * WS + s) * H + h) * DH + e];
    static_cast<bf16*>(p.out)[((int64_t)b * H + h) * DH + e] = static_cast<bf16>(v * inv[bl]);
  }
}

}  // namespace

bool maps_wide_supports(const DecodeParams& p) {
  return p.bf16 && (p.dh == 64 || p.dh == 96 || p.dh == 128) && p.rv % 8 == 0 && p.S + p.WS <= 512;
}

hipError_t launch_qmap_wide(const DecodeParams& p, hipStream_t s) {
  if (!maps_wide_supports(p)) return hipErrorNotSupported;
  const int slab = p.rope_base != 0.f ? (kThreads / p.dh) * p.dh : kThreads;
  const dim3 grid((p.rk + slab - 1) / slab, p.H);
  switch (p.dh) {
    case 64: hipLaunchKernelGGL(k_qmap_wide<64>, grid, dim3(kThreads), 0, s, p); break;
    case 96: hipLaunchKernelGGL(k_qmap_wide<96>, grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL(k_qmap_wide<128>, grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_wide(const DecodeParams& p, hipStream_t s) {
  if (!maps_wide_supports(p) || p.mode != kAbsorbed) return hipErrorNotSupported;
  const dim3 grid(p.H, (p.B + kSeqChunk - 1) / kSeqChunk);
  const size_t lds = (size_t)kSeqChunk * (p.S + p.WS) * sizeof(float);
  switch (p.dh) {
    case 64: hipLaunchKernelGGL(k_combine_wide<64>, grid, dim3(kThreads), lds, s, p); break;
    case 96: hipLaunchKernelGGL(k_combine_wide<96>, grid, dim3(kThreads), lds, s, p); break;
    default: hipLaunchKernelGGL(k_combine_wide<128>, grid, dim3(kThreads), lds, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace lla
