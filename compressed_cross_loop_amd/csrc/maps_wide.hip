// Query map and combine for the absorbed read of one wide latent shared by
// all heads ("Hybrid Latent Attention" summary, "Latent Reader": q~ = A_t^T q
// before the scan, o = B_t^T O~ / l after it; LLA-D of the Looped Latent
// Attention abstract).  With r in the thousands each head's A_t and B_t^T are
// about a MiB, so these kernels take every sequence of a head together and
// read each map once per workgroup, instead of once per (sequence, head).
//
//   k_qmap_wide     workgroup = (slab of latent dims, head): the slab of A_t
//                   staged in LDS once, then every sequence on the matrix
//                   cores.  RoPE on the latent (frequency-paired decoders)
//                   rotates dim pairs (f, f + d_h/2) inside each d_h block,
//                   exchanged in LDS.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSeqChunk = 16;   // sequences per LDS round of the query map / per combine workgroup

// ---------------------------------------------------------------- query map
// q~^T[n][b] = sum_e A_t[e][n] q[b][e] for a slab of latent dims n and every
// sequence b, on the matrix cores (v_mfma_f32_16x16x16_bf16, M = 16 latent
// dims, N = 16 sequences, K = d_h).  The slab of A_t (d_h rows of 512
// contiguous bytes) is staged in LDS once; A_t is stored with the latent axis
// contiguous, so its fragments (four consecutive e of one n per lane) come
// back through the transposing LDS read ds_read_b64_tr_b16.  q fragments are
// 8-byte loads.  Rows are padded by 32 bytes so that the 16 rows one
// transposing read touches fall in different banks.
template <int DH, bool ROPE>
__global__ __launch_bounds__(kThreads) void k_qmap_wide(DecodeParams p) {
  constexpr int HALF = DH / 2, KS = DH / 16, LDA = kThreads + 16;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) bf16 at[DH * LDA];
  // rotation exchange buffers (one element when there is no rotation, so that
  // more workgroups fit a CU)
  __shared__ float ub[ROPE ? kSeqChunk : 1][ROPE ? kThreads + 4 : 1];
  __shared__ float cs[ROPE ? kSeqChunk : 1][ROPE ? HALF : 1][2];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int H = p.H, rk = p.rk, B = p.B;
  constexpr bool rope = ROPE;   // = (rope_base != 0)
  const int slab = rope ? (kThreads / DH) * DH : kThreads;   // whole d_h blocks when rotating
  const int n0 = blockIdx.x * slab;
  {
    // A_t[e][n0 .. n0 + slab): 16-byte pieces, columns past r_k clamped (never
    // stored); every load of a thread is issued before the first LDS write
    constexpr int NP = DH * (kThreads / 8) / kThreads;   // pieces per thread at the widest slab
    const bf16* Ah = static_cast<const bf16*>(p.A) + (int64_t)h * DH * rk;
    const int pr = slab / 8, npc = DH * pr;
    u32x4 r[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int x = min(tid + kThreads * k, npc - 1), e = x / pr, c = x % pr;
      r[k] = *reinterpret_cast<const u32x4*>(Ah + (int64_t)e * rk + min(n0 + 8 * c, rk - 8));
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int x = tid + kThreads * k, e = x / pr, c = x % pr;
      if (x < npc) *reinterpret_cast<u32x4*>(&at[e * LDA + 8 * c]) = r[k];
    }
  }
  __syncthreads();
  // q~ leaves as bf16 hi and lo parts (lo = the rounding remainder, at
  // qlat + B H r_k), so that the score pass keeps it at fp32-level accuracy
  bf16* ql = static_cast<bf16*>(p.qlat);
  const int64_t qlo = (int64_t)B * H * rk;
  const int nblk = slab / 16;
  // B operand: q[b0 + col][16 ks + 4 grp .. + 3], one chunk ahead
  s16x4 qn[KS];
  auto q_load = [&](int b0) {
    const bf16* q = static_cast<const bf16*>(p.q) + ((int64_t)min(b0 + col, B - 1) * H + h) * DH + 4 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qn[ks] = *reinterpret_cast<const s16x4*>(q + 16 * ks);
  };
  q_load(0);
  for (int b0 = 0; b0 < B; b0 += kSeqChunk) {
    const int nb = min(kSeqChunk, B - b0);
    if (rope) {
      for (int x = tid; x < nb * HALF; x += kThreads) {
        const int bb = x / HALF, f = x % HALF;
        float c, s;
        rope_cs(p.rope_base, DH, f, p.pos[b0 + bb], c, s);
        cs[bb][f][0] = c;
        cs[bb][f][1] = s;
      }
    }
    s16x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
    if (b0 + kSeqChunk < B) q_load(b0 + kSeqChunk);
    for (int blk = wave; blk < nblk; blk += 4) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // lane l of the 16-lane group points at A_t[16 ks + 4 grp + l / 4][16 blk + 4 (l % 4)]
        const bf16* a = &at[(16 * ks + 4 * grp + (col >> 2)) * LDA + 16 * blk + 4 * (col & 3)];
        const s16x4 af = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, qf[ks], acc, 0, 0, 0);
      }
      // lane holds q~[sequence b0 + col][n0 + 16 blk + 4 grp + r]
      const int nl = 16 * blk + 4 * grp;
      if (rope) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ub[col][nl + r] = acc[r];
      } else if (col < nb && n0 + nl < rk) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v, w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[r] * p.scale;
          v[r] = static_cast<bf16>(x);
          w[r] = static_cast<bf16>(x - static_cast<float>(v[r]));
        }
        const int64_t o = ((int64_t)(b0 + col) * H + h) * rk + n0 + nl;
        *reinterpret_cast<bf16x4*>(ql + o) = v;
        *reinterpret_cast<bf16x4*>(ql + qlo + o) = w;
      }
    }
    if (rope) {
      __syncthreads();
      for (int x = tid; x < nb * slab; x += kThreads) {
        const int bb = x / slab, t = x % slab, n = n0 + t;
        if (n >= rk) continue;
        const int f = t % DH;   // n0 is a multiple of d_h, so the partner is in this slab
        const int fp = f < HALF ? f : f - HALF;
        const float c = cs[bb][fp][0], sn = cs[bb][fp][1];
        const float u = ub[bb][t];
        const float v = f < HALF ? u * c - ub[bb][t + HALF] * sn : ub[bb][t - HALF] * sn + u * c;
        const float xs = v * p.scale;
        const bf16 hi = static_cast<bf16>(xs);
        const int64_t o = ((int64_t)(b0 + bb) * H + h) * rk + n;
        ql[o] = hi;
        ql[qlo + o] = static_cast<bf16>(xs - static_cast<float>(hi));
      }
      __syncthreads();   // ub and cs are refilled next round
    }
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
  // workgroups are dealt to the 8 XCDs round-robin: every 16-sequence chunk of
  // head h gets an id = h (mod 8), so B_h is fetched into one L2 only
  const int span = 8 * ((p.B + kSeqChunk - 1) / kSeqChunk);
  const int h = (blockIdx.x / span) * 8 + (blockIdx.x % 8), b0 = (blockIdx.x % span) / 8 * kSeqChunk;
  if (h >= p.H) return;   // the id padding of the last 8 heads; before any barrier
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
  // the wide scan leaves its partials in bf16 (rows of Dp elements)
  const bf16* po = reinterpret_cast<const bf16*>(p.part_o) + ((int64_t)bA * S * H + h) * p.Dp;   // split s at + s H Dp
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
    bf16x8 oa[KB];
    bf16x8 ba[KB][NB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int ks = min(ks0 + 4 * u, nk - 1);
      const int k = min(32 * ks + 8 * grp, rv - 8);   // clamped; zeroed below when past r_v
      oa[u] = *reinterpret_cast<const bf16x8*>(po + k);
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
        o[e] = w0 * static_cast<float>(oa[u][e]);
        o[e + 4] = w0 * static_cast<float>(oa[u][e + 4]);
      }
      for (int s = 1; s < S; ++s) {                  // further context splits (forced or long contexts)
        const float ws = wrow[s];
        const bf16x8 ps = *reinterpret_cast<const bf16x8*>(po + s * split_stride + min(k, rv - 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += ws * static_cast<float>(ps[e]);
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

template <int DH>
void launch_qmap_dh(const DecodeParams& p, dim3 grid, hipStream_t s) {
  if (p.rope_base != 0.f)
    hipLaunchKernelGGL((k_qmap_wide<DH, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_qmap_wide<DH, false>), grid, dim3(kThreads), 0, s, p);
}

hipError_t launch_qmap_wide(const DecodeParams& p, hipStream_t s) {
  if (!maps_wide_supports(p)) return hipErrorNotSupported;
  const int slab = p.rope_base != 0.f ? (kThreads / p.dh) * p.dh : kThreads;
  const dim3 grid((p.rk + slab - 1) / slab, p.H);
  switch (p.dh) {
    case 64: launch_qmap_dh<64>(p, grid, s); break;
    case 96: launch_qmap_dh<96>(p, grid, s); break;
    default: launch_qmap_dh<128>(p, grid, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_wide(const DecodeParams& p, hipStream_t s) {
  if (!maps_wide_supports(p) || p.mode != kAbsorbed || !p.part_bf16) return hipErrorNotSupported;
  const dim3 grid((p.H + 7) / 8 * 8 * ((p.B + kSeqChunk - 1) / kSeqChunk));
  const size_t lds = (size_t)kSeqChunk * (p.S + p.WS) * sizeof(float);
  switch (p.dh) {
    case 64: hipLaunchKernelGGL(k_combine_wide<64>, grid, dim3(kThreads), lds, s, p); break;
    case 96: hipLaunchKernelGGL(k_combine_wide<96>, grid, dim3(kThreads), lds, s, p); break;
    default: hipLaunchKernelGGL(k_combine_wide<128>, grid, dim3(kThreads), lds, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace lla
