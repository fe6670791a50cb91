// Latent writer on the gfx950 matrix cores ("Hybrid Latent Attention"
// summary, "Latent Writer", Eq. 2).  Per group, the writer is one GEMM
//     c[tokens x (r_k+r_v)] = sum_t X_t[tokens x d_in] . E_t^T[d_in x (r_k+r_v)]
// with the loops concatenated along K.  The matrices are short and wide
// (a decode step writes one token per sequence), so the GEMM is split along
// K across workgroups: each writes an fp32 partial tile to the workspace, and
// a second kernel sums the partials in a fixed order, rotates the key part
// by R~_p when the set bakes rotary embedding, rounds to bf16 and scatters
// into the paged store.
//   v_mfma_f32_16x16x32_bf16: A = 8 consecutive inputs of one token (16-B
//   load from x), B = 8 consecutive inputs of one encoder row (16-B load
//   from E_t), both in their natural row-major layouts.
#include <algorithm>

#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileM = 64;   // tokens per workgroup (16 per wave)
constexpr int kTileN = 64;   // latent outputs per workgroup
constexpr int kUnroll = 4;   // K steps whose loads are issued together

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<bf16>(0.f);
  return z;
}

__global__ __launch_bounds__(kThreads) void k_writer_mfma(WriterParams p) {
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int g = blockIdx.z / p.ksplit, ks = blockIdx.z % p.ksplit;
  const int M = p.B * p.n_tok, R = p.R, d_in = p.d_in, G = p.G;
  const int ksteps = p.n_loops * d_in / 32;
  const int per = (ksteps + p.ksplit - 1) / p.ksplit;
  const int s0 = ks * per, s1 = min(ksteps, s0 + per);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int m = mt * kTileM + wave * 16 + col;       // A-operand row (token)
  const bool m_ok = m < M;
  const bf16* x = static_cast<const bf16*>(p.x);
  const bf16* enc = static_cast<const bf16*>(p.enc);
  f32x4 acc[kTileN / 16];
#pragma unroll
  for (int j = 0; j < kTileN / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool n_ok[kTileN / 16];
#pragma unroll
  for (int j = 0; j < kTileN / 16; ++j) n_ok[j] = nt * kTileN + 16 * j + col < R;

  for (int st = s0; st < s1; st += kUnroll) {
    bf16x8 a[kUnroll], bb[kUnroll][kTileN / 16];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k0 = (st + u) * 32;
      const bool ok = st + u < s1;
      const int t = k0 / d_in, kk = k0 % d_in + grp * 8;
      a[u] = (ok && m_ok) ? *reinterpret_cast<const bf16x8*>(
                                x + (((int64_t)m * p.n_loops + t) * G + g) * d_in + kk)
                          : zero8();
#pragma unroll
      for (int j = 0; j < kTileN / 16; ++j) {
        const int n = nt * kTileN + 16 * j + col;
        bb[u][j] = (ok && n_ok[j]) ? *reinterpret_cast<const bf16x8*>(
                                         enc + (((int64_t)t * G + g) * R + n) * d_in + kk)
                                   : zero8();
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < kTileN / 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bb[u][j], acc[j], 0, 0, 0);
  }
  // lane holds C[row 4*grp + r][col] of each 16x16 tile
#pragma unroll
  for (int j = 0; j < kTileN / 16; ++j) {
    const int n = nt * kTileN + 16 * j + col;
    if (!n_ok[j]) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = mt * kTileM + wave * 16 + 4 * grp + r;
      if (mm < M) p.acc[(((int64_t)ks * M + mm) * G + g) * R + n] = acc[j][r];
    }
  }
}

// Sum the K-split partials of one (token, group), then rotate/round/scatter.
__global__ __launch_bounds__(kThreads) void k_writer_reduce(WriterParams p) {
  extern __shared__ float c[];
  __shared__ double theta[128];     // d_h / 2 <= 128
  const int m = blockIdx.x, g = blockIdx.y;
  if (p.rope_baked && (int)threadIdx.x < p.dh / 2) theta[threadIdx.x] = rope_theta(p.rope_base, p.dh, threadIdx.x);
  const int M = p.B * p.n_tok, R = p.R, G = p.G;
  for (int o = threadIdx.x; o < R; o += kThreads) {
    float v = 0.f;
    for (int ks = 0; ks < p.ksplit; ++ks) v += p.acc[(((int64_t)ks * M + m) * G + g) * R + o];
    c[o] = v;
  }
  __syncthreads();
  const int b = m / p.n_tok, n = m % p.n_tok;
  const int R_ = R, rk = p.rk, dh = p.dh, half = dh / 2;
  const int pos = p.pos[(int64_t)b * p.n_tok + n];
  const int64_t page = p.bt[(int64_t)b * p.max_pages + pos / p.P];
  const int slot = pos % p.P;
  bf16* pages = static_cast<bf16*>(p.pages);
  for (int o = threadIdx.x; o < R_; o += kThreads) {
    float v = c[o];
    int64_t off;
    if (o < rk) {
      if (p.rope_baked) {
        const int f = o % dh;
        float cs, sn;
        if (f < half) {
          rope_cs_theta(theta[f], pos, cs, sn);
          v = c[o] * cs - c[o + half] * sn;
        } else {
          rope_cs_theta(theta[f - half], pos, cs, sn);
          v = c[o - half] * sn + c[o] * cs;
        }
      }
      off = key_off(page, g, slot, o, G, p.P, R_, rk);
    } else {
      off = val_off(page, g, slot, o - rk, G, p.P, R_, rk);
    }
    pages[off] = static_cast<bf16>(v);
  }
}

}  // namespace

bool writer_mfma_supports(const WriterParams& p) { return p.bf16 && p.d_in % 32 == 0; }

int writer_mfma_ksplit(int M, int G, int R, int n_loops, int d_in) {
  const int64_t tiles = (int64_t)((R + kTileN - 1) / kTileN) * ((M + kTileM - 1) / kTileM) * G;
  const int ksteps = n_loops * d_in / 32;
  int64_t ks = (512 + tiles - 1) / tiles;
  ks = std::min<int64_t>(ks, std::max(1, ksteps / 8));
  return (int)std::max<int64_t>(ks, 1);
}

hipError_t launch_writer_mfma(const WriterParams& p, hipStream_t s) {
  if (!writer_mfma_supports(p)) return hipErrorNotSupported;
  const int M = p.B * p.n_tok;
  const dim3 grid((p.R + kTileN - 1) / kTileN, (M + kTileM - 1) / kTileM, p.G * p.ksplit);
  hipLaunchKernelGGL(k_writer_mfma, grid, dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_writer_reduce, dim3(M, p.G), dim3(kThreads), (size_t)p.R * sizeof(float), s, p);
  return hipGetLastError();
}

}  // namespace lla
