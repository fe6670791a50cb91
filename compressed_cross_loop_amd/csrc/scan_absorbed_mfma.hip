// Absorbed latent scan on the gfx950 matrix cores: the hot loop of the
// direct latent read ("Hybrid Latent Attention" summary, "Latent Reader",
// Eqs. 3-4; LLA-D of the Looped Latent Attention abstract).
//
// One workgroup = one (context split, sequence, latent group); its four waves
// take interleaved 16-token tiles of the split.  Every head of the group
// reads the same latent row, so a tile is streamed from HBM once for all
// heads: the heads are the N dimension of both contractions.
//
//   scores   S^T[16 tok x 16 heads] = C^K[16 x r_k] . Q~^T[r_k x 16]
//            v_mfma_f32_16x16x32_bf16, A = key rows straight from the store
//            (token-major: 8 consecutive dims per lane, one 16-B load)
//   softmax  per head, online, exp2 domain (q~ carries log2(e)/sqrt(d_h));
//            the tile max is reduced over the 4 lane groups holding a head
//   values   O^T[r_v x 16 heads] += C^V^T[r_v x 16 tok] . P^T[16 tok x 16]
//            v_mfma_f32_16x16x16_bf16, A = value sub-blocks straight from
//            the store (dimension-major 16x16 blocks: one 8-B load per lane,
//            512 contiguous bytes per wave), B = the probabilities exactly
//            as the score MFMA left them in registers (its C layout is this
//            MFMA's B layout), rounded to bf16
//
// The tile loop is software-pipelined: the next tile's key loads are issued
// right after the score MFMAs, its value loads right after the value MFMAs.  At the end the
// four waves are merged (same-max rescale, fixed order) in LDS and one
// partial (m, l, O_latent) per head is written for the combine kernel.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int RK>
__device__ __forceinline__ void load_keys(bf16x8 (&k)[RK / 32], const bf16* tile, int col, int grp) {
  const bf16* kp = tile + col * RK + grp * 8;
#pragma unroll
  for (int st = 0; st < RK / 32; ++st) k[st] = *reinterpret_cast<const bf16x8*>(kp + st * 32);
}

template <int RK, int RV>
__device__ __forceinline__ void load_values(s16x4 (&v)[RV / 16], const bf16* tile, int col, int grp) {
  const bf16* vp = tile + 16 * RK + col * 16 + grp * 4;
#pragma unroll
  for (int vt = 0; vt < RV / 16; ++vt) v[vt] = *reinterpret_cast<const s16x4*>(vp + vt * 256);
}

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, static_cast<bf16>(x));
}

// Scores of one tile; lane (head = lane&15, grp) gets tokens 4*grp + r.
template <int RK>
__device__ __forceinline__ f32x4 tile_scores(const bf16x8 (&k)[RK / 32], const bf16x8 (&qreg)[RK / 32]) {
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < RK / 32; ++st)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[st], qreg[st], sc, 0, 0, 0);
  return sc;
}

// Online-softmax update for one tile; returns the bf16 probabilities in the
// B-operand layout of the value MFMA.
template <int RV>
__device__ __forceinline__ s16x4 tile_softmax(f32x4 sc, f32x4 (&acc)[RV / 16], float& m, float& lsum,
                                              int nvalid, int grp) {
  if (nvalid < 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * grp + r >= nvalid) sc[r] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(m, mx);
  const float alpha = exp2_diff(m, mn);
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = exp2f(sc[r] - mn);
  lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  m = mn;
  // rescale only when some head's running max moved (rare after a few tiles)
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int vt = 0; vt < RV / 16; ++vt) acc[vt] *= alpha;
  }
  s16x4 pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) pb[r] = bf16_bits(pr[r]);
  return pb;
}

template <int RV>
__device__ __forceinline__ void tile_values(s16x4 (&v)[RV / 16], s16x4 pb, f32x4 (&acc)[RV / 16],
                                            int nvalid, int grp) {
  if (nvalid < 16) {
    // tokens past the end may hold anything (even NaN): zero their values
#pragma unroll
    for (int vt = 0; vt < RV / 16; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * grp + r >= nvalid) v[vt][r] = 0;
  }
#pragma unroll
  for (int vt = 0; vt < RV / 16; ++vt)
    acc[vt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v[vt], pb, acc[vt], 0, 0, 0);
}

template <int RK, int RV>
__global__ __launch_bounds__(kThreads, 1) void k_scan_absorbed_mfma(DecodeParams p) {
  const int s = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int hpg = p.hpg, G = p.G, P = p.P;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;

  // q~ of the group's heads, as the B operand of the score MFMA
  bf16x8 qreg[RK / 32];
  {
    const bf16* qsrc = static_cast<const bf16*>(p.qlat) +
                       ((int64_t)b * p.H + (int64_t)g * hpg + col) * RK + grp * 8;
#pragma unroll
    for (int st = 0; st < RK / 32; ++st) {
      if (col < hpg) {
        qreg[st] = *reinterpret_cast<const bf16x8*>(qsrc + st * 32);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[st][e] = static_cast<bf16>(0.f);
      }
    }
  }
  f32x4 acc[RV / 16];
#pragma unroll
  for (int vt = 0; vt < RV / 16; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const int R = RK + RV;
  const int ntiles = (t1 - t0 + 15) / 16;
  auto tile_ptr = [&](int ti) -> const bf16* {
    const int j0 = t0 + ti * 16;
    const int64_t page = bt[j0 / P];
    return pages + tile_base(page, g, j0 % P, G, P, R);
  };
  auto tile_valid = [&](int ti) -> int { return min(16, t1 - (t0 + ti * 16)); };

  // Staggered pipeline: the next tile's keys are requested as soon as the
  // score MFMAs have consumed the current ones, its values as soon as the
  // value MFMAs have; about one tile per wave stays in flight.
  bf16x8 kreg[RK / 32];
  s16x4 vreg[RV / 16];
  int ti = wave;
  if (ti < ntiles) {
    const bf16* tp = tile_ptr(ti);
    load_keys<RK>(kreg, tp, col, grp);
    load_values<RK, RV>(vreg, tp, col, grp);
  }
  while (ti < ntiles) {
    const int tn = ti + kWaves;
    const int nvalid = tile_valid(ti);
    const bf16* np = (tn < ntiles) ? tile_ptr(tn) : nullptr;
    const f32x4 sc = tile_scores<RK>(kreg, qreg);
    if (np) load_keys<RK>(kreg, np, col, grp);
    const s16x4 pb = tile_softmax<RV>(sc, acc, m, lsum, nvalid, grp);
    tile_values<RV>(vreg, pb, acc, nvalid, grp);
    if (np) load_values<RK, RV>(vreg, np, col, grp);
    ti = tn;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // ---- merge the four waves (fixed order) and write the split's partial
  __shared__ float mw[kWaves][16];
  __shared__ float lw[kWaves][16];
  __shared__ float osum[16 * (RV + 1)];   // [head][dim], padded rows
  if (grp == 0) {
    mw[wave][col] = m;
    lw[wave][col] = lsum;
  }
  __syncthreads();
  float M = mw[0][col];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w][col]);
  const float f = exp2_diff(m, M);
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int vt = 0; vt < RV / 16; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int idx = col * (RV + 1) + vt * 16 + grp * 4 + r;
          const float v = f * acc[vt][r];
          osum[idx] = (w == 0) ? v : osum[idx] + v;
        }
    }
    __syncthreads();
  }
  const int64_t row0 = ((int64_t)b * p.S + s) * p.H + (int64_t)g * hpg;
  if (tid < hpg) {
    float Mh = mw[0][tid], l = 0.f;
    for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, mw[w][tid]);
    for (int w = 0; w < kWaves; ++w) l += exp2_diff(mw[w][tid], Mh) * lw[w][tid];
    p.part_ml[(row0 + tid) * 2 + 0] = Mh;
    p.part_ml[(row0 + tid) * 2 + 1] = l;
  }
  for (int x = tid; x < hpg * RV; x += kThreads) {
    const int h = x / RV, d = x % RV;
    p.part_o[(row0 + h) * p.Dp + d] = osum[h * (RV + 1) + d];
  }
}

template <int RK, int RV>
hipError_t launch_rk(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((k_scan_absorbed_mfma<RK, RV>), dim3(p.S, p.B, p.G), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool scan_absorbed_mfma_supports(const DecodeParams& p) {
  if (!p.bf16 || p.hpg > 16 || p.rk != p.rv) return false;
  switch (p.rk) {
    case 32: case 64: case 128: case 256: case 512: return true;
    default: return false;
  }
}

hipError_t launch_scan_absorbed_mfma(const DecodeParams& p, hipStream_t s) {
  if (!scan_absorbed_mfma_supports(p)) return hipErrorNotSupported;
  switch (p.rk) {
    case 32: return launch_rk<32, 32>(p, s);
    case 64: return launch_rk<64, 64>(p, s);
    case 128: return launch_rk<128, 128>(p, s);
    case 256: return launch_rk<256, 256>(p, s);
    default: return launch_rk<512, 512>(p, s);
  }
}

}  // namespace lla
