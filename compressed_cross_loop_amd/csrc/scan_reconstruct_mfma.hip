// Reconstruct-on-read latent scan for per-head Looped Latent Attention on the
// gfx950 matrix cores ("Looped Latent Attention" abstracts: the codec
// "reconstructs loop-specific K/V vectors only when attention reads them").
//
// One wave per head (each head has its own latent group), four waves per
// workgroup, one workgroup per (context split, sequence, 4 heads).  Per
// 16-token tile the wave rebuilds, for its head,
//   K^ [16 tok x d_h] = S^K [16 x r] . A^T [r x d_h]   (v_mfma_f32_16x16x32_bf16)
//   V^ [16 tok x d_h] = S^V [16 x r] . B_t [r x d_h]   (same)
// then scores K^ q' (the 16 lanes holding one token row reduce), an online
// softmax over the tile, and o += p . V^.  Both decoders are stored [d_h][r]
// (rows contiguous along the latent axis), so each B-operand fragment is one
// 16-byte load; they are held in registers for the whole scan.  Key rows are
// token-major in the store (one 16-byte load per lane); the tile's value block
// is stored dimension-major (for the absorbed read), so each wave transposes
// it through its own LDS slice before the V^ product.  Several tiles are kept
// in flight.
#include <type_traits>

#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int R, int DH>
__global__ __launch_bounds__(kThreads, 2) void k_scan_reconstruct_mfma(DecodeParams p) {
  constexpr int NT = DH / 16;     // column tiles of d_h
  constexpr int KS = R / 32;      // K steps over the latent width
  constexpr int VC = R / 32;      // 16-byte value chunks per lane per tile (16 tok x R / 64 lanes / 8)
  constexpr int kPF = R == 32 ? 8 : 2;   // tiles in flight per wave
  __shared__ __attribute__((aligned(16))) bf16 vt[kWaves][16][R + 8];
  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.z * kWaves + wave;
  if (h >= p.H) return;
  const int g = h / p.hpg;
  const int G = p.G, P = p.P, Rt = 2 * R;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;

  // decoders of this head, in B-operand layout (lane: column e = 16 nt + col,
  // 8 consecutive latent dims 32 st + 8 grp ..)
  const bf16* Ah = static_cast<const bf16*>(p.A) + (int64_t)h * DH * R;   // [DH][R]
  const bf16* Bh = static_cast<const bf16*>(p.Bm) + (int64_t)h * DH * R;  // B_t^T: [DH][R]
  bf16x8 af[NT][KS], bfr[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      af[nt][st] = *reinterpret_cast<const bf16x8*>(Ah + (int64_t)(16 * nt + col) * R + 32 * st + 8 * grp);
      bfr[nt][st] = *reinterpret_cast<const bf16x8*>(Bh + (int64_t)(16 * nt + col) * R + 32 * st + 8 * grp);
    }
  float qv[NT];
  {
    const float* qh = p.qhead + ((int64_t)b * p.H + h) * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qv[nt] = qh[16 * nt + col];
  }

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const int ntiles = (t1 - t0 + 15) / 16;
  auto tile_ptr = [&](int ti) -> const bf16* {
    const int j0 = t0 + min(ti, ntiles - 1) * 16;
    return pages + tile_base(bt[j0 / P], g, j0 % P, G, P, Rt);
  };
  struct Buf {
    bf16x8 k[KS];
    bf16x8 v[VC];
  };
  auto load = [&](Buf& buf, int ti) {
    const bf16* tp = tile_ptr(ti);
#pragma unroll
    for (int st = 0; st < KS; ++st)
      buf.k[st] = *reinterpret_cast<const bf16x8*>(tp + col * R + 32 * st + 8 * grp);
#pragma unroll
    for (int c = 0; c < VC; ++c)   // value block: 16 * R contiguous elements
      buf.v[c] = *reinterpret_cast<const bf16x8*>(tp + 16 * R + (c * 64 + lane) * 8);
  };

  float m = -INFINITY, lsum = 0.f, o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = 0.f;

  // FULL: all 16 tokens of the tile are valid (every tile but a ragged last
  // one), so no masking
  auto step = [&](const Buf& buf, int nvalid, auto full) {
    constexpr bool FULL = decltype(full)::value;
    // rebuild keys: lane holds K^[tok 4 grp + r][e = 16 nt + col]
    f32x4 kh[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      kh[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        kh[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(buf.k[st], af[nt][st], kh[nt], 0, 0, 0);
    }
    // value block -> LDS, token-major: element x of the block is
    // (sub-block x/256, dim-in-block (x%256)/16, token x%16)
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      const int x0 = (c * 64 + lane) * 8;
      const int r = (x0 / 256) * 16 + (x0 % 256) / 16, tk = x0 % 16;
#pragma unroll
      for (int k = 0; k < 8; ++k) vt[wave][tk + k][r] = buf.v[c][k];
    }
    // scores of the rebuilt keys against q'
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) a += qv[nt] * kh[nt][r];
      a = row_sum16(a);   // the 16 lanes of this lane group hold one token row
      sc[r] = (FULL || 4 * grp + r < nvalid) ? a : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_diff(m, mn);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - mn);
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = mn;
    if (alpha != 1.f) {   // uniform: the wave holds one head
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
    }
    // rebuild values: A operand = token rows of the transposed block
    bf16x8 sv[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) sv[st] = *reinterpret_cast<const bf16x8*>(&vt[wave][col][32 * st + 8 * grp]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 vh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) vh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv[st], bfr[nt][st], vh, 0, 0, 0);
      float acc = o[nt];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += (FULL || 4 * grp + r < nvalid) ? pr[r] * vh[r] : 0.f;
      o[nt] = acc;
    }
  };

  if (ntiles > 0) {
    Buf buf[kPF];
#pragma unroll
    for (int u = 0; u < kPF; ++u) load(buf[u], u);
    for (int base = 0; base < ntiles; base += kPF) {
#pragma unroll
      for (int u = 0; u < kPF; ++u) {
        if (base + u < ntiles) {
          const int nvalid = min(16, t1 - (t0 + (base + u) * 16));
          if (nvalid == 16)
            step(buf[u], 16, std::true_type{});
          else
            step(buf[u], nvalid, std::false_type{});
        }
        load(buf[u], base + u + kPF);   // clamped: always a valid tile
      }
    }
  }
  // totals over the four lane groups (each held 4 tokens per tile)
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    o[nt] += __shfl_xor(o[nt], 16);
    o[nt] += __shfl_xor(o[nt], 32);
  }
  const int64_t row = ((int64_t)b * p.S + s) * p.H + h;
  if (lane == 0) {
    p.part_ml[row * 2 + 0] = m;
    p.part_ml[row * 2 + 1] = lsum;
  }
  if (grp == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) p.part_o[row * p.Dp + 16 * nt + col] = o[nt];
  }
}

template <int R, int DH>
hipError_t launch_r(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(p.S, p.B, (p.H + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((k_scan_reconstruct_mfma<R, DH>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool scan_reconstruct_mfma_supports(const DecodeParams& p) {
  return p.bf16 && p.hpg == 1 && p.rk == p.rv && (p.rk == 32 || p.rk == 64) &&
         (p.dh == 64 || p.dh == 128);
}

hipError_t launch_scan_reconstruct_mfma(const DecodeParams& p, hipStream_t s) {
  if (!scan_reconstruct_mfma_supports(p)) return hipErrorNotSupported;
  if (p.rk == 32) return p.dh == 128 ? launch_r<32, 128>(p, s) : launch_r<32, 64>(p, s);
  return p.dh == 128 ? launch_r<64, 128>(p, s) : launch_r<64, 64>(p, s);
}

}  // namespace lla
