// Reconstruct-on-read for head-folded latents (LLA-2D: one K and one V latent
// per token shared by all heads; "Looped Latent Attention" abstracts) on the
// gfx950 matrix cores.  Rebuilding every head's keys and values is a GEMM per
// sequence,
//   K^[tokens x H d_h] = S^K[tokens x r] . A^T[r x H d_h]
//   V^[tokens x H d_h] = S^V[tokens x r] . B_t[r x H d_h]
// with an attention epilogue per head, so it is tiled like a GEMM: one
// workgroup per (context split, sequence, 2 heads), 128-token tiles, K-loop
// over the latent width in steps of 32.  Each step stages four operand tiles
// in LDS (key rows and both decoders' rows as they are stored; the
// dimension-major value blocks transposed on the way in) while the next
// step's global loads are in flight.  Eight waves: wave w computes K^ (w even) or V^
// (w odd) of head (w/2)%2 for token half w/4 (4 x d_h/16
// v_mfma_f32_16x16x32_bf16 tiles).  After a tile, the K waves score against
// q' into LDS and the V waves run the online softmax and o += p . V^.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int TM = 128;     // tokens per tile
constexpr int KC = 32;      // latent dims per K step
constexpr int LD = KC + 8;  // padded LDS row (80 bytes: 16 lanes hit distinct bank quads)

template <int DH>
__global__ __launch_bounds__(kThreads, 1) void k_scan_reconstruct_gemm(DecodeParams p) {
  constexpr int NT = DH / 16;        // column tiles per head
  constexpr int MT = TM / 2 / 16;    // row tiles per wave (half of the token tile)
  __shared__ __attribute__((aligned(16))) bf16 sk[TM][LD];
  __shared__ __attribute__((aligned(16))) bf16 sv[TM][LD];
  __shared__ __attribute__((aligned(16))) bf16 uk[2 * DH][LD];
  __shared__ __attribute__((aligned(16))) bf16 uv[2 * DH][LD];
  __shared__ float sc[2][TM];
  __shared__ float ox[2][DH + 1];    // second token half's o and l, per head

  const int s = blockIdx.x, b = blockIdx.y, hb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int kind = wave & 1, hl = (wave >> 1) & 1, mh = wave >> 2;   // K^/V^, head, token half
  const int H = p.H, R = p.rk, Rt = 2 * p.rk, P = p.P;
  const int h = 2 * hb + hl;
  const bool head_ok = h < H;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;
  const int ntile = (t1 - t0 + TM - 1) / TM;
  const int nks = R / KC;

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const bf16* A = static_cast<const bf16*>(p.A);    // [H][DH][R]
  const bf16* Bm = static_cast<const bf16*>(p.Bm);  // B_t^T: [H][DH][R]

  float qv[NT];
  {
    const float* qh = p.qhead + ((int64_t)b * H + (head_ok ? h : 0)) * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qv[nt] = qh[16 * nt + col];
  }

  // ---- staging.  Thread tid stages one key chunk and one value chunk of
  // 16-token sub-tile `wave` (its base pointer is resolved once per tile and
  // clamped so that a sub-tile past the end rereads the last valid one,
  // masked later), plus A-row and B-row chunks of the two heads.
  constexpr int NU = (2 * DH * KC / 8 + kThreads - 1) / kThreads;
  bf16x8 rsk, rsv, ruk[NU], ruv[NU];
  const bf16* sub = pages;
  auto set_tile = [&](int tile) {
    int j = min(t0 + tile * TM + 16 * wave, t1 - 1);
    j -= j & 15;
    sub = pages + tile_base(bt[j / P], 0, j % P, 1, P, Rt);
  };
  const int krow = (tid >> 2) & 15, kpart = tid & 3;
  const int vb = (tid >> 5) & 1, r16 = (tid >> 1) & 15, vhalf = tid & 1;
  auto load_step = [&](int ks) {
    rsk = *reinterpret_cast<const bf16x8*>(sub + krow * R + ks * KC + kpart * 8);
    rsv = *reinterpret_cast<const bf16x8*>(sub + 16 * R + (2 * ks + vb) * 256 + r16 * 16 + 8 * vhalf);
#pragma unroll
    for (int u = 0; u < NU; ++u) {   // A rows: 2 heads x DH rows x 4 chunks
      const int c = min(tid + u * kThreads, 2 * DH * KC / 8 - 1);
      const int row = c / 4, part = c % 4;
      const int hh = min(2 * hb + row / DH, H - 1), e = row % DH;
      ruk[u] = *reinterpret_cast<const bf16x8*>(A + ((int64_t)hh * DH + e) * R + ks * KC + part * 8);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {   // B_t^T rows: 2 heads x DH rows x 4 chunks
      const int c = min(tid + u * kThreads, 2 * DH * KC / 8 - 1);
      const int row = c / 4, part = c % 4;
      const int hh = min(2 * hb + row / DH, H - 1), e = row % DH;
      ruv[u] = *reinterpret_cast<const bf16x8*>(Bm + ((int64_t)hh * DH + e) * R + ks * KC + part * 8);
    }
  };
  auto store_step = [&]() {
    *reinterpret_cast<bf16x8*>(&sk[16 * wave + krow][kpart * 8]) = rsk;
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[16 * wave + 8 * vhalf + k][16 * vb + r16] = rsv[k];   // transpose
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = tid + u * kThreads;
      if (c < 2 * DH * KC / 8) *reinterpret_cast<bf16x8*>(&uk[c / 4][(c % 4) * 8]) = ruk[u];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = tid + u * kThreads;
      if (c < 2 * DH * KC / 8) *reinterpret_cast<bf16x8*>(&uv[c / 4][(c % 4) * 8]) = ruv[u];
    }
  };

  float m = -INFINITY, l = 0.f, o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = 0.f;

  if (ntile > 0) {
    set_tile(0);
    load_step(0);
    for (int tile = 0; tile < ntile; ++tile) {
      f32x4 acc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < nks; ++ks) {
        __syncthreads();
        store_step();
        __syncthreads();
        // next step's operands; unconditional (the very last step reloads
        // itself) so no register set has to survive a skipped load
        int kn = ks + 1;
        if (kn == nks) {
          kn = 0;
          if (tile + 1 < ntile)
            set_tile(tile + 1);
          else
            kn = ks;
        }
        load_step(kn);
        const bf16 (*X)[LD] = kind ? sv : sk;
        const bf16 (*U)[LD] = kind ? uv : uk;
        bf16x8 bfr[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bfr[nt] = *reinterpret_cast<const bf16x8*>(&U[hl * DH + 16 * nt + col][8 * grp]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&X[64 * mh + 16 * mt + col][8 * grp]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfr[nt], acc[mt][nt], 0, 0, 0);
        }
      }
      // ---- attention epilogue; lane holds token 64 mh + 16 mt + 4 grp + r,
      // column 16 nt + col
      const int j0 = t0 + tile * TM;
      if (kind == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) a += qv[nt] * acc[mt][nt][r];
            a = row_sum16(a);
            const int tok = 64 * mh + 16 * mt + 4 * grp + r;
            if (col == 0) sc[hl][tok] = (j0 + tok < t1) ? a : -INFINITY;
          }
      }
      __syncthreads();
      if (kind == 1) {
        // both token halves of a head see all 128 scores: same max, same rescale
        float mx = fmaxf(sc[hl][lane], sc[hl][lane + 64]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float mn = fmaxf(m, mx);
        const float alpha = exp2_diff(m, mn);
        float lp = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 64 * mh + 16 * mt + 4 * grp + r;
            const bool ok = j0 + tok < t1;
            const float pw = ok ? exp2f(sc[hl][tok] - mn) : 0.f;
            lp += pw;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) o[nt] += ok ? pw * acc[mt][nt][r] : 0.f;
          }
        lp += __shfl_xor(lp, 16);
        lp += __shfl_xor(lp, 32);
        l = l * alpha + lp;
        m = mn;
      }
    }
  }
  // ---- add the two token halves of each head, write the split's partial
  if (kind == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      o[nt] += __shfl_xor(o[nt], 16);
      o[nt] += __shfl_xor(o[nt], 32);
    }
  }
  __syncthreads();
  if (kind == 1 && mh == 1) {
    if (grp == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ox[hl][16 * nt + col] = o[nt];
    }
    if (lane == 0) ox[hl][DH] = l;
  }
  __syncthreads();
  if (kind == 1 && mh == 0 && head_ok) {
    const int64_t row = ((int64_t)b * p.S + s) * H + h;
    if (lane == 0) {
      p.part_ml[row * 2 + 0] = m;
      p.part_ml[row * 2 + 1] = l + ox[hl][DH];
    }
    if (grp == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p.part_o[row * p.Dp + 16 * nt + col] = o[nt] + ox[hl][16 * nt + col];
    }
  }
}

}  // namespace

bool scan_reconstruct_gemm_supports(const DecodeParams& p) {
  return p.bf16 && p.G == 1 && p.rk == p.rv && p.rk % KC == 0 && (p.dh == 96 || p.dh == 128 || p.dh == 64);
}

int scan_reconstruct_gemm_tile() { return TM; }

hipError_t launch_scan_reconstruct_gemm(const DecodeParams& p, hipStream_t s) {
  if (!scan_reconstruct_gemm_supports(p)) return hipErrorNotSupported;
  const dim3 grid(p.S, p.B, (p.H + 1) / 2);
  if (p.dh == 96)
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<96>, grid, dim3(kThreads), 0, s, p);
  else if (p.dh == 128)
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<64>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace lla
