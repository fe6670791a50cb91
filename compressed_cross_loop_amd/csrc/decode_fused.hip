// Fused single-launch decode for small batches: the query map A_t, the latent
// scan, the exact window and the value map B_t of one (layer, loop) call in
// one kernel ("Hybrid Latent Attention" summary: Latent Reader, Eqs. 3-4;
// its future work names kernel fusion against the maps' fixed per-step cost).
//
// One workgroup per (context split s, head h, sequence b), four waves:
//   1. q~ = R~_i A_h^T q_h and q' = R_i q_h, both times log2(e)/sqrt(d_h),
//      from this head's decoder alone (A_h: d_h x R, into LDS);
//   2. the split's latent tokens (the head's group latent), 16-token tiles,
//      wave w taking tiles w, w+4, ...: each lane holds R/64 dimensions, a
//      score is a wave-wide dot product, online softmax per wave (exp2
//      domain), O~ += a c^V in latent space;
//   3. window slice s (exact tokens max(0, i-W) .. i, ring then the current
//      token), wave w taking every fourth token, in the same softmax,
//      o_w += a v in head space; the slice holding the current token also
//      appends R_i k_cur, v_cur to the ring;
//   4. the waves merged in LDS, the split's partial (m, l, O~, o_w) stored;
//   5. the last workgroup of (b, h) to take a ticket (one atomic add, no
//      waiting) merges the splits and writes o = (B_h^T O~ + o_w) / l.
// A one-line launch before it zeroes the tickets (no memset, so a caller can
// capture both in a graph).
//
// Every latent byte is read by all H/G heads of its group (from L2 after the
// first), and A_h by every split of its head, so this path pays only where the
// three-kernel path is bound by fixed latency: small batch x context.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// n consecutive bf16 (n = 2, 4, 8 or 16) as floats
template <int N>
__device__ __forceinline__ void load_bf16(const bf16* p, float (&x)[N]) {
  if constexpr (N >= 8) {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 8 * c);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[8 * c + k] = static_cast<float>(v[k]);
    }
  } else {
    typedef __bf16 vec __attribute__((ext_vector_type(N)));
    const vec v = *reinterpret_cast<const vec*>(p);
#pragma unroll
    for (int k = 0; k < N; ++k) x[k] = static_cast<float>(v[k]);
  }
}

// sums over the 64 lanes of N independent values at once: DPP row sums
// (no LDS), then two cross-row exchanges issued back to back
template <int N>
__device__ __forceinline__ void wave_sums(float (&v)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) v[t] = row_sum16(v[t]);
#pragma unroll
  for (int t = 0; t < N; ++t) v[t] += __shfl_xor(v[t], 16);
#pragma unroll
  for (int t = 0; t < N; ++t) v[t] += __shfl_xor(v[t], 32);
}

__global__ void k_fused_tickets_zero(int32_t* t, int n) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x < n) t[x] = 0;
}

template <int R, int DH>
__global__ __launch_bounds__(kThreads) void k_fused_decode(DecodeParams p) {
  constexpr int DK = R / 64;           // latent dims per lane
  constexpr int DW = DH / 64;          // head dims per lane (window)
  constexpr int CG = R / 8, EG = kThreads / CG;   // q map: column chunks x row groups
  static_assert(EG >= 1 && kThreads % CG == 0, "R <= 2048");
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H, W = p.W, S = p.S, P = p.P;
  const int g = h / p.hpg;
  const int i = p.pos[b];
  const int n_lat = max(0, i - W);
  int t0 = s * p.chunk;
  const int t1 = (s == S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > t1) t0 = t1;
  const bool rope = p.rope_base != 0.f;

  // ---- 1. query maps
  __shared__ float qin[DH];
  __shared__ float cs[DH / 2][2];
  __shared__ float red[EG][R];
  __shared__ float qraw[R];
  __shared__ float qt[R];
  __shared__ float qh[DH];
  const bf16* qsrc = static_cast<const bf16*>(p.q) + ((int64_t)b * H + h) * DH;
  if (tid < DH) qin[tid] = static_cast<float>(qsrc[tid]);
  if (tid < DH / 2) {
    float c = 1.f, sn = 0.f;
    if (rope) rope_cs(p.rope_base, DH, tid, i, c, sn);
    cs[tid][0] = c;
    cs[tid][1] = sn;
  }
  __syncthreads();
  {
    const int cg = tid % CG, eg = tid / CG;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    const bf16* A = static_cast<const bf16*>(p.A) + (int64_t)h * DH * R + 8 * cg;
    // rows eg, eg + EG, ...: issued U at a time, so each thread waits on
    // one memory round trip per batch rather than per row
    constexpr int NR = DH / EG, U = NR < 32 ? NR : 32;
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += U) {
      bf16x8 rows[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rows[u] = *reinterpret_cast<const bf16x8*>(A + (int64_t)(eg + EG * (r0 + u)) * R);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float qe = qin[eg + EG * (r0 + u)];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += static_cast<float>(rows[u][k]) * qe;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) red[eg][8 * cg + k] = acc[k];
  }
  __syncthreads();
  for (int c = tid; c < R; c += kThreads) {
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < EG; ++e) v += red[e][c];
    qraw[c] = v;
  }
  __syncthreads();
  // rotation pairs (f, f + d_h/2) inside every d_h-block of the latent, and in head space
  for (int c = tid; c < R + DH; c += kThreads) {
    const bool lat = c < R;
    const int cc = lat ? c : c - R;
    const int f = cc % DH, base = cc - f;
    const float* src = lat ? qraw : qin;
    float v = src[cc];
    if (rope) {
      const int fr = f < DH / 2 ? f : f - DH / 2;
      const float co = cs[fr][0], sn = cs[fr][1];
      v = f < DH / 2 ? src[cc] * co - src[base + f + DH / 2] * sn : src[base + f - DH / 2] * sn + src[cc] * co;
    }
    if (lat)
      qt[cc] = v * p.scale;
    else
      qh[cc] = v * p.scale;
  }
  __syncthreads();

  // ---- 2. latent tokens t0 .. t1-1
  float qv[DK];
#pragma unroll
  for (int k = 0; k < DK; ++k) qv[k] = qt[lane * DK + k];
  float m = -INFINITY, l = 0.f, ov[DK], ow[DW];
#pragma unroll
  for (int k = 0; k < DK; ++k) ov[k] = 0.f;
#pragma unroll
  for (int k = 0; k < DW; ++k) ow[k] = 0.f;
  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  for (int ti = wave; ti < ntiles; ti += kWaves) {
    const int j0 = t0 + ti * kTile;
    const int nvalid = min(kTile, t1 - j0);
    const int64_t page = bt[j0 / P];
    const bf16* tile = pages + ((page * p.G + g) * (P / kTile) + (j0 % P) / kTile) * kTile * (2 * R);
    // every key row and value row of the tile requested before any is used
    float kk[kTile][DK];
#pragma unroll
    // key row t, dims lane DK .. (wide rows are chunk-major; DK <= 16 dims
    // never cross a 32-dim chunk)
    for (int t = 0; t < kTile; ++t) load_bf16<DK>(tile + key_in_tile(t, lane * DK, R), kk[t]);
    // values: dimension d of the tile sits in sub-block d/16, row d%16, 16 tokens contiguous
    const bf16* vb = tile + kTile * R;
    float vv[DK][kTile];
#pragma unroll
    for (int k = 0; k < DK; ++k) {
      const int d = lane * DK + k;
      load_bf16<kTile>(vb + (d / kTile) * kTile * kTile + (d % kTile) * kTile, vv[k]);
    }
    float sc[kTile];
#pragma unroll
    for (int t = 0; t < kTile; ++t) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < DK; ++k) d += qv[k] * kk[t][k];
      sc[t] = d;
    }
    wave_sums(sc);
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTile; ++t) {
      if (t >= nvalid) sc[t] = -INFINITY;
      mx = fmaxf(mx, sc[t]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_diff(m, mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < DK; ++k) ov[k] *= alpha;
#pragma unroll
    for (int t = 0; t < kTile; ++t) {
      sc[t] = exp2_diff(sc[t], mn);
      l += sc[t];
    }
    m = mn;
#pragma unroll
    for (int k = 0; k < DK; ++k) {
      float a = 0.f;
#pragma unroll
      for (int t = 0; t < kTile; ++t) a += t < nvalid ? sc[t] * vv[k][t] : 0.f;   // tokens past the end may hold NaN
      ov[k] += a;
    }
  }

  // ---- 3. window slice s: exact tokens j0w + u for u = us .. ue-1 (u = nw is the current token)
  const int j0w = max(0, i - W), nw = i - j0w;
  const int us = s * p.tw, ue = min(us + p.tw, nw + 1);
  const bf16* rk = static_cast<const bf16*>(p.ring_k);
  const bf16* rv = static_cast<const bf16*>(p.ring_v);
  const int64_t hd = (int64_t)h * DH + lane * DW;
  // each wave takes every fourth token, UW at a time (their loads in flight together)
  constexpr int UW = 4;
  for (int u0 = us + wave; u0 < ue; u0 += kWaves * UW) {
    float kk[UW][DW], vv[UW][DW], sc[UW];
#pragma unroll
    for (int x = 0; x < UW; ++x) {
      const int u = min(u0 + kWaves * x, ue - 1);   // past the slice: reread a valid token, masked below
      if (u < nw) {
        const int64_t row = ((int64_t)b * (W + 1) + (j0w + u) % (W + 1)) * H * DH + hd;
        load_bf16<DW>(rk + row, kk[x]);
        load_bf16<DW>(rv + row, vv[x]);
      } else {
        // the current token: R_i k_cur (partner dims d +- d_h/2 live 32 lanes away), v_cur
        float kc[DW];
        load_bf16<DW>(static_cast<const bf16*>(p.k_cur) + ((int64_t)b * H) * DH + hd, kc);
        load_bf16<DW>(static_cast<const bf16*>(p.v_cur) + ((int64_t)b * H) * DH + hd, vv[x]);
#pragma unroll
        for (int k = 0; k < DW; ++k) {
          const float other = __shfl_xor(kc[k], 32);
          const int d = lane * DW + k, f = d < DH / 2 ? d : d - DH / 2;
          const float co = cs[f][0], sn = cs[f][1];
          kk[x][k] = d < DH / 2 ? kc[k] * co - other * sn : other * sn + kc[k] * co;
        }
        if (u0 + kWaves * x == nw) {
          // append to the ring: slot i mod (W+1) held token i-W-1, which no slice reads
          const int64_t so = ((int64_t)b * (W + 1) + i % (W + 1)) * H * DH + hd;
#pragma unroll
          for (int k = 0; k < DW; ++k) {
            static_cast<bf16*>(p.ring_k)[so + k] = static_cast<bf16>(kk[x][k]);
            static_cast<bf16*>(p.ring_v)[so + k] = static_cast<bf16>(vv[x][k]);
          }
        }
      }
    }
#pragma unroll
    for (int x = 0; x < UW; ++x) {
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < DW; ++k) d += qh[lane * DW + k] * kk[x][k];
      sc[x] = d;
    }
    wave_sums(sc);
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < UW; ++x) {
      if (u0 + kWaves * x >= ue) sc[x] = -INFINITY;
      mx = fmaxf(mx, sc[x]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_diff(m, mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < DK; ++k) ov[k] *= alpha;
#pragma unroll
    for (int k = 0; k < DW; ++k) ow[k] *= alpha;
#pragma unroll
    for (int x = 0; x < UW; ++x) {
      const float pw = exp2_diff(sc[x], mn);
      l += pw;
#pragma unroll
      for (int k = 0; k < DW; ++k) ow[k] += pw * vv[x][k];   // a reread token has pw = 0 and finite values
    }
    m = mn;
  }

  // ---- 4. merge the waves, store the split's partial (m, l, O~[R], o_w[d_h])
  __shared__ float mw[kWaves], lw[kWaves];
  __shared__ float ovw[kWaves][R];
  __shared__ float oww[kWaves][DH];
  if (lane == 0) {
    mw[wave] = m;
    lw[wave] = l;
  }
#pragma unroll
  for (int k = 0; k < DK; ++k) ovw[wave][lane * DK + k] = ov[k];
#pragma unroll
  for (int k = 0; k < DW; ++k) oww[wave][lane * DW + k] = ow[k];
  __syncthreads();
  float M = mw[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
  float fw[kWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    fw[w] = exp2_diff(mw[w], M);
    L += fw[w] * lw[w];
  }
  constexpr int PW = 2 + R + DH;   // partial row: m, l, O~, o_w
  const int64_t bh = (int64_t)b * H + h;
  float* part = p.fpart + (bh * S + s) * PW;
  if (tid == 0) {
    part[0] = M;
    part[1] = L;
  }
  for (int c = tid; c < R + DH; c += kThreads) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += fw[w] * (c < R ? ovw[w][c] : oww[w][c - R]);
    part[2 + c] = v;
  }

  // ---- 5. the last split of (b, h) to arrive merges and applies B_h
  // The barrier waits for every wave's stores to reach this XCD's L2; one
  // device-scope release by the ticket holder then writes them back for the
  // other XCDs (each release or acquire fence is an L2 write-back or
  // invalidate here, so one per workgroup and direction, not one per wave).
  __shared__ int last;
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    last = atomicAdd(&p.tickets[bh], 1) == S - 1;
    if (last) __threadfence();   // acquire the other splits' partials
  }
  __syncthreads();
  if (!last) return;
  const float* parts = p.fpart + bh * S * PW;
  // the splits' weights exp2(m_s - M) once, in LDS (S <= kMaxFusedSplits)
  __shared__ float wsp[kMaxFusedSplits];
  __shared__ float Lsh;
  if (tid < 64) {
    float mloc = -INFINITY;
    for (int q = tid; q < S; q += 64) mloc = fmaxf(mloc, parts[q * PW]);
    const float Mg = wave_max(mloc);
    float lloc = 0.f;
    for (int q = tid; q < S; q += 64) {
      const float f = exp2_diff(parts[q * PW], Mg);
      wsp[q] = f;
      lloc += f * parts[q * PW + 1];
    }
    lloc = wave_sum(lloc);
    if (tid == 0) Lsh = lloc;
  }
  __syncthreads();
  const float Lg = Lsh;
  for (int c = tid; c < R + DH; c += kThreads) {
    float v = 0.f;
#pragma unroll 8
    for (int q = 0; q < S; ++q) v += wsp[q] * parts[q * PW + 2 + c];
    if (c < R)
      qraw[c] = v;       // merged O~ (latent space)
    else
      qin[c - R] = v;    // merged o_w (head space)
  }
  __syncthreads();
  // o[e] = (B_t^T[h][e][:] . O~ + o_w[e]) / l: TPE threads per output row
  constexpr int TPE = kThreads / DH, CPT = R / TPE;
  const int e = tid / TPE, part_id = tid % TPE;
  const bf16* brow = static_cast<const bf16*>(p.Bm) + ((int64_t)h * DH + e) * R + part_id * CPT;
  float acc = 0.f;
  constexpr int UB = CPT / 8 < 16 ? CPT / 8 : 16;
#pragma unroll
  for (int c0 = 0; c0 < CPT; c0 += 8 * UB) {
    bf16x8 bv[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) bv[u] = *reinterpret_cast<const bf16x8*>(brow + c0 + 8 * u);
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += static_cast<float>(bv[u][k]) * qraw[part_id * CPT + c0 + 8 * u + k];
  }
#pragma unroll
  for (int o = 1; o < TPE; o <<= 1) acc += __shfl_xor(acc, o);
  if (part_id == 0)
    static_cast<bf16*>(p.out)[bh * DH + e] = static_cast<bf16>((acc + qin[e]) / Lg);
}

template <int R, int DH>
hipError_t launch_rd(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((k_fused_decode<R, DH>), dim3(p.S, p.H, p.B), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_d(const DecodeParams& p, hipStream_t st) {
  switch (p.rk) {
    case 128: return launch_rd<128, DH>(p, st);
    case 256: return launch_rd<256, DH>(p, st);
    case 512: return launch_rd<512, DH>(p, st);
    default: return launch_rd<1024, DH>(p, st);
  }
}

}  // namespace

bool fused_decode_supports(const DecodeParams& p) {
  if (!p.bf16 || p.fp8 || p.rk != p.rv) return false;
  if (p.dh != 64 && p.dh != 128) return false;
  return p.rk == 128 || p.rk == 256 || p.rk == 512 || p.rk == 1024;
}

int fused_partial_floats(int rk, int dh) { return 2 + rk + dh; }

hipError_t launch_fused_decode(const DecodeParams& p, hipStream_t s) {
  if (!fused_decode_supports(p)) return hipErrorNotSupported;
  const int n = p.B * p.H;
  hipLaunchKernelGGL(k_fused_tickets_zero, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p.tickets, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return p.dh == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
}

}  // namespace lla
