// General decode kernels (VALU, fp32 arithmetic, any supported shape, fp32 or
// bf16 storage).  They implement, per (sequence, head):
//   qmap      q' = s R_i q            and, for the absorbed read,
//             q~ = s R~_i A_t^T q     ("Hybrid Latent Attention" summary,
//                                      "Latent Reader", Eq. 3)
//   window    exact tokens i-W <= j <= i of Eq. 4 (ring + current token),
//             and the ring append of the current token
//   scan      latent tokens j < i-W of one context split, online softmax:
//             absorbed    -- scores q~ . sK_j, accumulate sum a_j sV_j
//             reconstruct -- rebuild k_j = A sK_j and v_j = B^T sV_j first
//                            (Looped Latent Attention abstracts: keys and
//                            values are rebuilt from the latents when
//                            attention reads them)
//   combine   merge split and window partials (one softmax over all tokens,
//             Eq. 4) and apply B_t^T to the latent sum (absorbed)
// with s = log2(e)/sqrt(d_h): scores live in the exp2 domain.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_qmap(DecodeParams p, int want_qlat) {
  extern __shared__ float sm[];
  const int dh = p.dh, rk = p.rk, half = dh / 2;
  float* qs = sm;        // [dh]
  float* u = sm + dh;    // [rk]
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int i = p.pos[b];
  const T* q = static_cast<const T*>(p.q) + ((int64_t)b * p.H + h) * dh;
  for (int e = tid; e < dh; e += kThreads) qs[e] = to_f(q[e]);
  __syncthreads();
  float* qh = p.qhead + ((int64_t)b * p.H + h) * dh;
  for (int f = tid; f < half; f += kThreads) {
    float c = 1.f, s = 0.f;
    if (p.rope_base != 0.f) rope_cs(p.rope_base, dh, f, i, c, s);
    const float x1 = qs[f], x2 = qs[f + half];
    qh[f] = p.scale * (x1 * c - x2 * s);
    qh[f + half] = p.scale * (x1 * s + x2 * c);
  }
  if (!want_qlat) return;
  const T* Ah = static_cast<const T*>(p.A) + (int64_t)h * dh * rk;
  for (int k = tid; k < rk; k += kThreads) {
    float acc = 0.f;
    for (int e = 0; e < dh; ++e) acc += to_f(Ah[(int64_t)e * rk + k]) * qs[e];
    u[k] = acc;
  }
  __syncthreads();
  T* ql = static_cast<T*>(p.qlat) + ((int64_t)b * p.H + h) * rk;
  for (int k = tid; k < rk; k += kThreads) {
    float v = u[k];
    if (p.rope_base != 0.f) {
      const int f = k % dh;
      float c, s;
      if (f < half) {
        rope_cs(p.rope_base, dh, f, i, c, s);
        v = u[k] * c - u[k + half] * s;
      } else {
        rope_cs(p.rope_base, dh, f - half, i, c, s);
        v = u[k - half] * s + u[k] * c;
      }
    }
    ql[k] = from_f<T>(v * p.scale);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_window(DecodeParams p) {
  extern __shared__ float sm[];
  const int dh = p.dh, W = p.W, half = dh / 2, H = p.H;
  float* qv = sm;            // [dh]
  float* ks = sm + dh;       // [dh]  rotated current key
  float* sc = sm + 2 * dh;   // [W+1] scores, then weights
  __shared__ float red[kThreads / 64];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = p.pos[b];
  const int j0 = max(0, i - W);
  const int nw = i - j0;  // exact tokens from the ring
  const float* qh = p.qhead + ((int64_t)b * H + h) * dh;
  const T* kc = static_cast<const T*>(p.k_cur) + ((int64_t)b * H + h) * dh;
  const T* vc = static_cast<const T*>(p.v_cur) + ((int64_t)b * H + h) * dh;
  const T* rk_ = static_cast<const T*>(p.ring_k);
  const T* rv_ = static_cast<const T*>(p.ring_v);
  for (int e = tid; e < dh; e += kThreads) qv[e] = qh[e];
  for (int f = tid; f < half; f += kThreads) {
    float c = 1.f, s = 0.f;
    if (p.rope_base != 0.f) rope_cs(p.rope_base, dh, f, i, c, s);
    const float x1 = to_f(kc[f]), x2 = to_f(kc[f + half]);
    ks[f] = x1 * c - x2 * s;
    ks[f + half] = x1 * s + x2 * c;
  }
  __syncthreads();
  for (int t = wave; t <= nw; t += kThreads / 64) {
    float acc = 0.f;
    if (t < nw) {
      const int slot = (j0 + t) % (W + 1);
      const T* kr = rk_ + (((int64_t)b * (W + 1) + slot) * H + h) * dh;
      for (int e = lane; e < dh; e += 64) acc += qv[e] * to_f(kr[e]);
    } else {
      for (int e = lane; e < dh; e += 64) acc += qv[e] * ks[e];
    }
    acc = wave_sum(acc);
    if (lane == 0) sc[t] = acc;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int t = tid; t <= nw; t += kThreads) mx = fmaxf(mx, sc[t]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < kThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float ls = 0.f;
  for (int t = tid; t <= nw; t += kThreads) {
    const float w = exp2f(sc[t] - mx);
    sc[t] = w;
    ls += w;
  }
  ls = wave_sum(ls);
  if (lane == 0) red[wave] = ls;
  __syncthreads();
  ls = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) ls += red[w];
  float* wo = p.win_o + ((int64_t)b * p.WS * H + h) * dh;
  for (int e = tid; e < dh; e += kThreads) {
    float acc = 0.f;
    for (int t = 0; t < nw; ++t) {
      const int slot = (j0 + t) % (W + 1);
      acc += sc[t] * to_f(rv_[(((int64_t)b * (W + 1) + slot) * H + h) * dh + e]);
    }
    acc += sc[nw] * to_f(vc[e]);
    wo[e] = acc;
  }
  if (tid == 0) {
    p.win_ml[((int64_t)b * p.WS * H + h) * 2 + 0] = mx;
    p.win_ml[((int64_t)b * p.WS * H + h) * 2 + 1] = ls;
  }
  for (int ws = 1; ws < p.WS; ++ws) {
    const int64_t row = ((int64_t)b * p.WS + ws) * H + h;
    if (tid == 0) {
      p.win_ml[row * 2 + 0] = -INFINITY;
      p.win_ml[row * 2 + 1] = 0.f;
    }
    for (int e = tid; e < dh; e += kThreads) p.win_o[row * dh + e] = 0.f;
  }
  // ring append: slot i mod (W+1) was token i-W-1, which no read above touches
  const int si = i % (W + 1);
  T* rkw = static_cast<T*>(p.ring_k) + (((int64_t)b * (W + 1) + si) * H + h) * dh;
  T* rvw = static_cast<T*>(p.ring_v) + (((int64_t)b * (W + 1) + si) * H + h) * dh;
  for (int e = tid; e < dh; e += kThreads) {
    rkw[e] = from_f<T>(ks[e]);
    rvw[e] = vc[e];
  }
}

__device__ __forceinline__ void split_range(const DecodeParams& p, int s, int n_lat, int& t0, int& t1) {
  t0 = s * p.chunk;
  t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_scan_absorbed_generic(DecodeParams p) {
  extern __shared__ float sm[];
  const int rk = p.rk, rv = p.rv, P = p.P, G = p.G, R = rk + rv;
  float* ql = sm;              // [rk]
  float* o = sm + rk;          // [rv]
  __shared__ float sc[kChunk];
  __shared__ int64_t pg[kChunk];
  __shared__ float kscale[kChunk], vscale[kChunk];   // fp8 stores: per-token scales
  const int s = blockIdx.x, b = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = h / p.hpg;
  const uint8_t* bytes = static_cast<const uint8_t*>(p.pages);
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0, t1;
  split_range(p, s, n_lat, t0, t1);
  const T* qsrc = static_cast<const T*>(p.qlat) + ((int64_t)b * p.H + h) * rk;
  for (int k = tid; k < rk; k += kThreads) ql[k] = to_f(qsrc[k]);
  for (int k = tid; k < rv; k += kThreads) o[k] = 0.f;
  const T* pages = static_cast<const T*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  float m = -INFINITY, l = 0.f;
  __syncthreads();
  for (int c0 = t0; c0 < t1; c0 += kChunk) {
    const int n = min(kChunk, t1 - c0);
    if (tid < n) {
      pg[tid] = bt[(c0 + tid) / P];
      if (p.fp8) {
        const int slot = (c0 + tid) % P;
        kscale[tid] = *reinterpret_cast<const float*>(bytes + scale_off8(pg[tid], g, slot, 0, G, P, rk, rv));
        vscale[tid] = *reinterpret_cast<const float*>(bytes + scale_off8(pg[tid], g, slot, 1, G, P, rk, rv));
      }
    }
    __syncthreads();
    for (int t = wave; t < n; t += kThreads / 64) {
      const int slot = (c0 + t) % P;
      float acc = 0.f;
      if (p.fp8) {
        const uint8_t* kr = bytes + key_off8(pg[t], g, slot, 0, G, P, rk, rv);
        for (int k = lane; k < rk; k += 64) acc += ql[k] * e4m3_to_f(kr[k]);
      } else {
        const T* kt = pages + tile_base(pg[t], g, slot, G, P, R);
        for (int k = lane; k < rk; k += 64) acc += ql[k] * to_f(kt[key_in_tile(slot & 15, k, rk)]);
      }
      acc = wave_sum(acc);
      if (lane == 0) sc[t] = p.fp8 ? acc * kscale[t] : acc;
    }
    __syncthreads();
    float cm = -INFINITY;
    for (int t = 0; t < n; ++t) cm = fmaxf(cm, sc[t]);
    const float mn = fmaxf(m, cm);
    const float alpha = exp2_diff(m, mn);
    float ps = 0.f;
    for (int t = 0; t < n; ++t) ps += exp2f(sc[t] - mn);
    l = l * alpha + ps;
    m = mn;
    for (int k = tid; k < rv; k += kThreads) {
      float acc = o[k] * alpha;
      for (int t = 0; t < n; ++t) {
        const int slot = (c0 + t) % P;
        acc += p.fp8 ? exp2f(sc[t] - mn) * vscale[t] * e4m3_to_f(bytes[val_off8(pg[t], g, slot, k, G, P, rk, rv)])
                     : exp2f(sc[t] - mn) * to_f(pages[val_off(pg[t], g, slot, k, G, P, R, rk)]);
      }
      o[k] = acc;
    }
    __syncthreads();
  }
  const int64_t row = ((int64_t)b * p.S + s) * p.H + h;
  if (tid == 0) {
    p.part_ml[row * 2 + 0] = m;
    p.part_ml[row * 2 + 1] = l;
  }
  for (int k = tid; k < rv; k += kThreads) p.part_o[row * p.Dp + k] = o[k];
}

constexpr int kRecTok = 16;   // tokens rebuilt per step
constexpr int kRecR = 128;    // latent dims staged per step

template <typename T>
__global__ __launch_bounds__(kThreads) void k_scan_reconstruct_generic(DecodeParams p) {
  const int rk = p.rk, rv = p.rv, P = p.P, G = p.G, R = rk + rv, dh = p.dh;
  __shared__ float qv[256];
  __shared__ float skt[kRecTok][kRecR];
  __shared__ float svt[kRecTok][kRecR];
  __shared__ float red[kThreads / 64][kRecTok];
  __shared__ int64_t pg[kRecTok];
  const int s = blockIdx.x, b = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = h / p.hpg;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0, t1;
  split_range(p, s, n_lat, t0, t1);
  const float* qh = p.qhead + ((int64_t)b * p.H + h) * dh;
  const T* Ah = static_cast<const T*>(p.A) + (int64_t)h * dh * rk;   // [dh][rk]
  const T* Bh = static_cast<const T*>(p.Bm) + (int64_t)h * dh * rv;  // B_t^T: [dh][rv]
  const T* pages = static_cast<const T*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const int e = tid;
  const float qe = (e < dh) ? qh[e] : 0.f;
  float oe = 0.f, m = -INFINITY, l = 0.f;
  for (int c0 = t0; c0 < t1; c0 += kRecTok) {
    const int n = min(kRecTok, t1 - c0);
    if (tid < n) pg[tid] = bt[(c0 + tid) / P];
    float kacc[kRecTok], vacc[kRecTok];
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) kacc[t] = vacc[t] = 0.f;
    const int rmax = max(rk, rv);
    for (int r0 = 0; r0 < rmax; r0 += kRecR) {
      __syncthreads();
      for (int x = tid; x < kRecTok * kRecR; x += kThreads) {
        const int t = x / kRecR, r = x % kRecR;
        float kvl = 0.f, vvl = 0.f;
        if (t < n) {
          const int slot = (c0 + t) % P;
          if (r0 + r < rk) kvl = to_f(pages[key_off(pg[t], g, slot, r0 + r, G, P, R, rk)]);
          if (r0 + r < rv) vvl = to_f(pages[val_off(pg[t], g, slot, r0 + r, G, P, R, rk)]);
        }
        skt[t][r] = kvl;
        svt[t][r] = vvl;
      }
      __syncthreads();
      if (e < dh) {
        const int rkn = min(kRecR, rk - r0), rvn = min(kRecR, rv - r0);
        for (int r = 0; r < rkn; ++r) {
          const float a = to_f(Ah[(int64_t)e * rk + r0 + r]);
#pragma unroll
          for (int t = 0; t < kRecTok; ++t) kacc[t] += a * skt[t][r];
        }
        for (int r = 0; r < rvn; ++r) {
          const float bb = to_f(Bh[(int64_t)e * rv + r0 + r]);
#pragma unroll
          for (int t = 0; t < kRecTok; ++t) vacc[t] += bb * svt[t][r];
        }
      }
    }
    // scores of the rebuilt keys against q' (block reduction over e)
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) {
      const float v = wave_sum(qe * kacc[t]);
      if (lane == 0) red[wave][t] = v;
    }
    __syncthreads();
    float sc[kRecTok];
    float cm = -INFINITY;
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) {
      float v = 0.f;
      for (int w = 0; w < kThreads / 64; ++w) v += red[w][t];
      sc[t] = (t < n) ? v : -INFINITY;
      cm = fmaxf(cm, sc[t]);
    }
    const float mn = fmaxf(m, cm);
    const float alpha = exp2_diff(m, mn);
    float ps = 0.f, acc = oe * alpha;
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) {
      const float w = (t < n) ? exp2f(sc[t] - mn) : 0.f;
      ps += w;
      acc += w * vacc[t];
    }
    l = l * alpha + ps;
    m = mn;
    oe = acc;
  }
  const int64_t row = ((int64_t)b * p.S + s) * p.H + h;
  if (tid == 0) {
    p.part_ml[row * 2 + 0] = m;
    p.part_ml[row * 2 + 1] = l;
  }
  if (e < dh) p.part_o[row * p.Dp + e] = oe;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_combine(DecodeParams p) {
  extern __shared__ float sm[];
  const int S = p.S, WS = p.WS, H = p.H, dh = p.dh;
  float* ws = sm;            // [S]   latent split weights
  float* ww = sm + S;        // [WS]  window slice weights
  float* ob = sm + S + WS;   // [Dp]  (absorbed: latent-space sum)
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  __shared__ float red[kThreads / 64];
  // block-wide max / sum of one value per thread (every thread gets the result)
  auto block_reduce = [&](float v, bool is_max) {
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();   // red is free
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float t = red[0];
    for (int w = 1; w < kThreads / 64; ++w) t = is_max ? fmaxf(t, red[w]) : t + red[w];
    return t;
  };
  // (m, l) of every split and window slice: threads take parts tid, tid + kThreads, ..
  auto part_m = [&](int j) {
    return j < S ? p.part_ml[(((int64_t)b * S + j) * H + h) * 2] : p.win_ml[(((int64_t)b * WS + (j - S)) * H + h) * 2];
  };
  auto part_l = [&](int j) {
    return j < S ? p.part_ml[(((int64_t)b * S + j) * H + h) * 2 + 1]
                 : p.win_ml[(((int64_t)b * WS + (j - S)) * H + h) * 2 + 1];
  };
  float mloc = -INFINITY;
  for (int j = tid; j < S + WS; j += kThreads) mloc = fmaxf(mloc, part_m(j));
  const float M = block_reduce(mloc, true);
  float lloc = 0.f;
  for (int j = tid; j < S + WS; j += kThreads) {
    const float w = exp2_diff(part_m(j), M);
    lloc += w * part_l(j);
    if (j < S) ws[j] = w; else ww[j - S] = w;
  }
  const float l = block_reduce(lloc, false);
  const float inv = 1.f / l;
  __syncthreads();
  T* out = static_cast<T*>(p.out) + ((int64_t)b * H + h) * dh;
  auto window_sum = [&](int e) {
    float acc = 0.f;
    for (int s = 0; s < WS; ++s) acc += ww[s] * p.win_o[(((int64_t)b * WS + s) * H + h) * dh + e];
    return acc;
  };
  if (p.mode == kAbsorbed) {
    const int rv = p.rv;
    for (int k = tid; k < rv; k += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < S; ++s) acc += ws[s] * p.part_o[(((int64_t)b * S + s) * H + h) * p.Dp + k];
      ob[k] = acc;
    }
    __syncthreads();
    const T* Bh = static_cast<const T*>(p.Bm) + (int64_t)h * dh * rv;   // B_t^T: [dh][rv]
    for (int e = tid; e < dh; e += kThreads) {
      float acc = 0.f;
      for (int k = 0; k < rv; ++k) acc += to_f(Bh[(int64_t)e * rv + k]) * ob[k];
      out[e] = from_f<T>((acc + window_sum(e)) * inv);
    }
  } else if (dh <= kThreads) {
    // thread -> (dim e, split group sg): the groups take splits sg, sg + ng, ..
    // eight at a time (addresses clamped to the last split, weight 0), so a
    // long context's many splits cost a few memory round trips, not one each;
    // the groups' sums then add through LDS in a fixed order
    __shared__ float gsum[kThreads];
    const int ng = kThreads / dh, e = tid % dh, sg = tid / dh;
    float acc = 0.f;
    if (sg < ng) {
      const float* base = p.part_o + ((int64_t)b * S * H + h) * p.Dp + e;
      const int64_t sstride = (int64_t)H * p.Dp;
      constexpr int UL = 8;
      for (int s0 = sg; s0 < S; s0 += UL * ng) {
        float v[UL];
#pragma unroll
        for (int u = 0; u < UL; ++u) v[u] = base[min(s0 + u * ng, S - 1) * sstride];
#pragma unroll
        for (int u = 0; u < UL; ++u) acc += (s0 + u * ng < S ? ws[s0 + u * ng] : 0.f) * v[u];
      }
    }
    gsum[tid] = acc;
    __syncthreads();
    if (tid < dh) {
      float t = 0.f;
      for (int g = 0; g < ng; ++g) t += gsum[g * dh + tid];
      out[tid] = from_f<T>((t + window_sum(tid)) * inv);
    }
  } else {
    for (int e = tid; e < dh; e += kThreads) {
      float acc = 0.f;
      for (int s = 0; s < S; ++s) acc += ws[s] * p.part_o[(((int64_t)b * S + s) * H + h) * p.Dp + e];
      out[e] = from_f<T>((acc + window_sum(e)) * inv);
    }
  }
}

template <typename T>
hipError_t launch_all_qmap(const DecodeParams& p, bool want_qlat, hipStream_t st) {
  const size_t lds = (size_t)(p.dh + (want_qlat ? p.rk : 0)) * sizeof(float);
  hipLaunchKernelGGL(k_qmap<T>, dim3(p.B, p.H), dim3(kThreads), lds, st, p, want_qlat ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmap(const DecodeParams& p, bool want_qlat, hipStream_t s) {
  return p.bf16 ? launch_all_qmap<bf16>(p, want_qlat, s) : launch_all_qmap<float>(p, want_qlat, s);
}

hipError_t launch_window(const DecodeParams& p, hipStream_t s) {
  const size_t lds = (size_t)(2 * p.dh + p.W + 1) * sizeof(float);
  if (p.bf16)
    hipLaunchKernelGGL(k_window<bf16>, dim3(p.B, p.H), dim3(kThreads), lds, s, p);
  else
    hipLaunchKernelGGL(k_window<float>, dim3(p.B, p.H), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_scan_absorbed_generic(const DecodeParams& p, hipStream_t s) {
  const size_t lds = (size_t)(p.rk + p.rv) * sizeof(float);
  if (p.bf16)
    hipLaunchKernelGGL(k_scan_absorbed_generic<bf16>, dim3(p.S, p.B, p.H), dim3(kThreads), lds, s, p);
  else
    hipLaunchKernelGGL(k_scan_absorbed_generic<float>, dim3(p.S, p.B, p.H), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_scan_reconstruct_generic(const DecodeParams& p, hipStream_t s) {
  if (p.bf16)
    hipLaunchKernelGGL(k_scan_reconstruct_generic<bf16>, dim3(p.S, p.B, p.H), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_scan_reconstruct_generic<float>, dim3(p.S, p.B, p.H), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeParams& p, hipStream_t s) {
  const size_t lds = (size_t)(p.S + p.WS + (p.mode == kAbsorbed ? p.rv : 0)) * sizeof(float);
  if (p.bf16)
    hipLaunchKernelGGL(k_combine<bf16>, dim3(p.B, p.H), dim3(kThreads), lds, s, p);
  else
    hipLaunchKernelGGL(k_combine<float>, dim3(p.B, p.H), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace lla
