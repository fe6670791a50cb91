// The last step of the latent writer ("Hybrid Latent Attention" summary,
// "Latent Writer", Eq. 2), shared by the general and the matrix-core writer:
// a finished latent c (fp32, in LDS) is rotated and stored.
#pragma once
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

// Called by every thread of a workgroup of NT threads (NT a multiple of 64)
// for the latent of one (token, group) at position pos, page `page`, slot
// `slot`.  The key part is rotated in place by R~_p when the set bakes rotary
// embedding (csn: the (cos, sin) of pos * theta_f per frequency, or null to
// compute them here).  16-bit stores round to nearest even and scatter; fp8
// stores take max |x| of the key part and of the value part, scale = max /
// 448 (1 for an all-zero part), round each element of x / scale to an e4m3
// code and write the two scales.
template <typename T, int NT>
__device__ void finish_latent(const WriterParams& p, float* c, const float (*csn)[2], int pos, int64_t page,
                              int slot, int g) {
  const int R = p.R, rk = p.rk, rv = p.rv, dh = p.dh, half = dh / 2;
  const int tid = threadIdx.x;
  if (p.rope_baked) {
    for (int x = tid; x < rk / 2; x += NT) {
      const int blk = x / half, f = x % half;
      const int lo = blk * dh + f, hi = lo + half;
      float cs, sn;
      if (csn) {
        cs = csn[f][0];
        sn = csn[f][1];
      } else {
        rope_cs(p.rope_base, dh, f, pos, cs, sn);
      }
      const float a = c[lo], b = c[hi];
      c[lo] = a * cs - b * sn;
      c[hi] = a * sn + b * cs;
    }
    __syncthreads();
  }
  if (!p.fp8) {
    T* pages = static_cast<T*>(p.pages);
    for (int o = tid; o < R; o += NT) {
      const int64_t off = o < rk ? key_off(page, g, slot, o, p.G, p.P, R, rk)
                                 : val_off(page, g, slot, o - rk, p.G, p.P, R, rk);
      pages[off] = from_f<T>(c[o]);
    }
    return;
  }
  // fp8: per-part scales from the part's max |x|
  __shared__ float red[2][NT / 64];
  __shared__ float scale[2];
  float mk = 0.f, mv = 0.f;
  for (int o = tid; o < R; o += NT) {
    const float a = fabsf(c[o]);
    if (o < rk)
      mk = fmaxf(mk, a);
    else
      mv = fmaxf(mv, a);
  }
  mk = wave_max(mk);
  mv = wave_max(mv);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mk;
    red[1][tid >> 6] = mv;
  }
  __syncthreads();
  if (tid < 2) {
    float m = 0.f;
    for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, red[tid][w]);
    scale[tid] = m > 0.f ? m / 448.f : 1.f;
  }
  __syncthreads();
  uint8_t* bytes = static_cast<uint8_t*>(p.pages);
  const float sk = scale[0], sv = scale[1];
  for (int o = tid; o < R; o += NT) {
    if (o < rk)
      bytes[key_off8(page, g, slot, o, p.G, p.P, rk, rv)] = (uint8_t)f_to_e4m3(c[o] / sk);
    else
      bytes[val_off8(page, g, slot, o - rk, p.G, p.P, rk, rv)] = (uint8_t)f_to_e4m3(c[o] / sv);
  }
  if (tid < 2)
    *reinterpret_cast<float*>(bytes + scale_off8(page, g, slot, tid, p.G, p.P, rk, rv)) = scale[tid];
}

}  // namespace lla
