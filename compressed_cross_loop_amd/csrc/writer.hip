// Latent writer ("Hybrid Latent Attention" summary, "Latent Writer", Eq. 2):
// for each token and group, c = sum over the set's loops of E_t x_t in fp32,
// the key part rotated by R~_p when the set bakes rotary embedding into its
// key latents, then rounded to the storage dtype (or to e4m3 codes with
// per-token scales) and scattered into the paged store at
// (block_table[b][p/P], p % P).
#include "device_common.h"
#include "lla_internal.h"
#include "writer_common.h"

namespace lla {

namespace {

constexpr int kThreads = 256;
constexpr int kXChunk = 4096;   // input elements staged in LDS at a time

// One workgroup per (token, group): plain fp32 dot products.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_writer_generic(WriterParams p) {
  extern __shared__ float sm[];
  float* c = sm;              // [R]
  float* xs = sm + p.R;       // [kXChunk]
  const int tok = blockIdx.x, g = blockIdx.y;
  const int b = tok / p.n_tok, n = tok % p.n_tok;
  const int R = p.R, d_in = p.d_in;
  for (int o = threadIdx.x; o < R; o += kThreads) c[o] = 0.f;
  const T* x = static_cast<const T*>(p.x);
  const T* enc = static_cast<const T*>(p.enc);
  for (int t = 0; t < p.n_loops; ++t) {
    const T* xr = x + ((((int64_t)b * p.n_tok + n) * p.n_loops + t) * p.G + g) * d_in;
    for (int k0 = 0; k0 < d_in; k0 += kXChunk) {
      const int kn = min(kXChunk, d_in - k0);
      __syncthreads();
      for (int k = threadIdx.x; k < kn; k += kThreads) xs[k] = to_f(xr[k0 + k]);
      __syncthreads();
      for (int o = threadIdx.x; o < R; o += kThreads) {
        const T* er = enc + (((int64_t)t * p.G + g) * R + o) * d_in + k0;
        float acc = 0.f;
        for (int k = 0; k < kn; ++k) acc += to_f(er[k]) * xs[k];
        c[o] += acc;
      }
    }
  }
  __syncthreads();
  const int pos = p.pos[(int64_t)b * p.n_tok + n];
  const int64_t page = p.bt[(int64_t)b * p.max_pages + pos / p.P];
  finish_latent<T, kThreads>(p, c, nullptr, pos, page, pos % p.P, g);
}

}  // namespace

hipError_t launch_writer_generic(const WriterParams& p, hipStream_t s) {
  const size_t lds = (size_t)(p.R + kXChunk) * sizeof(float);
  const dim3 grid(p.B * p.n_tok, p.G);
  if (p.bf16)
    hipLaunchKernelGGL(k_writer_generic<bf16>, grid, dim3(kThreads), lds, s, p);
  else
    hipLaunchKernelGGL(k_writer_generic<float>, grid, dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace lla
