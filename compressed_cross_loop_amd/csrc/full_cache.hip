// Uncompressed (full-cache) looped decode attention: the baseline the latent
// codec replaces.  Every loop keeps exact keys and values of every token
// ("Hybrid Latent Attention" summary, "Key Problem"), so one decode call of
// one (layer, loop) is ordinary attention over the paged exact cache.
//
// grid (context split, sequence, head block); thread (head hl = tid / (d_h/8),
// c = tid % (d_h/8)) owns dims 8c..8c+7 of one head: one token's keys (or
// values) for all heads of the block are one contiguous row, read with
// 16-byte loads by the whole workgroup.  Scores are reduced over the d_h/8
// lanes of a head with DPP; the online softmax runs per head over batches of
// 8 tokens (the loads of the next batch in flight while one is consumed).
// The last split also takes the current token R_i k_cur, v_cur and appends
// it to the cache at position i, which no split reads.  Each split writes a
// head-space partial (m, l, o); the merge is the common combine kernel.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

constexpr int kThreads = 256;
constexpr int U = 8;   // tokens per batch (a batch never straddles a page: P % 8 == 0)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements as floats
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = static_cast<float>(v[k]);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[k] = a[k];
    x[k + 4] = b[k];
  }
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = static_cast<bf16>(x[k]);
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// raw storage of one 8-element row chunk (kept packed while in flight)
// Cached keys and values are read exactly once per call: non-temporal loads
// (measured: 193.7 -> 175.3 us per call at batch 32, 4k, 16 x 128 heads).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p)); }
  __device__ __forceinline__ float get(int k) const { return static_cast<float>(v[k]); }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ float get(int k) const { return k < 4 ? a[k] : b[k - 4]; }
};

template <typename T, int DH>
__global__ __launch_bounds__(kThreads) void k_full_scan(FullParams p) {
  constexpr int TPH = DH / 8;             // lanes per head
  constexpr int HPB = kThreads / TPH;     // heads per block
  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, hl = tid / TPH, c = tid % TPH;
  const int h = blockIdx.z * HPB + hl;
  if (h >= p.H) return;                   // whole TPH-lane groups leave together; no barriers follow
  const int H = p.H, P = p.P;
  const int i = p.pos[b];
  int t0 = s * p.chunk;
  const int t1 = (s == p.S - 1) ? i : min(i, t0 + p.chunk);
  if (t0 > t1) t0 = t1;
  const bool has_self = s == p.S - 1;

  // rotated, scaled query and (last split) current key for this thread's dims
  const bool rope = p.rope_base != 0.f;
  const int pc = (8 * c < DH / 2) ? 8 * c + DH / 2 : 8 * c - DH / 2;   // partner dims of the rotation
  auto rotate = [&](const T* row, float (&out)[8], float scale) {
    float x[8], xp[8];
    load8(row + 8 * c, x);
    load8(row + pc, xp);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = 8 * c + k;
      const int f = d < DH / 2 ? d : d - DH / 2;
      float cc = 1.f, sn = 0.f;
      if (rope) rope_cs(p.rope_base, DH, f, i, cc, sn);
      out[k] = scale * (d < DH / 2 ? x[k] * cc - xp[k] * sn : xp[k] * sn + x[k] * cc);
    }
  };
  const int64_t hrow = ((int64_t)b * H + h) * DH;
  float qf[8];
  rotate(static_cast<const T*>(p.q) + hrow, qf, p.scale);

  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  const T* kp = static_cast<const T*>(p.k_pages);
  const T* vp = static_cast<const T*>(p.v_pages);
  // element offset of this thread's chunk of token j (its page looked up once
  // per batch: a batch lies in one page)
  auto row_of = [&](int j) -> int64_t {
    const int64_t page = bt[j / P];
    return ((page * P + j % P) * H + h) * DH + 8 * c;
  };

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;

  Raw8<T> kA[U], vA[U], kB[U], vB[U];
  auto load_batch = [&](Raw8<T> (&kr)[U], Raw8<T> (&vr)[U], int tb) {
    const int tc = min(tb, t1 - 1);            // past the end: reread a valid token
    const int64_t base = row_of(tc - tc % U);  // the batch's first token (same page)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = base + (int64_t)u * H * DH;
      kr[u].load(kp + off);
      vr[u].load(vp + off);
    }
  };
  auto consume = [&](const Raw8<T> (&kr)[U], const Raw8<T> (&vr)[U], int tb) {
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) a += qf[k] * kr[u].get(k);
      sc[u] = group_sum(a, TPH);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t1) sc[u] = -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_diff(m, mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pw = fast_exp2(sc[u] - mn);
      l += pw;
      if (tb + u < t1) {   // a token past the end may hold anything: select, not multiply
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] += pw * vr[u].get(k);
      }
    }
    m = mn;
  };
  if (t0 < t1) {
    // t0 is a multiple of the split chunk (a multiple of 64), so batches are
    // aligned to U
    load_batch(kA, vA, t0);
    for (int tb = t0; tb < t1; tb += 2 * U) {
      load_batch(kB, vB, tb + U);
      consume(kA, vA, tb);
      if (tb + U >= t1) break;
      load_batch(kA, vA, tb + 2 * U);
      consume(kB, vB, tb + U);
    }
  }

  if (has_self) {
    float kself[8], vself[8];
    rotate(static_cast<const T*>(p.k_cur) + hrow, kself, 1.f);
    load8(static_cast<const T*>(p.v_cur) + hrow + 8 * c, vself);
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a += qf[k] * kself[k];
    a = group_sum(a, TPH);
    const float mn = fmaxf(m, a);
    const float alpha = exp2_diff(m, mn);
    const float pw = fast_exp2(a - mn);
    l = l * alpha + pw;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = o[k] * alpha + pw * vself[k];
    m = mn;
    // append the current token at position i (no split reads it)
    const int64_t so = row_of(i);
    store8(static_cast<T*>(p.k_pages) + so, kself);
    store8(static_cast<T*>(p.v_pages) + so, vself);
  }

  const int64_t row = ((int64_t)b * p.S + s) * H + h;
  if (c == 0) {
    p.part_ml[row * 2 + 0] = m;
    p.part_ml[row * 2 + 1] = l;
  }
  store8(p.part_o + row * DH + 8 * c, o);
}

template <typename T, int DH>
hipError_t launch_t(const FullParams& p, hipStream_t st) {
  constexpr int HPB = kThreads / (DH / 8);
  const dim3 grid(p.S, p.B, (p.H + HPB - 1) / HPB);
  hipLaunchKernelGGL((k_full_scan<T, DH>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int full_scan_heads_per_block(int dh) { return kThreads / (dh / 8); }

hipError_t launch_full_scan(const FullParams& p, hipStream_t s) {
  if (p.dh != 64 && p.dh != 128) return hipErrorNotSupported;
  if (p.bf16) return p.dh == 128 ? launch_t<bf16, 128>(p, s) : launch_t<bf16, 64>(p, s);
  return p.dh == 128 ? launch_t<float, 128>(p, s) : launch_t<float, 64>(p, s);
}

}  // namespace lla
