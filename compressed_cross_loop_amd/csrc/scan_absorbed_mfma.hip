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
// With fuse_window set, split s also handles slice s of the exact window
// (window_slice below), so those bytes stream in the same launch.
//
// Latent tiles and ring rows are read exactly once per call, so their loads
// are non-temporal (measured: 211.7 -> 201.0 us per main-set call on the
// Ouro-1.4B shape at batch 128, 4k).
//
// The tile loop is software-pipelined (keys two to four tiles ahead, values
// one to four, by latent width).  q~ is read from LDS to leave registers for
// the key pipeline.  At the end the
// four waves are merged (same-max rescale, fixed order) in LDS and one
// partial (m, l, O_latent) per head is written for the combine kernel.
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Page ids of a split are staged in LDS: a block-table read inside the tile
// loop is a vector load, and waiting for it (vmcnt counts loads in issue
// order) would also wait for every tile load the pipeline has in flight.
constexpr int kPageTab = 8192;

// Prefetch depth per latent width (measured): narrow tiles carry few bytes,
// so they run further ahead to keep enough of HBM's latency covered; wide
// tiles already keep enough in flight, and every CU streaming its own pages
// with more requests outstanding only adds DRAM contention (r = 512 is
// fastest one tile ahead).
template <int RK> struct Pipe { static constexpr int keys = 4, values = 4, unroll = 4; };
template <> struct Pipe<128> { static constexpr int keys = 4, values = 2, unroll = 4; };
template <> struct Pipe<256> { static constexpr int keys = 3, values = 2, unroll = 6; };
template <> struct Pipe<512> { static constexpr int keys = 1, values = 1, unroll = 1; };
// fp8 tiles hold half the bytes (and registers) of bf16 ones: deeper at
// narrow widths, and again shallow at r = 512
template <int RK> struct Pipe8 { static constexpr int keys = 4, values = 4, unroll = 4; };
template <> struct Pipe8<256> { static constexpr int keys = 4, values = 2, unroll = 4; };
template <> struct Pipe8<512> { static constexpr int keys = 2, values = 1, unroll = 2; };

template <int RK, bool NT>
__device__ __forceinline__ void load_keys(bf16x8 (&k)[RK / 32], const char* tile_b, int col, int grp) {
  const bf16* kp = reinterpret_cast<const bf16*>(tile_b) + col * RK + grp * 8;
#pragma unroll
  for (int st = 0; st < RK / 32; ++st) k[st] = load_once<NT>(reinterpret_cast<const bf16x8*>(kp + st * 32));
}

template <int RK, int RV, bool NT>
__device__ __forceinline__ void load_values(s16x4 (&v)[RV / 16], const char* tile_b, int col, int grp) {
  const bf16* vp = reinterpret_cast<const bf16*>(tile_b) + 16 * RK + col * 16 + grp * 4;
#pragma unroll
  for (int vt = 0; vt < RV / 16; ++vt) v[vt] = load_once<NT>(reinterpret_cast<const s16x4*>(vp + vt * 256));
}

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, static_cast<bf16>(x));
}

// Scores of one tile; lane (head = lane&15, grp) gets tokens 4*grp + r.
// q~ rows live in LDS (row stride RK + 8 bf16, so the 16 lanes of a group
// read 16 distinct bank quads).
template <int RK>
__device__ __forceinline__ f32x4 tile_scores(const bf16x8 (&k)[RK / 32], const bf16* qrow) {
  // two independent accumulator chains over the K steps
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < RK / 32; ++st) {
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + st * 32);
    if (st & 1)
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[st], qv, s1, 0, 0, 0);
    else
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[st], qv, s0, 0, 0, 0);
  }
  return s0 + s1;
}

// Online-softmax update for one tile; returns the bf16 probabilities in the
// B-operand layout of the value MFMA.
template <int RV, bool SCALED = false>
__device__ __forceinline__ s16x4 tile_softmax(f32x4 sc, f32x4 (&acc)[RV / 16], float& m, float& lsum,
                                              int nvalid, int grp, f32x4 vscale = f32x4{1.f, 1.f, 1.f, 1.f}) {
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
  for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - mn);
  lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  m = mn;
  // rescale only when some head's running max moved (rare after a few tiles)
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int vt = 0; vt < RV / 16; ++vt) acc[vt] *= alpha;
  }
  s16x4 pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // fp8 values carry a per-token scale; a token past the end may hold
    // anything (even NaN) there: select, not multiply
    const float w = SCALED ? ((4 * grp + r < nvalid) ? pr[r] * vscale[r] : 0.f) : pr[r];
    pb[r] = bf16_bits(w);
  }
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

// ---- fp8 latents (OCP e4m3 codes + per-token fp32 scales, the byte tile
// layout of device_common.h).  Key codes are read 16 per lane (dims
// 64u + 16 grp ..); the score MFMA sums over its 32 K values, so the two
// 8-dim halves of a load feed two K steps, each against the q~ dims they hold.
// Value codes: one 16-byte load per lane gives its 4 tokens of 4 sub-blocks.
// Codes are converted exactly to bf16 (gfx950 converter), the MFMAs are the
// bf16 ones; scales multiply the scores (key) and the probabilities (value).
template <int RK> struct Keys8 {
  u32x4 v[RK / 64];
  f32x4 s;   // key scales of tokens 4 grp .. 4 grp + 3
};
template <int RV> struct Vals8 {
  u32x4 v[RV / 64];
  f32x4 s;   // value scales of tokens 4 grp .. 4 grp + 3
};

template <int RK, int RV, bool NT>
__device__ __forceinline__ void load_keys8(Keys8<RK>& k, const char* tile, int col, int grp) {
  const char* kp = tile + col * RK + grp * 16;
#pragma unroll
  for (int u = 0; u < RK / 64; ++u) k.v[u] = load_once<NT>(reinterpret_cast<const u32x4*>(kp + u * 64));
  k.s = load_once<NT>(reinterpret_cast<const f32x4*>(tile + 16 * (RK + RV) + 16 * grp));
}

template <int RK, int RV, bool NT>
__device__ __forceinline__ void load_values8(Vals8<RV>& v, const char* tile, int col, int grp) {
  const char* vp = tile + 16 * RK + col * 64 + grp * 16;
#pragma unroll
  for (int q = 0; q < RV / 64; ++q) v.v[q] = load_once<NT>(reinterpret_cast<const u32x4*>(vp + q * 1024));
  v.s = load_once<NT>(reinterpret_cast<const f32x4*>(tile + 16 * (RK + RV) + 64 + 16 * grp));
}

// two bf16 from the e4m3 codes in bytes (2 hi, 2 hi + 1) of w
template <bool HI>
__device__ __forceinline__ unsigned e4m3x2_to_bf16x2(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int RK, int RV>
__device__ __forceinline__ f32x4 tile_scores8(const Keys8<RK>& k, const bf16* qcol, int grp) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < RK / 64; ++u) {
    u32x4 a0, a1;   // dims 64u + 16 grp + 0..7 and + 8..15, as bf16 pairs
    a0[0] = e4m3x2_to_bf16x2<false>(k.v[u][0]);
    a0[1] = e4m3x2_to_bf16x2<true>(k.v[u][0]);
    a0[2] = e4m3x2_to_bf16x2<false>(k.v[u][1]);
    a0[3] = e4m3x2_to_bf16x2<true>(k.v[u][1]);
    a1[0] = e4m3x2_to_bf16x2<false>(k.v[u][2]);
    a1[1] = e4m3x2_to_bf16x2<true>(k.v[u][2]);
    a1[2] = e4m3x2_to_bf16x2<false>(k.v[u][3]);
    a1[3] = e4m3x2_to_bf16x2<true>(k.v[u][3]);
    const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qcol + 64 * u + 16 * grp);
    const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(qcol + 64 * u + 16 * grp + 8);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), q0, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), q1, s1, 0, 0, 0);
  }
  return (s0 + s1) * k.s;
}

template <int RV>
__device__ __forceinline__ void tile_values8(const Vals8<RV>& v, s16x4 pb, f32x4 (&acc)[RV / 16], int nvalid,
                                             int grp) {
  // tokens past the end may hold anything (even NaN codes): byte r of a word
  // is token 4 grp + r, so one AND per word turns them into +0 codes
  const int nv = nvalid - 4 * grp;
  const unsigned keep = nv >= 4 ? 0xFFFFFFFFu : (nv <= 0 ? 0u : 0xFFFFFFFFu >> (8 * (4 - nv)));
#pragma unroll
  for (int q = 0; q < RV / 64; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // sub-block 4q + j, tokens 4 grp .. 4 grp + 3 of this lane's dim row
      const unsigned w = v.v[q][j] & keep;
      unsigned w2[2] = {e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
      acc[4 * q + j] =
          __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, w2), pb, acc[4 * q + j], 0, 0, 0);
    }
}

// Exact tokens i-W <= j <= i of Eq. 4 (ring slots and the current token) for
// window slice `slice` of sequence b, heads of group g: thread (head hl, c)
// owns dims 8c..8c+7 of head hl (16-byte loads of the [H][d_h] ring rows),
// per-head online softmax, partial (m, l, o) in head space.  The slice that
// holds the current token also appends R_i k_cur, v_cur to the ring.
// cs[f] = (cos, sin) of i * theta_f.
template <bool NT>
__device__ void window_slice(const DecodeParams& p, int b, int slice, int g, const float (*cs)[2]) {
  const int DH = p.dh, TPH = DH / 8, H = p.H, W = p.W;
  const int tid = threadIdx.x;
  const int hl = tid / TPH, c = tid % TPH;
  if (hl >= p.hpg) return;                 // whole TPH-lane groups drop out together
  const int h = g * p.hpg + hl;
  const int i = p.pos[b];
  const int j0 = max(0, i - W);
  const int nw = i - j0;
  const int t0 = slice * p.tw, t1 = min(t0 + p.tw, nw + 1);
  const bool rope = p.rope_base != 0.f;
  const int pc = (8 * c < DH / 2) ? 8 * c + DH / 2 : 8 * c - DH / 2;
  auto rotate = [&](const bf16x8& x, const bf16x8& xp, float* out, float scale) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = 8 * c + k;
      const int f = d < DH / 2 ? d : d - DH / 2;
      const float cc = rope ? cs[f][0] : 1.f, sn = rope ? cs[f][1] : 0.f;
      const float a = to_f(x[k]), bp = to_f(xp[k]);
      out[k] = scale * (d < DH / 2 ? a * cc - bp * sn : bp * sn + a * cc);
    }
  };
  const int64_t hrow = ((int64_t)b * H + h) * DH;
  float qf[8];
  {
    const bf16* qr = static_cast<const bf16*>(p.q) + hrow;
    rotate(*reinterpret_cast<const bf16x8*>(qr + 8 * c), *reinterpret_cast<const bf16x8*>(qr + pc), qf,
           p.scale);
  }
  const bool has_self = t0 <= nw && nw < t1;
  float kself[8], vself[8];
  if (has_self) {
    const bf16* kc = static_cast<const bf16*>(p.k_cur) + hrow;
    rotate(*reinterpret_cast<const bf16x8*>(kc + 8 * c), *reinterpret_cast<const bf16x8*>(kc + pc), kself,
           1.f);
    const bf16x8 vv = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.v_cur) + hrow + 8 * c);
#pragma unroll
    for (int k = 0; k < 8; ++k) vself[k] = to_f(vv[k]);
  }
  const bf16* ring_k = static_cast<const bf16*>(p.ring_k);
  const bf16* ring_v = static_cast<const bf16*>(p.ring_v);
  const int64_t rs = (int64_t)H * DH;
  const int64_t base = (int64_t)b * (W + 1) * rs + (int64_t)h * DH + 8 * c;
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  // batches of U ring tokens, double-buffered: batch n+1 is requested before
  // batch n is consumed.  Loads past the slice reread a valid slot, so every
  // refill is unconditional.
  constexpr int U = 8;
  auto slot_of = [&](int t) { return (j0 + min(t, max(nw - 1, 0))) % (W + 1); };
  auto load_batch = [&](bf16x8 (&kr)[U], bf16x8 (&vr)[U], int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = base + slot_of(tb + u) * rs;
      kr[u] = load_once<NT>(reinterpret_cast<const bf16x8*>(ring_k + off));
      vr[u] = load_once<NT>(reinterpret_cast<const bf16x8*>(ring_v + off));
    }
  };
  // one batch: U independent score reductions, one max, then the weighted
  // sum (no per-token dependency chain)
  auto consume = [&](const bf16x8 (&kr)[U], const bf16x8 (&vr)[U], int tb) {
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u;
      float a = 0.f;
      if (t < nw) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a += qf[k] * to_f(kr[u][k]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) a += qf[k] * kself[k];
      }
      sc[u] = group_sum(a, TPH);   // the TPH lanes of this head
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
      const int t = tb + u;
      const float pw = fast_exp2(sc[u] - mn);
      l += pw;
      if (t < nw) {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] += pw * to_f(vr[u][k]);
      } else if (t < t1) {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] += pw * vself[k];
      }
    }
    m = mn;
  };
  if (t0 < t1) {
    bf16x8 kA[U], vA[U], kB[U], vB[U];
    load_batch(kA, vA, t0);
    for (int tb = t0; tb < t1; tb += 2 * U) {
      load_batch(kB, vB, tb + U);
      consume(kA, vA, tb);
      if (tb + U >= t1) break;
      load_batch(kA, vA, tb + 2 * U);
      consume(kB, vB, tb + U);
    }
  }
  const int64_t row = ((int64_t)b * p.WS + slice) * H + h;
  if (c == 0) {
    p.win_ml[row * 2 + 0] = m;
    p.win_ml[row * 2 + 1] = l;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) p.win_o[row * DH + 8 * c + k] = o[k];
  if (has_self) {
    // slot i mod (W+1) held token i-W-1, which no slice reads
    const int64_t so = (int64_t)b * (W + 1) * rs + (int64_t)(i % (W + 1)) * rs + (int64_t)h * DH + 8 * c;
    bf16x8 kw, vw;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      kw[k] = static_cast<bf16>(kself[k]);
      vw[k] = static_cast<bf16>(vself[k]);
    }
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.ring_k) + so) = kw;
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.ring_v) + so) = vw;
  }
}

template <int RK, int RV, bool F8, bool NT>
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

  // q~ of the group's heads (B operand of the score MFMA), staged in LDS
  __shared__ __attribute__((aligned(16))) bf16 qs[16][RK + 8];
  {
    const bf16* qsrc = static_cast<const bf16*>(p.qlat) + ((int64_t)b * p.H + (int64_t)g * hpg) * RK;
    for (int x = tid; x < 16 * RK / 8; x += kThreads) {
      const int hh = x / (RK / 8), c8 = (x % (RK / 8)) * 8;
      bf16x8 v;
      if (hh < hpg) {
        v = *reinterpret_cast<const bf16x8*>(qsrc + (int64_t)hh * RK + c8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(0.f);
      }
      *reinterpret_cast<bf16x8*>(&qs[hh][c8]) = v;
    }
  }
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  __shared__ int32_t ptab[kPageTab];
  const int pfirst = t0 / P;
  {
    // pages of tokens t0 .. t1-1; never more than max_pages <= kPageTab
    const int npt = t1 > t0 ? (t1 - 1) / P - pfirst + 1 : 0;
    for (int x = tid; x < npt; x += kThreads) ptab[x] = bt[pfirst + x];
  }
  __syncthreads();
  const bf16* qrow = &qs[col][grp * 8];
  f32x4 acc[RV / 16];
#pragma unroll
  for (int vt = 0; vt < RV / 16; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const char* pages = static_cast<const char*>(p.pages);
  const int R = RK + RV;
  const int ntiles = (t1 - t0 + 15) / 16;
  auto tile_ptr = [&](int ti) -> const char* {   // byte address of a 16-token tile
    const int j0 = t0 + ti * 16;
    const int64_t page = ptab[j0 / P - pfirst];
    if constexpr (F8) return pages + tile_base8(page, g, j0 % P, G, P, RK, RV);
    return pages + 2 * tile_base(page, g, j0 % P, G, P, R);
  };
  auto tile_valid = [&](int ti) -> int { return min(16, t1 - (t0 + ti * 16)); };

  // Keys run NK tiles (of this wave) ahead, values NV: tile n+NK's keys are
  // requested as soon as the score MFMAs have consumed tile n's, tile n+NV's
  // values as soon as tile n's value MFMAs are issued.  The register sets
  // rotate with the loop unrolled by lcm(NK, NV), so every index is static.
  // Refills are unconditional (clamped to the last tile, still cached) so no
  // register set has to survive a skipped refill.
  if constexpr (!F8) {
    constexpr int NK = Pipe<RK>::keys, NV = Pipe<RK>::values, UN = Pipe<RK>::unroll;
    bf16x8 kb[NK][RK / 32];
    s16x4 vb[NV][RV / 16];
    int ti = wave;
    if (ti < ntiles) {
#pragma unroll
      for (int u = 0; u < NK; ++u) load_keys<RK, NT>(kb[u], tile_ptr(min(ti + u * kWaves, ntiles - 1)), col, grp);
#pragma unroll
      for (int u = 0; u < NV; ++u)
        load_values<RK, RV, NT>(vb[u], tile_ptr(min(ti + u * kWaves, ntiles - 1)), col, grp);
    }
    while (ti < ntiles) {
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const f32x4 sc = tile_scores<RK>(kb[u % NK], qrow);
        __builtin_amdgcn_sched_barrier(0);   // keep each refill below its consumer
        load_keys<RK, NT>(kb[u % NK], tile_ptr(min(ti + NK * kWaves, ntiles - 1)), col, grp);
        const s16x4 pb = tile_softmax<RV>(sc, acc, m, lsum, tile_valid(ti), grp);
        tile_values<RV>(vb[u % NV], pb, acc, tile_valid(ti), grp);
        __builtin_amdgcn_sched_barrier(0);
        load_values<RK, RV, NT>(vb[u % NV], tile_ptr(min(ti + NV * kWaves, ntiles - 1)), col, grp);
        ti += kWaves;
        if (ti >= ntiles) break;
      }
    }
  } else {
    constexpr int NK = Pipe8<RK>::keys, NV = Pipe8<RK>::values, UN = Pipe8<RK>::unroll;
    Keys8<RK> kb[NK];
    Vals8<RV> vb[NV];
    const bf16* qcol = &qs[col][0];
    int ti = wave;
    if (ti < ntiles) {
#pragma unroll
      for (int u = 0; u < NK; ++u)
        load_keys8<RK, RV, NT>(kb[u], tile_ptr(min(ti + u * kWaves, ntiles - 1)), col, grp);
#pragma unroll
      for (int u = 0; u < NV; ++u)
        load_values8<RK, RV, NT>(vb[u], tile_ptr(min(ti + u * kWaves, ntiles - 1)), col, grp);
    }
    while (ti < ntiles) {
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        f32x4 sc = tile_scores8<RK, RV>(kb[u % NK], qcol, grp);
        __builtin_amdgcn_sched_barrier(0);
        const f32x4 vs = vb[u % NV].s;
        load_keys8<RK, RV, NT>(kb[u % NK], tile_ptr(min(ti + NK * kWaves, ntiles - 1)), col, grp);
        const s16x4 pb = tile_softmax<RV, true>(sc, acc, m, lsum, tile_valid(ti), grp, vs);
        tile_values8<RV>(vb[u % NV], pb, acc, tile_valid(ti), grp);
        __builtin_amdgcn_sched_barrier(0);
        load_values8<RK, RV, NT>(vb[u % NV], tile_ptr(min(ti + NV * kWaves, ntiles - 1)), col, grp);
        ti += kWaves;
        if (ti >= ntiles) break;
      }
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // ---- this split's slice of the exact window (same launch, same HBM stream)
  if (p.fuse_window) {
    __shared__ float cs[64][2];
    if (tid < p.dh / 2) {
      float c = 1.f, sn = 0.f;
      if (p.rope_base != 0.f) rope_cs(p.rope_base, p.dh, tid, i, c, sn);
      cs[tid][0] = c;
      cs[tid][1] = sn;
    }
    __syncthreads();
    window_slice<NT>(p, b, s, g, cs);
  }

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

template <int RK, int RV, bool NT>
hipError_t launch_rk_nt(const DecodeParams& p, hipStream_t st) {
  if (p.fp8) {
    if constexpr (RK % 64 == 0)
      hipLaunchKernelGGL((k_scan_absorbed_mfma<RK, RV, true, NT>), dim3(p.S, p.B, p.G), dim3(kThreads), 0, st, p);
    else
      return hipErrorNotSupported;
  } else {
    hipLaunchKernelGGL((k_scan_absorbed_mfma<RK, RV, false, NT>), dim3(p.S, p.B, p.G), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

// streaming loads when the launch keeps every CU busy (load_once)
template <int RK, int RV>
hipError_t launch_rk(const DecodeParams& p, hipStream_t st) {
  if ((int64_t)p.S * p.B * p.G >= kStreamWorkgroups) return launch_rk_nt<RK, RV, true>(p, st);
  return launch_rk_nt<RK, RV, false>(p, st);
}

}  // namespace

bool scan_absorbed_mfma_supports(const DecodeParams& p) {
  if (!p.bf16 || p.hpg > 16 || p.rk != p.rv || p.max_pages > kPageTab) return false;
  if (p.fp8 && p.rk % 64) return false;
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
