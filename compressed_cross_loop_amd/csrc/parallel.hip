// Parallel HLA attention over whole sequences: the second pass of the
// two-pass procedure ("Hybrid Latent Attention" summary, "Training
// Procedure"), i.e. Eq. 4 at every position i of a sequence, with Eq. 3
// scores for the latent tokens j < i - W and the loop's exact keys and values
// for max(0, i-W) <= j <= i.
//
// With many queries per latent token the keys and values are rebuilt once per
// token, k^_j = A_t s^K_j and v^_j = B_t^T s^V_j, and attention runs in head
// space (d_h-wide products instead of r_k- and r_v-wide ones); this equals
// Eq. 3 when A_t commutes with the rotation (frequency-paired decoders) or
// without rotary embedding.  Five launches:
//
//   k_par_prep    q' = R_i q * log2(e)/sqrt(d_h) and k' = R_j k (token-major,
//                 bf16); zero past n_tok
//   k_par_gather  the latents a position can read (j < n_tok - 1 - W) as
//                 token-major rows; the store's dimension-major value
//                 sub-blocks are transposed through LDS; zero rows elsewhere
//   k_gemm_nt     K^ [tokens][H d_h] = S^K A_t^T, per latent group
//   k_gemm_nt     V^ [tokens][H d_h] = S^V B_t, per latent group
//   k_par_attn    causal flash attention over the two key sources, one
//                 online softmax per (position, head), exp2 domain
//
// k_par_attn: workgroup = (128 positions, sequence, head), four waves of 32
// positions (two query blocks of 16), two workgroups per CU (the second
// wave on each SIMD runs its MFMAs while the first works through its
// softmax; a wave of 64 positions needs more than the 256 registers that
// allows and was 1.6x slower).  Key tiles of 64 tokens are staged in
// LDS (keys and values token-major: the exact values straight from the
// caller's v), the next tile's global loads in flight while the current one
// is consumed; a source is staged only when some position of the workgroup
// reads it.  Per 16-token sub-tile and query block:
//   scores  S^T[16 tok x 16 pos] = K[16 x d_h] . Q'^T   (v_mfma_f32_16x16x32_bf16)
//           per element: j > i masked, j < i - W from the rebuilt keys, else
//           from the exact keys
//   values  O^T[d_h x 16 pos] += V^T[d_h x 32 tok] . P^T[32 tok x 16 pos]
//           (v_mfma_f32_16x16x32_bf16; the 32 tokens are two sub-tiles, and
//           each lane's 8 K values are tokens 4g..4g+3 of both, which is the
//           score MFMA's output layout, so P never leaves registers), the
//           latent and exact parts of P against their own values.  The V^T
//           operand comes out of the token-major value tile through the gfx950
//           transposing read ds_read_b64_tr_b16 (inside each 16-lane group lane
//           i receives element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4 and
//           12 + i / 4): two reads give a lane dim 16 db + i of its 8 tokens.
// Workgroups are issued longest (last positions) first.
#include "device_common.h"
#include "gemm_nt.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLazy = 8.f;   // running-max slack of the attention softmax (exp2 units)
// Initial running maximum of the attention softmax: finite, so that 2^(s - m)
// needs no special case (a masked score is -inf and gives 0; the first real
// maximum replaces it and scales the empty sums by 2^(-huge) = 0)
constexpr float kMinMax = -1e30f;
constexpr int kAttnQB = 2;                  // query blocks of 16 positions per wave
constexpr int kAttnWaves = 8;               // waves per attention workgroup
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnQT = kAttnWaves * 16 * kAttnQB;   // positions per attention workgroup
static_assert(kParQueryTile % kAttnQT == 0, "padding must cover whole query tiles");

// ------------------------------------------------------------------ prep
// workgroup = (64 positions, sequence, hpw heads); every thread first loads
// all of its items, then rotates and stores them (one memory round trip)
constexpr int kPrepTokens = 64;

template <int DH>
__global__ __launch_bounds__(kThreads) void k_par_prep(ParParams p, int hpw) {
  constexpr int T = kPrepTokens;
  constexpr int C8 = DH / 8;                      // 16-byte chunks per head row
  constexpr int IPT = 4;                          // items per thread per round
  const int b = blockIdx.y, i0 = blockIdx.x * T, h0 = blockIdx.z * hpw, tid = threadIdx.x;
  const int n = p.n_tok[b], H = p.H;
  __shared__ float cs[T][DH / 2][2];
  __shared__ double theta[DH / 2];
  const bool rope = p.rope_base != 0.f;
  if (tid < DH / 2) theta[tid] = rope ? rope_theta(p.rope_base, DH, tid) : 0.0;
  __syncthreads();
  for (int x = tid; x < T * DH / 2; x += kThreads) {
    const int t = x / (DH / 2), f = x % (DH / 2);
    float c = 1.f, s = 0.f;
    if (rope && i0 + t < n) rope_cs_theta(theta[f], i0 + t, c, s);
    cs[t][f][0] = c;
    cs[t][f][1] = s;
  }
  __syncthreads();
  const bf16* q = static_cast<const bf16*>(p.q);
  const bf16* k = static_cast<const bf16*>(p.k);
  bf16* qr = static_cast<bf16*>(p.qr);
  bf16* kr = static_cast<bf16*>(p.kr);
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<bf16>(0.f);
  // q' and k': item = (token, head, 8 dims); pair (f, f + d_h/2)
  const int items = T * hpw * C8;
  for (int x0 = 0; x0 < items; x0 += IPT * kThreads) {
    bf16x8 qa[IPT], qp[IPT], ka[IPT], kp[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int x = x0 + u * kThreads + tid;
      const int c8 = x % C8, th = x / C8, h = h0 + th % hpw, t = th / hpw, i = i0 + t;
      qa[u] = qp[u] = ka[u] = kp[u] = z;
      if (x < items && i < n) {
        const int64_t row = (((int64_t)b * p.n_max + i) * H + h) * DH;
        const int d0 = 8 * c8, pd = d0 < DH / 2 ? d0 + DH / 2 : d0 - DH / 2;
        qa[u] = *reinterpret_cast<const bf16x8*>(q + row + d0);
        qp[u] = *reinterpret_cast<const bf16x8*>(q + row + pd);
        ka[u] = *reinterpret_cast<const bf16x8*>(k + row + d0);
        kp[u] = *reinterpret_cast<const bf16x8*>(k + row + pd);
      }
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int x = x0 + u * kThreads + tid;
      if (x >= items) continue;
      const int c8 = x % C8, th = x / C8, h = h0 + th % hpw, t = th / hpw, i = i0 + t;
      const int d0 = 8 * c8;
      bf16x8 qo, ko;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + e;
        const int f = d < DH / 2 ? d : d - DH / 2;
        const float c = cs[t][f][0], sn = cs[t][f][1];
        // first half: x_f c - x_{f+h} s; second half: x_f s + x_{f+h} c
        const float qv = d < DH / 2 ? (float)qa[u][e] * c - (float)qp[u][e] * sn
                                    : (float)qp[u][e] * sn + (float)qa[u][e] * c;
        const float kv = d < DH / 2 ? (float)ka[u][e] * c - (float)kp[u][e] * sn
                                    : (float)kp[u][e] * sn + (float)ka[u][e] * c;
        qo[e] = static_cast<bf16>(qv * p.scale);
        ko[e] = static_cast<bf16>(kv);
      }
      const int64_t orow = (((int64_t)b * p.n_pad + i) * H + h) * DH;
      *reinterpret_cast<bf16x8*>(qr + orow + d0) = qo;
      *reinterpret_cast<bf16x8*>(kr + orow + d0) = ko;
    }
  }
}

// ------------------------------------------------------------------ gather
// one 16-token store tile of one group per workgroup
constexpr int kGatherDims = 512;   // value dimensions transposed per LDS round

__global__ __launch_bounds__(kThreads) void k_par_gather(ParParams p) {
  const int j0 = blockIdx.x * kTile, b = blockIdx.y, g = blockIdx.z, tid = threadIdx.x;
  const int n = p.n_tok[b];
  const int nl = max(0, n - 1 - p.W);    // tokens some position reads as latents
  const int G = p.G, rk = p.rk, rv = p.rv, R = rk + rv;
  bf16* sk = static_cast<bf16*>(p.sk) + (((int64_t)b * p.n_pad + j0) * G + g) * rk;   // row t: + t G rk
  bf16* sv = static_cast<bf16*>(p.sv) + (((int64_t)b * p.n_pad + j0) * G + g) * rv;
  const int nv = min(kTile, max(0, nl - j0));   // valid rows of this tile
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<bf16>(0.f);
  const bf16* tile = nullptr;
  if (nv > 0) {
    const int64_t page = p.bt[(int64_t)b * p.max_pages + j0 / p.P];
    tile = static_cast<const bf16*>(p.pages) + ((page * G + g) * (p.P / kTile) + (j0 % p.P) / kTile) * kTile * R;
  }
  // keys: 16 rows of r_k, token-major in the store as here
  for (int x = tid; x < kTile * (rk / 8); x += kThreads) {
    const int t = x / (rk / 8), c = 8 * (x % (rk / 8));
    const bf16x8 val = t < nv ? *reinterpret_cast<const bf16x8*>(tile + t * rk + c) : z;
    *reinterpret_cast<bf16x8*>(sk + (int64_t)t * G * rk + c) = val;
  }
  // values: sub-block d/16 holds [16 dims][16 tokens]
  __shared__ __attribute__((aligned(16))) bf16 vs[kGatherDims / kTile][kTile][kTile + 8];
  for (int d0 = 0; d0 < rv; d0 += kGatherDims) {
    const int nd = min(kGatherDims, rv - d0);
    if (nv > 0) {
      for (int x = tid; x < nd * (kTile / 8); x += kThreads) {
        const int dd = x / 2, half = 8 * (x % 2);   // dim row d0 + dd, tokens half .. half+7
        const int d = d0 + dd;
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(tile + kTile * rk + (d / kTile) * kTile * kTile +
                                                             (d % kTile) * kTile + half);
        *reinterpret_cast<bf16x8*>(&vs[dd / kTile][dd % kTile][half]) = val;
      }
    }
    __syncthreads();
    for (int x = tid; x < kTile * (nd / 8); x += kThreads) {
      const int t = x / (nd / 8), c = 8 * (x % (nd / 8));
      bf16x8 o = z;
      if (t < nv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = vs[(c + e) / kTile][(c + e) % kTile][t];
      }
      *reinterpret_cast<bf16x8*>(sv + (int64_t)t * G * rv + d0 + c) = o;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ attention
template <int DH>
__global__ __launch_bounds__(kAttnThreads, 1) void k_par_attn(ParParams p) {
  constexpr int KT = 64;            // keys per tile
  constexpr int QB = kAttnQB;       // query blocks of 16 per wave
  constexpr int KS = DH / 32;       // K steps of the score MFMA
  constexpr int DB = DH / 16;       // 16-dim blocks of the output
  constexpr int LDK = DH + 8;       // LDS row of a key tile (bf16): 16-byte reads of 16 rows hit distinct banks
  constexpr int LDV = DH + 16;      // LDS row of a value tile: the 4 rows x 32 bytes of a transposing read do
  constexpr int CK = KT * DH / 8 / kAttnThreads;   // 16-B chunks per thread per tile and operand
  static_assert(CK >= 1, "tile too small for the workgroup");
  // two buffers of each staged tile: tile jt + 1 is stored while tile jt is read
  __shared__ __attribute__((aligned(16))) bf16 kl_s[2][KT * LDK];
  __shared__ __attribute__((aligned(16))) bf16 ke_s[2][KT * LDK];
  __shared__ __attribute__((aligned(16))) bf16 vl_s[2][KT * LDV];
  __shared__ __attribute__((aligned(16))) bf16 ve_s[2][KT * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int H = p.H, W = p.W;
  const int nqt = p.n_pad / kAttnQT, BH = p.B * H;
  const int L = blockIdx.x;
  const int qt = nqt - 1 - L / BH, bh = L % BH, b = bh / H, h = bh % H;
  const int n = p.n_tok[b];
  const int q0 = qt * kAttnQT;
  if (q0 >= n) return;                                // whole workgroup
  const int qe = min(q0 + kAttnQT, n) - 1;            // last position of the workgroup
  const int qw0 = q0 + 16 * QB * wave;                // this wave's first position
  const bool wave_on = qw0 <= qe;
  const int qw1 = min(qw0 + 16 * QB - 1, qe);         // its last valid position

  const int64_t trow = (int64_t)H * DH;               // token row stride of [tokens][H][d_h]
  const bf16* qr = static_cast<const bf16*>(p.qr) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* kh = static_cast<const bf16*>(p.kh) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* kr = static_cast<const bf16*>(p.kr) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* vh = static_cast<const bf16*>(p.vh) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* vx = static_cast<const bf16*>(p.v) + (int64_t)b * p.n_max * trow + h * DH;   // caller's v

  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qr + (int64_t)(qw0 + 16 * qb + col) * trow + 32 * ks + 8 * grp);
  f32x4 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kMinMax;
    l[qb] = 0.f;
  }

  // a tile's sources, for the whole workgroup: rebuilt when some j of the
  // tile is below i - W for some position i <= qe, exact when some j lies in
  // [i - W, i] for some i in [q0, qe]
  auto need_lat = [&](int jt) { return jt * KT + W < qe; };
  auto need_ex = [&](int jt) { return jt * KT + KT - 1 >= q0 - W; };
  const int ntile = qe / KT + 1;

  // The next tile's keys and values wait in registers (both sources of the
  // one to three tiles around the window edge, else the one the workgroup
  // reads) while the current tile is consumed, and are stored into the other
  // LDS buffer right after the barrier that ends the reads of the tile before.
  u32x4 rkl[CK], rvl[CK], rke[CK], rve[CK];
  // chunk c of this thread: token row j0 + idx / (DH/8) (clamped to rmax),
  // dims 8 (idx % (DH/8)) ..
  auto chunk = [&](const bf16* src, int j0, int c, int rmax) {
    const int idx = tid + kAttnThreads * c;
    return reinterpret_cast<const u32x4*>(src + (int64_t)min(j0 + idx / (DH / 8), rmax) * trow +
                                          8 * (idx % (DH / 8)));
  };
  auto lds_k = [&](bf16* dst, int c) {
    const int idx = tid + kAttnThreads * c;
    return reinterpret_cast<u32x4*>(dst + (idx / (DH / 8)) * LDK + 8 * (idx % (DH / 8)));
  };
  auto lds_v = [&](bf16* dst, int c) {
    const int idx = tid + kAttnThreads * c;
    return reinterpret_cast<u32x4*>(dst + (idx / (DH / 8)) * LDV + 8 * (idx % (DH / 8)));
  };
  // rows past the sequence are never read by a valid position; the caller's
  // v has n_max rows only, so its rows are clamped to n - 1
  auto load_tile = [&](int jt) {
    const int j0 = jt * KT;
    if (need_lat(jt)) {
#pragma unroll
      for (int c = 0; c < CK; ++c) {
        rkl[c] = *chunk(kh, j0, c, p.n_pad - 1);
        rvl[c] = *chunk(vh, j0, c, p.n_pad - 1);
      }
    }
    if (need_ex(jt)) {
#pragma unroll
      for (int c = 0; c < CK; ++c) {
        rke[c] = *chunk(kr, j0, c, p.n_pad - 1);
        rve[c] = *chunk(vx, j0, c, n - 1);
      }
    }
  };
  auto store_tile = [&](int jt, int buf) {
    if (need_lat(jt)) {
#pragma unroll
      for (int c = 0; c < CK; ++c) {
        *lds_k(kl_s[buf], c) = rkl[c];
        *lds_v(vl_s[buf], c) = rvl[c];
      }
    }
    if (need_ex(jt)) {
#pragma unroll
      for (int c = 0; c < CK; ++c) {
        *lds_k(ke_s[buf], c) = rke[c];
        *lds_v(ve_s[buf], c) = rve[c];
      }
    }
  };

  // one tile: two halves of 32 keys (sub-tiles 2u, 2u+1), each scored,
  // folded into the online softmax and multiplied into the values in turn
  auto compute = [&](int jt, int buf) {
    const int j0 = jt * KT;
    const bf16* KL = kl_s[buf];
    const bf16* KE = ke_s[buf];
    const bf16* VL = vl_s[buf];
    const bf16* VE = ve_s[buf];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc[2][QB];
      // every key of the half is a latent token for every position of the
      // wave (the common case, away from the window edge): no masks
      const bool pure = j0 + 32 * u + 31 < qw0 - W;
      bool lat_u = pure, ex_u = false;
      if (pure) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sc[hs][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf =
                *reinterpret_cast<const bf16x8*>(&KL[(16 * (2 * u + hs) + col) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sc[hs][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], sc[hs][qb], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int ts = 2 * u + hs;
        const int jl = j0 + 16 * ts;   // first key of the sub-tile
        // sources this wave needs for the sub-tile (over its positions qw0 .. qw1)
        const bool any_l = jl + W < qw1;                       // some j < i - W
        const bool any_e = jl + 15 >= qw0 - W && jl <= qw1;    // some i - W <= j <= i
        lat_u |= any_l;
        ex_u |= any_e;
        // masked (j > i) by default; the rebuilt keys' scores where j < i - W,
        // then the exact keys' where i - W <= j <= i
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[hs][qb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (any_l) {
          f32x4 sl[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sl[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&KL[(16 * ts + col) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sl[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], sl[qb], 0, 0, 0);
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (jl + 4 * grp + r < qw0 + 16 * qb + col - W) sc[hs][qb][r] = sl[qb][r];
        }
        if (any_e) {
          f32x4 se[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) se[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&KE[(16 * ts + col) * LDK + 32 * ks + 8 * grp]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              se[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], se[qb], 0, 0, 0);
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = jl + 4 * grp + r, i = qw0 + 16 * qb + col;
              if (j >= i - W && j <= i) sc[hs][qb][r] = se[qb][r];
            }
        }
      }
      }
      if (!lat_u && !ex_u) continue;   // every key of the half follows every position
      // online softmax per position (column) over the 32 keys; sc becomes P
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // The running max moves only when a new score exceeds it by more than
        // kLazy (exp2 units): weights relative to a slightly stale max stay
        // below 2^kLazy, exact in fp32 and bf16, and the output divides by a
        // sum taken relative to the same max.  Each lane first checks its own
        // 8 scores; only when some lane of the wave sees such a score is the
        // maximum of each position reduced over its four lane groups and the
        // accumulators rescaled, which is rare after the first tiles.
        const float lmx = fmaxf(fmaxf(fmaxf(sc[0][qb][0], sc[0][qb][1]), fmaxf(sc[0][qb][2], sc[0][qb][3])),
                                fmaxf(fmaxf(sc[1][qb][0], sc[1][qb][1]), fmaxf(sc[1][qb][2], sc[1][qb][3])));
        if (__any(lmx > m[qb] + kLazy)) {
          float mx = fmaxf(lmx, __shfl_xor(lmx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mn = mx > m[qb] + kLazy ? mx : m[qb];
          const float alpha = fast_exp2(m[qb] - mn);
          m[qb] = mn;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
        }
        const float mn = m[qb];
        float sum = 0.f;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(sc[hs][qb][r] - mn);
            sc[hs][qb][r] = pr;
            sum += pr;
          }
        l[qb] += sum;
      }
      // values: the latent and exact parts of P against their own values.
      // The value MFMA's K index e of this lane is token 4 grp + e % 4 of
      // sub-tile 2u + e / 4.
      // V^T[dims 16 db ..][tokens of this half] as the value MFMA's A operand:
      // lane (col, grp) needs dim 16 db + col of tokens 32 u + 4 grp + e and
      // 32 u + 16 + 4 grp + e (e < 4); each transposing read takes 4 token
      // rows x 4 dims per lane group and hands lane i its dim i
      auto v_operand = [&](const bf16* vt_s, int db) {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const bf16* base = vt_s + (32 * u + 4 * grp + (col >> 2)) * LDV + 16 * db + 4 * (col & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 16 * LDV));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      auto p_part = [&](int qb, bool latent) {
        const int i = qw0 + 16 * qb + col;
        bf16x8 pp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 16 * (2 * u + e / 4) + 4 * grp + e % 4;
          pp[e] = static_cast<bf16>((pure || (j < i - W) == latent) ? sc[e / 4][qb][e % 4] : 0.f);
        }
        return pp;
      };
      if (lat_u) {
        bf16x8 pl[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (pure) {   // every key of the half is a latent token for every position
#pragma unroll
            for (int e = 0; e < 8; ++e) pl[qb][e] = static_cast<bf16>(sc[e / 4][qb][e % 4]);
          } else {
            pl[qb] = p_part(qb, true);
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = v_operand(VL, db);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[qb], acc[qb][db], 0, 0, 0);
        }
      }
      if (ex_u) {
        bf16x8 pe[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pe[qb] = p_part(qb, false);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = v_operand(VE, db);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pe[qb], acc[qb][db], 0, 0, 0);
        }
      }
    }
  };

  load_tile(0);
  store_tile(0, 0);
  if (ntile > 1) load_tile(1);
  for (int jt = 0; jt < ntile; ++jt) {
    // tile jt is in LDS, and every wave is done with tile jt - 1's buffer
    __syncthreads();
    if (jt + 1 < ntile) store_tile(jt + 1, (jt + 1) & 1);
    if (jt + 2 < ntile) load_tile(jt + 2);
    // a wave whose positions all precede the tile has nothing to add
    if (wave_on && jt * KT <= qw1) compute(jt, jt & 1);
  }

  if (!wave_on) return;
  bf16* out = static_cast<bf16*>(p.out);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l[qb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int i = qw0 + 16 * qb + col;
    if (i > qe) continue;
    const float inv = 1.f / lt;
    bf16* orow = out + (((int64_t)b * p.n_max + i) * H + h) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[qb][db][r] * inv);
      *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * grp) = o;
    }
  }
}

template <int DH>
hipError_t launch_dh(const ParParams& p, hipStream_t s, hipEvent_t* ev) {
  const int hpw = p.H % 4 == 0 ? 4 : (p.H % 2 == 0 ? 2 : 1);   // heads per prep workgroup
  hipLaunchKernelGGL((k_par_prep<DH>), dim3(p.n_pad / kPrepTokens, p.B, p.H / hpw), dim3(kThreads), 0, s, p, hpw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_par_gather, dim3(p.n_pad / kTile, p.B, p.G), dim3(kThreads), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int hd = p.hpg * DH;   // output columns (rows) of one latent group
  // K^[b][t][g hd + c] = sum_d S^K[b][t][g][d] A[g hd + c][d]
  GemmParams<bf16> gk{};
  gk.X = static_cast<const bf16*>(p.sk);
  gk.Y = static_cast<const bf16*>(p.A);
  gk.C = static_cast<bf16*>(p.kh);
  gk.M = p.n_pad; gk.N = hd; gk.K = p.rk; gk.kseg = p.rk;
  gk.ldx = p.G * p.rk; gk.ldy = p.rk; gk.ldc = p.H * DH; gk.G = p.G;
  gk.sxb = (int64_t)p.n_pad * p.G * p.rk; gk.sxg = p.rk;
  gk.syb = 0; gk.syg = (int64_t)hd * p.rk;
  gk.scb = (int64_t)p.n_pad * p.H * DH; gk.scg = hd;
  if ((e = launch_gemm(gk, p.B, s)) != hipSuccess) return e;
  // V^[b][t][g hd + c] = sum_d S^V[b][t][g][d] B^T[g hd + c][d]
  GemmParams<bf16> gv{};
  gv.X = static_cast<const bf16*>(p.sv);
  gv.Y = static_cast<const bf16*>(p.Bm);
  gv.C = static_cast<bf16*>(p.vh);
  gv.M = p.n_pad; gv.N = hd; gv.K = p.rv; gv.kseg = p.rv;
  gv.ldx = p.G * p.rv; gv.ldy = p.rv; gv.ldc = p.H * DH; gv.G = p.G;
  gv.sxb = (int64_t)p.n_pad * p.G * p.rv; gv.sxg = p.rv;
  gv.syb = 0; gv.syg = (int64_t)hd * p.rv;
  gv.scb = (int64_t)p.n_pad * p.H * DH; gv.scg = hd;
  if ((e = launch_gemm(gv, p.B, s)) != hipSuccess) return e;
  const int wgs = (p.n_pad / kAttnQT) * p.B * p.H;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_par_attn<DH>), dim3(wgs), dim3(kAttnThreads), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return ev ? hipEventRecord(ev[1], s) : hipSuccess;
}

}  // namespace

hipError_t launch_parallel(const ParParams& p, hipStream_t s, hipEvent_t* events) {
  if (p.dh == 128) return launch_dh<128>(p, s, events);
  if (p.dh == 64) return launch_dh<64>(p, s, events);
  return hipErrorNotSupported;
}

}  // namespace lla
