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
//   k_rope_table  (cos, sin) of every position and frequency, once per call
//                 (the attention rotates its query rows and exact keys with it)
//   k_par_gather  the latents a position can read (j < n_tok - 1 - W) as
//                 token-major rows; the store's dimension-major value
//                 sub-blocks are transposed through LDS; zero rows elsewhere
//   k_gemm_nt     K^ [tokens][H d_h] = S^K A_t^T, per latent group
//   k_gemm_nt     V^ [tokens][H d_h] = S^V B_t, per latent group
//   k_par_attn    causal flash attention over the two key sources, one
//                 online softmax per (position, head), exp2 domain
//
// k_par_attn: workgroup = (256 positions, sequence, head), eight waves of 32
// positions (two query blocks of 16), one workgroup per CU.  Key and value
// tiles of 64 tokens are copied straight into LDS (global_load_lds, 1 KiB
// per instruction; rows of d_h with their 16-byte chunks XOR-swizzled by row
// against bank conflicts), double buffered: tile jt + 1's copies are in
// flight while tile jt is read, one barrier per tile; a source is copied only
// when some position of the workgroup reads it.  The exact keys are copied
// from the caller's k and rotated in LDS once they land (R_j k, with the
// angles of the table by angle addition), behind one more barrier; the query
// rows are rotated in registers.  Per 16-token sub-tile and
// query block:
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
// A wave's tiles whose keys are all latent tokens for all of its positions
// (most of them) run a separate mask-free loop: scores start from -m so the
// products give s - m, the lazy running-max test is an integer max3 chain on
// the score bits, P is packed pairwise to bf16, and its row sums come from one
// more product against ones.  Keeping that loop apart from the masked one
// lets the value accumulators stay in place (a shared loop body made the
// register allocator shuffle them every half-tile).
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

// ------------------------------------------------------------------ rotary table
// (cos, sin) of position i and frequency f, for every position up to the
// padded length: one thread per entry, fp64 angles (the same for every
// sequence, layer and loop of the call)
template <int DH>
__global__ __launch_bounds__(kThreads) void k_rope_table(ParParams p) {
  const int x = blockIdx.x * kThreads + threadIdx.x;
  if (x >= p.n_pad * (DH / 2)) return;
  const int i = x / (DH / 2), f = x % (DH / 2);
  float c = 1.f, s = 0.f;
  if (p.rope_base != 0.f) rope_cs(p.rope_base, DH, f, i, c, s);
  static_cast<float2*>(p.rtab)[x] = make_float2(c, s);
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
    const bf16x8 val = t < nv ? *reinterpret_cast<const bf16x8*>(tile + key_in_tile(t, c, rk)) : z;
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
  // Tiles sit in LDS as plain [KT][d_h] rows with the 16-byte chunks of row r
  // stored at chunk position c ^ (r % NCH), so that the 16-row key reads and
  // the transposing value reads spread over the banks.  They are copied
  // straight from global memory (copy_to_lds: 1 KiB per instruction, RPC rows
  // each), the next tile's copies in flight while the current one is read.
  constexpr int NCH = DH / 8;                 // 16-byte chunks per row
  constexpr int RPC = 512 / DH;               // rows per 1 KiB copy
  constexpr int NCP = KT * DH / 512;          // copies per source tile
  constexpr int CPW = NCP / kAttnWaves;       // ... per wave
  static_assert(NCP % kAttnWaves == 0, "tile copies must divide over the waves");
  // two buffers of each staged tile: tile jt + 1 is copied while tile jt is read
  __shared__ __attribute__((aligned(1024))) bf16 kl_s[2][KT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 ke_s[2][KT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 vl_s[2][KT * DH];
  __shared__ __attribute__((aligned(1024))) bf16 ve_s[2][KT * DH];
  // (cos, sin) rows for the exact keys' rotation, R_j = R_(j - j % 16) R_(j % 16),
  // per wave for the RPC x CPW rows its own copies bring: its RPC offset rows
  // (j % 16, the same for every tile; 2 KiB) and, per buffer, the rows of
  // the 16-token blocks its rows fall in (one per copy; 1 KiB)
  __shared__ __attribute__((aligned(1024))) char tb_s[kAttnWaves][2048];
  __shared__ __attribute__((aligned(1024))) char ta_s[2][kAttnWaves][1024];
  static_assert(RPC * 4 * DH == 2048 && CPW * 4 * DH <= 1024 && 16 % RPC == 0, "rotation table slots");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: per-wave choices are scalar branches
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
  const bf16* qx = static_cast<const bf16*>(p.q) + (int64_t)b * p.n_max * trow + h * DH;     // caller's q
  const bf16* kh = static_cast<const bf16*>(p.kh) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* kx = static_cast<const bf16*>(p.k) + (int64_t)b * p.n_max * trow + h * DH;     // caller's k
  const bf16* vh = static_cast<const bf16*>(p.vh) + (int64_t)b * p.n_pad * trow + h * DH;
  const bf16* vx = static_cast<const bf16*>(p.v) + (int64_t)b * p.n_max * trow + h * DH;   // caller's v

  bf16x8 qf[QB][KS];   // q', filled once tile 0's copies are in flight (below)
  f32x4 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[QB], l[QB];
  f32x4 accl[QB];   // row sums of P from the no-mask halves (every entry: the position's sum)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kMinMax;
    l[qb] = 0.f;
    accl[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<bf16>(1.f);

  // a tile's sources, for the whole workgroup: rebuilt when some j of the
  // tile is below i - W for some position i <= qe, exact when some j lies in
  // [i - W, i] for some i in [q0, qe]
  auto need_lat = [&](int jt) { return jt * KT + W < qe; };
  auto need_ex = [&](int jt) { return jt * KT + KT - 1 >= q0 - W; };
  const int ntile = qe / KT + 1;

  // this lane's row and source chunk in copy q of the wave (copy wave + 8 q)
  int crow[CPW], cchunk[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    crow[q] = (wave + kAttnWaves * q) * RPC + lane / NCH;
    cchunk[q] = (lane % NCH) ^ (crow[q] % NCH);
  }
  // rows past the sequence are never read by a valid position; the caller's
  // v has n_max rows only, so its rows are clamped to n - 1
  auto copy_source = [&](const bf16* src, int j0, int rmax, bf16* dst) {
#pragma unroll
    for (int q = 0; q < CPW; ++q)
      copy_to_lds(src + (int64_t)min(j0 + crow[q], rmax) * trow + 8 * cchunk[q],
                  dst + (wave + kAttnWaves * q) * 512);
  };
  auto issue_tile = [&](int jt, int buf) {
    const int j0 = jt * KT;
    if (need_lat(jt)) {
      copy_source(kh, j0, p.n_pad - 1, kl_s[buf]);
      copy_source(vh, j0, p.n_pad - 1, vl_s[buf]);
    }
    if (need_ex(jt)) {
      copy_source(kx, j0, n - 1, ke_s[buf]);
      copy_source(vx, j0, n - 1, ve_s[buf]);
      // block rows: lane group q (64 / CPW lanes) takes the row of copy q's
      // 16-token block; a row is 4 d_h bytes (lanes past it repeat it)
      const int qg = lane / (64 / CPW);
      copy_to_lds(static_cast<const char*>(p.rtab) +
                      (int64_t)(j0 + 16 * (((wave + kAttnWaves * qg) * RPC) / 16)) * (4 * DH) +
                      16 * (lane % (DH / 4)),
                  &ta_s[buf][wave][0]);
    }
  };
  // R_j k of the exact keys this wave copied (rows (wave + 8 q) RPC + x),
  // in place once they have landed: lane -> (row, dims 8 c .. 8 c + 7 and
  // their partners d + d_h/2); nothing another wave wrote is read
  auto rotate_own = [&](int buf) {
    constexpr int PPR = NCH / 2;   // chunk pairs per row
    if (lane >= CPW * RPC * PPR) return;
    const int ri = lane / PPR, c = lane % PPR, qg = ri / RPC, x = ri % RPC;
    const int r = (wave + kAttnWaves * qg) * RPC + x;
    bf16x8* plo = reinterpret_cast<bf16x8*>(&ke_s[buf][r * DH + 8 * (c ^ (r % NCH))]);
    bf16x8* phi = reinterpret_cast<bf16x8*>(&ke_s[buf][r * DH + 8 * ((c + PPR) ^ (r % NCH))]);
    const bf16x8 lo = *plo, hi = *phi;
    const float4* ta = reinterpret_cast<const float4*>(&ta_s[buf][wave][qg * (1024 / CPW) + 64 * c]);
    const float4* tb = reinterpret_cast<const float4*>(&tb_s[wave][x * 4 * DH + 64 * c]);
    bf16x8 olo, ohi;
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const float4 a4 = ta[c2], b4 = tb[c2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * c2 + u;
        const float ca = u ? a4.z : a4.x, sa = u ? a4.w : a4.y;
        const float cb = u ? b4.z : b4.x, sb = u ? b4.w : b4.y;
        const float cc = ca * cb - sa * sb, sn = sa * cb + ca * sb;
        const float x0 = (float)lo[e], x1 = (float)hi[e];
        // first half: x_f c - x_{f+h} s; second half: x_f s + x_{f+h} c
        olo[e] = static_cast<bf16>(x0 * cc - x1 * sn);
        ohi[e] = static_cast<bf16>(x0 * sn + x1 * cc);
      }
    }
    *plo = olo;
    *phi = ohi;
  };
  // key row 16 ts + col, chunk 4 ks + grp (the row's swizzle is col % NCH)
  auto key_frag = [&](const bf16* kt_s, int ts, int ks) {
    return *reinterpret_cast<const bf16x8*>(&kt_s[(16 * ts + col) * DH + 8 * ((4 * ks + grp) ^ (col % NCH))]);
  };
  // V^T[dims 16 db ..][tokens of half u] as the value MFMA's A operand: lane
  // (col, grp) needs dim 16 db + col of tokens 32 u + 4 grp + e and
  // 32 u + 16 + 4 grp + e (e < 4); each transposing read takes 4 token rows x
  // 4 dims per lane group and hands lane i its dim i.  Rows r and r + 16 share
  // their chunk swizzle.
  auto value_frag = [&](const bf16* vt_s, int u, int db) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int r = 32 * u + 4 * grp + (col >> 2);
    const int c = 2 * db + ((col & 3) >> 1);
    const bf16* base = vt_s + r * DH + 8 * (c ^ (r % NCH)) + 4 * (col & 1);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 16 * DH));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // one tile: two halves of 32 keys (sub-tiles 2u, 2u+1), each scored,
  // folded into the online softmax and multiplied into the values in turn
  // A tile whose keys are all latent tokens for every position of the wave
  // (the common case, away from the window edge): no masks.  The score
  // products start from -m, so they yield s - m directly; the lazy-max test
  // reads the scores' bits as signed integers (for a positive threshold
  // x > k exactly when int(x) > int(k)), which needs no float
  // canonicalisation; the row sums of P come from one more product against
  // ones.  Runs only once every position's running maximum is a real score.
  auto fast_tile = [&](int buf) {
    const bf16* KL = kl_s[buf];
    const bf16* VL = vl_s[buf];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc[2][QB];

#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float nm = -m[qb];
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) sc[hs][qb] = f32x4{nm, nm, nm, nm};
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf = key_frag(KL, 2 * u + hs, ks);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sc[hs][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], sc[hs][qb], 0, 0, 0);
          }
        }
        bf16x8 pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int b0i = max(max(__float_as_int(sc[0][qb][0]), __float_as_int(sc[0][qb][1])),
                              __float_as_int(sc[0][qb][2]));
          const int b1i = max(max(__float_as_int(sc[0][qb][3]), __float_as_int(sc[1][qb][0])),
                              __float_as_int(sc[1][qb][1]));
          const int b2i = max(max(__float_as_int(sc[1][qb][2]), __float_as_int(sc[1][qb][3])), b0i);
          if (__any(max(b1i, b2i) > __float_as_int(kLazy))) {
            float lmx = -INFINITY;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
              for (int r = 0; r < 4; ++r) lmx = fmaxf(lmx, sc[hs][qb][r]);
            float mx = fmaxf(lmx, __shfl_xor(lmx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float d = mx > kLazy ? mx : 0.f;   // the position's maximum moves up by d
            const float alpha = fast_exp2(-d);
            m[qb] += d;
            l[qb] *= alpha;
            accl[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
              for (int r = 0; r < 4; ++r) sc[hs][qb][r] -= d;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[qb][e] = static_cast<bf16>(fast_exp2(sc[e / 4][qb][e % 4]));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = value_frag(VL, u, db);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], acc[qb][db], 0, 0, 0);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) accl[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb], accl[qb], 0, 0, 0);
    }
  };

  // general tile (masks): tiles near the window edge or the diagonal, and a
  // wave's first tile
  auto compute = [&](int jt, int buf) {
    const int j0 = jt * KT;
    const bf16* KL = kl_s[buf];
    const bf16* KE = ke_s[buf];
    const bf16* VL = vl_s[buf];
    const bf16* VE = ve_s[buf];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc[2][QB];

      // general path (masks): halves near the window edge or the diagonal,
      // and a wave's first half
      bool lat_u = false, ex_u = false;
      {
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
            const bf16x8 kf = key_frag(KL, ts, ks);
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
            const bf16x8 kf = key_frag(KE, ts, ks);
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
          accl[qb] *= alpha;
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
      auto v_operand = [&](const bf16* vt_s, int db) { return value_frag(vt_s, u, db); };
      auto p_part = [&](int qb, bool latent) {
        const int i = qw0 + 16 * qb + col;
        bf16x8 pp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 16 * (2 * u + e / 4) + 4 * grp + e % 4;
          pp[e] = static_cast<bf16>((j < i - W) == latent ? sc[e / 4][qb][e % 4] : 0.f);
        }
        return pp;
      };
      if (lat_u) {
        bf16x8 pl[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pl[qb] = p_part(qb, true);
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

  // Every tile starts with the same step: this wave's copies of tile jt have
  // landed; after the barrier everyone's have, and every wave is done with
  // tile jt - 1's buffer, which takes tile jt + 1.  Each wave passes one
  // barrier per tile, in whichever of the loops below it is.
  // A tile with exact keys has each wave rotate the rows it copied before
  // the barrier.
  auto tile_start = [&](int jt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (need_ex(jt)) rotate_own(jt & 1);
    __syncthreads();
    if (jt + 1 < ntile) issue_tile(jt + 1, (jt + 1) & 1);
  };
  // tiles 1 .. jp - 1 are all latent for every position of the wave and run
  // the mask-free loop (tile 0 sets the running maxima first)
  const int jp = wave_on ? min(ntile, max(0, (qw0 - W) / KT)) : 0;
  // q' = R_i q log2(e)/sqrt(d_h) as the score MFMA's B operand: lane (col,
  // grp) holds dims 32 ks + 8 grp .. + 7 of position i = qw0 + 16 qb + col,
  // and the rotation partner of a first-half dim d (ks < KS/2) is d + d_h/2,
  // in the same lane's fragment ks + KS/2.  The angles come from the (cos,
  // sin) table by angle addition, R_i = R_(i - col) R_col: row i - col is
  // shared by the 16 lanes of a query block and rows 0..15 by every wave, so
  // a workgroup reads a few KiB of the table instead of a row per position.
  // Rows past the sequence are clamped to its last token (those positions
  // write nothing).  The q rows and table entries are requested first, then
  // tile 0's copies, and the rotation runs while the copies travel: the
  // compiler's waits for the q loads do not wait for the younger copies.
  // Everything has landed before the tile loop, whose waits then count only
  // tile copies.
  bf16x8 raw[QB][KS];
  float4 csa[QB][KS / 2][4], csb[KS / 2][4];   // (cos, sin) of frequencies 32 ks + 8 grp + 2 c2, + 1
  {
    const float4* rt = static_cast<const float4*>(p.rtab);   // [n_pad][d_h/2] (cos, sin) pairs
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) csb[ks][c2] = rt[(col * (DH / 2) + 32 * ks + 8 * grp) / 2 + c2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int i = qw0 + 16 * qb + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        raw[qb][ks] = *reinterpret_cast<const bf16x8*>(qx + (int64_t)min(i, n - 1) * trow + 32 * ks + 8 * grp);
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2)
          csa[qb][ks][c2] = rt[((int64_t)(qw0 + 16 * qb) * (DH / 2) + 32 * ks + 8 * grp) / 2 + c2];
    }
  }
  // this wave's offset rows (j % 16 of its rows: RPC rows from (wave RPC) % 16)
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
    copy_to_lds(static_cast<const char*>(p.rtab) +
                    (int64_t)((wave * RPC) % 16 + k2 * (256 / DH) + lane / (DH / 4)) * (4 * DH) + 16 * (lane % (DH / 4)),
                &tb_s[wave][k2 * 1024]);
  issue_tile(0, 0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 ta = csa[qb][ks][e / 2], tb = csb[ks][e / 2];
        const float ca = (e & 1) ? ta.z : ta.x, sa = (e & 1) ? ta.w : ta.y;
        const float cb = (e & 1) ? tb.z : tb.x, sb = (e & 1) ? tb.w : tb.y;
        const float c = ca * cb - sa * sb, sn = sa * cb + ca * sb;
        const float x0 = (float)raw[qb][ks][e], x1 = (float)raw[qb][ks + KS / 2][e];
        qf[qb][ks][e] = static_cast<bf16>((x0 * c - x1 * sn) * p.scale);
        qf[qb][ks + KS / 2][e] = static_cast<bf16>((x0 * sn + x1 * c) * p.scale);
      }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  int jt = 0;
  if (ntile > 0) {
    tile_start(0);
    if (wave_on) compute(0, 0);
    jt = 1;
  }
  for (; jt < jp; ++jt) {
    tile_start(jt);
    fast_tile(jt & 1);
  }
  for (; jt < ntile; ++jt) {
    tile_start(jt);
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
    lt += accl[qb][0];
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
  hipLaunchKernelGGL((k_rope_table<DH>), dim3((p.n_pad * (DH / 2) + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
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
  // (the tiled GEMM, not the vendor's: with the vendor GEMM the rebuild took
  // 41 against 51 us, but the attention that reads its output 228 against
  // 210 us per call)
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
