// bf16 decode kernels around the latent scan, shaped for gfx950:
//   k_qmap_mfma     q~ = s R~_i A_t^T q for a block of 16 sequences and 128
//                   latent columns per workgroup (its waves split the d_h
//                   contraction), on the matrix cores; the latent rotation
//                   pairs (f, f + d_h/2) land one lane swap apart, so
//                   R~_i is applied in registers ("Hybrid Latent Attention"
//                   summary, "Latent Reader" Eq. 3, "Rotary Embedding
//                   Alignment")
//   k_window_fast   the exact tokens i-W <= j <= i of Eq. 4 for one sequence
//                   and one slice of the window: all heads at once, each
//                   thread owning 8 dims of one head (16-byte loads of the
//                   contiguous [H][d_h] ring rows), per-head online softmax
//   k_combine_mfma  merge of the latent and window partials of 16 sequences
//                   and one head, then o = (B_t^T O_latent + O_window) / l
//                   for 32 of the head's output dims per workgroup, with the
//                   B_t^T product on the bf16 matrix cores
#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// ------------------------------------------------------------------ q map
// grid (H, ceil(r_k / 128), ceil(B / 16)); the workgroup produces the 128
// latent columns n0 = 128 blockIdx.y .. n0 + 127 of q~ for 16 sequences, its
// four waves splitting the contraction over the head dims (wave w takes the
// 32-wide k steps w, w + 4, ..): each wave reads a quarter of the
// workgroup's 32 KiB slab of A^(h), and the four partial products are summed
// through LDS.  q~[b][n] = sum_e q[b][e] A[e][n] runs on
// v_mfma_f32_16x16x32_bf16, which wants 8 consecutive e per lane while rows
// of A^(h) are contiguous along n: each lane loads 8 rows x 8 columns
// (columns n0 + 8c .. n0 + 8c + 7, c = lane % 16) and regroups them in
// registers, so product j yields the columns {n0 + 8c + j}.  With rotary the
// partner column n +- d_h/2 of a pair then sits in lane c ^ (d_h / 16) of the
// same product, one lane swap away; after the sum wave w holds rows
// 4 grp + w of the block, so the swap stays inside the wave.
// Nothing waits for the operand loads before the products: the sequences'
// rotation table is built while they are in flight (wave w takes sequences
// w, w + 4, .. with their positions as scalar loads, lane f frequency f),
// and q' = s R_i q for the window (first column block only) is formed after
// the products from q values requested at entry.
template <int DH>
__global__ __launch_bounds__(kThreads) void k_qmap_mfma(DecodeParams p, int want_qlat) {
  constexpr int KS = DH / 32;
  constexpr int KW = (KS + 3) / 4;          // k steps per wave
  constexpr int NF = DH / 2;                // rotary frequency pairs
  __shared__ __attribute__((aligned(16))) float csn[16][NF][2];   // (cos, sin)
  __shared__ float red[4][8][4][64];        // per-wave partial products [wave][j][r][lane]
  const int h = blockIdx.x, b0 = blockIdx.z * 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int H = p.H, rk = p.rk;
  const bool rope = p.rope_base != 0.f;
  const bf16* q = static_cast<const bf16*>(p.q);
  const int n0 = blockIdx.y * 128;
  const bool active = want_qlat && n0 < rk;   // uniform over the workgroup
  const int ncol = n0 + 8 * col;
  const bool do_qhead = blockIdx.y == 0 && p.need_qhead;
  const int fl = min(lane, NF - 1);

  // q of sequences wave + 4 k at dims fl and fl + NF (for q')
  float qa[4], qb[4];
  if (do_qhead) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16* qr = q + ((int64_t)min(b0 + wave + 4 * k, p.B - 1) * H + h) * DH;
      qa[k] = to_f(qr[fl]);
      qb[k] = to_f(qr[fl + NF]);
    }
  }
  // A^(h) rows e = 32 st + 8 grp + i of this wave's k steps, columns ncol ..
  // ncol + 7 (clamped into the row; lanes past r_k store nothing)
  bf16x8 araw[KW][8];
  bf16x8 aq[KW];
  const int brow = b0 + col;
  if (active) {
    const bf16* Ah = static_cast<const bf16*>(p.A) + (int64_t)h * DH * rk + min(ncol, rk - 8);
#pragma unroll
    for (int u = 0; u < KW; ++u) {
      const int st = wave + 4 * u;
      if (st < KS) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          araw[u][i] = *reinterpret_cast<const bf16x8*>(Ah + (int64_t)(32 * st + 8 * grp + i) * rk);
        // A operand: q row of sequence b0 + col (rows past the batch read the
        // last sequence and are zeroed), dims 32 st + 8 grp ..
        aq[u] = *reinterpret_cast<const bf16x8*>(q + ((int64_t)min(brow, p.B - 1) * H + h) * DH + st * 32 + grp * 8);
        if (brow >= p.B) {
#pragma unroll
          for (int k = 0; k < 8; ++k) aq[u][k] = static_cast<bf16>(0.f);
        }
      }
    }
  }
  if (rope) {
    const double th = rope_theta(p.rope_base, DH, fl);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int bl = wave + 4 * k;
      const int pos = p.pos[min(b0 + bl, p.B - 1)];
      float c, sn;
      rope_cs_theta(th, pos, c, sn);
      if (lane < NF) {
        csn[bl][lane][0] = c;
        csn[bl][lane][1] = sn;
      }
    }
  }

  if (active) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KW; ++u) {
      if (wave + 4 * u < KS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bf16x8 bj;
#pragma unroll
          for (int i = 0; i < 8; ++i) bj[i] = araw[u][i][j];
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[u], bj, acc[j], 0, 0, 0);
        }
      }
    }
    // lane: C[b0 + 4 grp + r][ncol + j] of this wave's k steps
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][j][r][lane] = acc[j][r];
  }
  __syncthreads();
  if (active) {
    // wave w: row r = w of every lane's 4 x 8 block, summed over the waves
    const int r = wave;
    float mine[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      mine[j] = (red[0][j][r][lane] + red[1][j][r][lane]) + (red[2][j][r][lane] + red[3][j][r][lane]);
    bf16* ql = static_cast<bf16*>(p.qlat);
    const bool lo_half = (8 * col) % DH < DH / 2;   // n0 is a multiple of d_h
    const int f0 = (8 * col) % (DH / 2);
    const int bl = 4 * grp + r, bb = b0 + bl;
    float v[8];
    if (rope) {
      const float4* cs = reinterpret_cast<const float4*>(&csn[bl][f0][0]);
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const float4 t = cs[j2];   // (cos, sin) of frequencies f0 + 2 j2, f0 + 2 j2 + 1
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * j2 + u;
          const float c = u ? t.z : t.x, sn = u ? t.w : t.y;
          const float other = __shfl_xor(mine[j], DH / 16);
          v[j] = lo_half ? (mine[j] * c - other * sn) : (other * sn + mine[j] * c);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = mine[j];
    }
    if (bb < p.B && ncol < rk) {
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = static_cast<bf16>(v[j] * p.scale);
      *reinterpret_cast<bf16x8*>(ql + ((int64_t)bb * H + h) * rk + ncol) = o;
    }
  }
  // q' = s R_i q (head space, fp32) when a later kernel reads it
  if (do_qhead) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int bl = wave + 4 * k, bb = b0 + bl;
      if (bb < p.B && lane < NF) {
        const float c = rope ? csn[bl][lane][0] : 1.f, sn = rope ? csn[bl][lane][1] : 0.f;
        float* qh = p.qhead + ((int64_t)bb * H + h) * DH;
        qh[lane] = p.scale * (qa[k] * c - qb[k] * sn);
        qh[lane + NF] = p.scale * (qa[k] * sn + qb[k] * c);
      }
    }
  }
}

// ------------------------------------------------------------------ window
// grid (B, WS); thread (h = tid / (DH/8), c = tid % (DH/8)) owns dims 8c..8c+7
template <int DH>
__global__ __launch_bounds__(kThreads) void k_window_fast(DecodeParams p) {
  constexpr int TPH = DH / 8;
  __shared__ double theta[DH / 2];
  const int b = blockIdx.x, ws = blockIdx.y, tid = threadIdx.x;
  if (p.rope_base != 0.f && tid < DH / 2) theta[tid] = rope_theta(p.rope_base, DH, tid);
  __syncthreads();
  const int H = p.H, W = p.W, WS = p.WS;
  const int h = tid / TPH, c = tid % TPH;
  const bool active = h < H;
  const int hh = active ? h : 0;
  const int i = p.pos[b];
  const int j0 = max(0, i - W);
  const int nw = i - j0;                       // ring tokens; token nw is the current one
  const int t0 = ws * p.tw, t1 = min(t0 + p.tw, nw + 1);
  float qf[8];
  if (p.need_qhead) {
    const float* qh = p.qhead + ((int64_t)b * H + hh) * DH + 8 * c;
#pragma unroll
    for (int k = 0; k < 8; ++k) qf[k] = qh[k];
  } else {
    // q' = s R_i q for this thread's 8 dims (partner dims are d +- DH/2)
    const bf16* qr = static_cast<const bf16*>(p.q) + ((int64_t)b * H + hh) * DH;
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qr + 8 * c);
    const int pc = (8 * c < DH / 2) ? 8 * c + DH / 2 : 8 * c - DH / 2;
    const bf16x8 qp = *reinterpret_cast<const bf16x8*>(qr + pc);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = 8 * c + k;
      const int f = d < DH / 2 ? d : d - DH / 2;
      float cs = 1.f, sn = 0.f;
      if (p.rope_base != 0.f) rope_cs_theta(theta[f], i, cs, sn);
      const float r = d < DH / 2 ? to_f(qv[k]) * cs - to_f(qp[k]) * sn : to_f(qp[k]) * sn + to_f(qv[k]) * cs;
      qf[k] = p.scale * r;
    }
  }
  const bf16* ring_k = static_cast<const bf16*>(p.ring_k);
  const bf16* ring_v = static_cast<const bf16*>(p.ring_v);
  const int64_t rs = (int64_t)H * DH;          // elements per ring slot
  const int64_t base = (int64_t)b * (W + 1) * rs + (int64_t)hh * DH + 8 * c;

  // current token: rotated key R_i k_cur and v_cur (only the slice holding it)
  float kself[8], vself[8];
  const bool has_self = t0 <= nw && nw < t1;
  if (has_self) {
    const bf16* kc = static_cast<const bf16*>(p.k_cur) + ((int64_t)b * H + hh) * DH;
    const bf16* vc = static_cast<const bf16*>(p.v_cur) + ((int64_t)b * H + hh) * DH;
    const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kc + 8 * c);
    const int pc = (8 * c < DH / 2) ? 8 * c + DH / 2 : 8 * c - DH / 2;
    const bf16x8 kp = *reinterpret_cast<const bf16x8*>(kc + pc);
    const bf16x8 vv = *reinterpret_cast<const bf16x8*>(vc + 8 * c);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = 8 * c + k;
      float cs = 1.f, sn = 0.f;
      const int f = d < DH / 2 ? d : d - DH / 2;
      if (p.rope_base != 0.f) rope_cs_theta(theta[f], i, cs, sn);
      kself[k] = d < DH / 2 ? to_f(kv[k]) * cs - to_f(kp[k]) * sn : to_f(kp[k]) * sn + to_f(kv[k]) * cs;
      vself[k] = to_f(vv[k]);
    }
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  constexpr int U = 8;
  for (int tb = t0; tb < t1; tb += U) {
    bf16x8 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u;
      if (t < t1 && t < nw) {
        const int slot = (j0 + t) % (W + 1);
        kr[u] = *reinterpret_cast<const bf16x8*>(ring_k + base + slot * rs);
        vr[u] = *reinterpret_cast<const bf16x8*>(ring_v + base + slot * rs);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      float kk[8], vv[8];
      if (t < nw) {
#pragma unroll
        for (int k = 0; k < 8; ++k) { kk[k] = to_f(kr[u][k]); vv[k] = to_f(vr[u][k]); }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) { kk[k] = kself[k]; vv[k] = vself[k]; }
      }
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) s += qf[k] * kk[k];
      s = group_sum(s, TPH);   // the TPH lanes of this head
      const float mn = fmaxf(m, s);
      const float alpha = exp2_diff(m, mn);
      const float pw = fast_exp2(s - mn);
      l = l * alpha + pw;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = o[k] * alpha + pw * vv[k];
      m = mn;
    }
  }
  if (active) {
    const int64_t row = ((int64_t)b * WS + ws) * H + h;
    if (c == 0) {
      p.win_ml[row * 2 + 0] = m;
      p.win_ml[row * 2 + 1] = l;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) p.win_o[row * DH + 8 * c + k] = o[k];
    if (has_self) {
      // ring append: slot i mod (W+1) held token i-W-1, read by no slice
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
}

// ------------------------------------------------------------------ combine
// grid (H, ceil(B / 16), 4); 4 waves; out[b][h] for 16 sequences and the 32
// output dims 32 blockIdx.z .. + 31 of d_h = 128 (the four workgroups of a
// (head, sequence block) each read a quarter of B_t; they sit 128 workgroup
// ids apart, on one XCD, and share its L2 for the partials they all merge).
// The B_t^T product runs on v_mfma_f32_16x16x32_bf16.  The value decoder is
// stored as B_t^T [d_h][r_v] (rows contiguous along the latent axis), so each
// B-operand fragment (8 consecutive latent dims of one output column) is one
// 16-byte load.  Wave w takes the 32-wide k steps w, w+4, ...; all its loads
// are issued at entry so their latency overlaps the merge.  The fp32 latent
// sums enter as bf16 hi + lo parts (two products), which keeps the product at
// fp32-level accuracy.  The four waves' partial results are summed through LDS
// and written as 16-byte rows.  With all 16 sequences present (large
// batches, few splits) the first two splits' latent sums and the first two
// window slices are requested at entry as well, so the merge barrier waits
// for one memory round trip instead of three.  PART: some workgroup may hold
// fewer than 16 sequences (the batch is not a multiple of 16); the path for
// those is compiled only then, so that it cannot change the register
// allocation of the full-workgroup path.
template <int RV, bool PART>
__global__ __launch_bounds__(kThreads) void k_combine_mfma(DecodeParams p) {
  constexpr int DH = 128;
  constexpr int NT = 2;                    // output column tiles of this workgroup
  constexpr int KS = RV / 32;              // k steps
  constexpr int KW = (KS + 3) / 4;         // k steps per wave
  __shared__ float ob[16][RV + 1];         // latent-space sums
  __shared__ float wo[16][DH];             // window sums
  __shared__ float wl[16];                 // 1 / l
  __shared__ __attribute__((aligned(16))) float red[4][16][16 * NT + 4];   // per-wave products
  const int H = p.H, S = p.S, WS = p.WS;
  const int h = blockIdx.x, b0 = blockIdx.y * 16, tid = threadIdx.x;
  const int e0 = 16 * NT * blockIdx.z;     // first output dim of this workgroup
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const bf16* Bh = static_cast<const bf16*>(p.Bm) + (int64_t)h * DH * RV;   // [DH][RV]
  bf16x8 bfr[KW][NT];
#pragma unroll
  for (int u = 0; u < KW; ++u) {
    const int st = wave + 4 * u;
    if (st < KS) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bfr[u][nt] = *reinterpret_cast<const bf16x8*>(Bh + (int64_t)(e0 + 16 * nt + col) * RV + 32 * st + 8 * grp);
    }
  }

  constexpr int C4 = RV / 4;               // float4 columns of a latent sum
  constexpr int PER = (C4 + 15) / 16;
  const bool full16 = !PART || p.B - b0 >= 16;
  // full16: thread -> (sequence fbl, float4 columns fk4, fk4 + 16, .., and 8
  // window dims from fe8)
  const int fbl = tid / 16, fk4 = tid % 16, fe8 = (tid % 16) * 8, fb = b0 + fbl;
  const bool wmine = (fe8 >> 5) == (int)blockIdx.z;   // window dims this workgroup outputs
  f32x4 pv[2][PER], wv[2][2];
  if (full16) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const float4* row = reinterpret_cast<const float4*>(p.part_o + (((int64_t)fb * S + min(ss, S - 1)) * H + h) * p.Dp);
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int cc = fk4 + 16 * u;
        if (cc < C4) {
          const float4 t = row[cc];
          pv[ss][u] = f32x4{t.x, t.y, t.z, t.w};
        } else {
          pv[ss][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      if (WS > 0 && wmine) {
        const float4* src = reinterpret_cast<const float4*>(
            p.win_o + (((int64_t)fb * WS + min(ss, WS - 1)) * H + h) * DH + fe8);
        const float4 a = src[0], c = src[1];
        wv[ss][0] = f32x4{a.x, a.y, a.z, a.w};
        wv[ss][1] = f32x4{c.x, c.y, c.z, c.w};
      } else {
        wv[ss][0] = wv[ss][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // (m, l) of every split and window slice of the 16 sequences: one load per
  // thread, all in flight together, then the per-sequence softmax merge
  __shared__ float pm[16][kCombineMaxParts], pl[16][kCombineMaxParts];
  {
    const int NP = S + WS;
    constexpr int MU = (16 * kCombineMaxParts + kThreads - 1) / kThreads;
    float2 ml[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int x = tid + u * kThreads, bl = x / NP, j = x % NP, b = b0 + bl;
      ml[u] = make_float2(-INFINITY, 0.f);
      if (x < 16 * NP && b < p.B) {
        const float* src = (j < S) ? p.part_ml + (((int64_t)b * S + j) * H + h) * 2
                                   : p.win_ml + (((int64_t)b * WS + (j - S)) * H + h) * 2;
        ml[u] = *reinterpret_cast<const float2*>(src);
      }
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int x = tid + u * kThreads, bl = x / NP, j = x % NP;
      if (x < 16 * NP) {
        pm[bl][j] = ml[u].x;
        pl[bl][j] = ml[u].y;
      }
    }
  }
  __syncthreads();
  {
    // the 16 lanes of a DPP row merge one sequence's parts: parts j = c,
    // c + 16, .. per lane, then row reductions
    const int NP = S + WS;
    const int bl = tid / 16, c = tid % 16;
    float M = -INFINITY;
    for (int j = c; j < NP; j += 16) M = fmaxf(M, pm[bl][j]);
    M = row_max16(M);
    float l = 0.f;
    for (int j = c; j < NP; j += 16) {
      const float w = exp2_diff(pm[bl][j], M);
      pm[bl][j] = w;         // from here on: merge weight of split / slice j
      l += w * pl[bl][j];
    }
    l = row_sum16(l);
    if (c == 0) wl[bl] = (b0 + bl < p.B) ? 1.f / l : 0.f;
  }
  __syncthreads();
  // A workgroup with all 16 sequences gives each thread one sequence; with
  // fewer (small batches, where the splits are many) the threads share the
  // splits of one sequence at a time and add their sums through LDS.
  const int nb = min(16, p.B - b0);
  float* rbuf = &red[0][0][0];
  if (!full16) {
    constexpr int SG = kThreads / C4;     // split groups
    const int c4 = tid % C4, sg = tid / C4;
    for (int bl = 0; bl < 16; ++bl) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      if (bl < nb) {
        // 16 splits' rows requested together (the address is clamped to the
        // last split, whose weight is then replaced by 0), so a sequence's
        // many splits cost a few memory round trips, not one each
        const int b = b0 + bl;
        const float* base = p.part_o + ((int64_t)b * S * H + h) * p.Dp + 4 * c4;
        const int64_t sstride = (int64_t)H * p.Dp;
        constexpr int UL = 16;
        for (int s0 = sg; s0 < S; s0 += UL * SG) {
          float4 t[UL];
#pragma unroll
          for (int u = 0; u < UL; ++u)
            t[u] = *reinterpret_cast<const float4*>(base + min(s0 + u * SG, S - 1) * sstride);
#pragma unroll
          for (int u = 0; u < UL; ++u) {
            const float w = (s0 + u * SG < S) ? pm[bl][s0 + u * SG] : 0.f;
            sum += w * f32x4{t[u].x, t[u].y, t[u].z, t[u].w};
          }
        }
      }
      reinterpret_cast<f32x4*>(rbuf)[tid] = sum;
      __syncthreads();
      if (tid < C4) {
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < SG; ++g) tot += reinterpret_cast<const f32x4*>(rbuf)[g * C4 + tid];
#pragma unroll
        for (int k = 0; k < 4; ++k) ob[bl][4 * tid + k] = tot[k];
      }
      __syncthreads();
      if (bl + 1 >= nb) {   // the remaining rows are zero
        for (int x = tid; x < (15 - bl) * RV; x += kThreads) ob[bl + 1 + x / RV][x % RV] = 0.f;
        break;
      }
    }
    // window sums: thread -> (8 consecutive dims, slice group of 16)
    const int e8 = (tid % 16) * 8, wg = tid / 16;
    for (int bl = 0; bl < nb; ++bl) {
      const int b = b0 + bl;
      f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
      constexpr int WL = 4;   // slices of this thread requested together (clamped, weight 0)
      for (int sl0 = wg; sl0 < WS; sl0 += WL * (kThreads / 16)) {
        float4 a[WL], c[WL];
#pragma unroll
        for (int u = 0; u < WL; ++u) {
          const int sl = min(sl0 + u * (kThreads / 16), WS - 1);
          const float4* src = reinterpret_cast<const float4*>(p.win_o + (((int64_t)b * WS + sl) * H + h) * DH + e8);
          a[u] = src[0];
          c[u] = src[1];
        }
#pragma unroll
        for (int u = 0; u < WL; ++u) {
          const int sl = sl0 + u * (kThreads / 16);
          const float w = sl < WS ? pm[bl][S + sl] : 0.f;
          w0 += w * f32x4{a[u].x, a[u].y, a[u].z, a[u].w};
          w1 += w * f32x4{c[u].x, c[u].y, c[u].z, c[u].w};
        }
      }
      reinterpret_cast<f32x4*>(rbuf)[2 * tid] = w0;
      reinterpret_cast<f32x4*>(rbuf)[2 * tid + 1] = w1;
      __syncthreads();
      if (tid < 16) {
        f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
        for (int g = 0; g < kThreads / 16; ++g) {
          t0 += reinterpret_cast<const f32x4*>(rbuf)[2 * (16 * g + tid)];
          t1 += reinterpret_cast<const f32x4*>(rbuf)[2 * (16 * g + tid) + 1];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wo[bl][e8 + k] = t0[k];
          wo[bl][e8 + 4 + k] = t1[k];
        }
      }
      __syncthreads();
    }
  } else {
    // thread -> (sequence fbl, float4 columns fk4, fk4 + 16, ...): splits 0, 1
    // from the registers filled at entry, the rest four at a time
    f32x4 sum[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) sum[u] = pm[fbl][0] * pv[0][u];
    if (S > 1) {
#pragma unroll
      for (int u = 0; u < PER; ++u) sum[u] += pm[fbl][1] * pv[1][u];
    }
    for (int s0 = 2; s0 < S; s0 += 4) {
      f32x4 v[4][PER];
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const int s = s0 + ss;
        const float4* row = reinterpret_cast<const float4*>(
            p.part_o + (((int64_t)fb * S + min(s, S - 1)) * H + h) * p.Dp);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int cc = fk4 + 16 * u;
          if (s < S && cc < C4) {
            const float4 t = row[cc];
            v[ss][u] = f32x4{t.x, t.y, t.z, t.w};
          } else {
            v[ss][u] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const float w = (s0 + ss < S) ? pm[fbl][s0 + ss] : 0.f;
#pragma unroll
        for (int u = 0; u < PER; ++u) sum[u] += w * v[ss][u];
      }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int cc = fk4 + 16 * u;
      if (cc < C4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) ob[fbl][4 * cc + k] = sum[u][k];
      }
    }
    // window sums: slices 0, 1 from the entry registers, the rest four at a time
    f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      if (ss < WS) {
        const float w = pm[fbl][S + ss];
        w0 += w * wv[ss][0];
        w1 += w * wv[ss][1];
      }
    }
    for (int s0 = 2; s0 < (wmine ? WS : 0); s0 += 4) {
      f32x4 v[4][2];
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const int sl = min(s0 + ss, WS - 1);
        const float4* src = reinterpret_cast<const float4*>(
            p.win_o + (((int64_t)fb * WS + sl) * H + h) * DH + fe8);
        const float4 a = src[0], c = src[1];
        v[ss][0] = f32x4{a.x, a.y, a.z, a.w};
        v[ss][1] = f32x4{c.x, c.y, c.z, c.w};
      }
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const float w = (s0 + ss < WS) ? pm[fbl][S + s0 + ss] : 0.f;
        w0 += w * v[ss][0];
        w1 += w * v[ss][1];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wo[fbl][fe8 + k] = w0[k];
      wo[fbl][fe8 + 4 + k] = w1[k];
    }
  }
  __syncthreads();
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KW; ++u) {
    const int st = wave + 4 * u;
    if (st < KS) {
      // A operand: row b = col of the latent sums, k = 32 st + 8 grp + i
      bf16x8 ahi, alo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = ob[col][32 * st + 8 * grp + i];
        const bf16 hi = static_cast<bf16>(x);
        ahi[i] = hi;
        alo[i] = static_cast<bf16>(x - static_cast<float>(hi));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfr[u][nt], acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr[u][nt], acc[nt], 0, 0, 0);
      }
    }
  }
  // lane holds C[b = 4 grp + r][e = e0 + 16 nt + col]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * grp + r][16 * nt + col] = acc[nt][r];
  __syncthreads();
  if (tid < 16 * (16 * NT / 8)) {
    const int bl = tid / (2 * NT), e8 = (tid % (2 * NT)) * 8, b = b0 + bl;
    if (b < p.B) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = wo[bl][e0 + e8 + k];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 x0 = *reinterpret_cast<const float4*>(&red[w][bl][e8]);
        const float4 x1 = *reinterpret_cast<const float4*>(&red[w][bl][e8 + 4]);
        v[0] += x0.x; v[1] += x0.y; v[2] += x0.z; v[3] += x0.w;
        v[4] += x1.x; v[5] += x1.y; v[6] += x1.z; v[7] += x1.w;
      }
      bf16x8 o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = static_cast<bf16>(v[k] * wl[bl]);
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + ((int64_t)b * H + h) * DH + e0 + e8) = o;
    }
  }
}

template <int DH>
hipError_t qmap_launch(const DecodeParams& p, bool want, hipStream_t s) {
  const dim3 grid(p.H, want ? (p.rk + 127) / 128 : 1, (p.B + 15) / 16);
  hipLaunchKernelGGL((k_qmap_mfma<DH>), grid, dim3(kThreads), 0, s, p, want ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

bool qmap_mfma_supports(const DecodeParams& p) {
  if (!p.bf16) return false;
  if (p.dh != 64 && p.dh != 128) return false;
  if (p.rope_base != 0.f) return p.rk % p.dh == 0;
  return p.rk % 8 == 0;
}

hipError_t launch_qmap_mfma(const DecodeParams& p, bool want_qlat, hipStream_t s) {
  if (!qmap_mfma_supports(p)) return hipErrorNotSupported;
  return p.dh == 128 ? qmap_launch<128>(p, want_qlat, s) : qmap_launch<64>(p, want_qlat, s);
}

bool window_fast_supports(const DecodeParams& p) {
  return p.bf16 && (p.dh == 64 || p.dh == 128) && p.H * (p.dh / 8) <= kThreads;
}

hipError_t launch_window_fast(const DecodeParams& p, hipStream_t s) {
  if (!window_fast_supports(p)) return hipErrorNotSupported;
  const dim3 grid(p.B, p.WS);
  if (p.dh == 128)
    hipLaunchKernelGGL(k_window_fast<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_window_fast<64>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

bool combine_mfma_supports(const DecodeParams& p) {
  if (!p.bf16 || p.mode != kAbsorbed || p.dh != 128 || p.S + p.WS > kCombineMaxParts) return false;
  return p.rv == 32 || p.rv == 64 || p.rv == 128 || p.rv == 256 || p.rv == 512;
}

hipError_t launch_combine_mfma(const DecodeParams& p, hipStream_t s) {
  if (!combine_mfma_supports(p)) return hipErrorNotSupported;
  const dim3 grid(p.H, (p.B + 15) / 16, 4);
  if (p.B % 16 != 0) {
    switch (p.rv) {
      case 32: hipLaunchKernelGGL((k_combine_mfma<32, true>), grid, dim3(kThreads), 0, s, p); break;
      case 64: hipLaunchKernelGGL((k_combine_mfma<64, true>), grid, dim3(kThreads), 0, s, p); break;
      case 128: hipLaunchKernelGGL((k_combine_mfma<128, true>), grid, dim3(kThreads), 0, s, p); break;
      case 256: hipLaunchKernelGGL((k_combine_mfma<256, true>), grid, dim3(kThreads), 0, s, p); break;
      default: hipLaunchKernelGGL((k_combine_mfma<512, true>), grid, dim3(kThreads), 0, s, p); break;
    }
  } else {
    switch (p.rv) {
      case 32: hipLaunchKernelGGL((k_combine_mfma<32, false>), grid, dim3(kThreads), 0, s, p); break;
      case 64: hipLaunchKernelGGL((k_combine_mfma<64, false>), grid, dim3(kThreads), 0, s, p); break;
      case 128: hipLaunchKernelGGL((k_combine_mfma<128, false>), grid, dim3(kThreads), 0, s, p); break;
      case 256: hipLaunchKernelGGL((k_combine_mfma<256, false>), grid, dim3(kThreads), 0, s, p); break;
      default: hipLaunchKernelGGL((k_combine_mfma<512, false>), grid, dim3(kThreads), 0, s, p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace lla
