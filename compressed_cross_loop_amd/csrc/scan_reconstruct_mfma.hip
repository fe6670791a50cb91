// Reconstruct-on-read latent scan for per-head Looped Latent Attention on the
// gfx950 matrix cores ("Looped Latent Attention" abstracts: the codec keeps
// only latents and rebuilds a loop's keys and values when attention reads them).
//
// One workgroup per (context split, sequence, head); each head has its own
// latent group, and the four waves take interleaved 16-token tiles of the
// split (wave w: tiles w, w + 4, ..), so a workgroup streams one contiguous
// run of its group's tiles per page.  Per 16-token tile the wave rebuilds,
// for the head, the transposed keys and values
//   K^T [d_h x 16 tok] = A_t [d_h x r] . S^K^T [r x 16]   (v_mfma_f32_16x16x32_bf16)
//   V^T [d_h x 16 tok] = B_t^T [d_h x r] . S^V^T [r x 16]
// so that every lane ends with 4 dims of each 16-dim block for ONE token
// (token = lane % 16).  Then, per lane and without cross-lane traffic except
// one 4-lane reduction of the score:
//   score  q' . k^_tok   (the lane's 4 NT partial dims, summed over the 4 lane
//          groups holding the same token)
//   p      2^(score - m), running maximum m moved lazily (only when a tile's
//          maximum exceeds it by more than 2^8), so rescaling is rare
//   o      += p v^_tok for the lane's dims; o and the weight sum stay per
//          token lane and are summed over the 16 token lanes once per split;
//          the four waves' (m, l, o) are then merged in LDS (same-max
//          rescale, fixed order) into the split's one partial.
// Both decoders are stored [d_h][r] (rows contiguous along the latent axis),
// i.e. directly in A-operand layout; they are held in registers for the whole
// scan.  Key rows are token-major in the store: one 16-byte load per lane is
// the B operand.  The tile's value block is dimension-major (for the absorbed
// read); it is loaded into registers like the keys (16 contiguous bytes per
// lane and KiB), written to a wave-private KiB of LDS when the tile is
// consumed and read back as token-major B operands with the gfx950
// transposing read ds_read_b64_tr_b16 (inside each 16-lane group lane i
// receives element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4).
// A wave's LDS operations run in order, so one slot per wave needs no
// barrier.  Several tiles are in flight per wave, all in registers; the page
// ids of the split are staged in LDS first.
//
// The whole call is this kernel and the split merge: each wave rotates and
// scales its head's query itself (q' = s R_i q at the lane's dims; the
// partner of dim d is d +- d_h/2, i.e. block nt +- NT/2 of the same lane),
// and split s also takes slice s of the exact tokens of Eq. 4 (ring tokens
// i-W .. i-1 and the current one, 16 per step in the same token-per-lane
// layout, read straight from the ring rows, the steps dealt to the waves in
// turn) into the same running softmax; the lanes holding the current token
// append R_i k_cur, v_cur to the ring.
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPageTab = 4096;            // page ids of a split, staged in LDS
constexpr float kLazy = 8.f;              // running-max slack (exp2 units)

template <typename F, int... U>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ short bf16_bits(float x) {
  return __builtin_bit_cast(short, static_cast<bf16>(x));
}

// 16-byte chunk slot of a value copy: bit 3 ^= bit 4, so that the two
// 16-lane groups a transposing read serves together hit different banks
__device__ __forceinline__ int val_slot(int ch) { return ch ^ (((ch >> 4) & 1) << 3); }

template <int R, int DH>
__global__ __launch_bounds__(kThreads, (R == 32 || DH == 64) ? 2 : 1) void k_scan_reconstruct_mfma(DecodeParams p) {
  constexpr int NT = DH / 16;            // 16-dim blocks of d_h
  constexpr int KS = R / 32;             // K steps over the latent width = KiB of values per tile
  constexpr int kPF = 3;                 // tiles in flight per wave
  __shared__ int32_t ptab[kPageTab];
  __shared__ __attribute__((aligned(16))) unsigned char vlds[kWaves][KS * 1024];
  __shared__ float csn[DH / 2][2];       // (cos, sin) of i theta_f
  __shared__ float mrg_o[kWaves][DH];    // per-wave (m, l, o) for the merge
  __shared__ float mrg_ml[kWaves][2];
  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.z;
  const int G = p.G, P = p.P, Rt = 2 * R;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;
  // page ids of tokens t0 .. t1-1 (never more than max_pages <= kPageTab):
  // a block-table read in the loop would be a vector load, and waiting for it
  // (load counts complete in issue order) would drain the tiles in flight
  const int pfirst = t0 / P;
  const int npg = t1 > t0 ? (t1 - 1) / P - pfirst + 1 : 0;
  for (int x = tid; x < npg; x += kThreads) ptab[x] = p.bt[(int64_t)b * p.max_pages + pfirst + x];
  const bool rope = p.rope_base != 0.f;
  if (rope && tid < DH / 2) {
    float c, sn;
    rope_cs(p.rope_base, DH, tid, i, c, sn);
    csn[tid][0] = c;
    csn[tid][1] = sn;
  }
  __syncthreads();
  const int g = h / p.hpg;
  // R_i x at this lane's dims 16 nt + 4 grp + r, from x at the same dims
  auto rotate = [&](f32x4 (&x)[NT]) {
    if (!rope) return;
    f32x4 y[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = (16 * nt + 4 * grp + r) % (DH / 2);
        const float c = csn[f][0], sn = csn[f][1];
        const float other = x[(nt + NT / 2) % NT][r];
        y[nt][r] = nt < NT / 2 ? x[nt][r] * c - other * sn : other * sn + x[nt][r] * c;
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) x[nt] = y[nt];
  };
  // 4 consecutive bf16 of a head row at the lane's dims of block nt (a bf16
  // is the upper half of the fp32 with the same value)
  auto load4 = [&](const bf16* row, int nt) {
    const uint2 u = *reinterpret_cast<const uint2*>(row + 16 * nt + 4 * grp);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  };

  // decoders of this head in A-operand layout (lane: row 16 nt + col, latent
  // dims 32 st + 8 grp ..)
  const bf16* Ah = static_cast<const bf16*>(p.A) + (int64_t)h * DH * R;   // [DH][R]
  const bf16* Bh = static_cast<const bf16*>(p.Bm) + (int64_t)h * DH * R;  // B_t^T: [DH][R]
  bf16x8 af[NT][KS], bfr[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      af[nt][st] = *reinterpret_cast<const bf16x8*>(Ah + (int64_t)(16 * nt + col) * R + 32 * st + 8 * grp);
      bfr[nt][st] = *reinterpret_cast<const bf16x8*>(Bh + (int64_t)(16 * nt + col) * R + 32 * st + 8 * grp);
    }
  // q' = s R_i q at this lane's dims 16 nt + 4 grp + r
  f32x4 qv[NT];
  {
    const bf16* qh = static_cast<const bf16*>(p.q) + ((int64_t)b * p.H + h) * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qv[nt] = load4(qh, nt);
    rotate(qv);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qv[nt] *= p.scale;
  }

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int ntiles = (t1 - t0 + 15) / 16;
  // this wave's tiles w, w + 4, ..: local index lt is tile w + 4 lt
  const int ntw = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  auto tile_ptr = [&](int lt) -> const bf16* {
    const int j0 = t0 + (wave + kWaves * min(lt, ntw - 1)) * 16;
    const int pg = __builtin_amdgcn_readfirstlane(ptab[j0 / P - pfirst]);
    return pages + tile_base(pg, g, j0 % P, G, P, Rt);
  };
  // transposing-read offsets (bytes inside a KiB of values): dims 8 grp + 4 hh + col / 4,
  // tokens 4 (col % 4) .. + 3
  int vro[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int d = 8 * grp + 4 * hh + (col >> 2), c4 = col & 3;
    vro[hh] = val_slot((d >> 4) * 32 + (d & 15) * 2 + (c4 >> 1)) * 16 + (c4 & 1) * 8;
  }
  // Tiles are read exactly once per call: non-temporal loads.
  // This lane's 16-byte chunk of each value KiB: read from chunk
  // val_slot(lane) of the block, stored at slot `lane` of the wave's LDS KiB
  const int vsrc = val_slot(lane) * 8;
  bf16x8 kbuf[kPF][KS], vbuf[kPF][KS];
  // tile ti -> register set U
  auto issue = [&](auto U, int ti) {
    constexpr int u = decltype(U)::value;
    const bf16* tp = tile_ptr(ti);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      kbuf[u][st] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(tp + col * R + 32 * st + 8 * grp));
      vbuf[u][st] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(tp + 16 * R + st * 512 + vsrc));
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // consume slot U holding tile ti (nvalid tokens valid; FULL: all 16).
  // Order: the value block goes through LDS first (its transposing reads
  // are in flight during the key products), then all key and value products
  // are issued into their own accumulators, so that the softmax arithmetic
  // reads results that have long landed instead of waiting on each product.
  auto step = [&](auto U, int nvalid, auto full) {
    constexpr int u = decltype(U)::value;
    constexpr bool FULL = decltype(full)::value;
    const bool valid = FULL || col < nvalid;
    bf16x8 vf[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      unsigned char* vb = &vlds[wave][st * 1024];
      *reinterpret_cast<bf16x8*>(vb + 16 * lane) = vbuf[u][st];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vro[0]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vro[1]));
      vf[st] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // keys: lane holds K^T[dim 16 nt + 4 grp + r][token col]; values likewise V^T
    f32x4 kh[NT], vh[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      kh[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        kh[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[nt][st], kbuf[u][st], kh[nt], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vh[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        vh[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nt][st], vf[st], vh[nt], 0, 0, 0);
    }
    // four independent partial sums (one per r), so the products do not
    // form one dependent chain
    f32x4 sc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sc4 += qv[nt] * kh[nt];
    float sc = (sc4[0] + sc4[1]) + (sc4[2] + sc4[3]);
    sc += __shfl_xor(sc, 16);
    sc += __shfl_xor(sc, 32);
    if (!FULL && !valid) sc = -INFINITY;
    const float mx = row_max16(sc);       // the same in every lane group
    if (mx > m + kLazy) {                 // wave-uniform
      const float alpha = exp2_diff(m, mx);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
      lsum *= alpha;
      m = mx;
    }
    const float pw = fast_exp2(sc - m);   // 0 for masked tokens
    lsum += pw;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (FULL) {
        o[nt] += pw * vh[nt];
      } else {
        // a masked token's rebuilt value may be anything (even NaN): select, not multiply
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nt][r] = valid ? o[nt][r] + pw * vh[nt][r] : o[nt][r];
      }
    }
  };

  // decoders and q' have landed before the tile loads start: the loop's waits
  // then only count tile loads, which complete in issue order
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (ntw > 0) {                         // wave-uniform
    // prologue in slot order (the loop's waits assume loads complete in it)
    static_for<kPF>([&](auto U) {
      issue(U, decltype(U)::value);
      __builtin_amdgcn_sched_barrier(0);
    });
    // main loop over whole groups of full tiles: no branches in the body, so
    // every register set is refilled in place and the waits count exactly
    const int nfull = (t1 - t0) / 16;
    const int nfw = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
    int base = 0;
    for (; base + kPF <= nfw; base += kPF) {
      static_for<kPF>([&](auto U) {
        step(U, 16, std::true_type{});
        __builtin_amdgcn_sched_barrier(0);   // keep each refill below its consumer
        issue(U, base + decltype(U)::value + kPF);   // clamped: always a valid tile
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // the rest (fewer than kPF full tiles and a ragged last one) is already in flight
    static_for<kPF>([&](auto U) {
      constexpr int u = decltype(U)::value;
      if (base + u < ntw) {
        const int nvalid = min(16, t1 - (t0 + (wave + kWaves * (base + u)) * 16));
        if (nvalid == 16)
          step(U, 16, std::true_type{});
        else
          step(U, nvalid, std::false_type{});
      }
    });
  }
  // exact tokens t = e0 .. e1-1 of 0..nw (ring tokens j0 + t, t == nw the
  // current one), 16 per step, token tb + col in this lane
  {
    const int W = p.W;
    const int j0 = max(0, i - W), nw = i - j0;
    const int e0 = s * p.tw, e1 = min(e0 + p.tw, nw + 1);
    const int64_t rs = (int64_t)p.H * DH;                 // elements per ring slot
    const bf16* ring_k = static_cast<const bf16*>(p.ring_k);
    const bf16* ring_v = static_cast<const bf16*>(p.ring_v);
    for (int tb = e0 + 16 * wave; tb < e1; tb += 16 * kWaves) {
      const int t = tb + col;
      const bool valid = t < e1;
      f32x4 kx[NT], vx[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) kx[nt] = vx[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (valid && t < nw) {
        const int64_t off = ((int64_t)b * (W + 1) + (j0 + t) % (W + 1)) * rs + (int64_t)h * DH;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          kx[nt] = load4(ring_k + off, nt);
          vx[nt] = load4(ring_v + off, nt);
        }
      } else if (valid) {
        const int64_t off = ((int64_t)b * p.H + h) * DH;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          kx[nt] = load4(static_cast<const bf16*>(p.k_cur) + off, nt);
          vx[nt] = load4(static_cast<const bf16*>(p.v_cur) + off, nt);
        }
        rotate(kx);
        // ring append: slot i mod (W+1) held token i-W-1, which no slice reads
        const int64_t so = ((int64_t)b * (W + 1) + i % (W + 1)) * rs + (int64_t)h * DH;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s16x4 kw, vw;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kw[r] = bf16_bits(kx[nt][r]);
            vw[r] = bf16_bits(vx[nt][r]);
          }
          *reinterpret_cast<s16x4*>(static_cast<bf16*>(p.ring_k) + so + 16 * nt + 4 * grp) = kw;
          *reinterpret_cast<s16x4*>(static_cast<bf16*>(p.ring_v) + so + 16 * nt + 4 * grp) = vw;
        }
      }
      f32x4 sc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc4 += qv[nt] * kx[nt];
      float sc = (sc4[0] + sc4[1]) + (sc4[2] + sc4[3]);
      sc += __shfl_xor(sc, 16);
      sc += __shfl_xor(sc, 32);
      if (!valid) sc = -INFINITY;
      const float mx = row_max16(sc);     // finite: token tb is valid
      if (mx > m + kLazy) {
        const float alpha = exp2_diff(m, mx);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
        lsum *= alpha;
        m = mx;
      }
      const float pw = fast_exp2(sc - m);
      lsum += pw;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] += pw * vx[nt];
    }
  }
  // totals over the 16 token lanes (the four lane groups hold the same tokens)
  lsum = row_sum16(lsum);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[nt][r] = row_sum16(o[nt][r]);
  // merge of the four waves (each m is wave-uniform)
  if (lane == 0) {
    mrg_ml[wave][0] = m;
    mrg_ml[wave][1] = lsum;
  }
  if (col == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(&mrg_o[wave][16 * nt + 4 * grp]) = o[nt];
  }
  __syncthreads();
  if (wave == 0) {
    float M = mrg_ml[0][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg_ml[w][0]);
    float wt[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wt[w] = exp2_diff(mrg_ml[w][0], M);
      L += wt[w] * mrg_ml[w][1];
    }
    const int64_t row = ((int64_t)b * p.S + s) * p.H + h;
    if (lane == 0) {
      p.part_ml[row * 2 + 0] = M;
      p.part_ml[row * 2 + 1] = L;
    }
#pragma unroll
    for (int d = lane; d < DH; d += 64) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += wt[w] * mrg_o[w][d];
      p.part_o[row * p.Dp + d] = v;
    }
  }
}

template <int R, int DH>
hipError_t launch_r(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(p.S, p.B, p.H);
  hipLaunchKernelGGL((k_scan_reconstruct_mfma<R, DH>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool scan_reconstruct_mfma_supports(const DecodeParams& p) {
  return p.bf16 && p.hpg == 1 && p.rk == p.rv && (p.rk == 32 || p.rk == 64) &&
         (p.dh == 64 || p.dh == 128) && p.max_pages <= kPageTab;
}

hipError_t launch_scan_reconstruct_mfma(const DecodeParams& p, hipStream_t s) {
  if (!scan_reconstruct_mfma_supports(p)) return hipErrorNotSupported;
  if (p.rk == 32) return p.dh == 128 ? launch_r<32, 128>(p, s) : launch_r<32, 64>(p, s);
  return p.dh == 128 ? launch_r<64, 128>(p, s) : launch_r<64, 64>(p, s);
}

}  // namespace lla
