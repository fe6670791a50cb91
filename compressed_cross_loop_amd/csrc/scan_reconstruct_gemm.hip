// Reconstruct-on-read for head-folded latents (LLA-2D: one K and one V latent
// per token shared by all heads; "Looped Latent Attention" abstracts) on the
// gfx950 matrix cores.  Rebuilding every head's keys and values is a GEMM per
// sequence,
//   K^[tokens x H d_h] = S^K[tokens x r] . A^T [r x H d_h]
//   V^[tokens x H d_h] = S^V[tokens x r] . B_t [r x H d_h]
// with an attention epilogue per head.  Two forms: the LDS-staged one further
// down (d_h = 64 or 96, the usual case) and the register-streamed one here
// (d_h = 128, and stores whose page table does not fit the staged form's LDS
// table).
//
// Register-streamed form: one workgroup = (context split, sequence, 2 heads),
// four waves = {K^, V^} x 2 heads; each wave rebuilds a 128-token x d_h tile
// of its head over the latent width in K steps of 32 on
// v_mfma_f32_16x16x32_bf16.
//
// No operand is shared between the waves of a workgroup (each wave owns one
// head's decoder and one latent half), so nothing goes through LDS: every
// wave streams its own operands from L2/HBM straight into registers with
// several K steps in flight and no barrier inside the K loop.
//   K^ wave: A fragment of row tile j = key row of token 16 j + (lane % 16),
//            8 consecutive latent dims (one 16-byte load from the store).
//   V^ wave: the value block is dimension-major, so each lane loads 8 dims x 8
//            tokens (eight 16-byte loads) and regroups them in registers; row
//            tile j then holds tokens {8 m + j : m = 0..15}.
//   both:    B fragment = 8 consecutive latent dims of one decoder row (A_t
//            and B_t^T are both stored [d_h][r]).
// After a tile the K^ waves reduce q' . k^ per token (DPP row sums) into LDS,
// one barrier, and the V^ waves run the online softmax and o += p . v^ for
// their (permuted) tokens.
//
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  The launch order is remapped so that each XCD works through a
// contiguous range of (4 sequence splits x head pairs): the workgroups in
// flight on one XCD share latent tiles (same split, other head pairs) and
// decoders (same head pair, other splits) in that XCD's L2.
#include <algorithm>

#include "device_common.h"
#include "lla_internal.h"

namespace lla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int TM = 128;          // tokens per tile
constexpr int MT = TM / 16;      // row tiles per tile
constexpr int KC = 32;           // latent dims per K step
constexpr int kXcds = 8;
constexpr int kGroupItems = 4;   // splits grouped per head-pair sweep

// K steps in flight per wave: limited by registers (the accumulators take
// MT x d_h/16 x 4 of them); chosen so the K loop runs without spills
template <int DH, int KIND> struct Stages {
  static constexpr int value = DH == 128 ? 1 : (DH == 96 ? 2 : 3);
};

// Everything one wave of role KIND (0: K^, 1: V^) does for its work item.
// The two roles are separate instantiations so that each gets its own
// register allocation; both pass the same barriers (one per tile).
template <int DH, int KIND>
__device__ __forceinline__ void wave_main(const DecodeParams& p, float (*sc)[2][TM], int b, int s, int hb) {
  constexpr int NT = DH / 16;        // column tiles per head
  constexpr int NS = Stages<DH, KIND>::value;
  const int lane = threadIdx.x & 63;
  const int hl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);   // head of the pair
  const int col = lane & 15, kg = lane >> 4;
  const int H = p.H, R = p.rk, Rt = 2 * p.rk, P = p.P;
  const int h = 2 * hb + hl;
  const bool head_ok = h < H;
  const int hc = head_ok ? h : H - 1;
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;
  const int ntile = (t1 - t0 + TM - 1) / TM;
  const int nks = R / KC;

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const int32_t* bt = p.bt + (int64_t)b * p.max_pages;
  // Addresses are a wave-uniform base (scalar registers) plus one 32-bit
  // lane offset, so the unrolled loads do not each hold a 64-bit pointer.
  // This wave's decoder (A_t or B_t^T, both [DH][R]): fragment nt is row
  // 16 nt + col, latent dims ks*32 + 8 kg ..
  const bf16* dec = static_cast<const bf16*>(KIND ? p.Bm : p.A) + (int64_t)hc * DH * R;
  const uint32_t lane_off = (uint32_t)(col * R + 8 * kg);   // row col, dims 8 kg .. (decoder rows)
  // key rows: token-major (row col, like the decoders), or chunk-major when wide
  const bool wide = wide_keys(R);
  const uint32_t key_lane_off = wide ? (uint32_t)(col * kKeyChunk + 8 * kg) : lane_off;
  const int key_step = wide ? 16 * kKeyChunk : KC;

  float qv[NT];
  if (KIND == 0) {
    const float* qh = p.qhead + ((int64_t)b * H + hc) * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qv[nt] = qh[16 * nt + col];
  }

  // start of a latent token's 16-token tile in the store (j uniform)
  auto tile_of = [&](int j) -> const bf16* {
    const int pg = __builtin_amdgcn_readfirstlane(bt[j / P]);
    return pages + tile_base(pg, 0, j % P, 1, P, Rt);
  };

  struct Set {
    bf16x8 a[MT];
    bf16x8 d[NT];
  };
  Set set[NS];
  const bf16* kbase[MT];   // K^: 16-token store tile of row tile j (uniform)
  const bf16* vbase;       // V^: value rows of this lane's 8 tokens, dims 8 (kg%2) .. of sub-block kg/2
  auto issue = [&](Set& st, int ks) {
    if (KIND == 0) {
#pragma unroll
      for (int j = 0; j < MT; ++j)
        st.a[j] = *reinterpret_cast<const bf16x8*>(kbase[j] + ks * key_step + key_lane_off);
    } else {
      // dims ks*32 + 8 kg + k (k = 0..7) of this lane's 8 tokens: sub-block
      // 2 ks + kg/2, dim row 8 (kg%2) + k
      const bf16* vp = vbase + ks * 512;
#pragma unroll
      for (int k = 0; k < 8; ++k) st.a[k] = *reinterpret_cast<const bf16x8*>(vp + k * 16);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      st.d[nt] = *reinterpret_cast<const bf16x8*>(dec + (nt * 16 * R + ks * KC) + lane_off);
  };

  f32x4 acc[MT][NT];
  auto consume = [&](const Set& st) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      bf16x8 af;
      if (KIND == 0) {
        af = st.a[j];
      } else {
        // regroup: fragment j (token 8 m + j) = element j of each dim row;
        // dword q packs rows 2q (low half) and 2q + 1 (high half), element j
        // being the low (j even) or high (j odd) half of dword j/2
        u32x4 f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned lo = __builtin_bit_cast(u32x4, st.a[2 * q])[j >> 1];
          const unsigned hi = __builtin_bit_cast(u32x4, st.a[2 * q + 1])[j >> 1];
          f[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        af = __builtin_bit_cast(bf16x8, f);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[j][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, st.d[nt], acc[j][nt], 0, 0, 0);
    }
  };

  float m = -INFINITY, l = 0.f, o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = 0.f;

  for (int tile = 0; tile < ntile; ++tile) {
    const int j0 = t0 + tile * TM;
    const int last = t1 - 1;
    if (KIND == 0) {
      // row tile j = tokens j0 + 16 j .. + 15, one 16-token store tile; a
      // tile wholly past the end rereads the last valid one (masked later)
#pragma unroll
      for (int j = 0; j < MT; ++j) kbase[j] = tile_of(min(j0 + 16 * j, last));
    } else {
      // tokens 8 col .. 8 col + 7 (one half of a 16-token tile)
      const int tok = min(j0 + 8 * col, last);
      const int64_t pg = bt[tok / P];
      vbase = pages + tile_base(pg, 0, tok % P, 1, P, Rt) + 16 * R + (kg >> 1) * 256 + 8 * (kg & 1) * 16 +
              (tok & 8);
    }
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K loop: NS steps in flight; refills are unconditional (clamped to the
    // last step) so no register set has to survive a skipped refill
#pragma unroll
    for (int u = 0; u < NS; ++u) issue(set[u], min(u, nks - 1));
    int ks = 0;
    while (ks < nks) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        consume(set[u]);
        __builtin_amdgcn_sched_barrier(0);   // keep the refill below its consumer
        issue(set[u], min(ks + NS, nks - 1));
        if (++ks >= nks) break;
      }
    }

    // ---- attention epilogue
    const int par = tile & 1;
    if (KIND == 0) {
      // lane holds K^[token 16 j + 4 kg + r][dim 16 nt + col]
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        __builtin_amdgcn_sched_barrier(0);   // one row tile's accumulators at a time
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) a += qv[nt] * acc[j][nt][r];
          a = row_sum16(a);
          const int tok = 16 * j + 4 * kg + r;
          if (col == 0) sc[par][hl][tok] = (j0 + tok < t1) ? a : -INFINITY;
        }
      }
    }
    __syncthreads();
    if (KIND == 1) {
      // lane holds V^[token 8 (4 kg + r) + j][dim 16 nt + col]
      float mx = fmaxf(sc[par][hl][lane], sc[par][hl][lane + 64]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m, mx);
      const float alpha = exp2_diff(m, mn);
      float lp = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        __builtin_amdgcn_sched_barrier(0);   // one row tile's accumulators at a time
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 8 * (4 * kg + r) + j;
          const bool ok = j0 + tok < t1;
          const float pw = ok ? fast_exp2(sc[par][hl][tok] - mn) : 0.f;
          lp += pw;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] += ok ? pw * acc[j][nt][r] : 0.f;
        }
      }
      lp += __shfl_xor(lp, 16);
      lp += __shfl_xor(lp, 32);
      l = l * alpha + lp;
      m = mn;
    }
  }

  // ---- the V^ wave of each head writes the split's partial
  if (KIND == 1 && head_ok) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      o[nt] += __shfl_xor(o[nt], 16);
      o[nt] += __shfl_xor(o[nt], 32);
    }
    const int64_t row = ((int64_t)b * p.S + s) * H + h;
    if (lane == 0) {
      p.part_ml[row * 2 + 0] = m;
      p.part_ml[row * 2 + 1] = l;
    }
    if (kg == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p.part_o[row * p.Dp + 16 * nt + col] = o[nt];
    }
  }
}

template <int DH>
__global__ __launch_bounds__(kThreads, 1) void k_scan_reconstruct_gemm(DecodeParams p, int n_hp, int n_wg) {
  __shared__ float sc[2][2][TM];     // scores: tile parity, head of the pair, token
  // work item, in XCD-aware order
  const int L = blockIdx.x;
  const int lam = (L % kXcds) * (n_wg / kXcds) + L / kXcds;
  const int grp_i = lam / (kGroupItems * n_hp), hb = (lam / kGroupItems) % n_hp;
  const int item = grp_i * kGroupItems + lam % kGroupItems;
  if (item >= p.B * p.S) return;     // padding: the whole workgroup leaves
  const int b = item / p.S, s = item % p.S;
  // waves 0, 2: K^ of heads 2 hb, 2 hb + 1; waves 1, 3: V^
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
    wave_main<DH, 1>(p, sc, b, s, hb);
  else
    wave_main<DH, 0>(p, sc, b, s, hb);
}

// ---------------------------------------------------------------------------
// LDS-staged form (d_h = 64 or 96).  One workgroup = (context split, sequence,
// 2 heads), eight waves = {K^, V^} x 2 heads x 2 token halves of a 256-token
// tile; each wave rebuilds 128 tokens x d_h of its head.  Per K step of 32
// latent dims every operand the step needs -- the key rows and value blocks
// of the 256 tokens, both heads' A_t and B_t^T rows -- is copied into LDS with
// direct global -> LDS loads (lane i's 16 bytes land at base + 16 i, one
// 1 KiB copy per instruction), in three buffers with one barrier per step:
// the copies run two K steps ahead of the products.
// The four K^ (V^) waves share the latent tiles and the two token halves
// share the decoder rows, so a latent or decoder byte crosses the load path
// once per workgroup instead of once per wave, and every load instruction
// covers whole 64-byte row pieces or a contiguous 1 KiB.
//   copy slots: rows x 64 B copies (keys, decoders) put chunk c of row r at
//   slot 4 r + (c ^ (r / 4 % 4)), so the 16 lanes of a 16-byte LDS read hit
//   16 different bank groups.  A value copy holds two 16 x 16 dimension-major
//   sub-blocks of a 16-token store tile; the V^ waves read it with the gfx950
//   transposing LDS read (ds_read_b64_tr_b16: inside each 16-lane group,
//   lane i receives element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4 and
//   12 + i / 4), which turns four dims x 16 tokens into the token-major
//   A-operand pieces of the MFMA; chunk slots are XOR-swizzled (bit 3 ^= bit
//   4) so the two 16-lane groups served together read different banks.
// The decoder rows come from a copy regrouped per K step ([H][A_t, B_t^T]
// [r/32][d_h][32], written by k_tile_decoders at the start of the call), so
// each decoder copy is a contiguous 1 KiB as well; a copy of 16 strided row
// pieces costs the address unit about twice as much.
// The two token halves of a head see the same scores, so they keep the same
// running maximum and their (l, o) simply add at the end.
namespace staged {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPageTab = 2048;      // page ids of the split, staged in LDS (with three
                                    // 48 KiB stage buffers the workgroup takes 157 KiB)

template <int DH> struct Shape {
  static constexpr int NT = DH / 16;            // column tiles per head
  static constexpr int MTW = DH == 96 ? 6 : 8;  // row tiles per wave (registers: MTW x NT accumulators)
  static constexpr int TMW = 16 * MTW;          // tokens per wave
  static constexpr int TM = 2 * TMW;            // tokens per tile (two halves)
  static constexpr int NTT = TM / 16;           // 16-token store tiles per tile
  // 1 KiB copies per step, in LDS order: key pieces, value pieces, A rows of
  // both heads, B rows of both heads
  static constexpr int QV = NTT, QA = 2 * NTT, QB = 2 * NTT + 2 * NT, NQ = 2 * NTT + 4 * NT;
  static constexpr int PER_WAVE = NQ / kWaves;   // copies per wave and step (< 16: vmcnt immediate)
  static constexpr int STAGE = NQ * 1024;
  static constexpr int MAXP = (NTT + kWaves - 1) / kWaves;   // store tiles per wave, at most
  static_assert(NQ % kWaves == 0 && PER_WAVE >= 2 * MAXP, "copies must divide evenly over the waves");
  static_assert(PER_WAVE < 16, "the step wait names the copies in flight as a vmcnt immediate");
};

__device__ __forceinline__ int row_slot(int row, int c) { return 4 * row + (c ^ ((row >> 2) & 3)); }
__device__ __forceinline__ int val_slot(int ch) { return ch ^ (((ch >> 4) & 1) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0), expcnt / lgkmcnt untouched

// The staged kernel's copies (copy_to_lds) are not tracked by the compiler's
// wait insertion, which cannot tell the three stage buffers' copies apart
// once the step loop's control flow joins; the kernel waits for them itself.
//

// LDS regions of the staged kernel.  The three stage buffers are separate
// LDS variables and every access names one of them statically: the compiler
// then knows that copies into one buffer cannot alias reads of the other and
// does not wait for the copies in flight before reading.
template <int DH> struct Smem {
  float sc[2][2][Shape<DH>::TM];   // scores: tile parity, head of the pair, token
  float qh[2][DH];                 // q' of both heads
  float mrg[2][DH + 1];            // second half's (o, l) per head
  int32_t ptab[kPageTab];          // page ids of the split
};

// Everything one wave of role KIND (0: K^, 1: V^) does for its work item;
// the roles are separate instantiations so that each gets its own register
// allocation.  Both pass the same barriers: one per K step, one per tile, one
// at the end.
template <int DH, int KIND>
__device__ __forceinline__ void staged_wave(const DecodeParams& p, Smem<DH>& sm, unsigned char* stage0,
                                            unsigned char* stage1, unsigned char* stage2, int b, int s,
                                            int hb, int hl,
                                            int th, int wave, int t0, int t1) {
  using Sh = Shape<DH>;
  constexpr int NT = Sh::NT, MTW = Sh::MTW, TMW = Sh::TMW, TM = Sh::TM;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int H = p.H, R = p.rk, Rt = 2 * p.rk, P = p.P;
  const int h = 2 * hb + hl;
  const int ntile = (t1 - t0 + TM - 1) / TM;
  const int nks = R / KC;
  const int last = t1 - 1;
  const int pfirst = t0 / P;

  const bf16* pages = static_cast<const bf16*>(p.pages);
  const bf16* dect = static_cast<const bf16*>(p.dect);

  // This wave's copies of a step: the key and value pieces of store tiles
  // wave, wave + 8, .. of the tile, then its share of the decoder rows.
  // Sources are uniform bases (a store tile, per tile) plus lane offsets plus
  // the K step times a uniform stride, so a step only adds and issues.
  const int np = (Sh::NTT - wave + kWaves - 1) / kWaves;   // store tiles of this wave
  int dstart = 0;                                          // first decoder copy of this wave
  for (int w = 0; w < wave; ++w) dstart += Sh::PER_WAVE - 2 * ((Sh::NTT - w + kWaves - 1) / kWaves);
  const int row = lane >> 2, cq = (lane & 3) ^ ((row >> 2) & 3);
  // key rows: row, chunk cq (token-major, or chunk-major when wide: then a
  // step's 16 rows x 64 B are one contiguous KiB)
  const bool wide = wide_keys(R);
  const uint32_t koff = wide ? row * kKeyChunk + 8 * cq : row * R + 8 * cq;
  const uint32_t kstep = wide ? 16 * kKeyChunk : KC;
  const int vch = val_slot(lane);
  const uint32_t voff = 16 * R + (vch >> 5) * 256 + ((vch >> 1) & 15) * 16 + (vch & 1) * 8;
  uint32_t doff[Sh::PER_WAVE];
  int dslot[Sh::PER_WAVE];
#pragma unroll
  for (int u = 0; u < Sh::PER_WAVE; ++u) {
    const int dq = min(max(dstart + u - 2 * np, 0), 4 * NT - 1);   // decoder copy (clamped where unused)
    const int which = dq / NT, nt = dq % NT;               // which: A h0, A h1, B h0, B h1
    const int hh = min(2 * hb + (which & 1), H - 1);
    doff[u] = (((uint32_t)hh * 2 + (which >> 1)) * nks * DH + 16 * nt + row) * KC + 8 * cq;
    dslot[u] = Sh::QA + dq;
  }
  const bf16* tbase[Sh::MAXP];
  auto prep = [&](int tile) {
    const int j0 = t0 + tile * TM;
#pragma unroll
    for (int k = 0; k < Sh::MAXP; ++k) {
      const int jt = min(j0 + 16 * (wave + kWaves * k), last);   // a piece wholly past the end rereads the last
      const int pg = __builtin_amdgcn_readfirstlane(sm.ptab[jt / P - pfirst]);
      tbase[k] = pages + tile_base(pg, 0, jt % P, 1, P, Rt);
    }
  };
  auto issue = [&](int ks, unsigned char* dst) {
#pragma unroll
    for (int u = 0; u < Sh::PER_WAVE; ++u) {
      const bf16* src;
      int slot;
      if (u < 2 * np) {
        const int k = u >> 1, tt = wave + kWaves * k;
        src = (u & 1) ? tbase[k] + (voff + (uint32_t)ks * 512) : tbase[k] + (koff + (uint32_t)ks * kstep);
        slot = (u & 1) ? Sh::QV + tt : tt;
      } else {
        src = dect + (doff[u] + (uint32_t)ks * (DH * KC));
        slot = dslot[u];
      }
      copy_to_lds(src, dst + slot * 1024);
    }
  };

  // operand read offsets inside a stage
  const int kslot = row_slot(col, kg) * 16;   // key / decoder rows: row col, chunk kg
  int vslot[2];                               // V^: dims 8 kg + 4 hh + col / 4, tokens 4 (col % 4) ..
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int d = 8 * kg + 4 * hh + (col >> 2), c4 = col & 3;
    vslot[hh] = val_slot((d >> 4) * 32 + (d & 15) * 2 + (c4 >> 1)) * 16 + (c4 & 1) * 8;
  }
  const int dec_off = ((KIND == 0 ? Sh::QA : Sh::QB) + hl * NT) * 1024 + kslot;
  const int lat_off = ((KIND == 0 ? 0 : Sh::QV) + th * MTW) * 1024;

  f32x4 acc[MTW][NT];
  float m = -INFINITY, l = 0.f, o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = 0.f;

  // one K step on the operands staged in `st`
  auto compute = [&](const unsigned char* st) {
    bf16x8 bb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bb[nt] = *reinterpret_cast<const bf16x8*>(st + dec_off + nt * 1024);
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      bf16x8 a;
      if (KIND == 0) {
        a = *reinterpret_cast<const bf16x8*>(st + lat_off + j * 1024 + kslot);
      } else {
        // token col of store tile j of this half, dims 8 kg .. 8 kg + 7
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const unsigned char* vb = st + lat_off + j * 1024;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vslot[0]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + vslot[1]));
        a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[j][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb[nt], acc[j][nt], 0, 0, 0);
    }
  };

  for (int tile = 0; tile < ntile; ++tile) {
#pragma unroll
    for (int j = 0; j < MTW; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Every tile starts in buffer 0 (K steps rotate 0, 1, 2, 0, ..).  Buffers 0
    // and 1 are free here: their last readers passed the previous tile's
    // score barrier.
    prep(tile);
    issue(0, stage0);
    if (nks > 1) issue(1, stage1);
    // Step k: this wave's copies of step k have landed once at most those of
    // step k + 1 are in flight; after the barrier everyone's have, and the
    // buffer of step k - 1 (read before the barrier) takes step k + 2.
    auto step = [&](int k, const unsigned char* cur, unsigned char* nxt) {
      if (k + 1 < nks)
        copy_barrier<Sh::PER_WAVE>();
      else
        copy_barrier<0>();
      if (k + 2 < nks) issue(k + 2, nxt);
      compute(cur);
    };
    for (int ks = 0; ks < nks; ks += 3) {
      step(ks, stage0, stage2);
      if (ks + 1 < nks) step(ks + 1, stage1, stage0);
      if (ks + 2 < nks) step(ks + 2, stage2, stage1);
    }

    // ---- attention epilogue; lane holds X^[token 16 j + 4 kg + r of this half][dim 16 nt + col]
    const int par = tile & 1;
    const int j0 = t0 + tile * TM;
    if (KIND == 0) {
      float qv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) qv[nt] = sm.qh[hl][16 * nt + col];
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) a += qv[nt] * acc[j][nt][r];
          a = row_sum16(a);
          const int tok = th * TMW + 16 * j + 4 * kg + r;
          if (col == 0) sm.sc[par][hl][tok] = (j0 + tok < t1) ? a : -INFINITY;
        }
      }
    }
    __syncthreads();
    if (KIND == 1) {
      // both halves take the maximum over all scores of the head's tile
      const float* sch = sm.sc[par][hl];
      float mx = -INFINITY;
#pragma unroll
      for (int x = 0; x < TM / 64; ++x) mx = fmaxf(mx, sch[lane + 64 * x]);
      mx = wave_max(mx);
      const float mn = fmaxf(m, mx);
      const float alpha = exp2_diff(m, mn);
      float lp = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = th * TMW + 16 * j + 4 * kg + r;
          const bool ok = j0 + tok < t1;
          const float pw = ok ? fast_exp2(sch[tok] - mn) : 0.f;
          lp += pw;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] += ok ? pw * acc[j][nt][r] : 0.f;
        }
      }
      lp += __shfl_xor(lp, 16);
      lp += __shfl_xor(lp, 32);
      l = l * alpha + lp;
      m = mn;
    }
  }

  // ---- merge the two token halves of each head and write the split's partial
  if (KIND == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      o[nt] += __shfl_xor(o[nt], 16);
      o[nt] += __shfl_xor(o[nt], 32);
    }
    if (th == 1 && kg == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm.mrg[hl][16 * nt + col] = o[nt];
      if (col == 0) sm.mrg[hl][DH] = l;
    }
  }
  __syncthreads();
  if (KIND == 1 && th == 0 && h < H) {
    const int64_t prow = ((int64_t)b * p.S + s) * H + h;
    if (lane == 0) {
      p.part_ml[prow * 2 + 0] = m;
      p.part_ml[prow * 2 + 1] = l + sm.mrg[hl][DH];
    }
    if (kg == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p.part_o[prow * p.Dp + 16 * nt + col] = o[nt] + sm.mrg[hl][16 * nt + col];
    }
  }
}

template <int DH>
__global__ __launch_bounds__(kThreads, 1) void k_scan_reconstruct_staged(DecodeParams p, int n_hp, int n_wg) {
  __shared__ __attribute__((aligned(1024))) Smem<DH> sm;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[Shape<DH>::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[Shape<DH>::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[Shape<DH>::STAGE];
  const int L = blockIdx.x;
  const int lam = (L % kXcds) * (n_wg / kXcds) + L / kXcds;
  const int grp_i = lam / (kGroupItems * n_hp), hb = (lam / kGroupItems) % n_hp;
  const int item = grp_i * kGroupItems + lam % kGroupItems;
  if (item >= p.B * p.S) return;      // padding: the whole workgroup leaves
  const int b = item / p.S, s = item % p.S;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = p.pos[b];
  const int n_lat = max(0, i - p.W);
  int t0 = s * p.chunk;
  const int t1 = (s == p.S - 1) ? n_lat : min(n_lat, t0 + p.chunk);
  if (t0 > n_lat) t0 = n_lat;

  // page ids of tokens t0 .. t1-1 (never more than max_pages <= kPageTab) and q' of both heads
  const int pfirst = t0 / p.P;
  const int npg = t1 > t0 ? (t1 - 1) / p.P - pfirst + 1 : 0;
  for (int x = tid; x < npg; x += kThreads) sm.ptab[x] = p.bt[(int64_t)b * p.max_pages + pfirst + x];
  for (int x = tid; x < 2 * DH; x += kThreads) {
    const int hh = min(2 * hb + x / DH, p.H - 1);
    sm.qh[x / DH][x % DH] = p.qhead[((int64_t)b * p.H + hh) * DH + x % DH];
  }
  __syncthreads();

  const int hl = (wave >> 1) & 1, th = wave >> 2;
  if (wave & 1)
    staged_wave<DH, 1>(p, sm, stage0, stage1, stage2, b, s, hb, hl, th, wave, t0, t1);
  else
    staged_wave<DH, 0>(p, sm, stage0, stage1, stage2, b, s, hb, hl, th, wave, t0, t1);
}

// dect[h][ab][ks][d][k] = (ab ? B_t^T : A_t)[h][d][32 ks + k], 16 bytes per thread
__global__ __launch_bounds__(256) void k_tile_decoders(const bf16* __restrict__ A, const bf16* __restrict__ Bt,
                                                       bf16* __restrict__ dect, int H, int DH, int R) {
  const int64_t n8 = (int64_t)2 * H * DH * R / 8;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n8; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 8 * x;                      // source element: [ab][h][d][r]
    const int r = (int)(e % R);
    const int64_t hd = e / R;                     // (ab, h, d)
    const int d = (int)(hd % DH);
    const int64_t abh = hd / DH;
    const int h = (int)(abh % H), ab = (int)(abh / H);
    const uint4 v = *reinterpret_cast<const uint4*>((ab ? Bt : A) + ((int64_t)h * DH + d) * R + r);
    *reinterpret_cast<uint4*>(dect + ((((int64_t)h * 2 + ab) * (R / KC) + r / KC) * DH + d) * KC + r % KC) = v;
  }
}

}  // namespace staged

}  // namespace

bool scan_reconstruct_gemm_supports(const DecodeParams& p) {
  return p.bf16 && p.G == 1 && p.rk == p.rv && p.rk % KC == 0 && (p.dh == 96 || p.dh == 128 || p.dh == 64);
}

bool scan_reconstruct_gemm_tiles_decoders(int dh, int G, int rk, int rv, int bf16) {
  return bf16 && G == 1 && rk == rv && rk % KC == 0 && (dh == 64 || dh == 96);
}

// the staged form serves d_h = 64, 96 when the split's page ids fit its LDS
// table and the call brought the regrouped decoder buffer
static bool staged_form(const DecodeParams& p) {
  return (p.dh == 64 || p.dh == 96) && p.max_pages <= staged::kPageTab && p.dect != nullptr;
}

hipError_t launch_scan_reconstruct_gemm_prep(const DecodeParams& p, hipStream_t s) {
  if (!scan_reconstruct_gemm_supports(p) || !staged_form(p)) return hipSuccess;
  const int64_t n8 = (int64_t)2 * p.H * p.dh * p.rk / 8;
  const int tb = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(staged::k_tile_decoders, dim3(tb), dim3(256), 0, s, static_cast<const bf16*>(p.A),
                     static_cast<const bf16*>(p.Bm), static_cast<bf16*>(p.dect), p.H, p.dh, p.rk);
  return hipGetLastError();
}

int scan_reconstruct_gemm_tile(int dh) {
  return dh == 96 ? staged::Shape<96>::TM : dh == 64 ? staged::Shape<64>::TM : TM;
}

hipError_t launch_scan_reconstruct_gemm(const DecodeParams& p, hipStream_t s) {
  if (!scan_reconstruct_gemm_supports(p)) return hipErrorNotSupported;
  const int n_hp = (p.H + 1) / 2;
  const int64_t items = (int64_t)p.B * p.S;
  const int64_t wg = (items + kGroupItems - 1) / kGroupItems * kGroupItems * n_hp;
  const int64_t n_wg = (wg + kXcds - 1) / kXcds * kXcds;
  if (n_wg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  if (staged_form(p)) {
    if (p.dh == 96)
      hipLaunchKernelGGL(staged::k_scan_reconstruct_staged<96>, grid, dim3(staged::kThreads), 0, s, p, n_hp,
                         (int)n_wg);
    else
      hipLaunchKernelGGL(staged::k_scan_reconstruct_staged<64>, grid, dim3(staged::kThreads), 0, s, p, n_hp,
                         (int)n_wg);
  } else if (p.dh == 96) {
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<96>, grid, dim3(kThreads), 0, s, p, n_hp, (int)n_wg);
  } else if (p.dh == 128) {
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<128>, grid, dim3(kThreads), 0, s, p, n_hp, (int)n_wg);
  } else {
    hipLaunchKernelGGL(k_scan_reconstruct_gemm<64>, grid, dim3(kThreads), 0, s, p, n_hp, (int)n_wg);
  }
  return hipGetLastError();
}

}  // namespace lla
