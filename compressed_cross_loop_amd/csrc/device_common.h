// Device helpers shared by the gfx950 kernels: element conversion, paged
// store addressing, rotary angles, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace lla {

typedef __bf16 bf16;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// Paged store: [page][group][P/16 tiles][16 key rows of rk | rv/16 x (16 dims x 16 tokens)]
__device__ __forceinline__ int64_t tile_base(int64_t page, int g, int slot, int G, int P, int R) {
  return ((page * G + g) * (int64_t)P + (slot & ~15)) * (int64_t)R;
}
// Inside a tile, key rows of up to kWideKeyRows numbers are token-major
// ([16][r_k]); wider ones are chunk-major: chunk c (dims 32c .. 32c + 31, the
// last one narrower when r_k % 32 != 0) holds the 16 tokens' pieces one after
// another, so that a 16-token x 32-dimension block is one contiguous 1 KiB.
constexpr int kWideKeyRows = 512;
constexpr int kKeyChunk = 32;
__device__ __forceinline__ bool wide_keys(int rk) { return rk > kWideKeyRows; }
// offset of key element d of the token in tile slot s (0..15) from the tile start
__device__ __forceinline__ int64_t key_in_tile(int s, int d, int rk) {
  if (!wide_keys(rk)) return (int64_t)s * rk + d;
  const int c = d / kKeyChunk;
  return (int64_t)c * (16 * kKeyChunk) + s * min(kKeyChunk, rk - kKeyChunk * c) + d % kKeyChunk;
}
__device__ __forceinline__ int64_t key_off(int64_t page, int g, int slot, int d, int G, int P, int R,
                                           int rk) {
  return tile_base(page, g, slot, G, P, R) + key_in_tile(slot & 15, d, rk);
}
__device__ __forceinline__ int64_t val_off(int64_t page, int g, int slot, int d, int G, int P, int R,
                                           int rk) {
  return tile_base(page, g, slot, G, P, R) + 16 * rk + (d >> 4) * 256 + (d & 15) * 16 + (slot & 15);
}

// fp8 latent store (byte offsets): a tile of 16 tokens of one group holds the
// key codes (token-major rows of rk), the value codes (rv/64 quads of four
// 16-dimension sub-blocks, inside a quad [dim % 16][token / 4][sub-block]
// [token % 4], so that the 4 tokens x 4 sub-blocks a lane feeds to the value
// MFMA are 16 contiguous bytes), then 16 fp32 key scales and 16 value scales.
__device__ __forceinline__ int64_t tile_bytes8(int rk, int rv) { return 16 * (int64_t)(rk + rv) + 128; }
__device__ __forceinline__ int64_t tile_base8(int64_t page, int g, int slot, int G, int P, int rk, int rv) {
  return ((page * G + g) * (P / 16) + slot / 16) * tile_bytes8(rk, rv);
}
__device__ __forceinline__ int64_t key_off8(int64_t page, int g, int slot, int d, int G, int P, int rk, int rv) {
  return tile_base8(page, g, slot, G, P, rk, rv) + (slot & 15) * rk + d;
}
__device__ __forceinline__ int64_t val_off8(int64_t page, int g, int slot, int d, int G, int P, int rk, int rv) {
  const int t = slot & 15;
  return tile_base8(page, g, slot, G, P, rk, rv) + 16 * rk + (d >> 6) * 1024 + (d & 15) * 64 + (t >> 2) * 16 +
         ((d >> 4) & 3) * 4 + (t & 3);
}
__device__ __forceinline__ int64_t scale_off8(int64_t page, int g, int slot, int part, int G, int P, int rk,
                                              int rv) {
  return tile_base8(page, g, slot, G, P, rk, rv) + 16 * (int64_t)(rk + rv) + part * 64 + (slot & 15) * 4;
}

// OCP e4m3 code -> float on the gfx950 converter (exact: every e4m3 value is
// a bf16 value)
__device__ __forceinline__ float e4m3_to_f(uint32_t code) {
  return static_cast<float>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false)[0]);
}
// float -> OCP e4m3 code, round to nearest even, saturating at +-448.  In
// the binade [2^e, 2^(e+1)) (e clipped below at -6, where the subnormals
// share the spacing 2^-9) the grid spacing is 2^(e-3); n = rint(|y| / 2^(e-3))
// is exact and lies in [0, 16], and the code is 8 (e + 7) + n - 8 (n = 16
// carries into the next binade, n < 8 at e = -6 are the subnormals).
__device__ __forceinline__ uint32_t f_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  const int e = max((int)((__float_as_uint(a) >> 23) & 0xFF) - 127, -6);
  const int n = (int)rintf(ldexpf(a, 3 - e));
  return sign | (uint32_t)(8 * e + 48 + n);
}

// Rotary angle p * theta_f, theta_f = base^(-2f/d_h).  theta_f and the
// product are fp64 (positions reach 16K and beyond, where an fp32 angle would
// be off by ~1e-3 rad); the product is reduced by whole turns in fp64 and
// only the reduced angle (|r| <= pi) goes through fp32 sincosf.
__device__ __forceinline__ double rope_theta(float base, int dh, int f) {
  return pow((double)base, -2.0 * (double)f / (double)dh);
}
__device__ __forceinline__ void rope_cs_theta(double theta, int pos, float& c, float& s) {
  const double two_pi = 6.283185307179586476925;
  const double a = (double)pos * theta;
  const double turns = rint(a / two_pi);
  const float r = (float)fma(-turns, two_pi, a);
  sincosf(r, &s, &c);
}
__device__ __forceinline__ void rope_cs(float base, int dh, int f, int pos, float& c, float& s) {
  rope_cs_theta(rope_theta(base, dh, f), pos, c, s);
}

// A load that is marked streaming (non-temporal) when NT: for data read once
// per call by a launch that keeps every CU busy.  Measured on the latent
// scans: with 256 or more workgroups streaming loads are 7-10% faster, with
// fewer (some CUs idle, or batch 1) plain cached loads are 5-12% faster.
template <bool NT, class T>
__device__ __forceinline__ T load_once(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// One 1 KiB copy global -> LDS: global_load_lds_dwordx4, lane i's 16 bytes
// land at LDS address lds + 16 i.  Written as an asm statement so that the
// compiler's wait insertion does not track it (it waits conservatively for
// every copy in flight before LDS reads it cannot prove disjoint); the caller
// waits itself.  A wave's copies complete in issue order, so after
// "vmcnt(n)" every copy but the wave's last n has landed, however many other
// memory operations were issued meanwhile.  m0 is an input of the statement
// (the compiler sets it); s_nop 0 keeps the one wait state that an SALU write
// of m0 needs before an LDS DMA reads it.
__device__ __forceinline__ void copy_to_lds(const void* src, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// Barrier after copy_to_lds copies: this wave's copies have landed but for its
// last N (the ones issued after those the barrier is for) and its LDS reads
// have returned, then all waves meet.  No fence: a workgroup fence, even one
// on LDS alone, would also wait for every copy in flight.  The asm statements
// keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void copy_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);   // vmcnt(N) lgkmcnt(0), expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier ordering LDS accesses only: unlike __syncthreads(), whose
// fence also covers global memory, it leaves the wave's global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Reductions over the 16 lanes of a DPP row (lanes 16k .. 16k+15) with DPP
// moves instead of LDS permutes: quad_perm [1,0,3,2] and [2,3,0,1] (xor 1,
// xor 2 inside each quad), row_half_mirror (lane i <-> 7-i inside each half
// row), row_mirror (lane i <-> 15-i inside the row).  Every lane ends with the
// row's total.  The 8-lane form stops after the half-row step.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum8(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v = row_sum8(v);
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return v;
}
// sum over groups of n = 8 or 16 consecutive lanes (n uniform)
__device__ __forceinline__ float group_sum(float v, int n) { return n == 16 ? row_sum16(v) : row_sum8(v); }

// 2^x on the hardware exp unit (v_exp_f32): -inf gives 0, results below the
// normal range flush to 0, which is harmless for softmax weights (they are
// relative to the running maximum, so at most 1)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 of (x - m) for the online softmax; m == -inf (nothing seen yet) gives 0
__device__ __forceinline__ float exp2_diff(float x, float m) {
  return (m == -INFINITY) ? 0.f : fast_exp2(x - m);
}

}  // namespace lla
