// Internal interface between the host layer (lla_api.cpp) and the gfx950
// kernels: plain parameter blocks passed by value, and launcher functions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

constexpr int kTile = 16;        // tokens per store tile
constexpr int kChunk = 64;       // split granularity in tokens

enum Mode : int32_t { kAbsorbed = 1, kReconstruct = 0 };

struct DecodeParams {
  // shapes
  int32_t B, H, dh, G, hpg, rk, rv, P, W;
  int32_t S, chunk;               // context splits and tokens per split
  int32_t WS, tw;                 // exact-window slices and tokens per slice
  int32_t Dp;                     // width of latent partial rows (r_v or d_h)
  int32_t max_pages;
  int32_t mode;
  int32_t bf16;                   // storage dtype: 1 = bf16, 0 = fp32
  int32_t fp8;                    // latents stored as e4m3 codes + per-token scales (bytes)
  int32_t need_qhead;             // a later kernel reads qhead (else the window
                                  // kernel rotates q itself)
  int32_t fuse_window;            // the matrix-core scan also does the exact
                                  // window: split s handles window slice s
  float rope_base;
  float scale;                    // log2(e) / sqrt(d_h)
  // caller buffers
  const int32_t* pos;
  const int32_t* bt;
  const void* pages;
  const void* q;
  const void* k_cur;
  const void* v_cur;
  void* ring_k;
  void* ring_v;
  const void* A;
  const void* Bm;
  void* out;
  // workspace regions
  void* qlat;                     // [B][H][rk]  storage dtype
  float* qhead;                   // [B][H][dh]
  float* part_ml;                 // [B][S][H][2]
  float* part_o;                  // [B][S][H][Dp] (bf16 elements when part_bf16)
  int32_t part_bf16;              // the wide scan leaves part_o in bf16 for the wide combine
  float* win_ml;                  // [B][WS][H][2]
  float* win_o;                   // [B][WS][H][dh]
  // head-folded reconstruct (LDS-staged form): A_t and B_t^T rows regrouped
  // per K step of 32 latent dims, [H][2][r/32][d_h][32] bf16
  void* dect;
  // two-pass absorbed scan of one wide shared latent: scores and
  // probabilities of every latent token, rows of lcap tokens
  int32_t lcap;
  int32_t wsplit;                 // parts of r_k the score pass is split into
  float* wscore;                  // [wsplit][B][H][lcap]
  void* wprob;                    // [B][H][lcap] bf16
  // fused single-launch path
  int32_t* tickets;               // [B][H] arrival counters
  float* fpart;                   // [B][H][S][2 + rv + dh]
};

struct WriterParams {
  int32_t B, n_tok, n_loops, G, rk, rv, R, d_in, P, dh, max_pages;
  int32_t rope_baked;
  int32_t bf16;
  int32_t fp8;                    // latents stored as e4m3 codes + per-token scales
  float rope_base;
  const int32_t* pos;
  const int32_t* bt;
  void* pages;
  const void* x;
  const void* enc;
  float* acc;                     // workspace [ksplit][B*n_tok][G][R] (MFMA path)
  int32_t ksplit;
};

// full-cache (uncompressed) decode scan
struct FullParams {
  int32_t B, H, dh, P, S, chunk, max_pages, bf16;
  float rope_base, scale;
  const int32_t* pos;
  const int32_t* bt;
  void* k_pages;
  void* v_pages;
  const void* q;
  const void* k_cur;
  const void* v_cur;
  float* part_ml;   // [B][S][H][2]
  float* part_o;    // [B][S][H][dh]
};
int full_scan_heads_per_block(int dh);
hipError_t launch_full_scan(const FullParams& p, hipStream_t s);

// parallel attention over whole sequences (bf16)
struct ParParams {
  int32_t B, H, dh, G, hpg, rk, rv, P, max_pages, W, n_max, n_pad;
  float rope_base;
  float scale;                    // log2(e) / sqrt(d_h), folded into q'
  const int32_t* n_tok;
  const int32_t* bt;
  const void* pages;
  const void* q;
  const void* k;
  const void* v;
  const void* A;                  // [H][d_h][r_k]
  const void* Bm;                 // [H][d_h][r_v]
  void* out;
  // workspace regions (bf16 unless noted)
  void* sk;                       // [B][n_pad][G][r_k]  latents some position reads, token-major
  void* sv;                       // [B][n_pad][G][r_v]
  void* rtab;                     // [n_pad][d_h/2] (cos, sin) of position i, frequency f (fp32 pairs)
  void* kh;                       // [B][n_pad][H][d_h]  rebuilt keys
  void* vh;                       // [B][n_pad][H][d_h]  rebuilt values
};
constexpr int kParQueryTile = 256;   // positions per attention workgroup (n_pad multiple)
// events: optional pair recorded around the attention kernel
hipError_t launch_parallel(const ParParams& p, hipStream_t s, hipEvent_t* events);

// C[m][n] = sum_k X[m][k] Y[n][k] on hipBLASLt (X, Y bf16 row-major, leading
// dims ldx, ldy; C fp32 or bf16, leading dim ldc), K made of nseg segments of
// kseg elements, segment t at X + t sxk and Y + t syk (elements), summed into
// C.  Returns false when the library does not take the shape or its setup
// would fall inside a graph capture (then nothing was launched), or when a
// launch failed; the caller then runs its own GEMM, which writes all of C.
bool lt_gemm_nt(const void* X, const void* Y, void* C, bool c_f32, int64_t M, int64_t N, int64_t kseg, int nseg,
                int64_t ldx, int64_t ldy, int64_t ldc, int64_t sxk, int64_t syk, hipStream_t s);

hipError_t launch_qmap(const DecodeParams& p, bool want_qlat, hipStream_t s);
hipError_t launch_window(const DecodeParams& p, hipStream_t s);
hipError_t launch_scan_absorbed_generic(const DecodeParams& p, hipStream_t s);
hipError_t launch_scan_reconstruct_generic(const DecodeParams& p, hipStream_t s);
hipError_t launch_combine(const DecodeParams& p, hipStream_t s);

// matrix-core kernels (bf16 only); return hipErrorNotSupported for shapes
// they do not cover, before launching anything
bool scan_absorbed_mfma_supports(const DecodeParams& p);
hipError_t launch_scan_absorbed_mfma(const DecodeParams& p, hipStream_t s);

// two passes (scores, then values) for a wide latent shared by all heads
// (G = 1, up to 64 heads, r_k % 32 == 0, r_v % 16 == 0); needs lcap, wscore
// and wprob, with every latent token of every sequence below lcap
constexpr int kWideMaxPages = 8192;       // block-table row length it stages in LDS
bool scan_absorbed_wide_supports(const DecodeParams& p);
int scan_absorbed_wide_slabs(int rv);      // value-pass workgroups per (split, sequence)
int scan_absorbed_wide_lcap(int max_pos);  // score row length covering positions <= max_pos
int scan_absorbed_wide_ksplit(int B, int lcap, int rk);   // score-pass parts of r_k (small batches)
hipError_t launch_scan_absorbed_wide(const DecodeParams& p, hipStream_t s);
// query map and combine of the wide absorbed read: every sequence of a head
// in one workgroup (d_h 64, 96 or 128, bf16)
bool maps_wide_supports(const DecodeParams& p);
hipError_t launch_qmap_wide(const DecodeParams& p, hipStream_t s);
hipError_t launch_combine_wide(const DecodeParams& p, hipStream_t s);

bool scan_reconstruct_mfma_supports(const DecodeParams& p);
hipError_t launch_scan_reconstruct_mfma(const DecodeParams& p, hipStream_t s);

bool scan_reconstruct_gemm_supports(const DecodeParams& p);
bool scan_reconstruct_gemm_tiles_decoders(int dh, int G, int rk, int rv, int bf16);   // needs DecodeParams::dect
int scan_reconstruct_gemm_tile(int dh);   // tokens per workgroup tile (split granularity)
hipError_t launch_scan_reconstruct_gemm(const DecodeParams& p, hipStream_t s);
// regroups the decoders into DecodeParams::dect when the scan will read them from there
hipError_t launch_scan_reconstruct_gemm_prep(const DecodeParams& p, hipStream_t s);

constexpr int kMaxFusedSplits = 1024;   // context splits per (sequence, head) of the fused path
bool fused_decode_supports(const DecodeParams& p);
int fused_partial_floats(int rk, int dh);
hipError_t launch_fused_decode(const DecodeParams& p, hipStream_t s);

bool qmap_mfma_supports(const DecodeParams& p);
hipError_t launch_qmap_mfma(const DecodeParams& p, bool want_qlat, hipStream_t s);
bool window_fast_supports(const DecodeParams& p);
hipError_t launch_window_fast(const DecodeParams& p, hipStream_t s);
// a launch of at least this many workgroups keeps every CU of MI355X busy;
// the latent scans then load their tiles as streaming (load_once)
constexpr int kStreamWorkgroups = 256;
constexpr int kCombineMaxParts = 160;   // splits + window slices the matrix-core combine merges
bool combine_mfma_supports(const DecodeParams& p);
hipError_t launch_combine_mfma(const DecodeParams& p, hipStream_t s);

hipError_t launch_writer_generic(const WriterParams& p, hipStream_t s);
bool writer_mfma_supports(const WriterParams& p);
int writer_mfma_ksplit(int M, int G, int R, int n_loops, int d_in);
hipError_t launch_writer_mfma(const WriterParams& p, hipStream_t s);

}  // namespace lla
