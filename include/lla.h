/*
 * lla.h -- C ABI of the MI355X (gfx950) decode-attention library for looped
 * Transformers whose per-loop KV cache is replaced by cross-loop latents:
 * Looped Latent Attention (LLA: reconstruct keys/values on read; LLA-D: read
 * latents directly) and Hybrid Latent Attention (HLA: direct latent read plus
 * an exact window of recent tokens).
 *
 * Sources (cited by page title and section / equation):
 *   [HLA]   "Hybrid Latent Attention" summary, picx.dev/p/a0K1YZ -- sections
 *           "Latent Writer" (Eq. 2), "Latent Reader" (Eqs. 3 and 4), "Rotary
 *           Embedding Alignment", "Key Insight", "Key Problem".
 *   [LLA-A] "Looped Latent Attention: Cross-Loop Key-Value Compression For
 *           Looped Transformers", abstract (acceptodds.com/papers/iclr2027-34396).
 *   [LLA-S] "Looped Latent Attention: Cross-Loop KV Compression for Looped
 *           Transformers", abstract (searcharxiv.org/abs/2607.15456).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless marked (host).  Every device buffer
 *     is owned by the caller; the library never allocates, frees or keeps a
 *     pointer after it returns, and never synchronises the stream.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream); buffers
 *     must stay alive until the stream has passed the call.
 *   - Arguments are validated on the host before anything is enqueued: an
 *     error status means nothing was launched and no buffer was touched.
 *     LLA_ERR_HIP means a launch failed; the store, ring or output may then
 *     be partly written.
 *   - Device-resident indices (positions, block tables) are not validated on
 *     the host; out-of-range values are undefined behaviour.
 *   - Every device pointer must be 16-byte aligned.
 *   - dtype LLA_BF16: latents, activations, maps, ring and outputs are bf16,
 *     arithmetic is fp32 with fp32 accumulation (roundings to bf16 are
 *     round-to-nearest-even).  LLA_F32: everything fp32.
 *   - Rotary embedding: pairs (f, f + d_h/2) of a head vector rotate by
 *     angle p*theta_f, theta_f = rope_base^(-2f/d_h), p the 0-based absolute
 *     position; in a key latent of m = r_k/d_h blocks every block rotates the
 *     same way (R~_p = I_m (x) R_p, [HLA] "Rotary Embedding Alignment").
 *     rope_base == 0 disables it.
 *   - The library is re-entrant and holds no state, except the per-GPU
 *     scratch array of hla_decode_windowed_noalloc.  Calls that share a
 *     workspace, store or ring must be ordered on one stream by the caller.
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLA_ABI_VERSION 5   /* 2: value decoder passed as B_t^T [H][d_h][r_v]; 3: latent_fp8;
                                4: parallel attention over whole sequences;
                                5: lla_decode_scan_kernel_for_store, lla_check_indices,
                                hla_decode_windowed_noalloc */

typedef void* lla_stream_t; /* a hipStream_t */

typedef enum {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARGUMENT = 1,
  LLA_ERR_UNSUPPORTED = 2,
  LLA_ERR_WORKSPACE_TOO_SMALL = 3,
  LLA_ERR_HIP = 4
} lla_status;

typedef enum { LLA_F32 = 0, LLA_BF16 = 1 } lla_dtype;

/* Decode flags (lla_decode_args.flags). */
#define LLA_FLAG_GENERIC 1 /* use the general VALU kernels even where a
                              matrix-core kernel exists (testing, tuning) */
#define LLA_FLAG_FUSED 2   /* absorbed / HLA reads: the query map, latent
                              scan, exact window and value map in one kernel
                              (workgroup per (split, head, sequence)) behind a
                              one-line ticket reset, instead of three kernels;
                              for small batch x context, where a call is bound
                              by fixed latency rather than bytes.
                              LLA_ERR_UNSUPPORTED where it does not apply
                              (reconstruct entry, fp32 or fp8 sets, r_k != r_v,
                              r not in {128, 256, 512, 1024}, d_h not in
                              {64, 128}); not combinable with LLA_FLAG_GENERIC */

/*
 * One latent set of one layer (host struct).  A set serves loops
 * loop_first..loop_last: HLA has a loop-1 set {1,1} and a main set {2,T}
 * ([HLA] "Latent Writer", Eq. 2); LLA has one set {1,T} ([LLA-A]).
 *   n_heads, head_dim   H, d_h of the attention that reads the set
 *   groups              G latents per token: 1 = shared by all heads (HLA,
 *                       LLA-2D), H = one per head (per-head LLA); head h
 *                       reads group h / (H/G).  H % G == 0.
 *   r_k, r_v            key / value latent width per group; multiples of 16
 *   page_size           tokens per store page; a multiple of 16
 *   rope_baked          1: key latents are stored rotated, R~_p c^K
 *                       (needs r_k % head_dim == 0 and rope_base > 0)
 *   rope_base           0 = no rotary embedding
 *   dtype               storage and map dtype
 *   latent_fp8          1: the latents are stored as OCP e4m3 codes with one
 *                       fp32 scale per token, group and part (key, value):
 *                       element = code value x scale, scale = max|x| / 448 of
 *                       the part ([HLA] "Summary (Overview)": the codec
 *                       combines with quantization).  Needs dtype == LLA_BF16
 *                       (maps, ring and activations stay bf16) and r_k, r_v
 *                       multiples of 64; the absorbed / HLA entry points read
 *                       it, lla_decode_reconstruct returns UNSUPPORTED.
 */
typedef struct {
  int32_t n_heads, head_dim;
  int32_t groups;
  int32_t r_k, r_v;
  int32_t loop_first, loop_last;
  int32_t page_size;
  int32_t rope_baked;
  float rope_base;
  lla_dtype dtype;
  int32_t latent_fp8;
} lla_set_desc;

/*
 * Paged latent store of one set of one layer.
 *   pages        [n_pages][G][P/16 tiles][tile], one tile = 16 tokens:
 *                  16 key rows of r_k numbers (token-major), then
 *                  r_v/16 value sub-blocks of 16 dims x 16 tokens, each
 *                  stored dimension-major (16 tokens of one dim contiguous).
 *                Element offset of key dim d of slot u, group g, page pg:
 *                  ((pg*G + g)*P + (u/16)*16)*(r_k+r_v) + (u%16)*r_k + d
 *                for r_k <= 512; key rows wider than 512 numbers are
 *                chunk-major (chunk c = dims 32c .. 32c+31, the last one
 *                w_c = min(32, r_k - 32c) wide, holds the 16 tokens' pieces
 *                in turn), key dim d then at
 *                  ((pg*G + g)*P + (u/16)*16)*(r_k+r_v) + 512*(d/32)
 *                    + (u%16)*w_(d/32) + d%32
 *                (fp8 stores keep token-major key rows at every width);
 *                and of value dim d:
 *                  ((pg*G + g)*P + (u/16)*16)*(r_k+r_v) + 16*r_k
 *                    + (d/16)*256 + (d%16)*16 + u%16
 *                With latent_fp8 the store is bytes: a tile is
 *                  TB = 16*(r_k+r_v) + 128 bytes, tile base
 *                  T = ((pg*G + g)*(P/16) + u/16)*TB; key code of dim d at
 *                  T + (u%16)*r_k + d; value code of dim d at
 *                  T + 16*r_k + (d/64)*1024 + (d%16)*64 + ((u%16)/4)*16
 *                    + ((d/16)%4)*4 + u%4;
 *                  fp32 key scale at T + 16*(r_k+r_v) + (u%16)*4 and value
 *                  scale 64 bytes further.
 *   block_table  [batch][max_pages_per_seq] physical page of logical page
 *                p/P of each sequence (host-side: only its shape is used)
 */
typedef struct {
  void* pages;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
} lla_store;

/*
 * Latent writer, [HLA] "Latent Writer" Eq. 2: for every token (b, n) at
 * position p = pos[b*n_tok + n] and every group g,
 *     c = sum over the set's loops t of E_t x_t      (fp32 accumulation)
 * the key part is replaced by R~_p c^K when rope_baked, the result is
 * rounded to the storage dtype and written to page block_table[b][p/P],
 * slot p % P.
 *   x     [batch][n_tok][n_loops][G][d_in]   per-loop inputs h_{j,t}
 *   enc   [n_loops][G][r_k + r_v][d_in]      encoders E_t, c = E_t x
 *   workspace  scratch of lla_write_workspace_bytes() bytes (may be NULL
 *              when that is 0)
 * Errors: INVALID_ARGUMENT (null pointer, bad sizes, misalignment),
 * UNSUPPORTED (rope_baked with r_k % head_dim != 0), WORKSPACE_TOO_SMALL.
 */
lla_status lla_write_latents(const lla_set_desc* desc, const lla_store* store,
                             int32_t batch, int32_t n_tok, const int32_t* pos,
                             const void* x, int32_t d_in, const void* enc,
                             void* workspace, size_t workspace_bytes,
                             lla_stream_t stream);
size_t lla_write_workspace_bytes(const lla_set_desc* desc, int32_t batch,
                                 int32_t n_tok, int32_t d_in);

/*
 * Arguments of one decode call: one layer, one loop t, every sequence b at
 * its current position i = pos[b] (N = i + 1 tokens attended).  Tokens
 * j < i - W are read from the latent store, tokens i-W <= j < i from the
 * exact ring, and the current token from k_cur / v_cur; one softmax spans
 * all of them ([HLA] "Latent Reader", Eq. 4).  Scores are scaled by
 * 1/sqrt(d_h) (Eq. 3).
 *   loop          t, in [loop_first, loop_last] of the set
 *   window        W >= 0; the ring has W+1 slots
 *   max_pos_hint  (host) an upper bound of pos[], used only to plan the
 *                 context split; a larger pos[] stays correct
 *   splits        0 = plan automatically; > 0 forces the number of context
 *                 splits (results then are bitwise reproducible)
 *   flags         LLA_FLAG_* bits
 *   pos           [batch] int32 current positions
 *   q, k_cur, v_cur  [batch][H][d_h]: this loop's query, key (both before
 *                 rotation) and value of the current token
 *   ring_k, ring_v   [batch][W+1][H][d_h]: slot j mod (W+1) holds the
 *                 rotated key / the value of exact token j.  The call writes
 *                 slot i mod (W+1) with R_i k_cur and v_cur (that slot's old
 *                 token, i-W-1, is a latent token from now on).
 *   A             [H][d_h][r_k]  key decoder A_t of this loop (per head)
 *   B             [H][d_h][r_v]  value decoder stored transposed, B_t^T
 *                 (v = B_t^T c^V), the same orientation as A: rows
 *                 contiguous along the latent axis
 *   out           [batch][H][d_h]
 *   workspace     scratch of lla_decode_workspace_bytes() bytes; contents
 *                 on entry are irrelevant
 *   scan_events   optional (host) array of two hipEvent_t, recorded on
 *                 `stream` right before and right after the latent-scan
 *                 kernel (profiling); NULL = none
 */
typedef struct {
  int32_t loop;
  int32_t window;
  int32_t max_pos_hint;
  int32_t splits;
  int32_t flags;
  const int32_t* pos;
  const void* q;
  const void* k_cur;
  const void* v_cur;
  void* ring_k;
  void* ring_v;
  const void* A;
  const void* B;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  void* scan_events;
} lla_decode_args;

/*
 * Reconstruct-on-read (LLA, [LLA-A] / [LLA-S]: the codec rebuilds a loop's
 * keys and values from the latents at the moment attention reads them, and
 * keeps only the latents): every latent token's key
 * k_j = A^(h) sK_j and value v_j = B^(h)T sV_j are rebuilt, then ordinary
 * attention with q' = R_i q runs over latent, window and current tokens.
 * With a baked store, A^(h) sK_j is the rotated key when A_t is
 * frequency-paired.  UNSUPPORTED when rope_base > 0 and rope_baked == 0.
 */
lla_status lla_decode_reconstruct(const lla_set_desc* desc, const lla_store* store,
                                  int32_t batch, const lla_decode_args* args,
                                  lla_stream_t stream);

/*
 * Absorbed read (LLA-D, [LLA-A]: attention reads the latents directly, with
 * no rebuilt keys or values;
 * [HLA] Eqs. 3-4): q~ = R~_i A_t^T q, latent scores q~ . sK_j / sqrt(d_h),
 * o = B_t^T sum_lat a_j sV_j + sum_exact a_j v_j.  Any G.  Needs
 * rope_baked == 1 or rope_base == 0 (else UNSUPPORTED).
 */
lla_status lla_decode_absorbed(const lla_set_desc* desc, const lla_store* store,
                               int32_t batch, const lla_decode_args* args,
                               lla_stream_t stream);

/*
 * Hybrid Latent Attention decode ([HLA] Eqs. 3-4 with the exact window of
 * "Key Insight"): the absorbed read on an HLA set (G == 1).  Pass the loop-1
 * set and its maps for t = 1 and the main set for t >= 2.
 */
lla_status hla_decode_windowed(const lla_set_desc* desc, const lla_store* store,
                               int32_t batch, const lla_decode_args* args,
                               lla_stream_t stream);

/*
 * hla_decode_windowed without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace lives in a file-scope
 * device array of LLA_NOALLOC_SCRATCH_BYTES per GPU, which the library holds
 * until the process ends; its address is looked up on the first call on
 * each device.  The call allocates nothing.
 *   args->workspace must be NULL and args->workspace_bytes 0 (else
 *   INVALID_ARGUMENT); WORKSPACE_TOO_SMALL when lla_decode_workspace_bytes()
 *   for these sizes exceeds LLA_NOALLOC_SCRATCH_BYTES (32 MiB: the HLA sets of
 *   the Ouro-1.4B shape need 16.1 MiB at batch 128 and 4k context); LLA_ERR_HIP
 *   when the array's address cannot be looked up; otherwise as
 *   hla_decode_windowed.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads
 * without ordering) race.
 */
#define LLA_NOALLOC_SCRATCH_BYTES (32u << 20)
lla_status hla_decode_windowed_noalloc(const lla_set_desc* desc, const lla_store* store,
                                       int32_t batch, const lla_decode_args* args,
                                       lla_stream_t stream);

/* Workspace bytes any decode entry point needs for these sizes (splits as
 * in lla_decode_args; 0 = automatic).  For bf16 sets with one latent shared
 * by all heads (groups == 1, r_k == r_v, d_h 64 or 96) it includes a copy of
 * A_t and B_t^T regrouped per 32 latent dims (2 H d_h r_k bf16), which the
 * reconstruct read refills on every call.  For bf16 sets whose absorbed read
 * takes the two-pass scan ("k_scan_absorbed_wide" below) it also includes a
 * bf16 probability per (sequence, head, latent token) and an fp32 score per
 * (part of r_k, sequence, head, latent token), for tokens up to max_pos + 1
 * rounded up to 512: (4 parts + 2) batch H L bytes, with one part at large
 * batches and up to r_k / 128 at small ones.  A decode
 * call uses that scan only when the store cannot hold more tokens than these
 * rows cover (max_pages_per_seq * page_size <= L with L from max_pos_hint);
 * otherwise it runs the one-pass general scan, so a larger pos[] stays
 * correct. */
size_t lla_decode_workspace_bytes(const lla_set_desc* desc, int32_t batch,
                                  int32_t max_pos, int32_t window, int32_t splits);

/* Number of context splits the planner uses for these sizes and entry
 * (0 = reconstruct, 1 = absorbed / HLA); 0 on invalid arguments. */
int32_t lla_decode_plan_splits(const lla_set_desc* desc, int32_t batch, int32_t max_pos,
                               int32_t window, int32_t splits, int32_t entry);

/* Name of the latent-scan kernel family a decode call with this set, entry
 * (0 = lla_decode_reconstruct, 1 = lla_decode_absorbed, 2 =
 * hla_decode_windowed) and flags launches: "k_scan_absorbed_mfma",
 * "k_scan_absorbed_wide" (bf16, one latent shared by up to 64 heads, r_k a
 * multiple of 32, shapes the one-pass matrix-core scan does not take: a
 * score pass, a softmax pass and a value pass, kernels named with this
 * prefix), "k_scan_absorbed_generic", "k_scan_reconstruct_mfma",
 * "k_scan_reconstruct_gemm" or "k_scan_reconstruct_generic" (static
 * strings, for profilers).  The name assumes a store whose block table fits
 * the matrix-core scans' page tables (at most 8192 columns for
 * "k_scan_absorbed_mfma" and "k_scan_absorbed_wide", 4096 for
 * "k_scan_reconstruct_mfma"); lla_decode_scan_kernel_for_store answers for a
 * given store.  NULL on invalid arguments.  Host only. */
const char* lla_decode_scan_kernel(const lla_set_desc* desc, int32_t entry, int32_t flags);

/* The latent-scan kernel family a decode call launches on a store whose
 * block table has max_pages_per_seq columns, with this max_pos_hint: as
 * lla_decode_scan_kernel, except that a table longer than a matrix-core
 * scan's page table, or (for "k_scan_absorbed_wide") a store holding more
 * tokens per sequence than the score rows planned from max_pos_hint cover,
 * names the general scan ("k_scan_absorbed_generic" /
 * "k_scan_reconstruct_generic"), which the call then runs.  NULL on invalid
 * arguments (max_pos_hint < 0, max_pages_per_seq <= 0).  Host only. */
const char* lla_decode_scan_kernel_for_store(const lla_set_desc* desc, int32_t entry, int32_t flags,
                                             int32_t max_pos_hint, int32_t max_pages_per_seq);

/*
 * Host-side check of the device-resident indices a decode or write call will
 * use, on host copies (pos_host, block_table_host).  Kernels do not check
 * these (out-of-range values there are undefined behaviour); a caller that
 * wants the check runs this on copies before enqueuing, and no debug build of
 * the kernels exists.  For every sequence b < batch: pos_host[b] >= 0 and
 * pos_host[b] < max_pages_per_seq * page_size (the page of the current
 * position exists), and every block-table entry of logical pages 0 ..
 * pos_host[b] / page_size lies in [0, n_pages).  Returns LLA_OK or
 * LLA_ERR_INVALID_ARGUMENT; never touches the GPU.
 *   pos_host          (host) [batch] positions (decode: i; writer: any token's)
 *   block_table_host  (host) [batch][max_pages_per_seq]
 *   n_pages           pages in the store
 */
lla_status lla_check_indices(const int32_t* pos_host, int32_t batch, const int32_t* block_table_host,
                             int32_t max_pages_per_seq, int32_t page_size, int32_t n_pages);

/* Bytes one set stores per token (all groups): G*(r_k + r_v)*sizeof(dtype)
 * ([HLA] "Latent Writer": r_k + r_v (+ 2 r_1) numbers per token per layer).
 * 0 on an invalid descriptor. */
size_t lla_bytes_per_token(const lla_set_desc* desc);

const char* lla_status_string(lla_status status);
int32_t lla_abi_version(void);

/*
 * ---------------------------------------------------------------------------
 * Uncompressed (full-cache) looped decode: the baseline the codec replaces.
 * Every loop keeps exact keys and values of every token ([HLA] "Key
 * Problem": 2 T d numbers per token per layer, 768 KiB per token on the
 * Ouro-1.4B shape in bf16), paged like the latent store.
 * ---------------------------------------------------------------------------
 *   n_heads, head_dim   H, d_h (d_h in {64, 128})
 *   page_size           P tokens per page, a positive multiple of 8
 *   rope_base           0 = no rotary embedding; keys are stored rotated
 *   dtype               storage dtype of the cache and the activations
 */
typedef struct {
  int32_t n_heads;
  int32_t head_dim;
  int32_t page_size;
  float rope_base;
  lla_dtype dtype;
} lla_kv_desc;

/* Exact cache of one (layer, loop): token j of sequence b lives in page
 * block_table[b][j / P], slot j % P; a page is [P][H][d_h] (all heads of a
 * token contiguous), keys post-rotation.  Device pointers, 16-byte aligned. */
typedef struct {
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;   /* [batch][max_pages_per_seq] */
  int32_t max_pages_per_seq;
} lla_kv_cache;

/*   max_pos_hint, splits, scan_events   as in lla_decode_args
 *   flags         must be 0
 *   pos           [batch] current positions i (tokens 0..i-1 are cached)
 *   q, k_cur, v_cur  [batch][H][d_h], q and k_cur before rotation
 *   out           [batch][H][d_h]
 *   workspace     lla_full_decode_workspace_bytes() bytes, contents irrelevant */
typedef struct {
  int32_t max_pos_hint;
  int32_t splits;
  int32_t flags;
  const int32_t* pos;
  const void* q;
  const void* k_cur;
  const void* v_cur;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  void* scan_events;
} lla_full_decode_args;

/*
 * One decode call of the uncompressed model for one (layer, loop): writes
 * R_i k_cur and v_cur at position i of the cache, then
 * o = softmax(q' K^T / sqrt(d_h)) V over tokens 0..i with q' = R_i q.
 * Errors as for the latent entry points (validation before any launch).
 */
lla_status lla_decode_full_cache(const lla_kv_desc* desc, const lla_kv_cache* cache,
                                 int32_t batch, const lla_full_decode_args* args,
                                 lla_stream_t stream);

/* Workspace bytes lla_decode_full_cache needs (splits 0 = automatic); 0 on
 * invalid arguments. */
size_t lla_full_decode_workspace_bytes(const lla_kv_desc* desc, int32_t batch,
                                       int32_t max_pos, int32_t splits);

/* Context splits the planner uses for a full-cache decode; 0 on invalid
 * arguments. */
int32_t lla_full_decode_plan_splits(const lla_kv_desc* desc, int32_t batch, int32_t max_pos,
                                    int32_t splits);

/*
 * ---------------------------------------------------------------------------
 * Parallel HLA attention over whole sequences: the second pass of the
 * two-pass procedure ([HLA] "Training Procedure": a first pass writes every
 * token's latents -- lla_write_latents over the whole sequence -- and the
 * second runs HLA attention at all positions at once).  Position i of
 * sequence b gets Eq. 4 as a decode call at position i would, with the exact
 * part taken from this loop's k, v of positions max(0, i-W) .. i:
 *   o_i = B_t^T sum_{j < i-W} a_ij s^V_j + sum_{max(0,i-W) <= j <= i} a_ij v_j,
 * latent scores from Eq. 3, exact scores (R_i q_i).(R_j k_j) / sqrt(d_h), one
 * softmax per (position, head).
 * The library rebuilds keys and values once per latent token
 * (A_t s^K_j, B_t^T s^V_j) and attends in head space: with many queries per
 * latent token that takes (r_k + r_v) / (2 d_h) times fewer products than
 * scoring every query in latent space.  It equals Eq. 3 when A_t commutes
 * with the rotation (frequency-paired decoders, [HLA] "Rotary Embedding
 * Alignment") or when rope_base = 0 -- the same condition as
 * lla_decode_reconstruct.
 * ---------------------------------------------------------------------------
 *   loop, window   t in [loop_first, loop_last]; W >= 0
 *   n_max          positions per sequence in q, k, v and out (>= 1)
 *   flags          must be 0
 *   n_tok          [batch] (device) sequence lengths, 0 <= n_tok[b] <= n_max;
 *                  positions 0 .. n_tok[b]-1.  Only latents of tokens
 *                  j < n_tok[b] - 1 - W are read (the store must hold them);
 *                  values outside 0..n_max are undefined behaviour
 *   q, k, v        [batch][n_max][H][d_h], q and k before rotation; rows at
 *                  or past n_tok[b] are never read
 *   A, B           key decoder A_t [H][d_h][r_k], value decoder B_t^T
 *                  [H][d_h][r_v], as for the decode entry points
 *   out            [batch][n_max][H][d_h]; rows at or past n_tok[b] are left
 *                  untouched
 *   workspace      lla_parallel_workspace_bytes() bytes, contents irrelevant
 *   attn_events    optional (host) array of two hipEvent_t, recorded on the
 *                  stream right before and after the attention kernel (for
 *                  timing); NULL for none
 * Supported: bf16 sets with latent_fp8 = 0, d_h in {64, 128}, r_k and r_v
 * multiples of 32, rope_base = 0 or rope_baked = 1; other valid sets return
 * LLA_ERR_UNSUPPORTED.  The block table must cover max(0, n_max - 1 - W)
 * tokens (max_pages_per_seq * page_size).  Pointers 16-byte aligned.  Errors
 * as for the decode entry points (validation before any launch).
 */
typedef struct {
  int32_t loop;
  int32_t window;
  int32_t n_max;
  int32_t flags;
  const int32_t* n_tok;
  const void* q;
  const void* k;
  const void* v;
  const void* A;
  const void* B;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  void* attn_events;
} lla_parallel_args;

lla_status hla_attention_parallel(const lla_set_desc* desc, const lla_store* store, int32_t batch,
                                  const lla_parallel_args* args, lla_stream_t stream);

/* Workspace bytes hla_attention_parallel needs; 0 on invalid arguments. */
size_t lla_parallel_workspace_bytes(const lla_set_desc* desc, int32_t batch, int32_t n_max);

#ifdef __cplusplus
}
#endif
#endif /* LLA_H */
