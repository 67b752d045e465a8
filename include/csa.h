/*
 * csa.h -- C ABI of libcsa, the gfx950 (MI355X) Compressed Sparse Attention path.
 *
 * The operations follow the equations of DeepSeek-V4's compressed attention as
 * summarised on the "Evidence Ledger" page (mailtotanvir,
 * mastering-deepseek-v4-architecture: CSA bullets = Section 2.3.1, Eqs 9-19;
 * HCA = Section 2.3.2, Eqs 20-26; shared details = Section 2.3.3, Eq 27; mixed
 * storage = Section 2.3.4) and on the "DeepSeek V4 study" page (shuhuayu,
 * section 03 "Two resolutions of history", section 06 cache ledger).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises, and keeps no state between calls.
 *  - Every call is asynchronous on `stream` (0 = the null stream).
 *  - Layouts are dense row-major in the order the shapes are written.
 *  - Sequences in a batch are independent (no packing): each has its own
 *    query positions and entry count.
 *  - All argument checks run on the host before anything is launched; a bad
 *    argument returns CSA_ERR_INVALID and launches nothing.  A dtype pairing the
 *    library has no kernel for returns CSA_ERR_UNSUPPORTED.  A launch failure
 *    returns CSA_ERR_LAUNCH.  No C++ exception crosses this boundary.
 *  - Workspace protocol (calls that take `ws`): with ws_bytes != NULL and
 *    ws == NULL the call writes the bytes it needs to *ws_bytes and returns
 *    CSA_OK without launching; with both non-NULL, *ws_bytes is the size of
 *    `ws` and must be at least that much (else CSA_ERR_WORKSPACE); with
 *    ws_bytes == NULL the caller offers no workspace, which is accepted when
 *    the call needs none and is CSA_ERR_WORKSPACE otherwise.  The size depends
 *    only on the host arguments.
 *  - Positions are zero-based.  A query at position q sees the compressed
 *    entries s < N(q) = min(n_entries, (q + 1) / m): an entry is visible once
 *    its whole block has been processed (strict block causality).
 *  - Outputs are bitwise reproducible run to run.  The split of long entry
 *    lists into partial softmaxes depends only on host sizes, never on the
 *    batch size, and partials are merged in a fixed order.
 *
 * Row formats (csa_dtype)
 * -----------------------
 *  CSA_F32     c fp32 values.
 *  CSA_BF16    c bf16 values (round-to-nearest-even when produced here).
 *  CSA_FP8MIX  KV rows only: (c - rope_dims) OCP e4m3 bytes (no scale,
 *              saturating at +-448) followed by rope_dims bf16 values; 576 B
 *              for c = 512, rope_dims = 64 (Evidence Ledger 2.3.4: BF16 RoPE
 *              dims, FP8 elsewhere).
 *  CSA_MXFP4   c/2 bytes of E2M1 pairs per row (element 2j in the low nibble of
 *              byte j) plus a separate scale array of c/32 e8m0 bytes per row,
 *              scale = 2^(floor(log2 max|x|) - 2) over each block of 32 (OCP MX;
 *              Evidence Ledger Section 5.2.1: MXFP4 in 1x32 tiles).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID = 1,
  CSA_ERR_UNSUPPORTED = 2,
  CSA_ERR_WORKSPACE = 3,
  CSA_ERR_LAUNCH = 4,
  /* range markers, never returned: every int is a value of the type, so
   * csa_status_string takes any code */
  CSA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  CSA_STATUS_RANGE_MAX_ = 2147483647
} csa_status;

typedef enum csa_dtype {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8MIX = 2,
  CSA_MXFP4 = 3,
  /* range markers, not formats: they make every int a value of the type, so
   * an unknown code passed across the ABI is rejected (CSA_ERR_UNSUPPORTED)
   * rather than being an out-of-range enum inside the library */
  CSA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  CSA_DTYPE_RANGE_MAX_ = 2147483647
} csa_dtype;

/* Library version string (static storage). */
const char* csa_version(void);

/* Human-readable name of a status code (static storage). */
const char* csa_status_string(csa_status s);

/*
 * csa_prep_rows -- RMSNorm, partial RoPE and storage-format encoding of rows.
 *
 * Evidence Ledger Section 2.3.3: RMSNorm is applied to every compressed KV
 * entry just before core attention and partial RoPE to its last 64 dims;
 * Section 2.3.4 / shuhuayu section 06: entries are stored FP8 + BF16 and index
 * keys in FP4.  This is the last stage of the compressor, exposed on its own so
 * that caches and window rows can be (re)encoded:
 *
 *   y_r = x_r                                   if norm_w == NULL
 *       = x_r / sqrt(mean(x_r^2) + eps) * norm_w  otherwise
 *   then the pairs (c - rope_dims + 2u, c - rope_dims + 2u + 1) are rotated by
 *   angle pos_r * rope_theta^(-2u / rope_dims)   (skipped if rope_dims == 0),
 *   then y_r is stored in out_t.
 *
 *  x        [rows, c] in x_t (CSA_F32 or CSA_BF16).
 *  rows     number of rows (>= 0; 0 launches nothing).
 *  c        row length; multiple of 32 for CSA_MXFP4, even, <= 4096.
 *  norm_w   [c] fp32 gains or NULL.
 *  pos      [rows] int32 positions, or NULL: then pos_r = pos_offset +
 *           pos_stride * (r % rows_per_seq)  (rows_per_seq >= 1).
 *  out      [rows, row bytes of out_t]; out_scale [rows, c/32] e8m0 bytes,
 *           required iff out_t == CSA_MXFP4 (else ignored).
 *  rope_dims even, 0 <= rope_dims <= c; CSA_FP8MIX requires rope_dims > 0.
 */
csa_status csa_prep_rows(const void* x, csa_dtype x_t, int64_t rows, int c,
                         const float* norm_w, float eps, int rope_dims, float rope_theta,
                         const int32_t* pos, int rows_per_seq, int pos_stride, int pos_offset,
                         void* out, uint8_t* out_scale, csa_dtype out_t, hipStream_t stream);

/*
 * csa_compress -- token compression into KV entries (Evidence Ledger Eqs 9-12
 * for CSA, Eqs 20-26 for HCA; shuhuayu section 03).
 *
 *   C^a = H W_kv_a, Z^a = H W_z_a, C^b = H W_kv_b, Z^b = H W_z_b      (Eqs 9-10)
 *   entry i, channel j: softmax over the candidates r of
 *       Z^a[m i + u, j] + bias_a[u, j]          (own block, u = 0..m-1)
 *       Z^b[m (i-1) + u, j] + bias_b[u, j]      (preceding block; overlap only,
 *                                                absent for entry 0)
 *   E_i[j] = sum_r softmax_r * C^{series}[pos_r, j]                    (Eqs 11-12)
 *   then RMSNorm(norm_w, eps) and partial RoPE at position
 *   pos_stride * i + pos_offset, exactly as csa_prep_rows, stored in out_t.
 *
 *  H       [B, T, d] in h_t (CSA_F32 or CSA_BF16); weights [d, c] in h_t.
 *  W_kv_b / W_z_b / bias_b: required iff overlap != 0 (CSA, m = 4), else NULL.
 *  W_z_a / bias_a may be NULL only for m == 1 without overlap: one candidate,
 *          so E_i = C^a row i (the per-token window projection).
 *  bias_*  [m, c] fp32.
 *  norm_w  [c] fp32 or NULL (no RMSNorm; index keys use NULL and rope_dims 0).
 *  out     [B, T / m, row bytes of out_t] (+ out_scale [B, T/m, c/32] for MXFP4).
 *          Tokens beyond the last complete block are not compressed.
 *  ws      fp32 projection scratch (see the workspace protocol above); with bf16
 *          H, d a multiple of 64 and B * T >= 256 it also holds the projection
 *          weights transposed to [c, d] (bf16).
 */
csa_status csa_compress(const void* H, csa_dtype h_t, int B, int T, int d,
                        const void* W_kv_a, const void* W_z_a,
                        const void* W_kv_b, const void* W_z_b,
                        const float* bias_a, const float* bias_b, int m, int overlap, int c,
                        const float* norm_w, float eps, int rope_dims, float rope_theta,
                        int pos_stride, int pos_offset,
                        void* out, uint8_t* out_scale, csa_dtype out_t,
                        void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * csa_compress_append -- decode-time compression: the one new entry of each
 * sequence whose latest block has just completed (Evidence Ledger Eqs 9-12,
 * 20-26; the entry is formed exactly as csa_compress forms entry i, from the
 * same candidates and in the same order, so the appended row equals the full
 * pass's row i bit for bit).
 *
 *  H        [B, Tt, d] h_t: per sequence the tail of hidden states, Tt = 2m with
 *           overlap (block i-1, then block i) or m without (block i).  For i = 0
 *           the preceding-block rows are present but unused.
 *  W_*, bias_*, m, overlap, c, norm_w, eps, rope_*, pos_stride, pos_offset:
 *           as csa_compress (W_z_a and bias_a required).
 *  entry    [B] int32 (device): the index i of the entry each sequence completes;
 *           a sequence with i outside [0, Nmax) is skipped.
 *  cache    [B, Nmax, row] in out_t; row entry[b] of sequence b is written,
 *           nothing else.  cache_scale [B, Nmax, c/32] for CSA_MXFP4.
 *  ws       fp32 projections of the tails: query with ws == NULL.
 * Errors as csa_compress; asynchronous on `stream`.
 */
csa_status csa_compress_append(const void* H, csa_dtype h_t, int B, int d,
                               const void* W_kv_a, const void* W_z_a,
                               const void* W_kv_b, const void* W_z_b,
                               const float* bias_a, const float* bias_b, int m, int overlap,
                               int c, const float* norm_w, float eps, int rope_dims,
                               float rope_theta, int pos_stride, int pos_offset,
                               const int32_t* entry, void* cache, uint8_t* cache_scale,
                               csa_dtype out_t, int Nmax, void* ws, size_t* ws_bytes,
                               hipStream_t stream);

/*
 * indexer_score -- lightning-indexer scores (Evidence Ledger Eqs 13-17;
 * shuhuayu section 03 score formula):
 *
 *   scores[b, t, s] = sum_h w[b, t, h] * max(0, qI[b, t, h, :] . kI[b, s, :])
 *   for s < N(q_pos[b, t]) = min(n_entries[b], (q_pos[b, t] + 1) / m).
 *
 *  One cI-dim key per compressed entry, shared by all nI indexer heads.
 *  qI      [B, Tq, nI, cI] in qI_t; kI [B, Nmax, cI] in kI_t; qI_t == kI_t in
 *          {CSA_F32, CSA_BF16, CSA_MXFP4}.  For CSA_MXFP4 the scale arrays
 *          qI_scale [B, Tq, nI, cI/32] and kI_scale [B, Nmax, cI/32] are
 *          required (else ignored).
 *  w       [B, Tq, nI] fp32.
 *  q_pos   [B, Tq] int32; n_entries [B] int32 with 0 <= n_entries <= Nmax.
 *  scores  [B, Tq, Nmax] in score_t (CSA_F32, or CSA_BF16 rounded RNE from the
 *          fp32 sum).  Entries s >= N(q) are NOT written.
 *  Accumulation is fp32.  The bf16 / MXFP4 products are exact in fp32.
 */
csa_status indexer_score(const void* qI, const uint8_t* qI_scale, csa_dtype qI_t,
                         const float* w,
                         const void* kI, const uint8_t* kI_scale, csa_dtype kI_t,
                         const int32_t* q_pos, const int32_t* n_entries,
                         int B, int Tq, int nI, int cI, int Nmax, int m,
                         void* scores, csa_dtype score_t, hipStream_t stream);

/*
 * topk_select -- top-k over the visible scores (Evidence Ledger Eqs 13-17: the
 * top-k scores choose which compressed blocks the core attention reads).
 *
 *   idx[b, t, :] = the min(k, N(q)) entries with the largest scores among
 *   s < N(q), ties to the LOWER entry index, in ascending entry order, padded
 *   with -1 up to k.
 *
 *  scores  [B, Tq, Nmax] in score_t (CSA_F32 or CSA_BF16); only s < N(q) read.
 *  idx     [B, Tq, k] int32.
 *  ws      int32 scratch for rows of more than 16,384 entries (per-slice
 *          digit histograms, row state and slice counts; workspace protocol
 *          above); size 0 for shorter rows.
 */
csa_status topk_select(const void* scores, csa_dtype score_t,
                       const int32_t* q_pos, const int32_t* n_entries,
                       int B, int Tq, int Nmax, int m, int k, int32_t* idx,
                       void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * sparse_mqa_attend -- CSA core attention (Evidence Ledger Eqs 18-19 and 27,
 * Section 2.3.3; shuhuayu section 03): shared-KV multi-query attention of every
 * query head over the selected compressed entries plus the sliding window, in
 * ONE softmax whose denominator also holds exp(sink[h]).
 *
 *   q_h  = RoPE(RMSNorm(q[b, t, h, :]; q_norm_w, eps), q_pos[b, t])
 *   rows = { kv[b, s] : s in idx[b, t, :], s >= 0 }
 *          U { win[b, p % win_len] : max(0, q - n_win + 1) <= p <= q }
 *   l_x  = scale * q_h . x;   M = max(sink[h], max_x l_x)
 *   o_h  = sum_x exp(l_x - M) x / (exp(sink[h] - M) + sum_x exp(l_x - M))
 *   out[b, t, h, :] = RoPE(o_h, -q)      (each row is both K and V)
 *
 *  q       [B, Tq, nh, c] in q_t (CSA_F32 / CSA_BF16); q_norm_w [c] fp32 or NULL.
 *  kv      [B, Nmax, row] stored entries (already normed and RoPE'd) in kv_t
 *          (CSA_F32, CSA_BF16, CSA_FP8MIX).
 *  idx     [B, Tq, k] int32 (-1 = unused slot; every other value < Nmax).
 *  win     [B, win_len, row] window rows in kv_t, row of position p at slot
 *          p % win_len; win_len >= n_win >= 0 (decode: a ring of 128; prefill:
 *          win_len = T, one row per token).  win may be NULL iff n_win == 0.
 *  sink    [nh] fp32 logits z'_h (not multiplied by scale).
 *  out     [B, Tq, nh, c] in out_t (CSA_F32 / CSA_BF16).
 *  ws      split-softmax partials (workspace protocol above): O / l in bf16 and
 *          (m, l) in fp32 per (query row, split, head); size 0 when the slot
 *          lists are not split (many query rows, or at most 256 slots).
 */
csa_status sparse_mqa_attend(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                             int rope_dims, float rope_theta, const int32_t* q_pos,
                             const void* kv, csa_dtype kv_t, int Nmax,
                             const int32_t* idx, int k,
                             const void* win, int win_len, int n_win,
                             const float* sink, float scale, int B, int Tq, int nh, int c,
                             void* out, csa_dtype out_t,
                             void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * hca_attend -- HCA core attention (Evidence Ledger Section 2.3.2, Eqs 20-26;
 * shuhuayu section 03: each query reads every completed compressed block).
 * Identical to sparse_mqa_attend with the selected set replaced by ALL visible
 * entries s < min(n_entries[b], (q + 1) / m_prime).
 *
 *  n_entries [B] int32, 0 <= n_entries <= Nmax.  Other arguments as above.
 */
csa_status hca_attend(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                      int rope_dims, float rope_theta, const int32_t* q_pos,
                      const void* kv, csa_dtype kv_t, int Nmax,
                      const int32_t* n_entries, int m_prime,
                      const void* win, int win_len, int n_win,
                      const float* sink, float scale, int B, int Tq, int nh, int c,
                      void* out, csa_dtype out_t,
                      void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * grouped_out_proj -- the grouped output projection (Evidence Ledger Section
 * 2.3.1: n_h heads -> g groups -> d_g intermediates -> d; shuhuayu section 03:
 * the attention outputs are rotated back by -q before it -- the attention
 * calls' epilogue does that -- and its configuration table: 8 groups of rank
 * 1024 for 64 heads x 512, 16 for 128 heads):
 *
 *   u[r, j*d_g + e] = sum_k o[r, j*K1 + k] * W_a[j, e, k],   K1 = nh/g * c
 *   y[r, n]         = sum_k u[r, k] * W_b[n, k]               k < g * d_g
 *
 *  o    [R, nh, c] in t (attention output rows, R = B * Tq); group j is heads
 *       j*nh/g .. (j+1)*nh/g - 1, concatenated head by head.
 *  W_a  [g, d_g, K1] and W_b [d, g*d_g] in t (linear-layer [out, in] layout).
 *  t    CSA_BF16 (matrix cores, fp32 accumulation; u is rounded to bf16
 *       between the products) or CSA_F32 (fp32 throughout).
 *  y    [R, d] in y_t (CSA_F32, or CSA_BF16 rounded RNE).
 *  ws   u (R * g * d_g elements of t) and, for R <= 64, fp32 partial sums of
 *       the K-slices (workspace protocol).
 *  CSA_BF16 needs K1 and g*d_g multiples of 32 and 16-byte aligned o, W_a,
 *  W_b, y and ws; nh must be a multiple of g.  Else CSA_ERR_INVALID.
 */
csa_status grouped_out_proj(const void* o, csa_dtype t, int R, int nh, int c, int g, int d_g,
                            const void* W_a, const void* W_b, int d, void* y, csa_dtype y_t,
                            void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * Paged caches (Evidence Ledger Section 3.5.1; "G2C Brief -- DeepSeek V4",
 * "Hybrid attention creates a hybrid cache"; shuhuayu section 06 "What grows
 * with context" for the per-entry bytes): compressed entries live in fixed-size
 * blocks covering lcm(m, m') tokens, so one block of 128 tokens holds 32 CSA
 * entries (main rows and index keys) and 1 HCA entry.  A block is a PAGE of a
 * caller-owned pool; the page holds each series in its own section at an
 * offset the caller chooses.  A series is named by its base pointer -- the
 * address of its slot 0 in page 0 (pool + section offset) -- and a csa_pages:
 *
 *   entry s of sequence b  ->  base + P * page_bytes + (s % E) * row_bytes,
 *   P = block_table[b * max_blocks + s / E],  E = 2^entries_log2.
 *
 * MXFP4 scale rows (cI/32 bytes) are a series of their own with the same
 * block table, page_bytes and E.  The sliding window stays in its dense ring
 * (the fixed-size state cache).  Preconditions the library cannot check on the
 * host: every block holding an entry the call reads or writes maps to a page
 * of the pool, page 0 exists (empty attention slots read it and discard the
 * data), and page ids are below 2^(31 - entries_log2).  Host checks: pages and
 * block_table non-NULL, max_blocks >= 1, 0 <= entries_log2 <= 16,
 * Nmax <= max_blocks * E, page_bytes a positive multiple of 16 with
 * E * row_bytes <= page_bytes, series bases 16-byte aligned; else
 * CSA_ERR_INVALID.  Results equal those of the dense calls on the same
 * logical entries bit for bit.
 */
typedef struct csa_pages {
  const int32_t* block_table; /* DEVICE [B, max_blocks] int32 page ids */
  int max_blocks;             /* row stride of block_table */
  int entries_log2;           /* log2 of the series' entries per page */
  int64_t page_bytes;         /* bytes from one page to the next */
} csa_pages;

/* csa_compress into pages: `out` / `out_scale` are series bases; entry i of
 * sequence b (i < T/m) is written to its page slot.  Nmax = T/m. */
csa_status csa_compress_paged(const void* H, csa_dtype h_t, int B, int T, int d,
                              const void* W_kv_a, const void* W_z_a,
                              const void* W_kv_b, const void* W_z_b,
                              const float* bias_a, const float* bias_b, int m, int overlap,
                              int c, const float* norm_w, float eps, int rope_dims,
                              float rope_theta, int pos_stride, int pos_offset,
                              void* out, uint8_t* out_scale, csa_dtype out_t,
                              const csa_pages* pages,
                              void* ws, size_t* ws_bytes, hipStream_t stream);

/* csa_compress_append into pages: `cache` / `cache_scale` are series bases. */
csa_status csa_compress_append_paged(const void* H, csa_dtype h_t, int B, int d,
                                     const void* W_kv_a, const void* W_z_a,
                                     const void* W_kv_b, const void* W_z_b,
                                     const float* bias_a, const float* bias_b, int m,
                                     int overlap, int c, const float* norm_w, float eps,
                                     int rope_dims, float rope_theta, int pos_stride,
                                     int pos_offset, const int32_t* entry, void* cache,
                                     uint8_t* cache_scale, csa_dtype out_t, int Nmax,
                                     const csa_pages* pages,
                                     void* ws, size_t* ws_bytes, hipStream_t stream);

/* indexer_score over paged index keys: `kI` / `kI_scale` are series bases. */
csa_status indexer_score_paged(const void* qI, const uint8_t* qI_scale, csa_dtype qI_t,
                               const float* w,
                               const void* kI, const uint8_t* kI_scale, csa_dtype kI_t,
                               const csa_pages* pages,
                               const int32_t* q_pos, const int32_t* n_entries,
                               int B, int Tq, int nI, int cI, int Nmax, int m,
                               void* scores, csa_dtype score_t, hipStream_t stream);

/* sparse_mqa_attend over paged main rows: `kv` is a series base. */
csa_status sparse_mqa_attend_paged(const void* q, csa_dtype q_t, const float* q_norm_w,
                                   float eps, int rope_dims, float rope_theta,
                                   const int32_t* q_pos,
                                   const void* kv, csa_dtype kv_t, int Nmax,
                                   const csa_pages* pages,
                                   const int32_t* idx, int k,
                                   const void* win, int win_len, int n_win,
                                   const float* sink, float scale, int B, int Tq, int nh, int c,
                                   void* out, csa_dtype out_t,
                                   void* ws, size_t* ws_bytes, hipStream_t stream);

/* hca_attend over paged HCA rows (one entry per 128-token block:
 * entries_log2 = 0 for m' = 128): `kv` is a series base. */
csa_status hca_attend_paged(const void* q, csa_dtype q_t, const float* q_norm_w, float eps,
                            int rope_dims, float rope_theta, const int32_t* q_pos,
                            const void* kv, csa_dtype kv_t, int Nmax,
                            const csa_pages* pages,
                            const int32_t* n_entries, int m_prime,
                            const void* win, int win_len, int n_win,
                            const float* sink, float scale, int B, int Tq, int nh, int c,
                            void* out, csa_dtype out_t,
                            void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * sparse_mqa_attend_noalloc -- sparse_mqa_attend that allocates nothing and
 * takes no workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.
 *
 *  Arguments, layouts and results are those of sparse_mqa_attend without
 *  ws / ws_bytes.  The split-softmax partials (sparse_mqa_attend's workspace)
 *  go to a scratch array of CSA_NOALLOC_SCRATCH_BYTES inside the library's
 *  device memory, one copy per GPU, held until the process ends.  A call whose
 *  partials need more returns CSA_ERR_WORKSPACE and launches nothing (32 MiB
 *  covers, e.g., 32 decode rows x 64 heads in 8 splits or 8 x 128 heads in 12
 *  splits, at k = 1024 and a 128-row window).
 *  Every call looks up the current device's scratch address the first time
 *  it runs on that device (CSA_ERR_LAUNCH if the lookup fails); an empty call
 *  (B == 0) does only that, e.g. before a graph capture.
 *  All calls on one GPU share its scratch, which keeps the last call's
 *  contents: calls that overlap in time on one GPU (several streams or host
 *  threads) race on it and must be serialised by the caller.  Every partial a
 *  call reads is written by that call first.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa_status sparse_mqa_attend_noalloc(const void* q, csa_dtype q_t, const float* q_norm_w,
                                     float eps, int rope_dims, float rope_theta,
                                     const int32_t* q_pos, const void* kv, csa_dtype kv_t,
                                     int Nmax, const int32_t* idx, int k,
                                     const void* win, int win_len, int n_win,
                                     const float* sink, float scale, int B, int Tq, int nh,
                                     int c, void* out, csa_dtype out_t, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
