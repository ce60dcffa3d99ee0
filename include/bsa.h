/*
 * bsa.h -- block-sparse self-attention for video diffusion transformers on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: pointers, sizes, status codes.
 *
 * The hot path, in call order:
 *   bsa_score_blocks      mean-pool Q and K over 64-token blocks (and 16-token
 *                         tiles) and form the pooled block scores;
 *   bsa_select_blocks     per query block, the key blocks to keep (top-k,
 *                         top-p, static window + rotating anchors, or the
 *                         micro tiles inside omitted blocks) as CSR lists;
 *   bsa_sparse_attn_fwd   block-sparse flash attention: O and per-row LSE;
 *   bsa_micro_residual_fwd attention over the selected 16x16 micro tiles;
 *   bsa_lse_merge         exact merge of two partial softmax results.
 *   bsa_dense_attn_fwd    the same attention engine over every key (baseline).
 *   bsa_attn_stage_v      the attention calls' V^T staging on its own (to
 *                         overlap it with scoring on another stream).
 *   bsa_pooled_rectify    add the pooled estimate of the omitted blocks to a
 *                         sparse result (exact LSE merge).
 *   bsa_local_window_cluster  3D local-window clustering of Q or K (the
 *                         front end of cluster-induced blocks).
 *   bsa_cluster_permute   tokens in cluster order (HVA Eq. 1).
 *   bsa_cluster_select    key clusters per query cluster (HVA Eq. 2-3).
 *   bsa_lowe_ratio_subset Lowe's ratio and the most ambiguous tokens (HVA Eq. 6).
 *   bsa_subset_refine     the intermediate-step update of those tokens
 *                         against every centroid (HVA section 4.2).
 *   bsa_cluster_merge     merging of query clusters by tiled cost (HVA Alg. 1).
 *   bsa_cluster_attn_fwd  attention over cluster-induced blocks (HVA Eq. 4).
 *   bsa_omission_risk     per-head share of the full softmax mass a sparse
 *                         support omits (offline head calibration).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors Q, K, V (and attention outputs O) are [B, H, N, d] with element
 * strides stride_b, stride_h, stride_n taken from bsa_shape and the last
 * dimension contiguous.  Q, K, V are bf16 (passed as uint16_t bit patterns);
 * base pointers must be 16-byte aligned and the strides multiples of 8.
 * Tokens are a video latent grid flattened t-major.  N is the number of
 * valid tokens: the last 64-token block (and 16-token tile) may be ragged;
 * padded positions are never read as keys nor written as queries.
 * Per-row LSE arrays are float32 [B, H, N], contiguous.  All other arrays are
 * contiguous as documented.  d must be 64 or 128; the block must be 64 and
 * the micro tile 16.
 *
 * Every pointer except those marked "host" is device memory owned by the
 * caller; the library keeps no state between calls and allocates nothing.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream) and never synchronise.  Arguments are validated before anything is
 * launched: a non-zero status means nothing was enqueued, and
 * bsa_last_error() (thread-local) says why.  A launch failure reported by
 * the HIP runtime returns BSA_ERR_HIP.  NaN/Inf inputs are not checked.
 *
 * Sources (pages as titled): "HyperVAttention: Efficient Sparse Attention
 * with Spatio-Temporal Clustering for Video Diffusion" (HVA), section 2,
 * Eq. 2-4; "HyMoR-Attn: Granularity-Matched Repair of Omitted Attention
 * Support for Video Diffusion" (abstract: Macro backbone, Micro residual,
 * exact LSE merging); "Rectified SpaAttn" (abstract: pooled query-key
 * interactions); the "Long Video Sparse Attention" (LVSA) abstract (window
 * pattern with rotating global anchors); "Mixture of Distributions Matters"
 * (MOD-DiT: block-wise attention, density = computed blocks / all blocks).
 */
#ifndef BSA_H_
#define BSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bsa_status;
enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, ... */
  BSA_ERR_UNSUPPORTED = 2, /* d not in {64,128}, block != 64, micro != 16, */
                           /* too many blocks for a scored selection       */
  BSA_ERR_CAPACITY = 3,    /* workspace smaller than required              */
  BSA_ERR_HIP = 4          /* the HIP runtime reported an error            */
};

/* Element type of attention outputs O (and of merge inputs). */
enum { BSA_F32 = 0, BSA_BF16 = 1 };

typedef struct bsa_shape {
  int32_t B, H, N, d;
  int64_t stride_b, stride_h, stride_n; /* elements; last dim contiguous */
} bsa_shape;

/* Library version string, e.g. "bsa 0.1.0 gfx950". */
const char* bsa_version(void);

/* Message describing the last non-OK status returned on this thread. */
const char* bsa_last_error(void);

/* ------------------------------------------------------------------------
 * bsa_score_blocks -- pooled block scores (Rectified SpaAttn: pooled
 * query-key interactions; HVA section 2, Eq. 2 left, with centroids = block
 * means).
 *
 *   qpool[b,h,i,:] = mean of Q[b,h,t,:] over the valid tokens t of block i
 *   kpool[b,h,j,:] = same for K
 *   scores[b,h,i,j] = scale * <qpool[b,h,i,:], kpool[b,h,j,:]>
 *
 * block: 64, or 128 (the block size of MOD-DiT's block-wise attention).
 *   nB = ceil(N / block).
 * qpool, kpool: float32 [B, H, nB, d] (required).
 * scores: float32 [B, H, nB, nB], or NULL to skip the score matrix.
 * micro: 0, or 16 to also write the 16-token tile means qpool16 / kpool16,
 *   float32 [B, H, nT, d] with nT = ceil(N / 16) (required when micro=16).
 * Accumulation is float32 (no bf16 rounding of the means or scores); the
 * dot products run on the bf16 matrix cores over exact three-part bf16
 * splits of the means, with float32-grade error.
 * ---------------------------------------------------------------------- */
bsa_status bsa_score_blocks(const uint16_t* Q, const uint16_t* K,
                            const bsa_shape* shape, int32_t block, float scale,
                            float* qpool, float* kpool, float* scores,
                            int32_t micro, float* qpool16, float* kpool16,
                            void* stream);

/* ------------------------------------------------------------------------
 * Selection parameters.
 *
 * mode BSA_SELECT_TOPK: keep the k key blocks of highest score, ties to the
 *   lower block index (the Top-K density budget of block-sparse selectors).
 * mode BSA_SELECT_TOPP: HVA Eq. 2 right and Eq. 3: size-weighted softmax
 *   P_ij = n_j e^{S_ij} / sum_o n_o e^{S_io} (n_j = valid tokens of block
 *   j); keep the smallest prefix in descending P whose cumulative mass is at
 *   least p, clamped to [k_min, k_cap] blocks (HVA appendix A.1 "Min-kc" is
 *   the floor; the density cap is the ceiling).
 * mode BSA_SELECT_STATIC: no scores; only the forced set below.
 * mode BSA_SELECT_MICRO: HyMoR Micro selection (reading: for query block i,
 *   candidates are pairs (a, beta) of a 16-row query sub-tile a = 0..3 of
 *   block i and a 16-key tile beta whose 64-block was omitted by the macro
 *   lists; score sigma = scale * <qpool16[4i+a], kpool16[beta]>; keep the
 *   micro_m best by (sigma descending, code ascending), code = 4*beta + a).
 *   Entries are codes, sorted by (a, beta).  Heads with head_mask[h] == 0 get
 *   empty rows.
 *
 * Forced set (a union on top of TOPK/TOPP, not counted in k or p; the whole
 * row in STATIC mode):
 *   force_diag: block i itself;
 *   use_static: the LVSA static mask -- key block j is kept when some token
 *   of j lies within window_frames latent frames of some token of block i
 *   (frame of token t = t / frame_tokens), plus n_anchors global anchor
 *   blocks (anchor_offset + a * floor(nB / n_anchors)) mod nB, a = 0..n-1.
 *   The caller draws anchor_offset per call (rotation).  window_frames = 0
 *   is MOD-DiT's block-diagonal (intra-frame) pattern;
 *   diagonals / columns: MOD-DiT's parallel-diagonal and vertical patterns
 *   (section "Pattern Mixtures"): query block i keeps key block i + delta
 *   for each offset delta (offsets off the block map mark nothing) and every
 *   listed key column.  Which patterns to use (MOD ranks them by intensities
 *   fitted to dense attention maps of a model) is the caller's choice.
 *
 * Blocks (all modes but MICRO): block = 64, or 128 for selection on 128-token
 * blocks -- scores, k, k_cap, the forced set, diagonals and columns are then
 * in 128-token blocks -- and the CSR is emitted on the 64-token tiles the
 * attention kernels run: 64-token query block i' takes the row of 128-token
 * block i'/2, each kept 128-token key block J becoming blocks 2J and 2J+1
 * (when 2J+1 exists), which leaves every query's token support unchanged.
 * MICRO mode needs block = 64 (it reads the 64-token macro CSR).
 * ---------------------------------------------------------------------- */
enum {
  BSA_SELECT_TOPK = 0,
  BSA_SELECT_TOPP = 1,
  BSA_SELECT_STATIC = 2,
  BSA_SELECT_MICRO = 3
};

typedef struct bsa_select_params {
  int32_t mode;
  int32_t k;        /* TOPK: blocks per row (0 <= k)                    */
  float p;          /* TOPP: threshold in (0, 1]                         */
  int32_t k_min;    /* TOPP: floor on the row length (>= 0)              */
  int32_t k_cap;    /* TOPP: ceiling on the row length (>= k_min)        */
  int32_t force_diag;
  int32_t use_static;
  int32_t frame_tokens;   /* > 0 when use_static                          */
  int32_t window_frames;  /* >= 0                                         */
  int32_t n_anchors;      /* >= 0                                         */
  int32_t anchor_offset;  /* any value; taken modulo nB                   */
  /* MICRO mode only */
  int32_t micro;          /* 16                                           */
  int32_t micro_m;        /* tiles kept per query block (>= 0)             */
  float scale;            /* softmax scale of the micro score              */
  const uint8_t* head_mask;      /* host [H]; NULL = every head            */
  const int32_t* macro_row_ptr;  /* device, macro CSR of this shape        */
  const int32_t* macro_col_idx;  /* device                                  */
  const float* qpool16;          /* device [B,H,nT,d] from bsa_score_blocks */
  const float* kpool16;          /* device [B,H,nT,d]                       */
  /* structural patterns (all modes but MICRO), at most 64 of each        */
  int32_t n_diagonals;
  const int32_t* diagonals;      /* host [n_diagonals]: offsets delta       */
  int32_t n_columns;
  const int32_t* columns;        /* host [n_columns]: key blocks in [0, nB) */
} bsa_select_params;

/* Bytes of device workspace bsa_select_blocks needs for these arguments
 * (returns -1 on invalid arguments; see bsa_last_error). */
int64_t bsa_select_workspace_bytes(const bsa_shape* shape, int32_t block,
                                   const bsa_select_params* params);

/* Upper bound on the total entries bsa_select_blocks can emit. */
int64_t bsa_select_max_nnz(const bsa_shape* shape, int32_t block,
                           const bsa_select_params* params);

/* ------------------------------------------------------------------------
 * bsa_select_blocks -- CSR block lists, one row per (b, h, 64-token query
 * block i), row index r = (b * H + h) * nB64 + i, nB64 = ceil(N / 64).
 *
 * scores: float32 [B, H, nB, nB] from bsa_score_blocks with the same block
 *   (TOPK/TOPP); NULL in STATIC and MICRO mode.
 * row_ptr: int32 [B*H*nB64 + 1]; row r is col_idx[row_ptr[r] .. row_ptr[r+1]).
 * col_idx: int32 [col_cap]: ascending key block indices (MICRO: codes
 *   4*beta + a, sorted by (a, beta)).  Entries at positions >= col_cap are
 *   not written; *out_nnz tells the caller whether col_cap sufficed.
 * out_nnz: device int64, receives the total number of entries.
 * workspace: device, at least bsa_select_workspace_bytes(...) bytes; its
 *   contents on entry do not matter.
 * Limits: TOPK/TOPP need nB <= 4096 selection blocks; every mode needs
 * nB64 <= 4096 (N <= 262144 tokens); totals must fit in int32.
 * ---------------------------------------------------------------------- */
bsa_status bsa_select_blocks(const float* scores, const bsa_shape* shape,
                             int32_t block, const bsa_select_params* params,
                             int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_cap, int64_t* out_nnz,
                             void* workspace, int64_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * bsa_select_blocks_noalloc -- bsa_select_blocks for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, results and
 * errors without the workspace.  Its scratch is a static device array of
 * bsa_select_scratch_limit() bytes (32 MiB) that each GPU the library runs
 * on holds until the process ends; the call allocates nothing (no
 * hipMalloc, no allocating library routine).  Selections whose
 * bsa_select_workspace_bytes exceeds the limit are refused with
 * BSA_ERR_CAPACITY before any HIP call (every TOPK, TOPP and STATIC
 * selection of up to 4096 blocks per row for B*H*nB up to ~60,000 rows
 * fits; MICRO fits only small layers: its tile scores take 4 (B*heads)
 * ceil(N/16)^2 bytes).  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (several streams or host threads) race and
 * must be serialised by the caller.  The first call on a device looks up
 * the array's device address (hipGetSymbolAddress) with that device
 * current.
 * ---------------------------------------------------------------------- */
bsa_status bsa_select_blocks_noalloc(const float* scores,
                                     const bsa_shape* shape, int32_t block,
                                     const bsa_select_params* params,
                                     int32_t* row_ptr, int32_t* col_idx,
                                     int64_t col_cap, int64_t* out_nnz,
                                     void* stream);

/* Bytes of the no-allocation entry point's static scratch (32 MiB). */
int64_t bsa_select_scratch_limit(void);

/* Bytes of device workspace the attention entry points need (the key-major
 * copy of V the PV products read, the micro residual's sub-tile order, and
 * a status word in the last 256 bytes).  Returns -1 on invalid arguments.
 * The status word (int32 at byte bsa_attn_workspace_bytes(shape) - 256)
 * must be zero when the workspace is first used: zero those bytes once
 * after allocating it, or call bsa_attn_take_status once. */
int64_t bsa_attn_workspace_bytes(const bsa_shape* shape);

/* ------------------------------------------------------------------------
 * bsa_sparse_attn_fwd -- block-sparse attention forward (HVA Eq. 4 on the
 * original token order; the HyMoR Macro backbone).  For every valid query
 * token t of block i, over the keys of the blocks in its CSR row:
 *   LSE[t] = ln sum_tau exp(scale * q_t . k_tau)
 *   O[t]   = sum_tau exp(scale * q_t . k_tau - LSE[t]) v_tau
 * QK^T runs as a bf16 matrix-core product on the inputs, PV as an fp16 one
 * (P rounded to fp16, V converted from bf16 exactly), both with float32
 * accumulation; the softmax is online (flash style) in float32.  Rows with
 * an empty list get O = 0 and LSE = -inf.
 *
 * row_ptr / col_idx: a CSR from bsa_select_blocks (or the caller); column
 *   indices must lie in [0, nB).  Order within a row does not matter.  A
 *   column index outside [0, nB) adds nothing to its row (the kernel reads
 *   an in-bounds tile instead and masks it out) and sets bit 1 of the
 *   workspace's status word (see bsa_attn_take_status).  row_ptr itself is
 *   trusted: rows must be in order and lie within col_idx (checked by
 *   bsa_check_csr / bsa_validate_csr_host, not by this call).
 * O: [B, H, N, d] with the strides of `shape`, element type o_dtype
 *   (BSA_F32 or BSA_BF16, round-to-nearest-even).
 * LSE: float32 [B, H, N].
 * workspace: device, >= bsa_attn_workspace_bytes(shape) bytes, 256-byte
 *   aligned.  The call first writes a key-major fp16 copy of V into it (the
 *   PV operand; V entries must lie within the fp16 range |v| <= 65504).
 * V may be NULL: the workspace then must already hold that copy, written by
 *   an earlier attention call on the same V and shape (all heads for the
 *   sparse/dense calls; the masked heads for the micro call), so that the
 *   macro, micro and dense passes over one V share a single conversion.
 * ---------------------------------------------------------------------- */
bsa_status bsa_sparse_attn_fwd(const uint16_t* Q, const uint16_t* K,
                               const uint16_t* V, const bsa_shape* shape,
                               int32_t block, float scale,
                               const int32_t* row_ptr, const int32_t* col_idx,
                               void* O, int32_t o_dtype, float* LSE,
                               void* workspace, int64_t workspace_bytes,
                               void* stream);

/* bsa_dense_attn_fwd -- the same engine over all N keys for every query
 * (full attention; the speedup baseline). Arguments as above. */
bsa_status bsa_dense_attn_fwd(const uint16_t* Q, const uint16_t* K,
                              const uint16_t* V, const bsa_shape* shape,
                              float scale, void* O, int32_t o_dtype,
                              float* LSE, void* workspace,
                              int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_attn_take_status -- copies the attention workspace's status word to
 * status_out (device int32) and clears it, in stream order.  Bit 1: some
 * call since the last clear met a column index (bsa_sparse_attn_fwd) or a
 * micro tile index (bsa_micro_residual_fwd) outside its range and skipped
 * it.  The word is sticky: every call ORs into it; nothing else clears it.
 * ---------------------------------------------------------------------- */
bsa_status bsa_attn_take_status(void* workspace, int64_t workspace_bytes,
                                const bsa_shape* shape, int32_t* status_out,
                                void* stream);

/* ------------------------------------------------------------------------
 * bsa_check_csr -- validates a device CSR of `rows` rows before attention:
 * counts[0] = rows whose pointers are out of order, negative or past
 * col_cap (row_ptr[0] must be 0), counts[1] = entries outside [0, n_cols),
 * counts[2] = entries not strictly above their predecessor in the row.
 * counts: device int32 [3], overwritten (zeroed by the call itself); read
 * it after a stream synchronisation.  Reads row_ptr [rows + 1] and, for
 * rows whose pointers pass, only col_idx[row_ptr[r] .. row_ptr[r+1]) within
 * [0, col_cap).  All zero means the CSR is safe for the attention calls
 * (n_cols = nB64 for macro lists, ceil(N / 16) * 4 codes for micro lists,
 * whose order rule is (a, beta) -- use counts[1] only there).
 * ---------------------------------------------------------------------- */
bsa_status bsa_check_csr(const int32_t* row_ptr, int64_t rows,
                         const int32_t* col_idx, int64_t col_cap,
                         int32_t n_cols, int32_t* counts, void* stream);

/* bsa_validate_csr_host -- the same rules on a HOST CSR, synchronously:
 * BSA_OK, or BSA_ERR_INVALID_ARG with the first failing row in *bad_row
 * (may be NULL; -1 when the arrays themselves are invalid) and the reason
 * in bsa_last_error().  Needs no GPU. */
bsa_status bsa_validate_csr_host(const int32_t* row_ptr, int64_t rows,
                                 const int32_t* col_idx, int64_t col_cap,
                                 int32_t n_cols, int64_t* bad_row);

/* ------------------------------------------------------------------------
 * bsa_attn_stage_v -- the fp16 V^T staging that bsa_sparse_attn_fwd,
 * bsa_dense_attn_fwd and bsa_micro_residual_fwd perform when given V, as a
 * call of its own, so that a caller can run it on another stream while the
 * scores and selections of the same step are computed, then pass V = NULL
 * to the attention calls (ordering between the streams is the caller's).
 * Writes only the V^T region of the workspace: [B*H, nB, 4, d, 16] fp16,
 * every 16-key chunk in the order the matrix-core operand reads it, zero
 * beyond N.  Same V layout rules as the attention calls.
 * workspace: >= bsa_attn_workspace_bytes(shape) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
bsa_status bsa_attn_stage_v(const uint16_t* V, const bsa_shape* shape,
                            void* workspace, int64_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * bsa_micro_residual_fwd -- HyMoR Micro residual: each 16-row query sub-tile
 * a of block i attends over the union of the 16-key tiles beta of the
 * entries (a, beta) in its micro row (codes 4*beta + a, as emitted by
 * BSA_SELECT_MICRO).  Output as bsa_sparse_attn_fwd; sub-tiles without a
 * tile get O = 0, LSE = -inf.  Heads with head_mask[h] == 0 (host [H];
 * NULL = all heads) are skipped and their O_mu / LSE_mu left untouched.
 * ---------------------------------------------------------------------- */
bsa_status bsa_micro_residual_fwd(const uint16_t* Q, const uint16_t* K,
                                  const uint16_t* V, const bsa_shape* shape,
                                  int32_t block, int32_t micro, float scale,
                                  const int32_t* mrow_ptr, const int32_t* midx,
                                  const uint8_t* head_mask, void* O_mu,
                                  int32_t o_dtype, float* LSE_mu,
                                  void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * bsa_lse_merge -- HyMoR exact LSE merging of two partial attention results
 * over disjoint key supports:
 *   L = ln(e^L1 + e^L2);  O = e^(L1 - L) O1 + e^(L2 - L) O2
 * Both -inf gives O = 0, L = -inf.  O1/O2/O share element type o_dtype and
 * the strides of `shape`; L arrays are float32 [B, H, N].  O may alias O1
 * and L may alias L1 (in-place).  Heads with head_mask[h] == 0 (host [H];
 * NULL = all) are left untouched.
 * ---------------------------------------------------------------------- */
bsa_status bsa_lse_merge(const void* O1, const float* L1, const void* O2,
                         const float* L2, const bsa_shape* shape,
                         int32_t o_dtype, const uint8_t* head_mask, void* O,
                         float* L, void* stream);

/* ------------------------------------------------------------------------
 * bsa_pooled_rectify -- pooled rectification of omitted blocks ("Rectified
 * SpaAttn", abstract: sparse attention over-weights the kept blocks and
 * loses the omitted ones; pooled query-key interactions correct both).  The
 * page gives no formulas.  Reading used here: for every valid query token t
 * of 64-token block i, each key block j NOT in row i contributes its pooled
 * estimate, with Kbar_j, Vbar_j the means of K, V over the n_j valid tokens
 * of block j:
 *   LSE_p[t] = ln sum_j n_j exp(scale q_t . Kbar_j)
 *   O_p[t]   = sum_j n_j exp(scale q_t . Kbar_j - LSE_p[t]) Vbar_j
 * (exact when block j's keys are all equal), and the call replaces the
 * sparse result (O, LSE) by its exact LSE merge with (O_p, LSE_p), as
 * bsa_lse_merge would.  A row that keeps every block is left as it is.
 *
 * gain_gate (0 or 1): the page's Gain-Aware Pooling Rectification (the
 *   recovered gain must exceed the pooling error it brings in), read as: the
 *   estimate of block j for query t recovers n_j exp(scale q_t . Kbar_j);
 *   if the block's keys scatter normally and isotropically about Kbar_j
 *   with per-coordinate variance v_j = sum |k - Kbar_j|^2 / (n_j d), the
 *   block's true mass is that estimate times exp(sigma^2 / 2), sigma^2 =
 *   scale^2 |q_t|^2 v_j, so the error stays below the gain while
 *   sigma^2 < 2 ln 2.  With gain_gate = 1 block j enters LSE_p[t] and
 *   O_p[t] only where |q_t|^2 v_j < 2 ln 2 / scale^2 (float32, |q_t|^2
 *   from the bf16 query, v_j from one more pass over K); a query with no
 *   block left keeps its sparse result.  scale must be > 0 with the gate.
 *
 * O, LSE: on entry the bsa_sparse_attn_fwd result for the same Q, K, V and
 *   CSR (o_dtype BSA_F32 or BSA_BF16); on return the rectified result.
 * row_ptr / col_idx: the 64-token CSR the sparse result was computed on.
 * block: 64.  Limits: nB = ceil(N / 64) <= 4096, B*H <= 65535.
 * Precision: q . Kbar on bf16 matrix-core products with Kbar split into
 *   bf16 high and low parts (about 16 mantissa bits), Vbar as fp16, float32
 *   accumulation and softmax.
 * workspace: device, >= bsa_pooled_rectify_workspace_bytes(shape) bytes,
 *   256-byte aligned (the pooled means and their matrix-core copies).
 * ---------------------------------------------------------------------- */
int64_t bsa_pooled_rectify_workspace_bytes(const bsa_shape* shape);

bsa_status bsa_pooled_rectify(const uint16_t* Q, const uint16_t* K,
                              const uint16_t* V, const bsa_shape* shape,
                              int32_t block, float scale, int32_t gain_gate,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              void* O, int32_t o_dtype, float* LSE,
                              void* workspace, int64_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * bsa_local_window_cluster -- 3D local-window clustering of one token
 * tensor per head (HyperVAttention section 4.1, Eq. 5; Appendix A.2,
 * Algorithm 2), the front end of its cluster-induced blocks.  The N tokens
 * form a T x Hg x W lattice, t-major (token n = (t * Hg + y) * W + x).  A
 * fixed grid of (kt, kh, kw) cells -- ceil(T/kt) x ceil(Hg/kh) x ceil(W/kw)
 * of them, numbered t-major -- carries one centroid per cell, initialised
 * at the cell's centre token (coordinates u*k + floor(k/2), clamped to the
 * lattice).  Each of `iters` iterations assigns every token to the nearest
 * centroid (squared Euclidean distance) among the cells of a (wt, wh, ww)
 * window around its own cell -- per axis the cells g - floor(w/2) .. +w-1,
 * shifted to stay inside the grid, w clipped to the cell count -- and then
 * moves every centroid to the mean of its tokens (one with none stays).
 * Reading where the page is silent: ties go to the lower centroid index.
 *
 * X: bf16 [B, H, N, d] with the strides of `shape` (queries or keys).
 * assign: int32 [B, H, N], the last iteration's centroid of every token.
 * centroids: float32 [B, H, cells, d] after the last update.
 * counts: int32 [B, H, cells], tokens per centroid in the last assignment.
 * workspace: >= bsa_cluster_workspace_bytes bytes, 16-byte aligned (the
 *   centroids' squared norms and their three bf16 parts).
 * Precision: distances as ||mu||^2 - 2 x.mu with x.mu from bf16 matrix
 *   products of the bf16 token and the centroid split exactly into three
 *   bf16 parts, summed in float32 (near-ties within float32 rounding may
 *   resolve either way); centroid sums in float32 in token order, so
 *   repeated calls give identical results.
 * ---------------------------------------------------------------------- */
typedef struct bsa_cluster_params {
  int32_t T, Hg, W;     /* token lattice, T * Hg * W == N                  */
  int32_t kt, kh, kw;   /* cell size (>= 1)                                 */
  int32_t wt, wh, ww;   /* window in cells (>= 1; clipped to the grid)      */
  int32_t iters;        /* >= 1                                             */
} bsa_cluster_params;

/* Number of cells (centroids) per head, or -1 on invalid arguments. */
int64_t bsa_cluster_cells(const bsa_shape* shape, const bsa_cluster_params* params);

int64_t bsa_cluster_workspace_bytes(const bsa_shape* shape,
                                    const bsa_cluster_params* params);

bsa_status bsa_local_window_cluster(const uint16_t* X, const bsa_shape* shape,
                                    const bsa_cluster_params* params,
                                    int32_t* assign, float* centroids,
                                    int32_t* counts, void* workspace,
                                    int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_subset_refine -- HyperVAttention section 4.2, the intermediate-step
 * update of its hybrid clustering: full local-window clustering runs only
 * at anchor steps, which also cache the tokens of largest Lowe's ratio
 * (bsa_lowe_ratio_subset); at the steps in between only that subset is
 * revisited.  Each subset token is reassigned by a standard k-means step
 * against EVERY centroid of its head (not only its local window): the
 * nearest by squared Euclidean distance, ties to the lower index.  Then the
 * centroids that a subset token left or joined move to the mean of their
 * members under the new assignment, using the current embeddings X; one
 * left without members keeps its position; every other centroid (and every
 * token outside the subset) is left as it is.
 *
 * X: bf16 [B, H, N, d] with the strides of `shape`: the CURRENT step's
 *   queries or keys.
 * cells: centroids per head.
 * subset: int32 [B, H, n_sub], distinct token indices per head (e.g. the
 *   output of bsa_lowe_ratio_subset at the anchor step); an index outside
 *   [0, N) is ignored.
 * assign: int32 [B, H, N], centroids: float32 [B, H, cells, d], counts: int32
 *   [B, H, cells]: the clustering state (bsa_local_window_cluster's outputs
 *   or a previous refinement), updated in place; counts must be the member
 *   counts of `assign`.
 * workspace: >= bsa_subset_refine_workspace_bytes(shape, cells) bytes,
 *   256-byte aligned (touched-centroid bitmaps, member counts and ranges, a
 *   member list of up to B*H*N tokens, the centroids' bf16 parts and norms).
 * Precision: distances as ||mu||^2 - 2 x.mu with float32-grade dot products
 *   (each centroid split exactly into three bf16 parts on the matrix cores,
 *   float32 sums; near-ties within that rounding may resolve either way);
 *   member sums in float64, exact while one coordinate's nonzero magnitudes
 *   over a centroid's n members lie within a factor 2^(45 - log2 n), so
 *   repeated calls agree; means rounded to float32.
 * Errors: BSA_ERR_UNSUPPORTED when B*H*N or B*H*cells reaches 2^31.
 * ---------------------------------------------------------------------- */
int64_t bsa_subset_refine_workspace_bytes(const bsa_shape* shape, int32_t cells);

bsa_status bsa_subset_refine(const uint16_t* X, const bsa_shape* shape,
                             int32_t cells, const int32_t* subset,
                             int32_t n_sub, int32_t* assign, float* centroids,
                             int32_t* counts, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_cluster_permute -- HyperVAttention Eq. 1: the permutation that places
 * each cluster's tokens contiguously, tokens ordered by (cluster, original
 * index), and every cluster's start.
 *
 * assign, counts: the outputs of bsa_local_window_cluster with the same
 *   shape and params (counts must be the number of tokens of each cluster;
 *   positions beyond a cluster's segment are not written otherwise).
 * perm: int32 [B, H, N], perm[b,h,k] = original index of the token at
 *   position k of the head's cluster order.
 * offsets: int32 [B, H, cells + 1], cluster u occupies positions
 *   offsets[u] .. offsets[u+1]-1 (offsets[cells] = N).
 * workspace: >= bsa_cluster_permute_workspace_bytes bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
int64_t bsa_cluster_permute_workspace_bytes(const bsa_shape* shape,
                                            const bsa_cluster_params* params);

bsa_status bsa_cluster_permute(const int32_t* assign, const int32_t* counts,
                               const bsa_shape* shape,
                               const bsa_cluster_params* params, int32_t* perm,
                               int32_t* offsets, void* workspace,
                               int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_cluster_select -- HyperVAttention section 2, Eq. 2-3 on clusters: for
 * every query cluster i of every (b, h), the key clusters of
 * TopP(P'_i; p) with P'_ij = s_j exp(S_ij) / sum_o s_o exp(S_io),
 * S_ij = scale <mu_i^q, mu_j^k>, s_j the key cluster sizes; the prefix
 * length clamped to [k_min, k_cap] (Min-kc of Appendix A.1 as the floor);
 * ties to the lower index.  A CSR with one row per (b, h, i), row index
 * (b * H + h) * Nq + i, ascending key cluster indices.
 *
 * mu_q: float32 [B, H, Nq, d]; mu_k: float32 [B, H, Nk, d] (the centroids of
 *   bsa_local_window_cluster); size_k: int32 [B, H, Nk] (its counts).
 * row_ptr: int32 [B*H*Nq + 1]; col_idx: int32 [col_cap]; out_nnz: device
 *   int64 total (entries beyond col_cap are not written).
 * workspace: >= bsa_cluster_select_workspace_bytes(B, H, Nq, Nk) bytes,
 *   256-byte aligned.  Limits: Nk <= 4096, d in {64, 128}.
 * ---------------------------------------------------------------------- */
int64_t bsa_cluster_select_workspace_bytes(int32_t B, int32_t H, int32_t Nq,
                                           int32_t Nk);

bsa_status bsa_cluster_select(const float* mu_q, const float* mu_k,
                              const int32_t* size_k, int32_t B, int32_t H,
                              int32_t Nq, int32_t Nk, int32_t d, float scale,
                              float p, int32_t k_min, int32_t k_cap,
                              int32_t* row_ptr, int32_t* col_idx,
                              int64_t col_cap, int64_t* out_nnz,
                              void* workspace, int64_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * bsa_lowe_ratio_subset -- Lowe's ratio of every token and the subset of the
 * most ambiguous ones (HyperVAttention section 4.2, Eq. 6): per token,
 *   rho = d_1 / d_2,
 * d_1 its Euclidean distance to the nearest of the given centroids and d_2
 * to the nearest other one, both over the centroids of its local window
 * (the candidates of bsa_local_window_cluster with the same params; 0 with
 * a single candidate, 1 when d_2 = 0).  Then, per (b, h), the n_sub tokens
 * of largest rho (equal ratios to the lower token index), ascending: the
 * subset the page re-assigns against all centroids between full
 * clusterings (the page caches the top 15%).  Distances in float32 as
 * ||mu||^2 - 2 x.mu + ||x||^2.
 *
 * X, shape, params: as bsa_local_window_cluster (params->iters unused, >= 1).
 * centroids: float32 [B, H, Nc, d] (typically bsa_local_window_cluster's).
 * n_sub: 0 .. N.  rho (out): float32 [B, H, N].  subset (out): int32
 *   [B, H, n_sub] (may be NULL when n_sub = 0).
 * workspace: >= bsa_cluster_workspace_bytes(shape, params) bytes.
 * ---------------------------------------------------------------------- */
bsa_status bsa_lowe_ratio_subset(const uint16_t* X, const bsa_shape* shape,
                                 const bsa_cluster_params* params,
                                 const float* centroids, int32_t n_sub,
                                 float* rho, int32_t* subset, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_cluster_merge -- hardware-aware merging of query clusters
 * (HyperVAttention section 4.3, Eq. 7-10, Algorithm 1).  A group S of query
 * clusters costs
 *   C(S) = tau_q ceil(s^q(S) / tau_q) * tau_k ceil(grain * K(S) / tau_k),
 *   K(S) = sum over key clusters j in the union of the members' rows of
 *          ceil(s_j^k / grain),
 * the tiled work of executing the group with its key clusters packed one
 * after another at a grain of `grain` tokens (grain = 1 is the page's Eq. 8;
 * bsa_cluster_attn_fwd packs at 16 on 64 x 64 tiles, so tau_q = tau_k = 64,
 * grain = 16 is the cost it executes).  Starting from singletons, each of
 * `rounds` rounds (the page uses 3) splits the current groups by
 * sides[b, h, round, name] (0 or 1, read at the group's name = its lowest
 * member; the page draws them at random, the caller does here); every side-0
 * group A takes the side-1 group B of smallest gain C(A u B) - C(A) - C(B)
 * (ties to the lower B); for each B the A of smallest negative gain is kept
 * (ties to the lower A), and all kept pairs merge.  Integer arithmetic:
 * results are exact and repeatable.
 *
 * off_q [B,H,Nq+1], off_k [B,H,Nk+1]: cluster offsets (bsa_cluster_permute;
 *   sizes are their differences).  crow_ptr / ccol: the cluster CSR of
 *   bsa_cluster_select (rows (b * H + h) * Nq + i, key clusters in [0, Nk)).
 * N: tokens per head (bounds the key cluster sizes).  Nq, Nk <= 4096.
 * sides: uint8 [B, H, rounds, Nq] (may be NULL when rounds = 0); rounds 0..64.
 * group_of (out): int32 [B, H, Nq], the name of every cluster's group.
 * workspace: >= bsa_cluster_merge_workspace_bytes(B, H, N, Nq, Nk, grain)
 *   bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
int64_t bsa_cluster_merge_workspace_bytes(int32_t B, int32_t H, int32_t N,
                                          int32_t Nq, int32_t Nk,
                                          int32_t grain);

bsa_status bsa_cluster_merge(const int32_t* off_q, const int32_t* off_k,
                             const int32_t* crow_ptr, const int32_t* ccol,
                             int32_t B, int32_t H, int32_t N, int32_t Nq,
                             int32_t Nk, const uint8_t* sides, int32_t rounds,
                             int32_t tau_q, int32_t tau_k, int32_t grain,
                             int32_t* group_of, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_cluster_attn_fwd -- attention over cluster-induced blocks
 * (HyperVAttention section 2, Eq. 4; merged groups of section 4.3, Eq. 8):
 * every query of query cluster i attends over the tokens of the key clusters
 * in the union of the rows of its group (its own row when group_of is NULL);
 * O and LSE are written in the original token order (O = Pi_q^-1 O').
 *   LSE[t] = ln sum_tau exp(scale q_t . k_tau), O[t] = sum_tau softmax v_tau
 * over those keys; a group with no key cluster gets O = 0, LSE = -inf.
 * Executed as Eq. 8 describes: each group's queries fill whole 64-query
 * tiles; the key clusters are padded to whole 16-key chunks and a group's
 * chunks are packed four to a 64-key tile; padding keys are masked, so the
 * result is exactly Eq. 4.  Precision as bsa_sparse_attn_fwd.
 *
 * perm_q / off_q: bsa_cluster_permute of the query clustering ([B,H,N],
 *   [B,H,Nq+1]); perm_k / off_k the same for the keys ([B,H,Nk+1]).
 *   Nq, Nk <= 4096.
 * crow_ptr / ccol: cluster CSR with rows (b * H + h) * Nq + i and key cluster
 *   indices in [0, Nk) (bsa_cluster_select); entries outside are ignored.
 * group_of: int32 [B, H, Nq] group names (bsa_cluster_merge: the lowest
 *   member) or NULL; a name outside [0, i] makes cluster i its own group.
 * O: [B, H, N, d] with the strides of `shape`, o_dtype BSA_F32 or BSA_BF16;
 *   LSE: float32 [B, H, N].
 * out_tile_pairs: device int64 or NULL; receives the number of executed
 *   (query tile, key tile) pairs, C(S) / 64^2 summed over the groups.
 * workspace: >= bsa_cluster_attn_workspace_bytes(shape, Nq, Nk, o_dtype)
 *   bytes, 256-byte aligned (the padded copy of K, the staged V^T by chunk,
 *   the query source map and the chunk lists): padded length per head
 *   64 * max(ceil(N/64) + Nq, ceil((ceil(N/16) + Nk + 1) / 4)).  Queries are
 *   read, and O and LSE written, in the caller's layout.
 * ---------------------------------------------------------------------- */
int64_t bsa_cluster_attn_workspace_bytes(const bsa_shape* shape, int32_t Nq,
                                         int32_t Nk, int32_t o_dtype);

bsa_status bsa_cluster_attn_fwd(const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const bsa_shape* shape,
                                float scale, int32_t Nq, int32_t Nk,
                                const int32_t* perm_q, const int32_t* off_q,
                                const int32_t* perm_k, const int32_t* off_k,
                                const int32_t* crow_ptr, const int32_t* ccol,
                                const int32_t* group_of, void* O,
                                int32_t o_dtype, float* LSE,
                                int64_t* out_tile_pairs, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * bsa_omission_risk -- per-head omission risk of a sparse support.  The
 * HyMoR-Attn abstract finds the risk of omitting valuable support stable per
 * layer and head and calibrates it offline to pick the heads that get the
 * Micro residual; it gives no formula.  Reading used here: the risk of a
 * query row is the share of its full softmax mass outside its support,
 *   w = 1 - exp(LSE_sparse - LSE_full),
 * and a repair over a disjoint support (the Micro residual merged by
 * bsa_lse_merge) brings back
 *   g = exp(LSE_repaired - LSE_full) - exp(LSE_sparse - LSE_full).
 * Rows whose LSE_full is -inf count 0 for both; an empty support
 * (LSE_sparse = -inf) has w = 1.
 *
 * lse_sparse, lse_full: float32 [B, H, N] (bsa_sparse_attn_fwd and
 *   bsa_dense_attn_fwd on the same Q, K); lse_repaired: float32 [B, H, N]
 *   or NULL (then g = 0).  Only B, H and N of `shape` are read; B*H must be
 *   at most 65535.
 * risk: float64 [B, H, 3]: mean of w over the N rows, largest w, mean of g.
 *   Per-row shares are computed in float32 (expm1 forms), sums in float64
 *   in a fixed order (deterministic).
 * workspace: device, >= bsa_omission_risk_workspace_bytes(shape) bytes,
 *   8-byte aligned; its contents on entry do not matter.
 * ---------------------------------------------------------------------- */
int64_t bsa_omission_risk_workspace_bytes(const bsa_shape* shape);

bsa_status bsa_omission_risk(const float* lse_sparse, const float* lse_full,
                             const float* lse_repaired, const bsa_shape* shape,
                             double* risk, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* bsa_heads_at_risk -- the offline calibration step that follows
 * bsa_omission_risk: head_mask[h] = 1 for the n heads of largest mean
 * omitted share (equal shares to the lower head index), 0 for the others;
 * the mask bsa_select_blocks (MICRO) and bsa_micro_residual_fwd take.
 * mean_omitted: host float64 [H] (risk[b, h, 0] of one batch, copied to
 * the host); head_mask: host uint8 [H].  n is clamped to [0, H].  NaN
 * shares are rejected (BSA_ERR_INVALID_ARG).  Needs no GPU. */
bsa_status bsa_heads_at_risk(const double* mean_omitted, int32_t H, int32_t n,
                             uint8_t* head_mask);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
