// Kernel argument structs and launchers shared by the C-ABI layer (api.hip)
// and the kernel translation units.  Host and device visible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kMaxHeads = 256;  // heads per (b) a head list can name

// Compact list of head indices, passed by value to kernels.
struct HeadList {
  int32_t n;
  int32_t h[kMaxHeads];
};

struct PoolArgs {
  const uint16_t* Q;
  const uint16_t* K;
  int64_t sb, sh, sn;
  int H, N, D, nB, nT;
  int block;       // tokens per pooled block: 64 or 128
  float* qpool;
  float* kpool;
  float* qpool16;  // may be null
  float* kpool16;  // may be null
};

struct GemmArgs {
  const float* A;   // [B*H, M, D]
  const float* Bm;  // [B*H, Nc, D]
  float* C;         // [nbatch, M, Nc]
  int H, M, Nc, D;
  float scale;
  HeadList heads;   // batch z -> (z / heads.n, heads.h[z % heads.n])
};

constexpr int kMaxPatterns = 64;  // diagonal offsets / columns per selection

struct SelectArgs {
  const float* scores;  // [rows, nB] or null
  uint32_t* bits;       // [rows, W]
  int32_t* counts;      // [rows]
  int N, nB, W;
  int block;            // tokens per selection block: 64 or 128
  int mode, k, k_min, k_cap;
  float p;
  int force_diag, use_static;
  int frame_tokens, window_frames, n_anchors, anchor_offset;
  const int32_t* col_sizes;          // top-p weights per key column [heads, nB], or null
  int rows_per_head;                 // rows of one (b, h): nB for blocks, Nq for clusters
  int n_diag, n_col;                 // MOD-DiT parallel-diagonal / vertical patterns
  int32_t diag[kMaxPatterns];        // offsets: key block i + diag[t]
  int32_t col[kMaxPatterns];         // key blocks
  // direct > 0: every row holds exactly `direct` blocks (plain top-k on
  // 64-token blocks), so the kernel writes the CSR itself: row r starts at
  // r * direct, no bitmask, count or scan
  int direct;
  int rows;
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t col_cap;
  int64_t* out_nnz;
};

struct MicroSelectArgs {
  const float* sigma;          // [B*nh, nT, nT]
  const int32_t* macro_row_ptr;
  const int32_t* macro_col_idx;
  int32_t* slots;              // [rows, m]
  int32_t* counts;             // [rows]
  int H, nB, nT, W, m;
  HeadList heads;
};

struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* Vt;  // [B*H, D, Npad] key-major, 16-key chunks permuted
  void* O;
  float* LSE;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t sb, sh, sn;
  int B, H, N, nB, Npad;
  float scale_log2;  // softmax scale * log2(e)
  int rows;          // B*H*nB
  int per_xcd;       // ceil(rows / 8)
  // chunk kernel only: group of every query tile (-1: none), groups per
  // head, the token of every padded query position (-1: none) and the
  // tokens per head of Q, O and LSE, and the strides of the padded K
  const int32_t* tile_group;
  int ngroups;
  const int32_t* qsrc;
  int Nout;
  int64_t ksb, ksh, ksn;
  // sparse kernel: bit kStatusBadIndex is OR-ed in when a column index lies
  // outside [0, nB) (that entry is skipped); a word of the workspace
  int32_t* status;
};

// Status bits of the attention workspace's status word.
constexpr int32_t kStatusBadIndex = 1;

// 16-key chunk codes of packed cluster-induced blocks: chunk index in the low
// 24 bits, its valid keys (0..16) above.
constexpr int kChunkShift = 24;
constexpr int32_t kChunkMask = (1 << kChunkShift) - 1;

// waves (query sub-tiles) per workgroup of the micro residual: one, so that
// a sub-tile that ends early frees its LDS slots at once (4.13-4.18 ms with
// two per workgroup, 3.98-4.11 with one, 4.50-4.52 with four on the
// HunyuanVideo micro heads, bit-identical)
constexpr int kMicroWaves = 1;

struct MicroAttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* Vt;
  void* O;
  float* LSE;
  const int32_t* row_ptr;
  const int32_t* idx;
  int64_t sb, sh, sn;
  int H, N, nB, Npad;
  float scale_log2;
  HeadList heads;
  // sub-tile order: entry k of `order` is sub-tile (z * nB + i) * 4 + a (z =
  // b * heads.n + micro head slot); workgroup slots are dealt to the XCDs in
  // contiguous ranges of that order
  int32_t* sig;      // [slots] global bin of each sub-tile (workspace)
  int32_t* order;    // [slots] (workspace)
  int32_t* hist;     // [bins] counts, then (after the scan) cursors
  int32_t* offsets;  // [bins + 1] (workspace)
  int64_t* nnz;      // scan total (workspace)
  int32_t* status;   // kStatusBadIndex when a tile index lies outside [0, nT)
  int slots, bins, nT, per_xcd;
};

struct CsrCheckArgs {
  const int32_t* row_ptr;  // [rows + 1]
  const int32_t* col_idx;  // [cap]
  int64_t cap;
  int rows, n_cols;
  int32_t* counts;         // [3]: bad row pointers, entries out of range, entries not ascending
};

struct TransposeArgs {
  const uint16_t* V;
  uint16_t* Vt;
  int64_t sb, sh, sn;
  int H, N, nB, Npad;
  HeadList heads;  // heads to transpose (all for macro/dense attention)
};

struct MergeArgs {
  const void* O1;
  const float* L1;
  const void* O2;
  const float* L2;
  void* O;
  float* L;
  int64_t sb, sh, sn;
  int H, N, D;
  HeadList heads;
};

// Omission risk: rows of one head are reduced in chunks of kRiskRowsPerChunk.
constexpr int kRiskRowsPerChunk = 2048;

struct RiskArgs {
  const float* Ls;  // [BH, N] sparse-support LSE
  const float* Lf;  // [BH, N] full-attention LSE
  const float* Lr;  // [BH, N] repaired LSE, or null
  double* partial;  // [BH, chunks, 3] workspace
  double* risk;     // [BH, 3]
  int N, chunks, BH;
};

// 3D local-window clustering.
struct ClusterArgs {
  const uint16_t* X;   // [B, H, N, D] with strides (Q or K)
  int64_t sb, sh, sn;
  int H, N, D;
  int T, Hg, W;        // token lattice, T * Hg * W = N
  int kt, kh, kw;      // cell size
  int Kt, Kh, Kw, Nc;  // cells per axis, centroids
  int wt, wh, ww;      // window in cells, clipped to the grid
  int32_t* assign;     // [BH, N]
  float* mu;           // [BH, Nc, D]
  float* norm;         // [BH, Nc] squared norms of the centroids (workspace)
  int32_t* counts;     // [BH, Nc]
  float* rho;          // [BH, N] Lowe's ratio (ratio pass only)
  uint16_t* mu3;       // [BH, Nc, 3, D] bf16 hi, mid, lo parts of the centroids (workspace)
  int32_t* bucket;     // [BH, Nc, kt*kh*kw] tokens of each cell by window slot, or NULL
  int32_t* bstart;     // [BH, Nc, wt*wh*ww + 1] slot starts
};
// Bucketed update limits: tokens per cell and window slots.
constexpr int kMaxBucketCell = 2048;
constexpr int kMaxBucketSlots = 1023;
constexpr int kMaxAssignWindow = 1024;  // window cells the prefetching assignment tabulates

// Attention over cluster-induced blocks (padded cluster order).
struct ClusterAttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  int64_t sb, sh, sn;      // strides of Q, K, V, O
  int H, N, Nq, Nk;
  int NP, nTP;             // padded length per head and its query tiles (NP / 64)
  int W;                   // 32-bit words of a key-cluster mask
  const int32_t* perm_q;   // [BH, N]
  const int32_t* off_q;    // [BH, Nq + 1]
  const int32_t* perm_k;
  const int32_t* off_k;    // [BH, Nk + 1]
  const int32_t* crow_ptr; // cluster lists [BH * Nq + 1]
  const int32_t* ccol;
  const int32_t* group_of; // [BH, Nq] lowest member of each cluster's group, or NULL
  int32_t* gtile;          // [BH, Nq + 1] first query tile of each group (at its lowest member)
  int32_t* qpos;           // [BH, Nq] padded position of each query cluster's first token
  int32_t* kc;             // [BH, Nk + 1] first 16-key chunk of each key cluster
  int32_t* tile_group;     // [BH, nTP]
  int32_t* srcq;           // [BH, NP] token at each padded query position, -1 in padding
  uint32_t* gmask;         // [BH, Nq, W] key clusters of each group
  int32_t* counts;         // [BH * Nq] chunk entries of each group (multiple of 4)
  int32_t* row_ptr;        // [BH * Nq + 1]
  int32_t* col_idx;        // chunk codes
  int64_t cap;
  unsigned long long* pairs;  // executed (query tile, key tile) pairs
  uint16_t* Kp;            // [BH, NP, D] keys by chunk
  uint16_t* Vt;            // [BH, NP / 16, D, 16] staged fp16 V^T by chunk
};

// HVA parallel agglomerative merging of query clusters.
struct ClusterMergeArgs {
  int Nq, Nk, W, nbits;    // W mask words, nbits bit planes of the key slot counts
  int rounds, round;
  int tau_q, tau_k, grain;
  const int32_t* off_q;    // [BH, Nq + 1]
  const int32_t* off_k;    // [BH, Nk + 1]
  const int32_t* crow_ptr; // [BH * Nq + 1]
  const int32_t* ccol;
  const uint8_t* sides;    // [BH, rounds, Nq]
  int32_t* grp;            // [BH, Nq] lowest member of each cluster's group (the output)
  int32_t* gsq;            // [BH, Nq] query tokens of each group (at its lowest member)
  int32_t* gk;             // [BH, Nq] key slots of each group
  uint32_t* gmask;         // [BH, Nq, W]
  uint32_t* planes;        // [BH, nbits, W] bit b of every key cluster's slot count
  int32_t* alist;          // [BH, Nq] choosing groups of this round, then their count
  int32_t* blist;          // [BH, Nq] target groups
  int32_t* nab;            // [BH, 2]
  int32_t* choice;         // [BH, Nq] best target of each chooser (-1 none)
  int64_t* gain;           // [BH, Nq]
  int32_t* ukeys;          // [BH, Nq] key slots of chooser + best target
  int32_t* hbits;          // [BH] bit planes in use per head (largest slot count)
};
// Most query or key clusters per head of the cluster attention plan and the
// merging (per-head tables held in LDS; key masks of at most 128 words).
constexpr int kMaxClusters = 4096;

// HVA subset refinement (intermediate-step update of the hybrid clustering).
struct RefineArgs {
  const uint16_t* X;        // [B, H, N, D] with strides
  int64_t sb, sh, sn;
  int H, N, Nc, W;          // W: 32-bit words of a head's touched bitmap
  const int32_t* subset;    // [BH, n_sub] token indices
  int n_sub;
  int32_t* assign;          // [BH, N] in/out
  float* mu;                // [BH, Nc, D] in/out
  int32_t* counts;          // [BH, Nc] in/out
  uint32_t* touched;        // [BH, W] (workspace)
  int32_t* tcount;          // [BH, Nc] members of touched centroids (workspace)
  int32_t* offs;            // [BH * Nc + 1] their ranges in `list` (workspace)
  int64_t* total;           // the scan's total (workspace)
  int32_t* list;            // [BH * N] members of touched centroids (workspace)
  uint16_t* mu3;            // [BH, Nc, 3, D] bf16 parts of the centroids (workspace)
  float* norm;              // [BH, Nc] squared norms of the centroids (workspace)
};

hipError_t launch_subset_refine(const RefineArgs& a, int BH, int D, hipStream_t s);

// Pooled rectification of omitted blocks.
constexpr int kMaxRowWords = 128;  // bitmap words of a row of up to 4096 blocks

struct RectifyArgs {
  const uint16_t* Q;
  const float* Kf;   // [BH, nB, D] 64-token means of K (workspace)
  const float* Vf;   // [BH, nB, D] 64-token means of V (workspace)
  uint16_t* Khi;     // [BH, nBp, D] bf16 high part of Kbar
  uint16_t* Klo;     // [BH, nBp, D] bf16 low part
  uint16_t* Vt;      // [BH, nBp/16, D, 16] fp16 Vbar, 16-block chunks
  const int32_t* row_ptr;
  const int32_t* col_idx;
  void* O;           // in: sparse result; out: rectified
  float* LSE;
  const uint16_t* K;  // the keys (gain-aware gate: spread of each block)
  float* spread;      // [BH, nBp] per-coordinate key variance of each block
  int64_t sb, sh, sn;
  int H, N, nB, nBp;
  float scale_log2;
  int gate;           // 1: keep block j for query q only if |q|^2 spread_j < gate_thr
  float gate_thr;     // 2 ln 2 / scale^2
};

hipError_t launch_pool(const PoolArgs& a, int B, hipStream_t s);
hipError_t launch_score_gemm(const GemmArgs& a, int nbatch, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_csr_check(const CsrCheckArgs& a, hipStream_t s);
hipError_t launch_take_status(int32_t* status, int32_t* out, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s);
hipError_t launch_expand_bits(const uint32_t* bits_sel, int W_sel, int nB_sel,
                              uint32_t* bits64, int32_t* counts64, int W64, int nB64,
                              int rows64, hipStream_t s);
hipError_t launch_scan(const int32_t* counts, int rows, int32_t* row_ptr,
                       int64_t* out_nnz, hipStream_t s);
hipError_t launch_emit_bits(const uint32_t* bits, int W, int rows,
                            const int32_t* row_ptr, int32_t* col_idx,
                            int64_t cap, hipStream_t s);
hipError_t launch_micro_select(const MicroSelectArgs& a, int B, hipStream_t s);
hipError_t launch_emit_slots(const int32_t* slots, int m, int rows,
                             const int32_t* row_ptr, int32_t* col_idx,
                             int64_t cap, hipStream_t s);
hipError_t launch_transpose_v(const TransposeArgs& a, int B, int D,
                              hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int D, bool dense, bool out_bf16,
                       hipStream_t s);
hipError_t launch_attn_chunks(const AttnArgs& a, int D, bool out_bf16, hipStream_t s);
hipError_t launch_micro_attn(const MicroAttnArgs& a, int B, int D,
                             bool out_bf16, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int B, bool bf16, hipStream_t s);
hipError_t launch_risk(const RiskArgs& a, hipStream_t s);
hipError_t launch_cluster(const ClusterArgs& a, int BH, int iters, hipStream_t s);
hipError_t launch_cluster_permute(const ClusterArgs& a, int BH, const int32_t* gofs,
                                  int32_t* perm, int32_t* offsets, int32_t* big, hipStream_t s);
hipError_t launch_cluster_attn_plan(const ClusterAttnArgs& a, int BH, int D, hipStream_t s);
hipError_t launch_cluster_attn_emit(const ClusterAttnArgs& a, int BH, int D, hipStream_t s);
hipError_t launch_cluster_merge(const ClusterMergeArgs& a, int BH, hipStream_t s);
hipError_t launch_lowe(const ClusterArgs& a, int BH, int n_sub, int32_t* subset, hipStream_t s);

hipError_t launch_rectify(const RectifyArgs& a, int BH, int D, bool out_bf16, hipStream_t s);

}  // namespace bsa
