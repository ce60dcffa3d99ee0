// C-ABI entry points declared in include/bsa.h: argument validation (before
// any HIP call), workspace carving and kernel launches on the caller's
// stream.  No state is kept between calls and nothing is allocated.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "bsa.h"
#include "bsa_internal.h"

namespace {

thread_local std::string g_last_error;

bsa_status fail(bsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bsa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bsa_status check_shape(const bsa_shape* s) {
  if (s == nullptr) return fail(BSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->N < 1)
    return fail(BSA_ERR_INVALID_ARG, "shape B=%d H=%d N=%d must all be >= 1", s->B, s->H, s->N);
  if (s->d != 64 && s->d != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", s->d);
  if (s->H > bsa::kMaxHeads)
    return fail(BSA_ERR_UNSUPPORTED, "H=%d exceeds %d heads", s->H, bsa::kMaxHeads);
  if (s->B > 32767) return fail(BSA_ERR_UNSUPPORTED, "B=%d exceeds 32767", s->B);
  if (s->stride_n < s->d || s->stride_h < 0 || s->stride_b < 0)
    return fail(BSA_ERR_INVALID_ARG, "strides (b=%lld h=%lld n=%lld) inconsistent with d=%d",
                (long long)s->stride_b, (long long)s->stride_h, (long long)s->stride_n, s->d);
  if (s->stride_n % 8 || s->stride_h % 8 || s->stride_b % 8)
    return fail(BSA_ERR_INVALID_ARG, "strides must be multiples of 8 elements");
  const int64_t nB = cdiv(s->N, 64);
  if ((int64_t)s->B * s->H * nB >= INT32_MAX / 2)
    return fail(BSA_ERR_UNSUPPORTED, "too many query blocks");
  return BSA_OK;
}

bsa_status check_ptr(const void* p, const char* name, uintptr_t align = 16) {
  if (p == nullptr) return fail(BSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align))
    return fail(BSA_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, (unsigned)align);
  return BSA_OK;
}

#define BSA_TRY(expr)                   \
  do {                                  \
    const bsa_status _st = (expr);      \
    if (_st != BSA_OK) return _st;      \
  } while (0)

// The omission-risk reduction reads only B, H and N (LSE arrays are
// contiguous [B, H, N]); heads map to grid rows, at most 65535 of them.
bsa_status check_risk_shape(const bsa_shape* s, int64_t* chunks) {
  if (s == nullptr) return fail(BSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->N < 1)
    return fail(BSA_ERR_INVALID_ARG, "shape B=%d H=%d N=%d must all be >= 1", s->B, s->H, s->N);
  const int64_t bh = (int64_t)s->B * s->H;
  if (bh > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)bh);
  *chunks = cdiv(s->N, bsa::kRiskRowsPerChunk);
  return BSA_OK;
}

struct RectifyPlan {
  int64_t nB, nBp, BH, bytes_f, bytes_h, bytes_s, total;
};

bsa_status plan_rectify(const bsa_shape* s, RectifyPlan* pl) {
  BSA_TRY(check_shape(s));
  pl->nB = cdiv(s->N, 64);
  if (pl->nB > 32 * bsa::kMaxRowWords)
    return fail(BSA_ERR_UNSUPPORTED, "nB=%lld exceeds %d blocks", (long long)pl->nB,
                32 * bsa::kMaxRowWords);
  pl->BH = (int64_t)s->B * s->H;
  if (pl->BH > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  pl->nBp = cdiv(pl->nB, 16) * 16;
  pl->bytes_f = align256(pl->BH * pl->nB * s->d * 4);   // each of Kbar, Vbar (float32)
  pl->bytes_h = align256(pl->BH * pl->nBp * s->d * 2);  // each of Khi, Klo, Vbar^T (16-bit)
  pl->bytes_s = align256(pl->BH * pl->nBp * 4);          // key spread per block (gate)
  pl->total = 2 * pl->bytes_f + 3 * pl->bytes_h + pl->bytes_s;
  return BSA_OK;
}

// Attention workspace: the fp16 V^T copy, then the micro residual's
// sub-tile ordering (signatures, order, bin counts and offsets, a total),
// sized for every head.
struct MicroOrderPlan {
  int64_t vt_bytes, sig_off, order_off, hist_off, offs_off, nnz_off, status_off, order_bytes;
};

MicroOrderPlan plan_micro_order(const bsa_shape* s) {
  MicroOrderPlan m{};
  const int64_t nB = cdiv(s->N, 64), nT = cdiv(s->N, 16);
  const int64_t bh = (int64_t)s->B * s->H;
  m.vt_bytes = align256(bh * s->d * nB * 64 * 2);
  const int64_t slots = bh * nB * 4, bins = bh * (nT + 1);
  m.sig_off = m.vt_bytes;
  m.order_off = m.sig_off + align256(slots * 4);
  m.hist_off = m.order_off + align256(slots * 4);
  m.offs_off = m.hist_off + align256(bins * 4);
  m.nnz_off = m.offs_off + align256((bins + 1) * 4);
  m.status_off = m.nnz_off + 256;  // the status word: the last 256 bytes
  m.order_bytes = m.status_off + 256 - m.vt_bytes;
  return m;
}

// Tokens of a whole cell, and cells of a window (clipped to the grid).
int64_t cell_tokens(const bsa_cluster_params* p) { return (int64_t)p->kt * p->kh * p->kw; }

int64_t window_slots(const bsa_cluster_params* p) {
  return std::min<int64_t>(p->wt, cdiv(p->T, p->kt)) * std::min<int64_t>(p->wh, cdiv(p->Hg, p->kh)) *
         std::min<int64_t>(p->ww, cdiv(p->W, p->kw));
}

// Largest number of cells whose windows contain one cell, along one axis of
// K cells with windows of w (shifted to stay inside the grid).
int64_t max_covering(int64_t K, int64_t w) {
  w = std::min(w, K);
  int64_t best = 0;
  for (int64_t v = 0; v < K; ++v) {
    int64_t n = 0;
    for (int64_t g = 0; g < K; ++g) {
      const int64_t s = std::min(std::max(g - w / 2, (int64_t)0), K - w);
      if (s <= v && v < s + w) ++n;
    }
    best = std::max(best, n);
  }
  return best;
}

// The bucketed centroid update keeps a cell's tokens, a window's slots and a
// centroid's covering cells in LDS tables of fixed size.
bool bucket_update_fits(const bsa_cluster_params* p) {
  const int64_t cov = max_covering(cdiv(p->T, p->kt), p->wt) *
                      max_covering(cdiv(p->Hg, p->kh), p->wh) *
                      max_covering(cdiv(p->W, p->kw), p->ww);
  return cell_tokens(p) <= bsa::kMaxBucketCell && window_slots(p) <= bsa::kMaxBucketSlots &&
         cov <= bsa::kMaxBucketSlots;
}

bsa_status plan_cluster(const bsa_shape* s, const bsa_cluster_params* p, int64_t* cells) {
  if (s == nullptr || p == nullptr) return fail(BSA_ERR_INVALID_ARG, "shape or params is NULL");
  if (s->B < 1 || s->H < 1 || s->N < 1)
    return fail(BSA_ERR_INVALID_ARG, "shape B=%d H=%d N=%d must all be >= 1", s->B, s->H, s->N);
  if (s->d != 64 && s->d != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", s->d);
  if ((int64_t)s->B * s->H > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  if (p->T < 1 || p->Hg < 1 || p->W < 1 || (int64_t)p->T * p->Hg * p->W != s->N)
    return fail(BSA_ERR_INVALID_ARG, "lattice %d x %d x %d does not hold N=%d tokens", p->T, p->Hg,
                p->W, s->N);
  if (p->kt < 1 || p->kh < 1 || p->kw < 1 || p->wt < 1 || p->wh < 1 || p->ww < 1)
    return fail(BSA_ERR_INVALID_ARG, "cell and window sizes must be >= 1");
  if (p->iters < 1) return fail(BSA_ERR_INVALID_ARG, "iters=%d < 1", p->iters);
  *cells = cdiv(p->T, p->kt) * cdiv(p->Hg, p->kh) * cdiv(p->W, p->kw);
  return BSA_OK;
}

// Workspace of bsa_cluster_attn_fwd, carved in this order.  Queries are
// padded per group to whole 64-tiles (at most ceil(N/64) + Nq tiles per
// head), keys per cluster to whole 16-chunks plus one all-padding chunk (at
// most ceil(N/16) + Nk + 1 chunks); both layouts share one length NP.
struct ClusterAttnPlan {
  int64_t NP, nTP, BH, W;
  int64_t gt, qpos, kc, tg, srcq, gmask, cnt, rp, pairs, nent, kp, vt, col, total, cap;
};

bsa_status plan_cluster_attn(const bsa_shape* s, int32_t Nq, int32_t Nk, int32_t o_dtype,
                             ClusterAttnPlan* pl) {
  BSA_TRY(check_shape(s));
  if (Nq < 1 || Nk < 1) return fail(BSA_ERR_INVALID_ARG, "Nq=%d, Nk=%d must be >= 1", Nq, Nk);
  if (Nq > bsa::kMaxClusters || Nk > bsa::kMaxClusters)
    return fail(BSA_ERR_UNSUPPORTED, "Nq=%d, Nk=%d: at most %d clusters per head", Nq, Nk,
                bsa::kMaxClusters);
  if (o_dtype != BSA_F32 && o_dtype != BSA_BF16)
    return fail(BSA_ERR_INVALID_ARG, "o_dtype=%d (BSA_F32 or BSA_BF16)", o_dtype);
  ClusterAttnPlan p{};
  p.BH = (int64_t)s->B * s->H;
  if (p.BH > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  const int64_t q_tiles = cdiv(s->N, 64) + Nq;
  const int64_t k_chunks = cdiv(s->N, 16) + Nk + 1;
  p.nTP = std::max(q_tiles, cdiv(k_chunks, 4));
  p.NP = 64 * p.nTP;
  p.W = cdiv(Nk, 32);
  // every label's row can hold every chunk, rounded up to a whole tile
  p.cap = p.BH * Nq * (k_chunks + 3);
  if (p.cap >= INT32_MAX || p.BH * p.NP * s->d >= ((int64_t)1 << 40))
    return fail(BSA_ERR_UNSUPPORTED, "cluster layout too large (%lld chunk entries)",
                (long long)p.cap);
  const int64_t d = s->d;
  int64_t at = 0;
  auto take = [&](int64_t bytes) {
    const int64_t here = at;
    at += align256(bytes);
    return here;
  };
  p.gt = take(p.BH * (Nq + 1) * 4);
  p.qpos = take(p.BH * Nq * 4);
  p.kc = take(p.BH * (Nk + 1) * 4);
  p.tg = take(p.BH * p.nTP * 4);
  p.srcq = take(p.BH * p.NP * 4);
  p.gmask = take(p.BH * Nq * p.W * 4);
  p.cnt = take(p.BH * Nq * 4);
  p.rp = take((p.BH * Nq + 1) * 4);
  p.pairs = take(8);
  p.nent = take(8);
  p.kp = take(p.BH * p.NP * d * 2);
  p.vt = take(p.BH * p.NP * d * 2);
  p.col = take(p.cap * 4);
  p.total = at;
  *pl = p;
  return BSA_OK;
}

// Workspace of bsa_cluster_merge.
struct ClusterMergePlan {
  int64_t BH, W, nbits;
  int64_t gsq, gk, alist, blist, nab, choice, gain, ukeys, gmask, planes, hbits, total;
};

bsa_status plan_cluster_merge(int32_t B, int32_t H, int32_t N, int32_t Nq, int32_t Nk,
                              int32_t grain, ClusterMergePlan* pl) {
  if (B < 1 || H < 1 || N < 1 || Nq < 1 || Nk < 1)
    return fail(BSA_ERR_INVALID_ARG, "B=%d H=%d N=%d Nq=%d Nk=%d must be >= 1", B, H, N, Nq, Nk);
  if (Nq > bsa::kMaxClusters || Nk > bsa::kMaxClusters)
    return fail(BSA_ERR_UNSUPPORTED, "Nq=%d, Nk=%d: at most %d clusters per head", Nq, Nk,
                bsa::kMaxClusters);
  if (grain < 1) return fail(BSA_ERR_INVALID_ARG, "grain=%d must be >= 1", grain);
  ClusterMergePlan p{};
  p.BH = (int64_t)B * H;
  if (p.BH > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  p.W = cdiv(Nk, 32);
  const int64_t cmax = cdiv(N, grain);  // largest slot count of a key cluster
  p.nbits = 1;
  while ((int64_t(1) << p.nbits) <= cmax) ++p.nbits;
  int64_t at = 0;
  auto take = [&](int64_t bytes) {
    const int64_t here = at;
    at += align256(bytes);
    return here;
  };
  p.gsq = take(p.BH * Nq * 4);
  p.gk = take(p.BH * Nq * 4);
  p.alist = take(p.BH * Nq * 4);
  p.blist = take(p.BH * Nq * 4);
  p.nab = take(p.BH * 2 * 4);
  p.choice = take(p.BH * Nq * 4);
  p.gain = take(p.BH * Nq * 8);
  p.ukeys = take(p.BH * Nq * 4);
  p.gmask = take(p.BH * Nq * p.W * 4);
  p.planes = take(p.BH * p.nbits * p.W * 4);
  p.hbits = take(p.BH * 4);
  p.total = at;
  *pl = p;
  return BSA_OK;
}

bsa::HeadList all_heads(int H) {
  bsa::HeadList l;
  l.n = H;
  for (int h = 0; h < H; ++h) l.h[h] = h;
  return l;
}

bsa::HeadList heads_from_mask(const uint8_t* mask, int H) {
  bsa::HeadList l;
  l.n = 0;
  for (int h = 0; h < H; ++h)
    if (mask == nullptr || mask[h]) l.h[l.n++] = h;
  return l;
}

// Selection of a (b, h) batch of rows.  `sel` quantities are counted in
// selection blocks (64 or 128 tokens), `rows`/`nB`/`W` in the 64-token tiles
// the CSR is emitted on (equal when block = 64).
struct SelectPlan {
  int64_t rows, nB, W, nT;
  int64_t block, rows_sel, nB_sel, W_sel;
  int64_t bytes_a, bytes_b, bytes_c, bytes_d, total;
  bsa::HeadList heads;
};

bsa_status plan_select(const bsa_shape* s, int32_t block, const bsa_select_params* p,
                       SelectPlan* out) {
  BSA_TRY(check_shape(s));
  if (block != 64 && block != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block=%d unsupported (64 or 128)", block);
  if (p == nullptr) return fail(BSA_ERR_INVALID_ARG, "params is NULL");
  SelectPlan pl{};
  pl.nB = cdiv(s->N, 64);
  pl.rows = (int64_t)s->B * s->H * pl.nB;
  pl.W = cdiv(pl.nB, 32);
  pl.nT = cdiv(s->N, 16);
  pl.block = block;
  pl.nB_sel = cdiv(s->N, block);
  pl.rows_sel = (int64_t)s->B * s->H * pl.nB_sel;
  pl.W_sel = cdiv(pl.nB_sel, 32);
  if (p->mode != BSA_SELECT_MICRO) {
    if (p->n_diagonals < 0 || p->n_diagonals > bsa::kMaxPatterns || p->n_columns < 0 ||
        p->n_columns > bsa::kMaxPatterns)
      return fail(BSA_ERR_INVALID_ARG, "n_diagonals=%d, n_columns=%d (0..%d each)",
                  p->n_diagonals, p->n_columns, bsa::kMaxPatterns);
    if ((p->n_diagonals > 0 && p->diagonals == nullptr) ||
        (p->n_columns > 0 && p->columns == nullptr))
      return fail(BSA_ERR_INVALID_ARG, "pattern list is NULL");
    for (int t = 0; t < p->n_diagonals; ++t)
      if (p->diagonals[t] < -(1 << 24) || p->diagonals[t] > (1 << 24))
        return fail(BSA_ERR_INVALID_ARG, "diagonal offset %d out of range", p->diagonals[t]);
    for (int t = 0; t < p->n_columns; ++t)
      if (p->columns[t] < 0 || p->columns[t] >= pl.nB_sel)
        return fail(BSA_ERR_INVALID_ARG, "column %d outside [0, %lld)", p->columns[t],
                    (long long)pl.nB_sel);
  }
  switch (p->mode) {
    case BSA_SELECT_TOPK:
    case BSA_SELECT_TOPP:
    case BSA_SELECT_STATIC:
      if (p->mode != BSA_SELECT_STATIC && pl.nB_sel > 4096)
        return fail(BSA_ERR_UNSUPPORTED, "scored selection needs nB <= 4096 (nB=%lld)",
                    (long long)pl.nB_sel);
      if (pl.W > 128) return fail(BSA_ERR_UNSUPPORTED, "nB=%lld exceeds 4096", (long long)pl.nB);
      pl.bytes_a = align256(pl.rows_sel * pl.W_sel * 4);  // row bitmasks
      pl.bytes_b = align256(pl.rows_sel * 4);             // row counts
      if (block != 64) {
        pl.bytes_c = align256(pl.rows * pl.W * 4);  // the rows on 64-token tiles
        pl.bytes_d = align256(pl.rows * 4);
      }
      break;
    case BSA_SELECT_MICRO: {
      if (block != 64)
        return fail(BSA_ERR_UNSUPPORTED, "MICRO selection works on the 64-token CSR (block=64)");
      if (p->micro != 16) return fail(BSA_ERR_UNSUPPORTED, "micro=%d unsupported (16)", p->micro);
      if (p->micro_m < 0) return fail(BSA_ERR_INVALID_ARG, "micro_m=%d < 0", p->micro_m);
      if (pl.W > 128) return fail(BSA_ERR_UNSUPPORTED, "nB=%lld exceeds 4096", (long long)pl.nB);
      pl.heads = heads_from_mask(p->head_mask, s->H);
      const int64_t nbatch = (int64_t)s->B * pl.heads.n;
      if (nbatch > 65535) return fail(BSA_ERR_UNSUPPORTED, "too many micro heads");
      pl.bytes_a = align256(nbatch * pl.nT * pl.nT * 4);        // tile scores
      pl.bytes_b = align256(pl.rows * (int64_t)p->micro_m * 4);  // per-row slots
      pl.bytes_c = align256(pl.rows * 4);                        // row counts
      break;
    }
    default:
      return fail(BSA_ERR_INVALID_ARG, "unknown selection mode %d", p->mode);
  }
  pl.total = pl.bytes_a + pl.bytes_b + pl.bytes_c + pl.bytes_d;
  *out = pl;
  return BSA_OK;
}

int64_t max_nnz(const bsa_shape* s, const bsa_select_params* p, const SelectPlan& pl) {
  if (p->mode == BSA_SELECT_MICRO) {
    const int64_t per = std::min<int64_t>(p->micro_m, 4 * pl.nT);
    return (int64_t)s->B * pl.heads.n * pl.nB * per;
  }
  int64_t per = pl.nB_sel;
  if (!p->use_static) {
    int64_t base = 0;
    if (p->mode == BSA_SELECT_TOPK) base = std::max(p->k, 0);
    else if (p->mode == BSA_SELECT_TOPP) base = std::max(p->k_cap, 1);
    per = std::min<int64_t>(pl.nB_sel, base + (p->force_diag ? 1 : 0) + p->n_diagonals +
                                           p->n_columns);
  }
  // each selection block covers block / 64 tiles
  per = std::min<int64_t>(pl.nB, per * (pl.block / 64));
  return pl.rows * per;
}

bsa_status check_attn_common(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                             const bsa_shape* s, const void* O, int32_t o_dtype,
                             const float* LSE, const void* ws, int64_t ws_bytes) {
  BSA_TRY(check_shape(s));
  BSA_TRY(check_ptr(Q, "Q"));
  BSA_TRY(check_ptr(K, "K"));
  if (V != nullptr) BSA_TRY(check_ptr(V, "V"));
  BSA_TRY(check_ptr(O, "O"));
  BSA_TRY(check_ptr(LSE, "LSE", 4));
  BSA_TRY(check_ptr(ws, "workspace", 256));
  if (o_dtype != BSA_F32 && o_dtype != BSA_BF16)
    return fail(BSA_ERR_INVALID_ARG, "o_dtype=%d (BSA_F32 or BSA_BF16)", o_dtype);
  const int64_t need = bsa_attn_workspace_bytes(s);
  if (ws_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld", (long long)ws_bytes,
                (long long)need);
  return BSA_OK;
}

bsa_status run_attn(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const bsa_shape* s,
                    float scale, const int32_t* row_ptr, const int32_t* col_idx, void* O,
                    int32_t o_dtype, float* LSE, void* ws, bool dense, hipStream_t st) {
  const int nB = (int)cdiv(s->N, 64);
  bsa::TransposeArgs t{};
  t.V = V;
  t.Vt = (uint16_t*)ws;
  t.sb = s->stride_b;
  t.sh = s->stride_h;
  t.sn = s->stride_n;
  t.H = s->H;
  t.N = s->N;
  t.nB = nB;
  t.Npad = nB * 64;
  t.heads = all_heads(s->H);
  if (V != nullptr)
    BSA_TRY(hip_status(bsa::launch_transpose_v(t, s->B, s->d, st), "transpose_v launch"));
  bsa::AttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.Vt = (const uint16_t*)ws;
  a.O = O;
  a.LSE = LSE;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.sb = s->stride_b;
  a.sh = s->stride_h;
  a.sn = s->stride_n;
  a.B = s->B;
  a.H = s->H;
  a.N = s->N;
  a.nB = nB;
  a.Npad = nB * 64;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rows = s->B * s->H * nB;
  a.per_xcd = (int)cdiv(a.rows, 8);
  a.status = (int32_t*)((char*)ws + plan_micro_order(s).status_off);
  return hip_status(bsa::launch_attn(a, s->d, dense, o_dtype == BSA_BF16, st), "attn launch");
}

// Scratch of the no-allocation selection entry point: a file-scope device
// array that every GPU the library runs on holds until the process ends.
// Host code uses only the device address hipGetSymbolAddress returns for it
// (one per device, taken with that device current), never the array's name.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

bsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

}  // namespace

extern "C" {

const char* bsa_version(void) { return "bsa 0.1.0 gfx950"; }

const char* bsa_last_error(void) { return g_last_error.c_str(); }

bsa_status bsa_score_blocks(const uint16_t* Q, const uint16_t* K, const bsa_shape* shape,
                            int32_t block, float scale, float* qpool, float* kpool,
                            float* scores, int32_t micro, float* qpool16, float* kpool16,
                            void* stream) {
  BSA_TRY(check_shape(shape));
  if (block != 64 && block != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block=%d unsupported (64 or 128)", block);
  BSA_TRY(check_ptr(Q, "Q"));
  BSA_TRY(check_ptr(K, "K"));
  BSA_TRY(check_ptr(qpool, "qpool"));
  BSA_TRY(check_ptr(kpool, "kpool"));
  if (scores != nullptr) BSA_TRY(check_ptr(scores, "scores", 4));
  if (micro != 0 && micro != 16) return fail(BSA_ERR_UNSUPPORTED, "micro=%d (0 or 16)", micro);
  if (micro == 16) {
    BSA_TRY(check_ptr(qpool16, "qpool16"));
    BSA_TRY(check_ptr(kpool16, "kpool16"));
  }
  const int nB = (int)cdiv(shape->N, block);
  if ((int64_t)shape->B * shape->H > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  hipStream_t st = (hipStream_t)stream;
  bsa::PoolArgs p{};
  p.Q = Q;
  p.K = K;
  p.sb = shape->stride_b;
  p.sh = shape->stride_h;
  p.sn = shape->stride_n;
  p.H = shape->H;
  p.N = shape->N;
  p.D = shape->d;
  p.nB = nB;
  p.nT = (int)cdiv(shape->N, 16);
  p.block = block;
  p.qpool = qpool;
  p.kpool = kpool;
  p.qpool16 = micro ? qpool16 : nullptr;
  p.kpool16 = micro ? kpool16 : nullptr;
  BSA_TRY(hip_status(bsa::launch_pool(p, shape->B, st), "pool launch"));
  if (scores != nullptr) {
    bsa::GemmArgs g{};
    g.A = qpool;
    g.Bm = kpool;
    g.C = scores;
    g.H = shape->H;
    g.M = nB;
    g.Nc = nB;
    g.D = shape->d;
    g.scale = scale;
    g.heads = all_heads(shape->H);
    BSA_TRY(hip_status(bsa::launch_score_gemm(g, shape->B * shape->H, st), "score launch"));
  }
  return BSA_OK;
}

int64_t bsa_select_workspace_bytes(const bsa_shape* shape, int32_t block,
                                   const bsa_select_params* params) {
  SelectPlan pl;
  if (plan_select(shape, block, params, &pl) != BSA_OK) return -1;
  return pl.total;
}

int64_t bsa_select_max_nnz(const bsa_shape* shape, int32_t block,
                           const bsa_select_params* params) {
  SelectPlan pl;
  if (plan_select(shape, block, params, &pl) != BSA_OK) return -1;
  return max_nnz(shape, params, pl);
}

bsa_status bsa_select_blocks(const float* scores, const bsa_shape* shape, int32_t block,
                             const bsa_select_params* p, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_cap, int64_t* out_nnz, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  SelectPlan pl;
  BSA_TRY(plan_select(shape, block, p, &pl));
  BSA_TRY(check_ptr(row_ptr, "row_ptr", 4));
  BSA_TRY(check_ptr(out_nnz, "out_nnz", 8));
  if (col_cap < 0) return fail(BSA_ERR_INVALID_ARG, "col_cap < 0");
  if (col_cap > 0) BSA_TRY(check_ptr(col_idx, "col_idx", 4));
  if (pl.total > 0) BSA_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < pl.total)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)pl.total);
  const int64_t bound = max_nnz(shape, p, pl);
  if (bound > INT32_MAX)
    return fail(BSA_ERR_UNSUPPORTED, "up to %lld entries exceed int32 row pointers",
                (long long)bound);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int rows = (int)pl.rows;

  if (p->mode == BSA_SELECT_MICRO) {
    if (p->macro_row_ptr == nullptr || p->macro_col_idx == nullptr)
      return fail(BSA_ERR_INVALID_ARG, "MICRO mode needs the macro CSR");
    BSA_TRY(check_ptr(p->qpool16, "qpool16"));
    BSA_TRY(check_ptr(p->kpool16, "kpool16"));
    float* sigma = (float*)ws;
    int32_t* slots = (int32_t*)(ws + pl.bytes_a);
    int32_t* counts = (int32_t*)(ws + pl.bytes_a + pl.bytes_b);
    BSA_TRY(hip_status(bsa::launch_fill_i32(counts, rows, 0, st), "fill launch"));
    if (pl.heads.n > 0 && p->micro_m > 0) {
      bsa::GemmArgs g{};
      g.A = p->qpool16;
      g.Bm = p->kpool16;
      g.C = sigma;
      g.H = shape->H;
      g.M = (int)pl.nT;
      g.Nc = (int)pl.nT;
      g.D = shape->d;
      g.scale = p->scale;
      g.heads = pl.heads;
      BSA_TRY(hip_status(bsa::launch_score_gemm(g, shape->B * pl.heads.n, st), "micro score"));
      bsa::MicroSelectArgs m{};
      m.sigma = sigma;
      m.macro_row_ptr = p->macro_row_ptr;
      m.macro_col_idx = p->macro_col_idx;
      m.slots = slots;
      m.counts = counts;
      m.H = shape->H;
      m.nB = (int)pl.nB;
      m.nT = (int)pl.nT;
      m.W = (int)pl.W;
      m.m = p->micro_m;
      m.heads = pl.heads;
      BSA_TRY(hip_status(bsa::launch_micro_select(m, shape->B, st), "micro select"));
    }
    BSA_TRY(hip_status(bsa::launch_scan(counts, rows, row_ptr, out_nnz, st), "scan launch"));
    BSA_TRY(hip_status(
        bsa::launch_emit_slots(slots, std::max(p->micro_m, 1), rows, row_ptr, col_idx, col_cap, st),
        "emit launch"));
    return BSA_OK;
  }

  const bool scored = p->mode == BSA_SELECT_TOPK || p->mode == BSA_SELECT_TOPP;
  if (scored) BSA_TRY(check_ptr(scores, "scores", 4));
  if (p->mode == BSA_SELECT_TOPK && p->k < 0) return fail(BSA_ERR_INVALID_ARG, "k=%d < 0", p->k);
  if (p->mode == BSA_SELECT_TOPP) {
    if (!(p->p > 0.f && p->p <= 1.f)) return fail(BSA_ERR_INVALID_ARG, "p=%g not in (0,1]", p->p);
    if (p->k_min < 0 || p->k_cap < p->k_min)
      return fail(BSA_ERR_INVALID_ARG, "need 0 <= k_min <= k_cap (k_min=%d k_cap=%d)", p->k_min,
                  p->k_cap);
  }
  if (p->use_static) {
    if (p->frame_tokens <= 0) return fail(BSA_ERR_INVALID_ARG, "frame_tokens must be > 0");
    if (p->window_frames < 0) return fail(BSA_ERR_INVALID_ARG, "window_frames must be >= 0");
    if (p->n_anchors < 0) return fail(BSA_ERR_INVALID_ARG, "n_anchors must be >= 0");
  }
  bsa::SelectArgs a{};
  a.scores = scores;
  a.bits = (uint32_t*)ws;
  a.counts = (int32_t*)(ws + pl.bytes_a);
  a.N = shape->N;
  a.nB = (int)pl.nB_sel;
  a.W = (int)pl.W_sel;
  a.block = (int)pl.block;
  a.rows_per_head = (int)pl.nB_sel;
  a.mode = p->mode;
  a.k = p->k;
  a.k_min = p->k_min;
  a.k_cap = p->k_cap;
  a.p = p->p;
  a.force_diag = p->force_diag ? 1 : 0;
  a.use_static = p->use_static ? 1 : 0;
  a.frame_tokens = p->frame_tokens;
  a.window_frames = p->window_frames;
  a.n_anchors = p->n_anchors;
  a.anchor_offset = p->anchor_offset;
  a.n_diag = p->n_diagonals;
  a.n_col = p->n_columns;
  for (int t = 0; t < a.n_diag; ++t) a.diag[t] = p->diagonals[t];
  for (int t = 0; t < a.n_col; ++t) a.col[t] = p->columns[t];
  // Plain top-k on 64-token blocks keeps exactly min(k, nB) blocks per row:
  // the selection kernel writes the CSR directly (no count, scan or emit)
  if (pl.block == 64 && p->mode == BSA_SELECT_TOPK && p->k > 0 && !p->force_diag &&
      !p->use_static && p->n_diagonals == 0 && p->n_columns == 0) {
    a.direct = std::min(p->k, (int)pl.nB);
    a.rows = rows;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.col_cap = col_cap;
    a.out_nnz = out_nnz;
    BSA_TRY(hip_status(bsa::launch_select(a, (int)pl.rows_sel, st), "select launch"));
    return BSA_OK;
  }
  BSA_TRY(hip_status(bsa::launch_select(a, (int)pl.rows_sel, st), "select launch"));
  const uint32_t* bits = a.bits;
  const int32_t* counts = a.counts;
  if (pl.block != 64) {
    uint32_t* bits64 = (uint32_t*)(ws + pl.bytes_a + pl.bytes_b);
    int32_t* counts64 = (int32_t*)(ws + pl.bytes_a + pl.bytes_b + pl.bytes_c);
    BSA_TRY(hip_status(bsa::launch_expand_bits(a.bits, a.W, a.nB, bits64, counts64, (int)pl.W,
                                               (int)pl.nB, rows, st),
                       "expand launch"));
    bits = bits64;
    counts = counts64;
  }
  BSA_TRY(hip_status(bsa::launch_scan(counts, rows, row_ptr, out_nnz, st), "scan launch"));
  BSA_TRY(hip_status(bsa::launch_emit_bits(bits, (int)pl.W, rows, row_ptr, col_idx, col_cap, st),
                     "emit launch"));
  return BSA_OK;
}

int64_t bsa_select_scratch_limit(void) { return kScratchBytes; }

bsa_status bsa_select_blocks_noalloc(const float* scores, const bsa_shape* shape, int32_t block,
                                     const bsa_select_params* p, int32_t* row_ptr,
                                     int32_t* col_idx, int64_t col_cap, int64_t* out_nnz,
                                     void* stream) {
  SelectPlan pl;
  BSA_TRY(plan_select(shape, block, p, &pl));
  if (pl.total > kScratchBytes)
    return fail(BSA_ERR_CAPACITY,
                "selection needs %lld bytes of scratch, more than the %lld the no-allocation "
                "entry point holds (use bsa_select_blocks with a workspace)",
                (long long)pl.total, (long long)kScratchBytes);
  void* ws = nullptr;
  BSA_TRY(scratch_of_current_device(&ws));
  return bsa_select_blocks(scores, shape, block, p, row_ptr, col_idx, col_cap, out_nnz, ws,
                           kScratchBytes, stream);
}

int64_t bsa_attn_workspace_bytes(const bsa_shape* shape) {
  if (check_shape(shape) != BSA_OK) return -1;
  const MicroOrderPlan m = plan_micro_order(shape);
  return m.vt_bytes + m.order_bytes;
}

bsa_status bsa_attn_stage_v(const uint16_t* V, const bsa_shape* shape, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  BSA_TRY(check_shape(shape));
  BSA_TRY(check_ptr(V, "V"));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  const int64_t need = bsa_attn_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  const int nB = (int)cdiv(shape->N, 64);
  bsa::TransposeArgs t{};
  t.V = V;
  t.Vt = (uint16_t*)workspace;
  t.sb = shape->stride_b;
  t.sh = shape->stride_h;
  t.sn = shape->stride_n;
  t.H = shape->H;
  t.N = shape->N;
  t.nB = nB;
  t.Npad = nB * 64;
  t.heads = all_heads(shape->H);
  return hip_status(bsa::launch_transpose_v(t, shape->B, shape->d, (hipStream_t)stream),
                    "transpose_v launch");
}

bsa_status bsa_sparse_attn_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                               const bsa_shape* shape, int32_t block, float scale,
                               const int32_t* row_ptr, const int32_t* col_idx, void* O,
                               int32_t o_dtype, float* LSE, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  BSA_TRY(check_attn_common(Q, K, V, shape, O, o_dtype, LSE, workspace, workspace_bytes));
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "block=%d unsupported (64)", block);
  BSA_TRY(check_ptr(row_ptr, "row_ptr", 4));
  if (col_idx == nullptr) return fail(BSA_ERR_INVALID_ARG, "col_idx is NULL");
  return run_attn(Q, K, V, shape, scale, row_ptr, col_idx, O, o_dtype, LSE, workspace, false,
                  (hipStream_t)stream);
}

bsa_status bsa_attn_take_status(void* workspace, int64_t workspace_bytes,
                                const bsa_shape* shape, int32_t* status_out, void* stream) {
  BSA_TRY(check_shape(shape));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  BSA_TRY(check_ptr(status_out, "status_out", 4));
  const int64_t need = bsa_attn_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  int32_t* status = (int32_t*)((char*)workspace + plan_micro_order(shape).status_off);
  return hip_status(bsa::launch_take_status(status, status_out, (hipStream_t)stream),
                    "status launch");
}

bsa_status bsa_check_csr(const int32_t* row_ptr, int64_t rows, const int32_t* col_idx,
                         int64_t col_cap, int32_t n_cols, int32_t* counts, void* stream) {
  if (rows < 0 || rows > INT32_MAX - 1) return fail(BSA_ERR_INVALID_ARG, "rows=%lld", (long long)rows);
  if (col_cap < 0) return fail(BSA_ERR_INVALID_ARG, "col_cap < 0");
  if (n_cols < 0) return fail(BSA_ERR_INVALID_ARG, "n_cols < 0");
  BSA_TRY(check_ptr(row_ptr, "row_ptr", 4));
  BSA_TRY(check_ptr(counts, "counts", 4));
  if (col_cap > 0) BSA_TRY(check_ptr(col_idx, "col_idx", 4));
  bsa::CsrCheckArgs a{};
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.cap = col_cap;
  a.rows = (int)rows;
  a.n_cols = n_cols;
  a.counts = counts;
  return hip_status(bsa::launch_csr_check(a, (hipStream_t)stream), "csr check launch");
}

bsa_status bsa_validate_csr_host(const int32_t* row_ptr, int64_t rows, const int32_t* col_idx,
                                 int64_t col_cap, int32_t n_cols, int64_t* bad_row) {
  if (bad_row != nullptr) *bad_row = -1;
  if (rows < 0) return fail(BSA_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  if (row_ptr == nullptr) return fail(BSA_ERR_INVALID_ARG, "row_ptr is NULL");
  if (col_cap < 0) return fail(BSA_ERR_INVALID_ARG, "col_cap < 0");
  if (col_cap > 0 && col_idx == nullptr) return fail(BSA_ERR_INVALID_ARG, "col_idx is NULL");
  if (row_ptr[0] != 0) {
    if (bad_row != nullptr) *bad_row = 0;
    return fail(BSA_ERR_INVALID_ARG, "row_ptr[0] = %d, not 0", row_ptr[0]);
  }
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t b = row_ptr[r], e = row_ptr[r + 1];
    if (e < b || e > col_cap) {
      if (bad_row != nullptr) *bad_row = r;
      return fail(BSA_ERR_INVALID_ARG, "row %lld: row_ptr %lld..%lld out of order or past col_cap %lld",
                  (long long)r, (long long)b, (long long)e, (long long)col_cap);
    }
    for (int64_t k = b; k < e; ++k) {
      const int32_t v = col_idx[k];
      if (v < 0 || v >= n_cols) {
        if (bad_row != nullptr) *bad_row = r;
        return fail(BSA_ERR_INVALID_ARG, "row %lld: column %d outside [0, %d)", (long long)r, v,
                    n_cols);
      }
      if (k > b && v <= col_idx[k - 1]) {
        if (bad_row != nullptr) *bad_row = r;
        return fail(BSA_ERR_INVALID_ARG, "row %lld: columns not strictly ascending (%d after %d)",
                    (long long)r, v, col_idx[k - 1]);
      }
    }
  }
  return BSA_OK;
}

bsa_status bsa_dense_attn_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                              const bsa_shape* shape, float scale, void* O, int32_t o_dtype,
                              float* LSE, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  BSA_TRY(check_attn_common(Q, K, V, shape, O, o_dtype, LSE, workspace, workspace_bytes));
  return run_attn(Q, K, V, shape, scale, nullptr, nullptr, O, o_dtype, LSE, workspace, true,
                  (hipStream_t)stream);
}

bsa_status bsa_micro_residual_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                  const bsa_shape* shape, int32_t block, int32_t micro,
                                  float scale, const int32_t* mrow_ptr, const int32_t* midx,
                                  const uint8_t* head_mask, void* O_mu, int32_t o_dtype,
                                  float* LSE_mu, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  BSA_TRY(check_attn_common(Q, K, V, shape, O_mu, o_dtype, LSE_mu, workspace, workspace_bytes));
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "block=%d unsupported (64)", block);
  if (micro != 16) return fail(BSA_ERR_UNSUPPORTED, "micro=%d unsupported (16)", micro);
  BSA_TRY(check_ptr(mrow_ptr, "mrow_ptr", 4));
  const bsa::HeadList heads = heads_from_mask(head_mask, shape->H);
  if (heads.n == 0) return BSA_OK;
  if ((int64_t)shape->B * heads.n > 65535)
    return fail(BSA_ERR_UNSUPPORTED, "B * micro heads exceeds 65535");
  if (midx == nullptr) return fail(BSA_ERR_INVALID_ARG, "midx is NULL");
  hipStream_t st = (hipStream_t)stream;
  const int nB = (int)cdiv(shape->N, 64);
  bsa::TransposeArgs t{};
  t.V = V;
  t.Vt = (uint16_t*)workspace;
  t.sb = shape->stride_b;
  t.sh = shape->stride_h;
  t.sn = shape->stride_n;
  t.H = shape->H;
  t.N = shape->N;
  t.nB = nB;
  t.Npad = nB * 64;
  t.heads = heads;
  if (V != nullptr)
    BSA_TRY(hip_status(bsa::launch_transpose_v(t, shape->B, shape->d, st), "transpose_v launch"));
  bsa::MicroAttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.Vt = (const uint16_t*)workspace;
  a.O = O_mu;
  a.LSE = LSE_mu;
  a.row_ptr = mrow_ptr;
  a.idx = midx;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.nB = nB;
  a.Npad = nB * 64;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.heads = heads;
  const MicroOrderPlan m = plan_micro_order(shape);
  char* ws = (char*)workspace;
  a.sig = (int32_t*)(ws + m.sig_off);
  a.order = (int32_t*)(ws + m.order_off);
  a.hist = (int32_t*)(ws + m.hist_off);
  a.offsets = (int32_t*)(ws + m.offs_off);
  a.nnz = (int64_t*)(ws + m.nnz_off);
  a.status = (int32_t*)(ws + m.status_off);
  a.nT = (int)cdiv(shape->N, 16);
  a.slots = (int)((int64_t)shape->B * heads.n * nB * 4);
  a.bins = shape->B * heads.n * (a.nT + 1);
  a.per_xcd = (int)cdiv(cdiv(a.slots, bsa::kMicroWaves), 8);
  return hip_status(bsa::launch_micro_attn(a, shape->B, shape->d, o_dtype == BSA_BF16, st),
                    "micro attn launch");
}

bsa_status bsa_lse_merge(const void* O1, const float* L1, const void* O2, const float* L2,
                         const bsa_shape* shape, int32_t o_dtype, const uint8_t* head_mask,
                         void* O, float* L, void* stream) {
  BSA_TRY(check_shape(shape));
  BSA_TRY(check_ptr(O1, "O1"));
  BSA_TRY(check_ptr(O2, "O2"));
  BSA_TRY(check_ptr(O, "O"));
  BSA_TRY(check_ptr(L1, "L1", 4));
  BSA_TRY(check_ptr(L2, "L2", 4));
  BSA_TRY(check_ptr(L, "L", 4));
  if (o_dtype != BSA_F32 && o_dtype != BSA_BF16)
    return fail(BSA_ERR_INVALID_ARG, "o_dtype=%d (BSA_F32 or BSA_BF16)", o_dtype);
  const bsa::HeadList heads = heads_from_mask(head_mask, shape->H);
  if (heads.n == 0) return BSA_OK;
  bsa::MergeArgs a{};
  a.O1 = O1;
  a.L1 = L1;
  a.O2 = O2;
  a.L2 = L2;
  a.O = O;
  a.L = L;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.D = shape->d;
  a.heads = heads;
  return hip_status(bsa::launch_merge(a, shape->B, o_dtype == BSA_BF16, (hipStream_t)stream),
                    "merge launch");
}

int64_t bsa_omission_risk_workspace_bytes(const bsa_shape* shape) {
  int64_t chunks = 0;
  if (check_risk_shape(shape, &chunks) != BSA_OK) return -1;
  return align256((int64_t)shape->B * shape->H * chunks * 3 * 8);
}

bsa_status bsa_omission_risk(const float* lse_sparse, const float* lse_full,
                             const float* lse_repaired, const bsa_shape* shape, double* risk,
                             void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t chunks = 0;
  BSA_TRY(check_risk_shape(shape, &chunks));
  BSA_TRY(check_ptr(lse_sparse, "lse_sparse", 4));
  BSA_TRY(check_ptr(lse_full, "lse_full", 4));
  if (lse_repaired != nullptr) BSA_TRY(check_ptr(lse_repaired, "lse_repaired", 4));
  BSA_TRY(check_ptr(risk, "risk", 8));
  BSA_TRY(check_ptr(workspace, "workspace", 8));
  const int64_t need = bsa_omission_risk_workspace_bytes(shape);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < %lld required",
                (long long)workspace_bytes, (long long)need);
  bsa::RiskArgs a{};
  a.Ls = lse_sparse;
  a.Lf = lse_full;
  a.Lr = lse_repaired;
  a.partial = (double*)workspace;
  a.risk = risk;
  a.N = shape->N;
  a.chunks = (int)chunks;
  a.BH = shape->B * shape->H;
  return hip_status(bsa::launch_risk(a, (hipStream_t)stream), "omission risk launch");
}

bsa_status bsa_heads_at_risk(const double* mean_omitted, int32_t H, int32_t n,
                             uint8_t* head_mask) {
  if (H <= 0) return fail(BSA_ERR_INVALID_ARG, "H=%d must be >= 1", H);
  if (mean_omitted == nullptr || head_mask == nullptr)
    return fail(BSA_ERR_INVALID_ARG, "mean_omitted / head_mask is NULL");
  for (int h = 0; h < H; ++h)
    if (std::isnan(mean_omitted[h])) return fail(BSA_ERR_INVALID_ARG, "share of head %d is NaN", h);
  const int take = std::max(0, std::min(n, H));
  // rank of head h in the order (share descending, index ascending)
  for (int h = 0; h < H; ++h) {
    int before = 0;
    for (int g = 0; g < H; ++g)
      before += mean_omitted[g] > mean_omitted[h] || (mean_omitted[g] == mean_omitted[h] && g < h);
    head_mask[h] = before < take ? 1 : 0;
  }
  return BSA_OK;
}

int64_t bsa_pooled_rectify_workspace_bytes(const bsa_shape* shape) {
  RectifyPlan pl;
  if (plan_rectify(shape, &pl) != BSA_OK) return -1;
  return pl.total;
}

bsa_status bsa_pooled_rectify(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                              const bsa_shape* shape, int32_t block, float scale,
                              int32_t gain_gate, const int32_t* row_ptr,
                              const int32_t* col_idx, void* O, int32_t o_dtype, float* LSE,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  RectifyPlan pl;
  BSA_TRY(plan_rectify(shape, &pl));
  if (block != 64) return fail(BSA_ERR_UNSUPPORTED, "block=%d unsupported (64)", block);
  BSA_TRY(check_ptr(Q, "Q"));
  BSA_TRY(check_ptr(K, "K"));
  BSA_TRY(check_ptr(V, "V"));
  BSA_TRY(check_ptr(O, "O"));
  BSA_TRY(check_ptr(LSE, "LSE", 4));
  BSA_TRY(check_ptr(row_ptr, "row_ptr", 4));
  BSA_TRY(check_ptr(col_idx, "col_idx", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  if (o_dtype != BSA_F32 && o_dtype != BSA_BF16)
    return fail(BSA_ERR_INVALID_ARG, "o_dtype=%d (BSA_F32 or BSA_BF16)", o_dtype);
  if (gain_gate != 0 && gain_gate != 1)
    return fail(BSA_ERR_INVALID_ARG, "gain_gate=%d (0 or 1)", gain_gate);
  if (gain_gate && !(scale > 0.f))
    return fail(BSA_ERR_INVALID_ARG, "the gain-aware gate needs scale > 0 (scale=%g)", scale);
  if (workspace_bytes < pl.total)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)pl.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* Kf = (float*)ws;
  float* Vf = (float*)(ws + pl.bytes_f);
  // block means of K and V: the pooling kernel with K in the query slot
  bsa::PoolArgs p{};
  p.Q = K;
  p.K = V;
  p.sb = shape->stride_b;
  p.sh = shape->stride_h;
  p.sn = shape->stride_n;
  p.H = shape->H;
  p.N = shape->N;
  p.D = shape->d;
  p.nB = (int)pl.nB;
  p.nT = (int)cdiv(shape->N, 16);
  p.block = 64;
  p.qpool = Kf;
  p.kpool = Vf;
  BSA_TRY(hip_status(bsa::launch_pool(p, shape->B, st), "pool launch"));
  bsa::RectifyArgs a{};
  a.Q = Q;
  a.Kf = Kf;
  a.Vf = Vf;
  a.Khi = (uint16_t*)(ws + 2 * pl.bytes_f);
  a.Klo = (uint16_t*)(ws + 2 * pl.bytes_f + pl.bytes_h);
  a.Vt = (uint16_t*)(ws + 2 * pl.bytes_f + 2 * pl.bytes_h);
  a.K = K;
  a.spread = (float*)(ws + 2 * pl.bytes_f + 3 * pl.bytes_h);
  a.gate = gain_gate;
  a.gate_thr = gain_gate ? (float)(2.0 * 0.6931471805599453 / ((double)scale * scale)) : 0.f;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.O = O;
  a.LSE = LSE;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.nB = (int)pl.nB;
  a.nBp = (int)pl.nBp;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(bsa::launch_rectify(a, (int)pl.BH, shape->d, o_dtype == BSA_BF16, st),
                    "rectify launch");
}

int64_t bsa_cluster_cells(const bsa_shape* shape, const bsa_cluster_params* params) {
  int64_t cells = 0;
  if (plan_cluster(shape, params, &cells) != BSA_OK) return -1;
  return cells;
}

int64_t bsa_cluster_workspace_bytes(const bsa_shape* shape, const bsa_cluster_params* params) {
  int64_t cells = 0;
  if (plan_cluster(shape, params, &cells) != BSA_OK) return -1;
  const int64_t BH = (int64_t)shape->B * shape->H;
  // centroid norms, the centroids' three bf16 parts, then the update buckets
  int64_t bytes = align256(BH * cells * 4) + align256(BH * cells * 3 * shape->d * 2);
  if (bucket_update_fits(params))
    bytes += align256(BH * cells * cell_tokens(params) * 4) +
             align256(BH * cells * (window_slots(params) + 1) * 4);
  return bytes;
}

bsa_status bsa_local_window_cluster(const uint16_t* X, const bsa_shape* shape,
                                    const bsa_cluster_params* p, int32_t* assign,
                                    float* centroids, int32_t* counts, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
  int64_t cells = 0;
  BSA_TRY(plan_cluster(shape, p, &cells));
  if (shape->stride_n < shape->d || shape->stride_n % 8 || shape->stride_h % 8 ||
      shape->stride_b % 8 || shape->stride_h < 0 || shape->stride_b < 0)
    return fail(BSA_ERR_INVALID_ARG, "strides must be multiples of 8 elements (n >= d)");
  BSA_TRY(check_ptr(X, "X"));
  BSA_TRY(check_ptr(assign, "assign", 4));
  BSA_TRY(check_ptr(centroids, "centroids", 16));
  BSA_TRY(check_ptr(counts, "counts", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 16));
  const int64_t need = bsa_cluster_workspace_bytes(shape, p);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  if (cells > INT32_MAX / 2) return fail(BSA_ERR_UNSUPPORTED, "too many cells");
  bsa::ClusterArgs a{};
  a.X = X;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.D = shape->d;
  a.T = p->T;
  a.Hg = p->Hg;
  a.W = p->W;
  a.kt = p->kt;
  a.kh = p->kh;
  a.kw = p->kw;
  a.Kt = (int)cdiv(p->T, p->kt);
  a.Kh = (int)cdiv(p->Hg, p->kh);
  a.Kw = (int)cdiv(p->W, p->kw);
  a.Nc = (int)cells;
  a.wt = std::min(p->wt, a.Kt);
  a.wh = std::min(p->wh, a.Kh);
  a.ww = std::min(p->ww, a.Kw);
  a.assign = assign;
  a.mu = centroids;
  a.norm = (float*)workspace;
  {
    const int64_t BH = (int64_t)shape->B * shape->H;
    char* w = (char*)workspace + align256(BH * cells * 4);
    a.mu3 = (uint16_t*)w;
    w += align256(BH * cells * 3 * shape->d * 2);
    if (bucket_update_fits(p)) {
      a.bucket = (int32_t*)w;
      w += align256(BH * cells * cell_tokens(p) * 4);
      a.bstart = (int32_t*)w;
    }
  }
  a.counts = counts;
  return hip_status(bsa::launch_cluster(a, shape->B * shape->H, p->iters, (hipStream_t)stream),
                    "cluster launch");
}

bsa_status bsa_lowe_ratio_subset(const uint16_t* X, const bsa_shape* shape,
                                 const bsa_cluster_params* p, const float* centroids,
                                 int32_t n_sub, float* rho, int32_t* subset, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  int64_t cells = 0;
  BSA_TRY(plan_cluster(shape, p, &cells));
  if (shape->stride_n < shape->d || shape->stride_n % 8 || shape->stride_h % 8 ||
      shape->stride_b % 8 || shape->stride_h < 0 || shape->stride_b < 0)
    return fail(BSA_ERR_INVALID_ARG, "strides must be multiples of 8 elements (n >= d)");
  if (n_sub < 0 || n_sub > shape->N)
    return fail(BSA_ERR_INVALID_ARG, "n_sub=%d outside [0, N=%d]", n_sub, shape->N);
  BSA_TRY(check_ptr(X, "X"));
  BSA_TRY(check_ptr(centroids, "centroids", 16));
  BSA_TRY(check_ptr(rho, "rho", 4));
  if (n_sub > 0) BSA_TRY(check_ptr(subset, "subset", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 16));
  const int64_t need = bsa_cluster_workspace_bytes(shape, p);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  if (cells > INT32_MAX / 2) return fail(BSA_ERR_UNSUPPORTED, "too many cells");
  bsa::ClusterArgs a{};
  a.X = X;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.D = shape->d;
  a.T = p->T;
  a.Hg = p->Hg;
  a.W = p->W;
  a.kt = p->kt;
  a.kh = p->kh;
  a.kw = p->kw;
  a.Kt = (int)cdiv(p->T, p->kt);
  a.Kh = (int)cdiv(p->Hg, p->kh);
  a.Kw = (int)cdiv(p->W, p->kw);
  a.Nc = (int)cells;
  a.wt = std::min(p->wt, a.Kt);
  a.wh = std::min(p->wh, a.Kh);
  a.ww = std::min(p->ww, a.Kw);
  a.mu = (float*)centroids;  // read only in this pass
  a.norm = (float*)workspace;
  a.mu3 = (uint16_t*)((char*)workspace + align256((int64_t)shape->B * shape->H * cells * 4));
  a.rho = rho;
  return hip_status(bsa::launch_lowe(a, shape->B * shape->H, n_sub, subset, (hipStream_t)stream),
                    "lowe launch");
}

int64_t bsa_subset_refine_workspace_bytes(const bsa_shape* shape, int32_t cells) {
  if (check_shape(shape) != BSA_OK) return -1;
  if (cells < 1) {
    fail(BSA_ERR_INVALID_ARG, "cells=%d must be >= 1", cells);
    return -1;
  }
  const int64_t bh = (int64_t)shape->B * shape->H;
  // touched bitmaps, member counts, member ranges, the scan total, the
  // member list, the centroids' bf16 parts and their squared norms
  return align256(bh * cdiv(cells, 32) * 4) + align256(bh * cells * 4) +
         align256((bh * cells + 1) * 4) + 256 + align256(bh * shape->N * 4) +
         align256(bh * cells * 3 * shape->d * 2) + align256(bh * cells * 4);
}

bsa_status bsa_subset_refine(const uint16_t* X, const bsa_shape* shape, int32_t cells,
                             const int32_t* subset, int32_t n_sub, int32_t* assign,
                             float* centroids, int32_t* counts, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  BSA_TRY(check_shape(shape));
  if (cells < 1) return fail(BSA_ERR_INVALID_ARG, "cells=%d must be >= 1", cells);
  if (n_sub < 0 || n_sub > shape->N)
    return fail(BSA_ERR_INVALID_ARG, "n_sub=%d outside [0, N=%d]", n_sub, shape->N);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  if ((int64_t)shape->B * shape->H * shape->N >= INT32_MAX ||
      (int64_t)shape->B * shape->H * cells >= INT32_MAX)
    return fail(BSA_ERR_UNSUPPORTED, "too many tokens or centroids for int32 member offsets");
  BSA_TRY(check_ptr(X, "X"));
  if (n_sub > 0) BSA_TRY(check_ptr(subset, "subset", 4));
  BSA_TRY(check_ptr(assign, "assign", 4));
  BSA_TRY(check_ptr(centroids, "centroids", 16));
  BSA_TRY(check_ptr(counts, "counts", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  const int64_t need = bsa_subset_refine_workspace_bytes(shape, cells);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  const int64_t bh = (int64_t)shape->B * shape->H;
  char* ws = (char*)workspace;
  bsa::RefineArgs a{};
  a.X = X;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.H = shape->H;
  a.N = shape->N;
  a.Nc = cells;
  a.W = (int)cdiv(cells, 32);
  a.subset = subset;
  a.n_sub = n_sub;
  a.assign = assign;
  a.mu = centroids;
  a.counts = counts;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    char* p = ws + off;
    off += align256(bytes);
    return p;
  };
  a.touched = (uint32_t*)take(bh * a.W * 4);
  a.tcount = (int32_t*)take(bh * cells * 4);
  a.offs = (int32_t*)take((bh * cells + 1) * 4);
  a.total = (int64_t*)take(256);
  a.list = (int32_t*)take(bh * shape->N * 4);
  a.mu3 = (uint16_t*)take(bh * cells * 3 * shape->d * 2);
  a.norm = (float*)take(bh * cells * 4);
  return hip_status(bsa::launch_subset_refine(a, (int)bh, shape->d, (hipStream_t)stream),
                    "subset refine launch");
}

int64_t bsa_cluster_permute_workspace_bytes(const bsa_shape* shape,
                                            const bsa_cluster_params* params) {
  int64_t cells = 0;
  if (plan_cluster(shape, params, &cells) != BSA_OK) return -1;
  const int64_t BH = (int64_t)shape->B * shape->H;
  // cluster starts, the scan total, then (bucketed path) the cell buckets,
  // their slot starts and the flags of clusters too large for LDS
  int64_t bytes = align256((BH * cells + 1) * 4) + 256;
  if (bucket_update_fits(params))
    bytes += align256(BH * cells * cell_tokens(params) * 4) +
             align256(BH * cells * (window_slots(params) + 1) * 4) + align256(BH * cells * 4);
  return bytes;
}

bsa_status bsa_cluster_permute(const int32_t* assign, const int32_t* counts,
                               const bsa_shape* shape, const bsa_cluster_params* p,
                               int32_t* perm, int32_t* offsets, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  int64_t cells = 0;
  BSA_TRY(plan_cluster(shape, p, &cells));
  BSA_TRY(check_ptr(assign, "assign", 4));
  BSA_TRY(check_ptr(counts, "counts", 4));
  BSA_TRY(check_ptr(perm, "perm", 4));
  BSA_TRY(check_ptr(offsets, "offsets", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  const int64_t need = bsa_cluster_permute_workspace_bytes(shape, p);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  const int64_t rows = (int64_t)shape->B * shape->H * cells;
  if (rows >= INT32_MAX / 2 || (int64_t)shape->B * shape->H * shape->N >= INT32_MAX)
    return fail(BSA_ERR_UNSUPPORTED, "too many tokens for int32 offsets");
  bsa::ClusterArgs a{};
  a.H = shape->H;
  a.N = shape->N;
  a.D = shape->d;
  a.T = p->T;
  a.Hg = p->Hg;
  a.W = p->W;
  a.kt = p->kt;
  a.kh = p->kh;
  a.kw = p->kw;
  a.Kt = (int)cdiv(p->T, p->kt);
  a.Kh = (int)cdiv(p->Hg, p->kh);
  a.Kw = (int)cdiv(p->W, p->kw);
  a.Nc = (int)cells;
  a.wt = std::min(p->wt, a.Kt);
  a.wh = std::min(p->wh, a.Kh);
  a.ww = std::min(p->ww, a.Kw);
  a.assign = const_cast<int32_t*>(assign);
  hipStream_t st = (hipStream_t)stream;
  int32_t* gofs = (int32_t*)workspace;
  int64_t* total = (int64_t*)((char*)workspace + align256((rows + 1) * 4));
  int32_t* big = nullptr;
  if (bucket_update_fits(p)) {
    char* w = (char*)workspace + align256((rows + 1) * 4) + 256;
    a.bucket = (int32_t*)w;
    w += align256(rows * cell_tokens(p) * 4);
    a.bstart = (int32_t*)w;
    w += align256(rows * (window_slots(p) + 1) * 4);
    big = (int32_t*)w;
  }
  BSA_TRY(hip_status(bsa::launch_scan(counts, (int)rows, gofs, total, st), "scan launch"));
  return hip_status(
      bsa::launch_cluster_permute(a, shape->B * shape->H, gofs, perm, offsets, big, st),
      "permute launch");
}

int64_t bsa_cluster_select_workspace_bytes(int32_t B, int32_t H, int32_t Nq, int32_t Nk) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || Nk > 4096) return -1;
  const int64_t rows = (int64_t)B * H * Nq;
  return align256(rows * Nk * 4) + align256(rows * cdiv(Nk, 32) * 4) + align256(rows * 4);
}

bsa_status bsa_cluster_select(const float* mu_q, const float* mu_k, const int32_t* size_k,
                              int32_t B, int32_t H, int32_t Nq, int32_t Nk, int32_t d,
                              float scale, float p, int32_t k_min, int32_t k_cap,
                              int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                              int64_t* out_nnz, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1)
    return fail(BSA_ERR_INVALID_ARG, "B=%d H=%d Nq=%d Nk=%d must all be >= 1", B, H, Nq, Nk);
  if (Nk > 4096) return fail(BSA_ERR_UNSUPPORTED, "Nk=%d exceeds 4096 key clusters", Nk);
  if (d != 64 && d != 128) return fail(BSA_ERR_UNSUPPORTED, "d=%d unsupported (64 or 128)", d);
  if ((int64_t)B * H > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  if (!(p > 0.f && p <= 1.f)) return fail(BSA_ERR_INVALID_ARG, "p=%g not in (0,1]", p);
  if (k_min < 0 || k_cap < k_min)
    return fail(BSA_ERR_INVALID_ARG, "need 0 <= k_min <= k_cap (k_min=%d k_cap=%d)", k_min,
                k_cap);
  BSA_TRY(check_ptr(mu_q, "mu_q", 16));
  BSA_TRY(check_ptr(mu_k, "mu_k", 16));
  BSA_TRY(check_ptr(size_k, "size_k", 4));
  BSA_TRY(check_ptr(row_ptr, "row_ptr", 4));
  BSA_TRY(check_ptr(out_nnz, "out_nnz", 8));
  if (col_cap < 0) return fail(BSA_ERR_INVALID_ARG, "col_cap < 0");
  if (col_cap > 0) BSA_TRY(check_ptr(col_idx, "col_idx", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  const int64_t need = bsa_cluster_select_workspace_bytes(B, H, Nq, Nk);
  if (workspace_bytes < need)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)need);
  const int64_t rows = (int64_t)B * H * Nq;
  if (rows * std::min<int64_t>(Nk, k_cap) > INT32_MAX)
    return fail(BSA_ERR_UNSUPPORTED, "entries exceed int32 row pointers");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* scores = (float*)ws;
  bsa::GemmArgs g{};
  g.A = mu_q;
  g.Bm = mu_k;
  g.C = scores;
  g.H = H;
  g.M = Nq;
  g.Nc = Nk;
  g.D = d;
  g.scale = scale;
  g.heads = all_heads(H);
  BSA_TRY(hip_status(bsa::launch_score_gemm(g, B * H, st), "score launch"));
  bsa::SelectArgs a{};
  a.scores = scores;
  a.bits = (uint32_t*)(ws + align256(rows * Nk * 4));
  a.counts = (int32_t*)(ws + align256(rows * Nk * 4) + align256(rows * cdiv(Nk, 32) * 4));
  a.N = Nk * 64;  // no ragged block: every weight comes from size_k
  a.nB = Nk;
  a.W = (int)cdiv(Nk, 32);
  a.block = 64;
  a.mode = BSA_SELECT_TOPP;
  a.p = p;
  a.k_min = k_min;
  a.k_cap = k_cap;
  a.col_sizes = size_k;
  a.rows_per_head = Nq;
  BSA_TRY(hip_status(bsa::launch_select(a, (int)rows, st), "select launch"));
  BSA_TRY(hip_status(bsa::launch_scan(a.counts, (int)rows, row_ptr, out_nnz, st), "scan launch"));
  return hip_status(
      bsa::launch_emit_bits(a.bits, a.W, (int)rows, row_ptr, col_idx, col_cap, st), "emit launch");
}

int64_t bsa_cluster_attn_workspace_bytes(const bsa_shape* shape, int32_t Nq, int32_t Nk,
                                         int32_t o_dtype) {
  ClusterAttnPlan pl;
  if (plan_cluster_attn(shape, Nq, Nk, o_dtype, &pl) != BSA_OK) return -1;
  return pl.total;
}

bsa_status bsa_cluster_attn_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                const bsa_shape* shape, float scale, int32_t Nq, int32_t Nk,
                                const int32_t* perm_q, const int32_t* off_q,
                                const int32_t* perm_k, const int32_t* off_k,
                                const int32_t* crow_ptr, const int32_t* ccol,
                                const int32_t* group_of, void* O, int32_t o_dtype, float* LSE,
                                int64_t* out_tile_pairs, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  ClusterAttnPlan pl;
  BSA_TRY(plan_cluster_attn(shape, Nq, Nk, o_dtype, &pl));
  BSA_TRY(check_ptr(Q, "Q"));
  BSA_TRY(check_ptr(K, "K"));
  BSA_TRY(check_ptr(V, "V"));
  BSA_TRY(check_ptr(O, "O"));
  BSA_TRY(check_ptr(LSE, "LSE", 4));
  BSA_TRY(check_ptr(perm_q, "perm_q", 4));
  BSA_TRY(check_ptr(off_q, "off_q", 4));
  BSA_TRY(check_ptr(perm_k, "perm_k", 4));
  BSA_TRY(check_ptr(off_k, "off_k", 4));
  BSA_TRY(check_ptr(crow_ptr, "crow_ptr", 4));
  if (ccol == nullptr) return fail(BSA_ERR_INVALID_ARG, "ccol is NULL");
  if (group_of != nullptr) BSA_TRY(check_ptr(group_of, "group_of", 4));
  if (out_tile_pairs != nullptr) BSA_TRY(check_ptr(out_tile_pairs, "out_tile_pairs", 8));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < pl.total)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)pl.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int D = shape->d;
  const int BH = (int)pl.BH;
  bsa::ClusterAttnArgs c{};
  c.Q = Q;
  c.K = K;
  c.V = V;
  c.sb = shape->stride_b;
  c.sh = shape->stride_h;
  c.sn = shape->stride_n;
  c.H = shape->H;
  c.N = shape->N;
  c.Nq = Nq;
  c.Nk = Nk;
  c.NP = (int)pl.NP;
  c.nTP = (int)pl.nTP;
  c.W = (int)pl.W;
  c.perm_q = perm_q;
  c.off_q = off_q;
  c.perm_k = perm_k;
  c.off_k = off_k;
  c.crow_ptr = crow_ptr;
  c.ccol = ccol;
  c.group_of = group_of;
  c.gtile = (int32_t*)(ws + pl.gt);
  c.qpos = (int32_t*)(ws + pl.qpos);
  c.kc = (int32_t*)(ws + pl.kc);
  c.tile_group = (int32_t*)(ws + pl.tg);
  c.srcq = (int32_t*)(ws + pl.srcq);
  c.gmask = (uint32_t*)(ws + pl.gmask);
  c.counts = (int32_t*)(ws + pl.cnt);
  c.row_ptr = (int32_t*)(ws + pl.rp);
  c.col_idx = (int32_t*)(ws + pl.col);
  c.cap = pl.cap;
  c.pairs = (unsigned long long*)(out_tile_pairs != nullptr ? (void*)out_tile_pairs
                                                            : (void*)(ws + pl.pairs));
  c.Kp = (uint16_t*)(ws + pl.kp);
  c.Vt = (uint16_t*)(ws + pl.vt);
  int64_t* entries = (int64_t*)(ws + pl.nent);  // total chunk entries (unused)
  BSA_TRY(hip_status(bsa::launch_cluster_attn_plan(c, BH, D, st), "cluster plan launch"));
  BSA_TRY(hip_status(bsa::launch_scan(c.counts, (int)(pl.BH * Nq), c.row_ptr, entries, st),
                     "scan launch"));
  BSA_TRY(hip_status(bsa::launch_cluster_attn_emit(c, BH, D, st), "cluster emit launch"));
  // padded keys: [BH, NP, D], contiguous; V^T staged by the gather
  const int64_t sn = D, sh = pl.NP * D, sb = shape->H * sh;
  // queries and outputs in the caller's layout (rows through the source
  // map), keys and staged values in the padded layout
  bsa::AttnArgs a{};
  a.Q = Q;
  a.K = c.Kp;
  a.Vt = c.Vt;
  a.O = O;
  a.LSE = LSE;
  a.row_ptr = c.row_ptr;
  a.col_idx = c.col_idx;
  a.sb = shape->stride_b;
  a.sh = shape->stride_h;
  a.sn = shape->stride_n;
  a.ksb = sb;
  a.ksh = sh;
  a.ksn = sn;
  a.qsrc = c.srcq;
  a.Nout = shape->N;
  a.B = shape->B;
  a.H = shape->H;
  a.N = c.NP;
  a.nB = c.nTP;
  a.Npad = c.NP;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rows = (int)(pl.BH * pl.nTP);
  a.per_xcd = (int)cdiv(a.rows, 8);
  a.tile_group = c.tile_group;
  a.ngroups = Nq;
  return hip_status(bsa::launch_attn_chunks(a, D, o_dtype == BSA_BF16, st), "attn launch");
}

int64_t bsa_cluster_merge_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t Nq, int32_t Nk,
                                          int32_t grain) {
  ClusterMergePlan pl;
  if (plan_cluster_merge(B, H, N, Nq, Nk, grain, &pl) != BSA_OK) return -1;
  return pl.total;
}

bsa_status bsa_cluster_merge(const int32_t* off_q, const int32_t* off_k, const int32_t* crow_ptr,
                             const int32_t* ccol, int32_t B, int32_t H, int32_t N, int32_t Nq,
                             int32_t Nk, const uint8_t* sides, int32_t rounds, int32_t tau_q,
                             int32_t tau_k, int32_t grain, int32_t* group_of, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  ClusterMergePlan pl;
  BSA_TRY(plan_cluster_merge(B, H, N, Nq, Nk, grain, &pl));
  if (rounds < 0 || rounds > 64) return fail(BSA_ERR_INVALID_ARG, "rounds=%d (0..64)", rounds);
  if (tau_q < 1 || tau_k < 1)
    return fail(BSA_ERR_INVALID_ARG, "tau_q=%d, tau_k=%d must be >= 1", tau_q, tau_k);
  BSA_TRY(check_ptr(off_q, "off_q", 4));
  BSA_TRY(check_ptr(off_k, "off_k", 4));
  BSA_TRY(check_ptr(crow_ptr, "crow_ptr", 4));
  if (ccol == nullptr) return fail(BSA_ERR_INVALID_ARG, "ccol is NULL");
  if (rounds > 0 && sides == nullptr) return fail(BSA_ERR_INVALID_ARG, "sides is NULL");
  BSA_TRY(check_ptr(group_of, "group_of", 4));
  BSA_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < pl.total)
    return fail(BSA_ERR_CAPACITY, "workspace %lld bytes < required %lld",
                (long long)workspace_bytes, (long long)pl.total);
  char* ws = (char*)workspace;
  bsa::ClusterMergeArgs m{};
  m.Nq = Nq;
  m.Nk = Nk;
  m.W = (int)pl.W;
  m.nbits = (int)pl.nbits;
  m.rounds = rounds;
  m.tau_q = tau_q;
  m.tau_k = tau_k;
  m.grain = grain;
  m.off_q = off_q;
  m.off_k = off_k;
  m.crow_ptr = crow_ptr;
  m.ccol = ccol;
  m.sides = sides;
  m.grp = group_of;
  m.gsq = (int32_t*)(ws + pl.gsq);
  m.gk = (int32_t*)(ws + pl.gk);
  m.alist = (int32_t*)(ws + pl.alist);
  m.blist = (int32_t*)(ws + pl.blist);
  m.nab = (int32_t*)(ws + pl.nab);
  m.choice = (int32_t*)(ws + pl.choice);
  m.gain = (int64_t*)(ws + pl.gain);
  m.ukeys = (int32_t*)(ws + pl.ukeys);
  m.gmask = (uint32_t*)(ws + pl.gmask);
  m.planes = (uint32_t*)(ws + pl.planes);
  m.hbits = (int32_t*)(ws + pl.hbits);
  return hip_status(bsa::launch_cluster_merge(m, (int)pl.BH, (hipStream_t)stream),
                    "cluster merge launch");
}

}  // extern "C"
