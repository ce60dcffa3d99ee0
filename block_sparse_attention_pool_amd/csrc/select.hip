// Block selection -> CSR lists.
//
// Macro rows (one wave per (b, h, query block i), select_wave_kernel):
//   top-k:  the k key blocks of highest pooled score, ties to the lower
//           index (block-sparse density budget);
//   top-p:  HyperVAttention section 2, Eq. 2 (size-weighted centroid
//           softmax) and Eq. 3 (smallest descending prefix with cumulative
//           probability at least p), clamped to [k_min, k_cap];
//   forced: diagonal and/or the LVSA temporal window + rotating anchors
//           and/or MOD-DiT structural patterns (parallel diagonals at given
//           offsets, vertical key columns).
// The row is built as a bitmask (one ballot per 64 key blocks), counted,
// prefix-summed across rows into row_ptr, and emitted as ascending column
// indices; plain top-k rows, which all hold the same count, are emitted by
// the selection kernel itself.  Blocks are 64 or 128 tokens; a 128-token
// selection is emitted on the 64-token tiles the attention kernels run
// (each kept 128 x 128 pair becomes its 2 x 2 tiles), through
// expand_bits_kernel.
//
// Micro rows (HyMoR-Attn Micro selection, 16-token tiles inside omitted
// blocks): one workgroup per (b, micro head, query block); the top-m
// candidate scores by a value histogram and an exact ranking of the
// threshold bin (a radix selection when that bin is too full), ties to the
// lower code, emitted in (sub-tile, key tile) order.
#include <climits>
#include <type_traits>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

enum { kTopK = 0, kTopP = 1, kStatic = 2 };

// ---------------------------------------------------------------- helpers

// Block-wide sum of an int over blockDim.x threads (multiple of 64).
template <typename T>
__device__ T block_sum(T v, T* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = 0;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

// Exclusive prefix over the threads of the block (in thread order); also
// returns the block total.
template <typename T>
__device__ T block_exclusive_scan(T v, T* red, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const T inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  T off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) off += red[w];
    tot += red[w];
  }
  *total = tot;
  return off + inc - v;
}

// ----------------------------------------------------------- macro select

// Top-k, top-p and static rows, one wave per row.  The row is held as
// order-preserving 32-bit keys, E per lane (element e of lane l is block
// 64e + l; E = 8 to 32 in steps of 4, then 40, 48, 56 or 64, the smallest
// that holds the row):
// keys of the pooled scores for top-k, of the size-weighted exponentials
// n_j exp(S_j - max S) for top-p.
//   top-p: the cut of the descending prefix is found without sorting.  The
//     block where the cumulative mass first reaches p * total has the
//     largest key T with mass(key >= T) >= p * total (a bitwise descent over
//     the key, masses summed in double); the prefix length is the number of
//     keys above T plus as many of the equal keys as that sum needs, then
//     clamped to [k_min, k_cap].
//   top-k (and top-p's prefix of that length): the k-th largest key T is
//     the largest T with at least k keys >= T, counted with one ballot per
//     element; keys above T are taken, and of the keys equal to T the lowest
//     block indices, so ties go to the lower index.
// The forced blocks (diagonal, window, anchors) are a union on top.  The
// ballot of element e is words 2e and 2e+1 of the row's bitmask.

// Sum over the wave, left in every lane, without LDS round trips: the two
// halves of the double move through DPP (partner lane l^1, l^2, then the
// mirrored lane within 8 and within 16) and the permlane swaps (rows l^16,
// l^32).  Every step adds the same two values in both partner lanes, so all
// lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm(1, 0, 3, 2): lane l ^ 1
  v += dpp_f64<0x4E>(v);   // quad_perm(2, 3, 0, 1): lane l ^ 2
  v += dpp_f64<0x141>(v);  // row_half_mirror: the other quad of the 8
  v += dpp_f64<0x140>(v);  // row_mirror: the other 8 of the row
  {
    const uint64_t u = __double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])) +
        __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  }
  {
    const uint64_t u = __double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])) +
        __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  }
  return v;
}

template <int E>
__global__ __launch_bounds__(256) void select_wave_kernel(SelectArgs a, int rows) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = r % a.nB;
  const bool scored = a.mode != kStatic;

  uint32_t key[E];
  float val[E];  // top-p: the size-weighted exponentials
  if (scored) {
    const float* row = a.scores + (int64_t)r * a.nB;
    // Every load is issued before any is used, from clamped (in-bounds)
    // addresses, so the lane waits once instead of once per candidate.
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = row[min(64 * e + lane, a.nB - 1)];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (64 * e + lane >= a.nB) x[e] = -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    float sz[E];  // top-p weight: the key block's valid tokens, or the given cluster size
    if (a.mode == kTopP) {
      const float tail_size = (float)(a.N - (a.nB - 1) * a.block);
      if (a.col_sizes != nullptr) {
        const int32_t* cs = a.col_sizes + (int64_t)(r / a.rows_per_head) * a.nB;
#pragma unroll
        for (int e = 0; e < E; ++e) sz[e] = (float)cs[min(64 * e + lane, a.nB - 1)];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) sz[e] = 64 * e + lane == a.nB - 1 ? tail_size : (float)a.block;
      }
      mx = wave_max(mx);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = 64 * e + lane;
      float v = x[e];
      if (a.mode == kTopP) v = sz[e] * expf(v - mx);
      val[e] = j < a.nB ? v : 0.f;
      key[e] = j < a.nB ? float_order_key(v) : 0u;
    }
  }
  // Keys of padding lanes are 0 and every candidate below is >= 1, so they
  // are never counted.
  int k = 0;
  if (a.mode == kTopK) {
    k = min(a.k, a.nB);
  } else if (a.mode == kTopP) {
    double tot = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) tot += (double)val[e];
    tot = wave_sum_f64(tot);
    const double thr = (double)a.p * tot;
    uint32_t T = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      double m = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) m += key[e] >= cand ? (double)val[e] : 0.0;
      if (wave_sum_f64(m) >= thr) T = cand;
    }
    double above = 0.0;
    float vT = 0.f;
    int n_above = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      above += key[e] > T ? (double)val[e] : 0.0;
      if (key[e] == T && 64 * e + lane < a.nB) vT = val[e];
      n_above += __popcll(__ballot(key[e] > T));
      n_eq += __popcll(__ballot(key[e] == T && 64 * e + lane < a.nB));
    }
    above = wave_sum_f64(above);
    vT = wave_max(vT);
    // equal keys are equal values: take the fewest that reach the threshold
    int t = n_eq;
    if (vT > 0.f) t = (int)ceil((thr - above) / (double)vT);
    t = max(1, min(t, n_eq));
    // (no key equal to T: p*total <= 0 gives T = ~0u and a prefix of one
    // block, p > 1 gives T = 0 and the whole row)
    int L = n_eq > 0 ? n_above + t : max(1, n_above);
    L = max(L, a.k_min);
    L = min(L, a.k_cap);
    k = min(L, a.nB);
  }
  const bool all = k >= a.nB;
  uint32_t T = 0;
  int take = 0;  // keys equal to T still to take, lowest index first
  if (k > 0 && !all) {
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      int c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= k) T = cand;
    }
    int gt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) gt += __popcll(__ballot(key[e] > T));
    take = k - gt;
  }

  const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one
  uint32_t word[2] = {0u, 0u};  // lane l holds words l and l + 64 (up to 4096 blocks)
  int ties_before = 0;
  if (k > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool valid = 64 * e + lane < a.nB;
      bool sel = valid && (all || key[e] > T);
      if (take > 0) {
        const bool tie = valid && key[e] == T;
        const uint64_t tb = __ballot(tie);
        if (tie && ties_before + (int)__popcll(tb & below) < take) sel = true;
        ties_before += (int)__popcll(tb);
      }
      // words 2e and 2e+1 belong to lanes (2e) % 64 and (2e+1) % 64, slot e / 32
      const uint64_t m = __ballot(sel);
      if (lane == (2 * e) % 64) word[e / 32] = (uint32_t)m;
      if (lane == (2 * e + 1) % 64) word[e / 32] = (uint32_t)(m >> 32);
    }
  }
  if (a.direct > 0) {
    // ascending indices of the set bits: words 64q + lane, q = 0 then 1
    const int64_t base = (int64_t)r * a.direct;
    int before = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int w = 64 * q + lane;
      uint32_t v = w < a.W ? word[q] : 0u;
      const int c = __popc(v);
      const int incl = wave_inclusive_scan(c);
      int64_t pos = base + before + incl - c;
      before += __shfl(incl, 63);
      while (v) {
        if (pos < a.col_cap) a.col_idx[pos] = 32 * w + __ffs(v) - 1;
        ++pos;
        v &= v - 1;
      }
    }
    if (lane == 0) {
      a.row_ptr[r] = (int32_t)base;
      if (r == rows - 1) {
        a.row_ptr[rows] = (int32_t)((int64_t)rows * a.direct);
        *a.out_nnz = (int64_t)rows * a.direct;
      }
    }
    return;
  }
  // Forced blocks, OR-ed word by word.  The window is an interval of key
  // blocks [ja, jb]: a block's first and last frames never decrease with its
  // index, so lo_j <= hi_i + r and hi_j >= lo_i - r each cut the row once.
  int ja = 1, jb = 0;
  int64_t stride = 0, off = 0;
  if (a.use_static) {
    const int64_t ft = a.frame_tokens;
    const int64_t bs = a.block;
    const int64_t lo_i = (int64_t)i * bs / ft;
    const int64_t hi_i = (min((int64_t)i * bs + bs, (int64_t)a.N) - 1) / ft;
    // hi_j >= F  <=>  min(bs j + bs - 1, N - 1) >= F ft  <=>  bs j + bs - 1 >= F ft
    // (when F ft <= N - 1), i.e. j >= ceil((F ft - bs + 1) / bs) = floor(F ft / bs)
    const int64_t F = lo_i - a.window_frames;
    const int64_t G = hi_i + a.window_frames;
    ja = F * ft <= bs - 1 ? 0 : (int)(F * ft / bs);
    if (F * ft > a.N - 1) ja = a.nB;  // no block reaches that frame
    // lo_j <= G  <=>  bs j / ft <= G  <=>  bs j <= (G + 1) ft - 1
    jb = G < 0 ? -1 : (int)min((int64_t)a.nB - 1, ((G + 1) * ft - 1) / bs);
    if (a.n_anchors > 0) {
      stride = a.nB / a.n_anchors;
      off = ((int64_t)a.anchor_offset % a.nB + a.nB) % a.nB;
    }
  }
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int w = 64 * q + lane;
    if (w >= a.W) continue;
    const int j0 = 32 * w;
    uint32_t f = 0u;
    if (a.force_diag && i >= j0 && i < j0 + 32) f |= 1u << (i - j0);
    if (a.use_static) {
      const int lo = max(ja, j0), hi = min(jb, j0 + 31);
      if (lo <= hi) f |= (uint32_t)((((uint64_t)1 << (hi - lo + 1)) - 1) << (lo - j0));
      for (int t = 0; t < a.n_anchors; ++t) {
        const int j = (int)((off + (int64_t)t * stride) % a.nB);
        if (j >= j0 && j < j0 + 32) f |= 1u << (j - j0);
      }
    }
    // MOD-DiT patterns: diagonal offsets off the block map mark nothing
    for (int t = 0; t < a.n_diag; ++t) {
      const int j = i + a.diag[t];
      if (j >= j0 && j < j0 + 32) f |= 1u << (j - j0);
    }
    for (int t = 0; t < a.n_col; ++t) {
      const int j = a.col[t];
      if (j >= j0 && j < j0 + 32) f |= 1u << (j - j0);
    }
    const uint32_t valid = a.nB - j0 >= 32 ? 0xFFFFFFFFu : ((1u << (a.nB - j0)) - 1u);
    word[q] = (word[q] | f) & valid;
    a.bits[(int64_t)r * a.W + w] = word[q];
    cnt += __popc(word[q]);
  }
  cnt = wave_sum(cnt);
  if (lane == 0) a.counts[r] = cnt;
}

// ---------------------------------------------- 128-token blocks on 64 tiles

// Spread the 16 low bits of x to the even bit positions of a 32-bit word.
__device__ __forceinline__ uint32_t spread16(uint32_t x) {
  x &= 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x;
}

// One wave per 64-token query block r = (b, h, i): it takes the row of its
// 128-token block (b, h, i / 2), every kept key block J becoming 64-token
// blocks 2J and 2J + 1 (the second only when it exists).  Word w of the
// 64-block row covers 128-blocks 16w .. 16w + 15: half (w & 1) of word
// w / 2 of the 128-block row, each bit doubled.
__global__ __launch_bounds__(256) void expand_bits_kernel(const uint32_t* bits_sel, int W_sel,
                                                          int nB_sel, uint32_t* bits64,
                                                          int32_t* counts64, int W64, int nB64,
                                                          int rows64) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows64) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = r / nB64;
  const int i = r % nB64;
  const uint32_t* src = bits_sel + (bh * nB_sel + i / 2) * W_sel;
  int cnt = 0;
  for (int w = lane; w < W64; w += 64) {
    const uint32_t half = w / 2 < W_sel ? src[w / 2] >> (16 * (w & 1)) : 0u;
    const uint32_t x = spread16(half);
    const int j0 = 32 * w;
    const uint32_t valid = nB64 - j0 >= 32 ? 0xFFFFFFFFu : ((1u << (nB64 - j0)) - 1u);
    const uint32_t word = (x | (x << 1)) & valid;
    bits64[(int64_t)r * W64 + w] = word;
    cnt += __popc(word);
  }
  cnt = wave_sum(cnt);
  if (lane == 0) counts64[r] = cnt;
}

// -------------------------------------------------------- row pointers

// Exclusive prefix of the per-row counts into row_ptr (and the total into
// row_ptr[rows] and *out_nnz), one workgroup: the counts stream through LDS
// in chunks of 16384 (coalesced loads and stores), each thread scans 16
// consecutive entries of a chunk, and a running carry links the chunks.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* counts, int rows,
                                                    int32_t* row_ptr, int64_t* out_nnz) {
  constexpr int kChunk = 16384, kPer = 16;
  __shared__ int32_t buf[kChunk + kChunk / kPer];  // one pad word per 16 entries
  __shared__ int64_t red[16];
  const int tid = threadIdx.x;
  auto at = [](int k) { return k + k / kPer; };
  int64_t carry = 0;
  for (int base = 0; base < rows; base += kChunk) {
    const int n = min(kChunk, rows - base);
    for (int k = tid; k < n; k += 1024) buf[at(k)] = counts[base + k];
    __syncthreads();
    int64_t local = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int k = tid * kPer + e;
      if (k < n) local += buf[at(k)];
    }
    int64_t total;
    int64_t run = carry + block_exclusive_scan(local, red, &total);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int k = tid * kPer + e;
      if (k < n) {
        const int v = buf[at(k)];
        buf[at(k)] = (int32_t)run;
        run += v;
      }
    }
    __syncthreads();
    for (int k = tid; k < n; k += 1024) row_ptr[base + k] = buf[at(k)];
    carry += total;
    __syncthreads();
  }
  if (tid == 0) {
    row_ptr[rows] = (int32_t)carry;
    *out_nnz = carry;
  }
}

// One wave per row: ascending indices of the set bits.
__global__ __launch_bounds__(256) void emit_bits_kernel(const uint32_t* bits, int W, int rows,
                                                        const int32_t* row_ptr,
                                                        int32_t* col_idx, int64_t cap) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int wpl = (W + 63) / 64;
  const int w0 = lane * wpl;
  const uint32_t* rb = bits + (int64_t)r * W;
  int cnt = 0;
  for (int e = 0; e < wpl; ++e)
    if (w0 + e < W) cnt += __popc(rb[w0 + e]);
  const int incl = wave_inclusive_scan(cnt);
  int64_t pos = (int64_t)row_ptr[r] + incl - cnt;
  for (int e = 0; e < wpl; ++e) {
    const int w = w0 + e;
    if (w >= W) break;
    uint32_t v = rb[w];
    while (v) {
      const int bit = __ffs(v) - 1;
      if (pos < cap) col_idx[pos] = w * 32 + bit;
      ++pos;
      v &= v - 1;
    }
  }
}

// One wave per row of a caller's CSR: counts rows whose pointers are out of
// order or out of [0, cap] (row 0 must start at 0), entries outside
// [0, n_cols), and entries not above their predecessor.  Entries are read
// only inside [row_ptr[r], row_ptr[r+1]) of rows whose pointers pass.
__global__ __launch_bounds__(256) void csr_check_kernel(CsrCheckArgs a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = a.row_ptr[r], e = a.row_ptr[r + 1];
  const bool bad_ptr = b < 0 || b > e || e > a.cap || (r == 0 && b != 0);
  if (bad_ptr) {
    if (lane == 0) atomicAdd(&a.counts[0], 1);
    return;
  }
  int out = 0, order = 0;
  for (int64_t k = b + lane; k < e; k += 64) {
    const int v = a.col_idx[k];
    out += (unsigned)v >= (unsigned)a.n_cols;
    order += k > b && v <= a.col_idx[k - 1];
  }
  out = wave_sum(out);
  order = wave_sum(order);
  if (lane == 0) {
    if (out) atomicAdd(&a.counts[1], out);
    if (order) atomicAdd(&a.counts[2], order);
  }
}

// Copies a status word out and clears it (one thread).
__global__ void take_status_kernel(int32_t* status, int32_t* out) {
  if (threadIdx.x == 0) {
    out[0] = status[0];
    status[0] = 0;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------- micro select

// Value-binned selection: bins of the score range, and the candidates of the
// threshold bin the LDS list holds at most.
constexpr int kMicroBins = 2048;
constexpr int kMicroList = 1024;

// The float a (nonzero) order key came from: the inverse of float_order_key.
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}

// Exclusive prefix over the threads of the block in reversed thread order
// (thread t gets the sum over threads t' > t); also returns the total.
template <typename T>
__device__ T block_exclusive_scan_rev(T v, T* red, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  // suffix sum within the wave: lanes above this one
  T suf = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T o = __shfl_down(suf, off);
    if (lane + off < 64) suf += o;
  }
  __syncthreads();
  if (lane == 0) red[wave] = suf;  // the whole wave's sum
  __syncthreads();
  T off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w > wave) off += red[w];
    tot += red[w];
  }
  *total = tot;
  return off + suf - v;
}

// Radix selection, most significant byte first, of the `remaining`-th
// largest 32-bit key among the keys each thread hands to the visitor
// (each(f) calls f(key) for every candidate key of the calling thread).
// On return `remaining` holds how many candidates equal to the returned
// threshold must still be taken.  All threads of the block call it.
template <class Each>
__device__ uint32_t block_radix_select(int& remaining, Each each, uint32_t* hist,
                                       int* shared_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int q = tid; q < 256; q += blockDim.x) hist[q] = 0u;
    __syncthreads();
    each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      const int b0 = 4 * lane;
      const int h0 = hist[b0], h1 = hist[b0 + 1], h2 = hist[b0 + 2], h3 = hist[b0 + 3];
      const int mine = h0 + h1 + h2 + h3;
      // suffix sum over lanes: count of keys in bins >= 4*lane
      int suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      const int above_lane = suf - mine;  // bins >= 4*(lane+1)
      if (above_lane < remaining && suf >= remaining) {
        int above = above_lane;
        const int hb[4] = {h0, h1, h2, h3};
        for (int q = 3; q >= 0; --q) {
          if (above + hb[q] >= remaining) {
            shared_out[0] = b0 + q;
            shared_out[1] = above;
            break;
          }
          above += hb[q];
        }
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)shared_out[0];
    remaining -= shared_out[1];
    prefix |= digit << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  return prefix;
}

// One workgroup per query block.  The row's scores are read once, E per
// thread (candidate c = e * 1024 + thread, c = a * nT + beta): the first
// E - KL into registers, the last KL into LDS, since 64 registers per lane
// (two 1024-thread workgroups per compute unit, so that one's score loads
// overlap the other's selection) do not hold all E with the pass state
// without spills.  A bitmask per thread marks the candidates (inside the
// row, outside the blocks the macro selection kept).  The m best by (score
// descending, code 4 beta + a ascending) are found from a histogram of the
// scores; a radix selection over the order-preserving keys is the fallback.
// Each pass walks the codes again from an opaque start (otherwise the
// compiler keeps all E codes live from the first pass and spills).  On the
// HunyuanVideo micro heads this took the micro-selection stage from 2.02 to
// 1.70 ms (identical lists) against keeping every score in registers.
template <int E>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(E <= 32 ? 8 : 1)))
void micro_select_kernel(MicroSelectArgs a) {
  __shared__ uint32_t omask[128];
  __shared__ uint32_t hist[256];
  __shared__ int sh_out[2];
  __shared__ int ired[16];
  __shared__ int wcnt[16][E];
  __shared__ uint32_t hist2[kMicroBins];
  __shared__ float fred[32];
  __shared__ uint32_t list_n;
  __shared__ uint32_t list_key[kMicroList];
  __shared__ uint32_t list_code[kMicroList];
  __shared__ uint32_t won[E * 32];  // bit c: candidate c won its place in the threshold bin

  const int i = blockIdx.x;
  const int z = blockIdx.y;
  const int nh = a.heads.n;
  const int b = z / nh;
  const int h = a.heads.h[z % nh];
  const int64_t r = ((int64_t)b * a.H + h) * a.nB + i;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  for (int w = tid; w < a.W; w += 1024) omask[w] = 0u;
  __syncthreads();
  const int rb = a.macro_row_ptr[r], re = a.macro_row_ptr[r + 1];
  for (int e = rb + tid; e < re; e += 1024) {
    const int j = a.macro_col_idx[e];
    atomicOr(&omask[j >> 5], 1u << (j & 31));
  }
  __syncthreads();

  const int nT = a.nT;
  const int nq = min(4, nT - 4 * i);
  const int ncand = nq * nT;
  const float* sig = a.sigma + ((int64_t)z * nT + 4 * i) * nT;
  // codes 4 beta + a of the thread's candidates, walked in element order
  // (c grows by 1024 per element: beta and a advance without a division)
  const int beta0 = tid % nT, a0 = tid / nT;
  auto advance = [&](int& beta, int& sub) {
    beta += 1024;
    if constexpr (E > 8) {  // rows of more than 8192 candidates: nT > 2048
      if (beta >= nT) {
        beta -= nT;
        ++sub;
      }
    } else {
      while (beta >= nT) {
        beta -= nT;
        ++sub;
      }
    }
  };
  auto for_codes = [&](auto f) {
    int beta = beta0, sub = a0;
    // opaque to the compiler, so that each pass walks the codes again
    // instead of keeping every element's code live from the first pass
    asm volatile("" : "+v"(beta), "+v"(sub));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      f(e, beta, 4u * (uint32_t)beta + (uint32_t)sub);
      advance(beta, sub);
    }
  };
  // elements e < ne of this thread lie inside the row (a count, so that the
  // test needs no per-element candidate index kept live)
  const int ne = ncand > tid ? (ncand - tid + 1023) >> 10 : 0;
  // Every score load is issued before any is used (in-bounds addresses, so
  // the loads need no branch and all of them are in flight at once).  With
  // 64 registers per lane (E = 32) the last KL = 12 elements go to LDS
  // (48 KB; 73 KB per workgroup in all, two per compute unit); each thread
  // reads back only its own, so they need no barrier.
  constexpr int KL = E == 32 ? 12 : 0;
  constexpr int ER = E - KL;
  __shared__ float sl[KL > 0 ? KL * 1024 : 1];
  float sv[ER];
#pragma unroll
  for (int e = 0; e < ER; ++e) sv[e] = sig[min(e * 1024 + tid, ncand - 1)];
#pragma unroll
  for (int e = ER; e < E; ++e) sl[(e - ER) * 1024 + tid] = sig[min(e * 1024 + tid, ncand - 1)];
  auto val = [&](int e) { return e < ER ? sv[e] : sl[(e - ER) * 1024 + tid]; };
  // bit e: element e is a candidate (inside the row, outside every block the
  // macro selection kept); the row's score range over the candidates
  using Mask = std::conditional_t<(E > 32), uint64_t, uint32_t>;
  Mask valid = 0u;
  float vmin = INFINITY, vmax = -INFINITY;
  for_codes([&](int e, int beta, uint32_t) {
    const int blk = beta >> 2;
    if (e < ne && ((omask[blk >> 5] >> (blk & 31)) & 1u) == 0u) {
      valid |= Mask(1) << e;
      vmin = fminf(vmin, val(e));
      vmax = fmaxf(vmax, val(e));
    }
  });
  const int nvalid = block_sum((int)__popcll((uint64_t)valid), ired);
  auto is_valid = [&](int e) { return ((valid >> e) & 1u) != 0u; };
  auto key_of = [&](int e) { return is_valid(e) ? max(1u, float_order_key(val(e))) : 0u; };

  const int m = a.m;
  Mask chosen = valid;  // bit e: element e is selected
  bool done = nvalid <= m;  // every candidate fits
  // The m best candidates by (score descending, code ascending).  Fast
  // path: a histogram of the scores over kMicroBins equal-width bins between
  // the row's smallest and largest candidate score (a monotone map, so every
  // candidate of a higher bin beats every candidate of a lower one; equal
  // scores share a bin) finds the bin holding the m-th best; the bins above
  // it are taken whole and its own few candidates are ranked exactly in LDS.
  // Bins by value, not by the top bits of the key: scores of one row share
  // their sign and exponent, so bit bins would put most candidates on a
  // handful of LDS counters.  When that bin holds more than kMicroList
  // candidates (many equal scores) a radix selection over the keys runs
  // instead.
  if (!done) {
    vmin = wave_min(vmin);
    vmax = wave_max(vmax);
    if (lane == 0) {
      fred[wave] = vmin;
      fred[16 + wave] = vmax;
    }
    for (int q = tid; q < kMicroBins; q += 1024) hist2[q] = 0u;
    for (int q = tid; q < E * 32; q += 1024) won[q] = 0u;
    if (tid == 0) list_n = 0;
    __syncthreads();
    vmin = INFINITY;
    vmax = -INFINITY;
    for (int w = 0; w < 16; ++w) {
      vmin = fminf(vmin, fred[w]);
      vmax = fmaxf(vmax, fred[16 + w]);
    }
    if (vmax > vmin) {
      const float sc = (float)kMicroBins / (vmax - vmin);
      auto bin_of = [&](float v) { return min(kMicroBins - 1, (int)((v - vmin) * sc)); };
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (is_valid(e)) atomicAdd(&hist2[bin_of(val(e))], 1u);
      __syncthreads();
      // bins 2t, 2t+1 per thread; candidates in the bins above them
      const int b0 = 2 * tid;
      const int h0 = (int)hist2[b0], h1 = (int)hist2[b0 + 1];
      int tot;
      // exclusive prefix in reversed thread order = suffix over higher bins
      const int above = block_exclusive_scan_rev(h0 + h1, ired, &tot);
      if (above < m && above + h1 >= m) {
        sh_out[0] = b0 + 1;
        sh_out[1] = above;
      } else if (above + h1 < m && above + h1 + h0 >= m) {
        sh_out[0] = b0;
        sh_out[1] = above + h1;
      }
      __syncthreads();
      const int bstar = sh_out[0];
      const int need = m - sh_out[1];
      const int cstar = (int)hist2[bstar];
      if (cstar <= kMicroList) {
        Mask upper = 0u, inb = 0u;  // elements above the bin, in the bin
        for_codes([&](int e, int, uint32_t code) {
          if (is_valid(e)) {
            const int bn = bin_of(val(e));
            upper |= Mask(bn > bstar) << e;
            inb |= Mask(bn == bstar) << e;
            if (bn == bstar) {
              const int pos = (int)atomicAdd(&list_n, 1u);
              list_key[pos] = max(1u, float_order_key(val(e)));
              list_code[pos] = code;
            }
          }
        });
        __syncthreads();
        // the need best of the threshold bin by (key descending, code ascending)
        for (int t = tid; t < cstar; t += 1024) {
          const uint32_t kt = list_key[t], ct = list_code[t];
          int rank = 0;
          for (int u2 = 0; u2 < cstar; ++u2) {
            const uint32_t ku = list_key[u2];
            rank += ku > kt || (ku == kt && list_code[u2] < ct);
          }
          if (rank < need) {
            const int cw = (int)(ct & 3u) * nT + (int)(ct >> 2);
            atomicOr(&won[cw >> 5], 1u << (cw & 31));
          }
        }
        __syncthreads();
        for (Mask rest = inb; rest != 0u; rest &= rest - 1u) {
          const int e = (int)__builtin_ctzll((uint64_t)rest);
          const int cw = e * 1024 + tid;
          upper |= Mask((won[cw >> 5] >> (cw & 31)) & 1u) << e;
        }
        chosen = upper;
        done = true;
      }
    }
  }
  if (!done) {
    // the order-preserving keys of the candidates, 0 for the rest
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = key_of(e);
    int remaining = m;
    const uint32_t T = block_radix_select(remaining, [&](auto f) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (key[e] != 0u) f(key[e]);
    }, hist, sh_out);
    int n_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) n_eq += key[e] == T;
    n_eq = block_sum(n_eq, ired);
    uint32_t C = 0xFFFFFFFFu;  // largest code taken at T
    if (remaining < n_eq) {
      // ties at the threshold: the lowest codes win (largest ~code)
      int rem2 = remaining;
      C = ~block_radix_select(rem2, [&](auto f) {
        for_codes([&](int e, int, uint32_t code) {
          if (key[e] == T) f(~code);
        });
      }, hist, sh_out);
    }
    chosen = 0u;
    for_codes([&](int e, int, uint32_t code) {
      chosen |= Mask(key[e] != 0u && (key[e] > T || (key[e] == T && code <= C))) << e;
    });
  }

  // Compaction in candidate order (sub-tile a major, key tile beta minor):
  // candidate e * 1024 + 64 w + lane comes after every candidate of
  // element e' < e and of wave w' < w at element e.
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int cnt = __popcll(__ballot((chosen >> e) & 1u));
    if (lane == 0) wcnt[wave][e] = cnt;
  }
  __syncthreads();
  // lane e: exclusive offset of (element e, this wave) and the row total
  int before_w = 0, tot_e = 0;
  if (lane < E) {
    for (int w = 0; w < 16; ++w) {
      const int v = wcnt[w][lane];
      tot_e += v;
      if (w < wave) before_w += v;
    }
  }
  const int incl = wave_inclusive_scan(tot_e);
  const int off_e = incl - tot_e + before_w;
  const int total = __shfl(incl, 63);
  const uint64_t below = (1ull << lane) - 1ull;
  int32_t* out = a.slots + r * (int64_t)m;
  for_codes([&](int e, int, uint32_t code) {
    const bool sel = (chosen >> e) & 1u;
    const uint64_t bal = __ballot(sel);
    const int pos = __shfl(off_e, e) + __popcll(bal & below);
    if (sel && pos < m) out[pos] = (int32_t)code;
  });
  if (tid == 0) a.counts[r] = min(total, m);
}

// One wave per row: copy the row's slots into the CSR column array.
__global__ __launch_bounds__(256) void emit_slots_kernel(const int32_t* slots, int m, int rows,
                                                         const int32_t* row_ptr,
                                                         int32_t* col_idx, int64_t cap) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = row_ptr[r];
  const int n = row_ptr[r + 1] - row_ptr[r];
  for (int e = lane; e < n; e += 64)
    if (b + e < cap) col_idx[b + e] = slots[(int64_t)r * m + e];
}

// -------------------------------------------------------------- launchers

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_csr_check(const CsrCheckArgs& a, hipStream_t s) {
  hipError_t e = launch_fill_i32(a.counts, 3, 0, s);
  if (e != hipSuccess || a.rows <= 0) return e;
  hipLaunchKernelGGL(csr_check_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_take_status(int32_t* status, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(take_status_kernel, dim3(1), dim3(64), 0, s, status, out);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  // the smallest E (keys per lane) that holds the row: padding keys cost
  // the same passes as real ones (top-p on 1182 blocks: E = 24 -> 20,
  // 0.554 -> 0.472 ms, identical lists)
  if (a.nB <= 512 || a.mode == kStatic) {
    hipLaunchKernelGGL(select_wave_kernel<8>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 768) {
    hipLaunchKernelGGL(select_wave_kernel<12>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 1024) {
    hipLaunchKernelGGL(select_wave_kernel<16>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 1280) {
    hipLaunchKernelGGL(select_wave_kernel<20>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 1536) {
    hipLaunchKernelGGL(select_wave_kernel<24>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 1792) {
    hipLaunchKernelGGL(select_wave_kernel<28>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 2048) {
    hipLaunchKernelGGL(select_wave_kernel<32>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 2560) {
    hipLaunchKernelGGL(select_wave_kernel<40>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 3072) {
    hipLaunchKernelGGL(select_wave_kernel<48>, grid, block, 0, s, a, rows);
  } else if (a.nB <= 3584) {
    hipLaunchKernelGGL(select_wave_kernel<56>, grid, block, 0, s, a, rows);
  } else {
    hipLaunchKernelGGL(select_wave_kernel<64>, grid, block, 0, s, a, rows);
  }
  return hipGetLastError();
}

hipError_t launch_expand_bits(const uint32_t* bits_sel, int W_sel, int nB_sel,
                              uint32_t* bits64, int32_t* counts64, int W64, int nB64,
                              int rows64, hipStream_t s) {
  hipLaunchKernelGGL(expand_bits_kernel, dim3((rows64 + 3) / 4), dim3(256), 0, s, bits_sel,
                     W_sel, nB_sel, bits64, counts64, W64, nB64, rows64);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int rows, int32_t* row_ptr, int64_t* out_nnz,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, rows, row_ptr, out_nnz);
  return hipGetLastError();
}

hipError_t launch_emit_bits(const uint32_t* bits, int W, int rows, const int32_t* row_ptr,
                            int32_t* col_idx, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(emit_bits_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, bits, W, rows,
                     row_ptr, col_idx, cap);
  return hipGetLastError();
}

hipError_t launch_micro_select(const MicroSelectArgs& a, int B, hipStream_t s) {
  const dim3 grid(a.nB, B * a.heads.n), block(1024);
  const int ncand = 4 * a.nT;  // candidates of one query block, at most
  if (ncand <= 8 * 1024) {
    hipLaunchKernelGGL(micro_select_kernel<8>, grid, block, 0, s, a);
  } else if (ncand <= 32 * 1024) {
    hipLaunchKernelGGL(micro_select_kernel<32>, grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(micro_select_kernel<64>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_emit_slots(const int32_t* slots, int m, int rows, const int32_t* row_ptr,
                             int32_t* col_idx, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(emit_slots_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, slots, m, rows,
                     row_ptr, col_idx, cap);
  return hipGetLastError();
}

}  // namespace bsa
