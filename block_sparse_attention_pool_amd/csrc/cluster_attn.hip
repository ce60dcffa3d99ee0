// Attention over cluster-induced blocks (HyperVAttention section 2, Eq. 4):
// every query of query cluster i attends over the tokens of the key clusters
// its row selects; the output goes back to the original token order.
//
// Executed on the 64-token tile engine with every cluster padded to whole
// tiles (the CTA-aligned cost of the page's Eq. 7 with a tile of 64 on both
// sides): in the padded cluster order a query tile belongs to one query
// cluster and a key tile to one key cluster, so the tile lists are exact --
// query tile T of cluster i lists every tile of every key cluster in row i --
// and the attention kernel masks each key tile's padding keys (its count of
// valid keys per tile).  Queries and keys share one padded length NP per
// head, 64 * (ceil(N / 64) + max(Nq, Nk)), which bounds both layouts.
//
// Kernels: per-head tile offsets of the clusters (a scan of ceil(size/64));
// padded gathers of Q, K, V in cluster order; valid keys per key tile; the
// tile lists (per-row counts, the row-pointer scan, emission); the masked
// attention; the scatter of O and LSE back to token order.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

// Exclusive scan of ceil(size_c / 64) over the clusters of one head (sizes
// from the cluster offsets), one workgroup of 1024 per (head, tensor).
__global__ __launch_bounds__(1024) void ctile_offsets_kernel(ClusterAttnArgs a) {
  __shared__ int part[1024];
  const int64_t bh = blockIdx.x;
  const bool keys = blockIdx.y == 1;
  const int n = keys ? a.Nk : a.Nq;
  const int32_t* off = (keys ? a.off_k : a.off_q) + bh * (n + 1);
  int32_t* tiles = (keys ? a.tk : a.tq) + bh * (n + 1);
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int c0 = tid * per, c1 = min(c0 + per, n);
  int s = 0;
  for (int c = c0; c < c1; ++c) s += (off[c + 1] - off[c] + 63) / 64;
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan of the partial sums
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int c = c0; c < c1; ++c) {
    tiles[c] = run;
    run += (off[c + 1] - off[c] + 63) / 64;
  }
  if (tid == 1023) tiles[n] = part[1023];
}

// Largest c in [0, n) with t[c] <= x (t ascending, t[0] = 0 <= x).
__device__ __forceinline__ int seg_of(const int32_t* t, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Padded cluster-order copies: position p of tensor (Q, K or V) holds token
// perm[off[c] + k] where c is the cluster of tile p / 64 and k = p - 64
// tq[c], or zeros in a cluster's padding and past the last tile.  One
// thread per 16-byte chunk.
template <int D>
__global__ __launch_bounds__(256) void cgather_kernel(ClusterAttnArgs a) {
  constexpr int C = D / 8;
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  const int which = blockIdx.z;  // 0 Q, 1 K, 2 V
  if (f >= (int64_t)a.NP * C) return;
  const int p = (int)(f / C), c = (int)(f % C);
  const bool keys = which != 0;
  const int n = keys ? a.Nk : a.Nq;
  const int32_t* tl = (keys ? a.tk : a.tq) + bh * (n + 1);
  const int32_t* off = (keys ? a.off_k : a.off_q) + bh * (n + 1);
  const int32_t* perm = (keys ? a.perm_k : a.perm_q) + bh * a.N;
  const uint16_t* src = which == 0 ? a.Q : which == 1 ? a.K : a.V;
  uint16_t* dst = (which == 0 ? a.Qp : which == 1 ? a.Kp : a.Vp) + (bh * a.NP + p) * D;
  u32x4 v = {0u, 0u, 0u, 0u};
  const int T = p / kBlock;
  if (T < tl[n]) {
    const int cl = seg_of(tl, n, T);
    const int k = p - kBlock * tl[cl];
    if (k < off[cl + 1] - off[cl]) {
      const int64_t tok = perm[off[cl] + k];
      const int b = (int)(bh / a.H), h = (int)(bh % a.H);
      v = *(const u32x4*)(src + (int64_t)b * a.sb + (int64_t)h * a.sh + tok * a.sn + 8 * c);
    }
  }
  *(u32x4*)(dst + 8 * c) = v;
}

// Valid keys of every key tile, and each query tile's cluster (-1 past the
// last tile).
__global__ __launch_bounds__(256) void ctile_info_kernel(ClusterAttnArgs a) {
  const int T = blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (T >= a.nTP) return;
  const int32_t* tk = a.tk + bh * (a.Nk + 1);
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  int valid = 0;
  if (T < tk[a.Nk]) {
    const int cl = seg_of(tk, a.Nk, T);
    valid = min(kBlock, ok[cl + 1] - ok[cl] - kBlock * (T - tk[cl]));
  }
  a.key_valid[bh * a.nTP + T] = valid;
  const int32_t* tq = a.tq + bh * (a.Nq + 1);
  a.qtile_cluster[bh * a.nTP + T] = T < tq[a.Nq] ? seg_of(tq, a.Nq, T) : -1;
}

// Entries of every query tile's row: the tiles of the key clusters its
// cluster selects.
__global__ __launch_bounds__(256) void crow_count_kernel(ClusterAttnArgs a) {
  const int T = blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (T >= a.nTP) return;
  const int cl = a.qtile_cluster[bh * a.nTP + T];
  int cnt = 0;
  if (cl >= 0) {
    const int64_t r = bh * a.Nq + cl;
    const int32_t* tk = a.tk + bh * (a.Nk + 1);
    for (int e = a.crow_ptr[r]; e < a.crow_ptr[r + 1]; ++e) {
      const int j = a.ccol[e];
      cnt += tk[j + 1] - tk[j];
    }
  }
  a.counts[bh * a.nTP + T] = cnt;
}

// One wave per query tile: lanes take the selected key clusters 64 at a time
// and write their tiles at positions given by a wave prefix of tile counts.
__global__ __launch_bounds__(256) void cemit_kernel(ClusterAttnArgs a) {
  const int T = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (T >= a.nTP) return;
  const int cl = a.qtile_cluster[bh * a.nTP + T];
  if (cl < 0) return;
  const int64_t r = bh * a.Nq + cl;
  const int32_t* tk = a.tk + bh * (a.Nk + 1);
  int64_t pos = a.row_ptr[bh * a.nTP + T];
  const int e0 = a.crow_ptr[r], e1 = a.crow_ptr[r + 1];
  for (int eb = e0; eb < e1; eb += 64) {
    const int e = eb + lane;
    int j = 0, nt = 0;
    if (e < e1) {
      j = a.ccol[e];
      nt = tk[j + 1] - tk[j];
    }
    const int incl = wave_inclusive_scan(nt);
    int64_t at = pos + incl - nt;
    for (int k = 0; k < nt; ++k, ++at)
      if (at < a.cap) a.col_idx[at] = tk[j] + k;
    pos += __shfl(incl, 63);
  }
}

// O and LSE back to token order: position n of the query order is token
// perm_q[n] of cluster c (off_q[c] <= n), found at padded position
// 64 tq[c] + n - off_q[c].  One thread per 4 output elements.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void cscatter_kernel(ClusterAttnArgs a) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (f >= (int64_t)a.N * (D / 4)) return;
  const int n = (int)(f / (D / 4)), c = (int)(f % (D / 4));
  const int32_t* oq = a.off_q + bh * (a.Nq + 1);
  const int cl = seg_of(oq, a.Nq, n);
  const int64_t src = bh * a.NP + (int64_t)kBlock * a.tq[bh * (a.Nq + 1) + cl] + (n - oq[cl]);
  const int64_t tok = a.perm_q[bh * a.N + n];
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int64_t dst = (int64_t)b * a.sb + (int64_t)h * a.sh + tok * a.sn + 4 * c;
  if constexpr (OUT_BF16) {
    *(u32x2*)((uint16_t*)a.O + dst) = *(const u32x2*)((const uint16_t*)a.Op + src * D + 4 * c);
  } else {
    *(f32x4*)((float*)a.O + dst) = *(const f32x4*)((const float*)a.Op + src * D + 4 * c);
  }
  if (c == 0) a.LSE[bh * a.N + tok] = a.Lp[src];
}

}  // namespace

hipError_t launch_cluster_attn_plan(const ClusterAttnArgs& a, int BH, int D, hipStream_t s) {
  hipLaunchKernelGGL(ctile_offsets_kernel, dim3(BH, 2), dim3(1024), 0, s, a);
  const dim3 ggrid((unsigned)(((int64_t)a.NP * (D / 8) + 255) / 256), BH, 3);
  if (D == 128) hipLaunchKernelGGL(cgather_kernel<128>, ggrid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(cgather_kernel<64>, ggrid, dim3(256), 0, s, a);
  const dim3 tgrid((a.nTP + 255) / 256, BH);
  hipLaunchKernelGGL(ctile_info_kernel, tgrid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(crow_count_kernel, tgrid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cluster_attn_emit(const ClusterAttnArgs& a, int BH, hipStream_t s) {
  hipLaunchKernelGGL(cemit_kernel, dim3((a.nTP + 3) / 4, BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cluster_attn_scatter(const ClusterAttnArgs& a, int BH, int D, bool out_bf16,
                                       hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)a.N * (D / 4) + 255) / 256), BH);
  if (D == 128) {
    if (out_bf16) hipLaunchKernelGGL((cscatter_kernel<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((cscatter_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((cscatter_kernel<64, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((cscatter_kernel<64, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
