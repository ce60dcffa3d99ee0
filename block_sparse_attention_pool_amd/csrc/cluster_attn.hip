// Attention over cluster-induced blocks (HyperVAttention section 2, Eq. 4),
// executed as the page's hardware cost model describes it (section 4.3,
// Eq. 7-8): every query of query cluster i attends over the tokens of the
// key clusters its row selects; query clusters may be merged into groups
// that share the union of their rows (Algorithm 1); the output goes back to
// the original token order.
//
// Layout.  Queries: the groups one after another, ordered by their lowest
// member, each group's clusters in ascending order and each padded to whole
// 64-query tiles (the tau_q ceil(s^q / tau_q) of Eq. 8).  Keys: the key
// clusters in order, each padded to whole 16-key chunks; a group's key tiles
// are its selected clusters' chunks packed four to a 64-key tile (the
// tau_k ceil(sum s^k / tau_k) of Eq. 8 at a 16-token grain), the last tile
// completed with an all-padding chunk.  The attention kernel gathers every
// key tile from its four chunks and masks each chunk's padding keys, so the
// result is exactly Eq. 4.
//
// Kernels: the per-head plan (group sizes and tiles, query positions, key
// chunk offsets), the padded query source map, the group key masks, the
// per-group chunk counts and lists, the gather of K by chunk and of V
// straight into the staged fp16 V^T chunks, and the masked attention, which
// reads every query row through the source map and writes O and LSE
// straight to token order.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

// Exclusive scan over n values val(c) by a workgroup of 1024: out[0..n],
// out[n] the total; also written to lds_out when given.  Each thread scans a
// contiguous segment and reads only its own values.
template <typename F>
__device__ void block_exscan(int n, F val, int32_t* out, int* lds_out, int* part) {
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int c0 = min(tid * per, n), c1 = min(c0 + per, n);
  int s = 0;
  for (int c = c0; c < c1; ++c) s += val(c);
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int c = c0; c < c1; ++c) {
    const int v = val(c);
    out[c] = run;
    if (lds_out != nullptr) lds_out[c] = run;
    run += v;
  }
  if (tid == 1023) {
    out[n] = part[1023];
    if (lds_out != nullptr) lds_out[n] = part[1023];
  }
  __syncthreads();
}

// Group label of query cluster i: its group's lowest member, or i itself
// when no grouping is given (a label outside [0, i] also stands alone).
__device__ __forceinline__ int group_label(const ClusterAttnArgs& a, int64_t bh, int i) {
  if (a.group_of == nullptr) return i;
  const int g = a.group_of[bh * a.Nq + i];
  return (g >= 0 && g <= i) ? g : i;
}

// Largest c in [0, n) with t[c] <= x (t ascending, t[0] = 0 <= x).  With
// repeated values it returns the last of them, the segment that holds x.
__device__ __forceinline__ int seg_of(const int32_t* t, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One workgroup of 1024 per head: group sizes, the groups' first query tiles
// (scan of ceil(size / 64) over labels), every query cluster's padded start
// (its group's start plus the sizes of the lower members), and the key
// clusters' first chunks (scan of ceil(size / 16)).
__global__ __launch_bounds__(1024) void cplan_kernel(ClusterAttnArgs a) {
  __shared__ int sg[kMaxClusters + 1];
  __shared__ int lab[kMaxClusters];
  __shared__ int part[1024];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* oq = a.off_q + bh * (a.Nq + 1);
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  for (int i = tid; i < a.Nq; i += 1024) {
    sg[i] = 0;
    lab[i] = group_label(a, bh, i);
  }
  __syncthreads();
  for (int i = tid; i < a.Nq; i += 1024) atomicAdd(&sg[lab[i]], oq[i + 1] - oq[i]);
  __syncthreads();
  // sg becomes the groups' first tiles
  block_exscan(a.Nq, [&](int i) { return (sg[i] + kBlock - 1) / kBlock; },
               a.gtile + bh * (a.Nq + 1), sg, part);
  for (int i = tid; i < a.Nq; i += 1024) {
    const int g = lab[i];
    int off = 0;
    for (int m = g; m < i; ++m)
      if (lab[m] == g) off += oq[m + 1] - oq[m];
    a.qpos[bh * a.Nq + i] = kBlock * sg[g] + off;
  }
  block_exscan(a.Nk, [&](int j) { return (ok[j + 1] - ok[j] + 15) / 16; }, a.kc + bh * (a.Nk + 1),
               nullptr, part);
}

// Group of every query tile (-1 past the last tile).
__global__ __launch_bounds__(256) void ctile_group_kernel(ClusterAttnArgs a) {
  const int T = blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (T >= a.nTP) return;
  const int32_t* gt = a.gtile + bh * (a.Nq + 1);
  a.tile_group[bh * a.nTP + T] = T < gt[a.Nq] ? seg_of(gt, a.Nq, T) : -1;
}

// The token at every padded query position (positions start at -1): query
// order position n of cluster c goes to qpos[c] + n - off_q[c].
__global__ __launch_bounds__(256) void cqsrc_kernel(ClusterAttnArgs a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (n >= a.N) return;
  const int32_t* oq = a.off_q + bh * (a.Nq + 1);
  const int c = seg_of(oq, a.Nq, n);
  a.srcq[bh * a.NP + a.qpos[bh * a.Nq + c] + n - oq[c]] = a.perm_q[bh * a.N + n];
}

// Key clusters of every group: the OR of its members' rows (masks start at
// zero; integer OR, so the result does not depend on the order).  One wave
// per query cluster.
__global__ __launch_bounds__(256) void cgmask_kernel(ClusterAttnArgs a) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (i >= a.Nq) return;
  const int g = group_label(a, bh, i);
  uint32_t* m = a.gmask + (bh * a.Nq + g) * a.W;
  const int64_t r = bh * a.Nq + i;
  for (int e = a.crow_ptr[r] + lane; e < a.crow_ptr[r + 1]; e += 64) {
    const int j = a.ccol[e];
    if (j >= 0 && j < a.Nk) atomicOr(m + (j >> 5), 1u << (j & 31));
  }
}

// Chunk entries of every group with query tiles: its key clusters' chunks,
// rounded up to whole tiles of four; executed tile pairs added up (integer
// atomics).  One wave per label.
__global__ __launch_bounds__(256) void ccount_kernel(ClusterAttnArgs a) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (i >= a.Nq) return;
  const int32_t* gt = a.gtile + bh * (a.Nq + 1);
  const int tiles = gt[i + 1] - gt[i];
  int chunks = 0;
  if (tiles > 0) {
    const uint32_t* m = a.gmask + (bh * a.Nq + i) * a.W;
    const int32_t* kc = a.kc + bh * (a.Nk + 1);
    for (int j = lane; j < a.Nk; j += 64)
      if ((m[j >> 5] >> (j & 31)) & 1u) chunks += kc[j + 1] - kc[j];
    chunks = wave_sum(chunks);
  }
  const int padded = (chunks + 3) & ~3;
  if (lane == 0) {
    a.counts[bh * a.Nq + i] = padded;
    if (padded > 0) atomicAdd(a.pairs, (unsigned long long)tiles * (unsigned long long)(padded / 4));
  }
}

// One wave per group: lanes take the key clusters 64 at a time and write the
// chunks of the selected ones at wave-prefix positions, in ascending order;
// the row is completed with the all-padding chunk (the last chunk of the
// padded key layout, valid count 0).
__global__ __launch_bounds__(256) void cemit_kernel(ClusterAttnArgs a) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (i >= a.Nq) return;
  const int64_t r = bh * a.Nq + i;
  const int64_t end = a.row_ptr[r + 1];
  int64_t pos = a.row_ptr[r];
  if (pos == end) return;
  const uint32_t* m = a.gmask + r * a.W;
  const int32_t* kc = a.kc + bh * (a.Nk + 1);
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  for (int jb = 0; jb < a.Nk; jb += 64) {
    const int j = jb + lane;
    int nt = 0;
    if (j < a.Nk && ((m[j >> 5] >> (j & 31)) & 1u)) nt = kc[j + 1] - kc[j];
    const int incl = wave_inclusive_scan(nt);
    int64_t at = pos + incl - nt;
    if (nt > 0) {
      const int size = ok[j + 1] - ok[j];
      for (int k = 0; k < nt; ++k, ++at) {
        const int valid = min(16, size - 16 * k);
        if (at < a.cap) a.col_idx[at] = (kc[j] + k) | (valid << kChunkShift);
      }
    }
    pos += __shfl(incl, 63);
  }
  const int null_chunk = a.NP / 16 - 1;
  for (int64_t p = pos + lane; p < end; p += 64)
    if (p < a.cap) a.col_idx[p] = null_chunk;
}

// Keys and staged values by chunk.  Key position p of chunk p / 16 in key
// cluster j holds token perm_k[off_k[j] + p - 16 kc[j]] while that is inside
// the cluster, zeros otherwise; the same chunk of V^T holds those tokens'
// values as fp16, transposed to [d][16] with the keys in the order the
// attention's PV operand takes them.  One workgroup per key cluster (z = 0
// keys, z = 1 values) takes its rows 64 at a time: all permutation entries
// are loaded, then all rows, so each pass waits on memory twice.  Workgroup
// Nk writes the all-padding chunk (the last chunk, zeros).  Chunks that no
// cluster owns are never read and stay unwritten.
template <int D>
__global__ __launch_bounds__(256) void cgather_kernel(ClusterAttnArgs a) {
  constexpr int C = D / 8;            // 16-byte pieces per row
  constexpr int PER = 64 * C / 256;   // pieces per thread per 64-row pass
  __shared__ uint32_t tile[64][D / 2 + 1];  // bf16 pairs; +1 word breaks bank aliasing
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const bool values = blockIdx.z == 1;
  const int tid = threadIdx.x;
  const int32_t* kc = a.kc + bh * (a.Nk + 1);
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  int chunk0, nch, size = 0;
  const int32_t* perm = a.perm_k + bh * a.N;
  if (j < a.Nk) {
    chunk0 = kc[j];
    nch = kc[j + 1] - chunk0;
    size = ok[j + 1] - ok[j];
    perm += ok[j];
  } else {
    chunk0 = a.NP / 16 - 1;
    nch = 1;
  }
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const uint16_t* src = (values ? a.V : a.K) + (int64_t)b * a.sb + (int64_t)h * a.sh;
  uint16_t* Kp = a.Kp + (bh * a.NP + 16 * (int64_t)chunk0) * D;
  uint16_t* Vt = a.Vt + (bh * (a.NP / 16) + chunk0) * (int64_t)D * 16;
  for (int r0 = 0; r0 < 16 * nch; r0 += 64) {
    int tok[PER];
    u32x4 v[PER];
    if (size > 0) {  // uniform; rows past the cluster read its last token, then zero
#pragma unroll
      for (int u = 0; u < PER; ++u) tok[u] = perm[min(r0 + (tid + 256 * u) / C, size - 1)];
#pragma unroll
      for (int u = 0; u < PER; ++u)
        v[u] = *(const u32x4*)(src + (int64_t)tok[u] * a.sn + 8 * ((tid + 256 * u) % C));
    }
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (size == 0 || r0 + (tid + 256 * u) / C >= size) v[u] = u32x4{0u, 0u, 0u, 0u};
    if (!values) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int f = tid + 256 * u, row = r0 + f / C;
        if (row < 16 * nch) *(u32x4*)(Kp + (int64_t)row * D + 8 * (f % C)) = v[u];
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int f = tid + 256 * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[f / C][(f % C) * 4 + e] = v[u][e];
    }
    __syncthreads();
    const uint16_t* t16 = (const uint16_t*)&tile[0][0];
    constexpr int RS = D + 2;  // row stride of the tile in bf16 elements
    for (int f = tid; f < D * 8; f += 256) {
      const int d = f >> 3, q = f & 7;  // 8 output keys at positions 8q..8q+7 of the pass
      const int c = r0 / 16 + (q >> 1);
      if (c >= nch) continue;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p0 = 8 * q + 2 * e;
        const int k0 = 16 * (p0 >> 4) + vt_key_of_pos(p0 & 15);
        const int k1 = 16 * ((p0 + 1) >> 4) + vt_key_of_pos((p0 + 1) & 15);
        w[e] = bf16_bits_to_f16_bits(t16[k0 * RS + d]) |
               (bf16_bits_to_f16_bits(t16[k1 * RS + d]) << 16);
      }
      *(u32x4*)(Vt + ((int64_t)c * D + d) * 16 + 8 * (q & 1)) = u32x4{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_cluster_attn_plan(const ClusterAttnArgs& a, int BH, int D, hipStream_t s) {
  (void)D;
  hipError_t e = launch_fill_i32(a.srcq, (int64_t)BH * a.NP, -1, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32((int32_t*)a.gmask, (int64_t)BH * a.Nq * a.W, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32((int32_t*)a.pairs, 2, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cplan_kernel, dim3(BH), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(ctile_group_kernel, dim3((a.nTP + 255) / 256, BH), dim3(256), 0, s, a);
  hipLaunchKernelGGL(cqsrc_kernel, dim3((a.N + 255) / 256, BH), dim3(256), 0, s, a);
  const dim3 wgrid((a.Nq + 3) / 4, BH);
  hipLaunchKernelGGL(cgmask_kernel, wgrid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(ccount_kernel, wgrid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cluster_attn_emit(const ClusterAttnArgs& a, int BH, int D, hipStream_t s) {
  hipLaunchKernelGGL(cemit_kernel, dim3((a.Nq + 3) / 4, BH), dim3(256), 0, s, a);
  const dim3 ggrid(a.Nk + 1, BH, 2);
  if (D == 128) hipLaunchKernelGGL(cgather_kernel<128>, ggrid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(cgather_kernel<64>, ggrid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
