// 3D local-window clustering (HyperVAttention section 4.1, Eq. 5; Appendix
// A.2, Algorithm 2).  Tokens form a T x Hg x W lattice (t-major); a fixed
// grid of (kt, kh, kw) cells carries one centroid per cell, initialised at
// the cell's centre token.  Each iteration assigns every token to the
// nearest centroid among the cells of a window (wt, wh, ww) around its own
// cell, clipped to the grid, then moves each centroid to the mean of its
// tokens (a centroid with none stays).  Ties go to the lower centroid index.
//
// Kernels (one launch each, per iteration for the last two):
//   cluster_init_kernel    centroid u <- its centre token; squared norms;
//   cluster_assign_kernel  one workgroup per cell, one token per thread
//                          (the token in float32 registers); the window's
//                          centroids stream through LDS in chunks of 32 and
//                          are read as broadcasts; distance ||mu||^2 -
//                          2 x.mu (the token's own norm does not change the
//                          argmin), strict < over ascending indices;
//   cluster_update_kernel  one workgroup per centroid: the tokens that can
//                          be assigned to it lie in the cells whose windows
//                          contain it -- a box of cells per axis; the box is
//                          scanned in token order in chunks of 256, members
//                          compacted in order and summed per dimension in
//                          that order, so the centroids do not depend on
//                          scheduling (no atomics).
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kCandChunk = 32;

// First cell of the window around cell g on one axis, clipped to [0, K - w].
__device__ __forceinline__ int win_start(int g, int w, int K) {
  return min(max(g - w / 2, 0), K - w);
}

template <int D>
__global__ __launch_bounds__(D) void cluster_init_kernel(ClusterArgs a) {
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  const int t = min(ut * a.kt + a.kt / 2, a.T - 1);
  const int hh = min(uh * a.kh + a.kh / 2, a.Hg - 1);
  const int w = min(uw * a.kw + a.kw / 2, a.W - 1);
  const int64_t tok = ((int64_t)t * a.Hg + hh) * a.W + w;
  const int e = threadIdx.x;
  const float v = bf16_bits_to_f32(a.X[(int64_t)b * a.sb + (int64_t)h * a.sh + tok * a.sn + e]);
  a.mu[(bh * a.Nc + u) * D + e] = v;
  __shared__ float red[D / 64];
  float sq = wave_sum(v * v);
  if ((e & 63) == 0) red[e >> 6] = sq;
  __syncthreads();
  if (e == 0) {
    float s = 0.f;
    for (int k = 0; k < D / 64; ++k) s += red[k];
    a.norm[bh * a.Nc + u] = s;
  }
}

template <int D>
__global__ __launch_bounds__(512) void cluster_assign_kernel(ClusterArgs a) {
  __shared__ __attribute__((aligned(16))) float cm[kCandChunk][D];
  __shared__ float cn[kCandChunk];
  __shared__ int cid[kCandChunk];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  const int st = win_start(ut, a.wt, a.Kt), sh = win_start(uh, a.wh, a.Kh),
            sw = win_start(uw, a.ww, a.Kw);
  const int ncand = a.wt * a.wh * a.ww;
  // tokens of this cell
  const int t0 = ut * a.kt, h0 = uh * a.kh, w0 = uw * a.kw;
  const int lt = min(a.kt, a.T - t0), lh = min(a.kh, a.Hg - h0), lw = min(a.kw, a.W - w0);
  const int ntok = lt * lh * lw;
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const float* mu = a.mu + bh * a.Nc * D;
  const float* nrm = a.norm + bh * a.Nc;

  for (int base = 0; base < ntok; base += blockDim.x) {
    const int p = base + (int)threadIdx.x;
    const bool has = p < ntok;
    int64_t tok = 0;
    float x[D];
    if (has) {
      const int pt = p / (lh * lw), ph = (p / lw) % lh, pw = p % lw;
      tok = ((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
      const uint16_t* xr = Xh + tok * a.sn;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 v = *(const u32x4*)(xr + 8 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * c + 2 * k] = bf16_bits_to_f32(v[k] & 0xFFFFu);
          x[8 * c + 2 * k + 1] = bf16_bits_to_f32(v[k] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < D; ++e) x[e] = 0.f;
    }
    float best = INFINITY;
    int best_u = -1;
    for (int c0 = 0; c0 < ncand; c0 += kCandChunk) {
      const int nc = min(kCandChunk, ncand - c0);
      __syncthreads();  // the previous chunk is no longer read
      for (int f = threadIdx.x; f < nc * (D / 4); f += blockDim.x) {
        const int c = f / (D / 4), e4 = f % (D / 4);
        const int k = c0 + c;
        const int vw = sw + k % a.ww, vh = sh + (k / a.ww) % a.wh, vt = st + k / (a.ww * a.wh);
        const int v = (vt * a.Kh + vh) * a.Kw + vw;
        *(f32x4*)&cm[c][4 * e4] = *(const f32x4*)(mu + (int64_t)v * D + 4 * e4);
        if (e4 == 0) {
          cn[c] = nrm[v];
          cid[c] = v;
        }
      }
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < D; e += 4) {
          const f32x4 m = *(const f32x4*)&cm[c][e];
          dot = __builtin_fmaf(x[e], m[0], dot);
          dot = __builtin_fmaf(x[e + 1], m[1], dot);
          dot = __builtin_fmaf(x[e + 2], m[2], dot);
          dot = __builtin_fmaf(x[e + 3], m[3], dot);
        }
        const float dist = __builtin_fmaf(-2.f, dot, cn[c]);
        if (dist < best) {  // candidates ascend: ties keep the lower index
          best = dist;
          best_u = cid[c];
        }
      }
    }
    if (has) a.assign[bh * a.N + tok] = best_u;
  }
}

// Cells g on one axis whose window contains cell v: an interval, since the
// window start never decreases with g.
__device__ __forceinline__ void covering_cells(int v, int w, int K, int& lo, int& hi) {
  lo = K;
  hi = -1;
  for (int g = 0; g < K; ++g) {
    const int s = win_start(g, w, K);
    if (s <= v && v < s + w) {
      lo = min(lo, g);
      hi = max(hi, g);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void cluster_update_kernel(ClusterArgs a) {
  __shared__ int64_t list[256];
  __shared__ int wcnt[4];
  __shared__ float red[4];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  int glt, ght, glh, ghh, glw, ghw;
  covering_cells(ut, a.wt, a.Kt, glt, ght);
  covering_cells(uh, a.wh, a.Kh, glh, ghh);
  covering_cells(uw, a.ww, a.Kw, glw, ghw);
  // token box of those cells
  const int t0 = glt * a.kt, t1 = min((ght + 1) * a.kt, a.T);
  const int h0 = glh * a.kh, h1 = min((ghh + 1) * a.kh, a.Hg);
  const int w0 = glw * a.kw, w1 = min((ghw + 1) * a.kw, a.W);
  const int Lt = max(t1 - t0, 0), Lh = max(h1 - h0, 0), Lw = max(w1 - w0, 0);
  const int64_t P = (int64_t)Lt * Lh * Lw;
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int32_t* asg = a.assign + bh * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float acc = 0.f;  // thread e < D owns dimension e
  int count = 0;
  for (int64_t base = 0; base < P; base += 256) {
    const int64_t p = base + tid;
    int64_t tok = 0;
    bool m = false;
    if (p < P) {
      const int pt = (int)(p / ((int64_t)Lh * Lw)), ph = (int)((p / Lw) % Lh), pw = (int)(p % Lw);
      tok = ((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
      m = asg[tok] == u;
    }
    // ordered compaction of this chunk's members
    const uint64_t bal = __ballot(m);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < 4; ++k) {
      if (k < wave) off += wcnt[k];
      tot += wcnt[k];
    }
    if (m) list[off + before] = tok;
    __syncthreads();
    if (tid < D)
      for (int k = 0; k < tot; ++k)
        acc += bf16_bits_to_f32(Xh[list[k] * a.sn + tid]);
    count += tot;
    __syncthreads();  // list and wcnt are rewritten by the next chunk
  }
  if (tid == 0) a.counts[bh * a.Nc + u] = count;
  if (count == 0) return;  // the centroid keeps its position (and norm)
  float v = 0.f;
  if (tid < D) {
    v = acc / (float)count;
    a.mu[(bh * a.Nc + u) * D + tid] = v;
  }
  const float sq = wave_sum(tid < D ? v * v : 0.f);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int k = 0; k < 4; ++k) s += red[k];
    a.norm[bh * a.Nc + u] = s;
  }
}

// Eq. 1: the tokens of centroid u, in token order, at its place in the
// head's permutation.  The same box of cells as the update is scanned; the
// cluster's start comes from the scan of all heads' counts (minus the head's
// first entry); writes stop at the segment's end, whatever the counts say.
__global__ __launch_bounds__(256) void cluster_permute_kernel(ClusterArgs a,
                                                              const int32_t* gofs,
                                                              int32_t* perm,
                                                              int32_t* offsets) {
  __shared__ int wcnt[4];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  const int64_t base = gofs[bh * a.Nc];
  const int start = (int)(gofs[bh * a.Nc + u] - base);
  const int end = u + 1 < a.Nc ? (int)(gofs[bh * a.Nc + u + 1] - base) : a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    offsets[bh * (a.Nc + 1) + u] = start;
    if (u + 1 == a.Nc) offsets[bh * (a.Nc + 1) + a.Nc] = a.N;
  }
  int glt, ght, glh, ghh, glw, ghw;
  covering_cells(ut, a.wt, a.Kt, glt, ght);
  covering_cells(uh, a.wh, a.Kh, glh, ghh);
  covering_cells(uw, a.ww, a.Kw, glw, ghw);
  const int t0 = glt * a.kt, t1 = min((ght + 1) * a.kt, a.T);
  const int h0 = glh * a.kh, h1 = min((ghh + 1) * a.kh, a.Hg);
  const int w0 = glw * a.kw, w1 = min((ghw + 1) * a.kw, a.W);
  const int Lt = max(t1 - t0, 0), Lh = max(h1 - h0, 0), Lw = max(w1 - w0, 0);
  const int64_t P = (int64_t)Lt * Lh * Lw;
  const int32_t* asg = a.assign + bh * a.N;
  int32_t* pr = perm + bh * a.N;
  int done = 0;
  for (int64_t b0 = 0; b0 < P; b0 += 256) {
    const int64_t p = b0 + tid;
    int tok = 0;
    bool m = false;
    if (p < P) {
      const int pt = (int)(p / ((int64_t)Lh * Lw)), ph = (int)((p / Lw) % Lh), pw = (int)(p % Lw);
      tok = ((t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
      m = asg[tok] == u;
    }
    const uint64_t bal = __ballot(m);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = done, tot = 0;
    for (int q = 0; q < 4; ++q) {
      if (q < wave) off += wcnt[q];
      tot += wcnt[q];
    }
    const int pos = start + off + __popcll(bal & ((1ull << lane) - 1ull));
    if (m && pos < end) pr[pos] = tok;
    done += tot;
    __syncthreads();  // wcnt is rewritten by the next chunk
  }
}

}  // namespace

hipError_t launch_cluster_permute(const ClusterArgs& a, int BH, const int32_t* gofs,
                                  int32_t* perm, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(cluster_permute_kernel, dim3(a.Nc, BH), dim3(256), 0, s, a, gofs, perm,
                     offsets);
  return hipGetLastError();
}

hipError_t launch_cluster(const ClusterArgs& a, int BH, int iters, hipStream_t s) {
  const dim3 grid(a.Nc, BH);
  const int ctok = a.kt * a.kh * a.kw;
  const int threads = min(512, ((ctok + 63) / 64) * 64);
  if (a.D == 128) {
    hipLaunchKernelGGL(cluster_init_kernel<128>, grid, dim3(128), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(cluster_assign_kernel<128>, grid, dim3(threads), 0, s, a);
      hipLaunchKernelGGL(cluster_update_kernel<128>, grid, dim3(256), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL(cluster_init_kernel<64>, grid, dim3(64), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(cluster_assign_kernel<64>, grid, dim3(threads), 0, s, a);
      hipLaunchKernelGGL(cluster_update_kernel<64>, grid, dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace bsa
