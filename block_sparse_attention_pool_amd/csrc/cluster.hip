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

// LOWE: instead of the assignment, Lowe's ratio (HVA Eq. 6) of every token
// over the same candidates: the two smallest ||mu||^2 - 2 x.mu pick the
// nearest and the nearest other centroid, whose distances are then taken
// directly as sum (x - mu)^2 (the short form cancels when a token sits on a
// centroid); rho = d_1 / d_2, 0 with a single candidate, 1 when d_2 is 0.
template <int D, bool LOWE = false>
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
    float best = INFINITY, second = INFINITY;
    int best_u = -1, second_u = -1;
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
        if constexpr (LOWE) {
          if (dist < best) {
            second = best;
            second_u = best_u;
          } else if (dist < second) {
            second = dist;
            second_u = cid[c];
          }
        }
        if (dist < best) {  // candidates ascend: ties keep the lower index
          best = dist;
          best_u = cid[c];
        }
      }
    }
    if constexpr (LOWE) {
      if (has) {
        float r = 0.f;
        if (ncand > 1) {
          const float* m1 = mu + (int64_t)best_u * D;
          const float* m2 = mu + (int64_t)second_u * D;
          float d1 = 0.f, d2 = 0.f;
#pragma unroll
          for (int e = 0; e < D; e += 4) {
            const f32x4 p1 = *(const f32x4*)(m1 + e), p2 = *(const f32x4*)(m2 + e);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float u1 = x[e + q] - p1[q], u2 = x[e + q] - p2[q];
              d1 = __builtin_fmaf(u1, u1, d1);
              d2 = __builtin_fmaf(u2, u2, d2);
            }
          }
          r = d2 > 0.f ? sqrtf(d1 / d2) : 1.f;
          if (!(r > 0.f)) r = 0.f;  // +0: the subset search orders the bit patterns
        }
        a.rho[bh * a.N + tok] = r;
      }
    } else {
      if (has) a.assign[bh * a.N + tok] = best_u;
    }
  }
}

// Every centroid as three bf16 parts hi + mid + lo: hi = bf16(mu), mid =
// bf16(mu - hi), lo = bf16(mu - hi - mid) (each difference exact in fp32),
// which carry the float32 value.  Token vectors are bf16, so the products
// of the matrix-core assignment are exact and only its float32 sums round.
template <int D>
__global__ __launch_bounds__(D) void centroid_split_kernel(ClusterArgs a) {
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int e = threadIdx.x;
  const float v = a.mu[(bh * a.Nc + u) * D + e];
  const uint16_t hi = f32_to_bf16_bits(v);
  const float r = v - bf16_bits_to_f32(hi);
  const uint16_t mid = f32_to_bf16_bits(r);
  const uint16_t lo = f32_to_bf16_bits(r - bf16_bits_to_f32(mid));
  uint16_t* o = a.mu3 + (bh * a.Nc + u) * 3 * D;
  o[e] = hi;
  o[D + e] = mid;
  o[2 * D + e] = lo;
}

// Assignment on the matrix cores: one workgroup per cell, one wave per 32
// tokens (B operand: the token's bf16 row, held in registers); the window's
// centroids are staged 32 at a time in LDS as their three bf16 parts (A
// operand, 16-byte pieces XOR-swizzled by row), and S^T = mu x^T accumulates
// hi, mid and lo products in float32 (32x32x16 bf16).  A lane then holds 16
// candidates of one token (its lane pair the other 16): distance ||mu||^2 -
// 2 S, lowest (distance, index) wins, so ties keep the lower index.
template <int D>
__global__ __launch_bounds__(1024) void cluster_assign_mfma_kernel(ClusterArgs a) {
  constexpr int DC = D / 8;   // 16-byte pieces per row
  constexpr int KS = D / 16;  // k-steps
  __shared__ __attribute__((aligned(16))) uint16_t cm[3 * 32 * D];
  __shared__ __attribute__((aligned(16))) float cn[32];
  __shared__ int cid[32];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  const int st = win_start(ut, a.wt, a.Kt), sh = win_start(uh, a.wh, a.Kh),
            sw = win_start(uw, a.ww, a.Kw);
  const int ncand = a.wt * a.wh * a.ww;
  const int t0 = ut * a.kt, h0 = uh * a.kh, w0 = uw * a.kw;
  const int lt = min(a.kt, a.T - t0), lh = min(a.kh, a.Hg - h0), lw = min(a.kw, a.W - w0);
  const int ntok = lt * lh * lw;
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* m3 = a.mu3 + bh * a.Nc * 3 * D;
  const float* nrm = a.norm + bh * a.Nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int n = lane & 31, g = lane >> 5;

  for (int tb = 0; tb < ntok; tb += 32 * nwaves) {
    const int p = tb + 32 * wave + n;  // this lane's token (column n)
    const bool active = tb + 32 * wave < ntok;  // wave-uniform
    int64_t tok = 0;
    bf16x8 xf[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) xf[s2] = bf16x8{};
    if (p < ntok) {
      const int pt = p / (lh * lw), ph = (p / lw) % lh, pw = p % lw;
      tok = ((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
      const uint16_t* xr = Xh + tok * a.sn + 8 * g;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        xf[s2] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xr + 16 * s2));
    }
    float best = INFINITY;
    int best_u = 0x7fffffff;
    for (int c0 = 0; c0 < ncand; c0 += 32) {
      const int nc = min(32, ncand - c0);
      __syncthreads();  // the previous chunk is no longer read
      for (int f = tid; f < 3 * 32 * DC; f += blockDim.x) {
        const int part = f / (32 * DC), m = (f / DC) % 32, c = f % DC;
        u32x4 v = {0u, 0u, 0u, 0u};
        int vid = 0;
        if (m < nc) {
          const int k = c0 + m;
          const int vw = sw + k % a.ww, vh = sh + (k / a.ww) % a.wh, vt = st + k / (a.ww * a.wh);
          vid = (vt * a.Kh + vh) * a.Kw + vw;
          v = *(const u32x4*)(m3 + ((int64_t)vid * 3 + part) * D + 8 * c);
        }
        *(u32x4*)&cm[(part * 32 + m) * D + ((c ^ (m % DC)) * 8)] = v;
        if (part == 0 && c == 0) {
          cn[m] = m < nc ? nrm[vid] : 0.f;
          cid[m] = m < nc ? vid : 0x7fffffff;
        }
      }
      __syncthreads();
      if (!active) continue;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const bf16x8 af = *(const bf16x8*)&cm[(part * 32 + n) * D + (((2 * s2 + g) ^ (n % DC)) * 8)];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[s2], acc, 0, 0, 0);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 nn = *(const f32x4*)&cn[8 * j + 4 * g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 8 * j + 4 * g + q;
          const float dist = __builtin_fmaf(-2.f, acc[4 * j + q], nn[q]);
          const int id = cid[m];
          if (m < nc && (dist < best || (dist == best && id < best_u))) {
            best = dist;
            best_u = id;
          }
        }
      }
    }
    if (!active) continue;
    // the other 16 candidates of this token sit in lane n ^ 32
    const float ob = __shfl_xor(best, 32);
    const int ou = __shfl_xor(best_u, 32);
    if (ob < best || (ob == best && ou < best_u)) best_u = ou;
    if (g == 0 && p < ntok) a.assign[bh * a.N + tok] = best_u;
  }
}

// The same assignment with the window's centroid ids and norms tabulated
// once per cell (windows of at most kMaxAssignWindow cells) and the next
// 32-centroid chunk loaded into registers while the current one is
// multiplied, so the chunk copies overlap the matrix work.  PER 16-byte
// pieces per thread cover a chunk's three parts; the results are those of
// cluster_assign_mfma_kernel bit for bit (same products in the same order).
// LOWE: Lowe's ratio (HVA Eq. 6) instead of the assignment: the two
// smallest (||mu||^2 - 2 x.mu, index) pick the nearest and the nearest other
// centroid, whose distances are then taken directly as sum (x - mu)^2 over
// the float32 centroids (the short form cancels when a token sits on a
// centroid); rho = sqrt(d_1 / d_2), 0 with a single candidate, 1 when d_2 is 0.
template <int D, int PER, bool LOWE = false>
__global__ __launch_bounds__(PER >= 4 ? 512 : 1024) void cluster_assign_pf_kernel(ClusterArgs a) {
  constexpr int DC = D / 8;          // 16-byte pieces per row
  constexpr int KS = D / 16;         // k-steps
  constexpr int NPC = 3 * 32 * DC;   // pieces per chunk
  __shared__ __attribute__((aligned(16))) uint16_t cm[3 * 32 * D];
  __shared__ int tid_of[kMaxAssignWindow];
  __shared__ float tnorm[kMaxAssignWindow];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  const int st = win_start(ut, a.wt, a.Kt), sh = win_start(uh, a.wh, a.Kh),
            sw = win_start(uw, a.ww, a.Kw);
  const int ncand = a.wt * a.wh * a.ww;
  const int t0 = ut * a.kt, h0 = uh * a.kh, w0 = uw * a.kw;
  const int lt = min(a.kt, a.T - t0), lh = min(a.kh, a.Hg - h0), lw = min(a.kw, a.W - w0);
  const int ntok = lt * lh * lw;
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* m3 = a.mu3 + bh * a.Nc * 3 * D;
  const float* nrm = a.norm + bh * a.Nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, nwaves = nthr >> 6;
  const int n = lane & 31, g = lane >> 5;

  for (int k = tid; k < ncand; k += nthr) {
    const int vw = sw + k % a.ww, vh = sh + (k / a.ww) % a.wh, vt = st + k / (a.ww * a.wh);
    const int vid = (vt * a.Kh + vh) * a.Kw + vw;
    tid_of[k] = vid;
    tnorm[k] = nrm[vid];
  }
  __syncthreads();
  // one chunk's pieces: loads from clamped (in-bounds) candidates, then the
  // LDS stores with zeros past the window
  u32x4 stage[PER];
  auto gload = [&](int c0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int f = min(tid + nthr * q, NPC - 1);
      const int part = f / (32 * DC), m = (f / DC) % 32, c = f % DC;
      const int vid = tid_of[min(c0 + m, ncand - 1)];
      stage[q] = *(const u32x4*)(m3 + ((int64_t)vid * 3 + part) * D + 8 * c);
    }
  };
  auto lstore = [&](int c0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int f = tid + nthr * q;
      if (f < NPC) {
        const int part = f / (32 * DC), m = (f / DC) % 32, c = f % DC;
        const u32x4 v = c0 + m < ncand ? stage[q] : u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)&cm[(part * 32 + m) * D + ((c ^ (m % DC)) * 8)] = v;
      }
    }
  };

  for (int tb = 0; tb < ntok; tb += 32 * nwaves) {
    const int p = tb + 32 * wave + n;  // this lane's token (column n)
    const bool active = tb + 32 * wave < ntok;  // wave-uniform
    int64_t tok = 0;
    bf16x8 xf[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) xf[s2] = bf16x8{};
    if (p < ntok) {
      const int pt = p / (lh * lw), ph = (p / lw) % lh, pw = p % lw;
      tok = ((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
      const uint16_t* xr = Xh + tok * a.sn + 8 * g;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        xf[s2] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xr + 16 * s2));
    }
    float best = INFINITY, second = INFINITY;
    int best_u = 0x7fffffff, second_u = 0x7fffffff;
    __syncthreads();  // the previous token batch no longer reads the chunk buffer
    gload(0);
    lstore(0);
    __syncthreads();
    for (int c0 = 0; c0 < ncand; c0 += 32) {
      const bool more = c0 + 32 < ncand;
      if (more) gload(c0 + 32);
      if (active) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) {
            const bf16x8 af =
                *(const bf16x8*)&cm[(part * 32 + n) * D + (((2 * s2 + g) ^ (n % DC)) * 8)];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[s2], acc, 0, 0, 0);
          }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = 8 * j + 4 * g + q;
            const int k = min(c0 + m, ncand - 1);
            const float dist = __builtin_fmaf(-2.f, acc[4 * j + q], tnorm[k]);
            const int id = tid_of[k];
            if constexpr (LOWE) {
              if (c0 + m < ncand) {
                if (dist < best || (dist == best && id < best_u)) {
                  second = best;
                  second_u = best_u;
                  best = dist;
                  best_u = id;
                } else if (dist < second || (dist == second && id < second_u)) {
                  second = dist;
                  second_u = id;
                }
              }
            } else if (c0 + m < ncand && (dist < best || (dist == best && id < best_u))) {
              best = dist;
              best_u = id;
            }
          }
        }
      }
      __syncthreads();  // every wave is done with this chunk
      if (more) {
        lstore(c0 + 32);
        __syncthreads();
      }
    }
    if (!active) continue;
    // the other 16 candidates of this token sit in lane n ^ 32
    const float ob = __shfl_xor(best, 32);
    const int ou = __shfl_xor(best_u, 32);
    if constexpr (LOWE) {
      const float os = __shfl_xor(second, 32);
      const int osu = __shfl_xor(second_u, 32);
      auto lt = [](float d1, int u1, float d2, int u2) { return d1 < d2 || (d1 == d2 && u1 < u2); };
      // merge the lane pair's two ordered pairs
      if (lt(ob, ou, best, best_u)) {
        if (lt(best, best_u, os, osu)) {
          second = best;
          second_u = best_u;
        } else {
          second = os;
          second_u = osu;
        }
        best = ob;
        best_u = ou;
      } else if (lt(ob, ou, second, second_u)) {
        second = ob;
        second_u = ou;
      }
      // direct squared distances over this lane's half of the row (elements
      // 16 s + 8 g .. +7), the halves added across the lane pair
      const bool two = (unsigned)second_u < (unsigned)a.Nc && (unsigned)best_u < (unsigned)a.Nc;
      float d1 = 0.f, d2 = 0.f;
      if (two) {
        const float* m1 = a.mu + (bh * a.Nc + best_u) * D + 8 * g;
        const float* m2 = a.mu + (bh * a.Nc + second_u) * D + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const u32x4 xv = __builtin_bit_cast(u32x4, xf[s2]);
#pragma unroll
          for (int hq = 0; hq < 2; ++hq) {
            const f32x4 p1 = *(const f32x4*)(m1 + 16 * s2 + 4 * hq);
            const f32x4 p2 = *(const f32x4*)(m2 + 16 * s2 + 4 * hq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t w2 = xv[2 * hq + (e >> 1)];
              const float xe = bf16_bits_to_f32((e & 1) ? (w2 >> 16) : (w2 & 0xFFFFu));
              const float u1 = xe - p1[e], u2 = xe - p2[e];
              d1 = __builtin_fmaf(u1, u1, d1);
              d2 = __builtin_fmaf(u2, u2, d2);
            }
          }
        }
      }
      d1 += __shfl_xor(d1, 32);
      d2 += __shfl_xor(d2, 32);
      float r = 0.f;
      if (two) {
        r = d2 > 0.f ? sqrtf(d1 / d2) : 1.f;
        if (!(r > 0.f)) r = 0.f;  // +0: the subset search orders the bit patterns
      }
      if (g == 0 && p < ntok) a.rho[bh * a.N + tok] = r;
    } else {
      if (ob < best || (ob == best && ou < best_u)) best_u = ou;
      if (g == 0 && p < ntok) a.assign[bh * a.N + tok] = best_u;
    }
  }
}

// Squared norms of given centroids (for the ratio pass).
template <int D>
__global__ __launch_bounds__(D) void centroid_norm_kernel(ClusterArgs a) {
  __shared__ float red[D / 64];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int e = threadIdx.x;
  const float v = a.mu[(bh * a.Nc + u) * D + e];
  const float sq = wave_sum(v * v);
  if ((e & 63) == 0) red[e >> 6] = sq;
  __syncthreads();
  if (e == 0) {
    float s = 0.f;
    for (int k = 0; k < D / 64; ++k) s += red[k];
    a.norm[bh * a.Nc + u] = s;
  }
}

// The n_sub tokens of largest ratio per head (equal ratios to the lower
// index), ascending: the threshold is found by a radix selection, a byte at
// a time, over the ratios' bit patterns (order-preserving for values >= 0),
// then the tokens above it and the first of those equal to it are compacted
// in token order.  One workgroup of 1024 per head.
__global__ __launch_bounds__(1024) void lowe_subset_kernel(ClusterArgs a, int n_sub,
                                                           int32_t* subset) {
  __shared__ int red[16];
  __shared__ int wc[2][16];
  const int64_t bh = blockIdx.x;
  const float* r = a.rho + bh * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_count = [&](int c) {
    c = wave_sum(c);
    if (lane == 0) red[wave] = c;
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += red[w];
    __syncthreads();
    return tot;
  };
  // the n_sub-th largest bit pattern, one byte at a time (most significant
  // first): a 256-bin histogram of the patterns that match the bytes found so
  // far, and the bin where the count from the top reaches what remains
  __shared__ uint32_t hist[256];
  __shared__ int pick[2];
  uint32_t T = 0, pmask = 0;
  int remaining = n_sub;
  for (int shift = 24; shift >= 0 && n_sub > 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < a.N; i += 1024) {
      const uint32_t k = __float_as_uint(r[i]);
      if ((k & pmask) == T) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const int b0 = 4 * lane;
      const int hq[4] = {(int)hist[b0], (int)hist[b0 + 1], (int)hist[b0 + 2], (int)hist[b0 + 3]};
      const int mine = hq[0] + hq[1] + hq[2] + hq[3];
      int suf = mine;  // patterns in bins >= b0
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
      }
      int above = suf - mine;  // patterns in bins >= b0 + 4
      if (above < remaining && suf >= remaining) {
        for (int q = 3; q >= 0; --q) {
          if (above + hq[q] >= remaining) {
            pick[0] = b0 + q;
            pick[1] = above;
            break;
          }
          above += hq[q];
        }
      }
    }
    __syncthreads();
    T |= (uint32_t)pick[0] << shift;
    pmask |= 0xFFu << shift;
    remaining -= pick[1];
    __syncthreads();
  }
  int c = 0;
  for (int i = tid; i < a.N; i += 1024) c += __float_as_uint(r[i]) > T ? 1 : 0;
  const int need_eq = n_sub - block_count(c);
  int done = 0, eq_done = 0;
  for (int i0 = 0; i0 < a.N && done < n_sub; i0 += 1024) {
    const int i = i0 + tid;
    const uint32_t key = i < a.N ? __float_as_uint(r[i]) : 0u;
    const bool gt = i < a.N && key > T, eq = i < a.N && key == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wc[0][wave] = __popcll(beq);
    __syncthreads();
    int eq_before = eq_done + __popcll(beq & ((1ull << lane) - 1ull)), eq_tot = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) eq_before += wc[0][w];
      eq_tot += wc[0][w];
    }
    const bool sel = gt || (eq && eq_before < need_eq);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wc[1][wave] = __popcll(bsel);
    __syncthreads();
    int pos = done + __popcll(bsel & ((1ull << lane) - 1ull)), tot = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) pos += wc[1][w];
      tot += wc[1][w];
    }
    if (sel && pos < n_sub) subset[bh * n_sub + pos] = i;
    done += tot;
    eq_done += eq_tot;
    __syncthreads();  // wc is rewritten by the next chunk
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

// Update through per-cell buckets.  cell_bucket_kernel: one workgroup per
// cell sorts the cell's tokens by the slot of their centroid in the cell's
// window (a counting sort; ties in token order): bucket[c][...] holds token
// indices, bstart[c][k] the start of slot k.  cluster_update_bucket_kernel:
// one workgroup per centroid walks the cells whose windows contain it in
// ascending order, gathers the tokens of its slot in each, and sums their
// rows in that order -- a fixed order, so results do not vary from run to
// run, and only member rows are read (the box scan reads an assignment for
// every token of the box).
__global__ __launch_bounds__(256) void cell_bucket_kernel(ClusterArgs a) {
  __shared__ int slot[kMaxBucketCell];
  __shared__ int hist[kMaxBucketSlots + 1];
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int uw = c % a.Kw, uh = (c / a.Kw) % a.Kh, ut = c / (a.Kw * a.Kh);
  const int st = win_start(ut, a.wt, a.Kt), sh = win_start(uh, a.wh, a.Kh),
            sw = win_start(uw, a.ww, a.Kw);
  const int ncand = a.wt * a.wh * a.ww;
  const int t0 = ut * a.kt, h0 = uh * a.kh, w0 = uw * a.kw;
  const int lt = min(a.kt, a.T - t0), lh = min(a.kh, a.Hg - h0), lw = min(a.kw, a.W - w0);
  const int ntok = lt * lh * lw;
  const int cmax = a.kt * a.kh * a.kw;
  const int32_t* asg = a.assign + bh * a.N;
  const int tid = threadIdx.x;
  for (int k = tid; k <= ncand; k += 256) hist[k] = 0;
  __syncthreads();
  for (int p = tid; p < ntok; p += 256) {
    const int pt = p / (lh * lw), ph = (p / lw) % lh, pw = p % lw;
    const int64_t tok = ((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw);
    const int v = asg[tok];
    const int vw = v % a.Kw, vh = (v / a.Kw) % a.Kh, vt = v / (a.Kw * a.Kh);
    const int k = ((vt - st) * a.wh + (vh - sh)) * a.ww + (vw - sw);
    const bool in = vt >= st && vt < st + a.wt && vh >= sh && vh < sh + a.wh && vw >= sw &&
                    vw < sw + a.ww;
    slot[p] = in ? k : ncand;  // outside the window (never, for this clustering): dropped
    atomicAdd(&hist[in ? k : ncand], 1);
  }
  __syncthreads();
  if (tid == 0) {  // exclusive scan of at most kMaxBucketSlots counts
    int run = 0;
    for (int k = 0; k <= ncand; ++k) {
      const int v = hist[k];
      hist[k] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t* bs = a.bstart + (bh * a.Nc + c) * (ncand + 1);
  for (int k = tid; k <= ncand; k += 256) bs[k] = hist[k];
  int32_t* bk = a.bucket + (bh * a.Nc + c) * cmax;
  for (int p = tid; p < ntok; p += 256) {
    const int k = slot[p];
    if (k == ncand) continue;
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += slot[q] == k ? 1 : 0;
    const int pt = p / (lh * lw), ph = (p / lw) % lh, pw = p % lw;
    bk[hist[k] + rank] = (int32_t)(((int64_t)(t0 + pt) * a.Hg + (h0 + ph)) * a.W + (w0 + pw));
  }
}

// The cells whose windows contain centroid u, ascending, with u's slot range
// in each one's bucket: ccell[i], cb0[i], and exclusive member offsets
// cofs[0..ncov] (cofs[ncov] = members).  Block of 256 threads; returns ncov.
__device__ int gather_covering(const ClusterArgs& a, int64_t bh, int u, int* ccell, int* cb0,
                               int* ccnt, int* cofs) {
  const int uw = u % a.Kw, uh = (u / a.Kw) % a.Kh, ut = u / (a.Kw * a.Kh);
  int glt, ght, glh, ghh, glw, ghw;
  covering_cells(ut, a.wt, a.Kt, glt, ght);
  covering_cells(uh, a.wh, a.Kh, glh, ghh);
  covering_cells(uw, a.ww, a.Kw, glw, ghw);
  const int nt = max(ght - glt + 1, 0), nh = max(ghh - glh + 1, 0), nw = max(ghw - glw + 1, 0);
  const int ncov = nt * nh * nw;
  const int ncand = a.wt * a.wh * a.ww;
  for (int i = threadIdx.x; i < ncov; i += blockDim.x) {
    const int gt = glt + i / (nh * nw), gh = glh + (i / nw) % nh, gw = glw + i % nw;
    const int c = (gt * a.Kh + gh) * a.Kw + gw;
    const int st = win_start(gt, a.wt, a.Kt), sh = win_start(gh, a.wh, a.Kh),
              sw = win_start(gw, a.ww, a.Kw);
    const int k = ((ut - st) * a.wh + (uh - sh)) * a.ww + (uw - sw);
    const int32_t* bs = a.bstart + (bh * a.Nc + c) * (ncand + 1);
    ccell[i] = c;
    cb0[i] = bs[k];
    ccnt[i] = bs[k + 1] - bs[k];
  }
  __syncthreads();
  // exclusive offsets by a block scan: thread t takes items t*per .. t*per+per-1
  __shared__ int wsum[16];
  const int t = threadIdx.x, nthr = blockDim.x, lane = t & 63, wave = t >> 6;
  const int per = (ncov + nthr - 1) / nthr;
  int loc = 0;
  for (int q = 0; q < per; ++q) {
    const int i = t * per + q;
    if (i < ncov) loc += ccnt[i];
  }
  const int inc = wave_inclusive_scan(loc);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + inc - loc;
  for (int q = 0; q < per; ++q) {
    const int i = t * per + q;
    if (i < ncov) {
      cofs[i] = run;
      run += ccnt[i];
    }
  }
  if (t == nthr - 1) cofs[ncov] = before + inc;
  __syncthreads();
  return ncov;
}

// Member x (0 <= x < cofs[ncov]) of the gathered covering cells.
__device__ __forceinline__ int32_t covering_member(const ClusterArgs& a, int64_t bh, int ncov,
                                                   const int* ccell, const int* cb0,
                                                   const int* cofs, int x) {
  int lo = 0, hi = ncov - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cofs[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return a.bucket[(bh * a.Nc + ccell[lo]) * (a.kt * a.kh * a.kw) + cb0[lo] + (x - cofs[lo])];
}

template <int D>
__global__ __launch_bounds__(256) void cluster_update_bucket_kernel(ClusterArgs a) {
  __shared__ int cb0[kMaxBucketSlots], ccnt[kMaxBucketSlots], cofs[kMaxBucketSlots + 1];
  __shared__ int ccell[kMaxBucketSlots];
  __shared__ int list[1024];
  __shared__ float part[256 / (D / 8)][D + 1];
  __shared__ float red[4];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncov = gather_covering(a, bh, u, ccell, cb0, ccnt, cofs);
  const int count = cofs[ncov];
  // member rows 16 bytes per thread: G members per pass, thread (g, c) adds
  // dimensions 8c .. 8c+7 of members g, g + G, ... in order, four rows in
  // flight; the G partial sums are then added in order of g (a fixed order)
  constexpr int C = D / 8, G = 256 / C;
  const int c = tid % C, gi = tid / C;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto add = [&](const u32x4& w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_f32(w[e] & 0xFFFFu);
      acc[2 * e + 1] += bf16_bits_to_f32(w[e] >> 16);
    }
  };
  for (int base = 0; base < count; base += 1024) {
    const int nb = min(1024, count - base);
    for (int j = tid; j < nb; j += 256)
      list[j] = covering_member(a, bh, ncov, ccell, cb0, cofs, base + j);
    __syncthreads();
    int j = gi;
    for (; j + 3 * G < nb; j += 4 * G) {
      u32x4 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = *(const u32x4*)(Xh + (int64_t)list[j + q * G] * a.sn + 8 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) add(w[q]);
    }
    for (; j < nb; j += G) add(*(const u32x4*)(Xh + (int64_t)list[j] * a.sn + 8 * c));
    __syncthreads();  // list is rewritten by the next batch
  }
  if (tid == 0) a.counts[bh * a.Nc + u] = count;
  if (count == 0) return;  // the centroid keeps its position (and norm)
#pragma unroll
  for (int e = 0; e < 8; ++e) part[gi][8 * c + e] = acc[e];
  __syncthreads();
  float v = 0.f;
  if (tid < D) {
    float sum = 0.f;
    for (int k = 0; k < G; ++k) sum += part[k][tid];
    v = sum / (float)count;
    a.mu[(bh * a.Nc + u) * D + tid] = v;
  }
  const float sq = wave_sum(tid < D ? v * v : 0.f);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  if (tid == 0) {
    float s2 = 0.f;
    for (int k = 0; k < 4; ++k) s2 += red[k];
    a.norm[bh * a.Nc + u] = s2;
  }
}

// Eq. 1 through the buckets: centroid u's members gathered from its covering
// cells into LDS, each placed at its rank in token order (tokens are
// distinct), so the output equals the box scan's.  A cluster with more than
// kMaxPermMembers members takes the box scan below.
constexpr int kMaxPermMembers = 2048;

__global__ __launch_bounds__(256) void cluster_permute_bucket_kernel(ClusterArgs a,
                                                                     const int32_t* gofs,
                                                                     int32_t* perm,
                                                                     int32_t* offsets,
                                                                     int32_t* big) {
  __shared__ int cb0[kMaxBucketSlots], ccnt[kMaxBucketSlots], cofs[kMaxBucketSlots + 1];
  __shared__ int ccell[kMaxBucketSlots];
  __shared__ int mem[kMaxPermMembers];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t base = gofs[bh * a.Nc];
  const int start = (int)(gofs[bh * a.Nc + u] - base);
  const int end = u + 1 < a.Nc ? (int)(gofs[bh * a.Nc + u + 1] - base) : a.N;
  if (threadIdx.x == 0) {
    offsets[bh * (a.Nc + 1) + u] = start;
    if (u + 1 == a.Nc) offsets[bh * (a.Nc + 1) + a.Nc] = a.N;
  }
  const int ncov = gather_covering(a, bh, u, ccell, cb0, ccnt, cofs);
  const int n = cofs[ncov];
  if (n > kMaxPermMembers) {  // too many for LDS: the box scan handles it
    if (threadIdx.x == 0) big[bh * a.Nc + u] = 1;
    return;
  }
  if (threadIdx.x == 0) big[bh * a.Nc + u] = 0;
  for (int j = threadIdx.x; j < n; j += blockDim.x)
    mem[j] = covering_member(a, bh, ncov, ccell, cb0, cofs, j);
  __syncthreads();
  int32_t* pr = perm + bh * a.N;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int t = mem[j];
    int rank = 0;
    for (int q = 0; q < n; ++q) rank += mem[q] < t ? 1 : 0;
    if (start + rank < end) pr[start + rank] = t;
  }
}

// Eq. 1: the tokens of centroid u, in token order, at its place in the
// head's permutation.  The same box of cells as the update is scanned; the
// cluster's start comes from the scan of all heads' counts (minus the head's
// first entry); writes stop at the segment's end, whatever the counts say.
__global__ __launch_bounds__(256) void cluster_permute_kernel(ClusterArgs a,
                                                              const int32_t* gofs,
                                                              int32_t* perm,
                                                              int32_t* offsets,
                                                              const int32_t* big) {
  __shared__ int wcnt[4];
  const int u = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (big != nullptr && big[bh * a.Nc + u] == 0) return;  // placed through the buckets
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
                                  int32_t* perm, int32_t* offsets, int32_t* big, hipStream_t s) {
  const dim3 grid(a.Nc, BH);
  if (a.bucket != nullptr) {
    hipLaunchKernelGGL(cell_bucket_kernel, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(cluster_permute_bucket_kernel, grid, dim3(256), 0, s, a, gofs, perm,
                       offsets, big);
    // clusters too large for LDS (rare): the box scan, which skips the rest
    hipLaunchKernelGGL(cluster_permute_kernel, grid, dim3(256), 0, s, a, gofs, perm, offsets,
                       (const int32_t*)big);
  } else {
    hipLaunchKernelGGL(cluster_permute_kernel, grid, dim3(256), 0, s, a, gofs, perm, offsets,
                       (const int32_t*)nullptr);
  }
  return hipGetLastError();
}

// The prefetching assignment for windows of at most kMaxAssignWindow cells
// (4 to 16 waves, one per 32 tokens of a cell; four or more pieces per
// thread only with at most 448 threads), else the plain one.
template <int D, bool LOWE = false>
void launch_assign_pf(const ClusterArgs& a, dim3 grid, int ctok, hipStream_t s) {
  const int waves = min(16, (ctok + 31) / 32);
  const int threads = 64 * max(4, waves);
  const int per = (3 * 32 * (D / 8) + threads - 1) / threads;
  switch (per) {
    case 1: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 1, LOWE>), grid, dim3(threads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 2, LOWE>), grid, dim3(threads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 3, LOWE>), grid, dim3(threads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 4, LOWE>), grid, dim3(threads), 0, s, a); break;
    case 5: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 5, LOWE>), grid, dim3(threads), 0, s, a); break;
    default: hipLaunchKernelGGL((cluster_assign_pf_kernel<D, 6, LOWE>), grid, dim3(threads), 0, s, a); break;
  }
}

template <int D>
void launch_assign(const ClusterArgs& a, dim3 grid, int ncand, int ctok, hipStream_t s) {
  const int waves = min(16, (ctok + 31) / 32);
  if (ncand > kMaxAssignWindow) {
    hipLaunchKernelGGL(cluster_assign_mfma_kernel<D>, grid, dim3(64 * waves), 0, s, a);
    return;
  }
  launch_assign_pf<D>(a, grid, ctok, s);
}

// Lowe's ratios on the matrix cores for windows of at most kMaxAssignWindow
// cells (the centroids split into bf16 parts first), else with float32 FMAs.
hipError_t launch_lowe(const ClusterArgs& a, int BH, int n_sub, int32_t* subset, hipStream_t s) {
  const dim3 grid(a.Nc, BH);
  const int ctok = a.kt * a.kh * a.kw;
  const int threads = min(512, ((ctok + 63) / 64) * 64);
  const bool mfma = a.wt * a.wh * a.ww <= kMaxAssignWindow;
  if (a.D == 128) {
    hipLaunchKernelGGL(centroid_norm_kernel<128>, grid, dim3(128), 0, s, a);
    if (mfma) {
      hipLaunchKernelGGL(centroid_split_kernel<128>, grid, dim3(128), 0, s, a);
      launch_assign_pf<128, true>(a, grid, ctok, s);
    } else {
      hipLaunchKernelGGL((cluster_assign_kernel<128, true>), grid, dim3(threads), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL(centroid_norm_kernel<64>, grid, dim3(64), 0, s, a);
    if (mfma) {
      hipLaunchKernelGGL(centroid_split_kernel<64>, grid, dim3(64), 0, s, a);
      launch_assign_pf<64, true>(a, grid, ctok, s);
    } else {
      hipLaunchKernelGGL((cluster_assign_kernel<64, true>), grid, dim3(threads), 0, s, a);
    }
  }
  hipLaunchKernelGGL(lowe_subset_kernel, dim3(BH), dim3(1024), 0, s, a, n_sub, subset);
  return hipGetLastError();
}

hipError_t launch_cluster(const ClusterArgs& a, int BH, int iters, hipStream_t s) {
  const dim3 grid(a.Nc, BH);
  const int ctok = a.kt * a.kh * a.kw;
  const int threads = min(512, ((ctok + 63) / 64) * 64);
  const int ncand = a.wt * a.wh * a.ww;
  (void)threads;
  // bucketed update when a cell's tokens and a window's slots fit the LDS
  // tables (the workspace then holds the buckets), else the box scan
  const bool buckets = a.bucket != nullptr;
  if (a.D == 128) {
    hipLaunchKernelGGL(cluster_init_kernel<128>, grid, dim3(128), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(centroid_split_kernel<128>, grid, dim3(128), 0, s, a);
      launch_assign<128>(a, grid, ncand, ctok, s);
      if (buckets) {
        hipLaunchKernelGGL(cell_bucket_kernel, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(cluster_update_bucket_kernel<128>, grid, dim3(256), 0, s, a);
      } else {
        hipLaunchKernelGGL(cluster_update_kernel<128>, grid, dim3(256), 0, s, a);
      }
    }
  } else {
    hipLaunchKernelGGL(cluster_init_kernel<64>, grid, dim3(64), 0, s, a);
    for (int it = 0; it < iters; ++it) {
      hipLaunchKernelGGL(centroid_split_kernel<64>, grid, dim3(64), 0, s, a);
      launch_assign<64>(a, grid, ncand, ctok, s);
      if (buckets) {
        hipLaunchKernelGGL(cell_bucket_kernel, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(cluster_update_bucket_kernel<64>, grid, dim3(256), 0, s, a);
      } else {
        hipLaunchKernelGGL(cluster_update_kernel<64>, grid, dim3(256), 0, s, a);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace bsa
