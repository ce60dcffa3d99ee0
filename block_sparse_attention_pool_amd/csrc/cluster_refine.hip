// HyperVAttention section 4.2, the intermediate-step update of the hybrid
// clustering: the cached subset of tokens (the largest Lowe's ratios of the
// anchor step) is reassigned by a standard k-means step against every
// centroid of its head, not only its local window; then the centroids any
// subset token left or joined move to the mean of their members under the
// new assignment (a centroid left without members keeps its position).
//
// Four launches per call:
//   refine_assign_kernel  64 subset tokens per workgroup, four lanes per
//                         token (d/4 coordinates each, in registers); the
//                         head's centroids staged 32 at a time in LDS (the
//                         same row is a broadcast to the 16 tokens of a
//                         wave); squared distances sum(x - mu)^2 in float32,
//                         the four partial sums added across the lane quad;
//                         lowest (distance, index) wins; a token whose
//                         centroid changes marks both centroids touched;
//   refine_clear_kernel   zeroes the member sums and counts of touched
//                         centroids;
//   refine_sum_kernel     one thread per (token, 8 coordinates): members of
//                         touched centroids add their bf16 coordinates to the
//                         centroid's float64 sums (and count themselves);
//   refine_update_kernel  touched centroids: count, and mean when non-empty.
// Member sums of bf16 coordinates in float64 are exact (so independent of
// the order of the atomic adds) while a centroid's member coordinates span
// less than about 2^40 in magnitude.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kRefineTokens = 64;  // subset tokens per workgroup
constexpr int kRefineChunk = 32;   // centroids per LDS stage

template <int D>
__global__ __launch_bounds__(256) void refine_assign_kernel(RefineArgs a) {
  constexpr int P = D / 4;  // coordinates per lane
  __shared__ float smu[kRefineChunk][D];
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int tid = threadIdx.x;
  const int ts = tid >> 2, part = tid & 3;
  const int k = blockIdx.x * kRefineTokens + ts;
  int t = -1;
  if (k < a.n_sub) {
    t = a.subset[bh * a.n_sub + k];
    if ((unsigned)t >= (unsigned)a.N) t = -1;  // outside the head: ignored
  }
  float x[P];
  const uint16_t* xr = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh +
                       (int64_t)(t < 0 ? 0 : t) * a.sn + part * P;
#pragma unroll
  for (int e = 0; e < P / 8; ++e) {
    const u32x4 v = *(const u32x4*)(xr + 8 * e);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[8 * e + 2 * q] = bf16_bits_to_f32(v[q] & 0xFFFFu);
      x[8 * e + 2 * q + 1] = bf16_bits_to_f32(v[q] >> 16);
    }
  }
  const float* mu = a.mu + bh * (int64_t)a.Nc * D;
  float best_d = INFINITY;
  int best = 0;
  for (int c0 = 0; c0 < a.Nc; c0 += kRefineChunk) {
    const int nc = min(kRefineChunk, a.Nc - c0);
    __syncthreads();  // the previous chunk has been read
    for (int f = tid; f < kRefineChunk * D / 4; f += 256) {
      const int r = f / (D / 4), col = (f % (D / 4)) * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (r < nc) v = *(const f32x4*)(mu + (int64_t)(c0 + r) * D + col);
      *(f32x4*)&smu[r][col] = v;
    }
    __syncthreads();
    for (int r = 0; r < nc; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float dv = x[e] - smu[r][part * P + e];
        acc = __builtin_fmaf(dv, dv, acc);
      }
      // the four lanes of a token hold its four partial sums
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (acc < best_d) {  // strictly smaller: equal distances keep the lower index
        best_d = acc;
        best = c0 + r;
      }
    }
  }
  if (t >= 0 && part == 0) {
    int32_t* as = a.assign + bh * a.N + t;
    const int old = *as;
    *as = best;
    if (old != best) {
      uint32_t* tb = a.touched + bh * a.W;
      if ((unsigned)old < (unsigned)a.Nc) atomicOr(&tb[old >> 5], 1u << (old & 31));
      atomicOr(&tb[best >> 5], 1u << (best & 31));
    }
  }
}

// One thread per (head, centroid, 8 coordinates).
template <int D>
__global__ __launch_bounds__(256) void refine_clear_kernel(RefineArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= total) return;
  const int part = (int)(f % (D / 8));
  const int64_t bc = f / (D / 8);  // bh * Nc + c
  const int c = (int)(bc % a.Nc);
  const int64_t bh = bc / a.Nc;
  if (((a.touched[bh * a.W + (c >> 5)] >> (c & 31)) & 1u) == 0u) return;
  double* s = a.sums + bc * D + part * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  if (part == 0) a.tcount[bc] = 0;
}

// One thread per (head, token, 8 coordinates).
template <int D>
__global__ __launch_bounds__(256) void refine_sum_kernel(RefineArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= total) return;
  const int part = (int)(f % (D / 8));
  const int64_t bt = f / (D / 8);  // bh * N + t
  const int t = (int)(bt % a.N);
  const int64_t bh = bt / a.N;
  const int c = a.assign[bt];
  if ((unsigned)c >= (unsigned)a.Nc) return;
  if (((a.touched[bh * a.W + (c >> 5)] >> (c & 31)) & 1u) == 0u) return;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const u32x4 v = *(const u32x4*)(a.X + (int64_t)b * a.sb + (int64_t)h * a.sh +
                                  (int64_t)t * a.sn + part * 8);
  double* s = a.sums + (bh * a.Nc + c) * D + part * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    unsafeAtomicAdd(&s[2 * q], (double)bf16_bits_to_f32(v[q] & 0xFFFFu));
    unsafeAtomicAdd(&s[2 * q + 1], (double)bf16_bits_to_f32(v[q] >> 16));
  }
  if (part == 0) atomicAdd(&a.tcount[bh * a.Nc + c], 1);
}

// One thread per (head, centroid, 8 coordinates).
template <int D>
__global__ __launch_bounds__(256) void refine_update_kernel(RefineArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= total) return;
  const int part = (int)(f % (D / 8));
  const int64_t bc = f / (D / 8);
  const int c = (int)(bc % a.Nc);
  const int64_t bh = bc / a.Nc;
  if (((a.touched[bh * a.W + (c >> 5)] >> (c & 31)) & 1u) == 0u) return;
  const int n = a.tcount[bc];
  if (part == 0) a.counts[bc] = n;
  if (n == 0) return;  // no members left: the centroid keeps its position
  const double* s = a.sums + bc * D + part * 8;
  float* m = a.mu + bc * D + part * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = (float)(s[e] / (double)n);
}

}  // namespace

hipError_t launch_subset_refine(const RefineArgs& a, int BH, int D, hipStream_t s) {
  hipError_t e = launch_fill_i32((int32_t*)a.touched, (int64_t)BH * a.W, 0, s);
  if (e != hipSuccess) return e;
  if (a.n_sub > 0) {
    const dim3 grid((a.n_sub + kRefineTokens - 1) / kRefineTokens, BH);
    if (D == 128) hipLaunchKernelGGL(refine_assign_kernel<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(refine_assign_kernel<64>, grid, dim3(256), 0, s, a);
  }
  const int64_t ctot = (int64_t)BH * a.Nc * (D / 8);
  const int64_t ttot = (int64_t)BH * a.N * (D / 8);
  const dim3 cgrid((unsigned)((ctot + 255) / 256)), tgrid((unsigned)((ttot + 255) / 256));
  if (D == 128) {
    hipLaunchKernelGGL(refine_clear_kernel<128>, cgrid, dim3(256), 0, s, a, ctot);
    hipLaunchKernelGGL(refine_sum_kernel<128>, tgrid, dim3(256), 0, s, a, ttot);
    hipLaunchKernelGGL(refine_update_kernel<128>, cgrid, dim3(256), 0, s, a, ctot);
  } else {
    hipLaunchKernelGGL(refine_clear_kernel<64>, cgrid, dim3(256), 0, s, a, ctot);
    hipLaunchKernelGGL(refine_sum_kernel<64>, tgrid, dim3(256), 0, s, a, ttot);
    hipLaunchKernelGGL(refine_update_kernel<64>, cgrid, dim3(256), 0, s, a, ctot);
  }
  return hipGetLastError();
}

}  // namespace bsa
