// Per-head omission risk of a sparse support (HyMoR-Attn abstract: the risk
// of leaving valuable support out is stable per layer and head, so it is
// calibrated offline).  For a query row with full-attention log-sum-exp Lf,
// sparse-support LSE Ls and (optionally) repaired LSE Lr:
//   omitted share    w = 1 - e^(Ls - Lf)               = -expm1(Ls - Lf)
//   recovered share  g = e^(Lr - Lf) - e^(Ls - Lf)     = e^(Ls - Lf) expm1(Lr - Ls)
// (e^L is the softmax normaliser over a support, so the ratios are mass
// shares of the full distribution).  The expm1 forms keep small shares exact
// to float32 rounding instead of cancelling in 1 - e^x.
//
// The work is a streaming reduction: 8 or 12 bytes read per row, three
// numbers written per head.  Pass 1 reduces 2048-row chunks of one head per
// workgroup into float64 partials (coalesced 4-byte loads, 8 rows per
// thread); pass 2 sums each head's chunks in a fixed order, so the result
// does not depend on scheduling.
#include <cmath>

#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kRiskThreads = 256;
constexpr int kRiskRowsPerThread = 8;

struct RowShares {
  float w, g;
};

__device__ inline RowShares row_shares(float ls, float lf, const float* Lr, int64_t i) {
  RowShares s{0.f, 0.f};
  if (lf == -INFINITY) return s;  // no keys at all: nothing to omit
  const float dl = ls - lf;       // -inf for an empty support
  s.w = -expm1f(dl);
  if (Lr != nullptr) {
    const float lr = Lr[i];
    s.g = (ls == -INFINITY) ? expf(lr - lf) : expf(dl) * expm1f(lr - ls);
  }
  return s;
}

__global__ __launch_bounds__(kRiskThreads) void risk_partial_kernel(RiskArgs a) {
  const int chunk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const float* Ls = a.Ls + bh * a.N;
  const float* Lf = a.Lf + bh * a.N;
  const float* Lr = a.Lr ? a.Lr + bh * a.N : nullptr;
  const int r0 = chunk * kRiskRowsPerChunk;
  const int r1 = min(r0 + kRiskRowsPerChunk, a.N);

  double sw = 0.0, sg = 0.0;
  float mw = -INFINITY;
#pragma unroll
  for (int it = 0; it < kRiskRowsPerThread; ++it) {
    const int r = r0 + it * kRiskThreads + (int)threadIdx.x;
    if (r < r1) {
      const RowShares s = row_shares(Ls[r], Lf[r], Lr, r);
      sw += s.w;
      sg += s.g;
      mw = fmaxf(mw, s.w);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    sw += __shfl_xor(sw, off);
    sg += __shfl_xor(sg, off);
    mw = fmaxf(mw, __shfl_xor(mw, off));
  }
  __shared__ double red[kRiskThreads / 64][3];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    red[wave][0] = sw;
    red[wave][1] = sg;
    red[wave][2] = mw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double tw = 0.0, tg = 0.0, tm = -INFINITY;
    for (int v = 0; v < kRiskThreads / 64; ++v) {
      tw += red[v][0];
      tg += red[v][1];
      tm = fmax(tm, red[v][2]);
    }
    double* p = a.partial + (bh * a.chunks + chunk) * 3;
    p[0] = tw;
    p[1] = tg;
    p[2] = tm;
  }
}

__global__ __launch_bounds__(kRiskThreads) void risk_final_kernel(RiskArgs a) {
  const int64_t bh = (int64_t)blockIdx.x * kRiskThreads + threadIdx.x;
  if (bh >= a.BH) return;
  const double* p = a.partial + bh * a.chunks * 3;
  double tw = 0.0, tg = 0.0, tm = -INFINITY;
  for (int c = 0; c < a.chunks; ++c) {
    tw += p[3 * c + 0];
    tg += p[3 * c + 1];
    tm = fmax(tm, p[3 * c + 2]);
  }
  double* out = a.risk + bh * 3;
  out[0] = tw / a.N;
  out[1] = tm;
  out[2] = tg / a.N;
}

}  // namespace

static_assert(kRiskRowsPerChunk == kRiskThreads * kRiskRowsPerThread,
              "one chunk is eight rows per thread");

hipError_t launch_risk(const RiskArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(risk_partial_kernel, dim3(a.chunks, a.BH), dim3(kRiskThreads), 0, s, a);
  hipLaunchKernelGGL(risk_final_kernel, dim3((a.BH + kRiskThreads - 1) / kRiskThreads),
                     dim3(kRiskThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
