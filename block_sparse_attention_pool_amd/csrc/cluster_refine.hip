// HyperVAttention section 4.2, the intermediate-step update of the hybrid
// clustering: the cached subset of tokens (the largest Lowe's ratios of the
// anchor step) is reassigned by a standard k-means step against every
// centroid of its head, not only its local window; then the centroids any
// subset token left or joined move to the mean of their members under the
// new assignment (a centroid left without members keeps its position).
//
// Launches per call:
//   refine_split_kernel    every centroid as three bf16 parts hi + mid + lo
//                          (each difference exact in float32, so the parts
//                          carry the float32 value) and its squared norm;
//   refine_assign_kernel   32 subset tokens per wave, their bf16 rows the B
//                          operand (in registers); the head's centroids
//                          staged 32 at a time in LDS as their three parts
//                          (16-byte pieces XOR-swizzled by row; the next
//                          chunk loaded into registers while the current
//                          one is multiplied), S^T = mu x^T
//                          on 32x32x16 bf16 products (exact products, float32
//                          sums); distance ||mu||^2 - 2 S (||x||^2 is the
//                          same for every candidate), lowest (distance,
//                          index) wins; a token whose centroid changes marks
//                          both centroids touched;
//   refine_count_kernel    the members of touched centroids counted (one
//                          atomic per group of a wave's lanes that share a
//                          centroid);
//   scan                   each touched centroid's range in a member list;
//   refine_scatter_kernel  each such member's token index written into its
//                          centroid's range (in no particular order; again
//                          one atomic per group);
//   refine_mean_kernel     one workgroup per touched centroid: its members'
//                          bf16 rows gathered (16 bytes per thread, four rows
//                          in flight) and summed in float64, then the count
//                          and the mean.
// Member sums of bf16 coordinates in float64 are exact -- so the order of
// the members does not change them -- while the largest and smallest nonzero
// magnitudes of one coordinate over a centroid's n members lie within a
// factor 2^(45 - log2 n) (8 significant bits each, 53 in the sum): 2^28 for
// a centroid of 2^17 members.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kRefineWaves = 8;  // waves (of 32 subset tokens) per workgroup

__device__ __forceinline__ bool is_touched(const RefineArgs& a, int64_t bh, int c) {
  return (a.touched[bh * a.W + (c >> 5)] >> (c & 31)) & 1u;
}

template <int D>
__global__ __launch_bounds__(D) void refine_split_kernel(RefineArgs a) {
  __shared__ float red[D / 64];
  const int64_t bc = (int64_t)blockIdx.y * a.Nc + blockIdx.x;
  const int e = threadIdx.x;
  const float v = a.mu[bc * D + e];
  const uint16_t hi = f32_to_bf16_bits(v);
  const float r = v - bf16_bits_to_f32(hi);
  const uint16_t mid = f32_to_bf16_bits(r);
  const uint16_t lo = f32_to_bf16_bits(r - bf16_bits_to_f32(mid));
  uint16_t* o = a.mu3 + bc * 3 * D;
  o[e] = hi;
  o[D + e] = mid;
  o[2 * D + e] = lo;
  const float sq = wave_sum(v * v);
  if ((e & 63) == 0) red[e >> 6] = sq;
  __syncthreads();
  if (e == 0) {
    float s = 0.f;
    for (int k = 0; k < D / 64; ++k) s += red[k];
    a.norm[bc] = s;
  }
}

template <int D>
__global__ __launch_bounds__(64 * kRefineWaves) void refine_assign_kernel(RefineArgs a) {
  constexpr int DC = D / 8;   // 16-byte pieces per row
  constexpr int KS = D / 16;  // k-steps
  __shared__ __attribute__((aligned(16))) uint16_t cm[3 * 32 * D];
  __shared__ __attribute__((aligned(16))) float cn[32];
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int k0 = (blockIdx.x * kRefineWaves + wave) * 32;
  const bool active = k0 < a.n_sub;  // wave-uniform
  const int k = k0 + n;
  int t = -1;
  if (k < a.n_sub) {
    t = a.subset[bh * a.n_sub + k];
    if ((unsigned)t >= (unsigned)a.N) t = -1;  // outside the head: ignored
  }
  bf16x8 xf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) xf[s] = bf16x8{};
  if (t >= 0) {
    const uint16_t* xr = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)t * a.sn + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) xf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xr + 16 * s));
  }
  const uint16_t* m3 = a.mu3 + bh * a.Nc * 3 * D;
  const float* nrm = a.norm + bh * a.Nc;
  // one chunk's pieces, loaded into registers (from clamped, in-bounds
  // centroids) while the previous chunk is multiplied, then stored to LDS
  // with zeros past the last centroid
  constexpr int NT = 64 * kRefineWaves;
  constexpr int NPC = 3 * 32 * DC;             // 16-byte pieces per chunk
  constexpr int PER = (NPC + NT - 1) / NT;
  u32x4 stage[PER];
  float nstage = 0.f;
  auto gload = [&](int c0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int f = min(tid + NT * q, NPC - 1);
      const int part = f / (32 * DC), m = (f / DC) % 32, c = f % DC;
      const int cu = min(c0 + m, a.Nc - 1);
      stage[q] = *(const u32x4*)(m3 + ((int64_t)cu * 3 + part) * D + 8 * c);
    }
    if (tid < 32) nstage = nrm[min(c0 + tid, a.Nc - 1)];
  };
  auto lstore = [&](int c0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int f = tid + NT * q;
      if (f < NPC) {
        const int part = f / (32 * DC), m = (f / DC) % 32, c = f % DC;
        const u32x4 v = c0 + m < a.Nc ? stage[q] : u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)&cm[(part * 32 + m) * D + ((c ^ (m % DC)) * 8)] = v;
      }
    }
    if (tid < 32) cn[tid] = c0 + tid < a.Nc ? nstage : 0.f;
  };
  float best = INFINITY;
  int best_u = 0x7fffffff;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c0 = 0; c0 < a.Nc; c0 += 32) {
    const int nc = min(32, a.Nc - c0);
    const bool more = c0 + 32 < a.Nc;
    if (more) gload(c0 + 32);
    if (active) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 af =
              *(const bf16x8*)&cm[(part * 32 + n) * D + (((2 * s + g) ^ (n % DC)) * 8)];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xf[s], acc, 0, 0, 0);
        }
      // lane (n, g) holds candidates m = 8 j + 4 g + q of token n, visited in
      // ascending order, so a strict improvement keeps the lower index
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 nn = *(const f32x4*)&cn[8 * j + 4 * g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 8 * j + 4 * g + q;
          const float dist = __builtin_fmaf(-2.f, acc[4 * j + q], nn[q]);
          if (m < nc && dist < best) {
            best = dist;
            best_u = c0 + m;
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
  if (!active) return;
  // the other 16 candidates of each chunk sit in lane n ^ 32
  const float ob = __shfl_xor(best, 32);
  const int ou = __shfl_xor(best_u, 32);
  if (ob < best || (ob == best && ou < best_u)) best_u = ou;
  // best_u stays out of range only if every distance was NaN (non-finite
  // inputs): the token then keeps its centroid
  if (g == 0 && t >= 0 && best_u < a.Nc) {
    int32_t* as = a.assign + bh * a.N + t;
    const int old = *as;
    *as = best_u;
    if (old != best_u) {
      uint32_t* tb = a.touched + bh * a.W;
      if ((unsigned)old < (unsigned)a.Nc) atomicOr(&tb[old >> 5], 1u << (old & 31));
      atomicOr(&tb[best_u >> 5], 1u << (best_u & 31));
    }
  }
}

// Lanes of a wave whose tokens belong to the same touched centroid are
// served by one atomic (consecutive tokens mostly share a few centroids, so
// per-lane atomics would queue on the same counters): the lowest pending
// lane's centroid is taken each round, with every lane of that centroid.
// f(key, n, rank, first) runs on the group's lanes: key = bh * Nc + c, n
// lanes in the group, this lane's rank among them, first the group's lowest
// lane.
template <class F>
__device__ __forceinline__ void per_centroid_group(bool pending, int key, F f) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t pend = __ballot(pending);
  while (pend) {
    const int first = __ffsll((unsigned long long)pend) - 1;
    const int k0 = __shfl(key, first);
    const bool mine = pending && key == k0;
    const uint64_t same = __ballot(mine);
    if (mine) f(k0, __popcll(same), __popcll(same & below), first);
    pending = pending && !mine;
    pend &= ~same;
  }
}

// One thread per (head, token).
__global__ __launch_bounds__(256) void refine_count_kernel(RefineArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool pending = false;
  int key = 0;
  if (f < total) {
    const int64_t bh = f / a.N;
    const int c = a.assign[f];
    pending = (unsigned)c < (unsigned)a.Nc && is_touched(a, bh, c);
    key = (int)(bh * a.Nc + c);
  }
  const int lane = threadIdx.x & 63;
  per_centroid_group(pending, key, [&](int k, int n, int, int first) {
    if (lane == first) atomicAdd(&a.tcount[k], n);
  });
}

// One thread per (head, token); consumes the counts: each group takes the
// top n free places of its centroid's range.
__global__ __launch_bounds__(256) void refine_scatter_kernel(RefineArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool pending = false;
  int key = 0;
  int64_t bh = 0;
  if (f < total) {
    bh = f / a.N;
    const int c = a.assign[f];
    pending = (unsigned)c < (unsigned)a.Nc && is_touched(a, bh, c);
    key = (int)(bh * a.Nc + c);
  }
  const int lane = threadIdx.x & 63;
  per_centroid_group(pending, key, [&](int k, int n, int rank, int first) {
    int top = 0;
    if (lane == first) top = atomicSub(&a.tcount[k], n);
    top = __shfl(top, first);  // the group's lanes are active: first holds the count
    a.list[a.offs[k] + top - 1 - rank] = (int32_t)(f - bh * a.N);
  });
}

// One workgroup per (centroid, head).
template <int D>
__global__ __launch_bounds__(256) void refine_mean_kernel(RefineArgs a) {
  constexpr int TPR = D / 8;       // threads per member row (16 bytes each)
  constexpr int RPP = 256 / TPR;   // rows per pass
  constexpr int U = 4;             // rows in flight per thread
  __shared__ double red[RPP][D];
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  if (!is_touched(a, bh, c)) return;
  const int64_t bc = bh * a.Nc + c;
  const int s0 = a.offs[bc];
  const int n = a.offs[bc + 1] - s0;
  const int tid = threadIdx.x;
  if (tid == 0) a.counts[bc] = n;
  if (n == 0) return;  // no members left: the centroid keeps its position
  const int r = tid / TPR, part = tid % TPR;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const uint16_t* Xh = a.X + (int64_t)b * a.sb + (int64_t)h * a.sh + part * 8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int k0 = 0; k0 < n; k0 += U * RPP) {
    int tok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + u * RPP + r;
      tok[u] = kk < n ? a.list[s0 + kk] : -1;
    }
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (tok[u] >= 0) v[u] = *(const u32x4*)(Xh + (int64_t)tok[u] * a.sn);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += (double)bf16_bits_to_f32(v[u][q] & 0xFFFFu);
        acc[2 * q + 1] += (double)bf16_bits_to_f32(v[u][q] >> 16);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r][part * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int rr = 0; rr < RPP; ++rr) s += red[rr][tid];
    a.mu[bc * D + tid] = (float)(s / (double)n);
  }
}

}  // namespace

hipError_t launch_subset_refine(const RefineArgs& a, int BH, int D, hipStream_t s) {
  if (a.n_sub == 0) return hipSuccess;  // nothing moves
  hipError_t e = launch_fill_i32((int32_t*)a.touched, (int64_t)BH * a.W, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(a.tcount, (int64_t)BH * a.Nc, 0, s);
  if (e != hipSuccess) return e;
  const dim3 cgrid(a.Nc, BH);
  const dim3 grid((a.n_sub + 32 * kRefineWaves - 1) / (32 * kRefineWaves), BH);
  if (D == 128) {
    hipLaunchKernelGGL(refine_split_kernel<128>, cgrid, dim3(128), 0, s, a);
    hipLaunchKernelGGL(refine_assign_kernel<128>, grid, dim3(64 * kRefineWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL(refine_split_kernel<64>, cgrid, dim3(64), 0, s, a);
    hipLaunchKernelGGL(refine_assign_kernel<64>, grid, dim3(64 * kRefineWaves), 0, s, a);
  }
  const int64_t ttot = (int64_t)BH * a.N;
  const dim3 tgrid((unsigned)((ttot + 255) / 256));
  hipLaunchKernelGGL(refine_count_kernel, tgrid, dim3(256), 0, s, a, ttot);
  e = launch_scan(a.tcount, BH * a.Nc, a.offs, a.total, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(refine_scatter_kernel, tgrid, dim3(256), 0, s, a, ttot);
  const dim3 mgrid(a.Nc, BH);
  if (D == 128) hipLaunchKernelGGL(refine_mean_kernel<128>, mgrid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(refine_mean_kernel<64>, mgrid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
