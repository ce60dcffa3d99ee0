// Hardware-aware cluster merging (HyperVAttention section 4.3, Eq. 7-10,
// Algorithm 1): parallel agglomerative merging of query clusters that lowers
// the CTA-aligned cost
//   C(S) = tau_q ceil(s^q(S) / tau_q) * tau_k ceil(g * K(S) / tau_k),
//   K(S) = sum_j chi_j(S) ceil(s_j^k / g),
// where chi(S) is the union of the members' key-cluster rows and g the grain
// at which the executor packs a key cluster (g = 1 is the page's form).
//
// A group is named by its lowest member.  Per round, the active groups are
// split by the caller's side bits (read at each group's name); every side-0
// group A picks the side-1 group B of smallest gain C(A u B) - C(A) - C(B)
// (ties to the lower B); per target, the chooser of smallest negative gain
// is kept (ties to the lower A) and all kept pairs merge at once.
//
// Key-cluster masks are bitsets of W words.  K of a union is a weighted
// popcount: the slot counts are split into bit planes, so
// K(u) = sum_b 2^b popcount(u & plane_b), one lane per mask word.  Integer
// throughout: the result does not depend on scheduling.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

// t * ceil(x / t) for x >= 0, t >= 1: a 32-bit division whenever x fits
// (the usual case; 64-bit division is a long instruction sequence).
__device__ __forceinline__ int64_t ceil_multiple(uint64_t x, uint32_t t) {
  uint64_t q;
  if (x <= 0xFFFFFFFFull) {
    const uint32_t x32 = (uint32_t)x;
    q = x32 / t + (x32 % t != 0u ? 1u : 0u);
  } else {
    q = x / t + (x % t != 0u ? 1u : 0u);
  }
  return (int64_t)(q * t);
}

__device__ __forceinline__ int64_t group_cost(const ClusterMergeArgs& a, int64_t sq, int64_t k) {
  return ceil_multiple((uint64_t)sq, (uint32_t)a.tau_q) *
         ceil_multiple((uint64_t)a.grain * (uint64_t)k, (uint32_t)a.tau_k);
}

// Bit planes of the key clusters' slot counts ceil(s_j / g).  One thread per
// (head, mask word).
__global__ __launch_bounds__(256) void merge_planes_kernel(ClusterMergeArgs a) {
  const int w = blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (w >= a.W) return;
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  uint32_t* pl = a.planes + bh * a.nbits * a.W;
  for (int b = 0; b < a.nbits; ++b) {
    uint32_t word = 0;
    for (int t = 0; t < 32; ++t) {
      const int j = 32 * w + t;
      if (j < a.Nk) {
        const int c = (ok[j + 1] - ok[j] + a.grain - 1) / a.grain;
        word |= (uint32_t)((c >> b) & 1) << t;
      }
    }
    pl[b * a.W + w] = word;
  }
}

// Bits of the largest key-slot count of each head (planes above it are
// zero and are skipped).  One workgroup of 256 per head.
__global__ __launch_bounds__(256) void merge_bits_kernel(ClusterMergeArgs a) {
  __shared__ int red[4];
  const int64_t bh = blockIdx.x;
  const int32_t* ok = a.off_k + bh * (a.Nk + 1);
  int m = 0;
  for (int j = threadIdx.x; j < a.Nk; j += 256)
    m = max(m, (ok[j + 1] - ok[j] + a.grain - 1) / a.grain);
  for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    int bits = 0;
    while (bits < a.nbits && (m >> bits) != 0) ++bits;
    a.hbits[bh] = bits;
  }
}

// Weighted popcount of the union of two masks, one lane per word (W <= 128:
// two words per lane); the plane words come from LDS; nb planes.
__device__ __forceinline__ int union_slots(const ClusterMergeArgs& a, const uint32_t* pl,
                                           uint32_t u0, uint32_t u1, int lane, int nb) {
  int s = 0;
  for (int b = 0; b < nb; ++b) {
    int c = 0;
    if (lane < a.W) c += __popc(u0 & pl[b * a.W + lane]);
    if (lane + 64 < a.W) c += __popc(u1 & pl[b * a.W + lane + 64]);
    s += c << b;
  }
  return wave_sum(s);
}

// Singleton groups: name, query size, mask of the row (built in LDS by
// integer ORs), key slots.  One wave per query cluster.
__global__ __launch_bounds__(256) void merge_init_kernel(ClusterMergeArgs a) {
  __shared__ uint32_t words[4][128];
  __shared__ uint32_t pl[32 * 128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int64_t bh = blockIdx.y;
  for (int t = threadIdx.x; t < a.nbits * a.W; t += 256) pl[t] = a.planes[bh * a.nbits * a.W + t];
  for (int t = lane; t < 128; t += 64) words[wave][t] = 0u;
  __syncthreads();
  if (i >= a.Nq) return;
  const int64_t r = bh * a.Nq + i;
  for (int e = a.crow_ptr[r] + lane; e < a.crow_ptr[r + 1]; e += 64) {
    const int j = a.ccol[e];
    if (j >= 0 && j < a.Nk) atomicOr(&words[wave][j >> 5], 1u << (j & 31));
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const uint32_t u0 = lane < a.W ? words[wave][lane] : 0u;
  const uint32_t u1 = lane + 64 < a.W ? words[wave][lane + 64] : 0u;
  uint32_t* m = a.gmask + r * a.W;
  if (lane < a.W) m[lane] = u0;
  if (lane + 64 < a.W) m[lane + 64] = u1;
  const int k = union_slots(a, pl, u0, u1, lane, a.hbits[bh]);
  if (lane == 0) {
    a.grp[r] = i;
    a.gsq[r] = a.off_q[bh * (a.Nq + 1) + i + 1] - a.off_q[bh * (a.Nq + 1) + i];
    a.gk[r] = k;
  }
}

// The round's two sides, in ascending order of the groups' names (ordered
// compaction by ballots).  One workgroup of 1024 per head.
__global__ __launch_bounds__(1024) void merge_sides_kernel(ClusterMergeArgs a) {
  __shared__ int cnt[2][16];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint8_t* sd = a.sides + (bh * a.rounds + a.round) * a.Nq;
  int done[2] = {0, 0};
  for (int i0 = 0; i0 < a.Nq; i0 += 1024) {
    const int i = i0 + tid;
    bool act = false;
    int side = 0;
    if (i < a.Nq) {
      act = a.grp[bh * a.Nq + i] == i;
      side = sd[i] ? 1 : 0;
    }
    int pre[2], tot[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint64_t bal = __ballot(act && side == s);
      if (lane == 0) cnt[s][wave] = __popcll(bal);
      pre[s] = __popcll(bal & ((1ull << lane) - 1ull));
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      int before = 0;
      tot[s] = 0;
      for (int w = 0; w < 16; ++w) {
        if (w < wave) before += cnt[s][w];
        tot[s] += cnt[s][w];
      }
      pre[s] += before + done[s];
    }
    if (act) (side == 0 ? a.alist : a.blist)[bh * a.Nq + pre[side]] = i;
    done[0] += tot[0];
    done[1] += tot[1];
    __syncthreads();  // cnt is rewritten by the next chunk
  }
  if (tid == 0) {
    a.nab[bh * 2] = done[0];
    a.nab[bh * 2 + 1] = done[1];
  }
}

// One wave per chooser A: the target B of smallest gain over the side-1
// groups in ascending order (strict <, so ties keep the lower B).
// The four choosers of a workgroup scan the same targets, so the workgroup
// stages them together in LDS, kMergeChunk targets at a time (names, sizes
// and masks in one pass); all plane and mask reads in the scan are then LDS
// reads.
constexpr int kMergeChunk = 32;

__device__ __forceinline__ int union_slots_lds(const uint32_t* pl, int W, uint32_t u0,
                                               uint32_t u1, int w0, int w1, int nb) {
  // u0, u1 are zero on lanes past W, so the clamped plane words add nothing
  int s = 0;
  for (int b = 0; b < nb; ++b)
    s += (__popc(u0 & pl[b * W + w0]) + __popc(u1 & pl[b * W + w1])) << b;
  return wave_sum(s);
}

__global__ __launch_bounds__(256) void merge_gain_kernel(ClusterMergeArgs a) {
  extern __shared__ uint32_t dyn[];
  const int W = a.W;
  uint32_t* pl = dyn;                                   // [nbits][W]
  int* bl = (int*)(pl + a.nbits * W);                   // [kMergeChunk] target names
  int* bsq = bl + kMergeChunk;                          // their query sizes
  int* bgk = bsq + kMergeChunk;                         // their key slots
  uint32_t* cmk = (uint32_t*)(bgk + kMergeChunk);       // [kMergeChunk][W] their masks
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ai = blockIdx.x * 4 + wave;
  const int64_t bh = blockIdx.y;
  const int na = a.nab[bh * 2], nb = a.nab[bh * 2 + 1];
  const int32_t* blist = a.blist + bh * a.Nq;
  for (int t = tid; t < a.nbits * W; t += 256) pl[t] = a.planes[bh * a.nbits * W + t];
  const int hb = a.hbits[bh];
  const bool active = ai < na;  // inactive waves still stage and meet the barriers
  const int w0 = min(lane, W - 1), w1 = min(lane + 64, W - 1);
  uint32_t a0 = 0u, a1 = 0u;
  int64_t sqa = 0, ca = 0, ra = 0;
  if (active) {
    ra = bh * a.Nq + a.alist[bh * a.Nq + ai];
    const uint32_t* ma = a.gmask + ra * W;
    a0 = lane < W ? ma[lane] : 0u;
    a1 = lane + 64 < W ? ma[lane + 64] : 0u;
    sqa = a.gsq[ra];
    ca = group_cost(a, sqa, a.gk[ra]);
  }
  int64_t best = 0;
  int bestB = -1, bestK = 0;
  for (int c0 = 0; c0 < nb; c0 += kMergeChunk) {
    const int nc = min(kMergeChunk, nb - c0);
    for (int f = tid; f < nc * W; f += 256) {
      const int t = f / W, w = f - t * W;
      const int64_t rb = bh * a.Nq + blist[c0 + t];
      cmk[f] = a.gmask[rb * W + w];
      if (w == 0) {
        bl[t] = (int)(rb - bh * a.Nq);
        bsq[t] = a.gsq[rb];
        bgk[t] = a.gk[rb];
      }
    }
    __syncthreads();
    if (active) {
      for (int t = 0; t < nc; ++t) {
        const uint32_t* mb = cmk + t * W;
        const uint32_t u0 = a0 | (lane < W ? mb[w0] : 0u);
        const uint32_t u1 = a1 | (lane + 64 < W ? mb[w1] : 0u);
        const int k = union_slots_lds(pl, W, u0, u1, w0, w1, hb);
        const int64_t sqb = bsq[t];
        const int64_t gain = group_cost(a, sqa + sqb, k) - ca - group_cost(a, sqb, bgk[t]);
        if (bestB < 0 || gain < best) {
          best = gain;
          bestB = bl[t];
          bestK = k;
        }
      }
    }
    __syncthreads();  // the mask chunk is rewritten next
  }
  if (active && lane == 0) {
    a.choice[ra] = bestB;
    a.gain[ra] = best;
    a.ukeys[ra] = bestK;
  }
}

// Per target, the chooser of smallest negative gain (choosers scanned in
// ascending order, strict <); kept pairs merge into the lower name: sizes
// add, masks OR, key slots from the chooser's evaluation; then every
// cluster's group name follows.  One workgroup of 1024 per head.
__global__ __launch_bounds__(1024) void merge_apply_kernel(ClusterMergeArgs a) {
  __shared__ int newname[kMaxClusters];
  __shared__ int winner[kMaxClusters];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int na = a.nab[bh * 2], nb = a.nab[bh * 2 + 1];
  const int32_t* al = a.alist + bh * a.Nq;
  const int32_t* bl = a.blist + bh * a.Nq;
  for (int i = tid; i < a.Nq; i += 1024) newname[i] = i;
  for (int bi = tid; bi < nb; bi += 1024) {
    const int B = bl[bi];
    int w = -1;
    int64_t wg = 0;
    for (int ai = 0; ai < na; ++ai) {
      const int64_t ra = bh * a.Nq + al[ai];
      if (a.choice[ra] != B) continue;
      const int64_t g = a.gain[ra];
      if (g < 0 && (w < 0 || g < wg)) {
        w = al[ai];
        wg = g;
      }
    }
    winner[bi] = w;
  }
  __syncthreads();
  for (int bi = tid; bi < nb; bi += 1024) {
    const int A = winner[bi];
    if (A < 0) continue;
    const int B = bl[bi];
    const int lo = min(A, B), hi = max(A, B);
    const int64_t rl = bh * a.Nq + lo, rh = bh * a.Nq + hi;
    const int sq = a.gsq[rl] + a.gsq[rh];
    const int k = a.ukeys[bh * a.Nq + A];
    for (int w = 0; w < a.W; ++w) a.gmask[rl * a.W + w] |= a.gmask[rh * a.W + w];
    a.gsq[rl] = sq;
    a.gk[rl] = k;
    newname[A] = lo;
    newname[B] = lo;
  }
  __syncthreads();
  for (int i = tid; i < a.Nq; i += 1024) {
    int32_t* g = a.grp + bh * a.Nq + i;
    *g = newname[*g];
  }
}

}  // namespace

hipError_t launch_cluster_merge(const ClusterMergeArgs& a0, int BH, hipStream_t s) {
  ClusterMergeArgs a = a0;
  hipLaunchKernelGGL(merge_planes_kernel, dim3((a.W + 255) / 256, BH), dim3(256), 0, s, a);
  hipLaunchKernelGGL(merge_bits_kernel, dim3(BH), dim3(256), 0, s, a);
  const dim3 wgrid((a.Nq + 3) / 4, BH);
  // planes and one chunk of targets (at most (32*128 + 3*32 + 32*128) * 4 bytes)
  const size_t gain_lds =
      sizeof(uint32_t) * ((size_t)a.nbits * a.W + 3 * kMergeChunk + kMergeChunk * (size_t)a.W);
  hipLaunchKernelGGL(merge_init_kernel, wgrid, dim3(256), 0, s, a);
  for (int r = 0; r < a.rounds; ++r) {
    a.round = r;
    hipLaunchKernelGGL(merge_sides_kernel, dim3(BH), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(merge_gain_kernel, wgrid, dim3(256), gain_lds, s, a);
    hipLaunchKernelGGL(merge_apply_kernel, dim3(BH), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
