// Pooled rectification of omitted blocks (Rectified SpaAttn: sparse
// attention over-weights the kept blocks and drops the omitted ones; pooled
// query-key interactions recover both).  Reading implemented here: every
// key block j omitted by a query block's row contributes its pooled
// estimate -- softmax normaliser n_j exp(scale q . Kbar_j), value sum
// n_j exp(scale q . Kbar_j) Vbar_j, both exact when the block's keys are all
// equal -- and that pooled attention is merged into the sparse (O, LSE)
// by the exact LSE merge, in place.
//
// Gain-Aware Pooling Rectification (the abstract asks that the recovered
// gain exceed the pooling error it brings in), as read here: the estimate
// of block j for query q recovers the mass n_j exp(scale q . Kbar_j); with
// the block's keys spread normally and isotropically about their mean, the
// true mass is that estimate times exp(sigma^2 / 2), sigma^2 =
// scale^2 |q|^2 v_j (v_j the per-coordinate variance of the block's keys),
// so the estimate's error stays below its gain while exp(sigma^2 / 2) < 2:
// the gate keeps block j for query q when |q|^2 v_j < 2 ln 2 / scale^2.
// v_j comes from rect_spread_kernel (one more pass over K); |q|^2 is summed
// from the query fragments the kernel already holds.
//
// Three launches (four with the gate): the 64-token means of K and V (pool_kernel, float32,
// into the workspace); their conversion to the matrix-core operands
// (Kbar as bf16 high + low parts, so that q . Kbar carries about 16
// mantissa bits; Vbar as fp16 in 16-key chunks [d][16]); and the rectify
// kernel: one workgroup per query block, wave a on query rows 16a..16a+15,
// all four waves walking the pooled keys 16 at a time.  Each step's tiles
// (Kbar high and low rows, 4 KB each at d = 128, and the Vbar^T chunk, 4 KB)
// are copied once per workgroup into double-buffered LDS -- the next step's
// global loads are in flight while the current step computes, one barrier
// per step; the key rows are padded by 16 bytes so that the 16 rows a
// fragment read touches fall in distinct banks.  S^T = Kbar Q^T on 16x16x32
// bf16 products (twice: high and low parts), mask of the row's kept blocks
// from an LDS bitmap, log2 of the block size added, online softmax,
// O^T = Vbar^T P^T on 16x16x16 fp16 products, then the merge with the
// sparse result in the epilogue.  Steps whose 16 blocks are all kept are
// skipped.
#include <cmath>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

// Sum of the two fp16 halves of `packed` added to acc (dot with (1, 1)).
__device__ __forceinline__ float sum_f16x2(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// One thread per (head, padded block j, element d): Kbar -> bf16 high and
// low parts [BH][nBp][D], Vbar -> fp16 [BH][nBp/16][D][16].  Blocks
// j >= nB (padding to a multiple of 16) are zero.
template <int D>
__global__ __launch_bounds__(256) void rect_convert_kernel(RectifyArgs a, int64_t total) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= total) return;
  const int d = (int)(f % D);
  const int64_t jj = f / D;
  const int j = (int)(jj % a.nBp);
  const int64_t bh = jj / a.nBp;
  float k = 0.f, v = 0.f;
  if (j < a.nB) {
    k = a.Kf[(bh * a.nB + j) * D + d];
    v = a.Vf[(bh * a.nB + j) * D + d];
  }
  const uint16_t hi = f32_to_bf16_bits(k);
  const uint16_t lo = f32_to_bf16_bits(k - bf16_bits_to_f32(hi));
  a.Khi[(bh * a.nBp + j) * D + d] = hi;
  a.Klo[(bh * a.nBp + j) * D + d] = lo;
  a.Vt[((bh * (a.nBp / 16) + j / 16) * D + d) * 16 + (j % 16)] =
      __builtin_bit_cast(uint16_t, (_Float16)v);
}

// One workgroup per (head, padded block j): v_j = sum over the block's valid
// keys of |k - Kbar_j|^2 / (n_j D), summed in a fixed order (each thread
// its 16-byte chunks, then the block sum), 0 for padding blocks.
template <int D>
__global__ __launch_bounds__(256) void rect_spread_kernel(RectifyArgs a) {
  constexpr int C = D / 8;             // 16-byte chunks per key row
  constexpr int PER = 64 * C / 256;    // chunks per thread
  __shared__ float red[4];
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  float acc = 0.f;
  const int n = j < a.nB ? min(kBlock, a.N - j * kBlock) : 0;
  if (n > 0) {
    const int c = tid % C;  // the same coordinates for every chunk of this thread
    const float* mean = a.Kf + (bh * a.nB + j) * D + 8 * c;
    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = mean[e];
    const uint16_t* Kh = a.K + (int64_t)b * a.sb + (int64_t)h * a.sh;
    u32x4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = (tid + 256 * u) / C;  // token of the block
      v[u] = *(const u32x4*)(Kh + (int64_t)(j * kBlock + min(t, n - 1)) * a.sn + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = (tid + 256 * u) / C;
      if (t < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf16_bits_to_f32(v[u][e] & 0xFFFFu) - mu[2 * e];
          const float x1 = bf16_bits_to_f32(v[u][e] >> 16) - mu[2 * e + 1];
          acc = __builtin_fmaf(x0, x0, acc);
          acc = __builtin_fmaf(x1, x1, acc);
        }
      }
    }
  }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    a.spread[bh * a.nBp + j] = n > 0 ? tot / (float)(n * D) : 0.f;
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* O, int64_t off, float x0, float x1, float x2,
                                       float x3) {
  if constexpr (BF16) {
    const u32x2 v = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    *(u32x2*)((uint16_t*)O + off) = v;
  } else {
    const f32x4 v = {x0, x1, x2, x3};
    *(f32x4*)((float*)O + off) = v;
  }
}

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* O, int64_t off) {
  if constexpr (BF16) {
    const u32x2 v = *(const u32x2*)((const uint16_t*)O + off);
    return f32x4{bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16),
                 bf16_bits_to_f32(v[1] & 0xFFFFu), bf16_bits_to_f32(v[1] >> 16)};
  } else {
    return *(const f32x4*)((const float*)O + off);
  }
}

template <int D, bool OUT_BF16>
// Scheduled for four waves per SIMD (the compiler otherwise plans for three):
// 0.59 -> 0.51 ms on the 32K layer, 7.4 -> 6.9 ms on the 14B layer.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void rectify_kernel(RectifyArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int KP = D + 8;             // padded LDS row of a pooled key (conflict-free reads)
  constexpr int TILE = 2 * 16 * KP + 16 * D;  // Khi, Klo rows, then Vbar^T [D][16]
  constexpr int NCH = 6 * D;            // 16-byte chunks of one step's tiles (3 x 2D)
  __shared__ uint32_t kept[kMaxRowWords];
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][TILE];
  const int i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int tid = threadIdx.x;

  // bitmap of the key blocks this row keeps
  const int W = (a.nB + 31) / 32;
  for (int w = tid; w < W; w += 256) kept[w] = 0u;
  __syncthreads();
  const int64_t r = bh * a.nB + i;
  const int rb = a.row_ptr[r], re = a.row_ptr[r + 1];
  for (int e = rb + tid; e < re; e += 256) {
    const int j = a.col_idx[e];
    atomicOr(&kept[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // omitted blocks among j0 .. j0+15, and the next group that has any
  auto omitted_of = [&](int j0) {
    const uint32_t word = kept[j0 >> 5] >> (j0 & 31);
    const int nv = min(16, a.nB - j0);
    return ~word & ((1u << nv) - 1u);
  };
  auto next_active = [&](int j0) {
    while (j0 < a.nB && omitted_of(j0) == 0u) j0 += 16;
    return j0;
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int q0 = i * kBlock + wave * kMicro;
  const bool live = q0 < a.N;  // every wave takes part in the tile copies and barriers

  const int64_t base = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int q = q0 + n16;
  // the query rows are loaded together from clamped (in-bounds) rows, then
  // rows past N are zeroed
  const uint16_t* qrow = a.Q + base + (int64_t)min(q, a.N - 1) * a.sn + 8 * g4;
  u32x4 qv[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qv[s] = *(const u32x4*)(qrow + 32 * s);
  bf16x8 qf[KS];
  float qn2 = 0.f;  // |q|^2 of this lane's query (gate), from the fragments of all 4 lane groups
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (q >= a.N) qv[s] = u32x4{0u, 0u, 0u, 0u};
    qf[s] = __builtin_bit_cast(bf16x8, qv[s]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_bits_to_f32(qv[s][e] & 0xFFFFu), x1 = bf16_bits_to_f32(qv[s][e] >> 16);
      qn2 = __builtin_fmaf(x0, x0, qn2);
      qn2 = __builtin_fmaf(x1, x1, qn2);
    }
  }
  qn2 += __shfl_xor(qn2, 16);
  qn2 += __shfl_xor(qn2, 32);
  const bool gated = a.gate != 0;
  const float* spread = a.spread + bh * a.nBp;
  f32x4 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  const float lg_tail = __builtin_log2f((float)(a.N - (a.nB - 1) * kBlock));
  const uint16_t* Khi = a.Khi + bh * a.nBp * D;
  const uint16_t* Klo = a.Klo + bh * a.nBp * D;
  const uint16_t* Vt = a.Vt + bh * a.nBp * D;

  // one step's tiles: chunk c of Khi / Klo (rows j0.., contiguous) or of the
  // Vbar^T chunk j0/16 (contiguous), staged through registers
  constexpr int CPT = (NCH + 255) / 256;
  u32x4 stage[CPT];
  auto gload = [&](int j0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ch = tid + 256 * k;
      if (ch < NCH) {
        const int arr = ch / (2 * D), off = (ch % (2 * D)) * 8;
        const uint16_t* src = arr == 0 ? Khi + (int64_t)j0 * D
                            : arr == 1 ? Klo + (int64_t)j0 * D
                                       : Vt + (int64_t)(j0 / 16) * D * 16;
        stage[k] = *(const u32x4*)(src + off);
      }
    }
  };
  auto lstore = [&](uint16_t* buf) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ch = tid + 256 * k;
      if (ch < NCH) {
        const int arr = ch / (2 * D), off = (ch % (2 * D)) * 8;
        uint16_t* dst = arr < 2 ? buf + arr * 16 * KP + (off / D) * KP + off % D
                                : buf + 2 * 16 * KP + off;
        *(u32x4*)dst = stage[k];
      }
    }
  };

  // the spread of the lane's four pooled keys of a step (gate only)
  auto sload = [&](int j0) {
    return gated ? *(const f32x4*)(spread + j0 + 4 * g4) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  int j = next_active(0);
  int cur = 0;
  f32x4 sp = {0.f, 0.f, 0.f, 0.f};
  if (j < a.nB) {
    gload(j);
    sp = sload(j);
    lstore(tiles[0]);
  }
  __syncthreads();
  while (j < a.nB) {
    const int jn = next_active(j + 16);
    f32x4 sp_next = sp;
    if (jn < a.nB) {
      gload(jn);
      sp_next = sload(jn);
    }
    if (live) {
      const uint16_t* tk = tiles[cur];
      const uint32_t omitted = omitted_of(j);
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 khi = *(const bf16x8*)(tk + n16 * KP + 32 * s + 8 * g4);
        const bf16x8 klo = *(const bf16x8*)(tk + 16 * KP + n16 * KP + 32 * s + 8 * g4);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, qf[s], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(klo, qf[s], sacc, 0, 0, 0);
      }
      // lane holds pooled keys j + 4 g4 + rr of query q (log2 domain)
      float x[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int jj = 4 * g4 + rr;
        const float lg = j + jj == a.nB - 1 ? lg_tail : 6.0f;  // log2 of the block size
        const bool keep = ((omitted >> jj) & 1u) && (!gated || qn2 * sp[rr] < a.gate_thr);
        x[rr] = keep ? __builtin_fmaf(sacc[rr], c, lg) : -INFINITY;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      if (__any(m_new > m_run + 8.0f)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t] *= alpha;
        m_run = m_new;
      }
      float p[4];
      // a query whose blocks are all masked or gated so far keeps m_run = -inf:
      // its exponents are then taken against 0 (p = 0, not NaN)
      const float msafe = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = __builtin_amdgcn_exp2f(x[rr] - msafe);
      const u32x2 pk = {pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])};
      l_run = sum_f16x2(pk[0], sum_f16x2(pk[1], l_run));
      const f16x4 pb = __builtin_bit_cast(f16x4, pk);
      const uint16_t* tv = tk + 2 * 16 * KP;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const u32x2 vf = *(const u32x2*)(tv + (16 * t + n16) * 16 + 4 * g4);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vf), pb, o[t], 0,
                                                     0, 0);
      }
    }
    if (jn < a.nB) lstore(tiles[cur ^ 1]);
    __syncthreads();
    cur ^= 1;
    j = jn;
    sp = sp_next;
  }
  if (!live) return;

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float lp = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  if (q >= a.N) return;
  // exact LSE merge with the sparse result of this row, in place
  float* lse = a.LSE + bh * a.N + q;
  const float ls = *lse;
  const float mm = fmaxf(ls, lp);
  float ws = 0.f, wp = 0.f, L = -INFINITY;
  if (mm != -INFINITY) {
    const float es = __expf(ls - mm), ep = __expf(lp - mm);  // exp(-inf) = 0
    const float sum = es + ep;
    L = mm + __logf(sum);
    ws = es / sum;
    wp = ep > 0.f ? ep / (sum * l_tot) : 0.f;  // l_tot > 0 whenever ep > 0
  }
  const int64_t orow = base + (int64_t)q * a.sn;
  // the sparse output row is read whole before any of it is used; it is
  // taken only when its weight is positive (otherwise it may be unwritten)
  f32x4 osv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) osv[t] = load4<OUT_BF16>(a.O, orow + 16 * t + 4 * g4);
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int64_t off = orow + 16 * t + 4 * g4;
    const f32x4 os = ws > 0.f ? osv[t] : f32x4{0.f, 0.f, 0.f, 0.f};
    store4<OUT_BF16>(a.O, off, ws * os[0] + wp * o[t][0], ws * os[1] + wp * o[t][1],
                     ws * os[2] + wp * o[t][2], ws * os[3] + wp * o[t][3]);
  }
  if (g4 == 0) *lse = L;
}

}  // namespace

hipError_t launch_rectify(const RectifyArgs& a, int BH, int D, bool out_bf16, hipStream_t s) {
  const int64_t total = (int64_t)BH * a.nBp * D;
  const dim3 cgrid((unsigned)((total + 255) / 256));
  if (D == 128)
    hipLaunchKernelGGL(rect_convert_kernel<128>, cgrid, dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL(rect_convert_kernel<64>, cgrid, dim3(256), 0, s, a, total);
  const dim3 grid(a.nB, BH);
  if (a.gate) {
    const dim3 sgrid(a.nBp, BH);
    if (D == 128) hipLaunchKernelGGL(rect_spread_kernel<128>, sgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(rect_spread_kernel<64>, sgrid, dim3(256), 0, s, a);
  }
  if (D == 128) {
    if (out_bf16) hipLaunchKernelGGL((rectify_kernel<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rectify_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((rectify_kernel<64, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rectify_kernel<64, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
