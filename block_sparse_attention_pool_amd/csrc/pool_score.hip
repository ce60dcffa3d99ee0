// Block pooling and pooled block scores (Rectified SpaAttn: pooled query-key
// interactions; HyperVAttention section 2, Eq. 2 left, centroids = member
// means).  Pooling is HBM bound and runs on the vector ALUs in float32.  The
// scores feed an exact selection, so they are computed at float32 grade: the
// product runs on the bf16 matrix cores with every float32 operand split into
// three bf16 parts (score_gemm_kernel below).
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

// One workgroup per (BLK-token block i, head h, batch b, tensor Q|K), BLK =
// 64 or 128 (the 128-token blocks of MOD-DiT's block-wise attention).
// 256 threads: thread = (16-byte chunk c of a row, token group g).  Each
// group sums a run of consecutive tokens; groups are then combined into the
// BLK/16 16-token tile sums and the block sum.  Only valid tokens
// (index < N) contribute and the divisor is the valid count.
template <int D, int BLK>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int C = D / 8;        // 16-byte chunks per token row
  constexpr int G = 256 / C;      // token groups
  constexpr int TPG = BLK / G;    // tokens per group
  constexpr int GPT = 16 / TPG;   // groups per 16-token tile
  constexpr int NT = BLK / kMicro;  // 16-token tiles per block
  static_assert(GPT >= 1 && GPT * TPG == 16, "a token group never straddles two tiles");
  __shared__ float part[G][D + 4];
  __shared__ float tile[NT][D];

  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool isK = blockIdx.z & 1;
  const uint16_t* X = (isK ? a.K : a.Q) + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int g = tid / C;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // All of the group's rows are loaded before any is added (clamped to the
  // last token, so every address is in bounds); rows past N add nothing.
  u32x4 v[TPG];
#pragma unroll
  for (int t = 0; t < TPG; ++t) {
    const int tok = min(i * BLK + g * TPG + t, a.N - 1);
    v[t] = *(const u32x4*)(X + (int64_t)tok * a.sn + c * 8);
  }
#pragma unroll
  for (int t = 0; t < TPG; ++t) {
    if (i * BLK + g * TPG + t < a.N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_bits_to_f32(v[t][e] & 0xFFFFu);
        acc[2 * e + 1] += bf16_bits_to_f32(v[t][e] >> 16);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][c * 8 + e] = acc[e];
  __syncthreads();

  const int64_t bh = (int64_t)b * a.H + h;
  float* pool16 = isK ? a.kpool16 : a.qpool16;
  for (int idx = tid; idx < NT * D; idx += 256) {
    const int t = idx / D, e = idx % D;
    float s = 0.f;
#pragma unroll
    for (int gg = 0; gg < GPT; ++gg) s += part[t * GPT + gg][e];
    tile[t][e] = s;
    const int t0 = i * BLK + t * kMicro;
    const int cnt = min(kMicro, a.N - t0);
    if (pool16 != nullptr && cnt > 0)
      pool16[(bh * a.nT + NT * i + t) * D + e] = s / (float)cnt;
  }
  __syncthreads();
  float* pool = isK ? a.kpool : a.qpool;
  const int cnt = min(BLK, a.N - i * BLK);
  for (int e = tid; e < D; e += 256) {
    float s = (tile[0][e] + tile[1][e]) + (tile[2][e] + tile[3][e]);
    if constexpr (NT == 8) s += (tile[4][e] + tile[5][e]) + (tile[6][e] + tile[7][e]);
    pool[(bh * a.nB + i) * D + e] = s / (float)cnt;
  }
}

// Batched C = scale * A B^T with A [M, D], B [Nc, D] float32 per batch, on
// the bf16 matrix cores at float32 grade: every element is split exactly into
// bf16 parts hi + mid + lo (hi = bf16(x), mid = bf16(x - hi), lo = bf16(x -
// hi - mid), each difference exact in float32), and of the nine part products
// the six down to relative order 2^-16 are summed (lo*hi, mid*mid, hi*lo,
// mid*hi, hi*mid, hi*hi, smallest first) with float32 accumulation; the
// dropped ones are below 2^-23 of the hi*hi term.  64x64 output tile per
// workgroup, 4 waves of 32x32 (v_mfma_f32_32x32x16_bf16); the shared
// dimension in chunks of 32, split while staged into LDS, the next chunk
// loaded into registers while the current one is multiplied.  Batch z maps to
// the (b, h) pair through the head list so the same kernel serves the pooled
// block scores (all heads) and the micro tile scores (selected heads).
__global__ __launch_bounds__(256) void score_gemm_kernel(GemmArgs a) {
  constexpr int TK = 32, KP = TK + 8;  // chunk, padded LDS row (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t As[3][64][KP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][64][KP];

  const int z = blockIdx.z;
  const int b = z / a.heads.n;
  const int h = a.heads.h[z % a.heads.n];
  const int64_t src = (int64_t)b * a.H + h;
  const float* A = a.A + src * a.M * a.D;
  const float* Bm = a.Bm + src * a.Nc * a.D;
  float* Cm = a.C + (int64_t)z * a.M * a.Nc;

  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;  // this wave's quarter
  const int l32 = lane & 31, kh = lane >> 5;
  // staging: 64 rows x 32 floats per operand = 512 float4, 2 per thread each;
  // rows past M or Nc read the last row and are zeroed when staged
  f32x4 ra[2], rb[2];
  const float* pa[2];
  const float* pb[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int f = tid + 256 * it, row = f >> 3, c4 = (f & 7) * 4;
    pa[it] = A + (int64_t)min(m0 + row, a.M - 1) * a.D + c4;
    pb[it] = Bm + (int64_t)min(n0 + row, a.Nc - 1) * a.D + c4;
  }
  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      ra[it] = *(const f32x4*)(pa[it] + k0);
      rb[it] = *(const f32x4*)(pb[it] + k0);
    }
  };
  // element pairs: one packed round-to-nearest-even conversion per part
  auto split_store = [&](uint16_t(*dst)[64][KP], int row, int c4, f32x4 v, bool valid) {
    uint32_t w[3][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x0 = valid ? v[2 * e] : 0.f, x1 = valid ? v[2 * e + 1] : 0.f;
      const uint32_t hi = pack_bf16x2(x0, x1);
      const float r0 = x0 - __uint_as_float(hi << 16);
      const float r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
      const uint32_t mid = pack_bf16x2(r0, r1);
      const float s0 = r0 - __uint_as_float(mid << 16);
      const float s1 = r1 - __uint_as_float(mid & 0xFFFF0000u);
      w[0][e] = hi;
      w[1][e] = mid;
      w[2][e] = pack_bf16x2(s0, s1);
    }
#pragma unroll
    for (int part = 0; part < 3; ++part)
      *(u32x2*)&dst[part][row][c4] = u32x2{w[part][0], w[part][1]};
  };
  auto lstore = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int f = tid + 256 * it, row = f >> 3, c4 = (f & 7) * 4;
      split_store(As, row, c4, ra[it], m0 + row < a.M);
      split_store(Bs, row, c4, rb[it], n0 + row < a.Nc);
    }
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  gload(0);
  for (int k0 = 0; k0 < a.D; k0 += TK) {
    lstore();
    __syncthreads();
    if (k0 + TK < a.D) gload(k0 + TK);
#pragma unroll
    for (int s2 = 0; s2 < TK / 16; ++s2) {
      const int kc = 16 * s2 + 8 * kh;
      bf16x8 af[3], bf[3];
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        af[part] = *(const bf16x8*)&As[part][wm + l32][kc];
        bf[part] = *(const bf16x8*)&Bs[part][wn + l32][kc];
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[2], bf[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bf[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bf[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf[0], acc, 0, 0, 0);
    }
    __syncthreads();  // the chunk is no longer read
  }
  // lane holds rows 8 (r/4) + 4 kh + r%4 of column l32 of the quarter
  const int n = n0 + wn + l32;
  if (n < a.Nc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (m < a.M) Cm[(int64_t)m * a.Nc + n] = a.scale * acc[r];
    }
  }
}

hipError_t launch_pool(const PoolArgs& a, int B, hipStream_t s) {
  dim3 grid(a.nB, a.H, 2 * B);
  if (a.block == 128) {
    if (a.D == 128)
      hipLaunchKernelGGL((pool_kernel<128, 128>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((pool_kernel<64, 128>), grid, dim3(256), 0, s, a);
  } else {
    if (a.D == 128)
      hipLaunchKernelGGL((pool_kernel<128, 64>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((pool_kernel<64, 64>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_score_gemm(const GemmArgs& a, int nbatch, hipStream_t s) {
  dim3 grid((a.Nc + 63) / 64, (a.M + 63) / 64, nbatch);
  hipLaunchKernelGGL(score_gemm_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
