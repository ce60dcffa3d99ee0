// HyMoR-Attn Micro residual: attention of each 16-row query sub-tile over
// its selected 16-key tiles (the tiles a peak-preserving micro selection
// kept inside the blocks the macro selection omitted), on the fp16 V^T
// chunks the attention workspace stages.  Its output is merged with the
// macro result by the exact LSE merge.
#include "attn_util.h"
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

// One wave per 16-row query sub-tile over its selected 16-key tiles,
// kMicroWaves sub-tiles per workgroup.  16x16x32 products for S^T = K Q^T
// (lane holds 4 keys of one query), 16x16x16 products for O^T = V^T P^T
// (fp16) whose P^T operand is exactly those 4 accumulator registers.  A
// tile's K rows (4 KB) and V^T chunk (4 KB) are copied straight from global
// memory into one of two LDS slots of the wave (no registers, no barrier:
// each wave owns its slots), so the copies of tiles e+1 and e+2 are in
// flight while tile e is read from its slot and computed.  The kernel waits
// on memory latency: two slots of 8 KB per wave leave room for ten waves
// per compute unit (20 tiles in flight); against
// one tile prefetched in registers (12 waves) that took the HunyuanVideo
// micro heads from 5.63 to 4.40 ms, bit-identical, while three slots per
// wave (6 waves) gave 5.12 ms and four (5 waves) 6.25 ms.  The V^T rows are
// placed in the slot so that rows r and r + 8 of a fragment read fall on
// different banks (bank conflicts 7.4e8 -> 2.5e8 cycles per launch, 4.33 ->
// 4.15-4.28 ms).
//
// Sub-tiles run in the order of `order`: sorted, per head, by the first key
// tile each one selects, and dealt to the XCDs in contiguous ranges, so that
// sub-tiles gathering the same tiles run together on one XCD and share them
// through its L2.  Each sub-tile is computed on its own, so the order changes
// no result.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMicroWaves) void micro_attn_kernel(MicroAttnArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int DC = D / 8;             // 16-byte pieces per K row
  constexpr int NI = D / 32;            // 1 KB copies per K tile (and per V^T chunk)
  constexpr int SLOT = 2 * kMicro * D;  // uint16 elements of one slot: K rows, then V^T chunk
  __shared__ __attribute__((aligned(1024))) uint16_t ring[kMicroWaves][2][SLOT];
  const int w = blockIdx.x;
  const int Lw = (w & 7) * a.per_xcd + (w >> 3);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = kMicroWaves * Lw + wave;
  if (Lw >= (a.slots + kMicroWaves - 1) / kMicroWaves || slot >= a.slots) return;
  const int sid = a.order[slot];
  const int sub = sid & 3;
  const int i = (sid >> 2) % a.nB;
  const int z = (sid >> 2) / a.nB;
  const int nh = a.heads.n;
  const int b = z / nh, h = a.heads.h[z % nh];
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t r = bh * a.nB + i;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int q0 = i * kBlock + sub * kMicro;
  if (q0 >= a.N) return;

  // This sub-tile's segment of the row (entries sorted by sub-tile, then tile).
  const int rb = a.row_ptr[r], re = a.row_ptr[r + 1];
  int lt = 0, le = 0;
  for (int e = rb + lane; e < re; e += 64) {
    const int es_sub = a.idx[e] & 3;
    lt += es_sub < sub;
    le += es_sub <= sub;
  }
  lt = wave_sum(lt);
  le = wave_sum(le);
  const int es = __builtin_amdgcn_readfirstlane(rb + lt);
  const int ee = __builtin_amdgcn_readfirstlane(rb + le);

  const int64_t base = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* Qh = a.Q + base;
  const uint16_t* Kh = a.K + base;
  const uint16_t* Vth = a.Vt + bh * D * a.Npad;
  const int q = q0 + n16;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < a.N) v = *(const u32x4*)(Qh + (int64_t)q * a.sn + 32 * s + 8 * g4);
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }
  f32x4 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  // The Q fragments must have arrived before the copies start: the loop's
  // explicit waits count the copies only.
  wait_vmcnt<0>();

  // Tile copies straight into this wave's two LDS slots.  K: copy u, lane l
  // fills LDS byte 1024 u + 16 l = row (that / 2D), 16-byte position p of
  // the row, with global piece p ^ (row % DC) (rows XOR-swizzled, so the 16
  // rows a fragment read touches fall on distinct banks); rows past N read
  // row N-1 (their scores are masked).  V^T: the 16-key chunk is contiguous
  // and lands as it is.
  const int lastrow = a.N - 1 - (a.nT - 1) * kMicro;
  uint32_t koff[NI], kroff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int byte = 1024 * u + 16 * lane;
    const int row = byte / (2 * D), pc = (byte % (2 * D)) / 16;
    const int gp = pc ^ (row % DC);
    koff[u] = (uint32_t)(((int64_t)row * a.sn + gp * 8) * 2);
    kroff[u] = (uint32_t)(((int64_t)min(row, lastrow) * a.sn + gp * 8) * 2);
  }
  // V^T: LDS piece p (16 bytes) holds row p / 2, global half (p % 2) ^
  // ((row / 8) % 2): rows r and r + 8 of a fragment read then fall on
  // different banks
  uint32_t voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int pc = 64 * u + lane, row = pc >> 1;
    voff[u] = (uint32_t)(row * 32 + 16 * ((pc & 1) ^ ((row >> 3) & 1)));
  }
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring[wave][0][0]));
  const_i32* idx = (const_i32*)a.idx;
  // tile index and validity of an entry: an index outside [0, nT) reads
  // tile 0 and is masked out
  auto tile_of = [&](int e, bool& bad) {
    const int raw = idx[e] >> 2;
    bad = (unsigned)raw >= (unsigned)a.nT;
    return bad ? 0 : raw;
  };
  auto issue = [&](int e, int sl) {
    bool bad;
    const int beta = tile_of(e, bad);
    const uint32_t kb = ring0 + sl * (SLOT * 2);
    const uint32_t vb = kb + kMicro * D * 2;
    // every lane holds the same sub-tile, so the tile's addresses are uniform
    const uint16_t* ksrc = uniform_ptr(Kh + (int64_t)beta * kMicro * a.sn);
    const uint16_t* vsrc = uniform_ptr(Vth + (int64_t)beta * D * kMicro);
    const bool rag = beta == a.nT - 1;
    static_for<0, NI>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      dma16<u * 1024>(kb, ksrc, rag ? kroff[u] : koff[u]);
    });
    static_for<0, NI>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      dma16<u * 1024>(vb, vsrc, voff[u]);
    });
  };

  auto compute = [&](int e, int sl) {
    bool bad;
    const int beta = tile_of(e, bad);
    const uint16_t* ks = &ring[wave][sl][0];
    const uint16_t* vs = ks + kMicro * D;
    bf16x8 kf[KS];
    u32x2 vf[DT];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = *(const bf16x8*)(ks + n16 * D + (((4 * s + g4) ^ (n16 % DC)) * 8));
#pragma unroll
    // keys 4*g4 .. 4*g4+3 sit at chunk position 8 (g4 % 2) + 4 (g4 / 2), in
    // the half that the row's placement chose
    for (int t = 0; t < DT; ++t)
      vf[t] = *(const u32x2*)(vs + (16 * t + n16) * kMicro + 8 * ((g4 & 1) ^ ((n16 >> 3) & 1)) +
                              4 * (g4 >> 1));
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    // lane holds keys beta*16 + 4*g4 + rr of query q
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (bad || beta * kMicro + 4 * g4 + rr >= a.N) sacc[rr] = -INFINITY;
    if (bad && lane == 0) atomicOr(a.status, kStatusBadIndex);
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    if (__any(m_new > m_run + 8.0f)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      m_run = m_new;
    }
    float p[4];
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;  // all masked so far: p = 0, not NaN
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) p[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rr], c, mneg));
    const u32x2 pk = {pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])};
    // the row sum adds the rounded fp16 values the product uses
    l_run = add_f16x2(pk[0], add_f16x2(pk[1], l_run));
    const f16x4 pb = __builtin_bit_cast(f16x4, pk);
#pragma unroll
    for (int t = 0; t < DT; ++t)
      o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vf[t]), pb, o[t], 0, 0, 0);
  };

  // Two tiles in flight: tile e+1 and e+2 are being copied while tile e is
  // computed.  A slot is refilled once this wave's reads of it returned.
  if (es < ee) issue(es, 0);
  if (es + 1 < ee) issue(es + 1, 1);
  for (int e = es; e < ee; ++e) {
    const int sl = (e - es) & 1;
    if (e + 1 < ee) wait_vmcnt<2 * NI>();  // tile e has landed (e+1 may not)
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");         // the slot's reads stay behind the wait
    compute(e, sl);
    if (e + 2 < ee) {
      wait_lgkm0();                        // this wave's reads of the slot returned
      issue(e + 2, sl);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  if (q < a.N) {
    const int64_t orow = base + (int64_t)q * a.sn;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      store4<OUT_BF16>(a.O, orow + 16 * t + 4 * g4, o[t][0] * inv, o[t][1] * inv, o[t][2] * inv,
                       o[t][3] * inv);
    if (g4 == 0) a.LSE[bh * a.N + q] = lse;
  }
}

// Signature of every sub-tile: its global bin (z, first key tile selected),
// nT for an empty sub-tile; a row's entries are sorted by (sub-tile, key
// tile), so the first entry of sub-tile a is found by binary search.
__global__ __launch_bounds__(256) void micro_sig_kernel(MicroAttnArgs a) {
  const int sid = blockIdx.x * 256 + threadIdx.x;
  if (sid >= a.slots) return;
  const int sub = sid & 3;
  const int i = (sid >> 2) % a.nB;
  const int z = (sid >> 2) / a.nB;
  const int nh = a.heads.n;
  const int b = z / nh, h = a.heads.h[z % nh];
  const int64_t r = ((int64_t)b * a.H + h) * a.nB + i;
  int lo = a.row_ptr[r], hi = a.row_ptr[r + 1];
  const int end = hi;
  while (lo < hi) {  // first entry whose sub-tile is >= sub
    const int mid = (lo + hi) >> 1;
    if ((a.idx[mid] & 3) < sub) lo = mid + 1;
    else hi = mid;
  }
  // (a tile index outside [0, nT) sorts with the empty sub-tiles)
  int first = (lo < end && (a.idx[lo] & 3) == sub) ? (a.idx[lo] >> 2) : a.nT;
  if ((unsigned)first > (unsigned)a.nT) first = a.nT;
  const int bin = z * (a.nT + 1) + first;
  a.sig[sid] = bin;
  atomicAdd(&a.hist[bin], 1);
}

// Place every sub-tile at its bin's next position (any order inside a bin).
__global__ __launch_bounds__(256) void micro_scatter_kernel(MicroAttnArgs a) {
  const int sid = blockIdx.x * 256 + threadIdx.x;
  if (sid >= a.slots) return;
  const int pos = atomicAdd(&a.offsets[a.sig[sid]], 1);
  a.order[pos] = sid;
}


hipError_t launch_micro_attn(const MicroAttnArgs& a, int B, int D, bool out_bf16, hipStream_t s) {
  (void)B;
  hipError_t e = launch_fill_i32(a.hist, a.bins, 0, s);
  if (e != hipSuccess) return e;
  const dim3 sgrid((a.slots + 255) / 256);
  hipLaunchKernelGGL(micro_sig_kernel, sgrid, dim3(256), 0, s, a);
  e = launch_scan(a.hist, a.bins, a.offsets, a.nnz, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(micro_scatter_kernel, sgrid, dim3(256), 0, s, a);
  dim3 grid(8 * a.per_xcd);
  if (D == 128) {
    if (out_bf16) hipLaunchKernelGGL((micro_attn_kernel<128, true>), grid, dim3(64 * kMicroWaves), 0, s, a);
    else hipLaunchKernelGGL((micro_attn_kernel<128, false>), grid, dim3(64 * kMicroWaves), 0, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((micro_attn_kernel<64, true>), grid, dim3(64 * kMicroWaves), 0, s, a);
    else hipLaunchKernelGGL((micro_attn_kernel<64, false>), grid, dim3(64 * kMicroWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
