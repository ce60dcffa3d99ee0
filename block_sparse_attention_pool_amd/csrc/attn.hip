// Attention kernels for gfx950.
//
//  * transpose_v: V [N, d] bf16 -> key-major fp16 V^T per head, zero
//    padded, stored as [64-key block][16-key chunk][d][16]: one 16-key tile
//    (the micro tile) is 4 KB contiguous and a 64-key tile 16 KB.  Inside
//    each chunk the keys are in the order the matrix-core operand layout
//    consumes them, so every PV operand is one contiguous load.  The PV
//    product runs on fp16 operands: bf16 V converts to fp16 exactly (within
//    fp16 range) and P, bounded by 2^8 through the lazy rescale, keeps 3
//    more mantissa bits than bf16 would give it.
//  * attn_fwd: block-sparse (CSR rows) or dense flash attention forward.
//    HyperVAttention section 2, Eq. 4 (attention restricted to the selected
//    key blocks; identity permutation) and the HyMoR-Attn Macro backbone.
//  * merge: HyMoR-Attn exact LSE merging.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, wave64).  A wave owns
// 32 query rows.  It computes S^T = K Q^T (m = key, n = query, k = d) so that
// each lane holds 32 scores of ONE query (its column): the row max and sum of
// the online softmax are in-lane plus a single exchange with lane^32, and
// the rescale of the output is one scalar per lane.  The PV product is
// O^T = V^T P^T (m = d, n = query, k = key); the S^T accumulator registers
// of a lane are exactly its P^T operand for a 16-key chunk once the keys of
// the chunk are permuted consistently on the V^T side (done by transpose_v).
#include <type_traits>

#include "attn_util.h"
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

// ---------------------------------------------------------------- V^T

template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(TransposeArgs a) {
  constexpr int C = D / 8;
  __shared__ uint32_t tile[64][D / 2 + 1];  // bf16 pairs; +1 word breaks bank aliasing

  const int j = blockIdx.x;
  const int h = a.heads.h[blockIdx.y];
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const uint16_t* V = a.V + (int64_t)b * a.sb + (int64_t)h * a.sh;
  uint16_t* Vt = a.Vt + ((int64_t)b * a.H + h) * D * a.Npad;

  // every row load is issued before any is stored (rows past N read the
  // last row, then zeros are stored)
  constexpr int PER = 64 * C / 256;
  u32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int f = tid + 256 * u;
    v[u] = *(const u32x4*)(V + (int64_t)min(j * kBlock + f / C, a.N - 1) * a.sn + (f % C) * 8);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int f = tid + 256 * u, row = f / C, c = f % C;
    if (j * kBlock + row >= a.N) v[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[row][c * 4 + e] = v[u][e];
  }
  __syncthreads();
  const uint16_t* t16 = (const uint16_t*)&tile[0][0];
  constexpr int RS = D + 2;  // row stride of the tile in bf16 elements
  for (int f = tid; f < D * 8; f += 256) {
    const int d = f >> 3, u = f & 7;  // 8 output keys at positions 8u..8u+7
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * u + 2 * e;
      const int k0 = 16 * (p0 >> 4) + vt_key_of_pos(p0 & 15);
      const int k1 = 16 * ((p0 + 1) >> 4) + vt_key_of_pos((p0 + 1) & 15);
      w[e] = bf16_bits_to_f16_bits(t16[k0 * RS + d]) |
             (bf16_bits_to_f16_bits(t16[k1 * RS + d]) << 16);
    }
    const u32x4 out = {w[0], w[1], w[2], w[3]};
    // chunk u/2 of block j, row d, positions 8 (u%2) .. +7
    *(u32x4*)(Vt + ((int64_t)(4 * j + (u >> 1)) * D + d) * kMicro + 8 * (u & 1)) = out;
  }
}

// ---------------------------------------------------------- attention

// Per-lane byte offsets of the tile copies of one wave (loop invariant).
// K tile (64 x D bf16): instruction t covers rows t*RPI .. t*RPI+RPI-1; lane
// l of it lands at LDS row t*RPI + l/DC, 16-byte position l%DC, so it fetches
// global chunk (l%DC) ^ (row%DC) -- the row-XOR swizzle (a 128-bit LDS read
// is served 16 lanes at a time by 64 four-byte banks; K rows are 256 bytes,
// so r%16 separates 16 consecutive rows).  V^T tile: kept in LDS as it is
// in global memory, chunk-major [4][D][16] fp16 (32-byte rows), so every
// copy instruction reads 1 KB of contiguous global memory; the two 16-byte
// halves of a row are swapped when (row/8) is odd, which puts the 16 rows a
// PV operand read touches at once on distinct banks.  Wave w issues
// instructions t = w, w+2, ...: 1 KB of LDS each, 2 KB apart.
template <int D>
struct TileCopy {
  static constexpr int DC = D / 8;
  static constexpr int RPI = 64 / DC;
  static constexpr int NK = (64 / RPI) / 2;  // K instructions per wave
  static constexpr int NVI = (D / 8) / 2;    // V instructions per wave
  uint32_t koff[NK];
  uint32_t voff[NVI];
  uint32_t kbase, vbase;  // LDS byte address of this wave's first instruction

  uint32_t kr[NK];  // the same for the last key block, rows clamped to N-1
  __device__ __forceinline__ void init(int64_t sn, int wave, int lane,
                                       const uint16_t* sK, const uint16_t* sV, int N, int nB) {
    const int last = N - 1 - (nB - 1) * kBlock;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int t = wave + 2 * u;
      const int r = t * RPI + lane / DC;
      const int c = (lane % DC) ^ (r % DC);
      kr[u] = (uint32_t)((min(r, last) * sn + c * 8) * 2);
    }
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int t = wave + 2 * u;
      const int r = t * RPI + lane / DC;
      const int c = (lane % DC) ^ (r % DC);
      koff[u] = (uint32_t)((r * sn + c * 8) * 2);
    }
#pragma unroll
    for (int u = 0; u < NVI; ++u) {
      // LDS byte p = 1024 t + 16 lane of the chunk-major tile [4][D][16]:
      // chunk p / (32 D), row (p / 32) % D, half (p / 16) % 2, which holds
      // the global half h ^ ((row / 8) % 2) of the same chunk and row
      const int t = wave + 2 * u;
      const int pb = 1024 * t + 16 * lane;
      const int ch = pb / (32 * D), r = (pb / 32) % D, hf = (pb / 16) & 1;
      voff[u] = (uint32_t)((ch * D + r) * 32 + 16 * (hf ^ ((r >> 3) & 1)));
    }
    kbase = __builtin_amdgcn_readfirstlane(lds_addr(sK) + wave * 1024);
    vbase = __builtin_amdgcn_readfirstlane(lds_addr(sV) + wave * 1024);
  }

  // K rows past N (ragged last block) are clamped to row N-1; their scores
  // are masked to -inf, so only in-bounds reads matter.  The choice between
  // the two offset sets is a select, not a branch.
  __device__ __forceinline__ void k_tile(const uint16_t* Kh, int64_t sn, int j, int nB) const {
    const uint16_t* base = Kh + (int64_t)j * kBlock * sn;
    const bool rag = j == nB - 1;
    static_for<0, NK>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      dma16<u * 2048>(kbase, base, rag ? kr[u] : koff[u]);
    });
  }

  __device__ __forceinline__ void v_tile(const uint16_t* Vth, int j) const {
    const uint16_t* base = Vth + (int64_t)j * kBlock * D;
    static_for<0, NVI>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      dma16<u * 2048>(vbase, base, voff[u]);
    });
  }

  // Tiles gathered from four 16-key chunks (entries: chunk index in the low
  // 24 bits).  Instruction u of either wave covers rows of chunk 64 u / D
  // only, so its base moves to that chunk and the per-lane offsets stay the
  // ones of a contiguous tile.
  __device__ __forceinline__ void k_chunks(const uint16_t* Kh, int64_t sn, const_i32* ent) const {
    static_for<0, NK>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int cc = 64 * u / D;
      const int64_t ch = ent[cc] & kChunkMask;
      dma16<u * 2048>(kbase, Kh + (ch - cc) * 16 * sn, koff[u]);
    });
  }

  __device__ __forceinline__ void v_chunks(const uint16_t* Vth, const_i32* ent) const {
    static_for<0, NVI>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int cc = 64 * u / D;
      const int64_t ch = ent[cc] & kChunkMask;
      dma16<u * 2048>(vbase, Vth + (ch - cc) * 16 * D, voff[u]);
    });
  }
};

// max(a, b, c) in one instruction.  (fmaxf on matrix-core results compiles
// to an extra quieting max per operand.)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max(x[l], x[l ^ 32]): lanes l and l^32 exchange through one permlane swap.
__device__ __forceinline__ float pair_max32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Workgroup execution barrier without the memory fence __syncthreads()
// implies (that fence would also drain the asynchronous tile copies).  Every
// call is preceded by the explicit waits that make the LDS contents it
// publishes complete; the memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void exec_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The sparse kernel interleaves its rows across the XCDs when they average
// more key-tile bytes than twice the 4 MB L2 of one XCD and their runs of
// consecutive blocks average fewer than kShortRun blocks.
constexpr int64_t kWideRowBytes = int64_t(8) << 20;
constexpr int kShortRun = 8;

// One workgroup per (b, h, 64-row query block), two waves of 32 rows each.
// Per selected key block the 64 x D K tile (16-byte chunks XOR-swizzled by
// row) and the chunk-major V^T tile sit in LDS.  The K buffer is refilled with
// the next block as soon as both waves have finished QK^T, the V buffer as
// soon as they have finished PV, so each copy overlaps the other half of
// the iteration without a second buffer.  32 KB of LDS and at most 256
// registers per lane leave room for four workgroups (two waves per SIMD)
// per compute unit.
// CHUNK: rows are query tiles of groups; query tile L belongs to group
// a.tile_group[L] (-1: no work) whose entries row_ptr[bh * ngroups + g] ..
// are 16-key chunk codes (chunk | valid keys << 24), four per key tile; the
// keys of a chunk past its valid count are masked.  Used for packed
// cluster-induced blocks: K and the staged V^T hold whole chunks (so no load
// is clamped); query position q of a head is token a.qsrc[bh * N + q] of the
// caller's Q (-1: padding), whose O row and LSE (of a.Nout tokens) it writes.
template <int D, bool DENSE, bool OUT_BF16, bool CHUNK = false>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(AttnArgs a) {
  constexpr int DC = D / 8;      // 16-byte chunks per K row
  constexpr int KS = D / 16;     // k-steps of the QK^T product
  constexpr int DT = D / 32;     // 32-row d tiles of the PV product
  __shared__ __attribute__((aligned(1024))) uint16_t sK[64 * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[D * 64];

  // XCD-aware row order: dispatch w runs on XCD w % 8.  By default each XCD
  // takes a contiguous range of (head, query block) rows, so its L2 sees one
  // head's neighbouring query blocks, whose key selections overlap.  When
  // the rows' key supports average more than twice an XCD's 4 MB L2 and are
  // scattered (made of short runs of consecutive blocks), neighbouring rows
  // share little and that reuse is lost; the rows are then dealt to the XCDs
  // in interleaved chunks of 8, so that all XCDs work on neighbouring rows of
  // one head at a time and share its tiles through the Infinity Cache instead
  // of streaming eight heads' keys from HBM.  The choice reads the total
  // entry count and one sample row (the middle query block of the first
  // head, the same for every workgroup), so it needs no host round trip.
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  bool interleave = CHUNK;  // long rows of scattered short runs
  if constexpr (!DENSE && !CHUNK) {
    const_i32* rp = (const_i32*)a.row_ptr;
    const int64_t total = rp[a.rows];
    if (total * (kBlock * D * 2 * 2) > (int64_t)a.rows * kWideRowBytes) {
      __shared__ int run_starts[2];
      const int rs = a.nB / 2;
      const int sb = rp[rs], se = rp[rs + 1];
      int starts = 0;
      for (int e = sb + (int)threadIdx.x; e < se; e += 128)
        starts += (e == sb || a.col_idx[e] != a.col_idx[e - 1] + 1) ? 1 : 0;
      starts = wave_sum(starts);
      if ((threadIdx.x & 63) == 0) run_starts[threadIdx.x >> 6] = starts;
      __syncthreads();
      starts = run_starts[0] + run_starts[1];
      interleave = starts * kShortRun > se - sb;  // mean run shorter than kShortRun blocks
    }
  }
  int L;
  if (interleave) {
    L = ((slot >> 3) * 8 + xcd) * 8 + (slot & 7);
  } else {
    if (slot >= a.per_xcd) return;
    L = xcd * a.per_xcd + slot;
  }
  if (L >= a.rows) return;
  const int i = L % a.nB;
  const int bh = L / a.nB;
  const int b = bh / a.H, h = bh % a.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int64_t base = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* Qh = a.Q + base;
  // CHUNK: K lives in the padded chunk layout (its own strides); Q and O
  // keep the caller's layout, rows found through the query source map
  const uint16_t* Kh = a.K + (CHUNK ? (int64_t)b * a.ksb + (int64_t)h * a.ksh : base);
  const int64_t ksn = CHUNK ? a.ksn : a.sn;
  const uint16_t* Vth = a.Vt + (int64_t)bh * D * a.Npad;

  // Row pointers and column indices are read-only for the kernel's
  // lifetime: scalar loads (counted apart from the tile copies).
  const_i32* row_ptr = (const_i32*)a.row_ptr;
  const_i32* col_idx = (const_i32*)a.col_idx;
  int e0, e1;
  if constexpr (DENSE) {
    e0 = 0;
    e1 = a.nB;
  } else if constexpr (CHUNK) {
    const int gi = a.tile_group[L];
    e0 = gi < 0 ? 0 : row_ptr[(int64_t)bh * a.ngroups + gi];
    e1 = gi < 0 ? 0 : row_ptr[(int64_t)bh * a.ngroups + gi + 1];
  } else {
    e0 = row_ptr[L];
    e1 = row_ptr[L + 1];
  }

  const int q = i * kBlock + wave * 32 + n;
  // the row this lane's query is read from and written to
  int64_t qrow = q;
  bool has_q = q < a.N;
  if constexpr (CHUNK) {
    qrow = has_q ? a.qsrc[(int64_t)bh * a.N + q] : -1;
    has_q = qrow >= 0;
  }
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (has_q) v = *(const u32x4*)(Qh + qrow * a.sn + 16 * s + 8 * g);
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  // The Q fragments must have arrived before the loop: otherwise the
  // compiler places that wait inside the loop, where it would also drain
  // the tile copies in flight.
  wait_vmcnt<0>();
  TileCopy<D> cp;
  cp.init(ksn, wave, lane, sK, sV, a.N, a.nB);

  // O^T += V^T P^T for one key block whose V^T tile is in sV.
  // The V^T fragments of d tile t+1 are read while the products of tile t run.
  auto v_frags = [&](int t, f16x8(&va)[4]) {
    const int row = 32 * t + n;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      va[cc] = *(const f16x8*)(sV + (cc * D + row) * 16 + ((g ^ ((row >> 3) & 1)) * 8));
  };
  auto pv = [&](const f16x8(&pf)[4], const f16x8(&va0)[4]) {
    f16x8 va[2][4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) va[0][cc] = va0[cc];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      if (t + 1 < DT) v_frags(t + 1, va[(t + 1) & 1]);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[t & 1][cc], pf[cc], o[t], 0, 0, 0);
    }
  };

  // exp2 of the scaled scores against the running max, packed to fp16 (the
  // PV operand); the row sum adds exactly those rounded values (a dot with
  // (1, 1) in fp32), so numerator and normaliser agree.
  // While every key seen so far is masked (m_run = -inf) the exponent is
  // taken against 0, so masked scores give exp2(-inf) = 0, not NaN.
  auto softmax_pack = [&](f32x16& s0, f32x16& s1, f16x8(&pf)[4]) {
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, mneg));
      s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, mneg));
    }
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const f32x16& src = (cc < 2) ? s0 : s1;
      const int r0 = 8 * (cc & 1);
      const u32x4 pk = {pack_f16x2(src[r0 + 0], src[r0 + 1]), pack_f16x2(src[r0 + 2], src[r0 + 3]),
                        pack_f16x2(src[r0 + 4], src[r0 + 5]), pack_f16x2(src[r0 + 6], src[r0 + 7])};
      ps0 = add_f16x2(pk[0], add_f16x2(pk[1], ps0));
      ps1 = add_f16x2(pk[2], add_f16x2(pk[3], ps1));
      pf[cc] = __builtin_bit_cast(f16x8, pk);
    }
    l_run += ps0 + ps1;
  };

  // Software pipeline over the row's key blocks, two barriers per block.
  // Iteration e:
  //   A  K(e) has landed and every wave is done with sV  -> copy V(e-1)
  //      QK^T(e) from sK
  //   B  V(e-1) has landed and every wave is done with sK -> copy K(e+1)
  //      softmax(e) interleaved with the PV products of block e-1 (sV)
  // The first iteration runs its PV step on a zero P against V(e0) (a real,
  // finite tile), which adds exact zeros and keeps the loop body free of
  // branches between the softmax and the PV products.
  f16x8 pf_prev[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) pf_prev[cc] = f16x8{};
  // j: the key block (CHUNK: the position of its first chunk entry).  A
  // caller's column index outside [0, nB) becomes -1: its tiles are read
  // from block 0 (in bounds), its scores are masked out and the status word
  // records it, so such an entry adds nothing instead of reading outside K
  // and V^T.
  constexpr int STEP = CHUNK ? 4 : 1;
  auto key_block = [&](int e) {
    if constexpr (DENSE || CHUNK) {
      return e;
    } else {
      const int jr = col_idx[e];
      return (unsigned)jr < (unsigned)a.nB ? jr : -1;
    }
  };
  auto tile_of = [](int jj) { return jj < 0 ? 0 : jj; };
  int j = 0, jprev = 0;
  if (e0 < e1) {
    j = key_block(e0);
    jprev = j;
    if constexpr (CHUNK) cp.k_chunks(Kh, ksn, col_idx + j);
    else cp.k_tile(Kh, a.sn, tile_of(j), a.nB);
  }
  for (int e = e0; e < e1; e += STEP) {
    const int jn = (e + STEP < e1) ? key_block(e + STEP) : j;
    wait_lgkm0();      // this wave's reads of sV (block e-2) have returned
    wait_vmcnt<0>();   // this wave's copy of K(e) has landed
    exec_barrier();    // ... and the other wave's; sV is free
    if constexpr (CHUNK) cp.v_chunks(Vth, col_idx + jprev);
    else cp.v_tile(Vth, tile_of(jprev));

    // S^T for keys 0..31 (s0) and 32..63 (s1) of the block.
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int r0 = n, r1 = 32 + n;
      const bf16x8 k0 = *(const bf16x8*)(sK + r0 * D + (((2 * s + g) ^ (r0 % DC)) * 8));
      const bf16x8 k1 = *(const bf16x8*)(sK + r1 * D + (((2 * s + g) ^ (r1 % DC)) * 8));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], s1, 0, 0, 0);
    }
    // K fragments are read three k-steps ahead of their products.
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    static_for<0, KS - 3>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    __builtin_amdgcn_s_setprio(0);
    wait_lgkm0();      // this wave's reads of sK have returned
    wait_vmcnt<0>();   // V(e-1) has landed
    exec_barrier();    // both waves are done with sK; sV holds V(e-1)
    if (e + STEP < e1) {
      if constexpr (CHUNK) cp.k_chunks(Kh, ksn, col_idx + jn);
      else cp.k_tile(Kh, a.sn, tile_of(jn), a.nB);
    }

    f16x8 va0[4];  // V^T fragments of block e-1's first d tile, read early
    v_frags(0, va0);
    // Lane holds keys 8*(r/4) + 4*g + r%4 (+32 for s1) of query q.
    if constexpr (CHUNK) {
      // key 8*(r/4) + 4*g + r%4 of s0 lies in chunk r/8 at offset
      // 8*((r/4)%2) + 4*g + r%4; s1 is chunks 2 and 3
      int vc[4];
      bool partial = false;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        vc[cc] = (int)((uint32_t)col_idx[j + cc] >> kChunkShift);
        partial |= vc[cc] < 16;
      }
      if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * ((r >> 2) & 1) + 4 * g + (r & 3);
          if (off >= vc[r >> 3]) s0[r] = -INFINITY;
          if (off >= vc[2 + (r >> 3)]) s1[r] = -INFINITY;
        }
      }
    } else if (!DENSE && j < 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = -INFINITY;
        s1[r] = -INFINITY;
      }
      if (threadIdx.x == 0) atomicOr(a.status, kStatusBadIndex);
    } else if (j == a.nB - 1) {
      const int nvalid = a.N - j * kBlock;
      if (nvalid < kBlock) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * g + (r & 3);
          if (kk >= nvalid) s0[r] = -INFINITY;
          if (kk + 32 >= nvalid) s1[r] = -INFINITY;
        }
      }
    }
    // Row max over the lane's 32 scores (a tree of 3-input maxima), then
    // over the lane pair (l, l^32) that holds the other 32 keys.
    float m11[11];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      m11[k] = max3f(s0[3 * k], s0[3 * k + 1], s0[3 * k + 2]);
      m11[5 + k] = max3f(s1[3 * k], s1[3 * k + 1], s1[3 * k + 2]);
    }
    m11[10] = max3f(s0[15], s1[15], m11[0]);
    const float m3a = max3f(m11[1], m11[2], m11[3]);
    const float m3b = max3f(m11[4], m11[5], m11[6]);
    const float m3c = max3f(m11[7], m11[8], m11[9]);
    float mx = max3f(m3a, m3b, max3f(m3c, m11[10], m3c));
    mx = pair_max32(mx);
    const float m_new = fmaxf(m_run, mx * c);
    f16x8 pf[4];
    // Lazy rescale: keep a stale running max while the new one exceeds it
    // by at most 8 (in log2 units); probabilities then stay below 2^8, which
    // fp32 sums and fp16 operands hold.  The result is the same softmax
    // because the final normaliser uses the same max.
    if (__any(m_new > m_run + 8.0f)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      // block e-1 is not yet in O: bring its packed P to the new scale too
      const _Float16 ah = (_Float16)alpha;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) pf_prev[cc] *= ah;
      m_run = m_new;
    }
    // The vector work of block e and the (independent) PV products of block
    // e-1 share one basic block, so the compiler interleaves them.
    softmax_pack(s0, s1, pf);
    pv(pf_prev, va0);

#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pf_prev[cc] = pf[cc];
    jprev = j;
    j = jn;
  }
  if (e0 < e1) {
    wait_lgkm0();
    exec_barrier();    // every wave is done with sV
    if constexpr (CHUNK) cp.v_chunks(Vth, col_idx + jprev);
    else cp.v_tile(Vth, tile_of(jprev));
    wait_vmcnt<0>();
    exec_barrier();
    f16x8 va0[4];
    v_frags(0, va0);
    pv(pf_prev, va0);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  if (has_q) {
    const int64_t orow = base + qrow * a.sn;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * t + 8 * rr + 4 * g;
        store4<OUT_BF16>(a.O, orow + d0, o[t][4 * rr] * inv, o[t][4 * rr + 1] * inv,
                         o[t][4 * rr + 2] * inv, o[t][4 * rr + 3] * inv);
      }
    if (g == 0) a.LSE[(int64_t)bh * (CHUNK ? a.Nout : a.N) + qrow] = lse;
  }
}

// ---------------------------------------------------------------- merge

// Each row is handled by D/8 consecutive lanes of one wave, 8 elements per
// lane; every lane loads L1/L2 before any lane stores, so O/L may alias
// O1/L1.
template <bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int h = a.heads.h[blockIdx.y];
  const int b = blockIdx.z;
  const int C = a.D / 8;
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t q = f / C;
  const int cidx = (int)(f % C);
  if (q >= a.N) return;
  const int64_t lrow = ((int64_t)b * a.H + h) * a.N + q;
  const float l1 = a.L1[lrow], l2 = a.L2[lrow];
  const float mx = fmaxf(l1, l2);
  float Lm, w1, w2;
  if (mx == -INFINITY) {
    Lm = -INFINITY;
    w1 = 0.f;
    w2 = 0.f;
  } else {
    Lm = mx + logf(expf(l1 - mx) + expf(l2 - mx));
    w1 = expf(l1 - Lm);
    w2 = expf(l2 - Lm);
  }
  const int64_t off = (int64_t)b * a.sb + (int64_t)h * a.sh + q * a.sn + cidx * 8;
  if constexpr (BF16) {
    const u32x4 x = *(const u32x4*)((const uint16_t*)a.O1 + off);
    const u32x4 y = *(const u32x4*)((const uint16_t*)a.O2 + off);
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = w1 * bf16_bits_to_f32(x[e] & 0xFFFFu) + w2 * bf16_bits_to_f32(y[e] & 0xFFFFu);
      const float hi = w1 * bf16_bits_to_f32(x[e] >> 16) + w2 * bf16_bits_to_f32(y[e] >> 16);
      out[e] = pack_bf16x2(lo, hi);
    }
    *(u32x4*)((uint16_t*)a.O + off) = out;
  } else {
    const f32x4* x = (const f32x4*)((const float*)a.O1 + off);
    const f32x4* y = (const f32x4*)((const float*)a.O2 + off);
    const f32x4 x0 = x[0], x1 = x[1], y0 = y[0], y1 = y[1];
    f32x4* out = (f32x4*)((float*)a.O + off);
    out[0] = w1 * x0 + w2 * y0;
    out[1] = w1 * x1 + w2 * y1;
  }
  if (cidx == 0) a.L[lrow] = Lm;
}

// -------------------------------------------------------------- launchers

hipError_t launch_transpose_v(const TransposeArgs& a, int B, int D, hipStream_t s) {
  dim3 grid(a.nB, a.heads.n, B);
  if (D == 128)
    hipLaunchKernelGGL(transpose_v_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(transpose_v_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool DENSE>
static void launch_attn_t(const AttnArgs& a, bool out_bf16, hipStream_t s) {
  // room for either row order of the sparse kernel (8 XCDs x whole chunks of 8)
  dim3 grid(DENSE ? 8 * a.per_xcd : 64 * ((a.rows + 63) / 64));
  if (out_bf16)
    hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE, true>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE, false>), grid, dim3(128), 0, s, a);
}

hipError_t launch_attn_chunks(const AttnArgs& a, int D, bool out_bf16, hipStream_t s) {
  const dim3 grid(64 * ((a.rows + 63) / 64));
  if (D == 128) {
    if (out_bf16) hipLaunchKernelGGL((attn_fwd_kernel<128, false, true, true>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false, false, true>), grid, dim3(128), 0, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((attn_fwd_kernel<64, false, true, true>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false, false, true>), grid, dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int D, bool dense, bool out_bf16, hipStream_t s) {
  if (D == 128) {
    if (dense) launch_attn_t<128, true>(a, out_bf16, s);
    else launch_attn_t<128, false>(a, out_bf16, s);
  } else {
    if (dense) launch_attn_t<64, true>(a, out_bf16, s);
    else launch_attn_t<64, false>(a, out_bf16, s);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int B, bool bf16, hipStream_t s) {
  const int64_t threads = (int64_t)a.N * (a.D / 8);
  dim3 grid((unsigned)((threads + 255) / 256), a.heads.n, B);
  if (bf16) hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsa
