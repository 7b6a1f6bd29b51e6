// bf16 MFMA GEMM for gfx950 fed by direct HBM -> LDS DMA.
//
//   C[M x N] = A[M x K] . B[K x N]   (fp32 accumulate, K a multiple of 32)
//
// Same operand layouts and fused epilogues as the general kernel (gemm.hip);
// what changes is the data path, built for CDNA4:
//
//  * global_load_lds_dwordx4 moves each 16-byte granule straight from HBM
//    into LDS without passing through VGPRs, so a 6-stage ring of 32-deep
//    K-slabs can be in flight with no staging registers.  A wave's DMA
//    writes 1 KiB of LDS contiguously (lane i -> byte 16*i); the LDS layout
//    is chosen by which global granule each lane fetches.
//  * Operands stored k-contiguous (A in NN/NT, B in NT) keep rows of one
//    slab depth; fragment reads are ds_read_b128.  Granule c of row r sits
//    at c ^ swz_k(r), which spreads the 16 rows a read touches over all
//    banks.
//  * Operands stored m/n-contiguous (B in NN, A and B in TN) keep the global
//    [k][n] row layout; the MFMA operand (8 consecutive k of one column) is
//    produced by two ds_read_b64_tr_b16 transpose reads.  Within a 16-lane
//    group, lane j receives element (j & 3) of the 8-byte chunks addressed
//    by lanes 4e + (j >> 2), e = 0..3; lane s therefore addresses row
//    k0 + 8g + (s >> 2) (+4 for the second read), columns 4(s & 3) .. +3.
//    Granule index bits 1..3 are XOR-swizzled with the row so that the 8
//    rows a half-wave reads land on distinct banks.
//  * One barrier per K-slab; s_waitcnt vmcnt(n) waits only for the slab
//    about to be used while later slabs' DMA stays in flight.  The MFMA
//    operands of slab k+1 are read from LDS into a second register set
//    while slab k's MFMAs run (interleaved by sched_group_barrier), so LDS
//    latency hides under matrix-core work even at one wave per SIMD.
//  * Rows/columns past M or N are clamped to the last valid one (their
//    results are never stored), so no load leaves the operands.
#include <type_traits>

#include "gemm_common.hpp"
#include "lds_dma.hpp"

namespace tpcol {

// 16-byte output store with device scope (sc1): the line is written through
// to the memory side instead of staying dirty in this XCD's L2, so the
// writeback at the end of the kernel finds (almost) nothing left and the
// consumer, on whichever XCD, reads it from the Infinity Cache as before.
// Measured on the GPT-2-medium shard: row GEMM 25.5 -> 24.2 us, column GEMM
// 27.3 -> 26.7 us, consumers unchanged (nontemporal stores, by contrast,
// sped the producer up but sent the consumers to HBM).
typedef unsigned int u32x4_wt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_wt(void *dst, const void *lds_src) {
  const u32x4_wt v = *reinterpret_cast<const u32x4_wt *>(lds_src);
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(dst), "v"(v) : "memory");
}

// k-contiguous rows of BK elements (BK/8 granules); granule swizzle per row.
// For 32-deep slabs (64-byte rows) the fragment read (16 consecutive rows,
// one granule each, per 16-lane group) is free of bank conflicts on gfx950
// with granule c of row r stored at c ^ ((r >> 1) & 3), as measured with the
// LDS bank-conflict counter; XOR patterns that also mix in row bit 3 cost
// four conflict cycles per read.
template <int BK>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (BK == 64) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 1) & 3;
}
__device__ __forceinline__ int swz_mn(int r) { return ((r & 3) | (((r >> 3) & 1) << 2)) << 1; }

// ---------------------------------------------------------------- tile DMA
// k-contiguous operand: ROWS rows x BK k; one wave-DMA fills 1 KiB =
// 1024 / (2 BK) rows.
template <int ROWS, int BK, int NW>
struct KTileDma {
  static constexpr int GPR = BK / 8;          // granules per row
  static constexpr int RPB = 64 / GPR;        // rows per 1 KiB block
  static constexpr int NBLK = ROWS / RPB;
  static constexpr int PER_WAVE = NBLK / NW;
  static_assert(NBLK % NW == 0, "tile rows");
  const uint16_t *src[PER_WAVE];
  const uint16_t *src2[PER_WAVE];

  __device__ __forceinline__ void init(const uint16_t *g, int64_t ld, const uint16_t *g2, int64_t ld2,
                                       int row0, int rows_lim, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave + NW * j;
      const int row = blk * RPB + lane / GPR;
      const int c = (lane % GPR) ^ swz_k<BK>(row);
      const int64_t gr = min(row0 + row, rows_lim - 1);
      src[j] = g + gr * ld + c * 8;
      src2[j] = g2 ? g2 + gr * ld2 + c * 8 : nullptr;
    }
  }
  // k0: first k of the slab; use2: the slab lies in the second source, whose
  // k index starts at K1 (K1 a multiple of BK)
  __device__ __forceinline__ void issue(uint32_t lds, int k0, int K1, bool use2, int wave) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave + NW * j;
      const uint16_t *s = use2 ? src2[j] + (k0 - K1) : src[j] + k0;
      dma16(s, lds + blk * 1024);
    }
  }
};

// m/n-contiguous operand: BK k-rows x COLS, each row COLS/8 granules.
template <int COLS, int BK, int NW>
struct MNTileDma {
  static constexpr int GPR = COLS / 8;      // granules per row
  static constexpr int RPB = 64 / GPR;      // rows per 1 KiB block
  static constexpr int NBLK = BK / RPB;     // blocks per slab
  static constexpr int PER_WAVE = NBLK / NW;
  static_assert(GPR >= 16 && RPB >= 1 && NBLK % NW == 0, "MN tile needs at least 128 columns");
  const uint16_t *src[PER_WAVE];
  int64_t step;  // elements per slab (BK rows)

  __device__ __forceinline__ void init(const uint16_t *g, int64_t ld, int col0, int col_lim, int wave,
                                       int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave + NW * j;
      const int row = blk * RPB + lane / GPR;
      const int lg = (lane % GPR) ^ swz_mn(row);
      const int col = min(col0 + lg * 8, col_lim - 8);
      src[j] = g + (int64_t)row * ld + col;
    }
    step = (int64_t)BK * ld;
  }
  __device__ __forceinline__ void issue(uint32_t lds, int kt, int wave) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave + NW * j;
      dma16(src[j] + kt * step, lds + blk * 1024);
    }
  }
};

// ---------------------------------------------------------------- fragments
// k-contiguous tile (rows of BK): 8 k of row `row`, granule c = kc*4 + g.
template <int BK>
__device__ __forceinline__ uint4 frag_k(const uint16_t *t, int row, int c) {
  return *reinterpret_cast<const uint4 *>(t + row * BK + ((c ^ swz_k<BK>(row)) << 3));
}

// m/n-contiguous tile: 8 consecutive k (kc*32 + 8g ..) of column c0 + (lane & 15).
template <int COLS>
__device__ __forceinline__ uint4 frag_mn(const uint16_t *t, int kc, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int r1 = kc * 32 + 8 * g + (s >> 2);
  const int col = c0 + 4 * (s & 3);
  const int sw = swz_mn(r1);  // == swz_mn(r1 + 4)
  const int off = (((col >> 3) ^ sw) << 3) + (col & 4);
  const uint2 a = tr_read(t + r1 * COLS + off);
  const uint2 b = tr_read(t + (r1 + 4) * COLS + off);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// BM x BN tile per workgroup of WGM x WGN wave64s; LBK-deep K slabs through a
// STAGES-deep LDS ring.  PREFETCH: read the next slab's fragments while the
// current slab's MFMAs run (for one wave per SIMD); without it the second
// wave on each SIMD covers the LDS latency.
template <int BM, int BN, int LBK, int WGM, int WGN, int LAYOUT, int EPI, bool DUAL, bool KCAT,
          int STAGES, bool PREFETCH>
__global__ void __launch_bounds__(WGM * WGN * 64) gemm_lds_kernel(GemmParams pin) {
  GemmParams p = pin;
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr bool AT = (LAYOUT == LAY_TN);
  constexpr bool BT = (LAYOUT == LAY_NT);
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int A_EL = BM * LBK, B_EL = BN * LBK;
  constexpr int STAGE = A_EL + NB * B_EL;
  using ATile = typename std::conditional<AT, MNTileDma<BM, LBK, NW>, KTileDma<BM, LBK, NW>>::type;
  using BTile = typename std::conditional<BT, KTileDma<BN, LBK, NW>, MNTileDma<BN, LBK, NW>>::type;
  constexpr int LOADS = ATile::PER_WAVE + NB * BTile::PER_WAVE;  // DMA ops per wave per slab
  static_assert(STAGES >= 2 && LOADS * (STAGES - 1) < 64, "pipeline depth");

  // Single-output epilogues write the finished tile through LDS (the ring is
  // idle by then) when the whole tile fits in 144 KiB: every wave computes
  // its values at once, then the workgroup stores whole 16-byte chunks of
  // consecutive rows (the direct stores write 16 rows x 32 or 64 bytes per
  // instruction, which measured slower).  256 x 256 fp32 tiles (256 KiB)
  // keep the direct stores: staging them in two row bands idles half the
  // waves per band and measured slower than storing directly.
  constexpr int OES = EPI == EPI_STORE_F32 ? 4 : 2;  // output element bytes
  constexpr int SROW = BN * OES + 16;               // staged row bytes (16-byte pad)
  constexpr bool STAGED = (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_STORE_F32 || EPI == EPI_SWIGLU) &&
                          BM * SROW <= 144 * 1024;
  // The activation backward epilogues (dH read; GELU: dZ and H written,
  // SwiGLU: dZg, dZu and H) stage dH and then their outputs one tile at a
  // time the same way.  Reading dH element by element between the stores
  // would serialise: every load waits for the stores before it, which the
  // compiler cannot prove do not overlap it.
  constexpr bool STAGED3 = (EPI == EPI_SWIGLU_BWD || EPI == EPI_GELU_BWD) && 2 * BM * (BN * 2 + 16) <= 144 * 1024;
  constexpr int NOUT = EPI == EPI_SWIGLU_BWD ? 3 : 2;
  constexpr int RING_EL = STAGES * STAGE;
  constexpr int STG_EL = STAGED ? BM * SROW / 2 : (STAGED3 ? BM * (BN * 2 + 16) : 0);
  __shared__ __attribute__((aligned(1024))) uint16_t smem[RING_EL > STG_EL ? RING_EL : STG_EL];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int M = p.M, N = p.N;
  const int nk = p.K / LBK;
  constexpr bool PRIO = BM == 256 && LAYOUT != LAY_TN && !KCAT;

  int tm, tn;
  tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const uint16_t *Ag = static_cast<const uint16_t *>(p.A);
  const uint16_t *Bg = static_cast<const uint16_t *>(p.B);
  if constexpr (LAYOUT == LAY_TN) {
    // split-K: grid row z takes K rows [z K, (z+1) K) of both operands and
    // writes its own fp32 partial
    const int z = blockIdx.y;
    Ag += (int64_t)z * p.K * p.lda;
    Bg += (int64_t)z * p.K * p.ldb;
    p.C = static_cast<float *>(p.C) + (int64_t)z * p.zstride;
  }
  const uint16_t *B2g = static_cast<const uint16_t *>(p.B2);

  ATile ta;
  BTile tb;
  MNTileDma<BN, LBK, NW> tb2;
  if constexpr (AT) ta.init(Ag, p.lda, m0, M, wave, lane);
  else ta.init(Ag, p.lda, nullptr, 0, m0, M, wave, lane);
  if constexpr (BT) tb.init(Bg, p.ldb, KCAT ? B2g : nullptr, p.ldb2, n0, N, wave, lane);
  else tb.init(Bg, p.ldb, n0, N, wave, lane);
  if constexpr (DUAL) tb2.init(B2g, p.ldb2, n0, N, wave, lane);

  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int kt, int stage) {
    const uint32_t base = smem_lds + stage * (STAGE * 2);
    if constexpr (AT) ta.issue(base, kt, wave);
    else ta.issue(base, kt * LBK, 0, false, wave);
    if constexpr (BT) {
      const int k0 = kt * LBK;
      tb.issue(base + A_EL * 2, k0, p.K1, KCAT && k0 >= p.K1, wave);
    } else {
      tb.issue(base + A_EL * 2, kt, wave);
    }
    if constexpr (DUAL) tb2.issue(base + (A_EL + B_EL) * 2, kt, wave);
  };

  f32x4_t acc[TM][TN];
  f32x4_t acc2[DUAL ? TM : 1][DUAL ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  if constexpr (DUAL) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc2[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  const int g = lane >> 4, l16 = lane & 15;

  // Register fragments of one whole slab (both 32-deep k chunks).
  struct Frags {
    uint4 a[LBK / 32][TM];
    uint4 b[LBK / 32][TN];
    uint4 b2[LBK / 32][DUAL ? TN : 1];
  };
  auto load_frags = [&](Frags &F, int stage) {
    const uint16_t *As = smem + stage * STAGE;
    const uint16_t *Bs = As + A_EL;
    const uint16_t *B2s = Bs + B_EL;
#pragma unroll
    for (int kc = 0; kc < LBK / 32; ++kc) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (AT) F.a[kc][i] = frag_mn<BM>(As, kc, wm * WTM + i * 16, lane);
        else F.a[kc][i] = frag_k<LBK>(As, wm * WTM + i * 16 + l16, kc * 4 + g);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BT) F.b[kc][j] = frag_k<LBK>(Bs, wn * WTN + j * 16 + l16, kc * 4 + g);
        else F.b[kc][j] = frag_mn<BN>(Bs, kc, wn * WTN + j * 16, lane);
        if constexpr (DUAL) F.b2[kc][j] = frag_mn<BN>(B2s, kc, wn * WTN + j * 16, lane);
      }
    }
  };
  auto mma = [&](const Frags &F) {
#pragma unroll
    for (int kc = 0; kc < LBK / 32; ++kc) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(F.b[kc][j], F.a[kc][i], acc[i][j]);
      if constexpr (DUAL) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc2[i][j] = mfma16(F.b2[kc][j], F.a[kc][i], acc2[i][j]);
      }
    }
  };
  // LDS read instructions and MFMAs per slab, for the interleave hint
  constexpr int DS_A = (LBK / 32) * TM * (AT ? 2 : 1);
  constexpr int DS_B = (LBK / 32) * TN * (BT ? 1 : 2) * NB;
  constexpr int N_DS = DS_A + DS_B;
  constexpr int N_MFMA = (LBK / 32) * TM * TN * NB;
  constexpr int MFMA_PER_DS = (N_MFMA + N_DS - 1) / N_DS;

  // One slab: MFMAs on F (already in registers) while the next slab's
  // fragments stream from LDS into Fn.
  auto step = [&](int kt, Frags &F, Frags &Fn) {
    if (kt + 1 < nk) {
      if (kt + STAGES - 1 < nk) wait_vmcnt<LOADS * (STAGES - 2)>();
      else wait_vmcnt<0>();
      __syncthreads();  // slab kt+1 visible; every wave is done reading slab kt's stage
      if (kt + STAGES < nk) issue(kt + STAGES, kt % STAGES);
      load_frags(Fn, (kt + 1) % STAGES);
      mma(F);
#pragma unroll
      for (int q = 0; q < N_DS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_DS, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS read
      }
    } else {
      mma(F);
    }
  };

  if constexpr (PREFETCH) {
    // prologue: STAGES slabs in flight, slab 0's fragments into registers
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nk) issue(s, s);
    if (nk >= STAGES) wait_vmcnt<LOADS * (STAGES - 1)>();
    else wait_vmcnt<0>();
    __syncthreads();
    Frags F0, F1;
    load_frags(F0, 0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, F0, F1);
      step(kt + 1, F1, F0);
    }
    if (kt < nk) step(kt, F0, F1);
  } else {
    // prologue: STAGES-1 slabs in flight.  Iteration kt waits for slab kt,
    // and after the barrier refills the stage that held slab kt-1 with slab
    // kt+STAGES-1 (every wave finished reading it before the barrier).
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s, s);
    Frags F;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + STAGES - 2 < nk) wait_vmcnt<LOADS * (STAGES - 2)>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
      load_frags(F, kt % STAGES);
      // 256 x 256 NN / NT tiles: a wave issuing its MFMAs takes issue
      // priority over the other wave of its SIMD (still reading fragments or
      // issuing DMA), which keeps the matrix pipe fed: 1-4% on the Llama and
      // MHA shapes; TN and K-concatenated tiles measured no gain.
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
      mma(F);
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    }
  }

  // ---- epilogue: lane holds C[row][col .. col+3] of every 16x16 tile
  if constexpr (STAGED) {
    using OutT = typename std::conditional<EPI == EPI_STORE_F32, float, uint16_t>::type;
    char *stg = reinterpret_cast<char *>(smem);
    constexpr int CPR = BN * OES / 16;  // 16-byte chunks per tile row
    float bv[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 16 + g * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[j][r] = 0.f;
      if (p.bias != nullptr && col < N) {
        if constexpr (EPI == EPI_STORE_F32) load4(static_cast<const float *>(p.bias) + col, bv[j]);
        else load4(static_cast<const uint16_t *>(p.bias) + col, bv[j]);
      }
    }
    __syncthreads();  // every wave is done reading the ring
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][r] + bv[j][r];
          if constexpr (EPI == EPI_GELU) v[r] = gelu_f(v[r]);
          if constexpr (EPI == EPI_SWIGLU) v[r] = silu_f(v[r]) * acc2[DUAL ? i : 0][DUAL ? j : 0][r];
        }
        char *dst = stg + (wm * WTM + i * 16 + l16) * SROW + (wn * WTN + j * 16 + g * 4) * OES;
        store4(reinterpret_cast<OutT *>(dst), v);
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < BM * CPR; c += NW * 64) {
      const int rl = c / CPR, cc = c % CPR;
      const int row = m0 + rl, col = n0 + cc * (16 / OES);
      if (row < M && col < N)
        store16_wt(static_cast<OutT *>(p.C) + (int64_t)row * p.ldc + col, stg + rl * SROW + cc * 16);
    }
    return;
  }
  if constexpr (STAGED3) {
    // dH comes into LDS by coalesced 16-byte loads; then each output tile
    // (GELU: dZ, H; SwiGLU: dZg, dZu, H) in turn is computed from the
    // accumulators and dH, written to LDS and stored as whole row chunks.
    constexpr int SR = BN * 2 + 16;  // staged row bytes
    constexpr int CPR = BN * 2 / 16;
    char *dhs = reinterpret_cast<char *>(smem);
    char *out = dhs + BM * SR;
    if (p.bias != nullptr) {  // the bias belongs to the (gate) pre-activation
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WTN + j * 16 + g * 4;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (col < N) load4(static_cast<const uint16_t *>(p.bias) + col, bv);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += bv[r];
      }
    }
    __syncthreads();  // every wave is done reading the ring
    for (int c = threadIdx.x; c < BM * CPR; c += NW * 64) {
      const int rl = c / CPR, cc = c % CPR;
      const int row = m0 + rl, col = n0 + cc * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row < M && col < N)
        v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.D) + (int64_t)row * p.ldd + col);
      *reinterpret_cast<uint4 *>(dhs + rl * SR + cc * 16) = v;
    }
    __syncthreads();
#pragma unroll
    for (int which = 0; which < NOUT; ++which) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int off = (wm * WTM + i * 16 + l16) * SR + (wn * WTN + j * 16 + g * 4) * 2;
          float dh[4], o[4];
          load4(reinterpret_cast<const uint16_t *>(dhs + off), dh);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[i][j][r];
            if constexpr (EPI == EPI_GELU_BWD) {
              o[r] = which == 0 ? dh[r] * gelu_grad_f(gt) : gelu_f(gt);
            } else {
              const float ut = acc2[DUAL ? i : 0][DUAL ? j : 0][r];
              const float sg = sigmoid_f(gt);
              const float sl = gt * sg;
              o[r] = which == 0 ? dh[r] * ut * (sg * (1.0f + gt * (1.0f - sg))) : (which == 1 ? dh[r] * sl : sl * ut);
            }
          }
          store4(reinterpret_cast<uint16_t *>(out + off), o);
        }
      }
      __syncthreads();
      // SwiGLU: dZg -> C, dZu -> C3, H -> C2; GELU: dZ -> C, H -> C2
      void *C = which == 0 ? p.C : (which == NOUT - 1 ? p.C2 : p.C3);
      const int64_t ldc = which == 0 ? p.ldc : (which == NOUT - 1 ? p.ldc2 : p.ldc3);
      for (int c = threadIdx.x; c < BM * CPR; c += NW * 64) {
        const int rl = c / CPR, cc = c % CPR;
        const int row = m0 + rl, col = n0 + cc * 8;
        if (row < M && col < N)
          store16_wt(static_cast<uint16_t *>(C) + (int64_t)row * ldc + col, out + rl * SR + cc * 16);
      }
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = m0 + wm * WTM + i * 16 + l16;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 16 + g * 4;
      if (row >= M || col >= N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      float u[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DUAL) {
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = acc2[DUAL ? i : 0][DUAL ? j : 0][r];
      }
      epilogue4<uint16_t, EPI>(p, row, col, v, u);
    }
  }
}

// ---------------------------------------------------------------- host side
template <int BM, int BN, int LBK, int WGM, int WGN, int LAYOUT, int EPI, bool DUAL, bool KCAT,
          int STAGES, bool PREFETCH>
static hipError_t run_lds(const GemmArgs &a, hipStream_t s) {
  GemmParams p;
  p.colsum = nullptr;  // only the 64-deep kernel writes column sums
  p.A = a.A; p.lda = a.lda;
  p.B = a.B; p.ldb = a.ldb;
  p.B2 = a.B2; p.ldb2 = a.ldb2;
  p.bias = a.bias;
  p.D = a.D; p.ldd = a.ldd;
  p.C = a.C; p.ldc = a.ldc;
  p.C2 = a.C2; p.ldc2 = a.ldc2;
  p.C3 = a.C3; p.ldc3 = a.ldc3;
  p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K; p.K1 = (int)a.K1;
  p.tiles_m = (int)((a.M + BM - 1) / BM);
  p.tiles_n = (int)((a.N + BN - 1) / BN);
  p.zstride = a.zstride;
  hipLaunchKernelGGL(
      (gemm_lds_kernel<BM, BN, LBK, WGM, WGN, LAYOUT, EPI, DUAL, KCAT, STAGES, PREFETCH>),
      dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)a.splits), dim3(WGM * WGN * 64), 0, s, p);
  return hipGetLastError();
}

// Tile configurations measured on MI355X: 8 wave64 per
// workgroup (two per SIMD, so LDS and DMA latency of one wave hides under
// the other's MFMAs) and 256-wide tiles to cut L2 -> CU traffic per flop.
static int64_t cu_count() {
  // the attribute query is cached per host thread for its current device
  thread_local int cached_dev = -1, cached_n = 0;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev == cached_dev) return cached_n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  cached_dev = dev;
  cached_n = n;
  return n;
}

template <int LAYOUT, int EPI, bool DUAL, bool KCAT>
static hipError_t pick_lds(const GemmArgs &a, hipStream_t s) {
  const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int64_t t128x256 = ((a.M + 127) / 128) * ((a.N + 255) / 256);
  if constexpr (DUAL) {
    // four 40 KiB stages fill the 160 KiB of LDS (one workgroup per CU
    // either way: its 8 waves take all the VGPRs); measured 2-8% faster than
    // two or three stages on the Llama SwiGLU shard
    if constexpr (EPI == EPI_STORE_F32 && LAYOUT == LAY_NN) {
      // mid-size fp32 NN products (the row-parallel partial of a narrow
      // shard): 128 x 128 tiles stage in 67 KiB, so two workgroups share a
      // CU and one's fp32 stores overlap the other's loop (8192 x 1024 x
      // 1024: 23.9 -> 23.1 us; NT and split TN products measured slower)
      const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
      const int64_t cus = cu_count();
      if (a.splits == 1 && t128 >= cus && t128 <= 2 * cus)
        return run_lds<128, 128, 32, 2, 2, LAYOUT, EPI, DUAL, KCAT, 3, false>(a, s);
    }
    if (t128x256 >= 128) return run_lds<128, 256, 32, 2, 4, LAYOUT, EPI, DUAL, KCAT, 4, false>(a, s);
    return run_lds<128, 128, 32, 2, 2, LAYOUT, EPI, DUAL, KCAT, 3, false>(a, s);
  } else {
    if (t256 >= 192) {
      // Both large-tile configurations run one workgroup per CU, so a launch
      // takes ceil(tiles / CUs) rounds; a 256x256 tile costs about 65536 /
      // 1230 and a 128x256 tile 32768 / 1122 (their measured steady-state
      // TFLOP/s).  Where 256x256 tiles leave a half-empty last round (e.g.
      // 8192 x 3072: 384 tiles = 1.5 rounds) the smaller tiles fill theirs.
      const int64_t cus = cu_count();
      const double c256 = (double)((t256 + cus - 1) / cus) * (65536.0 / 1230.0);
      const double c128 = (double)((t128x256 + cus - 1) / cus) * (32768.0 / 1122.0);
      if (c256 <= c128) return run_lds<256, 256, 32, 2, 4, LAYOUT, EPI, DUAL, KCAT, 3, false>(a, s);
      return run_lds<128, 256, 32, 2, 4, LAYOUT, EPI, DUAL, KCAT, 4, false>(a, s);
    }
    if constexpr (EPI == EPI_STORE_F32 && LAYOUT == LAY_NN) {
      // mid-size fp32 NN products (the row-parallel partial of a narrow
      // shard): 128 x 128 tiles stage in 67 KiB, so two workgroups share a
      // CU and one's fp32 stores overlap the other's loop (8192 x 1024 x
      // 1024: 23.9 -> 23.1 us; NT and split TN products measured slower)
      const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
      const int64_t cus = cu_count();
      if (a.splits == 1 && t128 >= cus && t128 <= 2 * cus)
        return run_lds<128, 128, 32, 2, 2, LAYOUT, EPI, DUAL, KCAT, 3, false>(a, s);
    }
    if (t128x256 >= 128) return run_lds<128, 256, 32, 2, 4, LAYOUT, EPI, DUAL, KCAT, 4, false>(a, s);
    return run_lds<128, 128, 32, 2, 2, LAYOUT, EPI, DUAL, KCAT, 3, false>(a, s);
  }
}

hipError_t launch_gemm_lds(const GemmArgs &a, hipStream_t s) {
  constexpr int LBK = 32;  // slab depth of every instantiation below
  if (a.dtype != DT_BF16 || a.K <= 0 || a.K % LBK != 0) return hipErrorNotSupported;
  if (a.kcat && a.K1 % LBK != 0) return hipErrorNotSupported;
  // small problems stay on the general kernel (more, smaller tiles)
  if (((a.M + 127) / 128) * ((a.N + 127) / 128) * a.splits < 64) return hipErrorNotSupported;
  if (a.splits > 1 && (a.layout != LAY_TN || a.epi != EPI_STORE_F32)) return hipErrorInvalidValue;
  if (a.M < 8 || a.N < 8) return hipErrorNotSupported;
  switch (a.layout) {
    case LAY_NN:
      if (a.dual) {
        if (a.epi == EPI_SWIGLU) return pick_lds<LAY_NN, EPI_SWIGLU, true, false>(a, s);
        if (a.epi == EPI_SWIGLU_BWD) return pick_lds<LAY_NN, EPI_SWIGLU_BWD, true, false>(a, s);
        return hipErrorNotSupported;
      }
      switch (a.epi) {
        case EPI_STORE: return pick_lds<LAY_NN, EPI_STORE, false, false>(a, s);
        case EPI_STORE_F32: return pick_lds<LAY_NN, EPI_STORE_F32, false, false>(a, s);
        case EPI_GELU: return pick_lds<LAY_NN, EPI_GELU, false, false>(a, s);
        case EPI_GELU_BWD: return pick_lds<LAY_NN, EPI_GELU_BWD, false, false>(a, s);
        default: return hipErrorNotSupported;
      }
    case LAY_NT:
      if (a.dual) return hipErrorNotSupported;
      if (a.kcat) {
        if (a.epi == EPI_STORE_F32) return pick_lds<LAY_NT, EPI_STORE_F32, false, true>(a, s);
        return hipErrorNotSupported;
      }
      if (a.epi == EPI_STORE) return pick_lds<LAY_NT, EPI_STORE, false, false>(a, s);
      if (a.epi == EPI_STORE_F32) return pick_lds<LAY_NT, EPI_STORE_F32, false, false>(a, s);
      return hipErrorNotSupported;
    case LAY_TN:
      if (a.dual || a.kcat || a.epi != EPI_STORE_F32) return hipErrorNotSupported;
      return pick_lds<LAY_TN, EPI_STORE_F32, false, false>(a, s);
  }
  return hipErrorNotSupported;
}

}  // namespace tpcol
