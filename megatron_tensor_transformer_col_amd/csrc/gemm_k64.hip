// bf16 MFMA GEMM for gfx950 with 64-deep K slabs.
//
//   C[M x N] = A[M x K] . B[K x N]   (fp32 accumulate, K a multiple of 64)
//
// Same operand layouts (NN, NT, TN) and fused epilogues as the other GEMM
// kernels; the design choices, each measured on MI355X:
//
//  * 64-deep slabs.  A k-contiguous operand row then contributes 128 bytes
//    per slab, a whole cache line, so every L2 request of the HBM -> LDS DMA
//    carries a full line; with 32-deep slabs half of them were 64-byte
//    half-lines and the DMA topped out near 18 TB/s instead of ~23.
//  * 128 x 128 tiles: four wave64 per workgroup (one per SIMD, 64 x 64
//    each) and two workgroups per CU.  The next 32-deep chunk's fragments
//    are read from LDS while the current chunk's MFMAs run (two register
//    sets), and one barrier per slab sits between a slab's two chunks,
//    where every wave has finished reading the slab before.  While one
//    workgroup is in its epilogue (activation, staging, stores) the other
//    keeps the matrix cores busy, which hides the erf-GELU of the
//    column-parallel product.
//  * 256-row tiles (256 x 256, and the 128-row dual tiles): eight waves,
//    two per SIMD, in ping-pong: the two waves of a SIMD alternate between
//    a phase of MFMAs on fragments already in registers and a phase of LDS
//    reads (and DMA issue), switching at workgroup barriers, so the matrix
//    core of every SIMD always has one wave feeding it.  One workgroup per
//    CU; these tiles serve products with whole rounds of them.
//  * Dual products (SwiGLU: X.Wg and X.Wu) stage both weight slabs side by
//    side and keep both accumulators of an output element in one wave, so
//    the gate and up values meet in registers: 256 x 128 output tiles carry
//    the same per-slab traffic and MFMA work as a 256 x 256 single product.
//  * The compiler's register allocation is steered with the minimal-register
//    scheduling strategy (build flag); the default one shuffled accumulators
//    between AGPRs and VGPRs inside the loop.
//
// Operand staging in LDS (each stage one 64-deep slab of A and of B):
//  * k-contiguous rows (A in NN/NT, B in NT): 128 bytes = 8 granules of 16 B,
//    granule c of row r stored at slot c ^ swz_k(r); fragments by
//    ds_read_b128 (8 consecutive k of one row per lane).
//  * m/n-contiguous rows (B in NN, A and B in TN): 64 k-rows as in HBM with
//    the granule index XOR-swizzled by the row; the MFMA operand (8
//    consecutive k of one column) comes from two ds_read_b64_tr_b16.
//  * Rows / columns past M / N are clamped to the last valid one on load
//    (their results are never stored), so no load leaves the operands.
#include <algorithm>
#include <type_traits>

#include "gemm_common.hpp"
#include "lds_dma.hpp"

namespace tpcol {
namespace k64 {

constexpr int LBK = 64;  // slab depth
constexpr int NW = 4;    // waves per workgroup (one per SIMD); eight in the ping-pong kernel

// Workgroup barrier that the compiler may not schedule any instruction
// across (the ping-pong loop relies on the MFMAs and LDS reads of a phase
// staying between its two barriers).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// device-scope (write-through) 16-byte store from LDS; see gemm_lds.hip
typedef unsigned int u32x4_wt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_wt(void *dst, const void *lds_src) {
  const u32x4_wt v = *reinterpret_cast<const u32x4_wt *>(lds_src);
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(dst), "v"(v) : "memory");
}

// Bias of a lane's TF column groups (columns col0 + 16 f .. +3, zero from N
// on; N is a multiple of 4): all loads are issued before the first wait (a
// column past N reads column 0, so no load depends on a branch).
template <typename BT, int TF>
__device__ __forceinline__ void load_bias(const BT *bias, int col0, int N, float (&bv)[TF][4]) {
  using Raw = typename std::conditional<sizeof(BT) == 2, uint2, float4>::type;
  Raw raw[TF];
#pragma unroll
  for (int f = 0; f < TF; ++f) {
    const int col = col0 + 16 * f;
    raw[f] = *reinterpret_cast<const Raw *>(bias + (col < N ? col : 0));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < TF; ++f) {
    const bool ok = col0 + 16 * f < N;
    float v[4];
    if constexpr (sizeof(BT) == 2) {
      v[0] = bf2f((uint16_t)(raw[f].x & 0xffffu)); v[1] = bf2f((uint16_t)(raw[f].x >> 16));
      v[2] = bf2f((uint16_t)(raw[f].y & 0xffffu)); v[3] = bf2f((uint16_t)(raw[f].y >> 16));
    } else {
      v[0] = raw[f].x; v[1] = raw[f].y; v[2] = raw[f].z; v[3] = raw[f].w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) bv[f][r] = ok ? v[r] : 0.f;
  }
}

// k-contiguous 128-byte rows: slot of granule c in row r is c ^ swz_k(r)
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
// m/n-contiguous rows: granule index bits 1..3 XOR-ed with row bits
__device__ __forceinline__ int swz_mn(int r) { return ((r & 3) | (((r >> 3) & 1) << 2)) << 1; }

// DMA of a k-contiguous operand slab: ROWS rows x 64 k (8 rows per KiB),
// shared by NWI waves.  Per-lane 32-bit offsets relative to the tile's
// first row; the slab's base pointer is wave-uniform (SGPRs).  KCAT: rows
// of the second source (k >= K1) have their own offsets.
template <int ROWS, bool KCAT, int NWI>
struct KDma {
  static constexpr int PER_WAVE = ROWS / 8 / NWI;
  static_assert(ROWS % (8 * NWI) == 0, "rows");
  uint32_t off[PER_WAVE];
  uint32_t off2[KCAT ? PER_WAVE : 1];
  __device__ __forceinline__ void init(int64_t ld, int64_t ld2, int row0, int rows_lim, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int row = (wave + NWI * j) * 8 + lane / 8;
      const int c = (lane % 8) ^ swz_k(row);
      const int64_t gr = min(row0 + row, rows_lim - 1) - row0;
      off[j] = (uint32_t)(gr * ld * 2 + c * 16);
      if constexpr (KCAT) off2[j] = (uint32_t)(gr * ld2 * 2 + c * 16);
    }
  }
  __device__ __forceinline__ void issue(const uint16_t *base, bool second, uint32_t lds, int wave) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const uint32_t o = (KCAT && second) ? off2[KCAT ? j : 0] : off[j];
      dma16s(o, base, lds + (wave + NWI * j) * 1024);
    }
  }
};

// DMA of an m/n-contiguous operand slab: 64 k-rows x COLS, shared by NWI waves.
template <int COLS, int NWI>
struct NDma {
  static constexpr int GPR = COLS / 8;    // granules per row
  static constexpr int RPB = 64 / GPR;    // rows per KiB
  static constexpr int PER_WAVE = LBK / RPB / NWI;
  static_assert(GPR >= 16 && (LBK / RPB) % NWI == 0, "cols");
  uint32_t off[PER_WAVE];
  __device__ __forceinline__ void init(int64_t ld, int col0, int col_lim, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int row = (wave + NWI * j) * RPB + lane / GPR;
      const int lg = (lane % GPR) ^ swz_mn(row);
      const int col = min(col0 + lg * 8, col_lim - 8) - col0;
      off[j] = (uint32_t)((int64_t)row * ld * 2 + col * 2);
    }
  }
  __device__ __forceinline__ void issue(const uint16_t *base, uint32_t lds, int wave) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) dma16s(off[j], base, lds + (wave + NWI * j) * 1024);
  }
};

// Per-lane LDS byte offsets of one operand's fragments inside a stage, for
// chunk kc (0/1) and fragment f (16 rows / columns each).
template <bool KTYPE, int SPAN, int WT>
struct FragAddr {
  static constexpr int NF = WT / 16;
  uint32_t off[2][KTYPE ? 1 : NF];
  __device__ __forceinline__ void init(uint32_t region, int first, int lane) {
    const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      if constexpr (KTYPE) {
        const int row = first + l16;  // + 16 f: swz_k only reads row bits 1..3
        off[kc][0] = region + (uint32_t)(row * 128 + (((kc * 4 + g) ^ swz_k(row)) << 4));
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int r1 = kc * 32 + 8 * g + (l16 >> 2);
          const int col = first + f * 16 + 4 * (l16 & 3);
          const int o = (((col >> 3) ^ swz_mn(r1)) << 3) + (col & 4);  // swz_mn(r1) == swz_mn(r1 + 4)
          off[kc][f] = region + (uint32_t)((r1 * SPAN + o) * 2);
        }
      }
    }
  }
  __device__ __forceinline__ uint4 read(const char *stage, int kc, int f) const {
    if constexpr (KTYPE) {
      return *reinterpret_cast<const uint4 *>(stage + off[kc][0] + f * 2048);
    } else {
      const uint16_t *q = reinterpret_cast<const uint16_t *>(stage + off[kc][f]);
      const uint2 x = tr_read(q);
      const uint2 y = tr_read(q + 4 * SPAN);
      return make_uint4(x.x, x.y, y.x, y.y);
    }
  }
};

// BM x BN tile per workgroup of NWV waves (WGM x WGN), STAGES-deep ring of
// 64-deep slabs, OCC workgroups per CU.  NWV = 8: two waves per SIMD in
// alternation (the ping-pong loop below).
// DUAL (NN only): two products X.B and X.B2 of the same output tile, B's
// and B2's slabs side by side in the stage (BN = twice the output width);
// each wave holds both accumulators of its output columns, so the SwiGLU
// epilogues pair them in registers.
template <int BM, int BN, int WGM, int WGN, int STAGES, int OCC, int LAYOUT, int EPI, bool KCAT, bool DUAL,
          int NWV>
__global__ void __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(OCC * NWV / 4, OCC * NWV / 4)))
gemm_k64_kernel(GemmParams pin) {
  GemmParams p = pin;
  static_assert(WGM * WGN == NWV && (NWV == 4 || (NWV == 8 && STAGES == 2 && OCC == 1)), "waves");
  static_assert(!DUAL || (LAYOUT == LAY_NN && !KCAT), "dual products are NN");
  constexpr int BNO = DUAL ? BN / 2 : BN;  // output tile width
  constexpr int WTM = BM / WGM, WTNO = BNO / WGN;
  constexpr int TM = WTM / 16, TNO = WTNO / 16, TN = DUAL ? 2 * TNO : TNO;
  constexpr bool AK = LAYOUT != LAY_TN;  // A stored k-contiguous
  constexpr bool BK = LAYOUT == LAY_NT;  // B stored k-contiguous
  constexpr int A_EL = BM * LBK, B_EL = BN * LBK;
  constexpr int STAGE = A_EL + B_EL;  // elements
  constexpr int B2_OFF = BNO * LBK * 2;  // byte offset of B2's slab after B's (dual)
  using ADma = typename std::conditional<AK, KDma<BM, false, NWV>, NDma<BM, NWV>>::type;
  using BDma = typename std::conditional<BK, KDma<BNO, KCAT, NWV>, NDma<BNO, NWV>>::type;
  constexpr int LOADS = ADma::PER_WAVE + (DUAL ? 2 : 1) * BDma::PER_WAVE;  // DMA ops per wave per slab
  static_assert(STAGES >= 2 && LOADS * STAGES < 64, "pipeline depth");

  // epilogue staging: the finished tile goes through LDS (the ring is idle
  // by then) and leaves as 16-byte chunks of consecutive rows
  constexpr int LDS_CAP = 160 * 1024 / OCC;
  constexpr int OES = EPI == EPI_STORE_F32 ? 4 : 2;  // output element bytes
  constexpr int SROW = BNO * OES + 16;              // staged row bytes (16-byte pad)
  constexpr bool STAGED = (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_STORE_F32 || EPI == EPI_SWIGLU) &&
                          BM * SROW <= LDS_CAP;
  constexpr int SR3 = BNO * 2 + 16;
  constexpr bool BWD = EPI == EPI_GELU_BWD || EPI == EPI_SWIGLU_BWD;
  constexpr bool STAGED3 = BWD && 2 * BM * SR3 <= LDS_CAP;
  static_assert(!BWD || STAGED3, "the backward epilogues are staged");
  static_assert(DUAL == (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD), "SwiGLU epilogues need both products");
  constexpr int RING_B = STAGES * STAGE * 2;
  // GELU backward on 128 x 128 tiles of four waves: the per-row-tile column
  // sums of dZ (db1) reduce through a [16][BNO] fp32 area after the staging
  constexpr bool CSUM = EPI == EPI_GELU_BWD && BM == 128 && BNO == 128 && NWV == 4;
  constexpr int CSUM_B = CSUM ? 16 * BNO * 4 : 0;
  constexpr int STG_B = STAGED ? BM * SROW : (STAGED3 ? 2 * BM * SR3 + CSUM_B : 0);
  static_assert(RING_B <= LDS_CAP && STG_B <= LDS_CAP, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[RING_B > STG_B ? RING_B : STG_B];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int M = p.M, N = p.N;
  const int nk = p.K / LBK;
  int tm, tn;
  tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BNO;

  const uint16_t *Ag = static_cast<const uint16_t *>(p.A);
  const uint16_t *Bg = static_cast<const uint16_t *>(p.B);
  if constexpr (LAYOUT == LAY_TN) {
    // split-K: grid row y = g zsplit + z takes K rows [z K, (z+1) K) of
    // product g (g = 1: A2^T B2) and writes partial y
    const int y = blockIdx.y;
    const int g = y >= p.zsplit ? 1 : 0;
    const int z = y - g * p.zsplit;
    if (g) {
      Ag = static_cast<const uint16_t *>(p.A2);
      p.lda = p.lda2;
      Bg = static_cast<const uint16_t *>(p.B2);
      p.ldb = p.ldb2;
    }
    Ag += (int64_t)z * p.K * p.lda;
    Bg += (int64_t)z * p.K * p.ldb;
    p.C = static_cast<float *>(p.C) + (int64_t)y * p.zstride;
  }
  // wave-uniform slab bases: k-type operands advance LBK elements per slab,
  // m/n-type ones LBK rows
  const uint16_t *Ab = AK ? Ag + (int64_t)m0 * p.lda : Ag + m0;
  const uint16_t *Bb = BK ? Bg + (int64_t)n0 * p.ldb : Bg + n0;
  const uint16_t *B2b = KCAT   ? static_cast<const uint16_t *>(p.B2) + (int64_t)n0 * p.ldb2
                        : DUAL ? static_cast<const uint16_t *>(p.B2) + n0
                               : nullptr;
  const int64_t astep = AK ? LBK : (int64_t)LBK * p.lda;
  const int64_t bstep = BK ? LBK : (int64_t)LBK * p.ldb;
  const int64_t b2step = (int64_t)LBK * p.ldb2;  // dual

  const int dw = wave;  // every wave issues its share of each slab's DMA
  ADma da;
  BDma db, db2;
  if constexpr (AK) da.init(p.lda, 0, m0, M, dw, lane);
  else da.init(p.lda, m0, M, dw, lane);
  if constexpr (BK) db.init(p.ldb, p.ldb2, n0, N, dw, lane);
  else db.init(p.ldb, n0, N, dw, lane);
  if constexpr (DUAL) db2.init(p.ldb2, n0, N, dw, lane);

  const uint32_t sbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(TP_AS3 const void *)smem);
  auto issue = [&](int kt, int stage) {
    const uint32_t base = sbase + stage * (STAGE * 2);
    if constexpr (AK) da.issue(Ab + kt * astep, false, base, dw);
    else da.issue(Ab + kt * astep, base, dw);
    if constexpr (BK) {
      const int k0 = kt * LBK;
      const bool second = KCAT && k0 >= p.K1;
      db.issue(second ? B2b + (k0 - p.K1) : Bb + k0, second, base + A_EL * 2, dw);
    } else {
      db.issue(Bb + kt * bstep, base + A_EL * 2, dw);
      if constexpr (DUAL) db2.issue(B2b + kt * b2step, base + A_EL * 2 + B2_OFF, dw);
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  FragAddr<AK, BM, WTM> fa;
  FragAddr<BK, BNO, WTNO> fb;
  fa.init(0, wm * WTM, lane);
  fb.init(A_EL * 2, wn * WTNO, lane);
  struct Frags {
    uint4 a[TM];
    uint4 b[TN];
  };
  auto load_chunk = [&](Frags &F, int stage, int kc) {
    const char *st = smem + stage * (STAGE * 2);
#pragma unroll
    for (int i = 0; i < TM; ++i) F.a[i] = fa.read(st, kc, i);
#pragma unroll
    for (int j = 0; j < TNO; ++j) F.b[j] = fb.read(st, kc, j);
    if constexpr (DUAL) {
#pragma unroll
      for (int j = 0; j < TNO; ++j) F.b[TNO + j] = fb.read(st + B2_OFF, kc, j);
    }
  };
  constexpr int N_DS = TM * (AK ? 1 : 2) + TN * (BK ? 1 : 2);
  constexpr int N_MFMA = TM * TN;
  auto mma = [&](const Frags &F) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(F.b[j], F.a[i], acc[i][j]);
  };
  // interleave the next chunk's LDS reads with this chunk's MFMAs.  Two
  // workgroups per CU: the reads go out early (one after each of the first
  // MFMAs) so that they have landed before the chunk ends; one workgroup per
  // CU: spread evenly.
  auto interleave = [&]() {
    if constexpr (OCC > 1 && N_MFMA > N_DS) {
#pragma unroll
      for (int q = 0; q < N_DS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, N_MFMA - N_DS, 0);
    } else {
#pragma unroll
      for (int q = 0; q < N_DS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, N_MFMA / N_DS > 0 ? N_MFMA / N_DS : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // first half of slab kt: MFMAs on chunk 0 (F0) while chunk 1 is read into F1
  auto half0 = [&](int kt, Frags &F0, Frags &F1) {
    load_chunk(F1, kt % STAGES, 1);
    mma(F0);
    interleave();
  };
  // second half of slab kt < nk-1: wait for slab kt+1, barrier (every wave
  // has read both chunks of slab kt), refill slab kt's stage with slab
  // kt+STAGES, MFMAs on chunk 1 while chunk 0 of slab kt+1 is read into F0
  auto half1 = [&](int kt, Frags &F1, Frags &F0) {
    if (kt + STAGES - 1 < nk) wait_vmcnt<LOADS * (STAGES - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (kt + STAGES < nk) issue(kt + STAGES, kt % STAGES);
    load_chunk(F0, (kt + 1) % STAGES, 0);
    mma(F1);
    interleave();
  };

  // activation backward with four waves: the epilogue's dH tile is loaded
  // (coalesced 16-byte row chunks, DHE per thread) during the main loop
  constexpr bool DH_EARLY = STAGED3 && NWV == 4 && STAGES == 2;
  constexpr int DH_CPR = BNO * 2 / 16;
  constexpr int DHE = DH_EARLY ? (BM * DH_CPR + NWV * 64 - 1) / (NWV * 64) : 1;
  uint4 dhe[DHE];
  auto load_dh_early = [&]() {
    if constexpr (DH_EARLY) {
#pragma unroll
      for (int k = 0; k < DHE; ++k) {
        const int c = (int)threadIdx.x + k * NWV * 64;
        const int rl = c / DH_CPR, cc = c % DH_CPR;
        const int row = m0 + rl, col = n0 + cc * 8;
        dhe[k] = make_uint4(0u, 0u, 0u, 0u);
        if (c < BM * DH_CPR && row < M && col < N)
          dhe[k] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.D) + (int64_t)row * p.ldd + col);
      }
    }
  };
  bool dh_loaded = false;

  if constexpr (NWV == 4) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nk) issue(s, s);
    if (nk >= STAGES) wait_vmcnt<LOADS * (STAGES - 1)>();
    else wait_vmcnt<0>();
    __syncthreads();
    Frags F0, F1;
    load_chunk(F0, 0, 0);
    if constexpr (DH_EARLY) {
      // the dH loads go out right after the last slab's DMA (issued in
      // half1(nk - 3)) and are waited for with it in half1(nk - 2): their
      // latency passes under the last slabs' MFMAs instead of opening the
      // epilogue
      int kt = 0;
      if (nk >= 3) {
        for (; kt < nk - 3; ++kt) {
          half0(kt, F0, F1);
          half1(kt, F1, F0);
        }
        half0(kt, F0, F1);
        half1(kt, F1, F0);
        load_dh_early();
        dh_loaded = true;
        ++kt;
      }
      for (; kt < nk - 1; ++kt) {
        half0(kt, F0, F1);
        half1(kt, F1, F0);
      }
    } else {
      for (int kt = 0; kt < nk - 1; ++kt) {
        half0(kt, F0, F1);
        half1(kt, F1, F0);
      }
    }
    half0(nk - 1, F0, F1);
    mma(F1);
  } else {
    // Ping-pong: waves w and w + 4 share a SIMD.  Group 0 (waves 0..3)
    // starts one phase ahead of group 1, and every phase ends at a
    // workgroup barrier, so while one wave of a SIMD runs the MFMAs of a
    // 32-deep chunk (its fragments already in registers) the other reads
    // its fragments of the next chunk from LDS.  Chunk c = 2 kt + h is read
    // in phase 2c by group 0 and 2c + 1 by group 1.  Each wave issues an
    // eighth of every slab's DMA at the start of its read phase of the
    // slab's first chunk: slab kt + 1 goes into the stage of slab kt - 1 in
    // phases 4 kt (group 0) and 4 kt + 1 (group 1) -- slab kt - 1 was last
    // read in phase 4 kt - 1 and every reader waited for its reads before
    // that phase's barrier -- and every wave waits for its share before the
    // barrier that ends phase 4 kt + 3.  (Issuing a whole slab from one
    // group stalled that group's read phase behind the DMA queue: 10%
    // slower; issuing inside the MFMA phases stalled the MFMAs: 7%.)
    const bool g0 = wave < NW;
    issue(0, 0);
    if (nk > 1) {
      issue(1, 1);
      wait_vmcnt<LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    phase_barrier();
    if (!g0) phase_barrier();  // group 1 one phase behind
    Frags F;
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0 && kt >= 1 && kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
        load_chunk(F, kt & 1, h);
        if (h == 1 && !g0 && kt + 1 < nk) wait_vmcnt<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        phase_barrier();
        mma(F);
        if (h == 1 && g0 && kt + 1 < nk) wait_vmcnt<0>();
        phase_barrier();
      }
    }
    if (g0) phase_barrier();  // as many barriers as group 1
  }

  // ---- epilogue: lane holds C[row][col .. col+3] of every 16x16 tile
  const int g = lane >> 4, l16 = lane & 15;
  if constexpr (STAGED) {
    using OutT = typename std::conditional<EPI == EPI_STORE_F32, float, uint16_t>::type;
    constexpr int CPR = BNO * OES / 16;  // 16-byte chunks per tile row
    float bv[TNO][4];
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
      const int col = n0 + wn * WTNO + j * 16 + g * 4;
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
      for (int j = 0; j < TNO; ++j) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][r] + bv[j][r];
          if constexpr (EPI == EPI_GELU) v[r] = gelu_f(v[r]);
          if constexpr (EPI == EPI_SWIGLU) v[r] = silu_f(v[r]) * acc[i][DUAL ? TNO + j : j][r];
        }
        char *dst = smem + (wm * WTM + i * 16 + l16) * SROW + (wn * WTNO + j * 16 + g * 4) * OES;
        store4(reinterpret_cast<OutT *>(dst), v);
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < BM * CPR; c += NWV * 64) {
      const int rl = c / CPR, cc = c % CPR;
      const int row = m0 + rl, col = n0 + cc * (16 / OES);
      if (row < M && col < N)
        store16_wt(static_cast<OutT *>(p.C) + (int64_t)row * p.ldc + col, smem + rl * SROW + cc * 16);
    }
    return;
  }
  if constexpr (STAGED3) {
    // activation backward: dH comes into LDS by coalesced 16-byte loads,
    // then the outputs (GELU: dZ, H; SwiGLU: dZg, H, dZu) are computed from
    // the accumulators and dH, written to LDS and stored as whole row
    // chunks (reading dH element by element between stores would wait on
    // every store before it): GELU's two in one pass (dZ to a second tile,
    // H over dH), SwiGLU's three one tile at a time
    constexpr int CPR = BNO * 2 / 16;
    constexpr int NOUT = EPI == EPI_SWIGLU_BWD ? 3 : 2;
    constexpr int DHN = (BM * CPR + NWV * 64 - 1) / (NWV * 64);  // dH chunks per thread
    char *dhs = smem;
    char *out = smem + BM * SR3;
    float *red = reinterpret_cast<float *>(smem + 2 * BM * SR3);  // [16][BNO] (CSUM)
    // every dH load of the thread is in flight before the first one is
    // waited on (one memory latency per tile, not one per chunk), unless
    // the main loop has loaded the tile already
    uint4 dhv[DHN];
    if constexpr (DH_EARLY) {
      static_assert(DHE == DHN, "dH chunks per thread");
      if (!dh_loaded) load_dh_early();
#pragma unroll
      for (int k = 0; k < DHN; ++k) dhv[k] = dhe[k];
    } else {
#pragma unroll
      for (int k = 0; k < DHN; ++k) {
        const int c = (int)threadIdx.x + k * NWV * 64;
        const int rl = c / CPR, cc = c % CPR;
        const int row = m0 + rl, col = n0 + cc * 8;
        dhv[k] = make_uint4(0u, 0u, 0u, 0u);
        if (c < BM * CPR && row < M && col < N)
          dhv[k] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.D) + (int64_t)row * p.ldd + col);
      }
    }
    if (p.bias != nullptr) {
      float bv[TNO][4];
      load_bias(static_cast<const uint16_t *>(p.bias), n0 + wn * WTNO + g * 4, N, bv);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TNO; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] += bv[j][r];
    }
    __syncthreads();  // every wave is done reading the ring
#pragma unroll
    for (int k = 0; k < DHN; ++k) {
      const int c = (int)threadIdx.x + k * NWV * 64;
      if (c < BM * CPR) *reinterpret_cast<uint4 *>(dhs + (c / CPR) * SR3 + (c % CPR) * 16) = dhv[k];
    }
    __syncthreads();
    if constexpr (EPI == EPI_GELU_BWD) {
      // one pass: Phi(z) and phi(z) come from a single erf evaluation and
      // give both dZ = dH (Phi + z phi) (to `out`) and H = z Phi (over its
      // own dH, which this lane alone reads)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TNO; ++j) {
          const int off = (wm * WTM + i * 16 + l16) * SR3 + (wn * WTNO + j * 16 + g * 4) * 2;
          float dh[4], dz[4], h[4];
          load4(reinterpret_cast<const uint16_t *>(dhs + off), dh);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc[i][j][r];
            const PhiResult f = normal_cdf_pdf(z);
            dz[r] = dh[r] * fmaf(z, f.pdf, f.phi_cdf);
            h[r] = z * f.phi_cdf;
          }
          store4(reinterpret_cast<uint16_t *>(out + off), dz);
          store4(reinterpret_cast<uint16_t *>(dhs + off), h);
        }
      }
      __syncthreads();
      if constexpr (CSUM) {
        // db1's share of this tile: thread (row group rg, 8-column chunk
        // cc) adds the stored dZ values of rows rg, rg + 16, ... in order,
        // then (after a barrier) the 16 row groups are added in order
        if (p.colsum != nullptr) {
          const int cc = threadIdx.x & 15, rg = threadIdx.x >> 4;
          const int rows = min(BM, M - m0);
          float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < BM / 16; ++k) {
            const int rl = rg + 16 * k;
            if (rl < rows) {
              const uint4 v = *reinterpret_cast<const uint4 *>(out + rl * SR3 + cc * 16);
              const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                cs[2 * q] += bf2f((uint16_t)(w[q] & 0xffffu));
                cs[2 * q + 1] += bf2f((uint16_t)(w[q] >> 16));
              }
            }
          }
          *reinterpret_cast<f32x4_t *>(red + rg * BNO + cc * 8) = (f32x4_t){cs[0], cs[1], cs[2], cs[3]};
          *reinterpret_cast<f32x4_t *>(red + rg * BNO + cc * 8 + 4) = (f32x4_t){cs[4], cs[5], cs[6], cs[7]};
        }
      }
      // dZ -> C, H -> C2
      for (int c = threadIdx.x; c < BM * CPR; c += NWV * 64) {
        const int rl = c / CPR, cc = c % CPR;
        const int row = m0 + rl, col = n0 + cc * 8;
        if (row < M && col < N) {
          store16_wt(static_cast<uint16_t *>(p.C) + (int64_t)row * p.ldc + col, out + rl * SR3 + cc * 16);
          store16_wt(static_cast<uint16_t *>(p.C2) + (int64_t)row * p.ldc2 + col, dhs + rl * SR3 + cc * 16);
        }
      }
      if constexpr (CSUM) {
        if (p.colsum != nullptr) {
          __syncthreads();
          if ((int)threadIdx.x < BNO) {
            const int col = n0 + (int)threadIdx.x;
            if (col < N) {
              float t = red[threadIdx.x];
#pragma unroll
              for (int r = 1; r < 16; ++r) t += red[r * BNO + threadIdx.x];
              p.colsum[(int64_t)tm * N + col] = t;
            }
          }
        }
      }
    } else {
    // SwiGLU: the three outputs one after the other through `out`
#pragma unroll
    for (int which = 0; which < NOUT; ++which) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TNO; ++j) {
          const int off = (wm * WTM + i * 16 + l16) * SR3 + (wn * WTNO + j * 16 + g * 4) * 2;
          float dh[4], o[4];
          load4(reinterpret_cast<const uint16_t *>(dhs + off), dh);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // z = gate pre-activation, u = up projection
            const float z = acc[i][j][r];
            const float u = acc[i][DUAL ? TNO + j : j][r];
            const float sg = sigmoid_f(z);
            const float sl = z * sg;
            o[r] = which == 0 ? dh[r] * u * (sg * (1.0f + z * (1.0f - sg))) : (which == 1 ? sl * u : dh[r] * sl);
          }
          store4(reinterpret_cast<uint16_t *>(out + off), o);
        }
      }
      __syncthreads();
      // dZg -> C, H -> C2, dZu -> C3
      void *C = which == 0 ? p.C : (which == 1 ? p.C2 : p.C3);
      const int64_t ldc = which == 0 ? p.ldc : (which == 1 ? p.ldc2 : p.ldc3);
      for (int c = threadIdx.x; c < BM * CPR; c += NWV * 64) {
        const int rl = c / CPR, cc = c % CPR;
        const int row = m0 + rl, col = n0 + cc * 8;
        if (row < M && col < N)
          store16_wt(static_cast<uint16_t *>(C) + (int64_t)row * ldc + col, out + rl * SR3 + cc * 16);
      }
      __syncthreads();
    }
    }
    return;
  }
  // direct stores (fp32 tiles too large to stage)
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = m0 + wm * WTM + i * 16 + l16;
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
      const int col = n0 + wn * WTNO + j * 16 + g * 4;
      if (row >= M || col >= N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      const int ju = DUAL ? TNO + j : j;
      const float u[4] = {acc[i][ju][0], acc[i][ju][1], acc[i][ju][2], acc[i][ju][3]};
      epilogue4<uint16_t, EPI>(p, row, col, v, u);
    }
  }
}

// ---------------------------------------------------------------- host side
template <int BM, int BN, int WGM, int WGN, int STAGES, int OCC, int LAYOUT, int EPI, bool KCAT,
          bool DUAL = false, int NWV = 4>
static hipError_t run(const GemmArgs &a, hipStream_t s) {
  constexpr int BNO = DUAL ? BN / 2 : BN;
  GemmParams p;
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
  p.tiles_n = (int)((a.N + BNO - 1) / BNO);
  p.zstride = a.zstride;
  p.A2 = a.A2; p.lda2 = a.lda2;
  p.zsplit = a.splits;
  p.colsum = nullptr;
  if constexpr (EPI == EPI_GELU_BWD && BM == 128 && BNO == 128 && NWV == 4) {
    if (a.colsum != nullptr && a.splits * a.groups == 1) {
      p.colsum = a.colsum;
      if (a.colsum_tiles != nullptr) *a.colsum_tiles = p.tiles_m;
    }
  }
  hipLaunchKernelGGL((gemm_k64_kernel<BM, BN, WGM, WGN, STAGES, OCC, LAYOUT, EPI, KCAT, DUAL, NWV>),
                     dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)(a.splits * a.groups)), dim3(NWV * 64), 0, s,
                     p);
  return hipGetLastError();
}

static int64_t cus() {
  thread_local int cached_dev = -1, cached_n = 0;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev == cached_dev) return cached_n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  cached_dev = dev;
  cached_n = n;
  return n;
}

// The output columns [c0, c0 + nc) of a single product: B (and the second
// K source), C and the bias shifted by c0 columns (B's columns are its rows
// when it is stored [N x K]).
template <int LAYOUT, int EPI>
static GemmArgs single_cols(const GemmArgs &a, int64_t c0, int64_t nc) {
  constexpr size_t CE = EPI == EPI_STORE_F32 ? 4 : 2;  // output / bias element bytes
  GemmArgs b = a;
  b.N = nc;
  b.B = static_cast<const uint16_t *>(a.B) + (LAYOUT == LAY_NT ? c0 * a.ldb : c0);
  if (a.kcat) b.B2 = static_cast<const uint16_t *>(a.B2) + c0 * a.ldb2;  // NT: rows are columns
  b.C = static_cast<char *>(a.C) + c0 * CE;
  if (a.bias != nullptr) b.bias = static_cast<const char *>(a.bias) + c0 * CE;
  return b;
}

// Launch rounds of a plan, in units of a round of 256 x 256 tiles: a CU runs
// a pair of 128 x 128 tiles (half a 256 x 256 tile's work) in about 0.62 of
// a 256 x 256 tile's time (measured on 4096 x 3584 x 8192 and
// 8192 x 3584 x 4096 products); 128 x 128 tiles spread evenly over the two
// slots of every CU (counted in half rounds), while the last round of
// 256 x 256 tiles may leave CUs idle.  A second launch costs ~0.17.
static double plan_cost(int64_t big_tiles, int64_t small_tiles, int64_t n) {
  const double big = (double)((big_tiles + n - 1) / n);
  const double small = 0.5 * (double)((small_tiles + n - 1) / n);  // pair rounds, half-round steps
  return big + 0.62 * small + (big_tiles > 0 && small_tiles > 0 ? 0.17 : 0.0);
}

// 256 x 256 tiles: eight waves in ping-pong
template <int LAYOUT, int EPI, bool KCAT>
static hipError_t run_big(const GemmArgs &a, hipStream_t s) {
  return run<256, 256, 2, 4, 2, 1, LAYOUT, EPI, KCAT, false, 8>(a, s);
}

// 256 x 256 tiles (one workgroup per CU) for the leading c column-tiles and
// 128 x 128 tiles (two per CU) for the rest, c chosen by plan_cost (8192 x
// 3072 x 4096: 183 us with small tiles only, 197 us large only, 176 us with
// 8 of 12 column-tiles large).  The activation epilogues stay on 128 x 128
// tiles, where the other workgroup of the CU hides them; split-K and
// grouped products use one tile size.
template <int LAYOUT, int EPI, bool KCAT>
static hipError_t pick(const GemmArgs &a, hipStream_t s) {
  const int64_t n = cus();
  const int64_t tmb = (a.M + 255) / 256, tms = (a.M + 127) / 128;
  const int64_t tnb = (a.N + 255) / 256;
  constexpr bool BIG_OK = EPI == EPI_STORE || EPI == EPI_STORE_F32;
  if constexpr (BIG_OK) {
    const int64_t z = (int64_t)a.splits * a.groups;
    int64_t best_c = 0;
    double best = 1e30;
    const int64_t cmax = z > 1 ? 0 : tnb - 1;  // split / grouped products: no column split
    for (int64_t c = 0; c <= tnb; ++c) {
      if (c > cmax && c < tnb) continue;
      const int64_t rest = std::max<int64_t>(a.N - c * 256, 0);
      const double cost = plan_cost(tmb * c * z, tms * ((rest + 127) / 128) * z, n);
      if (cost < best - 1e-9) {
        best = cost;
        best_c = c;
      }
    }
    if (best_c >= tnb) return run_big<LAYOUT, EPI, KCAT>(a, s);
    if (best_c > 0) {
      const int64_t c0 = best_c * 256;
      const hipError_t e = run_big<LAYOUT, EPI, KCAT>(single_cols<LAYOUT, EPI>(a, 0, c0), s);
      if (e != hipSuccess) return e;
      return run<128, 128, 2, 2, 2, 2, LAYOUT, EPI, KCAT>(single_cols<LAYOUT, EPI>(a, c0, a.N - c0), s);
    }
  }
  return run<128, 128, 2, 2, 2, 2, LAYOUT, EPI, KCAT>(a, s);
}

// The output columns [c0, c0 + nc) of a dual (bf16, NN) product: the
// weights, outputs, epilogue input and bias shifted by c0 columns.
static GemmArgs dual_cols(const GemmArgs &a, int64_t c0, int64_t nc) {
  GemmArgs b = a;
  b.N = nc;
  auto sh = [c0](const void *q) { return q == nullptr ? nullptr : static_cast<const uint16_t *>(q) + c0; };
  auto shm = [c0](void *q) { return q == nullptr ? nullptr : static_cast<uint16_t *>(q) + c0; };
  b.B = sh(a.B);
  b.B2 = sh(a.B2);
  b.bias = sh(a.bias);
  b.D = sh(a.D);
  b.C = shm(a.C);
  b.C2 = shm(a.C2);
  b.C3 = shm(a.C3);
  return b;
}

// Dual (SwiGLU) products: 256 x 128 output tiles (a 256 x 256 stage with
// both weight slabs, one workgroup per CU) and 128 x 128 ones (one per CU
// too, half the work per tile).  The leading c column-tiles take the large
// tiles and the rest the small ones, with c chosen to minimise the number
// of rounds over the CUs, a large-tile round costing about 1.6 small-tile
// rounds (SwiGLU shard, 8192 x 3584 x 4096: 24 of the 28 column-tiles
// large, i.e. three whole rounds of them, 309-323 us, and one round of
// small ones, 72 us; with four waves per workgroup 397 us large tiles
// only, 428 us small ones, 375 us split).
template <int EPI>
static hipError_t pick_dual(const GemmArgs &a, hipStream_t s) {
  const int64_t n = cus();
  const int64_t tmb = (a.M + 255) / 256, tms = (a.M + 127) / 128, tn = (a.N + 127) / 128;
  auto rounds = [n](int64_t tiles) { return (tiles + n - 1) / n; };
  int64_t best_c = tn;
  double best = 1e30;
  for (int64_t c = tn; c >= 0; --c) {
    const double cost = 1.6 * (double)rounds(tmb * c) + (double)rounds(tms * (tn - c)) +
                        (c > 0 && c < tn ? 0.25 : 0.0);  // a second launch
    if (cost < best - 1e-9) {
      best = cost;
      best_c = c;
    }
  }
  const int64_t c0 = std::min(best_c * 128, a.N);
  if (c0 > 0) {
    const hipError_t e = run<256, 256, 2, 4, 2, 1, LAY_NN, EPI, false, true, 8>(c0 < a.N ? dual_cols(a, 0, c0) : a, s);
    if (e != hipSuccess || c0 == a.N) return e;
  }
  return run<128, 256, 2, 4, 2, 1, LAY_NN, EPI, false, true, 8>(c0 > 0 ? dual_cols(a, c0, a.N - c0) : a, s);
}

}  // namespace k64

hipError_t launch_gemm_k64(const GemmArgs &a, hipStream_t s) {
  using namespace k64;
  if (a.dtype != DT_BF16 || a.K <= 0 || a.K % LBK != 0) return hipErrorNotSupported;
  if (a.dual && (a.layout != LAY_NN || a.kcat || (a.epi != EPI_SWIGLU && a.epi != EPI_SWIGLU_BWD)))
    return hipErrorNotSupported;
  if (a.kcat && (a.K1 % LBK != 0 || a.layout != LAY_NT)) return hipErrorNotSupported;
  if (a.M < 8 || a.N < 8) return hipErrorNotSupported;
  // the DMA offsets are 32-bit (up to 256 rows of a k-contiguous operand or
  // 64 rows of an m/n-contiguous one, relative to the slab base)
  if (a.groups != 1 && (a.groups != 2 || a.layout != LAY_TN || a.A2 == nullptr || a.B2 == nullptr))
    return hipErrorInvalidValue;
  const int64_t ld_max = std::max(std::max(a.lda, a.groups > 1 ? a.lda2 : (int64_t)0),
                                  std::max(a.ldb, a.kcat || a.dual || a.groups > 1 ? a.ldb2 : (int64_t)0));
  if (ld_max * 2 * 256 >= ((int64_t)1 << 32)) return hipErrorNotSupported;
  // small products stay on the other kernels (more, smaller tiles)
  if (((a.M + 127) / 128) * ((a.N + 127) / 128) * a.splits * a.groups < 128) return hipErrorNotSupported;
  if ((a.splits > 1 || a.groups > 1) && (a.layout != LAY_TN || a.epi != EPI_STORE_F32)) return hipErrorInvalidValue;
  switch (a.layout) {
    case LAY_NN:
      if (a.dual) {
        if (a.epi == EPI_SWIGLU) return pick_dual<EPI_SWIGLU>(a, s);
        return pick_dual<EPI_SWIGLU_BWD>(a, s);
      }
      switch (a.epi) {
        case EPI_STORE: return pick<LAY_NN, EPI_STORE, false>(a, s);
        case EPI_STORE_F32: return pick<LAY_NN, EPI_STORE_F32, false>(a, s);
        case EPI_GELU: return pick<LAY_NN, EPI_GELU, false>(a, s);
        case EPI_GELU_BWD: return pick<LAY_NN, EPI_GELU_BWD, false>(a, s);
        default: return hipErrorNotSupported;
      }
    case LAY_NT:
      if (a.kcat) {
        if (a.epi == EPI_STORE_F32) return pick<LAY_NT, EPI_STORE_F32, true>(a, s);
        return hipErrorNotSupported;
      }
      if (a.epi == EPI_STORE) return pick<LAY_NT, EPI_STORE, false>(a, s);
      if (a.epi == EPI_STORE_F32) return pick<LAY_NT, EPI_STORE_F32, false>(a, s);
      return hipErrorNotSupported;
    case LAY_TN:
      if (a.epi != EPI_STORE_F32) return hipErrorNotSupported;
      return pick<LAY_TN, EPI_STORE_F32, false>(a, s);
  }
  return hipErrorNotSupported;
}

}  // namespace tpcol
