// Tiled MFMA GEMM for gfx950 with fused tensor-parallel epilogues.
//
//   C[M x N] = A[M x K] . B[K x N]   (fp32 accumulate)
//
// One kernel template serves every GEMM of the shard hot path:
//   NN  column-parallel X.W_i (+GELU / SwiGLU / none), row-parallel partial
//       X_i.W_i, QKV projection, and the backward recompute with the
//       activation-derivative epilogue;
//   NT  dgrad dY.W2_i^T and dZ.W1_i^T (the K-concatenated form covers
//       dZg.Wg^T + dZu.Wu^T in one pass);
//   TN  wgrad H^T.dY and X^T.dZ.
//
// Data path per workgroup (256 threads = 4 wave64):
//   global --16-byte vector loads--> registers --> LDS tile [rows][BK+pad]
//   (k contiguous; operands stored with the other dimension contiguous are
//   transposed in registers on the way, 8x8 bf16 / 4x4 fp32 blocks) -->
//   ds_read_b128 fragments --> v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4f32).
// The LDS tile is double-buffered: the next K-slab's global loads are in
// flight while the current slab is multiplied, and one barrier per slab
// separates reuse.  The MFMA is issued with B as the first operand so that
// each lane ends up holding 4 consecutive output columns of one row, which
// the epilogue writes as one vector.  The pre-activation never leaves
// registers.
//
// Workgroup -> tile mapping is XCD-aware: the hardware deals consecutive
// workgroup ids round-robin to the 8 XCDs, so ids are re-mapped so that each
// XCD receives a contiguous run of tiles, which are then walked in groups of
// GROUP_M tile-rows; neighbouring tiles share A rows / B columns in that
// XCD's L2.
#include <type_traits>

#include "gemm_common.hpp"

namespace tpcol {

// rows x BK slab, k contiguous in global memory -> LDS [rows][LDK].
template <typename T, int ROWS, int BK, int NT>
struct DirectTile {
  static constexpr int VW = Elem<T>::VW;
  static constexpr int VPR = BK / VW;
  static constexpr int NV = ROWS * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  uint4 r[PER];

  template <bool KCAT>
  __device__ __forceinline__ void load(const T *__restrict__ g, int64_t ld, const T *__restrict__ g2,
                                       int64_t ld2, int K1, int row0, int rows_lim, int k0, int k_lim,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      r[i] = make_uint4(0u, 0u, 0u, 0u);
      if ((NV % NT == 0) || v < NV) {
        const int row = v / VPR, kv = v % VPR;
        const int gr = row0 + row, gk = k0 + kv * VW;
        if (gr < rows_lim && gk < k_lim) {
          const T *src = (KCAT && gk >= K1) ? g2 + (int64_t)gr * ld2 + (gk - K1)
                                            : g + (int64_t)gr * ld + gk;
          r[i] = *reinterpret_cast<const uint4 *>(src);
        }
      }
    }
  }

  template <int LDK>
  __device__ __forceinline__ void store(T *s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * NT;
      if ((NV % NT == 0) || v < NV) {
        const int row = v / VPR, kv = v % VPR;
        *reinterpret_cast<uint4 *>(s + row * LDK + kv * VW) = r[i];
      }
    }
  }
};

// BK x cols slab with cols contiguous in global memory -> LDS [cols][LDK]
// (k contiguous): each thread moves VW x VW blocks and transposes them in
// registers.
template <typename T, int COLS, int BK, int NT>
struct TransTile {
  static constexpr int VW = Elem<T>::VW;
  static constexpr int CB = COLS / VW;
  static constexpr int KB = BK / VW;
  static constexpr int NU = CB * KB;
  static constexpr int PER = (NU + NT - 1) / NT;
  uint4 r[PER][VW];

  __device__ __forceinline__ void load(const T *__restrict__ g, int64_t ld, int col0, int col_lim,
                                       int k0, int k_lim, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      const bool valid = (NU % NT == 0) || u < NU;
      const int cb = u % CB, kb = u / CB;
      const int gc = col0 + cb * VW;
#pragma unroll
      for (int rr = 0; rr < VW; ++rr) {
        const int gk = k0 + kb * VW + rr;
        r[i][rr] = make_uint4(0u, 0u, 0u, 0u);
        if (valid && gc < col_lim && gk < k_lim)
          r[i][rr] = *reinterpret_cast<const uint4 *>(g + (int64_t)gk * ld + gc);
      }
    }
  }

  template <int LDK>
  __device__ __forceinline__ void store(T *s, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (!((NU % NT == 0) || u < NU)) continue;
      const int cb = u % CB, kb = u / CB;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = u4_word(r[i][2 * q], c >> 1);
            const uint32_t hi = u4_word(r[i][2 * q + 1], c >> 1);
            w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *reinterpret_cast<uint4 *>(s + (cb * 8 + c) * LDK + kb * 8) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *reinterpret_cast<uint4 *>(s + (cb * 4 + c) * LDK + kb * 4) =
              make_uint4(u4_word(r[i][0], c), u4_word(r[i][1], c), u4_word(r[i][2], c),
                         u4_word(r[i][3], c));
        }
      }
    }
  }
};

template <typename T, int BM, int BN, int BK, int WGM, int WGN, int LAYOUT, int EPI, bool DUAL,
          bool KCAT>
__global__ void __launch_bounds__(WGM * WGN * 64) gemm_kernel(GemmParams p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int VW = Elem<T>::VW, KP = Elem<T>::KP, KSTEP = Elem<T>::KSTEP;
  constexpr int LDK = BK + VW;  // 16-byte row pad: conflict-free ds_read_b128 columns
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int STAGE = (BM + NB * BN) * LDK;
  constexpr bool AT = (LAYOUT == LAY_TN);
  constexpr bool BT = (LAYOUT == LAY_NT);
  using Frag = typename std::conditional<sizeof(T) == 2, uint4, float>::type;
  static_assert(BK % KSTEP == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) T smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int M = p.M, N = p.N, K = p.K;

  int tm, tn;
  tile_of_block(p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const T *__restrict__ Ag = static_cast<const T *>(p.A);
  const T *__restrict__ Bg = static_cast<const T *>(p.B);
  const T *__restrict__ B2g = static_cast<const T *>(p.B2);

  typename std::conditional<AT, TransTile<T, BM, BK, NT>, DirectTile<T, BM, BK, NT>>::type la;
  typename std::conditional<BT, DirectTile<T, BN, BK, NT>, TransTile<T, BN, BK, NT>>::type lb;
  typename std::conditional<DUAL, TransTile<T, BN, BK, NT>, DirectTile<T, 16, BK, NT>>::type lb2;

  auto load_slab = [&](int k0) {
    if constexpr (AT) la.load(Ag, p.lda, m0, M, k0, K, tid);
    else la.template load<false>(Ag, p.lda, nullptr, 0, 0, m0, M, k0, K, tid);
    if constexpr (BT) lb.template load<KCAT>(Bg, p.ldb, B2g, p.ldb2, p.K1, n0, N, k0, K, tid);
    else lb.load(Bg, p.ldb, n0, N, k0, K, tid);
    if constexpr (DUAL) lb2.load(B2g, p.ldb2, n0, N, k0, K, tid);
  };
  auto store_slab = [&](int buf) {
    T *As = smem + buf * STAGE;
    la.template store<LDK>(As, tid);
    lb.template store<LDK>(As + BM * LDK, tid);
    if constexpr (DUAL) lb2.template store<LDK>(As + (BM + BN) * LDK, tid);
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

  const int nk = (K + BK - 1) / BK;
  load_slab(0);
  store_slab(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slab((kt + 1) * BK);

    const T *As = smem + cur * STAGE;
    const T *Bs = As + BM * LDK;
    const T *B2s = As + (BM + BN) * LDK;
#pragma unroll
    for (int kc = 0; kc < BK / KSTEP; ++kc) {
      const int koff = kc * KSTEP + (lane >> 4) * KP;
      Frag a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const Frag *>(As + (wm * WTM + i * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const Frag *>(Bs + (wn * WTN + j * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(b[j], a[i], acc[i][j]);
      if constexpr (DUAL) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[j] = *reinterpret_cast<const Frag *>(B2s + (wn * WTN + j * 16 + (lane & 15)) * LDK + koff);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc2[i][j] = mfma16(b[j], a[i], acc2[i][j]);
      }
    }

    if (kt + 1 < nk) store_slab(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[row][col .. col+3] of every 16x16 tile
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = m0 + wm * WTM + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 16 + (lane >> 4) * 4;
      if (row >= M || col >= N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      float u[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DUAL) {
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = acc2[DUAL ? i : 0][DUAL ? j : 0][r];
      }
      epilogue4<T, EPI>(p, row, col, v, u);
    }
  }
}

// ---------------------------------------------------------------- host side
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int LAYOUT, int EPI, bool DUAL,
          bool KCAT>
static hipError_t run_gemm(const GemmArgs &a, hipStream_t s) {
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
  p.zstride = 0;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WGM, WGN, LAYOUT, EPI, DUAL, KCAT>), grid,
                     dim3(WGM * WGN * 64), 0, s, p);
  return hipGetLastError();
}

template <typename T, int LAYOUT, int EPI, bool DUAL, bool KCAT>
static hipError_t pick_tile(const GemmArgs &a, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    return run_gemm<T, 64, 64, 32, 2, 2, LAYOUT, EPI, DUAL, KCAT>(a, s);
  } else if constexpr (DUAL) {
    const int64_t tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (tiles >= 128) return run_gemm<T, 128, 128, 64, 2, 2, LAYOUT, EPI, DUAL, KCAT>(a, s);
    return run_gemm<T, 64, 64, 64, 2, 2, LAYOUT, EPI, DUAL, KCAT>(a, s);
  } else {
    const int64_t tiles = ((a.M + 255) / 256) * ((a.N + 127) / 128);
    if (tiles >= 128) return run_gemm<T, 256, 128, 64, 2, 2, LAYOUT, EPI, DUAL, KCAT>(a, s);
    return run_gemm<T, 64, 64, 64, 2, 2, LAYOUT, EPI, DUAL, KCAT>(a, s);
  }
}

template <typename T>
static hipError_t dispatch(const GemmArgs &a, hipStream_t s) {
  switch (a.layout) {
    case LAY_NN:
      if (a.dual) {
        if (a.epi == EPI_SWIGLU) return pick_tile<T, LAY_NN, EPI_SWIGLU, true, false>(a, s);
        if (a.epi == EPI_SWIGLU_BWD) return pick_tile<T, LAY_NN, EPI_SWIGLU_BWD, true, false>(a, s);
        return hipErrorInvalidValue;
      }
      switch (a.epi) {
        case EPI_STORE: return pick_tile<T, LAY_NN, EPI_STORE, false, false>(a, s);
        case EPI_STORE_F32: return pick_tile<T, LAY_NN, EPI_STORE_F32, false, false>(a, s);
        case EPI_GELU: return pick_tile<T, LAY_NN, EPI_GELU, false, false>(a, s);
        case EPI_GELU_BWD: return pick_tile<T, LAY_NN, EPI_GELU_BWD, false, false>(a, s);
        default: return hipErrorInvalidValue;
      }
    case LAY_NT:
      if (a.dual) return hipErrorInvalidValue;
      if (a.kcat) {
        if (a.epi == EPI_STORE_F32) return pick_tile<T, LAY_NT, EPI_STORE_F32, false, true>(a, s);
        return hipErrorInvalidValue;
      }
      if (a.epi == EPI_STORE) return pick_tile<T, LAY_NT, EPI_STORE, false, false>(a, s);
      if (a.epi == EPI_STORE_F32) return pick_tile<T, LAY_NT, EPI_STORE_F32, false, false>(a, s);
      return hipErrorInvalidValue;
    case LAY_TN:
      if (a.dual || a.kcat || a.epi != EPI_STORE_F32) return hipErrorInvalidValue;
      return pick_tile<T, LAY_TN, EPI_STORE_F32, false, false>(a, s);
  }
  return hipErrorInvalidValue;
}

// K-range splits for a bf16 TN fp32 product with scratch: enough that the
// workgroups of the tile configuration the LDS kernel picks (256 x 256 from
// 192 tiles up, else 128 x 256 from 128 tiles up, else 128 x 128) times the
// splits fill about one round of 256 CUs, each split at least 512 deep, the
// partials inside the scratch.
static int split_k_factor(const GemmArgs &a) {
  if (a.part == nullptr || a.layout != LAY_TN || a.epi != EPI_STORE_F32 || a.bias != nullptr || a.dual ||
      a.kcat || a.dtype != DT_BF16)
    return 1;
  const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int64_t t128x256 = ((a.M + 127) / 128) * ((a.N + 255) / 256);
  if (t256 >= 192) return 1;
  const int64_t tiles = t128x256 >= 128 ? t128x256 : ((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (tiles > 128) return 1;
  const size_t one = (size_t)a.M * (size_t)a.N * sizeof(float);
  int S = 1;
  while (S < 8 && tiles * 2 * S <= 256 && (size_t)(2 * S) * one <= a.part_bytes && a.K % (64 * S) == 0 &&
         a.K / (2 * S) >= 512)
    S *= 2;
  return S;
}

// bf16 products on the LDS-DMA kernels: 64-deep slabs where they apply,
// else 32-deep ones
static hipError_t launch_lds(const GemmArgs &a, hipStream_t s) {
  const hipError_t e = launch_gemm_k64(a, s);
  if (e != hipErrorNotSupported) return e;
  return launch_gemm_lds(a, s);
}

// Both weight gradients of a backward in one launch: K-range splits of the
// two products share the grid (rows [0, S) the first, [S, 2S) the second),
// so that narrow outputs fill two workgroups per CU, then one launch adds
// each product's partials in split order (and takes on the column sum cj,
// if given, in spare workgroups of that launch).
hipError_t launch_gemm_tn_pair(const GemmArgs &a0, const GemmArgs &a1, hipStream_t s, const ColsumJob *cj,
                               bool *cj_done) {
  if (cj_done != nullptr) *cj_done = false;
  auto separate = [&]() -> hipError_t {
    const hipError_t e = launch_gemm(a0, s);
    if (e != hipSuccess) return e;
    return launch_gemm(a1, s);
  };
  if (a0.M <= 0 || a0.N <= 0 || a0.dtype != DT_BF16 || a1.dtype != DT_BF16 || a0.layout != LAY_TN ||
      a1.layout != LAY_TN || a0.epi != EPI_STORE_F32 || a1.epi != EPI_STORE_F32 || a0.bias != nullptr ||
      a1.bias != nullptr || a0.M != a1.M || a0.N != a1.N || a0.K != a1.K || a0.part == nullptr || a0.N % 4)
    return separate();
  const int64_t tiles = ((a0.M + 127) / 128) * ((a0.N + 127) / 128);
  const size_t one = (size_t)a0.M * (size_t)a0.N * sizeof(float);
  // two workgroups per CU over 256 CUs, splits at least 512 deep, the
  // partials of both products inside the scratch
  int S = 1;
  while (S < 8 && 2 * tiles * 2 * S <= 512 && (size_t)(2 * 2 * S) * one <= a0.part_bytes &&
         a0.K % (64 * 2 * S) == 0 && a0.K / (2 * S) >= 512)
    S *= 2;
  if (S == 1) return separate();
  GemmArgs b = a0;
  b.splits = S;
  b.groups = 2;
  b.K = a0.K / S;
  b.C = a0.part;
  b.ldc = a0.N;
  b.zstride = a0.M * a0.N;
  b.A2 = a1.A; b.lda2 = a1.lda;
  b.B2 = a1.B; b.ldb2 = a1.ldb;
  const hipError_t e = launch_gemm_k64(b, s);
  if (e == hipErrorNotSupported) return separate();
  if (e != hipSuccess) return e;
  const float *parts[16];
  for (int z = 0; z < 2 * S; ++z) parts[z] = a0.part + (int64_t)z * b.zstride;
  const hipError_t e2 = launch_shard_sum_pair(a0.M, a0.N, S, parts, a0.N, static_cast<float *>(a0.C), a0.ldc,
                                              static_cast<float *>(a1.C), a1.ldc, s, cj);
  if (e2 == hipSuccess && cj != nullptr && cj_done != nullptr) *cj_done = true;
  return e2;
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.dtype == DT_BF16) {
    const int S = split_k_factor(a);
    if (S > 1) {
      GemmArgs b = a;
      b.splits = S;
      b.K = a.K / S;
      b.C = a.part;
      b.ldc = a.N;
      b.zstride = a.M * a.N;
      const hipError_t e = launch_lds(b, s);
      if (e == hipSuccess) {
        const float *parts[8];
        for (int z = 0; z < S; ++z) parts[z] = a.part + (int64_t)z * b.zstride;
        return launch_shard_sum(DT_F32, a.M, a.N, S, parts, a.N, nullptr, a.C, a.ldc, s);
      }
      if (e != hipErrorNotSupported) return e;
    }
    GemmArgs b = a;
    b.splits = 1;
    const hipError_t e = launch_lds(b, s);
    if (e != hipErrorNotSupported) return e;
    return dispatch<uint16_t>(a, s);
  }
  if (a.dtype == DT_F32) return dispatch<float>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace tpcol
