// Pieces shared by the two GEMM kernels (register-staged general kernel and
// the LDS-DMA kernel): kernel parameters, 4-wide loads/stores and the fused
// tensor-parallel epilogues.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

struct GemmParams {
  const void *A; int64_t lda;
  const void *B; int64_t ldb;
  const void *B2; int64_t ldb2;
  const void *bias;
  const void *D; int64_t ldd;
  void *C; int64_t ldc;
  void *C2; int64_t ldc2;
  void *C3; int64_t ldc3;
  int M, N, K, K1;  // K: depth of one K-range split
  int tiles_m, tiles_n;
  int64_t zstride;   // elements between split outputs (TN split-K only)
  // grouped TN split-K: grid rows [zsplit, 2 zsplit) compute A2^T B2
  const void *A2; int64_t lda2;
  int zsplit;
  // GELU-backward epilogue: per row-tile column sums of C ([tiles_m][N]
  // fp32, the bf16 values as stored), or NULL
  float *colsum;
};

template <typename T>
__device__ __forceinline__ void load4(const T *p, float v[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf2f((uint16_t)(u.x & 0xffffu)); v[1] = bf2f((uint16_t)(u.x >> 16));
    v[2] = bf2f((uint16_t)(u.y & 0xffffu)); v[3] = bf2f((uint16_t)(u.y >> 16));
  } else {
    const float4 f = *reinterpret_cast<const float4 *>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T *p, const float v[4]) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
  } else {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Workgroup -> output tile.  The hardware deals consecutive workgroup ids
// round-robin to the 8 XCDs; re-map so each XCD gets a contiguous run of
// tiles, then walk them in groups of GROUP_M tile-rows so that neighbouring
// tiles share A rows / B columns in that XCD's L2.
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int GROUP_M = 4;
  const int nblk = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, idx = b >> 3, base = nblk >> 3, rem = nblk & 7;
  const int lin = xcd * base + (xcd < rem ? xcd : rem) + idx;
  const int per_group = GROUP_M * tiles_n;
  const int group = lin / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in = lin - group * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Epilogue for output C[row][col .. col+3]; v = first accumulator, u = the
// second (dual GEMMs).  The pre-activation only lives in these registers.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue4(const GemmParams &p, int row, int col, float v[4],
                                          const float u[4]) {
  if (p.bias != nullptr) {
    float bv[4];
    if constexpr (EPI == EPI_STORE_F32) load4(static_cast<const float *>(p.bias) + col, bv);
    else load4(static_cast<const T *>(p.bias) + col, bv);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += bv[r];
  }
  const int64_t rowi = row;
  if constexpr (EPI == EPI_STORE) {
    store4(static_cast<T *>(p.C) + rowi * p.ldc + col, v);
  } else if constexpr (EPI == EPI_STORE_F32) {
    store4(static_cast<float *>(p.C) + rowi * p.ldc + col, v);
  } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = gelu_f(v[r]);
    store4(static_cast<T *>(p.C) + rowi * p.ldc + col, v);
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = silu_f(v[r]) * u[r];
    store4(static_cast<T *>(p.C) + rowi * p.ldc + col, v);
  } else if constexpr (EPI == EPI_GELU_BWD) {
    float dh[4], dz[4], hh[4];
    load4(static_cast<const T *>(p.D) + rowi * p.ldd + col, dh);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dz[r] = dh[r] * gelu_grad_f(v[r]);
      hh[r] = gelu_f(v[r]);
    }
    store4(static_cast<T *>(p.C) + rowi * p.ldc + col, dz);
    store4(static_cast<T *>(p.C2) + rowi * p.ldc2 + col, hh);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    float dh[4], dzg[4], dzu[4], hh[4];
    load4(static_cast<const T *>(p.D) + rowi * p.ldd + col, dh);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float g = v[r];
      const float sg = sigmoid_f(g);
      const float sl = g * sg;
      dzu[r] = dh[r] * sl;
      dzg[r] = dh[r] * u[r] * (sg * (1.0f + g * (1.0f - sg)));
      hh[r] = sl * u[r];
    }
    store4(static_cast<T *>(p.C) + rowi * p.ldc + col, dzg);
    store4(static_cast<T *>(p.C3) + rowi * p.ldc3 + col, dzu);
    store4(static_cast<T *>(p.C2) + rowi * p.ldc2 + col, hh);
  }
}

// Launchers of the LDS-DMA kernels (bf16; gemm_lds: K a multiple of 32,
// gemm_k64: K a multiple of 64, dual products NN only); each returns
// hipErrorNotSupported when the shape/layout is not covered so that the
// caller falls back to the next kernel.
hipError_t launch_gemm_lds(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_k64(const GemmArgs &a, hipStream_t s);

}  // namespace tpcol
