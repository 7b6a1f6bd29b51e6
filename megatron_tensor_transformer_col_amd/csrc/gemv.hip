// Decode-phase GEMV (M <= 16 tokens), weight-streaming and HBM-bound.
//
// In decode every request contributes one token, so a linear layer reads the
// whole weight once for 2*M*K*N flops: arithmetic intensity is about
// 2*M / bytes_per_param (parallelism survey post, Prefill-Decode 分离,
// Decode 阶段), ~16 flop/byte for 16 bf16 tokens, far below the ridge.  The
// kernel therefore optimises for bytes in flight, not for flops:
//   * a wave owns a 128-column strip (16 lanes x 8 columns, 16-byte loads)
//     and streams 4 x 32 rows of W with all 32 loads per lane issued before
//     the first use (32 KiB in flight per wave);
//   * the 8x8 bf16 blocks are transposed in registers and multiplied with a
//     16 x 32 slab of x on the matrix cores (16x16x32 bf16 MFMA), M padded
//     to 16 with zeros, so the VALU only does the transposes;
//   * 4 waves of a workgroup cover consecutive row ranges and are summed in
//     LDS; workgroups split K (grid.y) and write fp32 partials; the last
//     workgroup to finish a strip (device-scope arrival counter) adds the
//     partials in split order and applies the epilogue.  The activation is
//     applied only after the full K reduction, since GELU does not
//     distribute over a sum ("张量并行", 两个矩阵相乘: GELU(sum) != sum GELU).
// The arrival counters are reset by the last workgroup, so the counter region
// of the workspace is left zeroed for the next call.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int GV_COLS = 128;   // columns per strip
static constexpr int GV_WAVES = 4;    // waves per workgroup
static constexpr int GV_STEPS = 4;    // 32-row steps per wave
static constexpr int GV_ROWS_WG = GV_WAVES * GV_STEPS * 32;

// Workspace layout (fixed for every shape, so that calls of different shapes
// can share one buffer): [0, GV_COUNTER_BYTES) arrival counters, one per
// 128-column strip, kept at zero between calls; then the fp32 partials
// [splits][16][N].
static constexpr int64_t GV_MAX_STRIPS = 16384;
static constexpr size_t GV_COUNTER_BYTES = GV_MAX_STRIPS * sizeof(uint32_t);

static inline int64_t gv_splits(int64_t K) { return (K + GV_ROWS_WG - 1) / GV_ROWS_WG; }
static inline int64_t gv_strips(int64_t N) { return (N + GV_COLS - 1) / GV_COLS; }

size_t gemv_workspace(int64_t K, int64_t N) {
  if (gv_splits(K) <= 1) return 0;
  return GV_COUNTER_BYTES + (size_t)gv_splits(K) * 16 * (size_t)N * sizeof(float);
}

int64_t gemv_max_n() { return GV_MAX_STRIPS * GV_COLS; }

template <int EPI>
__device__ __forceinline__ void gv_epilogue(float v[8], const uint16_t *bias, int col, void *Y,
                                            int64_t ldy, int m) {
  if (bias != nullptr) {
    const uint4 b = *reinterpret_cast<const uint4 *>(bias + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] += bf2f((uint16_t)(u4_word(b, j >> 1) >> ((j & 1) * 16)));
  }
  if constexpr (EPI == EPI_STORE_F32) {
    float *y = static_cast<float *>(Y) + (int64_t)m * ldy + col;
    *reinterpret_cast<float4 *>(y) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(y + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    if constexpr (EPI == EPI_GELU) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = gelu_f(v[j]);
    }
    uint16_t *y = static_cast<uint16_t *>(Y) + (int64_t)m * ldy + col;
    *reinterpret_cast<uint4 *>(y) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                               pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  }
}

template <int EPI>
__global__ void __launch_bounds__(GV_WAVES * 64)
gemv_kernel(const uint16_t *__restrict__ X, int64_t ldx, int M, const uint16_t *__restrict__ W,
            int64_t ldw, int K, int N, const uint16_t *bias, void *Y, int64_t ldy,
            float *part, uint32_t *counters) {
  __shared__ __attribute__((aligned(16))) float red[GV_WAVES][16][GV_COLS];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int strip = blockIdx.x, split = blockIdx.y, nsplit = gridDim.y;
  const int c0 = strip * GV_COLS + l16 * 8;
  const int row0 = split * GV_ROWS_WG + wave * (GV_STEPS * 32);

  // ---- issue every load of this wave first
  uint4 wv[GV_STEPS][8];
  uint4 xv[GV_STEPS];
#pragma unroll
  for (int st = 0; st < GV_STEPS; ++st) {
    const int kb = row0 + st * 32 + g * 8;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int k = kb + rr;
      wv[st][rr] = make_uint4(0u, 0u, 0u, 0u);
      if (k < K && c0 < N) wv[st][rr] = *reinterpret_cast<const uint4 *>(W + (int64_t)k * ldw + c0);
    }
    xv[st] = make_uint4(0u, 0u, 0u, 0u);
    if (l16 < M && kb < K) xv[st] = *reinterpret_cast<const uint4 *>(X + (int64_t)l16 * ldx + kb);
  }

  // ---- transpose 8x8 blocks and multiply: acc[j] lane holds
  //      Y[m = 4g + r][strip*128 + l16*8 + j]
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < GV_STEPS; ++st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = u4_word(wv[st][2 * q], j >> 1);
        const uint32_t hi = u4_word(wv[st][2 * q + 1], j >> 1);
        w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      acc[j] = mfma16(xv[st], make_uint4(w[0], w[1], w[2], w[3]), acc[j]);
    }
  }

  // ---- sum the 4 waves in LDS
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float *dst = &red[wave][4 * g + r][l16 * 8];
    *reinterpret_cast<float4 *>(dst) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
  }
  __syncthreads();
  const int m = tid >> 4, cc = (tid & 15) * 8;
  const int col = strip * GV_COLS + cc;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = ((red[0][m][cc + j] + red[1][m][cc + j]) + red[2][m][cc + j]) + red[3][m][cc + j];

  if (nsplit == 1) {
    if (m < M && col < N) gv_epilogue<EPI>(v, bias, col, Y, ldy, m);
    return;
  }

  // ---- split-K: publish this workgroup's partial, last arrival finishes
  if (m < M && col < N) {
    float *pp = part + ((int64_t)split * 16 + m) * N + col;
    *reinterpret_cast<float4 *>(pp) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(pp + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[strip], 1u);
    s_last = (prev == (uint32_t)(nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (m < M && col < N) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float *pp = part + ((int64_t)sp * 16 + m) * N + col;
      const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(pp));
      const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(pp + 4));
      v[0] += a[0]; v[1] += a[1]; v[2] += a[2]; v[3] += a[3];
      v[4] += b[0]; v[5] += b[1]; v[6] += b[2]; v[7] += b[3];
    }
    gv_epilogue<EPI>(v, bias, col, Y, ldy, m);
  }
  if (tid == 0) counters[strip] = 0u;
}

hipError_t launch_gemv(const GemvArgs &a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 16 || a.dtype != DT_BF16) return hipErrorInvalidValue;
  const int64_t splits = gv_splits(a.K < 1 ? 1 : a.K);
  const dim3 grid((unsigned)gv_strips(a.N), (unsigned)splits);
  float *part = nullptr;
  uint32_t *counters = nullptr;
  if (splits > 1) {
    if (a.ws == nullptr || a.ws_bytes < gemv_workspace(a.K, a.N)) return hipErrorInvalidValue;
    if (a.N > gemv_max_n()) return hipErrorInvalidValue;
    counters = static_cast<uint32_t *>(a.ws);
    part = reinterpret_cast<float *>(static_cast<char *>(a.ws) + GV_COUNTER_BYTES);
  }
  const uint16_t *X = static_cast<const uint16_t *>(a.X);
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const uint16_t *bias = static_cast<const uint16_t *>(a.bias);
  switch (a.epi) {
    case EPI_GELU:
      hipLaunchKernelGGL(gemv_kernel<EPI_GELU>, grid, dim3(GV_WAVES * 64), 0, s, X, a.ldx,
                         (int)a.M, W, a.ldw, (int)a.K, (int)a.N, bias, a.Y, a.ldy, part, counters);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL(gemv_kernel<EPI_STORE>, grid, dim3(GV_WAVES * 64), 0, s, X, a.ldx,
                         (int)a.M, W, a.ldw, (int)a.K, (int)a.N, bias, a.Y, a.ldy, part, counters);
      break;
    case EPI_STORE_F32:
      hipLaunchKernelGGL(gemv_kernel<EPI_STORE_F32>, grid, dim3(GV_WAVES * 64), 0, s, X, a.ldx,
                         (int)a.M, W, a.ldw, (int)a.K, (int)a.N, bias, a.Y, a.ldy, part, counters);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpcol
