// HBM-bound reductions: the N-shard partial sum and the bias-gradient column
// sum.  Both stream float4 / 16-byte vectors and keep one fp32 accumulator
// per element, adding terms in a fixed order (deterministic results).
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int kMaxShards = 64;

struct PartialPtrs {
  const float *p[kMaxShards];
};

// Y[m][c..c+3] = sum_{i<n} P_i[m][c..c+3] (+ bias[c..c+3]); one float4 per
// thread per grid-stride step.  Shard terms are added in index order.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
shard_sum_kernel(PartialPtrs pp, int n, int64_t M, int64_t N4, int64_t ldp, const float *bias,
                 void *Y, int64_t ldy) {
  const int64_t total = M * N4;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = v / N4, c = (v - row * N4) * 4;
    const int64_t off = row * ldp + c;
    float4 acc = *reinterpret_cast<const float4 *>(pp.p[0] + off);
    for (int i = 1; i < n; ++i) {
      const float4 t = *reinterpret_cast<const float4 *>(pp.p[i] + off);
      acc.x += t.x; acc.y += t.y; acc.z += t.z; acc.w += t.w;
    }
    if (bias != nullptr) {
      const float4 b = *reinterpret_cast<const float4 *>(bias + c);
      acc.x += b.x; acc.y += b.y; acc.z += b.z; acc.w += b.w;
    }
    if constexpr (OUT_BF16) {
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(Y) + row * ldy + c) =
          make_uint2(pack_bf2(acc.x, acc.y), pack_bf2(acc.z, acc.w));
    } else {
      *reinterpret_cast<float4 *>(static_cast<float *>(Y) + row * ldy + c) = acc;
    }
  }
}

// db[c] = sum over rows y < splits of part[y][c]: 16 lanes of a wave per
// column, lane l adding rows l, l + 16, ... in order, then the 16 lane
// sums added in lane order (a fixed order; one round trip of loads per
// 16 rows instead of a chain over all of them).  Block b covers columns
// 16 b .. 16 b + 15; every lane of the block takes part (the shuffles).
__device__ __forceinline__ void colsum_final_block(int64_t b, int splits, int64_t N, const float *__restrict__ part,
                                                   float *__restrict__ db) {
  const int lane = threadIdx.x & 63, l = lane & 15;
  const int64_t c = (b * 256 + threadIdx.x) >> 4;  // 4 columns per wave
  float t = 0.f;
  if (c < N) {
    for (int y0 = 0; y0 < splits; y0 += 64) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int y = y0 + 16 * j + l;
        v[j] = y < splits ? part[(int64_t)y * N + c] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (y0 + 16 * j + l < splits) t += v[j];
    }
  }
  // lane sums in lane order: lane 0 of each 16-lane group collects 1..15
  float tot = t;
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    const float o = __shfl(t, (lane & ~15) + k);
    if (l == 0) tot += o;
  }
  if (l == 0 && c < N) db[c] = tot;
}

__global__ void __launch_bounds__(256)
colsum_final_kernel(int splits, int64_t N, const float *__restrict__ part, float *__restrict__ db) {
  colsum_final_block(blockIdx.x, splits, N, part, db);
}

// Two sums of n partials each (fp32 out): element v of the combined range
// [0, 2 M N4) belongs to sum g = v / (M N4), whose terms are P_{g n + i}.
// Blocks past the first sum_blocks do colsum_final_block's work instead
// (cs_rows rows of cs_part, cs_N columns, into db).
__global__ void __launch_bounds__(256)
shard_sum_pair_kernel(PartialPtrs pp, int n, int64_t M, int64_t N4, int64_t ldp, float *Y0, int64_t ldy0,
                      float *Y1, int64_t ldy1, int sum_blocks, int cs_rows, int64_t cs_N,
                      const float *cs_part, float *db) {
  if ((int)blockIdx.x >= sum_blocks) {
    colsum_final_block((int64_t)blockIdx.x - sum_blocks, cs_rows, cs_N, cs_part, db);
    return;
  }
  const int64_t one = M * N4;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < 2 * one;
       v += (int64_t)sum_blocks * blockDim.x) {
    const int g = v >= one ? 1 : 0;
    const int64_t w = v - g * one;
    const int64_t row = w / N4, c = (w - row * N4) * 4;
    const int64_t off = row * ldp + c;
    const float *const *p = pp.p + g * n;
    float4 acc = *reinterpret_cast<const float4 *>(p[0] + off);
    for (int i = 1; i < n; ++i) {
      const float4 t = *reinterpret_cast<const float4 *>(p[i] + off);
      acc.x += t.x; acc.y += t.y; acc.z += t.z; acc.w += t.w;
    }
    *reinterpret_cast<float4 *>((g ? Y1 + row * ldy1 : Y0 + row * ldy0) + c) = acc;
  }
}

static unsigned colsum_final_blocks(int64_t N) { return (unsigned)((N * 16 + 255) / 256); }

hipError_t launch_shard_sum_pair(int64_t M, int64_t N, int n, const float *const *parts, int64_t ldp,
                                 float *Y0, int64_t ldy0, float *Y1, int64_t ldy1, hipStream_t s,
                                 const ColsumJob *cj) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (n < 1 || 2 * n > kMaxShards || N % 4) return hipErrorInvalidValue;
  if (cj != nullptr && (cj->rows < 0 || cj->N <= 0)) return hipErrorInvalidValue;
  PartialPtrs pp;
  for (int i = 0; i < kMaxShards; ++i) pp.p[i] = parts[i < 2 * n ? i : 0];
  const int64_t N4 = N / 4;
  const int64_t want = (2 * M * N4 + 255) / 256;
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  const unsigned extra = cj != nullptr ? colsum_final_blocks(cj->N) : 0u;
  hipLaunchKernelGGL(shard_sum_pair_kernel, dim3(grid + extra), dim3(256), 0, s, pp, n, M, N4, ldp, Y0, ldy0, Y1,
                     ldy1, (int)grid, cj != nullptr ? cj->rows : 0, cj != nullptr ? cj->N : (int64_t)0,
                     cj != nullptr ? cj->part : (const float *)nullptr, cj != nullptr ? cj->db : (float *)nullptr);
  return hipGetLastError();
}

hipError_t launch_shard_sum(int out_dtype, int64_t M, int64_t N, int n, const float *const *parts,
                            int64_t ldp, const float *bias, void *Y, int64_t ldy, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (n < 1 || n > kMaxShards) return hipErrorInvalidValue;
  PartialPtrs pp;
  for (int i = 0; i < kMaxShards; ++i) pp.p[i] = parts[i < n ? i : 0];
  const int64_t N4 = N / 4;
  const int64_t total = M * N4;
  // 256 CUs x 8 resident workgroups; a grid-stride loop covers the rest.
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
  if (out_dtype == DT_BF16)
    hipLaunchKernelGGL(shard_sum_kernel<true>, dim3(grid), dim3(256), 0, s, pp, n, M, N4, ldp,
                       bias, Y, ldy);
  else
    hipLaunchKernelGGL(shard_sum_kernel<false>, dim3(grid), dim3(256), 0, s, pp, n, M, N4, ldp,
                       bias, Y, ldy);
  return hipGetLastError();
}

// db[c] = sum_m dZ[m][c] in two passes, each in a fixed order.
// Pass 1: workgroup (y, column block) = 256 threads = 32 16-byte column
// vectors x 8 row lanes over the rows of split y; a thread adds rows
// lane, lane + 8, ... of its vector in row order (4 loads in flight), the 8
// lanes are added in lane order through LDS, and the sums go to part[y][c].
// Pass 2 (colsum_final_kernel): db[c] = sum over y of part[y][c] in a fixed
// order (see the kernel).
static constexpr int CS_MAX_SPLITS = 64;
static constexpr int CS_MIN_ROWS = 64;  // rows per split at least

static int colsum_splits(int64_t M) {
  const int64_t s = (M + CS_MIN_ROWS - 1) / CS_MIN_ROWS;
  return (int)(s < 1 ? 1 : (s > CS_MAX_SPLITS ? CS_MAX_SPLITS : s));
}

// room for the 64 row splits of colsum_partial_kernel or one row per 128
// rows of M (a GEMM epilogue's per-row-tile sums), whichever is more
int64_t colsum_rows(int64_t M) {
  const int64_t tiles = (M + 127) / 128;
  return tiles > CS_MAX_SPLITS ? tiles : CS_MAX_SPLITS;
}
size_t colsum_workspace(int64_t M, int64_t N) {
  return (size_t)colsum_rows(M) * (size_t)(N > 0 ? N : 0) * sizeof(float);
}

template <typename T>
__global__ void __launch_bounds__(256)
colsum_partial_kernel(int64_t M, int64_t N, const T *__restrict__ dZ, int64_t ldz, int64_t rows_per,
                      float *__restrict__ part) {
  constexpr int VW = Elem<T>::VW;
  __shared__ float red[8][32 * VW];
  const int vc = threadIdx.x & 31, lr = threadIdx.x >> 5;
  const int64_t c0 = ((int64_t)blockIdx.x * 32 + vc) * VW;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = M < r0 + rows_per ? M : r0 + rows_per;
  float acc[VW];
#pragma unroll
  for (int k = 0; k < VW; ++k) acc[k] = 0.f;
  auto add = [&](const uint4 &u) {
    if constexpr (VW == 8) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += bf2f((uint16_t)(w[k] & 0xffffu));
        acc[2 * k + 1] += bf2f((uint16_t)(w[k] >> 16));
      }
    } else {
      acc[0] += __uint_as_float(u.x); acc[1] += __uint_as_float(u.y);
      acc[2] += __uint_as_float(u.z); acc[3] += __uint_as_float(u.w);
    }
  };
  if (c0 < N) {
    const T *col = dZ + c0;
    int64_t m = r0 + lr;
    for (; m + 24 < r1; m += 32) {
      uint4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4 *>(col + (m + 8 * q) * ldz);
#pragma unroll
      for (int q = 0; q < 4; ++q) add(v[q]);
    }
    for (; m < r1; m += 8) add(*reinterpret_cast<const uint4 *>(col + m * ldz));
  }
#pragma unroll
  for (int k = 0; k < VW; ++k) red[lr][vc * VW + k] = acc[k];
  __syncthreads();
  if (lr == 0 && c0 < N) {
#pragma unroll
    for (int k = 0; k < VW; ++k) {
      float t = red[0][vc * VW + k];
#pragma unroll
      for (int l = 1; l < 8; ++l) t += red[l][vc * VW + k];
      part[(int64_t)blockIdx.y * N + c0 + k] = t;
    }
  }
}

hipError_t launch_colsum_final(int rows, int64_t N, const float *part, float *db, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (rows < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(colsum_final_kernel, dim3(colsum_final_blocks(N)), dim3(256), 0, s, rows, N, part, db);
  return hipGetLastError();
}

hipError_t launch_colsum(int dtype, int64_t M, int64_t N, const void *dZ, int64_t ldz, float *db,
                         float *part, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  int splits = 0;
  if (M > 0) {
    splits = colsum_splits(M);
    const int64_t rows_per = (M + splits - 1) / splits;
    splits = (int)((M + rows_per - 1) / rows_per);
    const int vw = dtype == DT_BF16 ? 8 : 4;
    const dim3 grid((unsigned)((N + 32 * vw - 1) / (32 * vw)), (unsigned)splits);
    if (dtype == DT_BF16)
      hipLaunchKernelGGL(colsum_partial_kernel<uint16_t>, grid, dim3(256), 0, s, M, N,
                         static_cast<const uint16_t *>(dZ), ldz, rows_per, part);
    else
      hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, s, M, N,
                         static_cast<const float *>(dZ), ldz, rows_per, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colsum_final_kernel, dim3(colsum_final_blocks(N)), dim3(256), 0, s, splits, N,
                     part, db);
  return hipGetLastError();
}

}  // namespace tpcol
