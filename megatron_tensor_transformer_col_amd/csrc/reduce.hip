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

// db[c] = sum_m dZ[m][c].  Workgroup = 64 columns x 4 row-slices; the four
// slice sums are combined in LDS in a fixed order.
template <typename T>
__global__ void __launch_bounds__(256)
colsum_kernel(int64_t M, int64_t N, const T *dZ, int64_t ldz, float *db) {
  __shared__ float part[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int slice = threadIdx.x >> 6;
  float acc = 0.f;
  if (c < N) {
    for (int64_t m = slice; m < M; m += 4) acc += Elem<T>::to_f(dZ[m * ldz + c]);
  }
  part[slice][threadIdx.x & 63] = acc;
  __syncthreads();
  if (slice == 0 && c < N) {
    const int t = threadIdx.x & 63;
    db[c] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
  }
}

hipError_t launch_colsum(int dtype, int64_t M, int64_t N, const void *dZ, int64_t ldz, float *db,
                         hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((N + 63) / 64));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(colsum_kernel<uint16_t>, grid, dim3(256), 0, s, M, N,
                       static_cast<const uint16_t *>(dZ), ldz, db);
  else
    hipLaunchKernelGGL(colsum_kernel<float>, grid, dim3(256), 0, s, M, N,
                       static_cast<const float *>(dZ), ldz, db);
  return hipGetLastError();
}

}  // namespace tpcol
