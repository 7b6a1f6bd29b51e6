// Vocabulary-parallel cross-entropy ("张量并行", 损失计算层的并行化).  The
// output layer's logits are split by vocabulary columns over the shards, so
// the softmax denominator of a row is a sum over all shards: each shard
// reduces its slice of every row to two numbers, the shards' row numbers are
// combined (a b*s-sized all-reduce instead of gathering b*s*v logits), and
// each shard then owns the loss terms of the rows whose target token lies
// in its slice; the shard losses are summed (an n-sized all-reduce).
//
// Row statistics are (max m, sum exp(z - m)) -- the pages sum exponentials
// directly; carrying the max keeps the same sum representable in fp32 --
// and two such pairs combine as M = max(m_a, m_b),
// s = s_a exp(m_a - M) + s_b exp(m_b - M).
//
// Kernels: row statistics (HBM-bound single pass over the logits, one
// workgroup per row, online max/sum over 16-byte vectors), the per-row
// log-sum-exp combination, the per-shard loss (gathers only the target
// logits) and the total.  Every reduction runs in a fixed order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int CE_NT = 256;
static constexpr int CE_MAX_SHARDS = 64;
static constexpr int CE_UNR = 2;       // 16-byte vectors in flight per thread (row statistics)
static constexpr int CE_LT = 1024;     // loss kernel: threads of its one workgroup
static constexpr int CE_LB = 8;        // loss kernel: rows per thread and round

struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum ms_combine(MaxSum a, MaxSum b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {M, 0.f};
  return {M, a.s * __expf(a.m - M) + b.s * __expf(b.m - M)};
}

template <typename T>
__device__ __forceinline__ void load8(const T *p, float v[8]);
// The logits are read exactly once: nontemporal loads (streamed past the
// caches) measured about 10% faster than plain ones on this pass.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float v[8]) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  const uint4 u = make_uint4(w.x, w.y, w.z, w.w);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = bf2f((uint16_t)(u4_word(u, j >> 1) >> ((j & 1) * 16)));
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
  const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p + 4));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// stats[row] = (max_j z[row][j], sum_j exp(z[row][j] - max)) over the shard's
// Vi columns.  Any width and row stride: each row is split into a scalar head
// up to the first 16-byte boundary, a body of 8-element vectors and a scalar
// tail (at most 7 elements each side).
template <typename T>
__global__ void __launch_bounds__(CE_NT)
vocab_stats_kernel(const T *__restrict__ Z, int64_t ldz, int64_t Vi, float *stats) {
  __shared__ MaxSum part[CE_NT / 64];
  const int64_t row = blockIdx.x;
  const T *z = Z + row * ldz;
  const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(z) & 15u) / sizeof(T));
  const int64_t head = mis ? min((int64_t)(16 / sizeof(T)) - mis, Vi) : 0;
  const int64_t V8 = (Vi - head) / 8;
  const int64_t body_end = head + V8 * 8;
  const T *zb = z + head;
  MaxSum acc = {-INFINITY, 0.f};
  // CE_UNR vectors per thread and round, all loaded before any is reduced
  // (more bytes in flight per CU); vectors are reduced in index order.
  for (int64_t v0 = threadIdx.x; v0 < V8; v0 += CE_NT * CE_UNR) {
    float x[CE_UNR][8];
#pragma unroll
    for (int u = 0; u < CE_UNR; ++u)
      if (v0 + u * CE_NT < V8) load8<T>(zb + (v0 + u * CE_NT) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < CE_UNR; ++u) {
      if (v0 + u * CE_NT >= V8) break;
      float cm = x[u][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[u][j]);
      const float M = fmaxf(acc.m, cm);
      if (M == -INFINITY) continue;  // every value so far is -inf: nothing to add
      float s = acc.s * __expf(acc.m - M);  // acc.m = -inf on the first vector: exp -> 0
#pragma unroll
      for (int j = 0; j < 8; ++j) s += __expf(x[u][j] - M);
      acc = {M, s};
    }
  }
  if (threadIdx.x < head) acc = ms_combine(acc, {(float)Elem<T>::to_f(z[threadIdx.x]), 1.f});
  if (threadIdx.x < Vi - body_end) acc = ms_combine(acc, {(float)Elem<T>::to_f(z[body_end + threadIdx.x]), 1.f});
  // wave tree (fixed order), then the 4 waves in index order
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) {
    MaxSum o = {__shfl_xor(acc.m, msk), __shfl_xor(acc.s, msk)};
    acc = (threadIdx.x & msk) ? ms_combine(o, acc) : ms_combine(acc, o);
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    MaxSum r = part[0];
#pragma unroll
    for (int w = 1; w < CE_NT / 64; ++w) r = ms_combine(r, part[w]);
    *reinterpret_cast<float2 *>(stats + 2 * row) = make_float2(r.m, r.s);
  }
}

struct StatPtrs {
  const float *p[CE_MAX_SHARDS];
};

// lse[t] = M + log sum_i s_i exp(m_i - M), shards in index order
__global__ void __launch_bounds__(CE_NT)
vocab_lse_kernel(StatPtrs sp, int n, int64_t T, float *lse) {
  const int64_t t = (int64_t)blockIdx.x * CE_NT + threadIdx.x;
  if (t >= T) return;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, sp.p[i][2 * t]);
  if (M == -INFINITY) {  // the whole row is -inf
    lse[t] = M;
    return;
  }
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += sp.p[i][2 * t + 1] * __expf(sp.p[i][2 * t] - M);
  lse[t] = M + __logf(s);
}

// shard_loss = sum over rows with target in [v0, v0 + Vi) of lse - z[target].
// One workgroup of CE_LT threads; rounds of CE_LT * CE_LB rows, thread k
// taking rows k, k + CE_LT, ... of a round: first every target of the round,
// then every gathered logit, so the two dependent loads of a row overlap with
// those of the thread's other rows.  Thread sums run in row order, then a
// fixed tree over the threads.
template <typename T>
__global__ void __launch_bounds__(CE_LT)
vocab_loss_kernel(const T *__restrict__ Z, int64_t ldz, int64_t T_, int64_t Vi, int64_t v0,
                  const int32_t *__restrict__ targets, const float *__restrict__ lse, float *row_loss,
                  float *shard_loss) {
  __shared__ float part[CE_LT];
  float acc = 0.f;
  for (int64_t r0 = threadIdx.x; r0 < T_; r0 += (int64_t)CE_LT * CE_LB) {
    // targets and lse of rows past T_ read row T_ - 1 (unused); the logit
    // gathers run only for this shard's targets, and nothing reads a
    // gathered value before every gather of the round is issued
    int64_t c[CE_LB];
#pragma unroll
    for (int u = 0; u < CE_LB; ++u) {
      const int64_t t = r0 + (int64_t)u * CE_LT;
      c[u] = (int64_t)targets[t < T_ ? t : T_ - 1] - v0;
    }
    bool mine[CE_LB];
    uint32_t zr[CE_LB];  // raw bits, each in its own 32-bit register
    float l[CE_LB];
#pragma unroll
    for (int u = 0; u < CE_LB; ++u) {
      const int64_t t = r0 + (int64_t)u * CE_LT;
      const int64_t tc = t < T_ ? t : T_ - 1;
      mine[u] = t < T_ && c[u] >= 0 && c[u] < Vi;
      zr[u] = 0u;
      if (mine[u]) {
        if constexpr (sizeof(T) == 2) zr[u] = (uint32_t)Z[tc * ldz + c[u]];  // widened only after every gather
        else zr[u] = __float_as_uint(Z[tc * ldz + c[u]]);
      }
      l[u] = lse[tc];
    }
#pragma unroll
    for (int u = 0; u < CE_LB; ++u) {
      const int64_t t = r0 + (int64_t)u * CE_LT;
      if (t >= T_) break;
      const float zf = __uint_as_float(sizeof(T) == 2 ? zr[u] << 16 : zr[u]);
      const float v = mine[u] ? l[u] - zf : 0.f;
      acc += v;
      if (row_loss != nullptr) row_loss[t] = v;
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = CE_LT / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) shard_loss[0] = part[0];
}

__global__ void vocab_total_kernel(StatPtrs sp, int n, float *total) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    float s = 0.f;
    for (int i = 0; i < n; ++i) s += sp.p[i][0];
    total[0] = s;
  }
}

hipError_t launch_vocab_stats(int dtype, int64_t T, int64_t Vi, const void *Z, int64_t ldz, float *stats,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(vocab_stats_kernel<uint16_t>, dim3((unsigned)T), dim3(CE_NT), 0, s,
                       static_cast<const uint16_t *>(Z), ldz, Vi, stats);
  else
    hipLaunchKernelGGL(vocab_stats_kernel<float>, dim3((unsigned)T), dim3(CE_NT), 0, s,
                       static_cast<const float *>(Z), ldz, Vi, stats);
  return hipGetLastError();
}

hipError_t launch_vocab_lse(int64_t T, int n, const float *const *stats, float *lse, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (n < 1 || n > CE_MAX_SHARDS) return hipErrorInvalidValue;
  StatPtrs sp;
  for (int i = 0; i < CE_MAX_SHARDS; ++i) sp.p[i] = stats[i < n ? i : 0];
  hipLaunchKernelGGL(vocab_lse_kernel, dim3((unsigned)((T + CE_NT - 1) / CE_NT)), dim3(CE_NT), 0, s, sp, n,
                     T, lse);
  return hipGetLastError();
}

hipError_t launch_vocab_loss(int dtype, int64_t T, int64_t Vi, int64_t v0, const void *Z, int64_t ldz,
                             const int32_t *targets, const float *lse, float *row_loss, float *shard_loss,
                             hipStream_t s) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(vocab_loss_kernel<uint16_t>, dim3(1), dim3(CE_LT), 0, s, static_cast<const uint16_t *>(Z),
                       ldz, T, Vi, v0, targets, lse, row_loss, shard_loss);
  else
    hipLaunchKernelGGL(vocab_loss_kernel<float>, dim3(1), dim3(CE_LT), 0, s, static_cast<const float *>(Z), ldz,
                       T, Vi, v0, targets, lse, row_loss, shard_loss);
  return hipGetLastError();
}

hipError_t launch_vocab_total(int n, const float *const *losses, float *total, hipStream_t s) {
  if (n < 1 || n > CE_MAX_SHARDS) return hipErrorInvalidValue;
  StatPtrs sp;
  for (int i = 0; i < CE_MAX_SHARDS; ++i) sp.p[i] = losses[i < n ? i : 0];
  hipLaunchKernelGGL(vocab_total_kernel, dim3(1), dim3(64), 0, s, sp, n, total);
  return hipGetLastError();
}

}  // namespace tpcol
