// Sequence-parallel end of a tensor-parallel block, one rank's row block:
//     Ysum = sum_{i<n} P_i (+ bias once) (+ residual)
//     Y    = gamma * (Ysum - mean) / sqrt(var + eps) + beta   per row
// The all-reduce of the row-parallel partials splits into a reduce-scatter
// (each rank sums its 1/N of the token rows) and an all-gather, and LayerNorm
// runs on the reduce-scatter's rows (parallelism overview post, 5 Sequence
// Parallelism).  LayerNorm needs the mean and the population variance of the
// full hidden row ("张量并行", 相关分析), which each rank has after the
// reduce-scatter.
//
// HBM-bound: one wave64 per row, the row held in registers as float4 chunks
// (4 consecutive columns per lane per chunk, so every load and store is a
// coalesced 16-byte vector), partials added in shard order, then the bias,
// then the residual (the order the reference sum uses).  Mean, then the
// centred sum of squares, by wave-wide butterfly reductions.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int LN_MAX_SHARDS = 64;
static constexpr int LN_ROWS_PER_WG = 4;  // one wave per row

struct LnPartials {
  const float *p[LN_MAX_SHARDS];
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// CH: float4 chunks per lane the row needs at most (N <= 256 * CH)
template <int CH, bool OUT_BF16>
__global__ void __launch_bounds__(64 * LN_ROWS_PER_WG)
rs_layernorm_kernel(LnPartials pp, int n, int64_t rows, int N, int64_t ldp, const float *bias,
                    const float *res, int64_t ldr, const float *gamma, const float *beta, float eps,
                    float *Ysum, int64_t ldys, void *Y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * LN_ROWS_PER_WG + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave: no barrier in this kernel
  // Every load of the row is issued before the first store: Ysum or Y may
  // share memory with the residual (an in-place update) or with gamma and
  // beta as far as the compiler knows, so a load placed after a store would
  // wait for it.  Loads of UNR shards are issued together before they are
  // added (in shard order).  Short rows (CH <= 4) also fetch the residual,
  // bias, gamma and beta with the first shard, so the row costs about one
  // memory latency.
  constexpr int UNR = CH <= 4 ? 4 : (CH <= 16 ? 2 : 1);
  constexpr bool EARLY = CH <= 4;
  auto ld4 = [&](const float *base, int col) {
    return col < N ? *reinterpret_cast<const f32x4_t *>(base + col) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
  };
  f32x4_t x[CH], r[EARLY ? CH : 1], bv[EARLY ? CH : 1], gm[EARLY ? CH : 1], bt[EARLY ? CH : 1];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (c * 64 + lane) * 4;
    x[c] = ld4(pp.p[0] + row * ldp, col);
    if constexpr (EARLY) {
      r[c] = res != nullptr ? ld4(res + row * ldr, col) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
      bv[c] = bias != nullptr ? ld4(bias, col) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
      gm[c] = ld4(gamma, col);
      bt[c] = ld4(beta, col);
    }
  }
  for (int i0 = 1; i0 < n; i0 += UNR) {
    f32x4_t t[UNR][CH];
#pragma unroll
    for (int j = 0; j < UNR; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int col = (c * 64 + lane) * 4;
        t[j][c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if (i0 + j < n && col < N) t[j][c] = *reinterpret_cast<const f32x4_t *>(pp.p[i0 + j] + row * ldp + col);
      }
#pragma unroll
    for (int j = 0; j < UNR; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (i0 + j < n) x[c] += t[j][c];
  }
  // shard sum, then the bias, then the residual (the reference sum's order)
  if constexpr (EARLY) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (bias != nullptr) x[c] += bv[c];
      if (res != nullptr) x[c] += r[c];
    }
  } else {
    if (bias != nullptr) {
#pragma unroll
      for (int c = 0; c < CH; ++c) x[c] += ld4(bias, (c * 64 + lane) * 4);
    }
    if (res != nullptr) {
      f32x4_t rr[CH];  // all chunks loaded before the first Ysum store
#pragma unroll
      for (int c = 0; c < CH; ++c) rr[c] = ld4(res + row * ldr, (c * 64 + lane) * 4);
#pragma unroll
      for (int c = 0; c < CH; ++c) x[c] += rr[c];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (c * 64 + lane) * 4;
    if (col < N) {
      const f32x4_t a = x[c];
      if (Ysum != nullptr) *reinterpret_cast<f32x4_t *>(Ysum + row * ldys + col) = a;
      s += (a[0] + a[1]) + (a[2] + a[3]);
    }
  }
  const float invN = 1.0f / (float)N;
  const float mean = wave_sum(s) * invN;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (c * 64 + lane) * 4;
    if (col < N) {
      const f32x4_t d = x[c] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * invN + eps);
  // gamma / beta of GB chunks at a time, loaded before those chunks' stores
  constexpr int GB = EARLY ? CH : 8;
#pragma unroll
  for (int c0 = 0; c0 < CH; c0 += GB) {
    f32x4_t g[GB], b[GB];
#pragma unroll
    for (int k = 0; k < GB; ++k) {
      if constexpr (EARLY) {
        g[k] = gm[c0 + k];
        b[k] = bt[c0 + k];
      } else {
        g[k] = ld4(gamma, ((c0 + k) * 64 + lane) * 4);
        b[k] = ld4(beta, ((c0 + k) * 64 + lane) * 4);
      }
    }
#pragma unroll
    for (int k = 0; k < GB; ++k) {
      const int col = ((c0 + k) * 64 + lane) * 4;
      if (col < N) {
        const f32x4_t y = (x[c0 + k] - mean) * rstd * g[k] + b[k];
        if constexpr (OUT_BF16)
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(Y) + row * ldy + col) =
              make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
        else
          *reinterpret_cast<f32x4_t *>(static_cast<float *>(Y) + row * ldy + col) = y;
      }
    }
  }
}

int64_t rs_layernorm_max_n() { return 8192; }

template <int CH>
static hipError_t run_ln(bool bf16, const LnPartials &pp, int n, int64_t rows, int N, int64_t ldp,
                         const float *bias, const float *res, int64_t ldr, const float *gamma,
                         const float *beta, float eps, float *Ysum, int64_t ldys, void *Y, int64_t ldy,
                         hipStream_t s) {
  const dim3 grid((unsigned)((rows + LN_ROWS_PER_WG - 1) / LN_ROWS_PER_WG));
  if (bf16)
    hipLaunchKernelGGL((rs_layernorm_kernel<CH, true>), grid, dim3(64 * LN_ROWS_PER_WG), 0, s, pp, n, rows,
                       N, ldp, bias, res, ldr, gamma, beta, eps, Ysum, ldys, Y, ldy);
  else
    hipLaunchKernelGGL((rs_layernorm_kernel<CH, false>), grid, dim3(64 * LN_ROWS_PER_WG), 0, s, pp, n, rows,
                       N, ldp, bias, res, ldr, gamma, beta, eps, Ysum, ldys, Y, ldy);
  return hipGetLastError();
}

hipError_t launch_rs_layernorm(int out_dtype, int64_t rows, int64_t N, int n, const float *const *parts,
                               int64_t ldp, const float *bias, const float *res, int64_t ldr,
                               const float *gamma, const float *beta, float eps, float *Ysum,
                               int64_t ldys, void *Y, int64_t ldy, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (n < 1 || n > LN_MAX_SHARDS || N < 4 || N > rs_layernorm_max_n() || N % 4) return hipErrorInvalidValue;
  LnPartials pp;
  for (int i = 0; i < LN_MAX_SHARDS; ++i) pp.p[i] = parts[i < n ? i : 0];
  const bool bf16 = out_dtype == DT_BF16;
  const int Ni = (int)N;
  if (N <= 1024) return run_ln<4>(bf16, pp, n, rows, Ni, ldp, bias, res, ldr, gamma, beta, eps, Ysum, ldys, Y, ldy, s);
  if (N <= 4096) return run_ln<16>(bf16, pp, n, rows, Ni, ldp, bias, res, ldr, gamma, beta, eps, Ysum, ldys, Y, ldy, s);
  return run_ln<32>(bf16, pp, n, rows, Ni, ldp, bias, res, ldr, gamma, beta, eps, Ysum, ldys, Y, ldy, s);
}

}  // namespace tpcol
