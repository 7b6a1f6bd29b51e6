// Decode-phase GEMV (M <= 16 tokens), weight-streaming and HBM-bound.
//
// In decode every request contributes one token, so a linear layer reads the
// whole weight once for 2*M*K*N flops: arithmetic intensity is about
// 2*M / bytes_per_param (parallelism survey post, Prefill-Decode 分离,
// Decode 阶段), ~16 flop/byte for 16 bf16 tokens, far below the ridge.  The
// kernel is therefore built for bytes in flight, not for flops:
//
//  * Workgroup = 4 wave64 over a 64-column strip of W and one K range
//    (split-K across workgroups so that a 3584 x 8192 or 8192 x 3584 shard
//    still spreads over all 256 CUs).  The K range of x (16 x Krange, zero
//    padded past M and K) is staged once in LDS.
//  * W streams HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) in
//    64-row slabs through a 4-deep ring (128-byte row segments); a slab is
//    8 KiB, two DMA ops per wave.
//  * Each wave owns 16 of the 64 columns.  The MFMA B operand (8 consecutive
//    k of one column) comes from ds_read_b64_tr_b16 transpose reads of the
//    [k][n] slab, the A operand from the x slice (ds_read_b128), and
//    v_mfma_f32_16x16x32_bf16 does the work, M padded to 16 with zeros.
//  * Rows past K read a clamped (valid) weight row against zero x, so they
//    add nothing; columns past N are clamped and never stored.
//  * Partial sums go to an fp32 workspace [splits][16][N]; a second small
//    kernel adds them in split order, adds the bias and applies the
//    activation.  The activation must come after the full K reduction
//    since GELU does not distribute over a sum ("张量并行", 两个矩阵相乘).
//    No workgroup waits on another and nothing has to be pre-zeroed.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

#define TP_AS3 __attribute__((address_space(3)))
typedef short gv_i16x4_t __attribute__((ext_vector_type(4)));

static constexpr int GV_BN = 64;       // columns per workgroup strip
static constexpr int GV_SLAB = 64;     // k rows per LDS slab
static constexpr int GV_STAGES = 4;    // slab ring depth
static constexpr int GV_NT = 256;      // 4 wave64
static constexpr int GV_MAX_KR = 1024; // max K range per workgroup (x slice in LDS)
static constexpr int GV_TARGET_WG = 512;

struct GvPlan {
  int strips, splits, krange;
};

static GvPlan gv_plan(int64_t K, int64_t N) {
  GvPlan p;
  p.strips = (int)((N + GV_BN - 1) / GV_BN);
  const int64_t kslabs = (K + GV_SLAB - 1) / GV_SLAB;
  int64_t splits = (GV_TARGET_WG + p.strips - 1) / p.strips;
  const int64_t min_splits = (kslabs * GV_SLAB + GV_MAX_KR - 1) / GV_MAX_KR;
  if (splits < min_splits) splits = min_splits;
  if (splits > kslabs) splits = kslabs;
  if (splits < 1) splits = 1;
  const int64_t slabs_per = (kslabs + splits - 1) / splits;
  p.krange = (int)(slabs_per * GV_SLAB);
  p.splits = (int)((kslabs + slabs_per - 1) / slabs_per);
  return p;
}

size_t gemv_workspace(int64_t K, int64_t N) {
  const GvPlan p = gv_plan(K, N);
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * 16 * (size_t)N * sizeof(float);
}

int64_t gemv_max_n() { return (int64_t)1 << 30; }

__device__ __forceinline__ void gv_dma16(const uint16_t *g, uint16_t *lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(TP_AS3 void *)lds_wave_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void gv_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// 64-column slab rows (8 granules): granule index bits 1..2 swizzled so that
// the 8 rows one half-wave transposes land on distinct banks.
__device__ __forceinline__ int gv_swz(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }

template <int EPI>
__device__ __forceinline__ void gv_store8(float v[8], const uint16_t *bias, int col, void *Y,
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

// FINAL: single split, apply the epilogue directly; else write fp32 partials.
template <int EPI, bool FINAL>
__global__ void __launch_bounds__(GV_NT)
gemv_partial_kernel(const uint16_t *__restrict__ X, int64_t ldx, int M, const uint16_t *__restrict__ W,
                    int64_t ldw, int K, int N, int krange, const uint16_t *bias, void *Y,
                    int64_t ldy, float *part) {
  constexpr int XLD = GV_MAX_KR + 8;  // padded x row (16 B pad: conflict-free b128 reads)
  __shared__ __attribute__((aligned(1024))) uint16_t slab[GV_STAGES][GV_SLAB * GV_BN];
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * XLD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int strip = blockIdx.x, split = blockIdx.y;
  const int n0 = strip * GV_BN;
  const int k_begin = split * krange;
  const int k_end = min(K, k_begin + krange);
  const int nslab = (k_end - k_begin + GV_SLAB - 1) / GV_SLAB;

  // ---- DMA sources: per slab 8 blocks of 8 rows x 8 granules; wave w owns
  //      blocks w and w + 4.  Lane i of a block fetches row i/8, granule
  //      (i%8) ^ swz(row), clamped into the matrix.
  int col_of[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (wave + 4 * j) * 8 + (lane >> 3);
    const int lg = (lane & 7) ^ gv_swz(row);
    col_of[j] = min(n0 + lg * 8, N - 8);
  }
  auto issue = [&](int s) {
    const int kr = k_begin + s * GV_SLAB;
    uint16_t *base = slab[s % GV_STAGES];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // rows past K are clamped to K-1: valid memory, multiplied by zero x
      const int row = min(kr + (wave + 4 * j) * 8 + (lane >> 3), K - 1);
      gv_dma16(W + (int64_t)row * ldw + col_of[j], base + (wave + 4 * j) * 512);
    }
  };
  // ---- x slice -> LDS (zero past M and past K)
  const int kv = nslab * (GV_SLAB / 8);  // 16-byte vectors per x row
  for (int v = tid; v < 16 * kv; v += GV_NT) {
    const int m = v / kv, kk = (v % kv) * 8;
    const int k = k_begin + kk;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (m < M && k < K) val = *reinterpret_cast<const uint4 *>(X + (int64_t)m * ldx + k);
    *reinterpret_cast<uint4 *>(&xs[m * XLD + kk]) = val;
  }

#pragma unroll
  for (int s = 0; s < GV_STAGES - 1; ++s)
    if (s < nslab) issue(s);

  // ---- stream the slabs
  f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int cw = wave * 16;  // this wave's columns within the strip
  const int s4 = l16 >> 2;
  const int colw = cw + 4 * (l16 & 3);
  for (int s = 0; s < nslab; ++s) {
    if (s + GV_STAGES - 2 < nslab) gv_wait_vmcnt<2 * (GV_STAGES - 2)>();
    else gv_wait_vmcnt<0>();
    __syncthreads();
    if (s + GV_STAGES - 1 < nslab) issue(s + GV_STAGES - 1);
    const uint16_t *t = slab[s % GV_STAGES];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int r1 = kc * 32 + 8 * g + s4;
      const int off = (((colw >> 3) ^ gv_swz(r1)) << 3) + (colw & 4);
      const gv_i16x4_t b0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_AS3 gv_i16x4_t *)(t + r1 * GV_BN + off));
      const gv_i16x4_t b1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_AS3 gv_i16x4_t *)(t + (r1 + 4) * GV_BN + off));
      const uint2 u0 = __builtin_bit_cast(uint2, b0), u1 = __builtin_bit_cast(uint2, b1);
      const uint4 bf = make_uint4(u0.x, u0.y, u1.x, u1.y);
      const uint4 af = *reinterpret_cast<const uint4 *>(&xs[l16 * XLD + s * GV_SLAB + kc * 32 + g * 8]);
      acc = mfma16(bf, af, acc);  // lane: token l16, columns cw + 4g .. +3
    }
  }

  // ---- this wave's 16 x 16 result: lane holds [m = l16][cw + 4g + r]
  const int m = l16;
  const int col = n0 + cw + 4 * g;
  if (m >= M || col >= N) return;
  if constexpr (FINAL) {
    float v[4] = {acc[0], acc[1], acc[2], acc[3]};
    if (bias != nullptr) {
      const uint2 b = *reinterpret_cast<const uint2 *>(bias + col);
      v[0] += bf2f((uint16_t)(b.x & 0xffffu)); v[1] += bf2f((uint16_t)(b.x >> 16));
      v[2] += bf2f((uint16_t)(b.y & 0xffffu)); v[3] += bf2f((uint16_t)(b.y >> 16));
    }
    if constexpr (EPI == EPI_STORE_F32) {
      *reinterpret_cast<float4 *>(static_cast<float *>(Y) + (int64_t)m * ldy + col) =
          make_float4(v[0], v[1], v[2], v[3]);
    } else {
      if constexpr (EPI == EPI_GELU) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = gelu_f(v[r]);
      }
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(Y) + (int64_t)m * ldy + col) =
          make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
    }
  } else {
    *reinterpret_cast<float4 *>(part + ((int64_t)split * 16 + m) * N + col) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// Y[m][c..c+7] = epi(sum_s part[s][m][c..c+7] + bias), splits added in order.
template <int EPI>
__global__ void __launch_bounds__(256)
gemv_finalize_kernel(const float *__restrict__ part, int splits, int M, int N,
                     const uint16_t *bias, void *Y, int64_t ldy) {
  const int n8 = N / 8;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= M * n8) return;
  const int m = v / n8, col = (v % n8) * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; ++sp) {
    const float *p = part + ((int64_t)sp * 16 + m) * N + col;
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
    s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
  }
  gv_store8<EPI>(s, bias, col, Y, ldy, m);
}

template <int EPI>
static hipError_t run_gemv(const GemvArgs &a, const GvPlan &pl, hipStream_t s) {
  const uint16_t *X = static_cast<const uint16_t *>(a.X);
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const uint16_t *bias = static_cast<const uint16_t *>(a.bias);
  const dim3 grid((unsigned)pl.strips, (unsigned)pl.splits);
  if (pl.splits == 1) {
    hipLaunchKernelGGL((gemv_partial_kernel<EPI, true>), grid, dim3(GV_NT), 0, s, X, a.ldx,
                       (int)a.M, W, a.ldw, (int)a.K, (int)a.N, pl.krange, bias, a.Y, a.ldy,
                       (float *)nullptr);
    return hipGetLastError();
  }
  float *part = static_cast<float *>(a.ws);
  hipLaunchKernelGGL((gemv_partial_kernel<EPI, false>), grid, dim3(GV_NT), 0, s, X, a.ldx,
                     (int)a.M, W, a.ldw, (int)a.K, (int)a.N, pl.krange, bias, a.Y, a.ldy, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = (int)a.M * (int)(a.N / 8);
  hipLaunchKernelGGL((gemv_finalize_kernel<EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, s, part, pl.splits, (int)a.M, (int)a.N, bias, a.Y, a.ldy);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs &a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 16 || a.dtype != DT_BF16 || a.K < 1 || a.N < 8) return hipErrorInvalidValue;
  const GvPlan pl = gv_plan(a.K, a.N);
  if (pl.krange > GV_MAX_KR) return hipErrorInvalidValue;
  if (pl.splits > 1 && (a.ws == nullptr || a.ws_bytes < gemv_workspace(a.K, a.N)))
    return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_GELU: return run_gemv<EPI_GELU>(a, pl, s);
    case EPI_STORE: return run_gemv<EPI_STORE>(a, pl, s);
    case EPI_STORE_F32: return run_gemv<EPI_STORE_F32>(a, pl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpcol
