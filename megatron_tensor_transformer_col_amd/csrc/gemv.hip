// Decode-phase GEMV (M <= 16 tokens), weight-streaming and HBM-bound.
//
// In decode every request contributes one token, so a linear layer reads the
// whole weight once for 2*M*K*N flops: arithmetic intensity is about
// 2*M / bytes_per_param (parallelism overview post, Prefill-Decode 分离,
// Decode 阶段), ~16 flop/byte for 16 bf16 tokens, far below the ridge.  The
// kernel is therefore built for bytes in flight, not for flops:
//
//  * Workgroup = 4 wave64 over a 64-column strip of W and one K range
//    (split-K across workgroups so that a 3584 x 8192 or 8192 x 3584 shard
//    spreads over all 256 CUs, two workgroups per CU).  W is row-major, or
//    packed once into 64-column panels (below), where a workgroup's share
//    is one contiguous run instead of 128 bytes from each of its rows.
//  * Each ring stage holds a 64-row slab of the strip (8 KiB) and the
//    matching 16 x 64 slice of x (2 KiB); both move HBM -> LDS with
//    global_load_lds_dwordx4 (no VGPR staging; the weights, read once per
//    call, with the nontemporal hint: 16.4 -> 15.5 us per column GEMV and
//    partial-sum pair over 8 rotating shards), three DMA ops per wave per
//    stage, through a 3-deep ring: two stages (20 KiB) in flight per
//    workgroup, ~10 MB over the chip.  Measured on the 58.7 MB decode
//    shards, deeper rings (up to 6 stages, 30 MB in flight) were ~1 us
//    slower per GEMV: the extra requests only queue at the memory.
//  * Each wave owns 16 of the 64 columns.  The MFMA B operand (8 consecutive
//    k of one column) comes from ds_read_b64_tr_b16 transpose reads of the
//    [k][n] slab, the A operand (x) from ds_read_b128, and
//    v_mfma_f32_16x16x32_bf16 does the work.  Token rows past M read the
//    last valid row (their results are never stored).
//  * A ragged K tail (the last slab of the last split) reads W rows clamped
//    to K-1 against a zero-padded copy of x built in registers, so those
//    rows add nothing and no load leaves x.
//  * Partial sums go to an fp32 workspace [splits][16][N]; a second small
//    kernel adds them in split order, adds the bias and applies the
//    activation.  The activation must come after the full K reduction
//    since GELU does not distribute over a sum ("张量并行", 两个矩阵相乘).
//    No workgroup waits on another and nothing has to be pre-zeroed.
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace tpcol {

static constexpr int GV_BN = 64;        // columns per workgroup strip
static constexpr int GV_SLAB = 64;      // k rows per slab
static constexpr int GV_STAGES = 3;     // ring depth
static constexpr int GV_NT = 256;       // 4 wave64
static constexpr int GV_TARGET_WG = 512;
static constexpr int GV_WSLAB = GV_SLAB * GV_BN;  // W elements per stage (8 KiB)
static constexpr int GV_XSLAB = 16 * GV_SLAB;     // x elements per stage (2 KiB)
static constexpr int GV_STAGE = GV_WSLAB + GV_XSLAB;
static constexpr int GV_DMA = 3;                  // DMA ops per wave per stage (2 W + 1 x)
static constexpr int64_t GV_MAX_LD = int64_t(1) << 26;  // 16 rows of either operand within 32-bit byte offsets

struct GvPlan {
  int strips, splits, krange;
};

static GvPlan gv_plan(int64_t K, int64_t N) {
  GvPlan p;
  p.strips = (int)((N + GV_BN - 1) / GV_BN);
  const int64_t kslabs = (K + GV_SLAB - 1) / GV_SLAB;
  // all workgroups in one wave of the launch (a partial second wave would
  // double the time): at most GV_TARGET_WG of them
  int64_t splits = GV_TARGET_WG / p.strips;
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

// 64-column slab rows (8 granules): granule index bits 1..2 swizzled so that
// the 8 rows one half-wave transposes land on distinct banks.
__device__ __forceinline__ int gv_swz(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }

// How a workgroup's 16 x 64 result leaves the kernel.
enum GvOut {
  GV_FINAL = 0,   // single split: bias + activation applied here
  GV_PARTIAL = 1  // fp32 partial to part[split]; gemv_finalize_kernel adds them
};

template <int EPI, int OUT>
__global__ void __launch_bounds__(GV_NT)
gemv_partial_kernel(const uint16_t *__restrict__ X, int64_t ldx, int M, const uint16_t *__restrict__ W,
                    int64_t ldw, int64_t sstride, int ncl, int K, int N, int krange, const uint16_t *bias,
                    void *Y, int64_t ldy, float *part) {
  constexpr bool FINAL = OUT == GV_FINAL;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[GV_STAGES * GV_STAGE + GV_XSLAB];
  uint16_t *xtail = smem + GV_STAGES * GV_STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int strip = blockIdx.x, split = blockIdx.y;
  const int n0 = strip * GV_BN;
  const int k_begin = split * krange;
  const int k_end = min(K, k_begin + krange);
  const int nslab = (k_end - k_begin + GV_SLAB - 1) / GV_SLAB;
  const int tail = ((k_end - k_begin) % GV_SLAB) ? nslab - 1 : -1;  // slab with rows past K

  // ---- DMA sources.  W: per slab 8 blocks of 8 rows x 8 granules; wave w
  //      owns blocks w and w + 4; lane i of a block fetches row i/8, granule
  //      (i%8) ^ swz(row), clamped into the matrix.  x: wave w fetches token
  //      rows 4w .. 4w+3 (lanes 0..31), granule (i%8) ^ (row & 7), token rows
  //      past M clamped to M-1.
  // Byte offsets below are 32-bit (launch_gemv checks the strides), added to
  // wave-uniform bases that the scalar unit computes per slab.
  uint32_t woff[2];  // this lane's W source relative to its block's first row
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (wave + 4 * j) * 8 + (lane >> 3);
    const int lg = (lane & 7) ^ gv_swz(row);
    const int colrel = min(n0 + lg * 8, ncl - 8) - n0;
    woff[j] = (uint32_t)(((int64_t)(lane >> 3) * ldw + colrel) * 2);
  }
  const int xrow = 4 * wave + ((lane >> 3) & 3);
  const uint32_t xoff_row = (uint32_t)((int64_t)min(xrow, M - 1) * ldx * 2);
  const uint32_t xoff = xoff_row + (uint32_t)(((lane & 7) ^ (xrow & 7)) * 16);
  const uint16_t *Wn = W + (int64_t)strip * sstride;  // this strip's column 0, row 0
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int s) {
    const int kr = k_begin + s * GV_SLAB;
    const uint32_t base = lds0 + (uint32_t)((s % GV_STAGES) * GV_STAGE * 2);
    if (s != tail) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        dma16s_nt(woff[j], Wn + (int64_t)(kr + (wave + 4 * j) * 8) * ldw, base + (wave + 4 * j) * 1024);
      if (lane < 32) dma16s(xoff, X + kr, base + GV_WSLAB * 2 + wave * 512);
    } else {
      // rows past K are clamped to K-1 (valid memory, matched by zero x in
      // xtail); the x DMA re-reads the first 8 elements of the row (valid for
      // any K) so every wave issues the same number of ops per stage
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rb = min(kr + (wave + 4 * j) * 8, K - 1);
        const int r = min(kr + (wave + 4 * j) * 8 + (lane >> 3), K - 1) - rb;
        const uint32_t off = woff[j] - (uint32_t)((int64_t)(lane >> 3) * ldw * 2) + (uint32_t)((int64_t)r * ldw * 2);
        dma16s_nt(off, Wn + (int64_t)rb * ldw, base + (wave + 4 * j) * 1024);
      }
      if (lane < 32) dma16s(xoff_row, X, base + GV_WSLAB * 2 + wave * 512);
    }
  };

  // ---- prologue: STAGES-1 slabs in flight, then the zero-padded tail of x
#pragma unroll
  for (int s = 0; s < GV_STAGES - 1; ++s)
    if (s < nslab) issue(s);
  if (tail >= 0) {
    // 16 rows x 64 k, 8 elements per thread (threads 0..127), zero past M / K
    if (tid < 128) {
      const int m = tid >> 3, c = tid & 7;
      const int k = k_begin + tail * GV_SLAB + c * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M && k < K) v = *reinterpret_cast<const uint4 *>(X + (int64_t)m * ldx + k);
      *reinterpret_cast<uint4 *>(xtail + m * GV_SLAB + ((c ^ (m & 7)) << 3)) = v;
    }
  }

  // ---- stream the slabs
  f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int cw = wave * 16;  // this wave's columns within the strip
  const int s4 = l16 >> 2;
  const int colw = cw + 4 * (l16 & 3);
  for (int s = 0; s < nslab; ++s) {
    if (s + GV_STAGES - 2 < nslab) wait_vmcnt<GV_DMA * (GV_STAGES - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();  // slab s visible to all; every wave is done with slab s-1's stage
    if (s + GV_STAGES - 1 < nslab) issue(s + GV_STAGES - 1);
    const uint16_t *t = smem + (s % GV_STAGES) * GV_STAGE;
    const uint16_t *xt = (s == tail) ? xtail : t + GV_WSLAB;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int r1 = kc * 32 + 8 * g + s4;
      const int off = (((colw >> 3) ^ gv_swz(r1)) << 3) + (colw & 4);
      const uint2 u0 = tr_read(t + r1 * GV_BN + off);
      const uint2 u1 = tr_read(t + (r1 + 4) * GV_BN + off);
      const uint4 bf = make_uint4(u0.x, u0.y, u1.x, u1.y);
      const uint4 af = *reinterpret_cast<const uint4 *>(xt + l16 * GV_SLAB + (((kc * 4 + g) ^ (l16 & 7)) << 3));
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
  } else if constexpr (OUT == GV_PARTIAL) {
    *reinterpret_cast<float4 *>(part + ((int64_t)split * 16 + m) * N + col) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// Y[m][c] = epi(sum_s part[s][m][c] + bias), splits added in order.  One
// thread per 4 adjacent outputs of a token row (N is a multiple of 8, so a
// group never straddles rows and every access is a 16- or 8-byte vector),
// all of its (at most 16 per batch) partial loads issued before the first
// add, so the kernel costs about one memory latency.  One wave per
// workgroup spreads those loads over as many CUs as there are waves (224 for
// a 16 x 3584 output, against 56 with 256-thread workgroups: 14.30 -> 14.10
// us per packed column GEMV, interleaved on one box).
template <int EPI>
__global__ void __launch_bounds__(64)
gemv_finalize_kernel(const float *__restrict__ part, int splits, int M, int N,
                     const uint16_t *bias, void *Y, int64_t ldy) {
  const int v = blockIdx.x * 64 + threadIdx.x;
  const int n4 = N >> 2;
  if (v >= M * n4) return;
  const int m = v / n4, col = (v - m * n4) * 4;
  const float4 *p = reinterpret_cast<const float4 *>(part + (int64_t)m * N + col);
  const int64_t step = (int64_t)4 * N;  // float4s between splits
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += 16) {
    float4 t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      t[j] = (s0 + j < splits) ? p[(int64_t)(s0 + j) * step] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s0 + j < splits) {
        sum[0] += t[j].x; sum[1] += t[j].y; sum[2] += t[j].z; sum[3] += t[j].w;
      }
  }
  if (bias != nullptr) {
    const uint2 b = *reinterpret_cast<const uint2 *>(bias + col);
    sum[0] += bf2f((uint16_t)(b.x & 0xffffu)); sum[1] += bf2f((uint16_t)(b.x >> 16));
    sum[2] += bf2f((uint16_t)(b.y & 0xffffu)); sum[3] += bf2f((uint16_t)(b.y >> 16));
  }
  if constexpr (EPI == EPI_STORE_F32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(Y) + (int64_t)m * ldy + col) =
        make_float4(sum[0], sum[1], sum[2], sum[3]);
  } else {
    if constexpr (EPI == EPI_GELU) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] = gelu_f(sum[r]);
    }
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(Y) + (int64_t)m * ldy + col) =
        make_uint2(pack_bf2(sum[0], sum[1]), pack_bf2(sum[2], sum[3]));
  }
}

// Where strip s of W starts and how its rows are laid out: row-major W
// (strip origin 64 s, row stride ldw, columns clamped to N) or the panel
// layout of gemv_pack_kernel (strip origin s * Kp * 64, row stride 64, every
// column of a panel present).
struct GvSrc {
  int64_t ldw, sstride;
  int ncl;
};
static GvSrc gv_src(const GemvArgs &a, const GvPlan &pl) {
  if (a.packed) return GvSrc{GV_BN, gemv_panel_rows(a.K) * GV_BN, pl.strips * GV_BN};
  return GvSrc{a.ldw, GV_BN, (int)a.N};
}

template <int EPI>
static hipError_t run_gemv(const GemvArgs &a, const GvPlan &pl, hipStream_t s) {
  const uint16_t *X = static_cast<const uint16_t *>(a.X);
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const uint16_t *bias = static_cast<const uint16_t *>(a.bias);
  const GvSrc src = gv_src(a, pl);
  const dim3 grid((unsigned)pl.strips, (unsigned)pl.splits);
  if (pl.splits == 1) {
    hipLaunchKernelGGL((gemv_partial_kernel<EPI, GV_FINAL>), grid, dim3(GV_NT), 0, s, X, a.ldx,
                       (int)a.M, W, src.ldw, src.sstride, src.ncl, (int)a.K, (int)a.N, pl.krange, bias, a.Y,
                       a.ldy, (float *)nullptr);
    return hipGetLastError();
  }
  float *part = static_cast<float *>(a.ws);
  hipLaunchKernelGGL((gemv_partial_kernel<EPI, GV_PARTIAL>), grid, dim3(GV_NT), 0, s, X, a.ldx,
                     (int)a.M, W, src.ldw, src.sstride, src.ncl, (int)a.K, (int)a.N, pl.krange, bias, a.Y,
                     a.ldy, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = (int)a.M * (int)(a.N / 4);
  hipLaunchKernelGGL((gemv_finalize_kernel<EPI>), dim3((unsigned)((total + 63) / 64)), dim3(64),
                     0, s, part, pl.splits, (int)a.M, (int)a.N, bias, a.Y, a.ldy);
  return hipGetLastError();
}

bool gemv_fits(int64_t ldx, int64_t ldw) { return ldx <= GV_MAX_LD && ldw <= GV_MAX_LD; }

// ---------------------------------------------------------------- panel layout
// For decode, where the same weight is streamed once per generated token, a
// weight can be stored once in the order the split-K pass reads it: panel s
// holds columns 64 s .. 64 s + 63 of every row k < Kp (K rounded up to the
// 64-row slab), 128 bytes per row, zeros past K and past N:
//     Wp[(s * Kp + k) * 64 + c] = W[k][64 s + c]
// A workgroup's K range of one strip is then one contiguous run of
// krange * 128 bytes instead of 128 bytes from each of krange rows
// ldw * 2 bytes apart, and every 1 KiB DMA op covers 8 whole rows of it.
// The arithmetic (slabs, MFMA order, split order) is unchanged, so the
// results equal the row-major path's bit for bit.
int64_t gemv_panel_rows(int64_t K) { return (K + GV_SLAB - 1) / GV_SLAB * GV_SLAB; }

size_t gemv_packed_bytes(int64_t K, int64_t N) {
  return (size_t)((N + GV_BN - 1) / GV_BN) * (size_t)gemv_panel_rows(K) * GV_BN * sizeof(uint16_t);
}

// One thread per 16-byte granule of Wp (8 columns of one panel row).
__global__ void __launch_bounds__(256)
gemv_pack_kernel(const uint16_t *__restrict__ W, int64_t ldw, int K, int N, int64_t Kp, int64_t granules,
                 uint16_t *__restrict__ Wp) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= granules) return;
  const int64_t row = v >> 3;  // panel row over all panels: s * Kp + k
  const int64_t s = row / Kp, k = row - s * Kp;
  const int64_t col = s * GV_BN + (v & 7) * 8;
  uint4 g = make_uint4(0u, 0u, 0u, 0u);
  if (k < K && col < N) g = *reinterpret_cast<const uint4 *>(W + k * ldw + col);  // N % 8 == 0
  reinterpret_cast<uint4 *>(Wp)[v] = g;
}

hipError_t launch_gemv_pack(const uint16_t *W, int64_t ldw, int64_t K, int64_t N, uint16_t *Wp, hipStream_t s) {
  if (K <= 0 || N <= 0) return hipSuccess;
  if (N % 8 != 0 || ldw < N) return hipErrorInvalidValue;
  const int64_t Kp = gemv_panel_rows(K);
  const int64_t granules = (int64_t)gemv_packed_bytes(K, N) / 16;
  if ((granules + 255) / 256 > (int64_t)0x7fffffff) return hipErrorInvalidValue;  // one grid dimension
  hipLaunchKernelGGL(gemv_pack_kernel, dim3((unsigned)((granules + 255) / 256)), dim3(256), 0, s, W, ldw,
                     (int)K, (int)N, Kp, granules, Wp);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs &a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 16 || a.dtype != DT_BF16 || a.K < 1 || a.N < 8 || a.N % 8 != 0) return hipErrorInvalidValue;
  if (!gemv_fits(a.ldx, a.packed ? GV_BN : a.ldw)) return hipErrorInvalidValue;
  const GvPlan pl = gv_plan(a.K, a.N);
  if (pl.splits > 1 && (a.ws == nullptr || a.ws_bytes < gemv_workspace(a.K, a.N)))
    return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_GELU: return run_gemv<EPI_GELU>(a, pl, s);
    case EPI_STORE: return run_gemv<EPI_STORE>(a, pl, s);
    case EPI_STORE_F32: return run_gemv<EPI_STORE_F32>(a, pl, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- allocation-free variant
// For callers that cannot allocate (graph capture, serving loops): the
// split-K partials live in this file-scope device array instead of a caller
// workspace, and the same two kernels run (split-K pass, then the finalize
// that adds the partials in split order), so the results are those of
// launch_gemv bit for bit.  Every partial a call reads was written by that
// call's split-K pass, so nothing is cleared.  Each GPU holds its own copy
// until the process ends; calls that overlap on one GPU share it and race.
// Any decode shape fits: the plan keeps splits * strips <= GV_TARGET_WG, so
// the partials (splits * 16 * N fp32) take at most 512 * 64 * 16 * 4 bytes.
static constexpr size_t NA_PART_BYTES = (size_t)GV_TARGET_WG * GV_BN * 16 * sizeof(float);  // 2 MiB
static __device__ __align__(256) unsigned char scratch[NA_PART_BYTES];

size_t gemv_noalloc_max_bytes() { return NA_PART_BYTES; }

bool gemv_noalloc_fits(int64_t K, int64_t N) { return gemv_workspace(K, N) <= NA_PART_BYTES; }

namespace {
std::mutex g_na_mu;
void *g_na_ptr[64] = {};  // per device: the device address of that GPU's copy of scratch
}  // namespace

// Device address of the current device's scratch, looked up once per device
// (with that device current); nullptr on failure.
static unsigned char *noalloc_scratch(hipError_t *err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_na_mu);
  if (g_na_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_na_ptr[dev] = ptr;
  }
  return static_cast<unsigned char *>(g_na_ptr[dev]);
}

hipError_t launch_gemv_noalloc(const GemvArgs &a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.packed || !gemv_noalloc_fits(a.K, a.N)) return hipErrorInvalidValue;
  GemvArgs b = a;
  b.ws = nullptr;
  b.ws_bytes = 0;
  if (gv_plan(a.K, a.N).splits > 1) {
    hipError_t e = hipSuccess;
    unsigned char *base = noalloc_scratch(&e);
    if (base == nullptr) return e;
    b.ws = base;
    b.ws_bytes = NA_PART_BYTES;
  }
  return launch_gemv(b, s);
}

}  // namespace tpcol
