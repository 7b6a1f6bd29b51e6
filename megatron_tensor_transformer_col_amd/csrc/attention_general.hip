// Head-local attention and its backward for the shapes the flash kernels
// (bf16, head dim 128) do not take: fp32 or bf16 operands, any head dim up
// to 256 -- the pages' own TP attention example runs 8 heads over a hidden
// size of 128 (d = 16) in fp32 ("Megatron-LM 实战 04", TPAttention).
//
// Same definitions and layouts as the flash path: per (sequence, head)
//     O = softmax(Q K^T / sqrt(d) [+ causal mask]) V
// ("张量并行", Multi-Head Attention 的并行化: heads are independent), grouped
// query heads reading kv head t / g ("张量并行", 相关分析: GQA), Q | K | V
// packed per token row, lse = log2 of each row's softmax denominator in the
// scaled base-2 score domain, and the backward
//     dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO O),
//     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
// by the chain rule through the two products and the row softmax.
//
// These are plain SIMT kernels with fp32 arithmetic (correctness path for
// small and odd shapes; the benchmark shapes take the flash kernels):
// 16-query / 16-key tiles in LDS as fp32, one thread per (query, key) score
// and one thread per (row, 16-strided dims) accumulator.  Every sum runs in
// a fixed order and no workgroup waits on another.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int AG_Q = 16;       // queries per tile
static constexpr int AG_K = 16;       // keys per tile
static constexpr int AG_DMAX = 256;   // largest head dim
static constexpr int AG_NT = 256;     // threads: 16 rows x 16
static constexpr int AG_J = AG_DMAX / 16;  // accumulator dims per thread

template <typename T>
__device__ __forceinline__ float ag_ld(const T *p) {
  if constexpr (sizeof(T) == 2) return bf2f(*p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void ag_st(T *p, float v) {
  if constexpr (sizeof(T) == 2) *p = f2bf(v);
  else *p = v;
}

struct AgArgs {
  const void *qkv;  // [b*s][(hl + 2 kvl) d]: Q heads, then K heads, then V heads
  int64_t ldq;
  const void *O;    // [b*s][hl d] (forward: written)
  int64_t ldo;
  const void *dO;   // backward
  int64_t lddo;
  float *lse;       // [b][hl][s], base 2, scaled scores
  float *Dr;        // [b][hl][s] (backward)
  void *dqkv;       // packed like qkv (backward)
  int s, hl, kvl, group, d;
  float scale_log2;  // log2(e) / sqrt(d)
  float scale;       // 1 / sqrt(d)
};

// rows x d tile of an operand (rows past s read as 0) into fp32 LDS
template <typename T, int LD>
__device__ __forceinline__ void ag_tile(float (*dst)[LD], const T *g, int64_t ld, int r0, int s, int d) {
  for (int e = threadIdx.x; e < 16 * d; e += AG_NT) {
    const int r = e / d, c = e - r * d;
    dst[r][c] = r0 + r < s ? ag_ld(g + (int64_t)(r0 + r) * ld + c) : 0.f;
  }
}

// ---------------------------------------------------------------- forward
// Workgroup: 16 queries of one (sequence, head); thread (qr, cl) keeps the
// running max / sum of query qr and its output dims cl, cl + 16, ...
template <typename T, bool CAUSAL>
__global__ void __launch_bounds__(AG_NT) attn_gen_fwd_kernel(AgArgs a) {
  __shared__ float Qs[AG_Q][AG_DMAX];
  __shared__ float Ks[AG_K][AG_DMAX + 1];
  __shared__ float Vs[AG_K][AG_DMAX];
  __shared__ float Ss[AG_Q][AG_K];
  const int tid = threadIdx.x;
  const int bi = blockIdx.y / a.hl, head = blockIdx.y % a.hl, kvh = head / a.group;
  const int d = a.d;
  const int64_t tok0 = (int64_t)bi * a.s;
  const T *qkv = static_cast<const T *>(a.qkv);
  const T *Qg = qkv + tok0 * a.ldq + (int64_t)head * d;
  const T *Kg = qkv + tok0 * a.ldq + (int64_t)(a.hl + kvh) * d;
  const T *Vg = qkv + tok0 * a.ldq + (int64_t)(a.hl + a.kvl + kvh) * d;
  const int q0 = blockIdx.x * AG_Q;
  ag_tile<T, AG_DMAX>(Qs, Qg, a.ldq, q0, a.s, d);

  const int qr = tid >> 4, cl = tid & 15;
  float o[AG_J];
#pragma unroll
  for (int j = 0; j < AG_J; ++j) o[j] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? min(a.s, q0 + AG_Q) : a.s;
  for (int k0 = 0; k0 < kend; k0 += AG_K) {
    __syncthreads();  // the Q tile is in; the previous tile's readers are done
    ag_tile<T, AG_DMAX + 1>(Ks, Kg, a.ldq, k0, a.s, d);
    ag_tile<T, AG_DMAX>(Vs, Vg, a.ldq, k0, a.s, d);
    __syncthreads();
    {
      const int sq = tid >> 4, sk = tid & 15;
      float acc = 0.f;
      for (int c = 0; c < d; ++c) acc += Qs[sq][c] * Ks[sk][c];
      const int q = q0 + sq, k = k0 + sk;
      const bool ok = k < a.s && (!CAUSAL || k <= q);
      Ss[sq][sk] = ok ? acc * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    float mx = m;
#pragma unroll
    for (int k = 0; k < AG_K; ++k) mx = fmaxf(mx, Ss[qr][k]);
    if (mx == -INFINITY) continue;  // every key so far masked for this query
    const float alpha = exp2f(m - mx);  // 0 on the first unmasked tile
    float p[AG_K];
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < AG_K; ++k) {
      p[k] = exp2f(Ss[qr][k] - mx);
      ps += p[k];
    }
    l = l * alpha + ps;
    m = mx;
#pragma unroll
    for (int j = 0; j < AG_J; ++j) {
      const int c = cl + 16 * j;
      if (c < d) {
        float acc = o[j] * alpha;
#pragma unroll
        for (int k = 0; k < AG_K; ++k) acc += p[k] * Vs[k][c];
        o[j] = acc;
      }
    }
  }
  const int q = q0 + qr;
  if (q >= a.s) return;
  const float inv = 1.0f / l;  // the diagonal key is never masked: l >= 1
  T *orow = static_cast<T *>(const_cast<void *>(a.O)) + (tok0 + q) * a.ldo + (int64_t)head * d;
#pragma unroll
  for (int j = 0; j < AG_J; ++j) {
    const int c = cl + 16 * j;
    if (c < d) ag_st(orow + c, o[j] * inv);
  }
  if (a.lse != nullptr && cl == 0) a.lse[((int64_t)bi * a.hl + head) * a.s + q] = m + log2f(l);
}

// ---------------------------------------------------------------- backward
// D[(bi*hl + head)*s + q] = sum_c dO[t][head d + c] O[t][head d + c]; one
// thread per (token, head)
template <typename T>
__global__ void __launch_bounds__(256) attn_gen_dot_kernel(AgArgs a, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int64_t t = r / a.hl;
  const int head = (int)(r % a.hl);
  const T *o = static_cast<const T *>(a.O) + t * a.ldo + (int64_t)head * a.d;
  const T *g = static_cast<const T *>(a.dO) + t * a.lddo + (int64_t)head * a.d;
  float acc = 0.f;
  for (int c = 0; c < a.d; ++c) acc += ag_ld(g + c) * ag_ld(o + c);
  const int64_t bi = t / a.s, q = t % a.s;
  a.Dr[(bi * a.hl + head) * a.s + q] = acc;
}

// P[sq][sk] and dS[sq][sk] of a 16 x 16 (query, key) tile from the Q, dO, K,
// V tiles in LDS; thread (sq, sk) = (tid / 16, tid % 16)
template <bool CAUSAL, int LQ, int LK>
__device__ __forceinline__ void ag_p_ds(const AgArgs &a, const float (*Qs)[LQ], const float (*dOs)[LQ],
                                        const float (*Ks)[LK], const float (*Vs)[LK], const float *lse2,
                                        const float *Dq, int q0, int k0, float &p, float &ds) {
  const int sq = threadIdx.x >> 4, sk = threadIdx.x & 15;
  float sc = 0.f, dp = 0.f;
  for (int c = 0; c < a.d; ++c) {
    sc += Qs[sq][c] * Ks[sk][c];
    dp += dOs[sq][c] * Vs[sk][c];
  }
  const int q = q0 + sq, k = k0 + sk;
  const bool ok = q < a.s && k < a.s && (!CAUSAL || k <= q);
  p = ok ? exp2f(sc * a.scale_log2 - lse2[sq]) : 0.f;
  ds = p * (dp - Dq[sq]);
}

// dQ for 16 queries of one (sequence, head): thread (qr, cl) accumulates
// dims cl, cl + 16, ... of query qr over the key tiles
template <typename T, bool CAUSAL>
__global__ void __launch_bounds__(AG_NT) attn_gen_dq_kernel(AgArgs a) {
  __shared__ float Qs[AG_Q][AG_DMAX];
  __shared__ float dOs[AG_Q][AG_DMAX];
  __shared__ float Ks[AG_K][AG_DMAX + 1];
  __shared__ float Vs[AG_K][AG_DMAX + 1];
  __shared__ float dSs[AG_Q][AG_K];
  __shared__ float lse2[AG_Q], Dq[AG_Q];
  const int tid = threadIdx.x;
  const int bi = blockIdx.y / a.hl, head = blockIdx.y % a.hl, kvh = head / a.group;
  const int d = a.d;
  const int64_t tok0 = (int64_t)bi * a.s;
  const T *qkv = static_cast<const T *>(a.qkv);
  const T *Kg = qkv + tok0 * a.ldq + (int64_t)(a.hl + kvh) * d;
  const T *Vg = qkv + tok0 * a.ldq + (int64_t)(a.hl + a.kvl + kvh) * d;
  const int q0 = blockIdx.x * AG_Q;
  ag_tile<T, AG_DMAX>(Qs, qkv + tok0 * a.ldq + (int64_t)head * d, a.ldq, q0, a.s, d);
  ag_tile<T, AG_DMAX>(dOs, static_cast<const T *>(a.dO) + tok0 * a.lddo + (int64_t)head * d, a.lddo, q0, a.s, d);
  if (tid < AG_Q) {
    const int q = min(q0 + tid, a.s - 1);
    const int64_t r = ((int64_t)bi * a.hl + head) * a.s + q;
    lse2[tid] = a.lse[r];
    Dq[tid] = a.Dr[r];
  }
  const int qr = tid >> 4, cl = tid & 15;
  float dq[AG_J];
#pragma unroll
  for (int j = 0; j < AG_J; ++j) dq[j] = 0.f;
  const int kend = CAUSAL ? min(a.s, q0 + AG_Q) : a.s;
  for (int k0 = 0; k0 < kend; k0 += AG_K) {
    __syncthreads();
    ag_tile<T, AG_DMAX + 1>(Ks, Kg, a.ldq, k0, a.s, d);
    ag_tile<T, AG_DMAX + 1>(Vs, Vg, a.ldq, k0, a.s, d);
    __syncthreads();
    float p, ds;
    ag_p_ds<CAUSAL>(a, Qs, dOs, Ks, Vs, lse2, Dq, q0, k0, p, ds);
    dSs[tid >> 4][tid & 15] = ds;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < AG_J; ++j) {
      const int c = cl + 16 * j;
      if (c < d) {
        float acc = dq[j];
#pragma unroll
        for (int k = 0; k < AG_K; ++k) acc += dSs[qr][k] * Ks[k][c];
        dq[j] = acc;
      }
    }
  }
  const int q = q0 + qr;
  if (q >= a.s) return;
  T *row = static_cast<T *>(a.dqkv) + (tok0 + q) * a.ldq + (int64_t)head * d;
#pragma unroll
  for (int j = 0; j < AG_J; ++j) {
    const int c = cl + 16 * j;
    if (c < d) ag_st(row + c, dq[j] * a.scale);
  }
}

// dK and dV for 16 keys of one (sequence, kv head), summed over the group's
// query heads in head order and over the query tiles in order: thread
// (kr, cl) accumulates dims cl, cl + 16, ... of key kr
template <typename T, bool CAUSAL>
__global__ void __launch_bounds__(AG_NT) attn_gen_dkdv_kernel(AgArgs a) {
  __shared__ float Qs[AG_Q][AG_DMAX];
  __shared__ float dOs[AG_Q][AG_DMAX];
  __shared__ float Ks[AG_K][AG_DMAX + 1];
  __shared__ float Vs[AG_K][AG_DMAX + 1];
  __shared__ float Ps[AG_Q][AG_K + 1];
  __shared__ float dSs[AG_Q][AG_K + 1];
  __shared__ float lse2[AG_Q], Dq[AG_Q];
  const int tid = threadIdx.x;
  const int bi = blockIdx.y / a.kvl, kvh = blockIdx.y % a.kvl;
  const int d = a.d;
  const int64_t tok0 = (int64_t)bi * a.s;
  const T *qkv = static_cast<const T *>(a.qkv);
  const int k0 = blockIdx.x * AG_K;
  ag_tile<T, AG_DMAX + 1>(Ks, qkv + tok0 * a.ldq + (int64_t)(a.hl + kvh) * d, a.ldq, k0, a.s, d);
  ag_tile<T, AG_DMAX + 1>(Vs, qkv + tok0 * a.ldq + (int64_t)(a.hl + a.kvl + kvh) * d, a.ldq, k0, a.s, d);
  const int kr = tid >> 4, cl = tid & 15;
  float dk[AG_J], dv[AG_J];
#pragma unroll
  for (int j = 0; j < AG_J; ++j) dk[j] = dv[j] = 0.f;
  for (int t = 0; t < a.group; ++t) {
    const int head = kvh * a.group + t;
    const T *Qg = qkv + tok0 * a.ldq + (int64_t)head * d;
    const T *dOg = static_cast<const T *>(a.dO) + tok0 * a.lddo + (int64_t)head * d;
    // causal: the queries before k0 see none of these keys
    for (int q0 = CAUSAL ? k0 : 0; q0 < a.s; q0 += AG_Q) {
      __syncthreads();  // the previous tile's readers are done (and K, V are in)
      ag_tile<T, AG_DMAX>(Qs, Qg, a.ldq, q0, a.s, d);
      ag_tile<T, AG_DMAX>(dOs, dOg, a.lddo, q0, a.s, d);
      if (tid < AG_Q) {
        const int q = min(q0 + tid, a.s - 1);
        const int64_t r = ((int64_t)bi * a.hl + head) * a.s + q;
        lse2[tid] = a.lse[r];
        Dq[tid] = a.Dr[r];
      }
      __syncthreads();
      float p, ds;
      ag_p_ds<CAUSAL>(a, Qs, dOs, Ks, Vs, lse2, Dq, q0, k0, p, ds);
      Ps[tid >> 4][tid & 15] = p;
      dSs[tid >> 4][tid & 15] = ds;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < AG_J; ++j) {
        const int c = cl + 16 * j;
        if (c < d) {
          float av = dv[j], ak = dk[j];
#pragma unroll
          for (int q = 0; q < AG_Q; ++q) {
            av += Ps[q][kr] * dOs[q][c];
            ak += dSs[q][kr] * Qs[q][c];
          }
          dv[j] = av;
          dk[j] = ak;
        }
      }
    }
  }
  const int k = k0 + kr;
  if (k >= a.s) return;
  T *krow = static_cast<T *>(a.dqkv) + (tok0 + k) * a.ldq + (int64_t)(a.hl + kvh) * d;
  T *vrow = static_cast<T *>(a.dqkv) + (tok0 + k) * a.ldq + (int64_t)(a.hl + a.kvl + kvh) * d;
#pragma unroll
  for (int j = 0; j < AG_J; ++j) {
    const int c = cl + 16 * j;
    if (c < d) {
      ag_st(krow + c, dk[j] * a.scale);
      ag_st(vrow + c, dv[j]);
    }
  }
}

// ---------------------------------------------------------------- host side
static AgArgs ag_args(const void *qkv, int64_t ldq, const void *O, int64_t ldo, float *lse, int64_t s,
                      int64_t hl, int64_t kvl, int64_t d) {
  AgArgs a{};
  a.qkv = qkv; a.ldq = ldq;
  a.O = O; a.ldo = ldo;
  a.lse = lse;
  a.s = (int)s; a.hl = (int)hl; a.kvl = (int)kvl; a.group = (int)(hl / kvl); a.d = (int)d;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  a.scale = 1.0f / sqrtf((float)d);
  return a;
}

bool attn_general_fits(int64_t s, int64_t d) { return d >= 1 && d <= AG_DMAX && s <= (int64_t(1) << 30); }

template <typename T>
static hipError_t gen_fwd(const AgArgs &a, int64_t b, bool causal, hipStream_t st) {
  const dim3 grid((unsigned)((a.s + AG_Q - 1) / AG_Q), (unsigned)(b * a.hl));
  if (causal) hipLaunchKernelGGL((attn_gen_fwd_kernel<T, true>), grid, dim3(AG_NT), 0, st, a);
  else hipLaunchKernelGGL((attn_gen_fwd_kernel<T, false>), grid, dim3(AG_NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_general(int dtype, const void *qkv, int64_t ldqkv, void *O, int64_t ldo, float *lse,
                               int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d, bool causal,
                               hipStream_t st) {
  if (b <= 0 || s <= 0 || hl <= 0) return hipSuccess;
  if (!attn_general_fits(s, d) || kvl < 1 || hl % kvl) return hipErrorInvalidValue;
  if (b * hl > 65535) return hipErrorInvalidValue;  // grid y
  const AgArgs a = ag_args(qkv, ldqkv, O, ldo, lse, s, hl, kvl, d);
  return dtype == DT_BF16 ? gen_fwd<uint16_t>(a, b, causal, st) : gen_fwd<float>(a, b, causal, st);
}

template <typename T>
static hipError_t gen_bwd(const AgArgs &a, int64_t b, bool causal, hipStream_t st) {
  const int64_t rows = b * (int64_t)a.s * a.hl;
  hipLaunchKernelGGL((attn_gen_dot_kernel<T>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)((a.s + 15) / 16);
  const dim3 gq(tiles, (unsigned)(b * a.hl)), gk(tiles, (unsigned)(b * a.kvl));
  if (causal) {
    hipLaunchKernelGGL((attn_gen_dq_kernel<T, true>), gq, dim3(AG_NT), 0, st, a);
    hipLaunchKernelGGL((attn_gen_dkdv_kernel<T, true>), gk, dim3(AG_NT), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_gen_dq_kernel<T, false>), gq, dim3(AG_NT), 0, st, a);
    hipLaunchKernelGGL((attn_gen_dkdv_kernel<T, false>), gk, dim3(AG_NT), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd_general(int dtype, const void *qkv, int64_t ldqkv, const void *O, int64_t ldo,
                                   const float *lse, const void *dO, int64_t lddo, float *Dr, void *dqkv,
                                   int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d, bool causal,
                                   hipStream_t st) {
  if (b <= 0 || s <= 0 || hl <= 0) return hipSuccess;
  if (!attn_general_fits(s, d) || kvl < 1 || hl % kvl) return hipErrorInvalidValue;
  if (b * hl > 65535) return hipErrorInvalidValue;
  AgArgs a = ag_args(qkv, ldqkv, O, ldo, const_cast<float *>(lse), s, hl, kvl, d);
  a.dO = dO; a.lddo = lddo;
  a.Dr = Dr;
  a.dqkv = dqkv;
  return dtype == DT_BF16 ? gen_bwd<uint16_t>(a, b, causal, st) : gen_bwd<float>(a, b, causal, st);
}

}  // namespace tpcol
