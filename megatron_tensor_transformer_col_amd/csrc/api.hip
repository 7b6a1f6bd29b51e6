// C ABI of the tensor-parallel shard library: argument validation, path
// selection and kernel sequencing.  Declarations and contracts are in
// include/tpcol.h.  Every check runs before the first launch, so a failing
// call enqueues nothing.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/tpcol.h"
#include "kernels.hpp"

using namespace tpcol;

namespace {

thread_local char g_err[512] = "";

// Initial GEMV threshold: TPCOL_GEMV_MAX_M from the environment when the
// library loads (an integer 0..16; anything else keeps the default 16).
int initial_gemv_max_m() {
  const char *v = getenv("TPCOL_GEMV_MAX_M");
  if (v == nullptr || *v == '\0') return 16;
  char *end = nullptr;
  const long m = strtol(v, &end, 10);
  return (*end == '\0' && m >= 0 && m <= 16) ? (int)m : 16;
}
std::atomic<int> g_gemv_max_m{initial_gemv_max_m()};

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return TP_OK;
}

size_t esize(int dtype) { return dtype == TP_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == TP_F32 || dtype == TP_BF16; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // kernels index rows/cols with int

// A [rows x cols] row-major matrix with row stride ld elements of size es.
// An empty matrix (rows == 0) may have a NULL pointer.
int check_mat(const void *p, int64_t rows, int64_t cols, int64_t ld, size_t es, const char *name,
              bool required = true) {
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim)
    return fail(TP_ERR_SHAPE, "%s has an invalid shape %lld x %lld", name, (long long)rows,
                (long long)cols);
  if (p == nullptr) {
    if (required && rows > 0) return fail(TP_ERR_ARG, "%s is NULL", name);
    return TP_OK;
  }
  if (ld < cols)
    return fail(TP_ERR_SHAPE, "%s: leading dimension %lld < width %lld", name, (long long)ld,
                (long long)cols);
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return fail(TP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (((size_t)ld * es) % 16 != 0)
    return fail(TP_ERR_ALIGN, "%s: leading dimension %lld is not a multiple of 16 bytes", name,
                (long long)ld);
  if (((size_t)cols * es) % 16 != 0)
    return fail(TP_ERR_ALIGN, "%s: width %lld is not a multiple of %zu elements", name,
                (long long)cols, 16 / es);
  return TP_OK;
}

int check_vec(const void *p, int64_t n, size_t es, const char *name) {
  if (p == nullptr) return TP_OK;  // optional vectors
  return check_mat(p, 1, n, n, es, name);
}

// a device array with no row-width rule: non-NULL (when required) and
// aligned to `align` bytes
int check_arr(const void *p, bool required, size_t align, const char *name) {
  if (p == nullptr) return required ? fail(TP_ERR_ARG, "%s is NULL", name) : TP_OK;
  if ((reinterpret_cast<uintptr_t>(p) % align) != 0)
    return fail(TP_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return TP_OK;
}

// a row-major matrix read element by element (any width and stride): non-NULL
// when it has rows, element-aligned, ld >= cols
int check_rows(const void *p, int64_t rows, int64_t cols, int64_t ld, size_t es, const char *name) {
  if (p == nullptr) return rows > 0 ? fail(TP_ERR_ARG, "%s is NULL", name) : TP_OK;
  if ((reinterpret_cast<uintptr_t>(p) % es) != 0) return fail(TP_ERR_ALIGN, "%s is not %zu-byte aligned", name, es);
  if (ld < cols)
    return fail(TP_ERR_SHAPE, "%s: leading dimension %lld < width %lld", name, (long long)ld, (long long)cols);
  return TP_OK;
}

int check_dims(std::initializer_list<int64_t> dims, const char *what) {
  for (int64_t d : dims)
    if (d < 0 || d > kMaxDim) return fail(TP_ERR_SHAPE, "%s: dimension %lld out of range", what, (long long)d);
  return TP_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TP_OK;
}

#define TRY(x)               \
  do {                       \
    const int _st = (x);     \
    if (_st != TP_OK) return _st; \
  } while (0)

bool use_gemv(int dtype, int64_t M) {
  return dtype == TP_BF16 && M >= 1 && M <= g_gemv_max_m.load(std::memory_order_relaxed);
}

// Backward workspace layout: dH [M x Ni], (GELU: as much again,) H [M x Ni],
// dZ [M x Ni] (GELU) or [M x 2Ni] = [dZg | dZu] (SwiGLU); each region
// 256-byte aligned.  Once the recompute has consumed dH, [dH, H) holds the
// fp32 K-range partials of the weight-gradient products.
struct BwdWs {
  size_t dH, H, dZ, cs, total;
};
// dH_i, H_i, dZ_i (SwiGLU: [dZg | dZu]); GELU / no activation also the
// fp32 column-sum partials of db1 and a second dH-sized region, so that the
// two weight gradients' partials fit together
BwdWs bwd_ws(int dtype, int act, int64_t M, int64_t Ni) {
  const size_t e = esize(dtype);
  const size_t one = round256((size_t)M * (size_t)Ni * e);
  BwdWs w;
  w.dH = 0;
  w.H = act == TP_ACT_SWIGLU ? one : 2 * one;
  w.dZ = w.H + one;
  w.cs = w.dZ + (act == TP_ACT_SWIGLU ? round256((size_t)M * 2 * (size_t)Ni * e) : one);
  w.total = w.cs + (act == TP_ACT_SWIGLU ? 0 : round256(colsum_workspace(M, Ni)));
  return w;
}

// the flash kernels take bf16 with head dim 128; every other shape runs the
// general attention kernels
bool attn_fast(int dtype, int64_t d) { return dtype == TP_BF16 && d == 128; }

// forward workspace: packed QKV_i, O_i (dtype) and the per-row softmax
// statistic (fp32 [b][hl][s]) the backward reads
struct AttnWs {
  size_t qkv, o, lse, total;
};
AttnWs attn_ws(int dtype, int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d) {
  const size_t T = (size_t)b * (size_t)s, e = esize(dtype);
  AttnWs w;
  w.qkv = 0;
  w.o = round256(T * (size_t)(hl + 2 * kvl) * (size_t)d * e);
  w.lse = w.o + round256(T * (size_t)hl * (size_t)d * e);
  w.total = w.lse + round256(T * (size_t)hl * 4);
  return w;
}

// backward workspace: dO_i (dtype [T x hl*d]), D (fp32 [b][hl][s]),
// dQKV_i (dtype, packed like QKV_i) and, for the flash kernels' split
// grouped-query heads, fp32 dK / dV partials
struct AttnBwdWs {
  size_t dO, D, dqkv, part, total;
};
AttnBwdWs attn_bwd_ws(int dtype, int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d) {
  const size_t T = (size_t)b * (size_t)s, e = esize(dtype);
  AttnBwdWs w;
  w.dO = 0;
  w.D = round256(T * (size_t)hl * (size_t)d * e);
  w.dqkv = w.D + round256(T * (size_t)hl * 4);
  w.part = w.dqkv + round256(T * (size_t)(hl + 2 * kvl) * (size_t)d * e);
  w.total = w.part + (attn_fast(dtype, d) ? round256(attn_bwd_part_bytes(b, s, hl, kvl)) : 0);
  return w;
}

}  // namespace

namespace {
// Shape rules of the attention entry points (after check_dims): head counts,
// kv grouping, head dim (128 for the flash kernels' bf16 path, 1..256
// otherwise), 16-byte rows of the packed Q|K|V and O buffers.
int check_attn_shape(int dtype, int64_t b, int64_t s_len, int64_t h, int64_t heads_local, int64_t kv_heads_local,
                     int64_t d) {
  if (h < 1 || heads_local < 1) return fail(TP_ERR_SHAPE, "h and heads_local must be >= 1");
  if (kv_heads_local < 1 || heads_local % kv_heads_local)
    return fail(TP_ERR_SHAPE, "heads_local %lld is not a multiple of kv_heads_local %lld",
                (long long)heads_local, (long long)kv_heads_local);
  if (!attn_fast(dtype, d) && !attn_general_fits(s_len, d))
    return fail(TP_ERR_SHAPE, "head dim %lld outside 1..256", (long long)d);
  if (b * s_len > kMaxDim) return fail(TP_ERR_SHAPE, "b*s too large");
  if (!attn_fast(dtype, d) && b * heads_local > 65535)
    return fail(TP_ERR_SHAPE, "b*heads_local must be <= 65535 for head dim %lld", (long long)d);
  const int64_t wqkv = (heads_local + 2 * kv_heads_local) * d;
  if (wqkv > (int64_t(1) << 24))
    return fail(TP_ERR_SHAPE, "(heads_local + 2*kv_heads_local)*d must be <= 2^24");
  if (((size_t)(heads_local * d) * esize(dtype)) % 16 != 0)
    return fail(TP_ERR_ALIGN, "heads_local*d*element size must be a multiple of 16 bytes");
  return TP_OK;
}

int attn_impl(const char *fn, int dtype, int64_t b, int64_t s_len, int64_t h, int64_t heads_local,
                     int64_t kv_heads_local, int64_t d, int causal, const void *X, int64_t ldx,
                     const void *Wqkv, int64_t ldwqkv, const void *Wo, int64_t ldwo, float *P,
                     int64_t ldp, void *ws, size_t ws_bytes, void *stream) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  TRY(check_dims({b, s_len, h, heads_local, kv_heads_local, d}, fn));
  TRY(check_attn_shape(dtype, b, s_len, h, heads_local, kv_heads_local, d));
  const size_t e = esize(dtype);
  const int64_t T = b * s_len;
  const int64_t w = heads_local * d;
  const int64_t wqkv = (heads_local + 2 * kv_heads_local) * d;
  TRY(check_mat(X, T, h, ldx, e, "X"));
  TRY(check_mat(Wqkv, h, wqkv, ldwqkv, e, "Wqkv"));
  TRY(check_mat(Wo, w, h, ldwo, e, "Wo"));
  TRY(check_mat(P, T, h, ldp, 4, "P"));
  if (T == 0) return ok();
  const AttnWs L = attn_ws(dtype, b, s_len, heads_local, kv_heads_local, d);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", L.total, ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  void *qkv = base + L.qkv;
  void *O = base + L.o;
  float *lse = reinterpret_cast<float *>(base + L.lse);

  GemmArgs q;
  q.dtype = dtype;
  q.layout = LAY_NN;
  q.epi = EPI_STORE;
  q.M = T; q.N = wqkv; q.K = h;
  q.A = X; q.lda = ldx;
  q.B = Wqkv; q.ldb = ldwqkv;
  q.C = qkv; q.ldc = wqkv;
  TRY(hip_status(launch_gemm(q, st), "QKV GEMM"));
  if (attn_fast(dtype, d))
    TRY(hip_status(launch_flash_attn(qkv, wqkv, O, w, lse, b, s_len, heads_local, kv_heads_local, d,
                                     causal != 0, st),
                   "attention"));
  else
    TRY(hip_status(launch_attn_general(dtype, qkv, wqkv, O, w, lse, b, s_len, heads_local, kv_heads_local, d,
                                       causal != 0, st),
                   "attention"));
  GemmArgs o;
  o.dtype = dtype;
  o.layout = LAY_NN;
  o.epi = EPI_STORE_F32;
  o.M = T; o.N = h; o.K = w;
  o.A = O; o.lda = w;
  o.B = Wo; o.ldb = ldwo;
  o.C = P; o.ldc = ldp;
  TRY(hip_status(launch_gemm(o, st), "output GEMM"));
  return ok();
}

int attn_bwd_impl(int dtype, int64_t b, int64_t s_len, int64_t h, int64_t heads_local,
                  int64_t kv_heads_local, int64_t d, int causal, const void *X, int64_t ldx,
                  const void *Wqkv, int64_t ldwqkv, const void *Wo, int64_t ldwo, const void *dY,
                  int64_t lddy, const void *fwd_ws, size_t fwd_ws_bytes, float *dWqkv, float *dWo,
                  float *dXi, int64_t lddx, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "tp_attn_shard_backward";
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  TRY(check_dims({b, s_len, h, heads_local, kv_heads_local, d}, fn));
  TRY(check_attn_shape(dtype, b, s_len, h, heads_local, kv_heads_local, d));
  const size_t e = esize(dtype);
  const int64_t T = b * s_len;
  const int64_t w = heads_local * d;
  const int64_t wqkv = (heads_local + 2 * kv_heads_local) * d;
  TRY(check_mat(X, T, h, ldx, e, "X"));
  TRY(check_mat(Wqkv, h, wqkv, ldwqkv, e, "Wqkv"));
  TRY(check_mat(Wo, w, h, ldwo, e, "Wo"));
  TRY(check_mat(dY, T, h, lddy, e, "dY"));
  TRY(check_mat(dWqkv, h, wqkv, wqkv, 4, "dWqkv"));
  TRY(check_mat(dWo, w, h, h, 4, "dWo"));
  TRY(check_mat(dXi, T, h, lddx, 4, "dXi"));
  if (dWqkv == nullptr || dWo == nullptr) return fail(TP_ERR_ARG, "dWqkv and dWo are required");
  const AttnWs F = attn_ws(dtype, b, s_len, heads_local, kv_heads_local, d);
  const AttnBwdWs L = attn_bwd_ws(dtype, b, s_len, heads_local, kv_heads_local, d);
  if (T > 0) {
    if (fwd_ws == nullptr || fwd_ws_bytes < F.total)
      return fail(TP_ERR_WORKSPACE, "the forward's workspace (%zu bytes) is required, got %zu", F.total,
                  fwd_ws_bytes);
    if (ws == nullptr || ws_bytes < L.total)
      return fail(TP_ERR_WORKSPACE, "attention backward needs %zu workspace bytes, got %zu", L.total, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || (reinterpret_cast<uintptr_t>(fwd_ws) & 255u) != 0)
      return fail(TP_ERR_ALIGN, "workspaces must be 256-byte aligned");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char *fb = static_cast<const char *>(fwd_ws);
  const void *qkv = fb + F.qkv;
  const void *O = fb + F.o;
  const float *lse = reinterpret_cast<const float *>(fb + F.lse);
  char *base = static_cast<char *>(ws);
  void *dO = base + L.dO;
  float *Dr = reinterpret_cast<float *>(base + L.D);
  void *dqkv = base + L.dqkv;
  float *part = L.total > L.part ? reinterpret_cast<float *>(base + L.part) : nullptr;

  if (T > 0) {
    // dO_i = dY Wo_i^T  (row-parallel output projection, input gradient)
    GemmArgs a;
    a.dtype = dtype; a.layout = LAY_NT; a.epi = EPI_STORE;
    a.M = T; a.N = w; a.K = h;
    a.A = dY; a.lda = lddy;
    a.B = Wo; a.ldb = ldwo;
    a.C = dO; a.ldc = w;
    TRY(hip_status(launch_gemm(a, st), "dO GEMM"));
  }
  // dWo_i = O_i^T dY  (row-parallel weight gradient)
  {
    GemmArgs g;
    g.dtype = dtype; g.layout = LAY_TN; g.epi = EPI_STORE_F32;
    g.M = w; g.N = h; g.K = T;
    g.A = O; g.lda = w;
    g.B = dY; g.ldb = lddy;
    g.C = dWo; g.ldc = h;
    // dQKV_i and the head-split partials are written only by the attention
    // kernels below: until then their regions hold split-K partials
    g.part = reinterpret_cast<float *>(dqkv); g.part_bytes = L.total - L.dqkv;
    TRY(hip_status(launch_gemm(g, st), "dWo GEMM"));
  }
  if (T > 0 && attn_fast(dtype, d))
    TRY(hip_status(launch_attn_bwd(qkv, wqkv, O, w, lse, dO, w, Dr, dqkv, part, b, s_len, heads_local,
                                   kv_heads_local, d, causal != 0, st),
                   "attention backward"));
  else if (T > 0)
    TRY(hip_status(launch_attn_bwd_general(dtype, qkv, wqkv, O, w, lse, dO, w, Dr, dqkv, b, s_len, heads_local,
                                           kv_heads_local, d, causal != 0, st),
                   "attention backward"));
  // dWqkv_i = X^T dQKV_i  (column-parallel weight gradient)
  {
    GemmArgs g;
    g.dtype = dtype; g.layout = LAY_TN; g.epi = EPI_STORE_F32;
    g.M = h; g.N = wqkv; g.K = T;
    g.A = X; g.lda = ldx;
    g.B = dqkv; g.ldb = wqkv;
    g.C = dWqkv; g.ldc = wqkv;
    TRY(hip_status(launch_gemm(g, st), "dWqkv GEMM"));
  }
  if (T > 0) {
    // dX_i = dQKV_i Wqkv_i^T  (this shard's partial of dX)
    GemmArgs x;
    x.dtype = dtype; x.layout = LAY_NT; x.epi = EPI_STORE_F32;
    x.M = T; x.N = h; x.K = wqkv;
    x.A = dqkv; x.lda = wqkv;
    x.B = Wqkv; x.ldb = ldwqkv;
    x.C = dXi; x.ldc = lddx;
    TRY(hip_status(launch_gemm(x, st), "dX GEMM"));
  }
  return ok();
}

}  // namespace

extern "C" {

const char *tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "TP_OK: success";
    case TP_ERR_ARG: return "TP_ERR_ARG: invalid or missing argument";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE: invalid shape or split";
    case TP_ERR_ALIGN: return "TP_ERR_ALIGN: pointer or stride not 16-byte vectorisable";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE: unsupported dtype";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_HIP: return "TP_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char *tp_last_error(void) { return g_err; }

int tp_set_gemv_max_m(int max_m) {
  if (max_m < 0 || max_m > 16) return fail(TP_ERR_ARG, "gemv threshold %d outside 0..16", max_m);
  return g_gemv_max_m.exchange(max_m);
}

int tp_check_split(int64_t h, int64_t ffn, int64_t heads, int64_t n) {
  if (n < 1) return fail(TP_ERR_SHAPE, "shard count %lld < 1", (long long)n);
  if (h < 1 || ffn < 0 || heads < 0) return fail(TP_ERR_SHAPE, "negative or zero size");
  if (ffn % n != 0)
    return fail(TP_ERR_SHAPE, "ffn %lld is not divisible by %lld shards", (long long)ffn, (long long)n);
  if (heads > 0) {
    if (h % heads != 0)
      return fail(TP_ERR_SHAPE, "hidden %lld is not divisible by %lld heads", (long long)h,
                  (long long)heads);
    if (heads % n != 0)
      return fail(TP_ERR_SHAPE, "heads %lld must be a multiple of the shard count %lld",
                  (long long)heads, (long long)n);
  }
  return ok();
}

size_t tp_col_linear_gelu_workspace(int dtype, int act, int64_t M, int64_t K, int64_t Ni) {
  if (act != TP_ACT_SWIGLU && use_gemv(dtype, M) && Ni <= gemv_max_n()) return gemv_workspace(K, Ni);
  return 0;
}

size_t tp_row_linear_partial_workspace(int dtype, int64_t M, int64_t Ki, int64_t N) {
  if (use_gemv(dtype, M) && N <= gemv_max_n()) return gemv_workspace(Ki, N);
  return 0;
}

size_t tp_attn_heads_shard_workspace(int dtype, int64_t b, int64_t s, int64_t heads_local,
                                     int64_t d) {
  if (!dtype_ok(dtype) || b < 0 || s < 0 || heads_local < 0 || d < 0) return 0;
  return attn_ws(dtype, b, s, heads_local, heads_local, d).total;
}

size_t tp_attn_shard_backward_workspace(int dtype, int64_t b, int64_t s, int64_t heads_local,
                                        int64_t kv_heads_local, int64_t d) {
  if (!dtype_ok(dtype) || b < 0 || s < 0 || heads_local < 0 || kv_heads_local < 0 || d < 0) return 0;
  return attn_bwd_ws(dtype, b, s, heads_local, kv_heads_local, d).total;
}

int tp_attn_shard_backward(int dtype, int64_t b, int64_t s, int64_t h, int64_t heads_local,
                           int64_t kv_heads_local, int64_t d, int causal, const void *X, int64_t ldx,
                           const void *Wqkv, int64_t ldwqkv, const void *Wo, int64_t ldwo, const void *dY,
                           int64_t lddy, const void *fwd_ws, size_t fwd_ws_bytes, float *dWqkv, float *dWo,
                           float *dXi, int64_t lddx, void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd_impl(dtype, b, s, h, heads_local, kv_heads_local, d, causal, X, ldx, Wqkv, ldwqkv, Wo, ldwo,
                       dY, lddy, fwd_ws, fwd_ws_bytes, dWqkv, dWo, dXi, lddx, ws, ws_bytes, stream);
}

size_t tp_attn_gqa_shard_workspace(int dtype, int64_t b, int64_t s, int64_t heads_local,
                                   int64_t kv_heads_local, int64_t d) {
  if (!dtype_ok(dtype) || b < 0 || s < 0 || heads_local < 0 || kv_heads_local < 0 || d < 0) return 0;
  return attn_ws(dtype, b, s, heads_local, kv_heads_local, d).total;
}

size_t tp_mlp_shard_backward_workspace(int dtype, int act, int64_t M, int64_t Ni) {
  if (M < 0 || Ni < 0) return 0;
  return bwd_ws(dtype, act, M, Ni).total;
}

}  // extern "C"

namespace {
// tp_col_linear_gelu and its allocation-free variant (noalloc: the decode
// path's split-K scratch is the library's static array, no ws)
int col_linear_impl(const char *fn, int dtype, int act, int64_t M, int64_t K, int64_t Ni, const void *X,
                    int64_t ldx, const void *W, int64_t ldw, const void *Wup, int64_t ldwu, const void *bias,
                    void *H, int64_t ldh, void *ws, size_t ws_bytes, void *stream, bool noalloc) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  if (act != TP_ACT_NONE && act != TP_ACT_GELU_ERF && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_ARG, "activation %d", act);
  TRY(check_dims({M, K, Ni}, fn));
  if (K < 1 || Ni < 1) return fail(TP_ERR_SHAPE, "K and Ni must be >= 1");
  const size_t e = esize(dtype);
  TRY(check_mat(X, M, K, ldx, e, "X"));
  TRY(check_mat(W, K, Ni, ldw, e, "W"));
  TRY(check_mat(H, M, Ni, ldh, e, "H"));
  if (act == TP_ACT_SWIGLU) {
    if (Wup == nullptr) return fail(TP_ERR_ARG, "SwiGLU needs Wup");
    if (bias != nullptr) return fail(TP_ERR_ARG, "SwiGLU takes no bias");
    TRY(check_mat(Wup, K, Ni, ldwu, e, "Wup"));
  } else if (Wup != nullptr) {
    return fail(TP_ERR_ARG, "Wup is only used by SwiGLU");
  }
  TRY(check_vec(bias, Ni, e, "bias"));
  if (M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (act != TP_ACT_SWIGLU && use_gemv(dtype, M) && Ni <= gemv_max_n() && gemv_fits(ldx, ldw)) {
    GemvArgs g;
    g.dtype = DT_BF16;
    g.epi = act == TP_ACT_GELU_ERF ? EPI_GELU : EPI_STORE;
    g.M = M; g.K = K; g.N = Ni;
    g.X = X; g.ldx = ldx; g.W = W; g.ldw = ldw; g.bias = bias;
    g.Y = H; g.ldy = ldh;
    if (noalloc) {
      if (!gemv_noalloc_fits(K, Ni))
        return fail(TP_ERR_SHAPE, "%s: decode partials of K %lld x Ni %lld exceed the %zu-byte static scratch", fn,
                    (long long)K, (long long)Ni, gemv_noalloc_max_bytes());
      TRY(hip_status(launch_gemv_noalloc(g, s), "gemv"));
      return ok();
    }
    const size_t need = gemv_workspace(K, Ni);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(TP_ERR_WORKSPACE, "decode path needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
      return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
    g.ws = ws; g.ws_bytes = ws_bytes;
    TRY(hip_status(launch_gemv(g, s), "gemv"));
    return ok();
  }

  GemmArgs a;
  a.dtype = dtype;
  a.layout = LAY_NN;
  a.M = M; a.N = Ni; a.K = K;
  a.A = X; a.lda = ldx;
  a.B = W; a.ldb = ldw;
  a.C = H; a.ldc = ldh;
  if (act == TP_ACT_SWIGLU) {
    a.dual = true;
    a.epi = EPI_SWIGLU;
    a.B2 = Wup; a.ldb2 = ldwu;
  } else {
    a.epi = act == TP_ACT_GELU_ERF ? EPI_GELU : EPI_STORE;
    a.bias = bias;
  }
  TRY(hip_status(launch_gemm(a, s), "column GEMM"));
  return ok();
}

}  // namespace

extern "C" {

int tp_col_linear_gelu(int dtype, int act, int64_t M, int64_t K, int64_t Ni, const void *X,
                       int64_t ldx, const void *W, int64_t ldw, const void *Wup, int64_t ldwu,
                       const void *bias, void *H, int64_t ldh, void *ws, size_t ws_bytes,
                       void *stream) {
  return col_linear_impl("tp_col_linear_gelu", dtype, act, M, K, Ni, X, ldx, W, ldw, Wup, ldwu, bias, H, ldh,
                         ws, ws_bytes, stream, false);
}

int tp_col_linear_gelu_noalloc(int dtype, int act, int64_t M, int64_t K, int64_t Ni, const void *X,
                               int64_t ldx, const void *W, int64_t ldw, const void *Wup, int64_t ldwu,
                               const void *bias, void *H, int64_t ldh, void *stream) {
  return col_linear_impl("tp_col_linear_gelu_noalloc", dtype, act, M, K, Ni, X, ldx, W, ldw, Wup, ldwu, bias, H,
                         ldh, nullptr, 0, stream, true);
}

int tp_row_linear_partial(int dtype, int64_t M, int64_t Ki, int64_t N, const void *Xi, int64_t ldx,
                          const void *Wi, int64_t ldw, float *P, int64_t ldp, void *ws,
                          size_t ws_bytes, void *stream) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  TRY(check_dims({M, Ki, N}, "tp_row_linear_partial"));
  if (Ki < 1 || N < 1) return fail(TP_ERR_SHAPE, "Ki and N must be >= 1");
  const size_t e = esize(dtype);
  TRY(check_mat(Xi, M, Ki, ldx, e, "Xi"));
  TRY(check_mat(Wi, Ki, N, ldw, e, "Wi"));
  TRY(check_mat(P, M, N, ldp, 4, "P"));
  if (M == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (use_gemv(dtype, M) && N <= gemv_max_n() && gemv_fits(ldx, ldw)) {
    const size_t need = gemv_workspace(Ki, N);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(TP_ERR_WORKSPACE, "decode path needs %zu workspace bytes, got %zu", need, ws_bytes);
    if (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
      return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
    GemvArgs g;
    g.dtype = DT_BF16;
    g.epi = EPI_STORE_F32;
    g.M = M; g.K = Ki; g.N = N;
    g.X = Xi; g.ldx = ldx; g.W = Wi; g.ldw = ldw;
    g.Y = P; g.ldy = ldp; g.ws = ws; g.ws_bytes = ws_bytes;
    TRY(hip_status(launch_gemv(g, s), "gemv"));
    return ok();
  }
  GemmArgs a;
  a.dtype = dtype;
  a.layout = LAY_NN;
  a.epi = EPI_STORE_F32;
  a.M = M; a.N = N; a.K = Ki;
  a.A = Xi; a.lda = ldx;
  a.B = Wi; a.ldb = ldw;
  a.C = P; a.ldc = ldp;
  TRY(hip_status(launch_gemm(a, s), "row GEMM"));
  return ok();
}

size_t tp_decode_packed_weight_bytes(int64_t K, int64_t N) {
  if (K < 1 || N < 1 || K > kMaxDim || N > kMaxDim) return 0;
  return gemv_packed_bytes(K, N);
}

int tp_decode_pack_weight(int dtype, int64_t K, int64_t N, const void *W, int64_t ldw, void *Wp,
                          size_t wp_bytes, void *stream) {
  if (dtype != TP_BF16) return fail(TP_ERR_DTYPE, "tp_decode_pack_weight: bf16 weights only");
  TRY(check_dims({K, N}, "tp_decode_pack_weight"));
  if (K < 1 || N < 1) return fail(TP_ERR_SHAPE, "K and N must be >= 1");
  TRY(check_mat(W, K, N, ldw, 2, "W"));
  if (Wp == nullptr) return fail(TP_ERR_ARG, "Wp is NULL");
  if ((reinterpret_cast<uintptr_t>(Wp) & 15u) != 0) return fail(TP_ERR_ALIGN, "Wp is not 16-byte aligned");
  const size_t need = gemv_packed_bytes(K, N);
  if (wp_bytes < need) return fail(TP_ERR_SHAPE, "Wp holds %zu bytes, the panels need %zu", wp_bytes, need);
  TRY(hip_status(launch_gemv_pack(static_cast<const uint16_t *>(W), ldw, K, N, static_cast<uint16_t *>(Wp),
                                  static_cast<hipStream_t>(stream)),
                 "decode weight pack"));
  return ok();
}

size_t tp_decode_linear_packed_workspace(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || M > 16 || K < 1 || N < 1 || N > gemv_max_n()) return 0;
  return gemv_workspace(K, N);
}

int tp_decode_linear_packed(int act, int out_dtype, int64_t M, int64_t K, int64_t N, const void *X, int64_t ldx,
                            const void *Wp, size_t wp_bytes, const void *bias, void *Y, int64_t ldy, void *ws,
                            size_t ws_bytes, void *stream) {
  if (act != TP_ACT_NONE && act != TP_ACT_GELU_ERF) return fail(TP_ERR_ARG, "activation %d", act);
  if (out_dtype != TP_BF16 && out_dtype != TP_F32) return fail(TP_ERR_DTYPE, "output dtype %d", out_dtype);
  if (out_dtype == TP_F32 && act != TP_ACT_NONE)
    return fail(TP_ERR_ARG, "an fp32 output (a row-parallel partial) takes no activation");
  TRY(check_dims({M, K, N}, "tp_decode_linear_packed"));
  if (K < 1 || N < 1) return fail(TP_ERR_SHAPE, "K and N must be >= 1");
  if (M > 16) return fail(TP_ERR_SHAPE, "the decode path takes at most 16 token rows, got %lld", (long long)M);
  if (N > gemv_max_n()) return fail(TP_ERR_SHAPE, "N %lld exceeds the decode path's %lld", (long long)N,
                                    (long long)gemv_max_n());
  TRY(check_mat(X, M, K, ldx, 2, "X"));
  TRY(check_mat(Y, M, N, ldy, out_dtype == TP_F32 ? 4 : 2, "Y"));
  TRY(check_vec(bias, N, 2, "bias"));
  if (Wp == nullptr) return fail(TP_ERR_ARG, "Wp is NULL");
  if ((reinterpret_cast<uintptr_t>(Wp) & 15u) != 0) return fail(TP_ERR_ALIGN, "Wp is not 16-byte aligned");
  if (wp_bytes < gemv_packed_bytes(K, N))
    return fail(TP_ERR_SHAPE, "Wp holds %zu bytes, the panels of K %lld x N %lld take %zu", wp_bytes,
                (long long)K, (long long)N, gemv_packed_bytes(K, N));
  if (!gemv_fits(ldx, 64)) return fail(TP_ERR_SHAPE, "ldx %lld too large for the decode path", (long long)ldx);
  if (M == 0) return ok();
  const size_t need = gemv_workspace(K, N);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(TP_ERR_WORKSPACE, "decode path needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
  GemvArgs g;
  g.dtype = DT_BF16;
  g.epi = out_dtype == TP_F32 ? EPI_STORE_F32 : (act == TP_ACT_GELU_ERF ? EPI_GELU : EPI_STORE);
  g.M = M; g.K = K; g.N = N;
  g.X = X; g.ldx = ldx; g.W = Wp; g.ldw = 0; g.packed = true;
  g.bias = bias; g.Y = Y; g.ldy = ldy; g.ws = ws; g.ws_bytes = ws_bytes;
  TRY(hip_status(launch_gemv(g, static_cast<hipStream_t>(stream)), "packed gemv"));
  return ok();
}

int tp_attn_heads_shard(int dtype, int64_t b, int64_t s_len, int64_t h, int64_t heads_local,
                        int64_t d, int causal, const void *X, int64_t ldx, const void *Wqkv,
                        int64_t ldwqkv, const void *Wo, int64_t ldwo, float *P, int64_t ldp,
                        void *ws, size_t ws_bytes, void *stream) {
  return attn_impl("tp_attn_heads_shard", dtype, b, s_len, h, heads_local, heads_local, d, causal, X,
                   ldx, Wqkv, ldwqkv, Wo, ldwo, P, ldp, ws, ws_bytes, stream);
}

int tp_attn_gqa_shard(int dtype, int64_t b, int64_t s_len, int64_t h, int64_t heads_local,
                      int64_t kv_heads_local, int64_t d, int causal, const void *X, int64_t ldx,
                      const void *Wqkv, int64_t ldwqkv, const void *Wo, int64_t ldwo, float *P,
                      int64_t ldp, void *ws, size_t ws_bytes, void *stream) {
  return attn_impl("tp_attn_gqa_shard", dtype, b, s_len, h, heads_local, kv_heads_local, d, causal, X,
                   ldx, Wqkv, ldwqkv, Wo, ldwo, P, ldp, ws, ws_bytes, stream);
}

int tp_shard_sum(int out_dtype, int64_t M, int64_t N, int n, const float *const *partials,
                 int64_t ldp, const float *bias, void *Y, int64_t ldy, void *stream) {
  if (!dtype_ok(out_dtype)) return fail(TP_ERR_DTYPE, "dtype %d", out_dtype);
  if (n < 1 || n > 64) return fail(TP_ERR_ARG, "shard count %d outside 1..64", n);
  if (partials == nullptr) return fail(TP_ERR_ARG, "partials array is NULL");
  TRY(check_dims({M, N}, "tp_shard_sum"));
  if (N < 1) return fail(TP_ERR_SHAPE, "N must be >= 1");
  for (int i = 0; i < n; ++i) {
    char name[32];
    snprintf(name, sizeof(name), "partials[%d]", i);
    TRY(check_mat(partials[i], M, N, ldp, 4, name));
  }
  TRY(check_vec(bias, N, 4, "bias"));
  TRY(check_mat(Y, M, N, ldy, esize(out_dtype), "Y"));
  if (M == 0) return ok();
  TRY(hip_status(launch_shard_sum(out_dtype, M, N, n, partials, ldp, bias, Y, ldy,
                                  static_cast<hipStream_t>(stream)),
                 "shard sum"));
  return ok();
}

int tp_shard_reduce_scatter_layernorm(int out_dtype, int64_t rows, int64_t N, int n,
                                      const float *const *partials, int64_t ldp, const float *bias,
                                      const float *residual, int64_t ldr, const float *gamma,
                                      const float *beta, float eps, float *Ysum, int64_t ldys, void *Y,
                                      int64_t ldy, void *stream) {
  if (!dtype_ok(out_dtype)) return fail(TP_ERR_DTYPE, "dtype %d", out_dtype);
  if (n < 1 || n > 64) return fail(TP_ERR_ARG, "shard count %d outside 1..64", n);
  if (partials == nullptr) return fail(TP_ERR_ARG, "partials array is NULL");
  if (gamma == nullptr || beta == nullptr) return fail(TP_ERR_ARG, "gamma and beta are required");
  if (!(eps >= 0.0f)) return fail(TP_ERR_ARG, "eps must be >= 0");
  TRY(check_dims({rows, N}, "tp_shard_reduce_scatter_layernorm"));
  if (N < 4 || N > rs_layernorm_max_n())
    return fail(TP_ERR_SHAPE, "hidden size %lld outside 4..%lld", (long long)N, (long long)rs_layernorm_max_n());
  for (int i = 0; i < n; ++i) {
    char name[32];
    snprintf(name, sizeof(name), "partials[%d]", i);
    TRY(check_mat(partials[i], rows, N, ldp, 4, name));
  }
  TRY(check_vec(bias, N, 4, "bias"));
  TRY(check_vec(gamma, N, 4, "gamma"));
  TRY(check_vec(beta, N, 4, "beta"));
  if (residual != nullptr) TRY(check_mat(residual, rows, N, ldr, 4, "residual"));
  if (Ysum != nullptr) TRY(check_mat(Ysum, rows, N, ldys, 4, "Ysum"));
  TRY(check_mat(Y, rows, N, ldy, esize(out_dtype), "Y"));
  if (rows == 0) return ok();
  TRY(hip_status(launch_rs_layernorm(out_dtype, rows, N, n, partials, ldp, bias, residual, ldr, gamma, beta,
                                     eps, Ysum, ldys, Y, ldy, static_cast<hipStream_t>(stream)),
                 "reduce-scatter layernorm"));
  return ok();
}

int tp_vocab_ce_shard_stats(int dtype, int64_t T, int64_t Vi, const void *logits, int64_t ldz,
                            float *stats, void *stream) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  TRY(check_dims({T, Vi}, "tp_vocab_ce_shard_stats"));
  if (Vi < 1) return fail(TP_ERR_SHAPE, "Vi must be >= 1");
  TRY(check_rows(logits, T, Vi, ldz, esize(dtype), "logits"));
  TRY(check_arr(stats, T > 0, 8, "stats"));
  if (T == 0) return ok();
  TRY(hip_status(launch_vocab_stats(dtype, T, Vi, logits, ldz, stats, static_cast<hipStream_t>(stream)),
                 "vocab stats"));
  return ok();
}

int tp_vocab_ce_lse(int64_t T, int n, const float *const *stats, float *lse, void *stream) {
  if (n < 1 || n > 64) return fail(TP_ERR_ARG, "shard count %d outside 1..64", n);
  if (stats == nullptr) return fail(TP_ERR_ARG, "stats array is NULL");
  TRY(check_dims({T}, "tp_vocab_ce_lse"));
  for (int i = 0; i < n; ++i) {
    char name[32];
    snprintf(name, sizeof(name), "stats[%d]", i);
    TRY(check_arr(stats[i], T > 0, 8, name));
  }
  TRY(check_arr(lse, T > 0, 4, "lse"));
  if (T == 0) return ok();
  TRY(hip_status(launch_vocab_lse(T, n, stats, lse, static_cast<hipStream_t>(stream)), "vocab lse"));
  return ok();
}

int tp_vocab_ce_shard_loss(int dtype, int64_t T, int64_t Vi, int64_t vocab_start, const void *logits,
                           int64_t ldz, const int32_t *targets, const float *lse, float *row_loss,
                           float *shard_loss, void *stream) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  TRY(check_dims({T, Vi, vocab_start}, "tp_vocab_ce_shard_loss"));
  if (Vi < 1) return fail(TP_ERR_SHAPE, "Vi must be >= 1");
  TRY(check_rows(logits, T, Vi, ldz, esize(dtype), "logits"));
  TRY(check_arr(targets, T > 0, 4, "targets"));
  TRY(check_arr(lse, T > 0, 4, "lse"));
  TRY(check_arr(row_loss, false, 4, "row_loss"));
  TRY(check_arr(shard_loss, true, 4, "shard_loss"));
  TRY(hip_status(launch_vocab_loss(dtype, T, Vi, vocab_start, logits, ldz, targets, lse, row_loss, shard_loss,
                                   static_cast<hipStream_t>(stream)),
                 "vocab loss"));
  return ok();
}

int tp_vocab_ce_total(int n, const float *const *shard_losses, float *total, void *stream) {
  if (n < 1 || n > 64) return fail(TP_ERR_ARG, "shard count %d outside 1..64", n);
  if (shard_losses == nullptr) return fail(TP_ERR_ARG, "shard_losses array is NULL");
  for (int i = 0; i < n; ++i) {
    char name[40];
    snprintf(name, sizeof(name), "shard_losses[%d]", i);
    TRY(check_arr(shard_losses[i], true, 4, name));
  }
  TRY(check_arr(total, true, 4, "total"));
  TRY(hip_status(launch_vocab_total(n, shard_losses, total, static_cast<hipStream_t>(stream)), "vocab total"));
  return ok();
}

int tp_mlp_shard_backward(int dtype, int act, int64_t M, int64_t K, int64_t Ni, const void *X,
                          int64_t ldx, const void *W1, int64_t ldw1, const void *Wup, int64_t ldwu,
                          const void *b1, const void *W2, int64_t ldw2, const void *dY,
                          int64_t lddy, float *dW1, float *dWup, float *dW2, float *db1,
                          float *dXi, int64_t lddx, void *ws, size_t ws_bytes, void *stream) {
  if (!dtype_ok(dtype)) return fail(TP_ERR_DTYPE, "dtype %d", dtype);
  if (act != TP_ACT_GELU_ERF && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_ARG, "backward supports GELU and SwiGLU, got activation %d", act);
  TRY(check_dims({M, K, Ni}, "tp_mlp_shard_backward"));
  if (K < 1 || Ni < 1) return fail(TP_ERR_SHAPE, "K and Ni must be >= 1");
  const size_t e = esize(dtype);
  const bool swiglu = act == TP_ACT_SWIGLU;
  TRY(check_mat(X, M, K, ldx, e, "X"));
  TRY(check_mat(W1, K, Ni, ldw1, e, "W1"));
  TRY(check_mat(W2, Ni, K, ldw2, e, "W2"));
  TRY(check_mat(dY, M, K, lddy, e, "dY"));
  TRY(check_mat(dW1, K, Ni, Ni, 4, "dW1"));
  TRY(check_mat(dW2, Ni, K, K, 4, "dW2"));
  TRY(check_mat(dXi, M, K, lddx, 4, "dXi"));
  if (swiglu) {
    if (Wup == nullptr || dWup == nullptr) return fail(TP_ERR_ARG, "SwiGLU needs Wup and dWup");
    if (b1 != nullptr || db1 != nullptr) return fail(TP_ERR_ARG, "SwiGLU takes no bias");
    TRY(check_mat(Wup, K, Ni, ldwu, e, "Wup"));
    TRY(check_mat(dWup, K, Ni, Ni, 4, "dWup"));
  } else {
    if (Wup != nullptr || dWup != nullptr) return fail(TP_ERR_ARG, "Wup/dWup are SwiGLU only");
    TRY(check_vec(b1, Ni, e, "b1"));
    TRY(check_vec(db1, Ni, 4, "db1"));
  }
  const BwdWs L = bwd_ws(dtype, act, M, Ni);
  if (M > 0) {
    if (ws == nullptr || ws_bytes < L.total)
      return fail(TP_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", L.total, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
      return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  void *dH = base + L.dH;
  void *H = base + L.H;
  void *dZ = base + L.dZ;
  const int64_t ldz = swiglu ? 2 * Ni : Ni;
  void *dZu = swiglu ? static_cast<void *>(base + L.dZ + (size_t)Ni * e) : nullptr;
  // dH is dead once the recompute has formed dZ: its region then holds the
  // split-K partials of the weight-gradient GEMMs
  float *dHpart = M > 0 ? reinterpret_cast<float *>(base + L.dH) : nullptr;
  const size_t dHpart_bytes = M > 0 ? L.H - L.dH : 0;
  int db1_tiles = 0;  // row-tiles of db1 partials the recompute's epilogue wrote

  if (M > 0) {
    // dH = dY W2^T  (row-parallel layer, input gradient of this shard's slice)
    GemmArgs a;
    a.dtype = dtype; a.layout = LAY_NT; a.epi = EPI_STORE;
    a.M = M; a.N = Ni; a.K = K;
    a.A = dY; a.lda = lddy;
    a.B = W2; a.ldb = ldw2;
    a.C = dH; a.ldc = Ni;
    TRY(hip_status(launch_gemm(a, s), "dH GEMM"));

    // recompute Z = X W1 (+b1) and apply the activation derivative
    GemmArgs r;
    r.dtype = dtype; r.layout = LAY_NN;
    r.M = M; r.N = Ni; r.K = K;
    r.A = X; r.lda = ldx;
    r.B = W1; r.ldb = ldw1;
    r.D = dH; r.ldd = Ni;
    r.C = dZ; r.ldc = ldz;
    r.C2 = H; r.ldc2 = Ni;
    if (swiglu) {
      r.dual = true; r.epi = EPI_SWIGLU_BWD;
      r.B2 = Wup; r.ldb2 = ldwu;
      r.C3 = dZu; r.ldc3 = ldz;
    } else {
      r.epi = EPI_GELU_BWD;
      r.bias = b1;
      // db1's per-row-tile partials straight from the epilogue, if the
      // kernel that takes the product can (else the column-sum kernels)
      if (db1 != nullptr) {
        r.colsum = reinterpret_cast<float *>(base + L.cs);
        r.colsum_tiles = &db1_tiles;
      }
    }
    TRY(hip_status(launch_gemm(r, s), "recompute GEMM"));
  }

  // dW2 = H^T dY (row-parallel weight gradient)
  GemmArgs w2;
  w2.dtype = dtype; w2.layout = LAY_TN; w2.epi = EPI_STORE_F32;
  w2.M = Ni; w2.N = K; w2.K = M;
  w2.A = H; w2.lda = Ni;
  w2.B = dY; w2.ldb = lddy;
  w2.C = dW2; w2.ldc = K;
  w2.part = dHpart; w2.part_bytes = dHpart_bytes;
  // dW1 = X^T dZ (column-parallel weight gradient; dWup = X^T dZu)
  GemmArgs w1;
  w1.dtype = dtype; w1.layout = LAY_TN; w1.epi = EPI_STORE_F32;
  w1.M = K; w1.N = Ni; w1.K = M;
  w1.A = X; w1.lda = ldx;
  w1.B = dZ; w1.ldb = ldz;
  w1.C = dW1; w1.ldc = Ni;
  w1.part = dHpart; w1.part_bytes = dHpart_bytes;
  if (swiglu) {
    // dWg and dWu have the same shape: one launch when they split
    GemmArgs wu = w1;
    wu.B = dZu;
    wu.C = dWup;
    TRY(hip_status(launch_gemm(w2, s), "dW2 GEMM"));
    TRY(hip_status(launch_gemm_tn_pair(w1, wu, s), "dW1 / dWup GEMMs"));
  }
  float *cs = M > 0 ? reinterpret_cast<float *>(base + L.cs) : nullptr;  // M == 0: db1 = 0
  bool db1_done = false;
  if (!swiglu) {
    // one launch for both when they have the same shape (K == Ni) and split;
    // its partial-sum launch also adds db1's row-tile partials when the
    // recompute wrote them
    ColsumJob cj;
    cj.rows = db1_tiles; cj.N = Ni; cj.part = cs; cj.db = db1;
    const bool with_db1 = db1 != nullptr && db1_tiles > 0;
    TRY(hip_status(launch_gemm_tn_pair(w2, w1, s, with_db1 ? &cj : nullptr, &db1_done), "dW2 / dW1 GEMMs"));
  }
  if (db1 != nullptr && !db1_done) {
    if (db1_tiles > 0)
      TRY(hip_status(launch_colsum_final(db1_tiles, Ni, cs, db1, s), "db1"));
    else
      TRY(hip_status(launch_colsum(dtype, M, Ni, dZ, ldz, db1, cs, s), "db1"));
  }

  if (M > 0) {
    // dX_i = dZ W1^T  (SwiGLU: [dZg | dZu] [Wg | Wu]^T in one K-concatenated pass)
    GemmArgs x;
    x.dtype = dtype; x.layout = LAY_NT; x.epi = EPI_STORE_F32;
    x.M = M; x.N = K; x.K = swiglu ? 2 * Ni : Ni;
    x.A = dZ; x.lda = ldz;
    x.B = W1; x.ldb = ldw1;
    if (swiglu) {
      x.kcat = true; x.K1 = Ni;
      x.B2 = Wup; x.ldb2 = ldwu;
    }
    x.C = dXi; x.ldc = lddx;
    TRY(hip_status(launch_gemm(x, s), "dX GEMM"));
  }
  return ok();
}

}  // extern "C"
