// Host-side interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpcol {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

// Epilogue applied to the float32 accumulator(s) of a GEMM tile.
enum Epi {
  EPI_STORE = 0,      // C (dtype)   = acc + bias
  EPI_STORE_F32 = 1,  // C (float32) = acc + bias
  EPI_GELU = 2,       // C (dtype)   = GELU(acc + bias)
  EPI_SWIGLU = 3,     // C (dtype)   = SiLU(acc) * acc2                  (dual)
  EPI_GELU_BWD = 4,   // z = acc + bias, dh = D:  C = dh * GELU'(z), C2 = GELU(z)
  EPI_SWIGLU_BWD = 5  // g = acc, u = acc2, dh = D: C = dh*u*SiLU'(g),
                      //   C3 = dh*SiLU(g), C2 = SiLU(g)*u               (dual)
};

// Operand storage.  A is [M x K] row-major (N) or stored as its transpose
// [K x M] row-major (T); B is [K x N] row-major (N) or stored as [N x K] (T).
enum Layout { LAY_NN = 0, LAY_NT = 1, LAY_TN = 2 };

struct GemmArgs {
  int dtype = DT_BF16;
  Layout layout = LAY_NN;
  Epi epi = EPI_STORE;
  bool dual = false;  // second B (B2) with its own accumulator (NN only)
  bool kcat = false;  // B rows k >= K1 are read from B2 (NT only)
  int64_t M = 0, N = 0, K = 0, K1 = 0;
  const void *A = nullptr;  int64_t lda = 0;
  const void *B = nullptr;  int64_t ldb = 0;
  const void *B2 = nullptr; int64_t ldb2 = 0;
  const void *bias = nullptr;                  // [N], dtype (f32 for EPI_STORE_F32)
  const void *D = nullptr;  int64_t ldd = 0;   // epilogue input (dH), dtype
  void *C = nullptr;  int64_t ldc = 0;
  void *C2 = nullptr; int64_t ldc2 = 0;
  void *C3 = nullptr; int64_t ldc3 = 0;
  // Optional fp32 scratch for split-K of TN fp32 products whose output has
  // too few tiles to fill the chip (weight gradients of narrow shards):
  // launch_gemm then writes `splits` K-range partials [splits][M][N] there
  // and adds them into C in split order.
  float *part = nullptr; size_t part_bytes = 0;
  // set by launch_gemm for the LDS kernel: K-range splits (grid y) and the
  // element stride between their outputs
  int splits = 1; int64_t zstride = 0;
  // grouped TN split-K (launch_gemm_tn_pair): a second product of the same
  // shape, A2 . B2 (B2 / ldb2 above), whose partials follow the first's
  const void *A2 = nullptr; int64_t lda2 = 0;
  int groups = 1;
  // EPI_GELU_BWD: where the kernel may also write the column sums of C per
  // row-tile ([row-tiles][N] fp32, rows added in order; colsum_rows() of
  // them at most); if it does, it stores the row-tile count in
  // *colsum_tiles (a host int), otherwise leaves it untouched
  float *colsum = nullptr;
  int *colsum_tiles = nullptr;
};

hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
// db[c] = sum over rows r < rows of part[r][c] (launch_colsum_final's work),
// for a launch that can take it on beside its own
struct ColsumJob {
  int rows = 0;
  int64_t N = 0;
  const float *part = nullptr;
  float *db = nullptr;
};
// Two bf16 TN fp32 products of the same shape (a0.C = A0^T B0, a1.C =
// A1^T B1): one K-split launch for both when a0.part holds their partials,
// else two launch_gemm calls.  cj (optional): a column sum whose inputs are
// complete before this call; when the split path's partial-sum launch has
// run it too, *cj_done is set (else the caller launches it).
hipError_t launch_gemm_tn_pair(const GemmArgs &a0, const GemmArgs &a1, hipStream_t s,
                               const ColsumJob *cj = nullptr, bool *cj_done = nullptr);

// Decode GEMV (M <= 16): y = act(x W + bias) with split-K partials in ws.
struct GemvArgs {
  int dtype = DT_BF16;  // bf16 only
  Epi epi = EPI_GELU;   // EPI_GELU / EPI_STORE (dtype out) or EPI_STORE_F32
  int64_t M = 0, K = 0, N = 0;
  const void *X = nullptr; int64_t ldx = 0;
  const void *W = nullptr; int64_t ldw = 0;
  const void *bias = nullptr;
  void *Y = nullptr; int64_t ldy = 0;
  void *ws = nullptr; size_t ws_bytes = 0;
  bool packed = false;  // W in the panel layout of launch_gemv_pack (ldw unused)
};
size_t gemv_workspace(int64_t K, int64_t N);  // the same for both weight layouts
// Panel layout for decode weights: Wp[(s * Kp + k) * 64 + c] = W[k][64 s + c]
// (zeros past K and N), Kp = gemv_panel_rows(K).
int64_t gemv_panel_rows(int64_t K);
size_t gemv_packed_bytes(int64_t K, int64_t N);
hipError_t launch_gemv_pack(const uint16_t *W, int64_t ldw, int64_t K, int64_t N, uint16_t *Wp, hipStream_t s);
int64_t gemv_max_n();  // widest N the split-K decode path accepts
bool gemv_fits(int64_t ldx, int64_t ldw);  // row strides the decode path's 32-bit offsets cover
hipError_t launch_gemv(const GemvArgs &a, hipStream_t s);
// The same with the split-K partials in the library's static scratch (no
// workspace; the same two kernels).  gemv_noalloc_fits: the shape's partials
// fit that scratch (gemv_noalloc_max_bytes(); true for every decode shape).
hipError_t launch_gemv_noalloc(const GemvArgs &a, hipStream_t s);
bool gemv_noalloc_fits(int64_t K, int64_t N);
size_t gemv_noalloc_max_bytes();

// Y = sum_i P_i (+ bias), float32 partials, float32 or bf16 output.
hipError_t launch_shard_sum(int out_dtype, int64_t M, int64_t N, int n, const float *const *parts,
                            int64_t ldp, const float *bias, void *Y, int64_t ldy, hipStream_t s);
// Two such sums in one launch (fp32 outputs, no bias): Y0 = sum_i P_i,
// Y1 = sum_i P_{n+i} for i < n; with cj, the same launch also does that
// column sum (in launch_colsum_final's order: bitwise the same db).
hipError_t launch_shard_sum_pair(int64_t M, int64_t N, int n, const float *const *parts, int64_t ldp,
                                 float *Y0, int64_t ldy0, float *Y1, int64_t ldy1, hipStream_t s,
                                 const ColsumJob *cj = nullptr);

// Head-local flash attention over a packed [Q|K|V] buffer (bf16, d = 128).
// lse (optional, [b][heads_local][s] fp32): log2 of each query row's softmax
// denominator in the scaled-score base-2 domain, for the backward
hipError_t launch_flash_attn(const void *qkv, int64_t ldqkv, void *O, int64_t ldo, float *lse, int64_t b,
                             int64_t s, int64_t heads_local, int64_t kv_heads_local, int64_t d,
                             bool causal, hipStream_t st);
// Attention backward from the forward's packed QKV, O and lse: D (fp32
// [b][heads_local][s], written) then dQ | dK | dV into dqkv (bf16, same
// packing and stride as qkv)
// (part: attn_bwd_part_bytes() of fp32 scratch for the split dK/dV partials,
// NULL allowed when that is 0)
hipError_t launch_attn_bwd(const void *qkv, int64_t ldqkv, const void *O, int64_t ldo, const float *lse,
                           const void *dO, int64_t lddo, float *Dr, void *dqkv, float *part, int64_t b, int64_t s,
                           int64_t heads_local, int64_t kv_heads_local, int64_t d, bool causal, hipStream_t st);
size_t attn_bwd_part_bytes(int64_t b, int64_t s, int64_t heads_local, int64_t kv_heads_local);
// The same two steps for any other shape: fp32 (DT_F32) or bf16 operands,
// head dim 1..256 (attn_general_fits), same packing, lse and D conventions;
// SIMT kernels, no scratch.
bool attn_general_fits(int64_t s, int64_t d);
hipError_t launch_attn_general(int dtype, const void *qkv, int64_t ldqkv, void *O, int64_t ldo, float *lse,
                               int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d, bool causal,
                               hipStream_t st);
hipError_t launch_attn_bwd_general(int dtype, const void *qkv, int64_t ldqkv, const void *O, int64_t ldo,
                                   const float *lse, const void *dO, int64_t lddo, float *Dr, void *dqkv,
                                   int64_t b, int64_t s, int64_t hl, int64_t kvl, int64_t d, bool causal,
                                   hipStream_t st);

// db[n] = sum_m dZ[m][n] (dZ dtype, db float32).
hipError_t launch_rs_layernorm(int out_dtype, int64_t rows, int64_t N, int n, const float *const *parts,
                               int64_t ldp, const float *bias, const float *res, int64_t ldr,
                               const float *gamma, const float *beta, float eps, float *Ysum,
                               int64_t ldys, void *Y, int64_t ldy, hipStream_t s);
int64_t rs_layernorm_max_n();
hipError_t launch_vocab_stats(int dtype, int64_t T, int64_t Vi, const void *Z, int64_t ldz, float *stats,
                              hipStream_t s);
hipError_t launch_vocab_lse(int64_t T, int n, const float *const *stats, float *lse, hipStream_t s);
hipError_t launch_vocab_loss(int dtype, int64_t T, int64_t Vi, int64_t v0, const void *Z, int64_t ldz,
                             const int32_t *targets, const float *lse, float *row_loss, float *shard_loss,
                             hipStream_t s);
hipError_t launch_vocab_total(int n, const float *const *losses, float *total, hipStream_t s);
// fp32 partial bytes launch_colsum needs for M x N, and which a GEMM's
// column-sum output of M rows fits
size_t colsum_workspace(int64_t M, int64_t N);
int64_t colsum_rows(int64_t M);  // rows of partials that workspace holds
hipError_t launch_colsum(int dtype, int64_t M, int64_t N, const void *dZ, int64_t ldz, float *db,
                         float *part, hipStream_t s);
// db[n] = sum over rows r < rows of part[r][n], in row order
hipError_t launch_colsum_final(int rows, int64_t N, const float *part, float *db, hipStream_t s);

}  // namespace tpcol
