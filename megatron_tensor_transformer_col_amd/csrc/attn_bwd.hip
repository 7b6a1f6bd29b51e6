// Backward of the head-local attention of one tensor-parallel shard (bf16,
// head dim 128), multi-head or grouped-query.
//
// A shard owns whole heads, so it differentiates them alone ("张量并行",
// Multi-Head Attention 的并行化: heads are independent).  For one
// (sequence, head), with the scaled scores S = Q K^T / sqrt(d), the
// probabilities P = softmax(S [+ causal mask]) and O = P V, the chain rule
// through the two products and the row softmax gives
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O),
//     dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d),
// and a key/value head read by g query heads receives the sum of their
// dK / dV.  P is recomputed from the forward's per-row statistic
// lse2 = log2 sum_j exp2(S_ij log2 e), so P_ij = exp2(S_ij log2 e - lse2_i).
//
// Three kernels, none of which waits on another workgroup, all bitwise
// repeatable:
//  * attn_bwd_dot_kernel: D for every (token, head).
//  * attn_bwd_dkdv_kernel: a workgroup of 8 waves owns 128 keys of one
//    (sequence, kv head), 16 per wave (two waves per SIMD; 32 keys per wave
//    need ~360 VGPRs and measured 7% slower at one wave per SIMD), and keeps
//    K, V (as MFMA B operands) and the fp32 dK^T, dV^T accumulators in
//    registers while 64-query tiles of Q and dO, with the tile's lse2 and D
//    rows, stream through LDS by direct DMA (two stages), issued by the
//    second wave of each SIMD only, so the first starts on the matrix cores
//    right after the barrier (all waves issuing: 2-3% slower).  Per tile:
//    S = Q K^T and dP = dO V^T (Q / dO fragments by ds_read_b128), then
//    P and dS in registers, then dV^T += dO^T P and dK^T += Q^T dS with the
//    dO^T / Q^T operands from ds_read_b64_tr_b16 transpose reads.  The
//    output tile of S (4 queries of one key per lane) is already the B
//    operand layout of the second pair of products.
//  * attn_bwd_dq_kernel: a workgroup owns 128 queries of one (sequence,
//    head), 32 per wave, with Q and dO in registers; 64-key tiles of K and V
//    stream through LDS.  Per tile: S^T = K Q^T and dP^T = V dO^T, then
//    dS^T, then dQ^T += K^T dS^T (K^T by transpose reads).  It fits in 256
//    VGPRs, so two workgroups share a CU (two waves per SIMD; 25% faster
//    than one).
//  S and dP are recomputed in both kernels rather than exchanging dS through
//  HBM or accumulating dQ with atomics: the sums stay in a fixed order.
//
// LDS tiles are [row][128] bf16 rows of 256 bytes (16 granules of 16 B);
// granule c of row r is stored at c ^ f(r & 15), f a bit-linear permutation
// of 0..15: f(r) = 2 (r & 7) ^ ((r >> 2) & 1) ^ (r & 8).  Both reads of a
// tile are then conflict free -- the 16-byte row reads (16 consecutive rows
// at one logical granule; every 8 lanes on distinct banks too) and the
// transpose reads (rows 4g + e, pairs of granules) -- which a brute-force
// check over the lane patterns confirms for both plausible bank models.  (A
// simpler f = 2 (r & 7) + (r >> 3) measured two conflict cycles per LDS
// instruction: its 8-lane groups of row reads collide.)
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace tpcol {

static constexpr int BW_D = 128;
static constexpr int BW_TROWS = 64;               // rows of one streamed tile
static constexpr int BW_TILE = BW_TROWS * BW_D;   // elements of one tile (16 KiB)
static constexpr int BW_NW = 4;                   // dQ: waves per workgroup ...
static constexpr int BW_WROWS = 32;               // ... of 32 queries each
static constexpr int BW_BLK = BW_NW * BW_WROWS;   // keys (dK/dV) / queries (dQ) per workgroup
static constexpr int DK_NW = 8;                   // dK/dV: waves per workgroup ...
static constexpr int DK_KT = 1;                   // ... of 16 * DK_KT keys each
static constexpr int64_t BW_MAX_LD = int64_t(1) << 24;

__device__ __forceinline__ int bw_swz(int r) { return ((r & 7) << 1) ^ ((r >> 2) & 1) ^ (r & 8); }

struct BwArgs {
  const uint16_t *qkv;  // forward's packed [Q (hl heads) | K (kvl) | V (kvl)], token-major
  int64_t ldq;
  const uint16_t *dO;   // [T x hl*d]
  int64_t lddo;
  const float *lse;     // [b][hl][s] lse2 of each query row
  const float *Dr;      // [b][hl][s] rowsum(dO * O)
  uint16_t *dqkv;       // gradients, same packing and stride as qkv
  int64_t lddq;
  int s, hl, kvl, group, nbh, nblk;
  int64_t T;            // b * s
  int hsplit;           // dK/dV: workgroups sharing one kv head's query heads
  float *part;          // hsplit > 1: fp32 dK/dV partials [hsplit][b*s][kvl][2][d]
  float scale_log2;     // log2(e) / sqrt(d)
  float scale;          // 1 / sqrt(d)
};

// Per-lane DMA slot of an NW-wave tile copy: lane i of wave w fetches row
// 4w + i/16 (+4 NW per further wave-DMA, a multiple of 16, so the row's
// swizzle stays the lane's) and the global granule that lands in LDS slot
// i % 16 of that row.
template <int NW>
struct BwDma {
  static constexpr int JN = BW_TROWS / (4 * NW);  // wave-DMAs per wave per tile
  static_assert((4 * NW) % 16 == 0 && JN >= 1, "a lane's rows must share their swizzle (16 apart)");
  int row_lo;
  uint32_t gran;  // byte offset of the fetched granule within its row
  __device__ __forceinline__ void init(int wave, int lane) {
    row_lo = 4 * wave + (lane >> 4);
    gran = (uint32_t)(((lane & 15) ^ bw_swz(row_lo & 15)) * 16);
  }
  // rows r0 .. r0+63 of the [rows x ld] bf16 matrix at G (column offset
  // included in G) into the LDS tile at byte address dst; rows at or past
  // `limit` read row limit-1 (their results are masked or discarded)
  __device__ __forceinline__ void tile(const uint16_t *G, int64_t ld, int r0, int limit, uint32_t dst,
                                       int wave) const {
    const uint32_t ldb = (uint32_t)ld * 2u;
    if (r0 + BW_TROWS <= limit) {
#pragma unroll
      for (int j = 0; j < JN; ++j)
        dma16s((uint32_t)row_lo * ldb + gran, G + (int64_t)(r0 + 4 * NW * j) * ld, dst + (wave + NW * j) * 1024);
    } else {
      const uint16_t *base = G + (int64_t)r0 * ld;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const uint32_t r = (uint32_t)min(4 * NW * j + row_lo, limit - 1 - r0);
        dma16s(r * ldb + gran, base, dst + (wave + NW * j) * 1024);
      }
    }
  }
};

// 16-byte fragment: row `row` (0..63) of an LDS tile, logical granule c
__device__ __forceinline__ uint4 lds_frag(const uint16_t *T, int row, int c) {
  return *reinterpret_cast<const uint4 *>(T + row * BW_D + ((c ^ bw_swz(row & 15)) << 3));
}

// Transposed operand from a [row][d] LDS tile: lane (g, l16) gets column
// d = dt*16 + l16 of rows {32kc + 4g + e, 32kc + 16 + 4g + e}, e = 0..3 --
// the k-slot order of a packed C-layout tile pair.
__device__ __forceinline__ uint4 lds_trans(const uint16_t *T, int kc, int dt, int g, int l16) {
  const int e = l16 >> 2, c = l16 & 3;
  const int row = 32 * kc + 4 * g + e;
  const int col = dt * 16 + 4 * c;
  const int off = (((col >> 3) ^ bw_swz(row & 15)) << 3) + (col & 4);
  const uint2 v0 = tr_read(T + row * BW_D + off);
  const uint2 v1 = tr_read(T + (row + 16) * BW_D + off);
  return make_uint4(v0.x, v0.y, v1.x, v1.y);
}

__device__ __forceinline__ uint4 pack8(const f32x4_t &lo, const f32x4_t &hi) {
  return make_uint4(pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                    pack_bf2(hi[2], hi[3]));
}

// workgroup -> (rank of its block in longest-first order, (sequence, head));
// consecutive workgroup indices of one (sequence, head) are nbh apart, so
// with nbh a multiple of 8 they all run on one XCD and share its L2
__device__ __forceinline__ void bw_place(const BwArgs &a, int &rank, int &bh) {
  rank = (int)blockIdx.x / a.nbh;
  bh = (int)blockIdx.x % a.nbh;
}

// ---------------------------------------------------------------- D
// D[(bi*hl + head)*s + q] = sum_c dO[t][head*d + c] * O[t][head*d + c]; 16
// lanes per row, 8 elements each
__global__ void __launch_bounds__(256) attn_bwd_dot_kernel(const uint16_t *__restrict__ dO, int64_t lddo,
                                                           const uint16_t *__restrict__ O, int64_t ldo, int64_t T,
                                                           int s, int hl, float *Dr) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // (token, head)
  const int part = threadIdx.x & 15;
  const bool live = row < T * hl;
  const int64_t t = live ? row / hl : 0;
  const int head = live ? (int)(row % hl) : 0;
  float acc = 0.f;
  if (live) {
    const uint4 a = *reinterpret_cast<const uint4 *>(dO + t * lddo + head * BW_D + part * 8);
    const uint4 b = *reinterpret_cast<const uint4 *>(O + t * ldo + head * BW_D + part * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc += bf2f((uint16_t)(u4_word(a, j >> 1) >> ((j & 1) * 16))) *
             bf2f((uint16_t)(u4_word(b, j >> 1) >> ((j & 1) * 16)));
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (live && part == 0) {
    const int64_t bi = t / s, q = t % s;
    Dr[(bi * hl + head) * s + q] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
// NW waves of 16*KT keys each, NW * 16 * KT == BW_BLK keys per workgroup
template <bool CAUSAL, int NW, int KT>
__global__ void __launch_bounds__(NW * 64) attn_bwd_dkdv_kernel(BwArgs a) {
  static_assert(NW * 16 * KT == BW_BLK, "keys per workgroup");
  // 2 stages x (Q tile, dO tile, the tile's lse2 and D rows: 1 KiB)
  constexpr int STG = 2 * BW_TILE + 512;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STG];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  // the second wave of every SIMD (waves NW/2 ..) issues the tile DMA
  constexpr int DW = NW / 2;
  const bool dmaw = wave >= DW;
  const int dwv = wave & (DW - 1);
  BwDma<DW> dma;
  dma.init(dwv, lane);
  const uint32_t lds0 = lds_addr(smem);

  int rank, bhs;
  bw_place(a, rank, bhs);
  const int kb = rank;  // key block 0 (longest under a causal mask) first
  const int hs = bhs % a.hsplit, bh = bhs / a.hsplit;
  const int bi = bh / a.kvl, kvh = bh % a.kvl;
  const int64_t tok0 = (int64_t)bi * a.s;
  const int key0 = kb * BW_BLK;
  const int k_w = key0 + wave * 16 * KT;

  // K, V of this wave's keys as B operands: lane supplies row key, d = dc*32 + g*8 ..
  const uint16_t *Kg = a.qkv + tok0 * a.ldq + (a.hl + kvh) * BW_D;
  const uint16_t *Vg = a.qkv + tok0 * a.ldq + (a.hl + a.kvl + kvh) * BW_D;
  uint4 kf[KT][4], vf[KT][4];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = k_w + kt * 16 + l16;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      kf[kt][dc] = make_uint4(0u, 0u, 0u, 0u);
      vf[kt][dc] = make_uint4(0u, 0u, 0u, 0u);
      if (key < a.s) {
        kf[kt][dc] = *reinterpret_cast<const uint4 *>(Kg + (int64_t)key * a.ldq + dc * 32 + g * 8);
        vf[kt][dc] = *reinterpret_cast<const uint4 *>(Vg + (int64_t)key * a.ldq + dc * 32 + g * 8);
      }
    }
  }
  f32x4_t dk[8][KT], dv[8][KT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      dk[dt][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      dv[dt][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

  const int nqt = (a.s + BW_TROWS - 1) / BW_TROWS;
  const int qt0 = CAUSAL ? key0 / BW_TROWS : 0;
  const float c = a.scale_log2;

  const int hper = a.group / a.hsplit;  // query heads of this workgroup
  for (int hg = hs * hper; hg < (hs + 1) * hper; ++hg) {
    const int head = kvh * a.group + hg;
    const uint16_t *Qg = a.qkv + tok0 * a.ldq + head * BW_D;
    const uint16_t *dOg = a.dO + tok0 * a.lddo + head * BW_D;
    const float *lse = a.lse + ((int64_t)bi * a.hl + head) * a.s;
    const float *Dr = a.Dr + ((int64_t)bi * a.hl + head) * a.s;

    // Tiles whose 64 rows all exist, with 16-byte aligned rows of lse2 / D
    // (s % 4 == 0), also bring those rows into LDS (the first DMA wave: lanes
    // 0..15 lse2, 16..31 D, 32..63 the same again); other tiles read them
    // from memory.
    auto issue = [&](int jt, uint32_t dst) {
      if (!dmaw) return;
      dma.tile(Qg, a.ldq, jt * BW_TROWS, a.s, dst, dwv);
      dma.tile(dOg, a.lddo, jt * BW_TROWS, a.s, dst + BW_TILE * 2, dwv);
      if (dwv == 0 && jt * BW_TROWS + BW_TROWS <= a.s && (a.s & 3) == 0)
        dma16(reinterpret_cast<const uint16_t *>(((lane & 16) ? Dr : lse) + jt * BW_TROWS + 4 * (lane & 15)),
              dst + 4 * BW_TILE);
    };
    __syncthreads();  // the previous head's readers are done with both stages
    issue(qt0, lds0);
    for (int j = qt0; j < nqt; ++j) {
      wait_vmcnt<0>();
      __syncthreads();  // tile j landed for every wave; the other stage is free
      const int st = (j - qt0) & 1;
      if (j + 1 < nqt) issue(j + 1, lds0 + (uint32_t)((st ^ 1) * STG * 2));
      const int q0 = j * BW_TROWS;
      if (CAUSAL && q0 + BW_TROWS - 1 < k_w) continue;  // every query precedes this wave's keys
      const uint16_t *Qs = smem + st * STG;
      const uint16_t *dOs = Qs + BW_TILE;
      const float *stats = reinterpret_cast<const float *>(Qs + 2 * BW_TILE);  // lse2 [64], D [64]
      const bool staged = q0 + BW_TROWS <= a.s && (a.s & 3) == 0;
      const bool edge = q0 + BW_TROWS > a.s || (CAUSAL && q0 < k_w + 16 * KT - 1);

      // two halves of 32 queries: kc selects query tiles 2kc, 2kc+1
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        f32x4_t S[2][KT], dP[2][KT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            S[h2][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            dP[h2][kt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int row = (2 * kc + h2) * 16 + l16;
            const uint4 qa = lds_frag(Qs, row, dc * 4 + g);
            const uint4 da = lds_frag(dOs, row, dc * 4 + g);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              S[h2][kt] = mfma16(qa, kf[kt][dc], S[h2][kt]);
              dP[h2][kt] = mfma16(da, vf[kt][dc], dP[h2][kt]);
            }
          }
        }
        // P and dS; lane holds queries q0 + (2kc+h2)*16 + 4g + r of key k_w + kt*16 + l16.
        // Only tiles that cross the diagonal or the end of the sequence need the
        // mask (keys past the end are discarded at the store; queries past it
        // must not contribute); the test is wave-uniform.
        uint4 pf[KT], sf[KT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int qb = q0 + (2 * kc + h2) * 16 + 4 * g;
          float lq[4], dq[4];
          if (staged) {
            const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(stats + qb - q0);
            const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(stats + BW_TROWS + qb - q0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              lq[r] = l4[r];
              dq[r] = d4[r];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int q = min(qb + r, a.s - 1);
              lq[r] = lse[q];
              dq[r] = Dr[q];
            }
          }
          if (edge) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
              const int key = k_w + kt * 16 + l16;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int q = qb + r;
                const bool ok = q < a.s && (!CAUSAL || key <= q);
                const float p = ok ? __builtin_amdgcn_exp2f(fmaf(S[h2][kt][r], c, -lq[r])) : 0.f;
                S[h2][kt][r] = p;
                dP[h2][kt][r] = p * (dP[h2][kt][r] - dq[r]);
              }
            }
          } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(S[h2][kt][r], c, -lq[r]));
                S[h2][kt][r] = p;
                dP[h2][kt][r] = p * (dP[h2][kt][r] - dq[r]);
              }
          }
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          pf[kt] = pack8(S[0][kt], S[1][kt]);
          sf[kt] = pack8(dP[0][kt], dP[1][kt]);
        }
        // dV^T[d][key] += dO^T P,  dK^T[d][key] += Q^T dS  (contraction over these 32 queries)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint4 ot = lds_trans(dOs, kc, dt, g, l16);
          const uint4 qt = lds_trans(Qs, kc, dt, g, l16);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            dv[dt][kt] = mfma16(ot, pf[kt], dv[dt][kt]);
            dk[dt][kt] = mfma16(qt, sf[kt], dk[dt][kt]);
          }
        }
      }
    }
    wait_vmcnt<0>();
  }

  // lane holds dK^T / dV^T rows d = dt*16 + 4g + r of key k_w + kt*16 + l16
  if (a.hsplit > 1) {  // fp32 partial of this head subset; attn_bwd_kv_sum_kernel adds them
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = k_w + kt * 16 + l16;
      if (key >= a.s) continue;
      float *pr = a.part + (((int64_t)hs * a.T + tok0 + key) * a.kvl + kvh) * 2 * BW_D;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        *reinterpret_cast<f32x4_t *>(pr + dt * 16 + 4 * g) = dk[dt][kt] * a.scale;
        *reinterpret_cast<f32x4_t *>(pr + BW_D + dt * 16 + 4 * g) = dv[dt][kt];
      }
    }
    return;
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = k_w + kt * 16 + l16;
    if (key >= a.s) continue;
    uint16_t *dKr = a.dqkv + (tok0 + key) * a.lddq + (a.hl + kvh) * BW_D;
    uint16_t *dVr = a.dqkv + (tok0 + key) * a.lddq + (a.hl + a.kvl + kvh) * BW_D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4_t k4 = dk[dt][kt] * a.scale;
      const f32x4_t v4 = dv[dt][kt];
      *reinterpret_cast<uint2 *>(dKr + dt * 16 + 4 * g) = make_uint2(pack_bf2(k4[0], k4[1]), pack_bf2(k4[2], k4[3]));
      *reinterpret_cast<uint2 *>(dVr + dt * 16 + 4 * g) = make_uint2(pack_bf2(v4[0], v4[1]), pack_bf2(v4[2], v4[3]));
    }
  }
}

// ---------------------------------------------------------------- dQ
template <bool CAUSAL>
__global__ void __launch_bounds__(BW_NW * 64, 2) attn_bwd_dq_kernel(BwArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * BW_TILE];  // 2 stages x (K, V)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  BwDma<BW_NW> dma;
  dma.init(wave, lane);
  const uint32_t lds0 = lds_addr(smem);

  int rank, bh;
  bw_place(a, rank, bh);
  const int qblk = CAUSAL ? a.nblk - 1 - rank : rank;  // the last query block is the longest
  const int bi = bh / a.hl, head = bh % a.hl;
  const int kvh = head / a.group;
  const int64_t tok0 = (int64_t)bi * a.s;
  const int q0 = qblk * BW_BLK;
  const int q_w = q0 + wave * BW_WROWS;

  const uint16_t *Qg = a.qkv + tok0 * a.ldq + head * BW_D;
  const uint16_t *dOg = a.dO + tok0 * a.lddo + head * BW_D;
  const uint16_t *Kg = a.qkv + tok0 * a.ldq + (a.hl + kvh) * BW_D;
  const uint16_t *Vg = a.qkv + tok0 * a.ldq + (a.hl + a.kvl + kvh) * BW_D;
  const float *lse = a.lse + ((int64_t)bi * a.hl + head) * a.s;
  const float *Dr = a.Dr + ((int64_t)bi * a.hl + head) * a.s;

  // Q and dO of this wave's 32 queries as B operands; lse2 and D of the
  // lane's query column
  uint4 qf[2][4], of[2][4];
  float lq[2], dq[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q_w + qt * 16 + l16;
    const int qc = min(q, a.s - 1);
    lq[qt] = lse[qc];
    dq[qt] = Dr[qc];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      qf[qt][dc] = make_uint4(0u, 0u, 0u, 0u);
      of[qt][dc] = make_uint4(0u, 0u, 0u, 0u);
      if (q < a.s) {
        qf[qt][dc] = *reinterpret_cast<const uint4 *>(Qg + (int64_t)q * a.ldq + dc * 32 + g * 8);
        of[qt][dc] = *reinterpret_cast<const uint4 *>(dOg + (int64_t)q * a.lddo + dc * 32 + g * 8);
      }
    }
  }
  f32x4_t dqa[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dqa[qt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nkt = CAUSAL ? (min(q0 + BW_BLK, a.s) + BW_TROWS - 1) / BW_TROWS : (a.s + BW_TROWS - 1) / BW_TROWS;
  const float c = a.scale_log2;

  dma.tile(Kg, a.ldq, 0, a.s, lds0, wave);
  dma.tile(Vg, a.ldq, 0, a.s, lds0 + BW_TILE * 2, wave);
  for (int j = 0; j < nkt; ++j) {
    wait_vmcnt<0>();
    __syncthreads();
    const int st = j & 1;
    if (j + 1 < nkt) {
      const uint32_t dst = lds0 + (uint32_t)((st ^ 1) * 2 * BW_TILE * 2);
      dma.tile(Kg, a.ldq, (j + 1) * BW_TROWS, a.s, dst, wave);
      dma.tile(Vg, a.ldq, (j + 1) * BW_TROWS, a.s, dst + BW_TILE * 2, wave);
    }
    const int k0 = j * BW_TROWS;
    if (q_w >= a.s || (CAUSAL && k0 > q_w + BW_WROWS - 1)) continue;  // no key of the tile is visible
    const uint16_t *Ks = smem + st * 2 * BW_TILE;
    const uint16_t *Vs = Ks + BW_TILE;

    // two halves of 32 keys: kc selects key tiles 2kc, 2kc+1
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f32x4_t S[2][2], dP[2][2];  // [key tile of the half][query tile]
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          S[h2][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          dP[h2][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
      // The MFMA blocks run at raised issue priority: of the two waves on a
      // SIMD (from the two resident workgroups), the one with matrix work
      // issues first while the other computes exponentials or reads LDS
      // (82 -> 74 us on the MHA shard; the dK/dV kernel measured slower).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int row = (2 * kc + h2) * 16 + l16;
          const uint4 ka = lds_frag(Ks, row, dc * 4 + g);
          const uint4 va = lds_frag(Vs, row, dc * 4 + g);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            S[h2][qt] = mfma16(ka, qf[qt][dc], S[h2][qt]);
            dP[h2][qt] = mfma16(va, of[qt][dc], dP[h2][qt]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // dS^T: lane holds keys k0 + (2kc+h2)*16 + 4g + r of query q_w + qt*16 + l16.
      // A key is visible when its offset (2kc+h2)*16 + r from the lane's first
      // key k0 + 4g is at most kmax: before the end of the sequence and, with
      // the causal mask, at or below the query.  Queries past the end only
      // feed their own, unstored dQ rows.
      uint4 sf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int q = q_w + qt * 16 + l16;
        const int kmax = (CAUSAL ? min(q, a.s - 1) : a.s - 1) - (k0 + 4 * g);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = (2 * kc + h2) * 16 + r <= kmax;
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(S[h2][qt][r], c, -lq[qt])) : 0.f;
            dP[h2][qt][r] = p * (dP[h2][qt][r] - dq[qt]);
          }
        sf[qt] = pack8(dP[0][qt], dP[1][qt]);
      }
      // dQ^T[d][q] += K^T dS^T (contraction over these 32 keys)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 kt = lds_trans(Ks, kc, dt, g, l16);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) dqa[qt][dt] = mfma16(kt, sf[qt], dqa[qt][dt]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q_w + qt * 16 + l16;
    if (q >= a.s) continue;
    uint16_t *dQr = a.dqkv + (tok0 + q) * a.lddq + head * BW_D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4_t v = dqa[qt][dt] * a.scale;
      *reinterpret_cast<uint2 *>(dQr + dt * 16 + 4 * g) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
    }
  }
}

// dK | dV = sum over the hsplit partials in order, rounded to bf16 into the
// K and V blocks of dqkv; one thread per 4 consecutive elements of a row
__global__ void __launch_bounds__(256) attn_bwd_kv_sum_kernel(const float *__restrict__ part, int hsplit, int64_t T,
                                                              int hl, int kvl, uint16_t *dqkv, int64_t lddq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (token, kv head, K|V, d/4)
  const int64_t per_tok = (int64_t)kvl * 2 * (BW_D / 4);
  if (i >= T * per_tok) return;
  const int64_t tok = i / per_tok;
  const int rem = (int)(i % per_tok);
  const int kvh = rem / (2 * (BW_D / 4));
  const int w = (rem / (BW_D / 4)) & 1;
  const int d4 = rem % (BW_D / 4);
  const int64_t src = ((tok * kvl + kvh) * 2 + w) * BW_D + d4 * 4;
  f32x4_t acc = *reinterpret_cast<const f32x4_t *>(part + src);
  for (int hs = 1; hs < hsplit; ++hs) acc += *reinterpret_cast<const f32x4_t *>(part + hs * T * kvl * 2 * BW_D + src);
  *reinterpret_cast<uint2 *>(dqkv + tok * lddq + (hl + w * kvl + kvh) * BW_D + d4 * 4) =
      make_uint2(pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]));
}

// Workgroups that share one kv head's query heads in the dK/dV pass: with
// fewer than 512 (sequence, kv head, key block) workgroups the group's heads
// are split (a power of two dividing the group) so the chip fills; each
// split writes an fp32 partial that attn_bwd_kv_sum_kernel adds in order.
int attn_bwd_hsplit(int64_t b, int64_t s, int64_t heads_local, int64_t kv_heads_local) {
  if (kv_heads_local < 1 || heads_local % kv_heads_local) return 1;
  const int64_t g = heads_local / kv_heads_local;
  const int64_t wgs = b * kv_heads_local * ((s + BW_BLK - 1) / BW_BLK);
  int64_t hs = 1;
  while (hs < g && g % (2 * hs) == 0 && wgs * hs < 512) hs *= 2;
  return (int)hs;
}

size_t attn_bwd_part_bytes(int64_t b, int64_t s, int64_t heads_local, int64_t kv_heads_local) {
  const int hs = attn_bwd_hsplit(b, s, heads_local, kv_heads_local);
  return hs > 1 ? (size_t)hs * (size_t)(b * s) * (size_t)kv_heads_local * 2 * BW_D * 4 : 0;
}

hipError_t launch_attn_bwd(const void *qkv, int64_t ldqkv, const void *O, int64_t ldo, const float *lse,
                           const void *dO, int64_t lddo, float *Dr, void *dqkv, float *part, int64_t b, int64_t s,
                           int64_t heads_local, int64_t kv_heads_local, int64_t d, bool causal, hipStream_t st) {
  if (b <= 0 || s <= 0 || heads_local <= 0) return hipSuccess;
  if (d != BW_D) return hipErrorInvalidValue;
  if (kv_heads_local < 1 || heads_local % kv_heads_local) return hipErrorInvalidValue;
  if (ldqkv > BW_MAX_LD || lddo > BW_MAX_LD) return hipErrorInvalidValue;  // 32-bit DMA offsets
  const int64_t T = b * s;
  const int64_t rows = T * heads_local;
  hipLaunchKernelGGL(attn_bwd_dot_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(dO), lddo, static_cast<const uint16_t *>(O), ldo, T, (int)s,
                     (int)heads_local, Dr);
  BwArgs a;
  a.qkv = static_cast<const uint16_t *>(qkv);
  a.ldq = ldqkv;
  a.dO = static_cast<const uint16_t *>(dO);
  a.lddo = lddo;
  a.lse = lse;
  a.Dr = Dr;
  a.dqkv = static_cast<uint16_t *>(dqkv);
  a.lddq = ldqkv;
  a.s = (int)s;
  a.hl = (int)heads_local;
  a.kvl = (int)kv_heads_local;
  a.group = (int)(heads_local / kv_heads_local);
  a.scale = 1.0f / sqrtf((float)d);
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  a.nblk = (int)((s + BW_BLK - 1) / BW_BLK);

  a.T = T;
  a.hsplit = attn_bwd_hsplit(b, s, heads_local, kv_heads_local);
  a.part = part;
  if (a.hsplit > 1 && part == nullptr) return hipErrorInvalidValue;
  a.nbh = (int)(b * kv_heads_local * a.hsplit);
  const dim3 g1((unsigned)(a.nbh * a.nblk));
  if (causal)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<true, DK_NW, DK_KT>), g1, dim3(DK_NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<false, DK_NW, DK_KT>), g1, dim3(DK_NW * 64), 0, st, a);
  if (a.hsplit > 1) {
    const int64_t n4 = T * kv_heads_local * 2 * (BW_D / 4);
    hipLaunchKernelGGL(attn_bwd_kv_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, a.hsplit,
                       T, (int)heads_local, (int)kv_heads_local, a.dqkv, a.lddq);
  }
  a.hsplit = 1;
  a.nbh = (int)(b * heads_local);
  const dim3 g2((unsigned)(a.nbh * a.nblk));
  if (causal)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<true>, g2, dim3(BW_NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<false>, g2, dim3(BW_NW * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpcol
