// Head-local attention for one tensor-parallel shard (bf16, head dim 128).
// Multi-head, or grouped-query with kv_heads_local key/value heads shared by
// consecutive groups of heads_local / kv_heads_local query heads
// ("张量并行", 相关分析: GQA).
//
// Each shard owns heads_local whole heads, so attention needs nothing from
// other shards ("张量并行", Multi-Head Attention 的并行化: heads are
// independent; "Infra: Tensor Parallel", MHA).  Per (sequence, head):
//     O = softmax(Q K^T / sqrt(d) [+ causal mask]) V
// computed flash-style: K/V are streamed in 64-key blocks through LDS and a
// running max / running sum keep the softmax exact without materialising
// the s x s score matrix.
//
// gfx950 design:
//  * Workgroup = 8 wave64 on one 128-query block of one (sequence, head):
//    two groups of 4 waves, 32 queries per wave, the same queries in both
//    groups.  Group 0 takes the even key blocks, group 1 the odd ones, and
//    the two partial softmax states (max, sum, unnormalised O) are merged
//    through LDS at the end.  Two waves share each SIMD, so one wave's
//    exponentials overlap the other's matrix-core work, while every wave
//    still owns 32 queries: the K/V fragments a wave reads from LDS per key
//    block are fixed, so fewer queries per wave would raise LDS traffic per
//    flop, and LDS (not the matrix cores) is the tighter limit on gfx950 for
//    the 8-byte transpose reads.
//  * With a causal mask a workgroup handles the query blocks p and nqb-1-p
//    one after the other, so every workgroup does the same number of key
//    blocks (the causal triangle otherwise leaves the short blocks' CUs idle
//    while the long ones finish).
//  * K and V tiles move HBM -> LDS by direct DMA (global_load_lds_dwordx4,
//    no staging registers) through two 4-deep rings of [key][d] tiles (K and
//    V): each step consumes two blocks while the next two land.  The L2 ->
//    LDS path takes a step's 64 KiB at ~44 B/cycle, and a wave cannot issue
//    past a full DMA queue, so the issue blocks the issuing wave for ~1,500
//    cycles.  Only the waves of group 0 issue it, right after their score
//    MFMAs, while group 1 (one block behind) runs the exponentials and P V of
//    its previous block: group 0's chain is the shorter one (4 x 2048-token,
//    8-head causal shard: all eight waves issuing at the step start 64 us,
//    group 1 at the step start 59, group 0 after its scores 57).  Group 1
//    runs one block behind group 0 inside each step (softmax and P V of its
//    previous block first, then the scores of its next one), so after every
//    barrier one wave of each SIMD starts on the matrix cores and the other
//    on the exponentials instead of both contending for one unit.  K is
//    read with ds_read_b128 (granule c of row r stored at c ^ (r & 15)); the
//    V^T operand of the second product comes from ds_read_b64_tr_b16
//    transpose reads (granule c of row r at c ^ 2(r & 7)).  Both layouts are
//    bank-conflict free for the reads they serve.
//  * S^T = K Q^T on the matrix cores (16x16x32 bf16, Q held in registers as
//    the B operand): each lane gets 4 keys of ONE query, so a row max needs
//    two cross-lane steps (gfx950 row swaps) and the probabilities already
//    sit in the B-operand layout of O^T += V^T P^T.
//  * The running max is updated lazily: the accumulator is rescaled only
//    when a block's max exceeds the reference by more than 2^8 (so every
//    probability stays <= 256 and the result is the same up to rounding).
//    The mask is evaluated only on blocks that cross the diagonal or the
//    end of the sequence; the row sum stays per lane until the end.
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace tpcol {

static constexpr int FA_D = 128;
static constexpr int FA_BQ = 128;     // queries per workgroup block
static constexpr int FA_BKV = 64;     // keys per block
static constexpr int FA_NW = 8;       // waves per workgroup (two groups of 4)
static constexpr int FA_QW = 32;      // queries per wave
static constexpr int FA_STAGES = 4;
static constexpr int FA_TILE = FA_BKV * FA_D;  // elements of one K or V tile (16 KiB)
static constexpr int FA_VRING = FA_STAGES * FA_TILE;  // element offset of the V ring (K ring first)
static constexpr int FA_DW = FA_NW / 2;       // waves that issue the K/V DMA (group 0)
static constexpr int FA_JN = 16 / FA_DW;       // wave-DMAs per issuing wave per tile
static constexpr int FA_ROWS_J = 4 * FA_DW;    // tile rows between one wave's DMA chunks
static constexpr float FA_RESCALE_LOG2 = 8.0f;
static constexpr int64_t FA_MAX_LD = int64_t(1) << 24;  // keeps 64 rows' byte offsets in 32 bits

// Butterfly steps across lanes i and i ^ 16 / i ^ 32 with the gfx950 row
// swaps: after v_permlane{16,32}_swap of a register with itself, one of the
// two results holds the lane's own value and the other its partner's.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct FaArgs {
  const uint16_t *qkv;
  int64_t ldq;
  uint16_t *O;
  int64_t ldo;
  int s, hl, nqb, items;  // items: workgroups per (sequence, head)
  int kvl, group;         // key/value heads in the shard; query heads per kv head
  float scale_log2;       // log2(e) / sqrt(d)
  float *lse;             // [b][hl][s]: log2 of each row's softmax denominator, or NULL
};

template <bool CAUSAL>
struct FaBlock {
  // per-lane constants
  int lane, wave, grp, wq, g, l16;
  int row_lo;          // tile row of this lane's first DMA slot (later ones are FA_ROWS_J apart)
  uint32_t koff, voff; // byte offset of that slot's source granule (K, V) from a chunk's first row
  int vsw;             // V read swizzle of this lane's rows
  uint32_t lds0;       // LDS byte address of stage 0
  uint16_t *smem;

  // DMA of one 64-key tile (K or V rows of key block kb) into the LDS tile
  // at byte address dst.  Full blocks use a scalar base per row chunk plus
  // one per-lane offset; the ragged last block clamps each lane's row to
  // the last key (those keys are masked).
  __device__ __forceinline__ void issue_tile(const FaArgs &a, const uint16_t *G, uint32_t off, int kb,
                                             uint32_t dst) const {
    const int key0 = kb * FA_BKV;
    if (key0 + FA_BKV <= a.s) {
#pragma unroll
      for (int j = 0; j < FA_JN; ++j)
        dma16s(off, G + (int64_t)(key0 + FA_ROWS_J * j) * a.ldq, dst + (wq + FA_DW * j) * 1024);
    } else {
      const uint16_t *base = G + (int64_t)key0 * a.ldq;
      const uint32_t ldb = (uint32_t)a.ldq * 2u;
#pragma unroll
      for (int j = 0; j < FA_JN; ++j) {
        const uint32_t r = (uint32_t)min(FA_ROWS_J * j + row_lo, a.s - 1 - key0);
        dma16s(r * ldb + (off - (uint32_t)row_lo * ldb), base, dst + (wq + FA_DW * j) * 1024);
      }
    }
  }
  // Block kb goes to ring stage kb % 4; block indexes past the last block
  // (nkb - 1) fetch nothing (every wait is for all of a wave's DMAs).
  __device__ __forceinline__ void issue_k(const FaArgs &a, const uint16_t *Kg, int kb, int nkb) const {
    if (kb < nkb) issue_tile(a, Kg, koff, kb, lds0 + (uint32_t)((kb % FA_STAGES) * FA_TILE * 2));
  }
  __device__ __forceinline__ void issue_v(const FaArgs &a, const uint16_t *Vg, int kb, int nkb) const {
    if (kb < nkb) issue_tile(a, Vg, voff, kb, lds0 + (uint32_t)((FA_VRING + (kb % FA_STAGES) * FA_TILE) * 2));
  }

  // S^T[key][q] for the 64 keys of a stage x the wave's 32 queries
  __device__ __forceinline__ void scores(int stage, const uint4 (&qf)[2][4], f32x4_t (&st)[4][2]) const {
    const uint16_t *Ks = smem + stage * FA_TILE;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) st[mt][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = mt * 16 + l16;
        const uint4 kf =
            *reinterpret_cast<const uint4 *>(Ks + row * FA_D + (((dc * 4 + g) ^ l16) << 3));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) st[mt][qt] = mfma16(kf, qf[qt][dc], st[mt][qt]);
      }
    }
  }

  // O^T[d][q] += V^T[d][key] P^T[key][q]; key slots of chunk kc are
  // {32kc + 4g + r, 32kc + 16 + 4g + r}, matching the packing of pf
  __device__ __forceinline__ void pv(int stage, const uint4 (&pf)[2][2], f32x4_t (&o)[2][8]) const {
    const uint16_t *Vs = smem + FA_VRING + stage * FA_TILE;
    const int e = l16 >> 2, c = l16 & 3;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int row = 32 * kc + 4 * g + e;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int col = dt * 16 + 4 * c;
        const int off = (((col >> 3) ^ vsw) << 3) + (col & 4);
        const uint2 v0 = tr_read(Vs + row * FA_D + off);
        const uint2 v1 = tr_read(Vs + (row + 16) * FA_D + off);
        const uint4 vf = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[qt][dt] = mfma16(vf, pf[qt][kc], o[qt][dt]);
      }
    }
  }

  // One 128-query block: queries qb*128 .. +127 of (sequence bi, head).
  __device__ __forceinline__ void run(const FaArgs &a, int bi, int head, int qb) const {
    const int64_t tok0 = (int64_t)bi * a.s;
    const uint16_t *Qg = a.qkv + tok0 * a.ldq + head * FA_D;
    const int kvh = head / a.group;  // grouped-query: the kv head this query head reads
    const uint16_t *Kg = a.qkv + tok0 * a.ldq + (a.hl + kvh) * FA_D;
    const uint16_t *Vg = a.qkv + tok0 * a.ldq + (a.hl + a.kvl + kvh) * FA_D;
    const int q0 = qb * FA_BQ;
    const int q_w = q0 + wq * FA_QW;

    // key blocks of the workgroup and of this wave (blocks 0 .. nkw-1, of
    // which this wave's group takes those with index parity grp)
    const int nkb = CAUSAL ? (min(q0 + FA_BQ, a.s) + FA_BKV - 1) / FA_BKV : (a.s + FA_BKV - 1) / FA_BKV;
    int nkw = 0;
    if (q_w < a.s) nkw = CAUSAL ? min(q_w + FA_QW - 1, a.s - 1) / FA_BKV + 1 : nkb;
    const int nsteps = (nkb + 1) / 2;

    // Q as the B operand: lane supplies Q[q][dc*32 + g*8 .. +7]
    uint4 qf[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int q = q_w + qt * 16 + l16;
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        qf[qt][dc] = make_uint4(0u, 0u, 0u, 0u);
        if (q < a.s) qf[qt][dc] = *reinterpret_cast<const uint4 *>(Qg + (int64_t)q * a.ldq + dc * 32 + g * 8);
      }
    }

    f32x4_t o[2][8];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[qt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float mref[2] = {-INFINITY, -INFINITY};  // reference max, log2 units
    float lsum[2] = {0.f, 0.f};              // this lane's part of the row sum
    const float c = a.scale_log2;

    // softmax of key block j: scores in st -> bf16 probabilities in pf
    auto softmax = [&](int j, f32x4_t(&st)[4][2], uint4(&pf)[2][2]) {
      const int key0 = j * FA_BKV;
      const bool masked = (key0 + FA_BKV > a.s) || (CAUSAL && key0 + FA_BKV - 1 > q_w);
      float mx[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int q = q_w + qt * 16 + l16;
        if (masked) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = key0 + mt * 16 + 4 * g + r;
              const bool ok = key < a.s && (!CAUSAL || key <= q);
              st[mt][qt][r] = ok ? st[mt][qt][r] : -INFINITY;
            }
        }
        float m = st[0][qt][0];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, st[mt][qt][r]);
        mx[qt] = max_xor32(max_xor16(m)) * c;
      }
      const bool grow = mx[0] > mref[0] + FA_RESCALE_LOG2 || mx[1] > mref[1] + FA_RESCALE_LOG2;
      if (__any(grow)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float mn = fmaxf(mref[qt], mx[qt]);
          const float alpha = __builtin_amdgcn_exp2f(mref[qt] - mn);
          mref[qt] = mn;
          lsum[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[qt][dt] *= alpha;
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float nm = -mref[qt];
        float p[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[mt][r] = __builtin_amdgcn_exp2f(fmaf(st[mt][qt][r], c, nm));
            lsum[qt] += p[mt][r];
          }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          pf[qt][kc] = make_uint4(pack_bf2(p[2 * kc][0], p[2 * kc][1]), pack_bf2(p[2 * kc][2], p[2 * kc][3]),
                                  pack_bf2(p[2 * kc + 1][0], p[2 * kc + 1][1]),
                                  pack_bf2(p[2 * kc + 1][2], p[2 * kc + 1][3]));
      }
    };

    // Step t: group 0 handles key block 2t (scores, softmax, O += P V);
    // group 1 first finishes block 2t-1 (softmax, O += P V, its scores were
    // computed in step t-1) and then computes the scores of block 2t+1.  So
    // after each barrier one wave of every SIMD starts on the matrix cores
    // and the other on the exponentials.  Resident in step t: K(2t), K(2t+1),
    // V(2t-1), V(2t); in flight: K(2t+2), K(2t+3), V(2t+1), V(2t+2), each in
    // ring stage (block % 4) of its own ring, issued by group 0 after its
    // scores (the stages they overwrite were last read in step t-1).
    __syncthreads();  // the previous query block's readers are done with the rings
    if (grp == 0) {
      issue_k(a, Kg, 0, nkb);
      issue_k(a, Kg, 1, nkb);
      issue_v(a, Vg, 0, nkb);
    }

    // One code path for both groups (wave-uniform conditions only):
    // group 0 scores block 2t and finishes it in the same step, group 1
    // finishes block 2t-1 (scored in step t-1) and then scores block 2t+1.
    f32x4_t st[4][2];
    for (int t = 0; t <= nsteps; ++t) {
      wait_vmcnt<0>();   // this wave's DMAs for step t have landed
      __syncthreads();   // ... and every wave's; the stages used in step t-1 are free
      const int jp = 2 * t - grp;        // block finished in this step
      const int jn = 2 * t + grp;        // block scored in this step
      if (grp == 0 && jn < nkw) scores(jn % FA_STAGES, qf, st);
      if (grp == 0) {
        issue_k(a, Kg, 2 * t + 2, nkb);
        issue_k(a, Kg, 2 * t + 3, nkb);
        issue_v(a, Vg, 2 * t + 1, nkb);
        issue_v(a, Vg, 2 * t + 2, nkb);
      }
      if (jp >= 0 && jp < nkw) {
        uint4 pf[2][2];
        softmax(jp, st, pf);
        pv(jp % FA_STAGES, pf, o);
      }
      if (grp == 1 && jn < nkw) scores(jn % FA_STAGES, qf, st);
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done reading the ring

    // ---- merge the two groups' states through LDS (the ring is free now):
    // group 1 stores (o, max, partial sums) in its own lane layout, group 0
    // (same queries, same lanes) combines and writes O
    float *xo = reinterpret_cast<float *>(smem) + wq * (2 * 8 * 4 * 64);  // 16 KiB per query slice
    float *xm = reinterpret_cast<float *>(smem) + 4 * (2 * 8 * 4 * 64) + wq * (4 * 64);
    if (grp == 1) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4_t *>(xo + ((qt * 8 + dt) * 64 + lane) * 4) = o[qt][dt];
        xm[(qt * 2 + 0) * 64 + lane] = mref[qt];
        xm[(qt * 2 + 1) * 64 + lane] = lsum[qt];
      }
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float m1 = xm[(qt * 2 + 0) * 64 + lane];
        const float l1 = xm[(qt * 2 + 1) * 64 + lane];
        const float m = fmaxf(mref[qt], m1);
        // a group with no key block for these queries has max -inf: weight 0
        const float a0 = mref[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref[qt] - m);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
        const float l = sum_xor32(sum_xor16(lsum[qt] * a0 + l1 * a1));
        const int q = q_w + qt * 16 + l16;
        const float inv = 1.0f / l;
        // the backward recomputes P = exp2(S log2(e)/sqrt(d) - lse2) from this
        if (a.lse != nullptr && g == 0 && q < a.s) a.lse[((int64_t)bi * a.hl + head) * a.s + q] = m + log2f(l);
        uint16_t *orow = a.O + (tok0 + q) * a.ldo + head * FA_D;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x4_t o1 = *reinterpret_cast<const f32x4_t *>(xo + ((qt * 8 + dt) * 64 + lane) * 4);
          const f32x4_t v = (o[qt][dt] * a0 + o1 * a1) * inv;
          if (q < a.s)
            *reinterpret_cast<uint2 *>(orow + dt * 16 + 4 * g) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
        }
      }
    }
  }
};

template <bool CAUSAL>
__global__ void __launch_bounds__(FA_NW * 64) flash_attn_kernel(FaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * FA_STAGES * FA_TILE];

  FaBlock<CAUSAL> fb;
  fb.lane = threadIdx.x & 63;
  fb.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  fb.grp = fb.wave >> 2;  // waves w and w+4 share a SIMD: one from each group
  fb.wq = fb.wave & 3;
  fb.g = fb.lane >> 4;
  fb.l16 = fb.lane & 15;
  // DMA slot of this lane: row 4*blk + lane/16, granule slot lane%16; rows
  // of one lane differ by multiples of 16, so the swizzles are per lane
  fb.row_lo = 4 * fb.wq + (fb.lane >> 4);
  const uint32_t row_bytes = (uint32_t)fb.row_lo * (uint32_t)a.ldq * 2u;
  fb.koff = row_bytes + (uint32_t)(((fb.lane & 15) ^ (fb.row_lo & 15)) * 16);
  fb.voff = row_bytes + (uint32_t)(((fb.lane & 15) ^ ((fb.row_lo & 7) << 1)) * 16);
  fb.vsw = ((4 * fb.g + (fb.l16 >> 2)) & 7) << 1;
  fb.smem = smem;
  fb.lds0 = lds_addr(smem);

  // workgroup -> (sequence, head, item); the 8 XCDs each get a contiguous
  // run of (sequence, head) pairs so their K/V stay in that XCD's L2 (query
  // heads of one kv group are consecutive, so they share it too)
  const int nwg = (int)gridDim.x;
  int logical = (int)blockIdx.x;
  if ((nwg & 7) == 0) logical = (logical & 7) * (nwg >> 3) + (logical >> 3);
  const int bh = logical / a.items, item = logical % a.items;
  const int bi = bh / a.hl, head = bh % a.hl;

  if (CAUSAL) {
    const int qb_long = a.nqb - 1 - item;
    fb.run(a, bi, head, qb_long);
    if (item != qb_long) fb.run(a, bi, head, item);
  } else {
    fb.run(a, bi, head, item);
  }
}

hipError_t launch_flash_attn(const void *qkv, int64_t ldqkv, void *O, int64_t ldo, float *lse, int64_t b,
                             int64_t s, int64_t heads_local, int64_t kv_heads_local, int64_t d,
                             bool causal, hipStream_t st) {
  if (b <= 0 || s <= 0 || heads_local <= 0) return hipSuccess;
  if (d != FA_D) return hipErrorInvalidValue;
  if (kv_heads_local < 1 || heads_local % kv_heads_local) return hipErrorInvalidValue;
  if (ldqkv > FA_MAX_LD) return hipErrorInvalidValue;  // 32-bit DMA offsets
  FaArgs a;
  a.qkv = static_cast<const uint16_t *>(qkv);
  a.ldq = ldqkv;
  a.O = static_cast<uint16_t *>(O);
  a.ldo = ldo;
  a.lse = lse;
  a.s = (int)s;
  a.hl = (int)heads_local;
  a.kvl = (int)kv_heads_local;
  a.group = (int)(heads_local / kv_heads_local);
  a.nqb = (int)((s + FA_BQ - 1) / FA_BQ);
  a.items = causal ? (a.nqb + 1) / 2 : a.nqb;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  const dim3 grid((unsigned)(a.items * b * heads_local));
  if (causal)
    hipLaunchKernelGGL(flash_attn_kernel<true>, grid, dim3(FA_NW * 64), 0, st, a);
  else
    hipLaunchKernelGGL(flash_attn_kernel<false>, grid, dim3(FA_NW * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace tpcol
