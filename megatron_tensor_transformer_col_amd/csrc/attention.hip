// Head-local attention for one tensor-parallel shard (bf16, head dim 128).
//
// Each shard owns heads_local whole heads, so attention needs nothing from
// other shards ("张量并行", Multi-Head Attention 的并行化: heads are
// independent; "Infra: Tensor Parallel", MHA).  Per (sequence, head):
//     O = softmax(Q K^T / sqrt(d) [+ causal mask]) V
// computed flash-style: K/V are streamed in 64-key blocks through LDS and a
// running max / running sum keep the softmax exact without materialising
// the s x s score matrix.
//
// Workgroup = 4 wave64 = 128 queries of one (sequence, head); each wave owns
// 32 queries.  The wave computes S^T = K Q^T on the matrix cores (16x16x32
// bf16 MFMA, Q held in registers as the B operand), so every lane ends up
// with 4 keys of ONE query column: the row max / row sum need only two
// cross-lane xor steps, and the probabilities already sit in the B-operand
// layout of the next product O^T += V^T P^T (no shuffle).  V is transposed
// into LDS ([d][key]) on the way in, K is stored [key][d]; both tiles are
// double-buffered.  Scores and the running statistics are fp32; P is rounded
// to bf16 for the second product.  Causal workgroups are issued
// longest-first.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tpcol {

static constexpr int FA_D = 128;
static constexpr int FA_BQ = 128;
static constexpr int FA_BKV = 64;
static constexpr int FA_LDK = FA_D + 8;
static constexpr int FA_LDV = FA_BKV + 8;
static constexpr int FA_NT = 256;

template <bool CAUSAL>
__global__ void __launch_bounds__(FA_NT)
flash_attn_kernel(const uint16_t *__restrict__ qkv, int64_t ldq, uint16_t *__restrict__ O,
                  int64_t ldo, int nb, int s, int hl, int nqb, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][FA_BKV * FA_LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][FA_D * FA_LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;

  // block -> (q-block, sequence, head); the longest causal rows go first
  const int per_qb = nb * hl;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);
  const int rest = blockIdx.x % per_qb;
  const int bi = rest / hl, head = rest % hl;

  const int64_t tok0 = (int64_t)bi * s;
  const uint16_t *Qg = qkv + tok0 * ldq + head * FA_D;
  const uint16_t *Kg = qkv + tok0 * ldq + (hl + head) * FA_D;
  const uint16_t *Vg = qkv + tok0 * ldq + (2 * hl + head) * FA_D;

  const int q_wg = qb * FA_BQ;
  const int q_w = q_wg + wave * 32;

  // Q as the B operand: lane supplies Q[q][dc*32 + g*8 .. +7]
  uint4 qf[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q_w + qt * 16 + l16;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      qf[qt][dc] = make_uint4(0u, 0u, 0u, 0u);
      if (q < s) qf[qt][dc] = *reinterpret_cast<const uint4 *>(Qg + (int64_t)q * ldq + dc * 32 + g * 8);
    }
  }

  f32x4_t o[2][8];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[qt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};

  const int kv_end = CAUSAL ? min(s, q_wg + FA_BQ) : s;
  const int nkb = (kv_end + FA_BKV - 1) / FA_BKV;

  // K block: 64 keys x 128 d, 16-byte vectors, [key][d] in LDS
  constexpr int KV_PER = FA_BKV * FA_D / 8 / FA_NT;  // 4
  uint4 kreg[KV_PER];
  // V block: 8x8 (key x d) blocks transposed to [d][key]; 128 blocks
  uint4 vreg[8];
  const bool v_owner = tid < (FA_BKV / 8) * (FA_D / 8);
  const int v_cb = tid % (FA_D / 8), v_kb = tid / (FA_D / 8);

  auto load_kv = [&](int kb) {
    const int key0 = kb * FA_BKV;
#pragma unroll
    for (int i = 0; i < KV_PER; ++i) {
      const int v = tid + i * FA_NT;
      const int row = v >> 4, dv = v & 15;
      const int key = key0 + row;
      kreg[i] = make_uint4(0u, 0u, 0u, 0u);
      if (key < s) kreg[i] = *reinterpret_cast<const uint4 *>(Kg + (int64_t)key * ldq + dv * 8);
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int key = key0 + v_kb * 8 + rr;
      vreg[rr] = make_uint4(0u, 0u, 0u, 0u);
      if (v_owner && key < s)
        vreg[rr] = *reinterpret_cast<const uint4 *>(Vg + (int64_t)key * ldq + v_cb * 8);
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KV_PER; ++i) {
      const int v = tid + i * FA_NT;
      const int row = v >> 4, dv = v & 15;
      *reinterpret_cast<uint4 *>(&Ks[buf][row * FA_LDK + dv * 8]) = kreg[i];
    }
    if (v_owner) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = u4_word(vreg[2 * q], c >> 1);
          const uint32_t hi = u4_word(vreg[2 * q + 1], c >> 1);
          w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<uint4 *>(&Vt[buf][(v_cb * 8 + c) * FA_LDV + v_kb * 8]) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) load_kv(kb + 1);

    const int key0 = kb * FA_BKV;
    if (!CAUSAL || key0 <= q_w + 31) {
      // ---- S^T[key][q] for 64 keys x 32 queries
      f32x4_t st[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) st[mt][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 kf =
              *reinterpret_cast<const uint4 *>(&Ks[cur][(mt * 16 + l16) * FA_LDK + dc * 32 + g * 8]);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) st[mt][qt] = mfma16(kf, qf[qt][dc], st[mt][qt]);
        }
      }

      // ---- online softmax per query column
      uint4 pf[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int q = q_w + qt * 16 + l16;
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + mt * 16 + 4 * g + r;
            const bool ok = key < s && (!CAUSAL || key <= q);
            const float v = ok ? st[mt][qt][r] * scale_log2 : -INFINITY;
            st[mt][qt][r] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(mrow[qt], mx);
        const float alpha = exp2f(mrow[qt] - m_new);
        float sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = exp2f(st[mt][qt][r] - m_new);
            st[mt][qt][r] = pv;
            sum += pv;
          }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        lrow[qt] = lrow[qt] * alpha + sum;
        mrow[qt] = m_new;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[qt][dt] *= alpha;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          pf[qt][kc] = make_uint4(pack_bf2(st[2 * kc][qt][0], st[2 * kc][qt][1]),
                                  pack_bf2(st[2 * kc][qt][2], st[2 * kc][qt][3]),
                                  pack_bf2(st[2 * kc + 1][qt][0], st[2 * kc + 1][qt][1]),
                                  pack_bf2(st[2 * kc + 1][qt][2], st[2 * kc + 1][qt][3]));
      }

      // ---- O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint16_t *vrow = &Vt[cur][(dt * 16 + l16) * FA_LDV + kc * 32 + 4 * g];
          const uint2 v0 = *reinterpret_cast<const uint2 *>(vrow);
          const uint2 v1 = *reinterpret_cast<const uint2 *>(vrow + 16);
          const uint4 vf = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) o[qt][dt] = mfma16(vf, pf[qt][kc], o[qt][dt]);
        }
      }
    }

    if (kb + 1 < nkb) store_kv(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise and write O[token][head*128 + d] (4 consecutive d per lane)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q_w + qt * 16 + l16;
    if (q >= s) continue;
    const float inv = 1.0f / lrow[qt];
    uint16_t *orow = O + (tok0 + q) * ldo + head * FA_D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      *reinterpret_cast<uint2 *>(orow + dt * 16 + 4 * g) =
          make_uint2(pack_bf2(o[qt][dt][0] * inv, o[qt][dt][1] * inv),
                     pack_bf2(o[qt][dt][2] * inv, o[qt][dt][3] * inv));
    }
  }
}

hipError_t launch_flash_attn(const void *qkv, int64_t ldqkv, void *O, int64_t ldo, int64_t b,
                             int64_t s, int64_t heads_local, int64_t d, bool causal,
                             hipStream_t st) {
  if (b <= 0 || s <= 0 || heads_local <= 0) return hipSuccess;
  if (d != FA_D) return hipErrorInvalidValue;
  const int nqb = (int)((s + FA_BQ - 1) / FA_BQ);
  const dim3 grid((unsigned)(nqb * b * heads_local));
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  if (causal)
    hipLaunchKernelGGL(flash_attn_kernel<true>, grid, dim3(FA_NT), 0, st,
                       static_cast<const uint16_t *>(qkv), ldqkv, static_cast<uint16_t *>(O), ldo,
                       (int)b, (int)s, (int)heads_local, nqb, scale_log2);
  else
    hipLaunchKernelGGL(flash_attn_kernel<false>, grid, dim3(FA_NT), 0, st,
                       static_cast<const uint16_t *>(qkv), ldqkv, static_cast<uint16_t *>(O), ldo,
                       (int)b, (int)s, (int)heads_local, nqb, scale_log2);
  return hipGetLastError();
}

}  // namespace tpcol
