// Causal GQA prefill, bf16 inputs, fp32 accumulation, MFMA 32x32x16 on gfx950.
//
// What is computed (per batch b, query head h, query row i):
//   o_i = sum_j softmax_j(scale * q_i . k_j + M_ij) v_j,  kv head = floor(h / g)
// which is the SDPA definition of "Module 5. Modern Attention Mechanisms",
// section 4, with the GQA head rule of its section 6. The work is organised as
// in the "FlashAttention" section of the "inference-attention" page: key/value
// tiles are streamed through on-chip memory, each query row carries a running
// max m, a running sum l and an unnormalised output O that is rescaled by
// 2^(m - m') whenever the max grows, and the output is O / l after the last
// tile. Tiles entirely above the causal diagonal are never visited.
//
// Mapping onto CDNA4:
//  * A work-group of NW waves owns BM = NW * QB * 32 consecutive query rows of
//    one (b, h). Each wave owns QB blocks of 32 rows.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims read from LDS, B = Q^T
//    held in registers for the whole kernel). In the MFMA result layout lane l
//    then holds 16 keys of query row l % 32, so the row max and row sum need
//    only in-lane reductions plus one exchange between the two lane halves.
//  * The same lane layout is exactly the B operand of O^T += V^T P^T (after
//    rounding P to bf16) provided the 16 keys of each MFMA k-step are taken in
//    the order the S^T accumulator hands them out. V is therefore written to
//    LDS transposed ([d][key]) with that key order, so each A-operand read of
//    V^T is one 16-byte LDS load. O^T lives in registers with the query row on
//    the lane, so the per-row rescale by alpha is in-lane as well.
//  * K and V tiles of BN keys go global -> registers -> LDS; the next tile's
//    global loads are issued before the current tile's MFMAs so their latency
//    hides behind compute.
//  * Rows of P are summed after rounding to bf16, so numerator and
//    denominator use the same weights.
//  * Work-groups are numbered so that each XCD receives whole (b, KV head)
//    groups (its L2 then holds those K/V), and within a group the heaviest
//    causal query tiles start first.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float bf16lo(unsigned x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16hi(unsigned x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

// Value held by the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32); }

template <int D, int QB, int NW, int BN>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * QB * 32;
  static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;            // 32-key blocks per tile
  static constexpr int PS = BN / 16;            // 16-key k-steps of O^T += V^T P^T
  static constexpr int DB = D / 32;             // 32-row blocks of O^T
  static constexpr int K_STRIDE = D * 2 + 16;   // bytes per key row of K in LDS
  static constexpr int V_STRIDE = BN * 2 + 16;  // bytes per dim row of V^T in LDS
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  // Staging: a chunk is KPC consecutive keys x 8 dims; one thread moves CPT chunks.
  static constexpr int KPC = ((BN / 4) * (D / 8) >= NT) ? 4 : 2;
  static constexpr int CHUNKS = (BN / KPC) * (D / 8);
  static constexpr int CPT = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0 && CPT >= 1, "tile does not split evenly over threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "bad tile");
};

// Position of tile-local key kt inside the V^T rows: within every 16-key group
// the 4-key quads are stored in the order 0, 2, 1, 3, which is the order in
// which the S^T accumulator hands keys to the P operand (lane half 0 holds keys
// 0-3 and 8-11 of the group, lane half 1 holds keys 4-7 and 12-15).
__device__ __forceinline__ int vt_pos(int kt) {
  const int quad = (kt >> 2) & 3;
  const int pq = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
  return (kt & ~15) | (pq << 2) | (kt & 3);
}

template <int D, int QB, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(PrefillParams p, int n_qtiles) {
  using C = Cfg<D, QB, NW, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::K_BYTES + C::V_BYTES];
  unsigned char* const k_lds = lds;
  unsigned char* const vt_lds = lds + C::K_BYTES;

  // ---- work decomposition --------------------------------------------------
  const int g = p.Hq / p.Hkv;
  const int total = p.B * p.Hq * n_qtiles;
  const int bid = blockIdx.x;
  // Hardware hands consecutive work-group ids to the 8 XCDs round-robin;
  // renumber so that each XCD gets one contiguous range of work items.
  int w;
  {
    const int xcd = bid & 7, slot = bid >> 3;
    const int q8 = total >> 3, r8 = total & 7;
    w = xcd * q8 + min(xcd, r8) + slot;
  }
  const int per_pair = n_qtiles * g;
  const int pair = w / per_pair;            // (b, kv head)
  const int rem = w - pair * per_pair;
  const int qtile = n_qtiles - 1 - rem / g; // heaviest causal tiles first
  const int hg = rem - (rem / g) * g;
  const int b = pair / p.Hkv;
  const int kvh = pair - b * p.Hkv;
  const int h = kvh * g + hg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 31;   // query column of S^T / O^T held by this lane
  const int h2 = lane >> 5;  // lane half

  const int N = p.N;
  const int q_tile0 = qtile * C::BM;
  const int qw0 = q_tile0 + wave * QB * 32;  // first query row of this wave

  const __bf16* __restrict__ qg = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + b * p.k_sb + kvh * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + b * p.k_sb + kvh * p.k_sh;

  // ---- Q^T operand in registers ---------------------------------------------
  u32x4_t qreg[QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + qb * 32 + c;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      if (qi < N)
        qreg[qb][s] = *(const u32x4_t*)(qg + (long long)qi * p.q_sn + s * 16 + h2 * 8);
      else
        qreg[qb][s] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // ---- running state --------------------------------------------------------
  f32x16_t oacc[QB][C::DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qb][db][e] = 0.f;
  }

  const int q_last_wg = min(q_tile0 + C::BM, N) - 1;
  const int n_tiles = p.causal ? (q_last_wg / BN + 1) : ((N + BN - 1) / BN);

  // ---- global -> register staging of one K/V tile ----------------------------
  u32x4_t kst[C::CPT][C::KPC], vst[C::CPT][C::KPC];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      const int kgrp = ch / (D / 8), dch = ch - kgrp * (D / 8);
#pragma unroll
      for (int r = 0; r < C::KPC; ++r) {
        const int key = k0 + kgrp * C::KPC + r;
        if (key < N) {
          const long long off = (long long)key * p.k_sn + dch * 8;
          kst[i][r] = *(const u32x4_t*)(kg + off);
          vst[i][r] = *(const u32x4_t*)(vg + off);
        } else {
          kst[i][r] = u32x4_t{0u, 0u, 0u, 0u};
          vst[i][r] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      const int kgrp = ch / (D / 8), dch = ch - kgrp * (D / 8);
      const int kt0 = kgrp * C::KPC;
#pragma unroll
      for (int r = 0; r < C::KPC; ++r)
        *(u32x4_t*)(k_lds + (kt0 + r) * C::K_STRIDE + dch * 16) = kst[i][r];
      // transpose KPC keys x 8 dims into 8 rows of KPC keys
      const int pos = vt_pos(kt0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (C::KPC == 4) {
          u32x2_t lo, hi;
          lo[0] = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(vst[i][3][e], vst[i][2][e], 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(vst[i][3][e], vst[i][2][e], 0x07060302u);
          *(u32x2_t*)(vt_lds + (dch * 8 + 2 * e) * C::V_STRIDE + pos * 2) = lo;
          *(u32x2_t*)(vt_lds + (dch * 8 + 2 * e + 1) * C::V_STRIDE + pos * 2) = hi;
        } else {
          const unsigned lo = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x05040100u);
          const unsigned hi = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x07060302u);
          *(unsigned*)(vt_lds + (dch * 8 + 2 * e) * C::V_STRIDE + pos * 2) = lo;
          *(unsigned*)(vt_lds + (dch * 8 + 2 * e + 1) * C::V_STRIDE + pos * 2) = hi;
        }
      }
    }
  };

  load_tile(0);
  store_tile();
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = j * BN;
    if (j + 1 < n_tiles) load_tile(k0 + BN);

    const bool wave_active = (qw0 < N) && (!p.causal || k0 <= qw0 + QB * 32 - 1);
    if (wave_active) {
      // ---- S^T = K Q^T ---------------------------------------------------------
      f32x16_t sacc[QB][C::KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[qb][kb][e] = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          const u32x4_t a = *(const u32x4_t*)(k_lds + (kb * 32 + c) * C::K_STRIDE + s * 32 + h2 * 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = mfma_32x32x16(a, qreg[qb][s], sacc[qb][kb]);
        }
      }

      // ---- online softmax, one 32-row block at a time ----------------------------
      u32x4_t pop[QB][C::PS];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow0 = qw0 + qb * 32;
        const int qi = qrow0 + c;
        const bool need_mask = (p.causal && k0 + BN - 1 > qrow0) || (k0 + BN > N);
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float s = sacc[qb][kb][e] * p.scale_log2;
            if (need_mask) {
              const int key = k0 + kb * 32 + (e >> 2) * 8 + h2 * 4 + (e & 3);
              if (key >= N || (p.causal && key > qi)) s = kNegInf;
            }
            sacc[qb][kb][e] = s;
            mx = fmaxf(mx, s);
          }
        mx = fmaxf(mx, other_half(mx));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
        m_run[qb] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int ps = 0; ps < C::PS; ++ps) {
          const int kb = ps >> 1, e0 = (ps & 1) * 8;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_amdgcn_exp2f(sacc[qb][kb][e0 + 2 * t] - m_use);
            const float p1 = __builtin_amdgcn_exp2f(sacc[qb][kb][e0 + 2 * t + 1] - m_use);
            const unsigned pk = pack_bf16x2(p0, p1);
            pop[qb][ps][t] = pk;
            rs += bf16lo(pk) + bf16hi(pk);
          }
        }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[qb][db][e] *= alpha;
      }

      // ---- O^T += V^T P^T ----------------------------------------------------------
#pragma unroll
      for (int ps = 0; ps < C::PS; ++ps) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const u32x4_t a = *(const u32x4_t*)(vt_lds + (db * 32 + c) * C::V_STRIDE + (ps * 16 + h2 * 8) * 2);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            // a 32-row block entirely above the diagonal has p == 0: skip its MFMAs
            if (!p.causal || k0 <= qw0 + qb * 32 + 31)
              oacc[qb][db] = mfma_32x32x16(a, pop[qb][ps], oacc[qb][db]);
          }
        }
      }
    }

    __syncthreads();
    if (j + 1 < n_tiles) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- epilogue: O / l -> bf16 ---------------------------------------------------
  __bf16* __restrict__ og = (__bf16*)p.o + b * p.o_sb + h * p.o_sh;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + qb * 32 + c;
    const float l_tot = l_run[qb] + other_half(l_run[qb]);
    if (qi < N) {
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          u32x2_t pk;
          pk[0] = pack_bf16x2(oacc[qb][db][vq * 4 + 0] * inv, oacc[qb][db][vq * 4 + 1] * inv);
          pk[1] = pack_bf16x2(oacc[qb][db][vq * 4 + 2] * inv, oacc[qb][db][vq * 4 + 3] * inv);
          *(u32x2_t*)(og + (long long)qi * p.o_sn + db * 32 + vq * 8 + h2 * 4) = pk;
        }
      if (p.lse && h2 == 0)
        p.lse[((long long)b * p.Hq + h) * N + qi] = (m_run[qb] + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int D, int QB, int NW, int BN>
hipError_t launch_cfg(const PrefillParams& p, hipStream_t stream) {
  using C = Cfg<D, QB, NW, BN>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long total = (long long)p.B * p.Hq * n_qtiles;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, QB, NW, BN>), dim3((unsigned)total), dim3(C::NT), 0,
                     stream, p, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 128) return launch_cfg<128, 2, 4, 64>(p, stream);
  if (d == 64) return launch_cfg<64, 2, 4, 64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
