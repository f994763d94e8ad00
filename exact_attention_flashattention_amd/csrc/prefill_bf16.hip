// Causal GQA prefill, bf16 inputs, fp32 accumulation, MFMA 32x32x16 on gfx950.
//
// What is computed (per batch b, query head h, query row i):
//   o_i = sum_j softmax_j(scale * q_i . k_j + M_ij) v_j,  kv head = floor(h / g)
// which is the SDPA definition of "Module 5. Modern Attention Mechanisms",
// section 4, with the GQA head rule of its section 6. The work is organised as
// in the "FlashAttention" section of the "inference-attention" page: key/value
// tiles are streamed through on-chip memory, each query row carries a running
// max m, a running sum l and an unnormalised output O that is rescaled by
// 2^(m - m') when the max moves, and the output is O / l after the last tile.
// Tiles entirely above the causal diagonal are never visited.
//
// Mapping onto CDNA4:
//  * A work-group of NW waves owns BM = NW * 32 consecutive query rows of one
//    (b, h); each wave owns one block of 32 rows. Two waves share a SIMD.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims read from LDS, B = Q^T
//    held in registers for the whole kernel). In the MFMA result layout lane l
//    then holds 16 keys of query row l % 32, so the row max and row sum are
//    in-lane reductions plus one v_permlane32_swap between the lane halves.
//  * The same lane layout is exactly the B operand of O^T += V^T P^T (after
//    rounding P to bf16) provided the 16 keys of each MFMA k-step are taken in
//    the order the S^T accumulator hands them out. V is therefore written to
//    LDS transposed ([d][key]) in that order, so each A-operand read of V^T is
//    one 16-byte LDS load. The 16-byte granules of a V^T row are XOR-swizzled
//    by row so that neither the transposing writes nor the operand reads
//    collide on LDS banks.
//  * Software pipeline: while tile j's scores are exponentiated and multiplied
//    into V (vector ALU + MFMA), the MFMAs of tile j+1's scores are already in
//    flight, all in one basic block, so the matrix cores and the vector ALU
//    work at the same time. Three LDS buffers rotate: tile j (V read), tile
//    j+1 (K read) and tile j+2 (being written from registers loaded earlier in
//    the same iteration); one barrier per tile.
//  * The reference point m used in 2^(s - m) is only moved when a row's max
//    exceeds it by more than 2^8 (then O and l are rescaled exactly); between
//    moves the weights are bounded by 2^8, which bf16 and fp32 represent with
//    the same relative precision. Results are identical in exact arithmetic;
//    the decision for tile j+1 is taken after tile j's P.V, outside the
//    pipelined block, so the accumulators are untouched on most tiles.
//  * Row sums of P are taken from the bf16-rounded weights (dot2 against
//    ones), so numerator and denominator use the same weights.
//  * Work-groups are numbered so that each XCD receives whole (b, KV head)
//    groups (its L2 then holds those K/V), and within a group the heaviest
//    causal query tiles start first.
//  * Inputs must be finite: rows past the end of the sequence are zero-filled
//    in LDS and masked, but a NaN in a visible key or value propagates, as it
//    does in the definition.
#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
// Lazy-rescale threshold in base-2 exponent units: the running reference is
// moved only when a row max exceeds it by more than this.
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

// lo + hi + acc for a packed pair of bf16 values (exact products with 1.0)
__device__ __forceinline__ float add_bf16x2(unsigned pk, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

// Reductions across the two lane halves (lane l with lane l ^ 32):
// v_permlane32_swap(x, x) returns (x of lanes 0-31 in both halves,
// x of lanes 32-63 in both halves).
__device__ __forceinline__ float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int D, int NW, int BN>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;            // 32-key blocks per tile
  static constexpr int PS = BN / 16;            // 16-key k-steps of O^T += V^T P^T
  static constexpr int DB = D / 32;             // 32-row blocks of O^T
  static constexpr int K_STRIDE = D * 2 + 16;   // bytes per key row of K in LDS
  static constexpr int V_STRIDE = BN * 2;       // bytes per dim row of V^T in LDS
  static constexpr int GR = BN / 8;             // 16-byte granules per V^T row
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  static constexpr int STAGE = K_BYTES + V_BYTES;  // one LDS buffer
  static constexpr int NBUF = 3;
  // Staging: a chunk is KPC consecutive keys x 8 dims; one thread moves up to
  // CPT chunks (when there are fewer chunks than threads, the surplus waves
  // stage nothing).
  static constexpr int KPC = ((BN / 4) * (D / 8) >= NT) ? 4 : 2;
  static constexpr int CHUNKS = (BN / KPC) * (D / 8);
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;
  static_assert(CHUNKS % NT == 0 || (NT % CHUNKS == 0 && CHUNKS % 64 == 0), "uneven staging");
  static_assert(BN % 32 == 0 && D % 32 == 0 && GR >= 4, "bad tile");
};

// Position of tile-local key kt inside a V^T row: within every 16-key group
// the 4-key quads are stored in the order 0, 2, 1, 3, which is the order in
// which the S^T accumulator hands keys to the P operand (lane half 0 holds keys
// 0-3 and 8-11 of the group, lane half 1 holds keys 4-7 and 12-15).
__device__ __forceinline__ int vt_pos(int kt) {
  const int quad = (kt >> 2) & 3;
  const int pq = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
  return (kt & ~15) | (pq << 2) | (kt & 3);
}

// Byte offset of (row r, key position pos) in the swizzled V^T buffer.
template <int GR, int V_STRIDE>
__device__ __forceinline__ int vt_off(int r, int pos) {
  const int swz = ((r & 7) ^ ((r >> 3) & 7)) & (GR - 1);
  return r * V_STRIDE + ((((pos >> 3) ^ swz)) << 4) + (pos & 7) * 2;
}

template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(PrefillParams p, int n_qtiles) {
  using C = Cfg<D, NW, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::NBUF * C::STAGE];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int c = lane & 31;   // query column of S^T / O^T held by this lane
  const int h2 = lane >> 5;  // lane half

  const int N = p.N;
  const int q_tile0 = qtile * C::BM;
  const int qw0 = q_tile0 + wave * 32;  // first query row of this wave
  const int qi = qw0 + c;               // this lane's query row

  const __bf16* __restrict__ qg = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + b * p.k_sb + kvh * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + b * p.k_sb + kvh * p.k_sh;

  // Scores are carried as raw q.k; c2 = scale * log2(e) > 0 is applied inside
  // the exponent. A negative scale is folded into Q by flipping its sign bits
  // (exact); a zero scale becomes a tiny positive one (every weight is then
  // 2^0 = 1 to fp32 precision, as for scale 0).
  float c2 = p.scale_log2;
  const unsigned qflip = c2 < 0.f ? 0x80008000u : 0u;
  c2 = fabsf(c2);
  if (c2 == 0.f) c2 = 1e-30f;

  // ---- Q^T operand in registers ---------------------------------------------
  u32x4_t qreg[C::KS];
  {
    const int qc = min(qi, N - 1);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qreg[s] = *(const u32x4_t*)(qg + (long long)qc * p.q_sn + s * 16 + h2 * 8) ^ qflip;
  }

  // ---- running state --------------------------------------------------------
  f32x16_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_ref = kNegInf, l_run = 0.f;

  const int q_last_wg = min(q_tile0 + C::BM, N) - 1;
  const int n_tiles = p.causal ? (q_last_wg / BN + 1) : ((N + BN - 1) / BN);
  // tiles 0 .. wave_tiles-1 hold keys visible to some row of this wave
  const int wave_tiles = (qw0 >= N) ? 0 : (p.causal ? min(n_tiles, (qw0 + 31) / BN + 1) : n_tiles);

  // ---- global -> register staging of one K/V tile ----------------------------
  u32x4_t kst[C::CPT][C::KPC], vst[C::CPT][C::KPC];
  // this thread's chunk offsets within a tile (element units), computed once
  long long st_off[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int ch = tid + i * C::NT;
    const int kgrp = ch / (D / 8), dch = ch - kgrp * (D / 8);
    st_off[i] = (long long)(kgrp * C::KPC) * p.k_sn + dch * 8;
  }
  auto load_tile = [&](int k0) {
    const long long tile_off = (long long)k0 * p.k_sn;  // scalar
    const bool tail = k0 + BN > N;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      if (C::CHUNKS < C::NT && ch >= C::CHUNKS) break;  // whole waves idle here
      if (!tail) {
        const __bf16* kp = kg + tile_off + st_off[i];
        const __bf16* vp = vg + tile_off + st_off[i];
#pragma unroll
        for (int r = 0; r < C::KPC; ++r) {
          kst[i][r] = *(const u32x4_t*)(kp + r * p.k_sn);
          vst[i][r] = *(const u32x4_t*)(vp + r * p.k_sn);
        }
      } else {
        const int kgrp = ch / (D / 8), dch = ch - kgrp * (D / 8);
#pragma unroll
        for (int r = 0; r < C::KPC; ++r) {
          // rows past the end are clamped here and zero-filled by store_tile
          const int key = min(k0 + kgrp * C::KPC + r, N - 1);
          const long long off = (long long)key * p.k_sn + dch * 8;
          kst[i][r] = *(const u32x4_t*)(kg + off);
          vst[i][r] = *(const u32x4_t*)(vg + off);
        }
      }
    }
  };
  auto buf_of = [&](int t) { return lds + (t % C::NBUF) * C::STAGE; };
  auto store_tile = [&](int t) {
    const int k0 = t * BN;
    unsigned char* const k_lds = buf_of(t);
    unsigned char* const vt_lds = k_lds + C::K_BYTES;
    const bool tail = k0 + BN > N;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + i * C::NT;
      if (C::CHUNKS < C::NT && ch >= C::CHUNKS) break;
      const int kgrp = ch / (D / 8), dch = ch - kgrp * (D / 8);
      const int kt0 = kgrp * C::KPC;
      if (tail) {
#pragma unroll
        for (int r = 0; r < C::KPC; ++r) {
          const bool dead = k0 + kt0 + r >= N;
          kst[i][r] = dead ? u32x4_t{0u, 0u, 0u, 0u} : kst[i][r];
          vst[i][r] = dead ? u32x4_t{0u, 0u, 0u, 0u} : vst[i][r];
        }
      }
#pragma unroll
      for (int r = 0; r < C::KPC; ++r)
        *(u32x4_t*)(k_lds + (kt0 + r) * C::K_STRIDE + dch * 16) = kst[i][r];
      // transpose KPC keys x 8 dims into 8 rows of KPC keys
      const int pos = vt_pos(kt0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r0 = dch * 8 + 2 * e;
        if constexpr (C::KPC == 4) {
          u32x2_t lo, hi;
          lo[0] = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x05040100u);
          lo[1] = __builtin_amdgcn_perm(vst[i][3][e], vst[i][2][e], 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x07060302u);
          hi[1] = __builtin_amdgcn_perm(vst[i][3][e], vst[i][2][e], 0x07060302u);
          *(u32x2_t*)(vt_lds + vt_off<C::GR, C::V_STRIDE>(r0, pos)) = lo;
          *(u32x2_t*)(vt_lds + vt_off<C::GR, C::V_STRIDE>(r0 + 1, pos)) = hi;
        } else {
          const unsigned lo = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x05040100u);
          const unsigned hi = __builtin_amdgcn_perm(vst[i][1][e], vst[i][0][e], 0x07060302u);
          *(unsigned*)(vt_lds + vt_off<C::GR, C::V_STRIDE>(r0, pos)) = lo;
          *(unsigned*)(vt_lds + vt_off<C::GR, C::V_STRIDE>(r0 + 1, pos)) = hi;
        }
      }
    }
  };

  // ---- the three steps of a tile ----------------------------------------------
  // S^T = K Q^T for tile t
  auto qk = [&](int t, f32x16_t (&s)[C::KB]) {
    const unsigned char* k_lds = buf_of(t);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const u32x4_t a = *(const u32x4_t*)(k_lds + (kb * 32 + c) * C::K_STRIDE + s_ * 32 + h2 * 16);
        s[kb] = mfma_32x32x16(a, qreg[s_], s[kb]);
      }
  };
  // mask tile t where it reaches past the diagonal or the end, then move the
  // reference max if this tile's max exceeds it by more than the threshold
  auto prep = [&](int t, f32x16_t (&s)[C::KB]) {
    const int k0 = t * BN;
    if ((p.causal && k0 + BN - 1 > qw0) || (k0 + BN > N)) {
      // key k0 + h2*4 + off (off a compile-time constant per element) is visible
      // iff off <= lim
      const int lim = (p.causal ? min(qi, N - 1) : N - 1) - k0 - h2 * 4;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kb * 32 + (e >> 2) * 8 + (e & 3);
          s[kb][e] = (off > lim) ? kNegInf : s[kb][e];
        }
    }
    float mr = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mr = fmaxf(mr, s[kb][e]);
    mr = halves_max(mr);
    const float mt = (mr == kNegInf) ? kNegInf : mr * c2;
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kRescaleTau)) {
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
  };
  // P = 2^(s - m) rounded to bf16, l += rowsum(P), O^T += V^T P^T for tile t
  auto pv = [&](int t, const f32x16_t (&s)[C::KB]) {
    const unsigned char* vt_lds = buf_of(t) + C::K_BYTES;
    const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
    u32x4_t pop[C::PS];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps) {
      const int kb = ps >> 1, e0 = (ps & 1) * 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][e0 + 2 * u], c2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][e0 + 2 * u + 1], c2, neg_m));
        const unsigned pk = pack_bf16x2(p0, p1);
        pop[ps][u] = pk;
        if (u & 1)
          rs1 = add_bf16x2(pk, rs1);
        else
          rs0 = add_bf16x2(pk, rs0);
      }
    }
    l_run += rs0 + rs1;
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x4_t a = *(const u32x4_t*)(vt_lds + vt_off<C::GR, C::V_STRIDE>(db * 32 + c, ps * 16 + h2 * 8));
        oacc[db] = mfma_32x32x16(a, pop[ps], oacc[db]);
      }
  };

  // ---- prologue: tiles 0 and 1 staged, scores of tile 0 --------------------------
  f32x16_t sa[C::KB], sb[C::KB];
  load_tile(0);
  store_tile(0);
  if (n_tiles > 1) {
    load_tile(BN);
    store_tile(1);
  }
  __syncthreads();
  if (wave_tiles > 0) {
    qk(0, sa);
    prep(0, sa);
  }

  // ---- main loop: iteration j consumes tile j and computes the scores of j+1 -------
  // Every wave runs n_tiles iterations (one barrier each); the loops only
  // differ in how much of the tile work the wave still has.
  auto staging = [&](int j) {
    if (j + 2 < n_tiles) load_tile((j + 2) * BN);
  };
  auto staging_store = [&](int j) {
    if (j + 2 < n_tiles) store_tile(j + 2);
  };
  int j = 0;
  for (; j + 1 < wave_tiles; ++j) {  // tiles j and j+1 both have work for this wave
    staging(j);
    qk(j + 1, sb);  // in flight while tile j is exponentiated
    pv(j, sa);
    staging_store(j);
    prep(j + 1, sb);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) sa[kb] = sb[kb];
    __syncthreads();
  }
  if (j < wave_tiles) {  // the wave's last tile
    staging(j);
    pv(j, sa);
    staging_store(j);
    __syncthreads();
    ++j;
  }
  for (; j < n_tiles; ++j) {  // no work left for this wave: keep staging tiles for the others
    staging(j);
    staging_store(j);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16 ---------------------------------------------------
  __bf16* __restrict__ og = (__bf16*)p.o + b * p.o_sb + h * p.o_sh;
  const float l_tot = halves_sum(l_run);
  if (qi < N) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        u32x2_t pk;
        pk[0] = pack_bf16x2(oacc[db][vq * 4 + 0] * inv, oacc[db][vq * 4 + 1] * inv);
        pk[1] = pack_bf16x2(oacc[db][vq * 4 + 2] * inv, oacc[db][vq * 4 + 3] * inv);
        *(u32x2_t*)(og + (long long)qi * p.o_sn + db * 32 + vq * 8 + h2 * 4) = pk;
      }
    // m_ref is in units of scale * log2(e) * q.k (the sign fold leaves that product unchanged)
    if (p.lse && h2 == 0)
      p.lse[((long long)b * p.Hq + h) * N + qi] = (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int NW, int BN>
hipError_t launch_cfg(const PrefillParams& p, hipStream_t stream) {
  using C = Cfg<D, NW, BN>;
  const int n_qtiles = (p.N + C::BM - 1) / C::BM;
  const long long total = (long long)p.B * p.Hq * n_qtiles;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BN>), dim3((unsigned)total), dim3(C::NT), 0,
                     stream, p, n_qtiles);
  return hipGetLastError();
}

}  // namespace

// Tile shapes (waves per work-group, keys per tile).
#ifndef ATTN_PREFILL_D128
#define ATTN_PREFILL_D128 8, 64
#endif
#ifndef ATTN_PREFILL_D64
#define ATTN_PREFILL_D64 8, 32
#endif

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  if (d == 128) return launch_cfg<128, ATTN_PREFILL_D128>(p, stream);
  if (d == 64) return launch_cfg<64, ATTN_PREFILL_D64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
