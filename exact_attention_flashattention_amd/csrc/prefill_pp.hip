// Causal GQA prefill, bf16 inputs, fp32 accumulation: the two-group
// ("ping-pong") form of the FlashAttention loop for gfx950.
//
// What is computed (per batch b, query head h, query row i):
//   o_i = sum_j softmax_j(scale * q_i . k_j + M_ij) v_j,  kv head = floor(h / g)
// the SDPA definition of "Module 5. Modern Attention Mechanisms", section 4,
// with the GQA head rule of its section 6, computed as in the "FlashAttention"
// section of the "inference-attention" page: key/value tiles stream through
// on-chip memory, each query row carries a running max m, a running sum l and
// an unnormalised output O rescaled by 2^(m - m') when the max moves, and the
// output is O / l after the last tile. Tiles with no visible key are skipped.
// The same page credits the third FlashAttention generation with overlapping
// the matrix products and the softmax; this kernel does that with two groups
// of waves that take turns on each SIMD.
//
// Mapping onto CDNA4:
//  * A work-group is 8 waves, 256 query rows of one (b, h), 32 rows per wave.
//    Waves 0-3 form group 0 and waves 4-7 group 1; the hardware places waves
//    w and w + 4 on the same SIMD, so each SIMD runs one wave of each group.
//  * Each key tile ("slot") is processed in two phases separated by
//    work-group barriers, the groups one phase apart. In its matrix phase a
//    wave issues only MFMAs: the scores of slot j+1 and the P V product of
//    slot j (16 MFMAs at d = 128). In its vector phase it runs the whole
//    softmax of slot j+1 (mask, row max, exponentials, rounding, row sums),
//    loads the next operands from LDS into registers and issues the
//    HBM -> LDS copies. Measured on this part: a wave's own v_exp_f32 stalls
//    its MFMA stream (about 4 cycles each), while the other wave's vector
//    work does not slow the MFMAs at all, so the matrix pipe of a SIMD stays
//    busy with one wave while its partner does the softmax.
//  * Per wave and slot: S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = 32 keys x
//    16 dims, B = Q^T held in registers for the whole kernel), so lane l holds
//    16 keys of query row l % 32 and the row max and sum are in-lane plus one
//    v_permlane32_swap; O^T += V^T P^T with the same MFMA, P^T being the
//    bf16-rounded scores in the accumulator's own lane layout (each 16-key
//    k-step takes the keys in that order), V^T read from LDS with
//    ds_read_b64_tr_b16 (four consecutive keys of one dimension per lane).
//  * K and V tiles go HBM -> LDS with global_load_lds_dwordx4 into rings of
//    R buffers each (R = 6 by default), every 16-byte chunk at a row-swizzled
//    position so the K operand reads and the transposed V reads are free of
//    bank conflicts. V copies run R-1 slots ahead and K copies R; each wave
//    waits for its own copies with an explicit vmcnt count before each
//    barrier (__syncthreads() would wait for every copy in flight).
//  * The reference point m of 2^(s - m) moves only when a row's max exceeds it
//    by more than 2^8 (then O and l are rescaled exactly), so the accumulators
//    are untouched on most slots; the weights stay below 2^8.
//  * Row sums of P are taken from the bf16-rounded weights (dot2 against
//    ones), so numerator and denominator use the same weights.
//  * Work-groups are numbered so that each XCD receives whole (b, KV head)
//    pairs (its L2 then holds their K/V) and the heaviest causal query tiles
//    start first.
//  * Inputs must be finite: key rows past the end of a sequence are loaded
//    from its last row and masked, so their weight is exactly 0.
#include "attn_internal.h"
#include "cdna4.h"

namespace attn {
namespace {

using namespace cdna4;

#ifndef ATTN_PP_RING
#define ATTN_PP_RING 6
#endif
constexpr int kPage = 16;           // tokens per page of a paged KV cache
constexpr float kRescaleTau = 8.0f; // lazy-rescale threshold, base-2 exponent units

template <int D>
struct PP {
  static constexpr int NW = 8;                   // waves per work-group
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;             // query rows per work-group
  static constexpr int BN = D == 128 ? 32 : 64;  // keys per tile
  static constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;             // 32-key blocks of S^T
  static constexpr int PS = BN / 16;             // 16-key k-steps of O^T += V^T P^T
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  static constexpr int NOP = KS * KB;            // operands per product per tile
  static constexpr int ROWB = D * 2;             // bytes per key row
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;           // rows per 1 KiB copy instruction
  static constexpr int TILE = BN * ROWB;         // bytes of one K (or V) tile
  static constexpr int RING = ATTN_PP_RING;      // buffers per ring
  static constexpr int VMW = 2 * (RING - 3);     // copies a wave may leave in flight at a barrier
  static constexpr int VBASE = RING * TILE;      // V ring after the K ring
  static constexpr int OROW = D * 2 + 16;        // padded bytes per staged output row
  static constexpr int LDS_BYTES = (2 * VBASE > NW * 32 * OROW) ? 2 * VBASE : NW * 32 * OROW;
  static_assert(NOP == DB * PS, "the K and the V^T operands of a tile are equally many");
  static_assert(TILE == NW * 1024, "one copy instruction per wave per tensor per tile");
};

template <int D, bool PAGED>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillParams p, int n_qtiles) {
  using C = PP<D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];

  // ---- work decomposition (as for every prefill launch) -----------------------
  const int g = p.Hq / p.Hkv;
  const int total = p.B * p.Hq * n_qtiles;
  const int w = xcd_remap(blockIdx.x, total);
  const int per_pair = n_qtiles * g;
  // (kv head, b) pairs with b fastest, heaviest query tiles first; pairs with
  // fewer work items than an XCD has CUs are grouped so that their query
  // tiles run heaviest-first across the whole group
  constexpr int kCusPerXcd = 32;
  const int n_pairs = p.B * p.Hkv;
  const int G = per_pair >= kCusPerXcd ? 1 : max(1, min(n_pairs, (total >> 3) / per_pair));
  const int grp_id = w / (G * per_pair);
  const int r_in = w - grp_id * G * per_pair;
  const int row_items = min(G, n_pairs - grp_id * G) * g;
  const int qrank = r_in / row_items;
  const int rest = r_in - qrank * row_items;
  const int pair = grp_id * G + rest / g;
  const int qtile = n_qtiles - 1 - qrank;
  const int hg = rest - (rest / g) * g;
  const int kvh = pair / p.B;
  const int b = pair - kvh * p.B;
  const int h = kvh * g + hg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  const int c = lane & 31;      // query column of S^T / O^T held by this lane
  const int h2 = lane >> 5;     // lane half

  const int q_tile0 = qtile * C::BM;
  int Nq, Nk, P;
  const __bf16* qg;
  __bf16* og;
  long long lse_row0;
  if constexpr (PAGED) {
    const int r0 = p.cu_q[b];
    Nq = p.cu_q[b + 1] - r0;
    Nk = p.seq_lens[b];
    P = max(Nk - Nq, 0);
    qg = (const __bf16*)p.q + (long long)r0 * p.q_sn + h * p.q_sh;
    og = (__bf16*)p.o + (long long)r0 * p.o_sn + h * p.o_sh;
    lse_row0 = (long long)h * p.total_q + r0;
  } else {
    Nq = Nk = p.N;
    P = 0;
    qg = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
    og = (__bf16*)p.o + b * p.o_sb + h * p.o_sh;
    lse_row0 = ((long long)b * p.Hq + h) * p.N;
  }
  if (q_tile0 >= Nq) return;  // the whole work-group: a chunk shorter than the launch
  // Query block of this wave: SIMD s holds blocks 2s (group 0) and 2s + 1
  // (group 1), so the two groups' causal limits differ by one block and both
  // have work until the last tiles.
  const int qblk = 2 * (wave & 3) + group;
  const int qw0 = q_tile0 + qblk * 32;
  const int qi = qw0 + c;

  const __bf16* __restrict__ kg = (const __bf16*)p.k + (PAGED ? 0 : b * p.k_sb) + kvh * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + (PAGED ? 0 : b * p.k_sb) + kvh * p.k_sh;

  // scores are raw q.k; c2 = scale * log2(e) > 0 is applied in the exponent,
  // a negative scale is folded into Q's sign bits (exact)
  float c2 = p.scale_log2;
  const unsigned qflip = c2 < 0.f ? 0x80008000u : 0u;
  c2 = fabsf(c2);
  if (c2 == 0.f) c2 = 1e-30f;

  u32x4_t qreg[C::KS];
  {
    const int qc = min(qi, Nq - 1);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qreg[s] = *(const u32x4_t*)(qg + (long long)qc * p.q_sn + s * 16 + h2 * 8) ^ qflip;
  }

  f32x16_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  // a learned sink logit s_h enters as the initial state m = s_h, l = 1, O = 0
  // m_ref starts at the most negative finite float ("no key yet"): a row
  // max of -inf (every key masked) never moves it and s*c2 - m_ref stays
  // -inf for masked scores, so no -inf guards are needed; the first finite
  // row max always moves it (then the rescale factor is exactly 0).
  float m_ref = -3.402823466e38f, l_run = 0.f;
  if (p.sinks) {
    m_ref = p.sinks[h] * 1.4426950408889634f;
    l_run = h2 == 0 ? 1.f : 0.f;  // the two lane halves' sums are added at the end
  }

  // ---- the key tiles of this work-group ("slots") ------------------------------
  // Sink tiles first, then the tiles of the window (or all causal tiles).
  const int q_last_wg = min(q_tile0 + C::BM, Nq) - 1;
  const int k_tiles = (Nk + BN - 1) / BN;
  const int n_tiles = p.causal ? min(k_tiles, (P + q_last_wg) / BN + 1) : k_tiles;
  const int W = p.window;
  const int sink_tiles = (W > 0 && p.n_sink > 0) ? min((p.n_sink + BN - 1) / BN, n_tiles) : 0;
  const int win_lo = W > 0 ? max(max(P + q_tile0 - W + 1, 0) / BN, sink_tiles) : 0;
  const int n_slots = sink_tiles + max(n_tiles - win_lo, 0);
  auto tile_of = [&](int j) __attribute__((always_inline)) { return j < sink_tiles ? j : win_lo + (j - sink_tiles); };
  auto slot_of = [&](int t) __attribute__((always_inline)) { return t < sink_tiles ? t : t - win_lo + sink_tiles; };
  // The slots this wave's group computes, [gf, ge): the union of the slots
  // holding keys visible to some row of its four query blocks (a gap between
  // sink slots and a later window is computed too, fully masked). Every wave
  // of the group computes every slot of the range; where none of its own
  // keys is visible the mask makes every weight exactly 0.
  int gf = n_slots, ge = 0;
#pragma unroll
  for (int s_ = 0; s_ < 4; ++s_) {
    const int qb0 = q_tile0 + (2 * s_ + group) * 32;
    if (qb0 >= Nq) continue;
    const int last = (p.causal ? min(n_tiles, (P + qb0 + 31) / BN + 1) : n_tiles) - 1;
    ge = max(ge, slot_of(last) + 1);
    int first = 0;
    if (W > 0 && sink_tiles == 0) first = slot_of(max(P + qb0 - W + 1, 0) / BN);
    gf = min(gf, first);
  }
  if (ge <= gf) gf = ge = 0;  // no row of this group has a visible key

  // ---- HBM -> LDS copies: one 1 KiB instruction per wave per tensor per tile ----
  const unsigned row_bytes = (unsigned)p.k_sn * 2u;
  const int ld_row = wave * C::RPI + lane / C::CPR;      // tile row of this lane's 16 bytes
  const int ld_chunk = (lane % C::CPR) ^ swz<C::CPR>(ld_row);
  const __attribute__((address_space(4))) int32_t* const table =
      PAGED ? (const __attribute__((address_space(4))) int32_t*)(p.block_table + (long long)b * p.max_pages_per_seq)
            : nullptr;
  const long long page_bytes = (long long)row_bytes * kPage;
  // Copies are issued for every slot index the schedule names, clamped to
  // the last slot: the copies past the end duplicate it into ring buffers
  // nobody reads, and every wave's count of copies in flight stays the same
  // on every slot (no tail cases in the waits).
  auto copy_tile = [&](const __bf16* __restrict__ base, int t, unsigned char* dst) __attribute__((always_inline)) {
    const int k0 = tile_of(min(t, n_slots - 1)) * BN;
    // rows past the end of the sequence repeat its last row (masked later)
    const int key = min(k0 + ld_row, Nk - 1);
    const char* src;
    unsigned off;
    if constexpr (PAGED) {
      src = (const char*)base + table[min(k0 + wave * C::RPI, Nk - 1) / kPage] * page_bytes;
      off = (unsigned)(key & (kPage - 1)) * row_bytes + (unsigned)ld_chunk * 16u;
    } else {
      src = (const char*)base + (long long)k0 * row_bytes;
      off = (unsigned)(key - k0) * row_bytes + (unsigned)ld_chunk * 16u;
    }
    load_to_lds(src + off, dst + wave * 1024);
  };
  auto kbuf = [&](int r) __attribute__((always_inline)) { return lds + (r % C::RING) * C::TILE; };
  auto vbuf = [&](int r) __attribute__((always_inline)) { return lds + C::VBASE + (r % C::RING) * C::TILE; };
  auto vrel = [&](int r) __attribute__((always_inline)) { return lds + (r % C::RING) * C::TILE; };

  // ---- LDS -> register operands ---------------------------------------------------
  // K operand of k-step s, key block kb: row c + 32 kb, chunk (2s + h2) ^ swz.
  unsigned kpart[C::KS];
#pragma unroll
  for (int s_ = 0; s_ < C::KS; ++s_)
    kpart[s_] = (unsigned)(c * C::ROWB + (((2 * s_ + h2) ^ swz<C::CPR>(c)) * 16));
  // V^T operand: lane l = 16 G + 4 t + u reads V[key][d] with key = ps*16 +
  // 8 r + 4 h2 + t and d = db*32 + 16 (G & 1) + 4 u; the 16-lane transpose
  // then hands lane l the keys ps*16 + 8 r + 4 h2 + 0..3 of dimension
  // db*32 + l % 32, the key order of the S^T accumulator. The parts include
  // the V ring's base.
  unsigned vpart[2][C::DB];
  {
    const int tr_t = (lane >> 2) & 3, tr_u = lane & 3, tr_g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int key = 8 * r + 4 * h2 + tr_t;
        const int d = db * 32 + 16 * tr_g + 4 * tr_u;
        vpart[r][db] = (unsigned)(C::VBASE + key * C::ROWB + ((d >> 3) ^ swz<C::CPR>(key)) * 16 + ((d >> 2) & 1) * 8);
      }
  }
  // Launder the lane parts once per slot: otherwise the address of every
  // (ring position, read) pair of the unrolled loop is hoisted into a
  // register of its own, far more than the register file holds.
  auto refresh_parts = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_) asm volatile("" : "+v"(kpart[s_]));
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) asm volatile("" : "+v"(vpart[r][db]));
  };
  u32x4_t kreg[C::NOP];  // K operands of the slot whose scores come next
  u32x4_t vreg[C::NOP];  // V^T operands of the slot whose P V comes next
  auto read_k = [&](const unsigned char* __restrict__ kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int s_ = 0; s_ < C::KS; ++s_)
        kreg[kb * C::KS + s_] = *(const u32x4_t*)(kt + kpart[s_] + kb * 32 * C::ROWB);
  };
  // vt: the V tile's buffer minus the V ring's base, which the lane parts
  // carry, so that the ring position stays within the 16-bit offset field
  auto read_v = [&](const unsigned char* __restrict__ vt) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt + vpart[r][db] + ps * 16 * C::ROWB));
          const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
          a[2 * r] = xx[0];
          a[2 * r + 1] = xx[1];
        }
        vreg[ps * C::DB + db] = a;
      }
  };

  // one operand of each, for the hand-ordered matrix phase
  auto read_k_op = [&](const unsigned char* __restrict__ kt, int i) __attribute__((always_inline)) {
    const int kb = i / C::KS, s_ = i % C::KS;
    kreg[i] = *(const u32x4_t*)(kt + kpart[s_] + kb * 32 * C::ROWB);
  };
  auto read_v_op = [&](const unsigned char* __restrict__ vt, int i) __attribute__((always_inline)) {
    const int ps = i / C::DB, db = i % C::DB;
    u32x4_t a;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vt + vpart[r][db] + ps * 16 * C::ROWB));
      const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
      a[2 * r] = xx[0];
      a[2 * r + 1] = xx[1];
    }
    vreg[i] = a;
  };

  // ---- the steps of a tile -------------------------------------------------------
  // S^T = K Q^T from the K operands in kv
  auto gemm0 = [&](f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) s[kb] = mfma_32x32x16(kreg[kb * C::KS + s_], qreg[s_], s[kb]);
  };
  // O^T += V^T P^T from the V^T operands in kv
  auto gemm1 = [&](const u32x4_t (&pop)[C::PS]) __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = mfma_32x32x16(vreg[ps * C::DB + db], pop[ps], oacc[db]);
  };
  // key k0 + h2*4 + off (off a constant per element) is visible iff off <= lim
  // and, with a window, off >= lo or it is one of the n_sink initial positions
  // First slot whose tile reaches past the causal limit of the wave's first
  // row or past the end of the sequence (tiles are visited in increasing
  // order, so every later slot needs the mask too); window edges are tested
  // per slot.
  const int t_mask = min(p.causal ? (P + qw0 + 1) / BN : k_tiles, Nk / BN);
  const int mask_from = t_mask < sink_tiles ? t_mask : sink_tiles + max(t_mask - win_lo, 0);
  auto mask = [&](int t, f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    const int k0 = tile_of(t) * BN;
    if (t >= mask_from || (W > 0 && k0 < P + qw0 + 31 - W + 1 && k0 + BN > p.n_sink)) {
      const int base = k0 + h2 * 4;
      const int lim = (p.causal ? min(P + qi, Nk - 1) : Nk - 1) - base;
      const int lo = W > 0 ? P + qi - W + 1 - base : -BN;
      const int sk = p.n_sink - base;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = kb * 32 + (e >> 2) * 8 + (e & 3);
          s[kb][e] = (off > lim || (off < lo && off >= sk)) ? kNegInf : s[kb][e];
        }
    }
  };
  // row max, the lazy move of the reference m (per row), then s := s*c2 - m
  float m_old = m_ref;
  auto alu0 = [&](f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    float rm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) rm[e & 3] = fmaxf(rm[e & 3], s[kb][e]);
    const float mr = halves_max(fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3])));
    const float mt = mr * c2;  // c2 > 0: -inf stays -inf
    m_old = m_ref;
    m_ref = mt > m_ref + kRescaleTau ? mt : m_ref;
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = fmaf(s[kb][e], c2, neg_m);
  };
  // rescale O and l for the rows whose reference moved (rare); a move always
  // changes m_ref, so the test needs only the two references
  auto rescale = [&]() __attribute__((always_inline)) {
    const bool mv = m_ref != m_old;
    if (__builtin_amdgcn_ballot_w64(mv)) {
      const float alpha = mv ? __builtin_amdgcn_exp2f(m_old - m_ref) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
  };
  // P = 2^s rounded to bf16 in the B-operand order, l += rowsum(P)
  auto alu1 = [&](const f32x16_t (&s)[C::KB], u32x4_t (&pop)[C::PS]) __attribute__((always_inline)) {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps) {
      const int kb = ps >> 1, e0 = (ps & 1) * 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float p0 = __builtin_amdgcn_exp2f(s[kb][e0 + 2 * u]);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][e0 + 2 * u + 1]);
        const unsigned pk = pack_bf16x2(p0, p1);
        pop[ps][u] = pk;
        if (u & 1)
          rs1 = add_bf16x2(pk, rs1);
        else
          rs0 = add_bf16x2(pk, rs0);
      }
    }
    l_run += rs0 + rs1;
  };
  // The common case: no score of this lane's keys is more than 2^8 above the
  // reference (the lazy rule's test, taken on the lane's own 16 or 32 keys
  // and combined across the wave), so the reference stays and the row max
  // across the two lane halves is not needed; then s := s*c2 - m.
  auto keep_ref = [&](const f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    float rm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) rm[e & 3] = fmaxf(rm[e & 3], s[kb][e]);
    const float mx = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
    return !__builtin_amdgcn_ballot_w64(mx * c2 > m_ref + kRescaleTau);
  };
  // the lazy move of the reference from the row max (both lane halves)
  auto move_ref = [&](const f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    float rm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) rm[e & 3] = fmaxf(rm[e & 3], s[kb][e]);
    const float mt = halves_max(fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]))) * c2;
    m_ref = mt > m_ref + kRescaleTau ? mt : m_ref;
  };
  auto shift = [&](f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = fmaf(s[kb][e], c2, neg_m);
  };
  u32x4_t pop[C::PS];  // P of the current slot, bf16 pairs in B-operand order
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_nofence();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Pin a phase's results to the phase: without a use here the compiler
  // sinks pure arithmetic (exponentials, packing, the max and the FMAs)
  // across the barriers toward the first use, into the other group's phase.
  auto pin_scores = [&](f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) asm volatile("" : "+v"(s[kb]));
  };
  auto pin_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps) asm volatile("" : "+v"(pop[ps]));
    asm volatile("" : "+v"(l_run));
  };

  // ---- prologue --------------------------------------------------------------------
  // Copies of K_0..K_5 and V_0..V_4 in the order the slots need them (K_0,
  // K_1, V_0, then K_t, V_{t-1}); the wait covers only the first three (and
  // the Q loads before them): the softmax of slot 0 and the operands of slot
  // 0's P V and slot 1's scores. Each later matrix phase finds the tiles it
  // reads complete under the loop's own vmcnt rule.
  f32x16_t sc[C::KB];
  copy_tile(kg, 0, kbuf(0));
  copy_tile(kg, 1, kbuf(1));
  copy_tile(vg, 0, vbuf(0));
#pragma unroll
  for (int t = 2; t < C::RING; ++t) {
    copy_tile(kg, t, kbuf(t));
    copy_tile(vg, t - 1, vbuf(t - 1));
  }
  wait_vmcnt<2 * C::RING - 4>();
  bar();
  if (gf == 0 && ge > 0) {
    read_k(kbuf(0));
    gemm0(sc);
    mask(0, sc);
    alu0(sc);
    rescale();
    alu1(sc, pop);
  }
  read_k(kbuf(1));
  read_v(vrel(0));

  // ---- main loop -----------------------------------------------------------------
  // Every wave runs, for each slot j, a matrix phase M(j) and a vector phase
  // X(j), each opened by a work-group barrier; group 1 runs one phase behind
  // group 0 (it opens with an empty phase, group 0 closes with one), so the
  // matrix phase of one wave of a SIMD meets the vector phase of the other.
  //   M(j): S_{j+1} = K_{j+1} Q^T and O += V_j P_j; then the K_{j+2} and
  //         V_{j+1} operands from LDS and the copies V_{j+R-1}, K_{j+R}
  //   X(j): mask, row max, exponentials and row sums of slot j+1
  // A wave issues at most one instruction every few cycles, so the data
  // movement rides in the matrix phase (between MFMAs a wave is idle) and
  // the vector phase holds only the softmax.
  // Copies: R buffers per ring. Slot t's K and V are read in M(t-2) and
  // M(t-1); their buffers are rewritten only from M(t) and M(t+1) on, after
  // the barriers that follow the waits for those reads (each wave waits for
  // its LDS reads at the start of its next matrix phase). Before every
  // barrier each wave waits until at most 2(R-3) of its copies are in flight
  // (those of its last R-3 matrix phases), which completes the copies of slot
  // j+2's K and j+1's V (issued in M(j+2-R) by both groups) before the
  // barrier that opens M(j) of group 0.
  constexpr int IDLE = 0, LEADIN = 1, FULL = 2, LEADOUT = 3;
  auto iteration = [&](int j, int jr, int kind) __attribute__((always_inline)) {
    refresh_parts();
    // M(j): the products, then the operands of M(j+1) (each read after the
    // MFMAs that consume the registers it overwrites) and the copies
    wait_vmcnt<C::VMW>();
    bar();
    wait_lgkmcnt<0>();  // this wave's operands from M(j-1)
    // (the fences keep each operand read behind the MFMAs that consume the
    // registers it overwrites, so one register set per operand suffices)
    if (kind == FULL) {
      // Hand-ordered (each fence stops the scheduler from moving anything
      // across): every MFMA is followed by the LDS read of the next slot's
      // operand of the same index, into the registers the MFMA has just
      // consumed, so the reads overlap the MFMAs.
      const unsigned char* const kt = kbuf(jr + 2);
      const unsigned char* const vt = vrel(jr + 1);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
#pragma unroll
      for (int i = 0; i < C::NOP; ++i) {
        const int kb = i / C::KS, s_ = i % C::KS;
        sc[kb] = mfma_32x32x16(kreg[i], qreg[s_], sc[kb]);
        __builtin_amdgcn_sched_barrier(0);
        read_k_op(kt, i);
        if (i == 1) copy_tile(vg, j + C::RING - 1, vbuf(jr + C::RING - 1));  // the copies ride early, in MFMA shadows
        if (i == 2) copy_tile(kg, j + C::RING, kbuf(jr + C::RING));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < C::NOP; ++i) {
        const int ps = i / C::DB, db = i % C::DB;
        oacc[db] = mfma_32x32x16(vreg[i], pop[ps], oacc[db]);
        __builtin_amdgcn_sched_barrier(0);
        read_v_op(vt, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if (kind == LEADIN) gemm0(sc);
      __builtin_amdgcn_sched_barrier(0);
      read_k(kbuf(jr + 2));  // unused when slot j+2 is not computed
      __builtin_amdgcn_sched_barrier(0);
      if (kind == LEADOUT) gemm1(pop);
      __builtin_amdgcn_sched_barrier(0);
      read_v(vrel(jr + 1));
      copy_tile(vg, j + C::RING - 1, vbuf(jr + C::RING - 1));
      copy_tile(kg, j + C::RING, kbuf(jr + C::RING));
    }
    // X(j): the softmax of slot j+1
    wait_vmcnt<C::VMW>();
    bar();
    if (kind == FULL) {
      mask(j + 1, sc);
      m_old = m_ref;
      if (!keep_ref(sc)) move_ref(sc);
      shift(sc);
      rescale();
      alu1(sc, pop);
      pin_p();
    } else if (kind == LEADIN) {
      mask(j + 1, sc);
      alu0(sc);
      rescale();
      alu1(sc, pop);
      pin_p();
    }
  };
  auto step = [&](int j, int kind) __attribute__((always_inline)) { iteration(j, j % C::RING, kind); };

  if (group == 1) bar();
  int j = 0;
  for (; j + 1 < gf; ++j) step(j, IDLE);
  if (gf > 0 && gf < ge) step(j++, LEADIN);
  // j == gf here when the group has work: slots j and j+1 both computed
  for (; j % C::RING && j + 1 < ge; ++j) step(j, FULL);
  // R slots per trip: ring positions are compile-time constants
  for (; j + C::RING < ge; j += C::RING) {
#pragma unroll
    for (int u = 0; u < C::RING; ++u) iteration(j + u, u, FULL);
  }
  for (; j + 1 < ge; ++j) step(j, FULL);
  if (j < ge) step(j++, LEADOUT);
  for (; j < n_slots; ++j) step(j, IDLE);
  if (group == 0) bar();

  // ---- epilogue: O / l -> bf16, whole rows through LDS ------------------------------
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();
  bar();
  constexpr int OROW = C::OROW;
  unsigned char* const ost = lds + wave * 32 * OROW;
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;  // a row with no key gets zeros
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      u32x2_t pk;
      pk[0] = pack_bf16x2(oacc[db][vq * 4 + 0] * inv, oacc[db][vq * 4 + 1] * inv);
      pk[1] = pack_bf16x2(oacc[db][vq * 4 + 2] * inv, oacc[db][vq * 4 + 3] * inv);
      *(u32x2_t*)(ost + c * OROW + (db * 32 + vq * 8 + h2 * 4) * 2) = pk;
    }
  __builtin_amdgcn_wave_barrier();
  constexpr int RPS = 64 / (D / 8);  // rows per wave store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int r = i * RPS + lane / (D / 8), ch = lane % (D / 8);
    const u32x4_t val = *(const u32x4_t*)(ost + r * OROW + ch * 16);
    if (qw0 + r < Nq) __builtin_nontemporal_store(val, (u32x4_t*)(og + (long long)(qw0 + r) * p.o_sn + ch * 8));
  }
  if (p.lse && h2 == 0 && qi < Nq)
    p.lse[lse_row0 + qi] = (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
}

template <int D, bool PAGED>
hipError_t launch_pp(const PrefillParams& p, int n_rows, hipStream_t stream) {
  using C = PP<D>;
  const int n_qtiles = (n_rows + C::BM - 1) / C::BM;
  const long long total = (long long)p.B * p.Hq * n_qtiles;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_pp_kernel<D, PAGED>), dim3((unsigned)total), dim3(C::NT), 0, stream, p, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_pp(const PrefillParams& p, int d, int n_rows, bool paged, hipStream_t stream) {
  if (d == 128) return paged ? launch_pp<128, true>(p, n_rows, stream) : launch_pp<128, false>(p, n_rows, stream);
  if (d == 64) return paged ? launch_pp<64, true>(p, n_rows, stream) : launch_pp<64, false>(p, n_rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
