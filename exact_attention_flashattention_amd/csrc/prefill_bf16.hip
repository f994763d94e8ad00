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
//    the order the S^T accumulator hands them out. V stays in its natural
//    [key][d] layout in LDS; the V^T operand is read with ds_read_b64_tr_b16,
//    whose 16-lane transpose hands each lane four consecutive keys of one
//    dimension, so two such reads form one A operand in exactly that key order.
//  * K and V tiles are copied HBM -> LDS with global_load_lds_dwordx4 (no
//    registers, no LDS store instructions). Each 16-byte chunk of a row is
//    stored at a position XOR-swizzled by the row, chosen so that both the K
//    operand reads (16 consecutive rows, one chunk each) and the transposed V
//    reads (4 consecutive rows, two chunks each) hit distinct LDS banks.
//  * Software pipeline: iteration j first issues the MFMAs of tile j+1's
//    scores, then takes tile j's row max (those scores finished an iteration
//    earlier, so nothing waits on an MFMA result), then exponentiates tile j
//    with its P.V MFMAs interleaved. Four LDS buffers rotate: tile j (V
//    read), tile j+1 (K read), tile j+2 (landed) and tile j+3 (loads in
//    flight, issued three iterations before use); one barrier per tile.
//  * The reference point m used in 2^(s - m) is only moved when a row's max
//    exceeds it by more than 2^8 (a wave-uniform ballot; then O and l are
//    rescaled exactly); between moves the weights are bounded by 2^8, which
//    bf16 and fp32 represent with the same relative precision. Results are
//    identical in exact arithmetic, and the accumulators are untouched on
//    most tiles.
//  * Row sums of P are taken from the bf16-rounded weights (dot2 against
//    ones), so numerator and denominator use the same weights.
//  * Work-groups are numbered so that each XCD receives whole (b, KV head)
//    pairs (its L2 then holds those K/V), and the heaviest causal query tiles
//    start first: within a pair, or across all of an XCD's pairs when a pair
//    has fewer work items than the XCD has CUs.
//  * Inputs must be finite: rows past the end of the sequence are filled with
//    the last row (finite) and masked out of the softmax, so their weight is
//    exactly 0.
#include "attn_internal.h"
#include "cdna4.h"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kPage = 16;  // tokens per page of a paged KV cache
// Lazy-rescale threshold in base-2 exponent units: the running reference is
// moved only when a row max exceeds it by more than this.
constexpr float kRescaleTau = 8.0f;

template <int D, int NW, int BN>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;       // 32-key blocks per tile
  static constexpr int PS = BN / 16;       // 16-key k-steps of O^T += V^T P^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int ROWB = D * 2;       // bytes per key row (K and V alike)
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;     // rows per wave load instruction (1 KiB)
  static constexpr int LPT = BN / RPI;     // load instructions per tensor per tile
  static constexpr int IPW = (LPT + NW - 1) / NW;  // of which one wave issues at most
  static constexpr int TILE = BN * ROWB;   // bytes of one K (or V) tile
  static constexpr int NBUF = 4;           // ring of tile buffers
  static constexpr int VREG = NBUF * TILE; // K tiles at [0, VREG), V tiles at [VREG, 2 VREG)
  static constexpr int OROW = D * 2 + 16;  // padded bytes per staged output row
  static constexpr int LDS_BYTES = (2 * VREG > NW * 32 * OROW) ? 2 * VREG : NW * 32 * OROW;
  static_assert(LPT % NW == 0 || NW % LPT == 0, "uneven tile loads");
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "bad tile");
};

// PAGED = false: one [B, N, H, d] or [B, H, N, d] sequence per batch entry,
// query row i at position i. PAGED = true: a chunk of queries per sequence
// (rows cu_q[b] ..) at positions P_b + i, keys read through the block table.
template <int D, int NW, int BN, bool PAGED>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(PrefillParams p, int n_qtiles) {
  using C = Cfg<D, NW, BN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];

  // ---- work decomposition --------------------------------------------------
  const int g = p.Hq / p.Hkv;
  const int total = p.B * p.Hq * n_qtiles;
  const int bid = blockIdx.x;
  // Hardware hands consecutive work-group ids to the 8 XCDs round-robin;
  // renumber so that each XCD gets one contiguous range of work items.
  const int w = xcd_remap(bid, total);
  const int per_pair = n_qtiles * g;
  // (kv head, b) pairs with b fastest: an XCD's contiguous range then holds
  // the same KV heads of different sequences, which keeps the XCDs balanced
  // when the sequences differ in length. Inside a group of G pairs the
  // heaviest causal query tiles of all G pairs come first (longest work
  // first). A pair with at least as many work items as an XCD has CUs keeps
  // G = 1; a smaller one (few query tiles, few query heads per KV head) would
  // leave its light tiles to run beside the next pair's heavy ones, so its
  // group is an XCD's whole share of pairs (measured: MHA at d = 64, N = 2048
  // 141 -> 95 us; larger pairs lose a little L2 locality when grouped).
  constexpr int kCusPerXcd = 32;
  const int n_pairs = p.B * p.Hkv;
  const int G = per_pair >= kCusPerXcd ? 1 : max(1, min(n_pairs, (total >> 3) / per_pair));
  const int grp = w / (G * per_pair);
  const int r_in = w - grp * G * per_pair;
  const int row_items = min(G, n_pairs - grp * G) * g;  // items per query-tile rank in this group
  const int qrank = r_in / row_items;
  const int rest = r_in - qrank * row_items;
  const int pair = grp * G + rest / g;
  const int qtile = n_qtiles - 1 - qrank;  // heaviest causal tiles first
  const int hg = rest - (rest / g) * g;
  const int kvh = pair / p.B;
  const int b = pair - kvh * p.B;
  const int h = kvh * g + hg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int c = lane & 31;   // query column of S^T / O^T held by this lane
  const int h2 = lane >> 5;  // lane half

  const int q_tile0 = qtile * C::BM;
  // Nq query rows and Nk keys for this (b, h); P is the position of query
  // row 0, so row i sees keys 0 .. P + i (causality compares positions).
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
  // Query block of this wave. Waves w and w + 4 share a SIMD; pairing block w
  // with block NW - 1 - (w - 4) gives every SIMD one early and one late block,
  // so the causal work per SIMD is balanced.
  const int qblk = (NW == 8 && wave >= 4) ? 11 - wave : wave;
  const int qw0 = q_tile0 + qblk * 32;  // first query row of this wave
  const int qi = qw0 + c;               // this lane's query row

  // contiguous: this (b, kv head)'s row 0; paged: the pools' kv head offset
  const __bf16* __restrict__ kg = (const __bf16*)p.k + (PAGED ? 0 : b * p.k_sb) + kvh * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + (PAGED ? 0 : b * p.k_sb) + kvh * p.k_sh;

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
    const int qc = min(qi, Nq - 1);
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
  // A learned sink logit s_h is an extra score column with zero value: it
  // enters as the initial state m = s_h, l = e^0 = 1, O = 0.
  // m_ref starts at the most negative finite float ("no key yet"): masked
  // scores stay -inf through s*c2 - m_ref, so no -inf guards are needed, and
  // the first finite row max always moves it (the rescale factor is then 0).
  float m_ref = -3.402823466e38f, l_run = 0.f;
  if (p.sinks) {
    m_ref = p.sinks[h] * 1.4426950408889634f;  // base-2 units, like the scores
    l_run = h2 == 0 ? 1.f : 0.f;  // the two lane halves' sums are added at the end
  }

  // ---- the key tiles this work-group visits -------------------------------------
  // Tiles past the causal limit of the last row are never visited; with a
  // window W, neither are the tiles before the window of the first row,
  // except the tiles holding the n_sink initial positions. The visited tiles
  // are numbered by "slots": sink tiles first, then the window tiles.
  const int q_last_wg = min(q_tile0 + C::BM, Nq) - 1;
  const int k_tiles = (Nk + BN - 1) / BN;
  const int n_tiles = p.causal ? min(k_tiles, (P + q_last_wg) / BN + 1) : k_tiles;
  const int W = p.window;
  const int sink_tiles = (W > 0 && p.n_sink > 0) ? min((p.n_sink + BN - 1) / BN, n_tiles) : 0;
  const int win_lo = W > 0 ? max(max(P + q_tile0 - W + 1, 0) / BN, sink_tiles) : 0;
  const int n_slots = sink_tiles + max(n_tiles - win_lo, 0);
  auto tile_of = [&](int j) __attribute__((always_inline)) { return j < sink_tiles ? j : win_lo + (j - sink_tiles); };
  auto slot_of = [&](int t) __attribute__((always_inline)) { return t < sink_tiles ? t : t - win_lo + sink_tiles; };
  // Slots w_first .. w_end-1 hold keys visible to some row of this wave. With
  // initial-token tiles the wave also visits the sink slots 0 .. sink_tiles-1
  // first; when its own window starts past them (sink_gap) the slots in
  // between are skipped like those of a later wave.
  int w_first = 0, w_end = 0;
  bool sink_gap = false;
  if (qw0 < Nq) {
    const int last = (p.causal ? min(n_tiles, (P + qw0 + 31) / BN + 1) : n_tiles) - 1;
    w_end = slot_of(last) + 1;
    if (W > 0) {
      const int t_w = max(P + qw0 - W + 1, 0) / BN;  // the wave's first window tile
      if (sink_tiles == 0) {
        w_first = slot_of(t_w);
      } else {
        // t_w >= sink_tiles implies t_w >= win_lo, so slot_of(t_w) is its slot
        const int ws = t_w >= sink_tiles ? slot_of(t_w) : 0;
        if (ws > sink_tiles && ws < w_end) {
          sink_gap = true;
          w_first = ws;
        }
      }
    }
  }

  // ---- HBM -> LDS copies of K/V tiles ----------------------------------------------
  // Buffer i of the ring: K tile at lds + i*TILE, V tile VREG bytes further.
  // With the K and V tiles in separate halves every LDS read below is a
  // per-lane register plus an immediate offset below 64 KiB, so once the ring
  // position is a compile-time constant no address arithmetic is left.
  auto kbuf = [&](int t) __attribute__((always_inline)) { return lds + (t % C::NBUF) * C::TILE; };
  auto vbuf = [&](int t) __attribute__((always_inline)) { return lds + C::VREG + (t % C::NBUF) * C::TILE; };
  // This lane's part of a load instruction: tile-local row, logical chunk and
  // the byte offset from the tile's first row (rows are k_sn elements apart).
  const int ld_row = lane / C::CPR;
  const int ld_pos = lane % C::CPR;
  const unsigned row_bytes = (unsigned)p.k_sn * 2u;
  // Paged: a load instruction covers RPI rows inside one 16-token page, so its
  // page is wave-uniform and the lane offset is from the page's first token.
  unsigned ld_off[C::IPW];
#pragma unroll
  for (int u = 0; u < C::IPW; ++u) {
    const int row = (wave + u * NW) * C::RPI + ld_row;
    const int prow = PAGED ? (row & (kPage - 1)) : row;
    ld_off[u] = (unsigned)prow * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
  }
  // block table row of this sequence, read with scalar loads
  const __attribute__((address_space(4))) int32_t* const table =
      PAGED ? (const __attribute__((address_space(4))) int32_t*)(p.block_table + (long long)b * p.max_pages_per_seq)
            : nullptr;
  const long long page_bytes = (long long)row_bytes * kPage;
  // issue the copies of tile t (this wave's share: instructions wave, wave+NW, ...)
  auto issue_tile = [&](int t, unsigned char* __restrict__ kl) __attribute__((always_inline)) {
    const int k0 = tile_of(t) * BN;
    unsigned char* const vl = kl + C::VREG;
    const bool ragged = k0 + BN > Nk;
#pragma unroll
    for (int u = 0; u < C::IPW; ++u) {
      const int i = wave + u * NW;
      if (C::LPT < NW && i >= C::LPT) break;  // wave-uniform
      const char* kt;
      const char* vt;
      if constexpr (PAGED) {
        // the page of this instruction's rows (the last key's page once past the end)
        const int page = table[min(k0 + i * C::RPI, Nk - 1) / kPage];
        kt = (const char*)kg + page * page_bytes;
        vt = (const char*)vg + page * page_bytes;
      } else {
        kt = (const char*)kg + (long long)k0 * row_bytes;  // wave-uniform
        vt = (const char*)vg + (long long)k0 * row_bytes;
      }
      unsigned off = ld_off[u];
      if (ragged) {
        // rows past the end repeat the last key's row (finite); the softmax masks them
        const int row = i * C::RPI + ld_row;
        const int chunk = ld_pos ^ swz<C::CPR>(row);
        const int key = min(k0 + row, Nk - 1);
        const int prow = PAGED ? (key & (kPage - 1)) : key - k0;
        off = (unsigned)prow * row_bytes + (unsigned)chunk * 16u;
      }
      load_to_lds(kt + off, kl + i * 1024);
      load_to_lds(vt + off, vl + i * 1024);
    }
  };
  // loads this wave issues per tile (all waves that issue any issue this many)
  constexpr int kLoadsPerTile = 2 * C::IPW;

  // ---- per-lane parts of the LDS read addresses (bytes from a tile's start) ------
  // K operand of k-step s: row c (+32 per key block), chunk (2s + h2) ^ swz(c).
  unsigned kpart[C::KS];
#pragma unroll
  for (int s_ = 0; s_ < C::KS; ++s_)
    kpart[s_] = (unsigned)(c * C::ROWB + (((2 * s_ + h2) ^ swz<C::CPR>(c)) * 16));
  // V^T operand: lane l = 16 G + 4 t + u addresses V[key][d] with
  // key = ps*16 + 8 r + 4 h2 + t and d = db*32 + 16 (G & 1) + 4 u; the
  // transpose read then gives lane l the keys ps*16 + 8 r + 4 h2 + 0..3 of
  // dimension db*32 + l % 32. The ps term is a multiple of 16 rows, which the
  // swizzle ignores, so it is an immediate offset. The parts include the V
  // half's base VREG, leaving ring position and ps to the 16-bit immediate.
  unsigned vpart[2][C::DB];
  {
    const int tr_t = (lane >> 2) & 3, tr_u = lane & 3, tr_g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int key = 8 * r + 4 * h2 + tr_t;
        const int d = db * 32 + 16 * tr_g + 4 * tr_u;
        vpart[r][db] = (unsigned)(C::VREG + key * C::ROWB + ((d >> 3) ^ swz<C::CPR>(key)) * 16 + ((d >> 2) & 1) * 8);
      }
  }
  // Hide the lane parts from loop-invariant code motion once per tile step:
  // otherwise every (buffer, read) address of the unrolled loop is hoisted
  // into a register of its own, far more than the register file holds.
  auto refresh_parts = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_) asm volatile("" : "+v"(kpart[s_]));
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) asm volatile("" : "+v"(vpart[r][db]));
  };

  // ---- the three steps of a tile ----------------------------------------------
  // S^T = K Q^T for tile t
  auto qk = [&](const unsigned char* __restrict__ k_lds, f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
    // operands of k-step s+1 are read before the products of k-step s
    u32x4_t a[2][C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) a[0][kb] = *(const u32x4_t*)(k_lds + kpart[0] + kb * 32 * C::ROWB);
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_) {
      if (s_ + 1 < C::KS) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
          a[(s_ + 1) & 1][kb] = *(const u32x4_t*)(k_lds + kpart[s_ + 1] + kb * 32 * C::ROWB);
      }
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) s[kb] = mfma_32x32x16(a[s_ & 1][kb], qreg[s_], s[kb]);
    }
    // keep the reads one k-step ahead of the products (the scheduler would
    // otherwise reuse one operand register and wait on every read)
    __builtin_amdgcn_sched_group_barrier(0x100, C::KB, 0);
#pragma unroll
    for (int s_ = 0; s_ < C::KS; ++s_) {
      if (s_ + 1 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, C::KB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, C::KB, 0);
    }
  };
  // mask tile t where it reaches past the diagonal or the end, then move the
  // reference max if this tile's max exceeds it by more than the threshold
  auto prep = [&](int t, f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {
    const int k0 = tile_of(t) * BN;
    const bool win_cut = W > 0 && k0 < P + qw0 + 31 - W + 1 && k0 + BN > p.n_sink;
    if ((p.causal && k0 + BN - 1 > P + qw0) || (k0 + BN > Nk) || win_cut) {
      // key k0 + h2*4 + off (off a compile-time constant per element) is visible
      // iff off <= lim, and with a window iff also off >= lo or it is one of
      // the n_sink initial positions (off < sk)
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
    // max of this lane's keys over four interleaved running maxima (one
    // running max would be a single chain of dependent v_max3 on the critical
    // path of every tile); a row's max exceeds the reference by more than the
    // threshold iff one of its two lane halves does, so the cross-lane row max
    // is taken only on the rare tiles that move the reference
    float rm[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) rm[e & 3] = fmaxf(rm[e & 3], s[kb][e]);
    const float mh = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
    if (__builtin_amdgcn_ballot_w64(mh * c2 > m_ref + kRescaleTau)) {
      const float m_new = fmaxf(m_ref, halves_max(mh) * c2);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
  };
  // P = 2^(s - m) rounded to bf16, l += rowsum(P), O^T += V^T P^T for tile t
  auto pv = [&](const unsigned char* __restrict__ vt_lds, const f32x16_t (&s)[C::KB]) __attribute__((always_inline)) {  // V tile of tile j
    const float neg_m = -m_ref;
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
        u32x4_t a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt_lds - C::VREG + vpart[r][db] + ps * 16 * C::ROWB));
          const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
          a[2 * r] = xx[0];
          a[2 * r + 1] = xx[1];
        }
        oacc[db] = mfma_32x32x16(a, pop[ps], oacc[db]);
      }
  };

  // ---- prologue: slots 0, 1, 2 in flight; scores of slot 0 -------------------------
  f32x16_t sa[C::KB], sb[C::KB];
  if (n_slots > 0) issue_tile(0, kbuf(0));
  if (n_slots > 1) issue_tile(1, kbuf(1));
  if (n_slots > 2) {
    issue_tile(2, kbuf(2));
    wait_vmcnt<kLoadsPerTile>();  // slots 0 and 1 have landed
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  if ((w_first == 0 || sink_gap) && w_end > 0) qk(kbuf(0), sa);

  // ---- main loop: iteration j consumes slot j and computes the scores of j+1 -------
  // Every wave runs n_slots iterations (one barrier each); the loops only
  // differ in how much of the tile work the wave has in each. Slot j+3 is
  // issued at the top of iteration j into the buffer slot j-1 used; slot j+2
  // must have landed before the barrier that ends iteration j. The buffers
  // reach the steps as distinct restrict pointers, which tells the compiler
  // that reading slots j and j+1 need not wait for the copy into j+3.
  auto end_iteration = [&](int j) __attribute__((always_inline)) {
    if (j + 3 < n_slots)
      wait_vmcnt<kLoadsPerTile>();
    else
      wait_vmcnt<0>();
    wait_lgkmcnt<0>();  // this wave's reads of the buffer the next copy overwrites
    barrier_nofence();
  };
  // b_issue: buffer receiving tile j+3; b_k: K tile of tile j+1; b_v: V tile of tile j.
  // The scores of tile j were computed in the previous iteration, so their
  // row max (prep) does not wait on an MFMA result and fills the shadow of
  // the MFMAs of tile j+1's scores; exponentiation then overlaps P V.
  auto full_step = [&](int j, unsigned char* __restrict__ b_issue, const unsigned char* __restrict__ b_k,
                       const unsigned char* __restrict__ b_v, f32x16_t (&s_cur)[C::KB],
                       f32x16_t (&s_nxt)[C::KB]) __attribute__((always_inline)) {
    refresh_parts();
    if (j + 3 < n_slots) issue_tile(j + 3, b_issue);
    qk(b_k, s_nxt);  // scores of tile j+1
    prep(j, s_cur);
    pv(b_v, s_cur);
  };
  auto last_step = [&](int j, unsigned char* __restrict__ b_issue, const unsigned char* __restrict__ b_v) __attribute__((always_inline)) {
    if (j + 3 < n_slots) issue_tile(j + 3, b_issue);
    prep(j, sa);
    pv(b_v, sa);
  };
  // the scores of slot j+1, the first of this wave's slots
  auto first_step = [&](int j, unsigned char* __restrict__ b_issue, const unsigned char* __restrict__ b_k) __attribute__((always_inline)) {
    refresh_parts();
    if (j + 3 < n_slots) issue_tile(j + 3, b_issue);
    qk(b_k, sa);
  };
  auto single_step = [&](int j) __attribute__((always_inline)) {  // a full step with run-time ring positions
    full_step(j, kbuf(j + 3), kbuf(j + 1), vbuf(j), sa, sb);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) sa[kb] = sb[kb];
    end_iteration(j);
  };
  auto idle_step = [&](int j) __attribute__((always_inline)) {  // no work for this wave: keep loading slots for the others
    if (j + 3 < n_slots) issue_tile(j + 3, kbuf(j + 3));
    end_iteration(j);
  };
  int j = 0;
  if (sink_gap) {  // the sink slots, then a gap up to the wave's window
    for (; j + 1 < sink_tiles; ++j) single_step(j);
    last_step(j, kbuf(j + 3), vbuf(j));
    end_iteration(j);
    ++j;
  }
  for (; j + 1 < w_first; ++j) idle_step(j);
  if (w_first > 0 && w_first < w_end) {
    first_step(j, kbuf(j + 3), kbuf(j + 1));
    end_iteration(j);
    ++j;
  }
  // (from here j == w_first) up to the next multiple of four one step at a time
  for (; (j & 3) && j + 1 < w_end; ++j) single_step(j);
  // Slots j .. j+4 all have work for this wave: unrolled by four, so the
  // ring positions are compile-time constants (j is a multiple of four) and
  // the score registers alternate instead of being copied.
  for (; j + 4 < w_end; j += 4) {
    full_step(j, kbuf(3), kbuf(1), vbuf(0), sa, sb);
    end_iteration(j);
    full_step(j + 1, kbuf(0), kbuf(2), vbuf(1), sb, sa);
    end_iteration(j + 1);
    full_step(j + 2, kbuf(1), kbuf(3), vbuf(2), sa, sb);
    end_iteration(j + 2);
    full_step(j + 3, kbuf(2), kbuf(0), vbuf(3), sb, sa);
    end_iteration(j + 3);
  }
  for (; j + 1 < w_end; ++j) single_step(j);
  if (j < w_end) {  // the wave's last slot
    last_step(j, kbuf(j + 3), vbuf(j));
    end_iteration(j);
    ++j;
  }
  for (; j < n_slots; ++j) idle_step(j);

  // ---- epilogue: O / l -> bf16, written as whole rows through LDS ---------------------
  // (every wave has passed the last barrier with no copy in flight, so the tile
  // buffers are free)
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
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;     // rows per wave instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, ch = lane % CPR;
    const u32x4_t val = *(const u32x4_t*)(ost + r * OROW + ch * 16);
    // non-temporal: O is written once and not read here, so its lines go out
    // to HBM while this compute-bound kernel runs instead of lingering dirty
    // in the caches until a later, bandwidth-bound kernel evicts them
    if (qw0 + r < Nq) __builtin_nontemporal_store(val, (u32x4_t*)(og + (long long)(qw0 + r) * p.o_sn + ch * 8));
  }
  // m_ref is in units of scale * log2(e) * q.k (the sign fold leaves that product unchanged)
  if (p.lse && h2 == 0 && qi < Nq)
    p.lse[lse_row0 + qi] = (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
}

// n_rows: query rows per sequence (the longest chunk when paged)
template <int D, int NW, int BN, bool PAGED>
hipError_t launch_cfg(const PrefillParams& p, int n_rows, hipStream_t stream) {
  using C = Cfg<D, NW, BN>;
  const int n_qtiles = (n_rows + C::BM - 1) / C::BM;
  const long long total = (long long)p.B * p.Hq * n_qtiles;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BN, PAGED>), dim3((unsigned)total), dim3(C::NT), 0,
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

#ifndef ATTN_PREFILL_PINGPONG
#define ATTN_PREFILL_PINGPONG 0
#endif

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream) {
  if (ATTN_PREFILL_PINGPONG) return launch_prefill_pp(p, d, p.N, false, stream);
  if (d == 128) return launch_cfg<128, ATTN_PREFILL_D128, false>(p, p.N, stream);
  if (d == 64) return launch_cfg<64, ATTN_PREFILL_D64, false>(p, p.N, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_paged(const PrefillParams& p, int d, int max_q_len, hipStream_t stream) {
  if (ATTN_PREFILL_PINGPONG) return launch_prefill_pp(p, d, max_q_len, true, stream);
  if (d == 128) return launch_cfg<128, ATTN_PREFILL_D128, true>(p, max_q_len, stream);
  if (d == 64) return launch_cfg<64, ATTN_PREFILL_D64, true>(p, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
