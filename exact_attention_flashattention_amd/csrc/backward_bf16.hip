// Backward of the causal (or full) GQA prefill, bf16 inputs, fp32 accumulation.
//
// For o = softmax(S) V with S = scale * Q K^T + M, the gradients given dO are
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// and a KV head's dK, dV sum over the g query heads that read it (GQA rule of
// "Module 5. Modern Attention Mechanisms", section 6). As the "inference-
// attention" page says of FlashAttention's backward ("FlashAttention"), S and
// P are recomputed tile by tile instead of stored: P = 2^(S log2(e) - lse2)
// with the forward's log-sum-exp, so no running max is needed.
//
// Two kernels, in this order:
//  * bwd_dq: a work-group owns 32 queries per wave of one (b, h) and streams
//    the K and V tiles, like the forward. Each wave also forms D_i and
//    lse2_i = lse_i * log2(e) of its rows and writes them to the workspace.
//  * bwd_dkdv: a work-group owns 128 keys of one (b, KV head), 32 per pair
//    of waves, and streams the Q and dO tiles (and their D, lse2) of every
//    query head of the group through LDS; one wave of a pair keeps dV^T and
//    the other dK^T in registers, so no atomics.
// Both kernels copy tiles HBM -> LDS with global_load_lds into a ring
// (one barrier per tile) and read them with the same XOR swizzle
// as the forward: row reads for the A operand of S = Q K^T / dP = dO V^T and
// ds_read_b64_tr_b16 transposed reads for the A operand of the dK, dV, dQ
// products. Score tiles are held in the MFMA accumulator layout whose lanes
// already form the B operand of the next product (the key/query order of each
// 16-wide k-step is the accumulator's), as in the forward.
#include <type_traits>

#include "attn_internal.h"
#include "cdna4.h"

namespace attn {
namespace {

using namespace cdna4;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Tile geometry shared by the two main kernels: NW waves, BN rows per streamed
// tile, head dimension D.
template <int D, int NW, int BN>
struct BCfg {
  static constexpr int NT = NW * 64;
  static constexpr int KS = D / 16;        // 16-dim k-steps of the row products
  static constexpr int RB = BN / 32;       // 32-row blocks of a streamed tile
  static constexpr int PS = BN / 16;       // 16-row k-steps of the transposed products
  static constexpr int DB = D / 32;        // 32-row blocks of the d x 32 accumulators
  static constexpr int ROWB = D * 2;       // bytes per row
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;     // rows per 1 KiB load instruction
  static constexpr int LPT = BN / RPI;     // load instructions per tensor per tile
  static constexpr int IPW = (LPT + NW - 1) / NW;
  static constexpr int TILE = BN * ROWB;
  static constexpr int NBUF = 4;
  static constexpr int BREG = NBUF * TILE;  // first tensor's tiles at [0, BREG), second's at [BREG, 2 BREG)
  static constexpr int OROW = D * 2 + 16;
  static_assert(LPT % NW == 0 || NW % LPT == 0, "uneven tile loads");
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "bad tile");
};

// ---------------------------------------------------------------------------
// dK and dV. A key block is 32*NP keys of one (b, KV head); its streamed
// slots are (query tile, query head of the group) over the tiles that hold a
// query at or after the block's first key (causal) or all tiles, tile-major.
// A work item takes key block j with its tiles in descending order and then
// key block n_kblk-1-j in ascending order. Under the causal mask the two
// blocks together stream the same number of tiles for every j, and at any
// time all items of one (b, KV head) stream one of two tiles (tile T-1-r in
// the first block, tile r-2 in the second, r counted from the item's start),
// so the work-groups that run side by side share their Q/dO reads in L2.
//
// The work of a 32-key block is split over a pair of waves that share a SIMD
// (waves w and w + NP): the "P wave" w computes S = Q K^T, the weights
// P = 2^(S c2 - lse2) and dV^T += dO^T P, and hands P (bf16) to its partner
// through LDS; the "dS wave" w + NP computes dP = dO V^T, dS = P (dP - D) and
// dK^T += Q^T dS. The dS wave runs one slot behind: in slot j it finishes
// slot j - 1 (whose P was written during slot j - 1) and then forms dP for
// slot j, which it keeps in registers. Each wave holds one of K, V and one of
// the two gradients, so two waves fit on a SIMD, and the exponentials of one
// wave overlap the products of the other.
template <int D, int NP, int BN>
__global__ __launch_bounds__(2 * NP * 64, 1) void bwd_dkdv_kernel(BwdParams p, int n_kblk) {
  constexpr int NW = 2 * NP;
  using C = BCfg<D, NW, BN>;
  constexpr int NB = 3;                          // ring: slot j-1 (dS wave), j (both), j+1 (landing)
  constexpr int RING = NB * C::TILE;             // Q tiles at [0, RING), dO tiles at [RING, 2 RING)
  constexpr int SREG = 2 * RING;                 // per-wave copies of (lse2, D) rows
  constexpr int SBUF = NW * 1024;
  constexpr int PREG = SREG + NB * SBUF;         // P hand-over: 2 slots x NP pairs x RB blocks x 2 KiB
  constexpr int PPAIR = C::RB * 2 * 1024;
  constexpr int PSLOT = NP * PPAIR;
  constexpr int LDS_MAIN = PREG + 2 * PSLOT;
  constexpr int LDS_OUT = NW * 32 * C::OROW;
  static_assert(LDS_MAIN <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT];

  const int g = p.Hq / p.Hkv;
  const int N = p.N;
  const int n_items = (n_kblk + 1) / 2;
  const int w = xcd_remap(blockIdx.x, p.B * p.Hkv * n_items);
  const int pair = w / n_items;                // (kv head, b), b fastest
  const int item = w - pair * n_items;
  const int kvh = pair / p.B, b = pair - kvh * p.B;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pi = wave % NP;                    // key block of the wave pair
  const bool ds_wave = wave >= NP;
  const int c = lane & 31, h2 = lane >> 5;

  // one key block, its tiles descending or ascending
  auto run_block = [&](const int kblk, const bool desc) __attribute__((always_inline)) {
    const int k_blk0 = kblk * NP * 32;
    const int kw0 = k_blk0 + pi * 32;            // the pair's first key
    const int kj = kw0 + c;                      // this lane's key (column of S)
    const float c2 = p.scale_log2;

    // K (P wave) or V (dS wave) of this lane's key as B operands (k-step s:
    // dims s*16 + h2*8 .. +7)
    u32x4_t kvreg[C::KS];
    {
      const int kc = min(kj, N - 1);
      const __bf16* src = (const __bf16*)(ds_wave ? p.v : p.k) + b * p.k_sb + (long long)kc * p.k_sn + kvh * p.k_sh;
  #pragma unroll
      for (int s = 0; s < C::KS; ++s) kvreg[s] = *(const u32x4_t*)(src + s * 16 + h2 * 8);
    }
    f32x16_t grad[C::DB];  // dV^T (P wave) or dK^T / scale (dS wave)
  #pragma unroll
    for (int db = 0; db < C::DB; ++db)
  #pragma unroll
      for (int e = 0; e < 16; ++e) grad[db][e] = 0.f;
    f32x16_t dp[C::RB];  // dS wave: dP of the current slot, carried into the next
  #pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
  #pragma unroll
      for (int e = 0; e < 16; ++e) dp[rb][e] = 0.f;

    // streamed slots: slot s is query head s % g of tile rank r = s / g, the
    // tile T - 1 - r (descending) or t0 + r (ascending)
    const int T = (N + BN - 1) / BN;
    const int t0 = p.causal ? k_blk0 / BN : 0;
    const int nT = T - t0;
    const int n_slots = g * nT;
    const int w_t = p.causal ? kw0 / BN : 0;  // the pair's first tile
    const bool pair_live = kw0 < N;
    auto tile_of = [&](int slot) __attribute__((always_inline)) {
      const int r = slot / g;
      return desc ? T - 1 - r : t0 + r;
    };
    auto live = [&](int slot) __attribute__((always_inline)) { return pair_live && tile_of(slot) >= w_t; };

    // Buffer addresses of a slot. The offset goes through an empty asm
    // statement so that it is formed once per slot in a scalar register: left
    // to itself the compiler precomputes every (buffer, lane offset) sum as a
    // loop-invariant vector register (most exceed the 16-bit immediate offset
    // of the LDS instructions) and runs out of registers.
    auto at = [&](unsigned off) __attribute__((always_inline)) {
      asm volatile("" : "+s"(off));
      return lds + off;
    };
    auto qbuf = [&](int s) __attribute__((always_inline)) { return at((unsigned)(s % NB) * C::TILE); };
    auto dbuf = [&](int s) __attribute__((always_inline)) { return at(RING + (unsigned)(s % NB) * C::TILE); };
    auto sbuf = [&](int s) __attribute__((always_inline)) {
      return at(SREG + (unsigned)(s % NB) * SBUF + wave * 1024);
    };
    auto pbuf = [&](int s) __attribute__((always_inline)) {
      return at(PREG + (unsigned)(s & 1) * PSLOT + pi * PPAIR);
    };

    const int ld_row = lane / C::CPR, ld_pos = lane % C::CPR;
    const unsigned row_bytes = (unsigned)p.q_sn * 2u;
    unsigned ld_off[C::IPW];
  #pragma unroll
    for (int u = 0; u < C::IPW; ++u) {
      const int row = (wave + u * NW) * C::RPI + ld_row;
      ld_off[u] = (unsigned)row * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
    }
    auto issue = [&](int slot) __attribute__((always_inline)) {
      const int hg = slot % g, t = tile_of(slot);
      const int h = kvh * g + hg;
      const int r0 = t * BN;
      const char* qt = (const char*)((const __bf16*)p.q + b * p.q_sb + h * p.q_sh) + (long long)r0 * row_bytes;
      const char* dt = (const char*)((const __bf16*)p.dout + b * p.q_sb + h * p.q_sh) + (long long)r0 * row_bytes;
      const bool ragged = r0 + BN > N;
  #pragma unroll
      for (int u = 0; u < C::IPW; ++u) {
        const int i = wave + u * NW;
        if (C::LPT < NW && i >= C::LPT) break;
        unsigned off = ld_off[u];
        if (ragged) {  // rows past the end repeat the last row (finite); they are masked
          const int row = i * C::RPI + ld_row;
          off = (unsigned)(min(r0 + row, N - 1) - r0) * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
        }
        load_to_lds(qt + off, qbuf(slot) + i * 1024);
        load_to_lds(dt + off, dbuf(slot) + i * 1024);
      }
      // stats rows r0 .. r0+63 (padded arrays): lanes 0-15 lse2, 16-31 D, 32-63 again
      const long long srow = ((long long)b * p.Hq + h) * p.Npad + r0;
      const int l32 = lane & 31;
      const float* src = (l32 < 16 ? p.lse2 : p.dvec) + srow + (l32 & 15) * 4;
      load_to_lds(src, sbuf(slot));
    };

    // per-lane parts of the LDS reads (bytes from a tile's start)
    unsigned rpart[C::KS];  // row reads: row c (+32 per block), chunk (2s + h2) ^ swz(c)
  #pragma unroll
    for (int s = 0; s < C::KS; ++s) rpart[s] = (unsigned)(c * C::ROWB + (((2 * s + h2) ^ swz<C::CPR>(c)) * 16));
    unsigned tpart[2][C::DB];  // transposed reads: rows ps*16 + 8r + 4h2 + t, dims db*32 + 16G + 4u
    {
      const int tr_t = (lane >> 2) & 3, tr_u = lane & 3, tr_g = (lane >> 4) & 1;
  #pragma unroll
      for (int r = 0; r < 2; ++r)
  #pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int row = 8 * r + 4 * h2 + tr_t;
          const int d = db * 32 + 16 * tr_g + 4 * tr_u;
          tpart[r][db] = (unsigned)(row * C::ROWB + ((d >> 3) ^ swz<C::CPR>(row)) * 16 + ((d >> 2) & 1) * 8);
        }
    }
    auto tr_read = [&](const unsigned char* base, int ps, int db) __attribute__((always_inline)) {
      u32x4_t a;
  #pragma unroll
      for (int r = 0; r < 2; ++r) {
        const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(base + tpart[r][db] + ps * 16 * C::ROWB));
        const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
        a[2 * r] = xx[0];
        a[2 * r + 1] = xx[1];
      }
      return a;
    };
    // 32 rows of a streamed tile times this pair's 32 keys: lane (key c) holds
    // query rows rb*32 + 8 (e/4) + 4 h2 + e%4
    auto row_product = [&](const unsigned char* tile, int rb) __attribute__((always_inline)) {
      f32x16_t acc;
  #pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  #pragma unroll
      for (int s = 0; s < C::KS; ++s)
        acc = mfma_32x32x16(*(const u32x4_t*)(tile + rpart[s] + rb * 32 * C::ROWB), kvreg[s], acc);
      return acc;
    };
    // P and dS words, in the accumulator's lane layout: k-step ps = 2 rb + kk
    // holds the rows of groups r = 2 kk, 2 kk + 1 (words 2(r&1), 2(r&1)+1), so
    // the packed words are the B operand of the transposed products as they are
    const int hand = lane * 16;  // byte offset of this lane's 16 bytes in a 1 KiB hand-over block

    // P wave, slot j: S, P (to LDS), dV^T += dO^T P
    auto p_step = [&](int slot) __attribute__((always_inline)) {
      const int t = tile_of(slot);
      const int r0 = t * BN;
      const unsigned char* qt = qbuf(slot);
      const unsigned char* dt = dbuf(slot);
      const unsigned char* st = sbuf(slot) + h2 * 16;  // this lane's rows 4 h2 .. 4 h2 + 3 of each group
      unsigned char* pt = pbuf(slot);
      const bool need_mask = (p.causal && r0 < kw0 + 31) || (r0 + BN > N) || (kw0 + 31 >= N);
  #pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        const f32x16_t sc = row_product(qt, rb);
        u32x4_t pp[2];
        auto make_p = [&](auto masked) __attribute__((always_inline)) {
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row4 = rb * 32 + 8 * r + 4 * h2;  // first of this lane's 4 rows in group r
            const f32x4_t l2 = *(const f32x4_t*)(st + (rb * 32 + 8 * r) * 4);
            float pv[4];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              float pe = __builtin_amdgcn_exp2f(fmaf(sc[4 * r + i], c2, -l2[i]));
              if constexpr (decltype(masked)::value) {
                const int qrow = r0 + row4 + i;
                const unsigned vis = (unsigned)(qrow < N) & (unsigned)(kj < N) & (unsigned)(!p.causal | (kj <= qrow));
                pe = __uint_as_float(__float_as_uint(pe) & (0u - vis));
              }
              pv[i] = pe;
            }
            const int kk = r >> 1, wd = (r & 1) * 2;
            pp[kk][wd] = pack_bf16x2(pv[0], pv[1]);
            pp[kk][wd + 1] = pack_bf16x2(pv[2], pv[3]);
          }
        };
        if (need_mask)
          make_p(std::true_type{});
        else
          make_p(std::false_type{});
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk) *(u32x4_t*)(pt + (rb * 2 + kk) * 1024 + hand) = pp[kk];
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
          for (int db = 0; db < C::DB; ++db) grad[db] = mfma_32x32x16(tr_read(dt, rb * 2 + kk, db), pp[kk], grad[db]);
      }
    };

    // dS wave, slot j - 1: dS = P (dP - D) with P from LDS, dK^T += Q^T dS
    auto ds_finish = [&](int slot) __attribute__((always_inline)) {
      const unsigned char* qt = qbuf(slot);
      const unsigned char* st = sbuf(slot) + h2 * 16;
      const unsigned char* pt = pbuf(slot);
  #pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        u32x4_t pw[2], ds[2];
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk) pw[kk] = *(const u32x4_t*)(pt + (rb * 2 + kk) * 1024 + hand);
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4_t dd = *(const f32x4_t*)(st + 256 + (rb * 32 + 8 * r) * 4);
          const int kk = r >> 1, wd = (r & 1) * 2;
          float dsv[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned word = pw[kk][wd + (i >> 1)];
            const float pe = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
            dsv[i] = pe * (dp[rb][4 * r + i] - dd[i]);
          }
          ds[kk][wd] = pack_bf16x2(dsv[0], dsv[1]);
          ds[kk][wd + 1] = pack_bf16x2(dsv[2], dsv[3]);
        }
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
          for (int db = 0; db < C::DB; ++db) grad[db] = mfma_32x32x16(tr_read(qt, rb * 2 + kk, db), ds[kk], grad[db]);
      }
    };
    // dS wave, slot j: dP = dO V^T, kept for the next slot
    auto ds_start = [&](int slot) __attribute__((always_inline)) {
      const unsigned char* dt = dbuf(slot);
  #pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) dp[rb] = row_product(dt, rb);
    };

    // ---- the stream: slot j+1 is copied during slot j (into the buffer of
    // slot j-2, which the dS wave finished in slot j-1); every copy has landed
    // at the barrier that ends the slot (__syncthreads waits for them). The two
    // roles run separate copies of the loop (the same barriers in the same
    // order), so each copy's registers are allocated for its own live values.
    if (n_slots > 0) issue(0);
    wait_vmcnt<0>();
    __syncthreads();
    if (!ds_wave) {
      for (int j = 0; j <= n_slots; ++j) {
        if (j + 1 < n_slots) issue(j + 1);
        if (j < n_slots && live(j)) p_step(j);
        wait_vmcnt<0>();
        __syncthreads();
      }
    } else {
      for (int j = 0; j <= n_slots; ++j) {
        if (j + 1 < n_slots) issue(j + 1);
        if (j > 0 && live(j - 1)) ds_finish(j - 1);
        if (j < n_slots && live(j)) ds_start(j);
        wait_vmcnt<0>();
        __syncthreads();
      }
    }

    // ---- epilogue: dV = dV^T (P wave), dK = scale dK^T (dS wave), bf16 rows through LDS
    unsigned char* const ost = lds + wave * 32 * C::OROW;
    constexpr int RPI_O = 64 / C::CPR;
    const float m = ds_wave ? p.scale : 1.f;
  #pragma unroll
    for (int db = 0; db < C::DB; ++db)
  #pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        u32x2_t pk;
        pk[0] = pack_bf16x2(grad[db][vq * 4 + 0] * m, grad[db][vq * 4 + 1] * m);
        pk[1] = pack_bf16x2(grad[db][vq * 4 + 2] * m, grad[db][vq * 4 + 3] * m);
        *(u32x2_t*)(ost + c * C::OROW + (db * 32 + vq * 8 + h2 * 4) * 2) = pk;
      }
    __builtin_amdgcn_wave_barrier();
    __bf16* og = (__bf16*)(ds_wave ? p.dk : p.dv) + b * p.k_sb + kvh * p.k_sh;
  #pragma unroll
    for (int i = 0; i < 32 / RPI_O; ++i) {
      const int r = i * RPI_O + lane / C::CPR, ch = lane % C::CPR;
      const u32x4_t val = *(const u32x4_t*)(ost + r * C::OROW + ch * 16);
      if (kw0 + r < N) *(u32x4_t*)(og + (long long)(kw0 + r) * p.k_sn + ch * 8) = val;
    }
  };  // run_block

  run_block(item, true);
  const int second = n_kblk - 1 - item;
  if (second != item) {
    __syncthreads();  // the epilogue's staging area overlaps the ring
    run_block(second, false);
  }
}

// ---------------------------------------------------------------------------
// dQ. Work item = (b, h, query block of 32*NW rows); streams the K and V tiles
// of the block's KV head up to the causal limit, like the forward.
template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdParams p, int n_qblk) {
  using C = BCfg<D, NW, BN>;
  constexpr int LDS_MAIN = 2 * C::BREG;
  constexpr int LDS_OUT = NW * 32 * C::OROW;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT];

  const int g = p.Hq / p.Hkv;
  const int N = p.N;
  const int w = xcd_remap(blockIdx.x, p.B * p.Hq * n_qblk);
  const int per_pair = n_qblk * g;
  const int pair = w / per_pair;
  const int rem = w - pair * per_pair;
  const int qblk = n_qblk - 1 - rem / g;  // heaviest causal blocks first
  const int hg = rem - (rem / g) * g;
  const int kvh = pair / p.B, b = pair - kvh * p.B;
  const int h = kvh * g + hg;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h2 = lane >> 5;
  const int q_blk0 = qblk * NW * 32;
  const int qw0 = q_blk0 + wave * 32;
  const int qi = qw0 + c;
  const float c2 = p.scale_log2;

  // Q and dO of this lane's row as B operands; D = sum_d dO O of the row
  // (each lane half holds half of the dimensions) and lse2 = lse log2(e),
  // also written to the workspace for the dK/dV kernel, which runs after
  // this one (padding rows up to Npad get 0)
  u32x4_t qreg[C::KS], doreg[C::KS];
  float l2, dd;
  {
    const int qc = min(qi, N - 1);
    const long long off = b * p.q_sb + (long long)qc * p.q_sn + h * p.q_sh;
    u32x4_t oreg[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      qreg[s] = *(const u32x4_t*)((const __bf16*)p.q + off + s * 16 + h2 * 8);
      doreg[s] = *(const u32x4_t*)((const __bf16*)p.dout + off + s * 16 + h2 * 8);
      oreg[s] = __builtin_nontemporal_load((const u32x4_t*)((const __bf16*)p.o + off + s * 16 + h2 * 8));
    }
    const long long bh = (long long)b * p.Hq + h;
    l2 = p.lse[bh * N + qc] * kLog2e;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part += __builtin_bit_cast(float, oreg[s][e] << 16) * __builtin_bit_cast(float, doreg[s][e] << 16);
        part += __builtin_bit_cast(float, oreg[s][e] & 0xffff0000u) * __builtin_bit_cast(float, doreg[s][e] & 0xffff0000u);
      }
    dd = halves_sum(part);
    if (h2 == 0 && qi < p.Npad) {
      p.dvec[bh * p.Npad + qi] = qi < N ? dd : 0.f;
      p.lse2[bh * p.Npad + qi] = qi < N ? l2 : 0.f;
    }
  }
  f32x16_t dq[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;

  const int q_last = min(q_blk0 + NW * 32, N) - 1;
  const int k_tiles = (N + BN - 1) / BN;
  const int n_tiles = p.causal ? min(k_tiles, q_last / BN + 1) : k_tiles;
  const int wave_tiles = (qw0 >= N) ? 0 : (p.causal ? min(n_tiles, (qw0 + 31) / BN + 1) : n_tiles);

  // ring slot t holds K at kbuf(t) and V right after it, at kbuf(t) + TILE, so
  // the K and V reads of one lane share an address register and differ by an
  // immediate offset; the slot's base goes through an empty asm statement so
  // that it is formed once per tile in a scalar register (left to itself the
  // compiler forms every (slot, lane offset) sum in a vector register)
  auto kbuf = [&](int t) __attribute__((always_inline)) {
    unsigned off = (unsigned)(t % C::NBUF) * (2 * C::TILE);
    asm volatile("" : "+s"(off));
    return lds + off;
  };
  auto vbuf = [&](int t) __attribute__((always_inline)) { return kbuf(t) + C::TILE; };
  const int ld_row = lane / C::CPR, ld_pos = lane % C::CPR;
  const unsigned row_bytes = (unsigned)p.k_sn * 2u;
  unsigned ld_off[C::IPW];
#pragma unroll
  for (int u = 0; u < C::IPW; ++u) {
    const int row = (wave + u * NW) * C::RPI + ld_row;
    ld_off[u] = (unsigned)row * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
  }
  constexpr int kLoads = 2 * C::IPW;
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    const char* kt = (const char*)((const __bf16*)p.k + b * p.k_sb + kvh * p.k_sh) + (long long)k0 * row_bytes;
    const char* vt = (const char*)((const __bf16*)p.v + b * p.k_sb + kvh * p.k_sh) + (long long)k0 * row_bytes;
    const bool ragged = k0 + BN > N;
#pragma unroll
    for (int u = 0; u < C::IPW; ++u) {
      const int i = wave + u * NW;
      if (C::LPT < NW && i >= C::LPT) break;
      unsigned off = ld_off[u];
      if (ragged) {
        const int row = i * C::RPI + ld_row;
        off = (unsigned)(min(k0 + row, N - 1) - k0) * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
      }
      load_to_lds(kt + off, kbuf(t) + i * 1024);
      load_to_lds(vt + off, vbuf(t) + i * 1024);
    }
  };
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {
    if (n >= 2)
      wait_vmcnt<2 * kLoads>();
    else if (n == 1)
      wait_vmcnt<kLoads>();
    else
      wait_vmcnt<0>();
  };

  unsigned rpart[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) rpart[s] = (unsigned)(c * C::ROWB + (((2 * s + h2) ^ swz<C::CPR>(c)) * 16));
  unsigned tpart[2][C::DB];
  {
    const int tr_t = (lane >> 2) & 3, tr_u = lane & 3, tr_g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int row = 8 * r + 4 * h2 + tr_t;
        const int d = db * 32 + 16 * tr_g + 4 * tr_u;
        tpart[r][db] = (unsigned)(row * C::ROWB + ((d >> 3) ^ swz<C::CPR>(row)) * 16 + ((d >> 2) & 1) * 8);
      }
  }
  auto tr_read = [&](const unsigned char* base, int ps, int db) __attribute__((always_inline)) {
    u32x4_t a;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(base + tpart[r][db] + ps * 16 * C::ROWB));
      const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
      a[2 * r] = xx[0];
      a[2 * r + 1] = xx[1];
    }
    return a;
  };

  auto compute = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    const unsigned char* kt = kbuf(t);
    const unsigned char* vt = kt + C::TILE;  // (one base for both)
    const bool need_mask = (p.causal && k0 + BN - 1 > qw0) || (k0 + BN > N);
#pragma unroll
    for (int kb = 0; kb < C::RB; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T: lane (query c) holds keys kb*32 + 8(e/4) + 4 h2 + e%4
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4_t a = *(const u32x4_t*)(kt + rpart[s] + kb * 32 * C::ROWB);
        const u32x4_t v = *(const u32x4_t*)(vt + rpart[s] + kb * 32 * C::ROWB);
        sc = mfma_32x32x16(a, qreg[s], sc);
        dp = mfma_32x32x16(v, doreg[s], dp);
      }
      u32x4_t ds[2];
      auto make_ds = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          float dsv[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int e = 2 * e2 + i;
            float pe = __builtin_amdgcn_exp2f(fmaf(sc[e], c2, -l2));
            if constexpr (decltype(masked)::value) {
              const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * h2 + (e & 3);
              const unsigned vis = (unsigned)(key < N) & (unsigned)(qi < N) & (unsigned)(!p.causal | (key <= qi));
              pe = __uint_as_float(__float_as_uint(pe) & (0u - vis));
            }
            dsv[i] = pe * (dp[e] - dd);
          }
          ds[e2 >> 2][e2 & 3] = pack_bf16x2(dsv[0], dsv[1]);
        }
      };
      if (need_mask)
        make_ds(std::true_type{});
      else
        make_ds(std::false_type{});
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) dq[db] = mfma_32x32x16(tr_read(kt, kb * 2 + kk, db), ds[kk], dq[db]);
    }
  };

  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  if (n_tiles > 2) issue(2);
  wait_tiles_after(min(n_tiles - 1, 2));
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    if (j + 3 < n_tiles) issue(j + 3);
    if (j < wave_tiles) compute(j);
    wait_tiles_after(min(n_tiles - j - 2, 2));
    __syncthreads();
  }

  // ---- epilogue: dQ = scale dQ^T, bf16 rows through LDS ---------------------------
  unsigned char* const ost = lds + wave * 32 * C::OROW;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      u32x2_t pk;
      pk[0] = pack_bf16x2(dq[db][vq * 4 + 0] * p.scale, dq[db][vq * 4 + 1] * p.scale);
      pk[1] = pack_bf16x2(dq[db][vq * 4 + 2] * p.scale, dq[db][vq * 4 + 3] * p.scale);
      *(u32x2_t*)(ost + c * C::OROW + (db * 32 + vq * 8 + h2 * 4) * 2) = pk;
    }
  __builtin_amdgcn_wave_barrier();
  __bf16* og = (__bf16*)p.dq + b * p.q_sb + h * p.q_sh;
  constexpr int RPI_O = 64 / C::CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI_O; ++i) {
    const int r = i * RPI_O + lane / C::CPR, ch = lane % C::CPR;
    const u32x4_t val = *(const u32x4_t*)(ost + r * C::OROW + ch * 16);
    if (qw0 + r < N) *(u32x4_t*)(og + (long long)(qw0 + r) * p.q_sn + ch * 8) = val;
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  constexpr int NPK = 4, NWQ = 8, BN = 64;
  {  // dQ first: it also writes D and lse2 for the dK/dV kernel
    const int n_qblk = (p.N + NWQ * 32 - 1) / (NWQ * 32);
    const long long total = (long long)p.B * p.Hq * n_qblk;
    if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ, BN>), dim3((unsigned)total), dim3(NWQ * 64), 0, stream, p,
                       n_qblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kblk = (p.N + NPK * 32 - 1) / (NPK * 32);
    const long long total = (long long)p.B * p.Hkv * ((n_kblk + 1) / 2);
    if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NPK, BN>), dim3((unsigned)total), dim3(2 * NPK * 64), 0, stream, p,
                       n_kblk);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdParams& p, int d, hipStream_t stream) {
  if (d == 128) return launch_bwd_d<128>(p, stream);
  if (d == 64) return launch_bwd_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
