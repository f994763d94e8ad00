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
// Three kernels:
//  * bwd_pre: D_i and lse2_i = lse_i * log2(e) per row, into the workspace.
//  * bwd_dkdv: a work-group owns 32 keys per wave of one (b, KV head) and
//    streams the Q and dO tiles (and their D, lse2) of every query head of the
//    group through LDS; dK^T and dV^T stay in registers, so no atomics.
//  * bwd_dq: a work-group owns 32 queries per wave of one (b, h) and streams
//    the K and V tiles, like the forward.
// Both main kernels copy tiles HBM -> LDS with global_load_lds into a ring of
// four buffers (one barrier per tile) and read them with the same XOR swizzle
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
// D_i = sum_d dO_id O_id (fp32) and lse2_i = lse_i * log2(e), rows in
// [B, Hq, Npad] order (Npad = N rounded up to 64; padding rows get 0).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int CPR = D / 8;
  const long long rows = (long long)p.B * p.Hq * p.Npad;
  const long long row = (long long)blockIdx.x * (256 / CPR) + threadIdx.x / CPR;
  const int ch = threadIdx.x % CPR;
  float acc = 0.f, l2 = 0.f;
  if (row < rows) {
    const int i = (int)(row % p.Npad);
    const long long bh = row / p.Npad;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    if (i < p.N) {
      const long long off = b * p.q_sb + (long long)i * p.q_sn + h * p.q_sh + ch * 8;
      const u32x4_t ov = *(const u32x4_t*)((const __bf16*)p.o + off);
      const u32x4_t dv = *(const u32x4_t*)((const __bf16*)p.dout + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += __builtin_bit_cast(float, ov[e] << 16) * __builtin_bit_cast(float, dv[e] << 16);
        acc += __builtin_bit_cast(float, ov[e] & 0xffff0000u) * __builtin_bit_cast(float, dv[e] & 0xffff0000u);
      }
      l2 = p.lse[(bh * p.N) + i] * kLog2e;
    }
  }
#pragma unroll
  for (int o = CPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < rows && ch == 0) {
    p.dvec[row] = acc;
    p.lse2[row] = l2;
  }
}

// ---------------------------------------------------------------------------
// dK and dV. Work item = (KV head, b, key block of 32*NW keys); the streamed
// slots are (query head of the group, query tile) with the tiles that hold a
// query at or after the block's first key (causal) or all tiles.
template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdParams p, int n_kblk) {
  using C = BCfg<D, NW, BN>;
  constexpr int SREG = 2 * C::BREG;              // per-wave copies of (lse2, D) rows
  constexpr int SBUF = NW * 1024;                // one buffer's stats: a 1 KiB copy per wave
  constexpr int LDS_MAIN = SREG + C::NBUF * SBUF;
  constexpr int LDS_OUT = NW * 32 * C::OROW;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT];

  const int g = p.Hq / p.Hkv;
  const int N = p.N;
  const int w = xcd_remap(blockIdx.x, p.B * p.Hkv * n_kblk);
  const int pair = w / n_kblk;                 // (kv head, b), b fastest
  const int kblk = w - pair * n_kblk;
  const int kvh = pair / p.B, b = pair - kvh * p.B;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h2 = lane >> 5;
  const int k_blk0 = kblk * NW * 32;
  const int kw0 = k_blk0 + wave * 32;  // this wave's first key
  const int kj = kw0 + c;              // this lane's key (column of S)
  const float c2 = p.scale_log2;

  // K and V of this lane's key as B operands (k-step s: dims s*16 + h2*8 .. +7)
  u32x4_t kreg[C::KS], vreg[C::KS];
  {
    const int kc = min(kj, N - 1);
    const __bf16* kg = (const __bf16*)p.k + b * p.k_sb + (long long)kc * p.k_sn + kvh * p.k_sh;
    const __bf16* vg = (const __bf16*)p.v + b * p.k_sb + (long long)kc * p.k_sn + kvh * p.k_sh;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      kreg[s] = *(const u32x4_t*)(kg + s * 16 + h2 * 8);
      vreg[s] = *(const u32x4_t*)(vg + s * 16 + h2 * 8);
    }
  }
  f32x16_t dk[C::DB], dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[db][e] = dv[db][e] = 0.f;

  // streamed slots: (query head hg, query tile T - 1 - r). The tiles of a
  // head run from the last one down to the block's first: the work-groups of
  // one (b, KV head) run side by side, and all of them start on the same last
  // tile, so they read the same Q/dO tiles at about the same time and L2
  // serves most of them (HBM reads of this kernel 1.67 GB -> 0.75 GB on the
  // headline backward; ascending order had each group start on its own tile).
  const int T = (N + BN - 1) / BN;
  const int t0 = p.causal ? k_blk0 / BN : 0;
  const int nT = T - t0;
  const int n_slots = g * nT;
  const int w_t0 = (p.causal ? kw0 / BN : 0) - t0;  // this wave's first tile within a head's run
  const bool wave_live = kw0 < N;

  auto qbuf = [&](int s) __attribute__((always_inline)) { return lds + (s % C::NBUF) * C::TILE; };
  auto dbuf = [&](int s) __attribute__((always_inline)) { return lds + C::BREG + (s % C::NBUF) * C::TILE; };
  auto sbuf = [&](int s) __attribute__((always_inline)) { return lds + SREG + (s % C::NBUF) * SBUF + wave * 1024; };

  const int ld_row = lane / C::CPR, ld_pos = lane % C::CPR;
  const unsigned row_bytes = (unsigned)p.q_sn * 2u;
  unsigned ld_off[C::IPW];
#pragma unroll
  for (int u = 0; u < C::IPW; ++u) {
    const int row = (wave + u * NW) * C::RPI + ld_row;
    ld_off[u] = (unsigned)row * row_bytes + (unsigned)(ld_pos ^ swz<C::CPR>(row)) * 16u;
  }
  constexpr int kLoads = 2 * C::IPW + 1;  // Q and dO pieces, plus the stats copy
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const int hg = slot / nT, t = T - 1 - (slot - hg * nT);
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
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {  // all but the n newest slots landed
    if (n >= 2)
      wait_vmcnt<2 * kLoads>();
    else if (n == 1)
      wait_vmcnt<kLoads>();
    else
      wait_vmcnt<0>();
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

  // one streamed slot: the query tile's contribution to this wave's dK, dV
  auto compute = [&](int slot) __attribute__((always_inline)) {
    const int hg = slot / nT, t = T - 1 - (slot - hg * nT);
    const int r0 = t * BN;
    const unsigned char* qt = qbuf(slot);
    const unsigned char* dt = dbuf(slot);
    const unsigned char* st = sbuf(slot);
    const bool need_mask = (p.causal && r0 < kw0 + 31) || (r0 + BN > N) || (kw0 + 31 >= N);
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys:
      // lane (key c) holds query rows rb*32 + 8 (e/4) + 4 h2 + e%4
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const u32x4_t a = *(const u32x4_t*)(qt + rpart[s] + rb * 32 * C::ROWB);
        const u32x4_t d = *(const u32x4_t*)(dt + rpart[s] + rb * 32 * C::ROWB);
        sc = mfma_32x32x16(a, kreg[s], sc);
        dp = mfma_32x32x16(d, vreg[s], dp);
      }
      // P = 2^(S c2 - lse2), dS = P (dP - D); both packed as B operands. The
      // mask is applied only on the tiles that need it (a uniform choice) and
      // with bit operations, so no lane-divergent branch enters the loop.
      u32x4_t pp[2], ds[2];
      auto make_p = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row4 = rb * 32 + 8 * r + 4 * h2;  // first of this lane's 4 rows in group r
          const f32x4_t l2 = *(const f32x4_t*)(st + row4 * 4);
          const f32x4_t dd = *(const f32x4_t*)(st + 256 + row4 * 4);
          float pv[4], dsv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * r + i;
            float pe = __builtin_amdgcn_exp2f(fmaf(sc[e], c2, -l2[i]));
            if constexpr (decltype(masked)::value) {
              const int qrow = r0 + row4 + i;
              const unsigned vis = (unsigned)(qrow < N) & (unsigned)(kj < N) & (unsigned)(!p.causal | (kj <= qrow));
              pe = __uint_as_float(__float_as_uint(pe) & (0u - vis));
            }
            pv[i] = pe;
            dsv[i] = pe * (dp[e] - dd[i]);
          }
          // k-step ps = 2 rb + r/2 holds rows (r even: e 0-7 -> elements 0..3 of
          // the pack, r odd: 4..7); words 2(r&1), 2(r&1)+1
          const int kk = r >> 1, wd = (r & 1) * 2;
          pp[kk][wd] = pack_bf16x2(pv[0], pv[1]);
          pp[kk][wd + 1] = pack_bf16x2(pv[2], pv[3]);
          ds[kk][wd] = pack_bf16x2(dsv[0], dsv[1]);
          ds[kk][wd + 1] = pack_bf16x2(dsv[2], dsv[3]);
        }
      };
      if (need_mask)
        make_p(std::true_type{});
      else
        make_p(std::false_type{});
      // dV^T += dO^T P and dK^T += Q^T dS (rows d, columns this wave's keys)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ps = rb * 2 + kk;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          dv[db] = mfma_32x32x16(tr_read(dt, ps, db), pp[kk], dv[db]);
          dk[db] = mfma_32x32x16(tr_read(qt, ps, db), ds[kk], dk[db]);
        }
      }
    }
  };

  // ---- the stream: issue slot j+3 at the top of iteration j (into the buffer
  // of slot j-1); slot j+1 must have landed before the barrier ending j
  if (n_slots > 0) issue(0);
  if (n_slots > 1) issue(1);
  if (n_slots > 2) issue(2);
  wait_tiles_after(min(n_slots - 1, 2));
  __syncthreads();
  for (int j = 0; j < n_slots; ++j) {
    if (j + 3 < n_slots) issue(j + 3);
    const int r = j % nT;
    if (wave_live && r <= nT - 1 - w_t0) compute(j);
    wait_tiles_after(min(n_slots - j - 2, 2));
    __syncthreads();
  }

  // ---- epilogue: dK = scale dK^T, dV = dV^T, bf16 rows through LDS ----------------
  unsigned char* const ost = lds + wave * 32 * C::OROW;
  constexpr int RPI_O = 64 / C::CPR;
  const float sc_k = p.scale;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const f32x16_t& acc = which ? dv[db] : dk[db];
        const float m = which ? 1.f : sc_k;
        u32x2_t pk;
        pk[0] = pack_bf16x2(acc[vq * 4 + 0] * m, acc[vq * 4 + 1] * m);
        pk[1] = pack_bf16x2(acc[vq * 4 + 2] * m, acc[vq * 4 + 3] * m);
        *(u32x2_t*)(ost + c * C::OROW + (db * 32 + vq * 8 + h2 * 4) * 2) = pk;
      }
    __builtin_amdgcn_wave_barrier();
    __bf16* og = (__bf16*)(which ? p.dv : p.dk) + b * p.k_sb + kvh * p.k_sh;
#pragma unroll
    for (int i = 0; i < 32 / RPI_O; ++i) {
      const int r = i * RPI_O + lane / C::CPR, ch = lane % C::CPR;
      const u32x4_t val = *(const u32x4_t*)(ost + r * C::OROW + ch * 16);
      if (kw0 + r < N) *(u32x4_t*)(og + (long long)(kw0 + r) * p.k_sn + ch * 8) = val;
    }
    __builtin_amdgcn_wave_barrier();
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

  // Q and dO of this lane's row as B operands, and its lse2, D
  u32x4_t qreg[C::KS], doreg[C::KS];
  float l2 = 0.f, dd = 0.f;
  {
    const int qc = min(qi, N - 1);
    const long long off = b * p.q_sb + (long long)qc * p.q_sn + h * p.q_sh;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      qreg[s] = *(const u32x4_t*)((const __bf16*)p.q + off + s * 16 + h2 * 8);
      doreg[s] = *(const u32x4_t*)((const __bf16*)p.dout + off + s * 16 + h2 * 8);
    }
    const long long srow = ((long long)b * p.Hq + h) * p.Npad + qc;
    l2 = p.lse2[srow];
    dd = p.dvec[srow];
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

  auto kbuf = [&](int t) __attribute__((always_inline)) { return lds + (t % C::NBUF) * C::TILE; };
  auto vbuf = [&](int t) __attribute__((always_inline)) { return lds + C::BREG + (t % C::NBUF) * C::TILE; };
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
    const unsigned char* vt = vbuf(t);
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
  constexpr int NWK = 4, NWQ = 8, BN = 64;
  {
    constexpr int CPR = D / 8;
    const long long rows = (long long)p.B * p.Hq * p.Npad;
    const long long blocks = (rows + 256 / CPR - 1) / (256 / CPR);
    if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kblk = (p.N + NWK * 32 - 1) / (NWK * 32);
    const long long total = (long long)p.B * p.Hkv * n_kblk;
    if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NWK, BN>), dim3((unsigned)total), dim3(NWK * 64), 0, stream, p,
                       n_kblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_qblk = (p.N + NWQ * 32 - 1) / (NWQ * 32);
    const long long total = (long long)p.B * p.Hq * n_qblk;
    if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ, BN>), dim3((unsigned)total), dim3(NWQ * 64), 0, stream, p,
                       n_qblk);
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
