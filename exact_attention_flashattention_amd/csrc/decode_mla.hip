// Decode for multi-head latent attention with absorbed projections.
//
// Every cached token is one row [c_t ; k^R_t] (latent d_c = 512, rotary key
// d_r = 64) shared by all query heads, so this is multi-query attention with
// d_k = 576 and d_v = 512, the values being the first 512 columns of the same
// rows ("inference-attention", section "DeepSeek Multi-head Latent
// Attention": attention runs directly over the cached latent vectors once the
// up-projections are absorbed). For sequence b with L cached tokens and head h:
//   o_h = sum_t softmax_t(scale * q_h . row_t) row_t[0:512].
// Token t of a sequence lives in page block_table[b][t / 16] at slot t % 16
// of a [pages][16][576] pool.
//
// Mapping onto CDNA4: a work-group of 8 waves takes one (sequence, split,
// 128-head chunk); wave w owns 16 heads. Each step stages two pages (32
// tokens, 36 KiB) into LDS with global_load_lds, rows padded to 1184 bytes
// (of the strides 1152..1280 with and without XOR swizzles of the 16-byte
// chunks, the one under which the row reads below ran fastest: ~140 B/clk
// per CU against 126 at 1168 and 64 unpadded); a ring of four step buffers
// keeps three steps of loads in flight.
//  * S^T (32 tokens x 16 heads) = K q^T with v_mfma_f32_16x16x32_bf16, A = K
//    rows from LDS, B = the wave's 16 queries (576 dims) held in registers.
//  * Online softmax per head (lane column), with the lazy rescale used by the
//    prefill (the reference max moves only when exceeded by more than 2^8).
//  * O^T (512 x 16 heads) += V^T P^T with the same MFMA: A = V^T from two
//    ds_read_b64_tr_b16 per 16 dims, B = P^T straight from the score lanes
//    (tokens 4g..4g+3 and 16+4g..16+4g+3 for lane group g, in that order).
//  * Rows past the end of the sequence are loaded from its last token (finite)
//    and masked, so a NaN left in an unused slot never meets a zero weight.
// Each (head, split) partial (m, l, O) goes to the workspace; a merge kernel
// combines the splits in a fixed order (Flash-Decoding, "inference-attention",
// section "FlashDecoding").
#include "attn_internal.h"
#include "cdna4.h"

namespace attn {
namespace {

using namespace cdna4;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int DC = 512, DR = 64, DK = DC + DR;
constexpr int PG = 16;                   // tokens per page
constexpr int NWM = 8;                   // waves per work-group (16 heads each)
constexpr int HPW = 16;                  // heads per wave
constexpr int ROWG = DK * 2;             // bytes of a cached row in HBM (1152)
constexpr int ROWP = ROWG + 32;          // bytes of a row in LDS (padded)
constexpr int SLOTS_ROW = ROWP / 16;     // 16-byte slots per LDS row (74)
constexpr int STEP_ROWS = 2 * PG;        // tokens per step
constexpr int STEP_SLOTS = STEP_ROWS * SLOTS_ROW;        // 2368
constexpr int IPW_M = (STEP_SLOTS + 64 * NWM - 1) / (64 * NWM);  // load instructions per wave (5)
constexpr int STEP_BYTES = IPW_M * NWM * 1024;           // one ring buffer (40 KiB)
constexpr int NBUF_M = 4;
constexpr int KS = DK / 32;              // 18 k-steps of S^T
constexpr int VB = DC / 16;              // 32 blocks of 16 dims of O^T
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kTau = 8.0f;

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(NWM * 64, 1) void mla_split_kernel(MlaParams p, int n_hchunk) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF_M * STEP_BYTES];

  const int S = p.num_splits;
  int w = blockIdx.x;
  const int split = w % S;
  w /= S;
  const int hchunk = w % n_hchunk;
  const int b = w / n_hchunk;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hcol = lane & 15;  // head column of S^T / O^T
  const int grp = lane >> 4;   // lane group: rows 4 grp .. 4 grp + 3 of the accumulators
  const int h0 = (hchunk * NWM + wave) * HPW;  // this wave's first head
  const bool wave_live = h0 < p.Hq;
  const int h = h0 + hcol;

  const int L = p.seq_lens[b];
  const int np = (L + PG - 1) / PG;
  int pps = (np + S - 1) / S;
  pps += pps & 1;  // whole steps of two pages
  const int pg_begin = min(np, split * pps);
  const int pg_end = min(np, pg_begin + pps);
  const int n_steps = (pg_end - pg_begin + 1) / 2;
  const int32_t* __restrict__ table = p.block_table + (long long)b * p.max_pages_per_seq;
  const unsigned char* __restrict__ pool = (const unsigned char*)p.kv_pages;

  // q of this lane's head as the B operand (k-step ks: dims ks*32 + grp*8 .. +7)
  u32x4_t qreg[KS];
  {
    const __bf16* qg = (const __bf16*)p.q + ((long long)b * p.Hq + (wave_live ? h : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = *(const u32x4_t*)(qg + ks * 32 + grp * 8);
  }
  f32x4_t oacc[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) oacc[vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_run = 0.f;

  // ---- staging: slot s of a step buffer holds row s / 74, chunk s % 74 ---------
  // (chunks 72 and 73 are the row's padding; slots past the 32 rows are spare). A row
  // past the end of the sequence, or the missing second page of the last
  // step, is loaded from the sequence's last token.
  auto issue = [&](int step) __attribute__((always_inline)) {
    const int pa = pg_begin + 2 * step, pb = pa + 1;
    const int page_a = table[pa];
    const int page_b = pb < pg_end ? table[pb] : page_a;
    const int page_last = table[np - 1];
    const int t_last = L - 1;
    unsigned char* const buf = lds + (step % NBUF_M) * STEP_BYTES;
#pragma unroll
    for (int u = 0; u < IPW_M; ++u) {
      const int i = wave + u * NWM;
      int s = i * 64 + lane;
      if (s >= STEP_SLOTS) s = 0;  // spare slot: a harmless copy of slot 0's source
      const int row = s / SLOTS_ROW;
      int chunk = s - row * SLOTS_ROW;
      if (chunk >= ROWG / 16) chunk = ROWG / 16 - 1;  // padding: any chunk of the row
      const int lp = row < PG ? pa : pb;                   // logical page of the row
      int t = lp * PG + (row & (PG - 1));
      int page = row < PG ? page_a : page_b;
      if (t > t_last || (row >= PG && pb >= pg_end)) {
        t = t_last;
        page = page_last;
      }
      const unsigned char* src = pool + ((long long)page * PG + (t & (PG - 1))) * ROWG + chunk * 16;
      load_to_lds_stream(src, buf + i * 1024);  // each latent row is read once per call
    }
  };

  // per-lane parts of the LDS reads
  const unsigned kpart = (unsigned)(hcol * ROWP + grp * 16);  // row hcol, dims grp*8: S^T A operand
  unsigned tpart[2];                                          // transposed V reads
  {
    const int tt = (lane & 15) >> 2, tu = lane & 3;
#pragma unroll
    for (int r = 0; r < 2; ++r) tpart[r] = (unsigned)((r * 16 + 4 * grp + tt) * ROWP + tu * 8);
  }

  auto compute = [&](int step) __attribute__((always_inline)) {
    const unsigned char* kt = lds + (step % NBUF_M) * STEP_BYTES;
    const int pa = pg_begin + 2 * step, pb = pa + 1;
    // S^T for tokens [pa*16, +16) (block 0) and [pb*16, +16) (block 1)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t a0 = *(const u32x4_t*)(kt + kpart + ks * 64);
      const u32x4_t a1 = *(const u32x4_t*)(kt + 16 * ROWP + kpart + ks * 64);
      s0 = mfma_16x16x32(a0, qreg[ks], s0);
      s1 = mfma_16x16x32(a1, qreg[ks], s1);
    }
    // visibility of this lane's 8 tokens
    const int lim0 = L - pa * PG - 4 * grp;                       // token 4grp+i of block 0 iff i < lim0
    const int lim1 = pb < pg_end ? L - pb * PG - 4 * grp : 0;     // block 1
    float sv[8];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = i < lim0 ? s0[i] * p.scale_log2 : kNegInf;
      sv[4 + i] = i < lim1 ? s1[i] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, fmaxf(sv[i], sv[4 + i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kTau)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) oacc[vb] *= alpha;
    }
    const float neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
    u32x4_t pb4;
    pb4[0] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[0] + neg_m), __builtin_amdgcn_exp2f(sv[1] + neg_m));
    pb4[1] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2] + neg_m), __builtin_amdgcn_exp2f(sv[3] + neg_m));
    pb4[2] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[4] + neg_m), __builtin_amdgcn_exp2f(sv[5] + neg_m));
    pb4[3] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[6] + neg_m), __builtin_amdgcn_exp2f(sv[7] + neg_m));
    l_run = add_bf16x2(pb4[3], add_bf16x2(pb4[2], add_bf16x2(pb4[1], add_bf16x2(pb4[0], l_run))));
    // O^T += V^T P^T, 16 dims at a time
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      u32x4_t a;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(kt + tpart[r] + vb * 32));
        const u32x2_t xx = __builtin_bit_cast(u32x2_t, x);
        a[2 * r] = xx[0];
        a[2 * r + 1] = xx[1];
      }
      oacc[vb] = mfma_16x16x32(a, pb4, oacc[vb]);
    }
  };

  constexpr int kLoads = IPW_M;
  auto wait_after = [&](int n) __attribute__((always_inline)) {  // all but the n newest steps landed
    if (n >= 2)
      wait_vmcnt<2 * kLoads>();
    else if (n == 1)
      wait_vmcnt<kLoads>();
    else
      wait_vmcnt<0>();
  };
  if (n_steps > 0) issue(0);
  if (n_steps > 1) issue(1);
  if (n_steps > 2) issue(2);
  wait_after(min(n_steps - 1, 2));
  __syncthreads();
  for (int j = 0; j < n_steps; ++j) {
    if (j + 3 < n_steps) issue(j + 3);
    if (wave_live) compute(j);
    wait_after(min(n_steps - j - 2, 2));
    __syncthreads();
  }

  // the four lane groups each summed their own tokens
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (wave_live && h < p.Hq) {
    const long long slot = ((long long)b * p.Hq + h) * S + split;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) *(f32x4_t*)(p.ws_o + slot * DC + vb * 16 + grp * 4) = oacc[vb];
    if (grp == 0) {
      p.ws_ml[slot * 2 + 0] = m_ref;
      p.ws_ml[slot * 2 + 1] = l_run;
    }
  }
}

// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, splits in order; zero
// when no split saw a token. One 256-thread work-group per (sequence, head),
// two output dims per thread.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams p) {
  const int bh = blockIdx.x;
  const int S = p.num_splits;
  const float* ml = p.ws_ml + (long long)bh * S * 2;
  const float* po = p.ws_o + (long long)bh * S * DC;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f, a0 = 0.f, a1 = 0.f;
  const int d = threadIdx.x * 2;
  for (int s = 0; s < S; ++s) {
    const float wgt = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml[2 * s] - M);
    den += wgt * ml[2 * s + 1];
    const float2 v = *(const float2*)(po + (long long)s * DC + d);
    a0 += wgt * v.x;
    a1 += wgt * v.y;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *(unsigned*)((__bf16*)p.o + (long long)bh * DC + d) = pack_bf16x2(a0 * inv, a1 * inv);
}

}  // namespace

int mla_auto_splits(int B, int Hq, int max_pages_per_seq) {
  // one round of work-groups, at most 256 (the CU count; one work-group fits
  // a CU), with at least 48 pages (768 tokens) of the table's width per split
  // so that a split's partial (Hq x 514 floats) stays small next to its rows.
  // Measured on the 16-sequence workload: 16 splits (256 work-groups)
  // 105-112 us, 15 splits 107-120 us, 20 to 32 splits 125-135 us.
  const long long chunks = (long long)B * ((Hq + NWM * HPW - 1) / (NWM * HPW));
  long long s = 256 / chunks;
  const long long cap = max(1, max_pages_per_seq / 48);
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode_mla(const MlaParams& p, hipStream_t stream) {
  const int n_hchunk = (p.Hq + NWM * HPW - 1) / (NWM * HPW);
  const long long total = (long long)p.B * n_hchunk * p.num_splits;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_split_kernel, dim3((unsigned)total), dim3(NWM * 64), 0, stream, p, n_hchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)(p.B * p.Hq)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
