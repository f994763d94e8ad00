// Single-token decode against a paged KV cache, split along the context and
// merged by log-sum-exp.
//
// Operator: for sequence b with L cached tokens and query head h,
//   o = sum_{t<L} softmax_t(scale * q . k_t) v_t,   kv head = floor(h / g),
// the query being the newest token, whose K/V are already cached ("USAAIO
// Lesson 90", KV-cache worked example; SDPA definition and GQA rule of
// "Module 5. Modern Attention Mechanisms", sections 4 and 6). Token t of a
// sequence lives in physical page block_table[b][t / 16] at slot t % 16, and a
// page holds [16][Hkv][d] ("Module 09: Efficient Attention", section "Paged
// Attention", subsection "Code: A Paged KV Cache from Scratch").
//
// Flash-Decoding ("inference-attention", section "FlashDecoding"): the pages
// of a sequence are cut into num_splits contiguous ranges. Kernel 1 turns each
// range into a partial (max m, sum l, unnormalised O) for every query head;
// kernel 2 rescales the partials by 2^(m_s - M) and sums them, the same
// rescaling the online softmax applies between tiles.
//
// Mapping onto CDNA4 (decode streams every cached byte once, so the design
// goal is the memory access pattern, not arithmetic):
//  * A "unit" is one KV head together with a group of <= 16 of its query
//    heads. A work-group is 8 independent waves, one unit each, all on the
//    same (sequence, split): the 8 waves walk the same pages in the same
//    order, so each page (all KV heads of 16 tokens) is read by one CU at
//    about the same time, as whole contiguous rows. The K/V of a page slice
//    are read from HBM once and shared by all query heads of the unit.
//  * K and V are loaded in 16-byte chunks laid out along the slot rows, so
//    every load instruction covers whole 2*D-byte rows (whole cache lines),
//    and staged through per-wave LDS regions. (Loading K straight into the
//    MFMA operand layout makes each instruction touch half of 16 different
//    lines; a streaming probe of the two patterns ran 5.8 against 7.0 TB/s,
//    and the long-context decode 311 -> 300 us with the staged K.)
//  * Scores for a page are S^T (16 slots x 16 heads) = K q^T with
//    v_mfma_f32_16x16x32_bf16, the K operand read back from LDS. Unused head
//    columns carry q = 0.
//  * V is read back transposed for O^T (d x heads) += V^T P^T with
//    v_mfma_f32_16x16x16_bf16; slots past the end of the sequence are
//    staged as zeros so that a NaN left in an unused slot cannot reach the
//    output (0 * NaN would).
//  * K and V are read with non-temporal loads: every cached byte is read once
//    per call, so it should not displace what other kernels keep in the
//    caches (measured: 330 -> 313 us for the long-context decode).
//  * Each wave issues the loads of the next ATTN_DECODE_PREFETCH pages before
//    it consumes the current one, and caches its next 64 block-table entries
//    in one register (lane t holds entry t), so no load waits on a table
//    lookup. (As compiled, the waits for the current page also take most of
//    the next page's loads; builds that keep them in flight measured slower.)
//  * Every wave writes its own partial; the split boundaries depend only on
//    logical page numbers, so the result is independent of where the pages
//    sit in the pool.
#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int PAGE = 16;
constexpr int NWU = 8;  // waves (units) per work-group

#ifndef ATTN_DECODE_WAVES_PER_SIMD
#define ATTN_DECODE_WAVES_PER_SIMD 2
#endif
#ifndef ATTN_DECODE_PREFETCH
#define ATTN_DECODE_PREFETCH 1
#endif

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
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

// Element offset of (physical page, slot, KV head, dim 0) in a
// [num_pages][16][Hkv][D] pool. Shared by the decode and the gather kernels.
__device__ __forceinline__ long long kv_row_offset(int phys, int slot, int kvh, int Hkv, int D) {
  return ((long long)phys * PAGE + slot) * Hkv * D + (long long)kvh * D;
}

template <int D>
struct DCfg {
  static constexpr int KS = D / 32;              // k-steps of S^T = K q^T
  static constexpr int DB = D / 16;              // 16-row blocks of O^T
  static constexpr int VROW = D * 2 + 16;        // bytes per slot row of a staged V page
  static constexpr int VCH = PAGE * D / 8 / 64;  // 16-byte V chunks per lane per page
  static constexpr int VPAGE = PAGE * VROW;      // bytes of one staged V page
};

template <int D>
__global__ __launch_bounds__(NWU * 64, ATTN_DECODE_WAVES_PER_SIMD) void decode_split_kernel(DecodeParams p, int HG) {
  using C = DCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * NWU * C::VPAGE];

  const int S = p.num_splits;
  const int units = p.Hkv * HG;
  const int UG = (units + NWU - 1) / NWU;
  int w = blockIdx.x;
  const int split = w % S;
  w /= S;
  const int ug = w % UG;
  const int b = w / UG;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int unit = ug * NWU + wave;
  if (unit >= units) return;  // no barrier below: idle waves may leave
  const int kvh = unit / HG;
  const int hgrp = unit - kvh * HG;

  const int g = p.Hq / p.Hkv;
  const int j = lane & 15;   // head column (B operand, S^T and O^T columns)
  const int rg = lane >> 4;  // row group: key slots rg*4..rg*4+3 of S^T, dims of O^T
  const int head_local = hgrp * 16 + j;
  const bool head_ok = head_local < g;
  const int h = kvh * g + head_local;

  // Visited logical pages: [0, np) or, with a window W, the pages holding the
  // n_sink initial positions, [0, sp), then the window's pages, [wp0, np).
  // The splits cut the visited pages (numbered 0 .. nv-1) into ranges.
  const int L = p.seq_lens[b];
  const int np = (L + PAGE - 1) / PAGE;
  int sp = 0, wp0 = 0;
  if (p.window > 0) {
    wp0 = max(L - p.window, 0) / PAGE;
    sp = min((p.n_sink + PAGE - 1) / PAGE, wp0);
  }
  const int nv = sp + (np - wp0);
  const int pps = (nv + S - 1) / S;
  const int v_begin = min(nv, split * pps);
  const int v_end = min(nv, v_begin + pps);
  auto page_of = [&](int vi) { return vi < sp ? vi : wp0 + (vi - sp); };
  // token t is visible iff t < L and (t >= lo_t or t < n_sink)
  const int lo_t = p.window > 0 ? L - p.window : 0;

  const __bf16* __restrict__ kp = (const __bf16*)p.k_pages;
  const __bf16* __restrict__ vp = (const __bf16*)p.v_pages;
  const int32_t* __restrict__ table = p.block_table + (long long)b * p.max_pages_per_seq;

  // q^T operand: lane holds q[head j][s*32 + rg*8 .. +7]
  u32x4_t qreg[C::KS];
  {
    const __bf16* qg = (const __bf16*)p.q + ((long long)b * p.Hq + (head_ok ? h : 0)) * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qreg[s] = head_ok ? *(const u32x4_t*)(qg + s * 32 + rg * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }

  f32x4_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  unsigned char* const vst = lds + wave * C::VPAGE;
  unsigned char* const kst = lds + (NWU + wave) * C::VPAGE;

  // Block-table entries of this wave's pages, 64 at a time in one VGPR (lane t
  // holds the entry of page tbase + t), so a page's loads never wait on a
  // dependent scalar load of its table entry.
  int tcache = 0, tbase = -64;
  auto phys_of = [&](int pg) {
    if (pg - tbase >= 64) {
      tbase = pg;
      const int mine = pg + lane;
      tcache = mine < np ? table[mine] : 0;
    }
    return __builtin_amdgcn_readlane(tcache, pg - tbase);
  };
  auto load_page = [&](int pg, u32x4_t (&kr)[C::VCH], u32x4_t (&vr)[C::VCH]) {
    const int phys = phys_of(pg);
    // K and V both as whole 16-byte chunks of consecutive slot rows (each
    // load instruction covers 64 / (D / 8) slots x 2 D bytes, whole cache lines)
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = lane + 64 * i;
      const int slot = ch / (D / 8), dch = ch - slot * (D / 8);
      kr[i] = __builtin_nontemporal_load((const u32x4_t*)(kp + kv_row_offset(phys, slot, kvh, p.Hkv, D) + dch * 8));
      vr[i] = __builtin_nontemporal_load((const u32x4_t*)(vp + kv_row_offset(phys, slot, kvh, p.Hkv, D) + dch * 8));
    }
  };

  // consume one page whose K and V are already in registers
  auto consume = [&](int pg, const u32x4_t (&kr)[C::VCH], const u32x4_t (&vr)[C::VCH]) {
    const int valid = min(PAGE, L - pg * PAGE);  // slots of this page that hold tokens
    const int lo_slot = lo_t - pg * PAGE, sink_slot = p.n_sink - pg * PAGE;
    auto visible = [&](int slot) { return slot < valid && (slot >= lo_slot || slot < sink_slot); };
    // stage K as it is and V with zeros in slots that are not visible
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = lane + 64 * i;
      const int slot = ch / (D / 8), dch = ch - slot * (D / 8);
      *(u32x4_t*)(kst + slot * C::VROW + dch * 16) = kr[i];
      const u32x4_t val = visible(slot) ? vr[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t*)(vst + slot * C::VROW + dch * 16) = val;
    }
    __builtin_amdgcn_wave_barrier();

    // S^T = K q^T : lane holds slots rg*4 + e for head j; K operand: slot j,
    // dims s*32 + rg*8 .. +7
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      sacc = mfma_16x16x32(*(const u32x4_t*)(kst + j * C::VROW + s * 64 + rg * 16), qreg[s], sacc);

    float sv[4];
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = rg * 4 + e;
      sv[e] = visible(slot) ? sacc[e] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    u32x2_t pb;
    pb[0] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[0] - m_use), __builtin_amdgcn_exp2f(sv[1] - m_use));
    pb[1] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2] - m_use), __builtin_amdgcn_exp2f(sv[3] - m_use));
    // partial over this lane's 4 slots; summed over row groups at the end
    l_run = add_bf16x2(pb[1], add_bf16x2(pb[0], l_run * alpha));

    __builtin_amdgcn_wave_barrier();
    // O^T += V^T P^T : A = V^T rows d = db*16 + j, keys rg*4 .. rg*4+3
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const unsigned short* col = (const unsigned short*)(vst + (db * 16 + j) * 2);
      const unsigned v0 = col[(rg * 4 + 0) * (C::VROW / 2)];
      const unsigned v1 = col[(rg * 4 + 1) * (C::VROW / 2)];
      const unsigned v2 = col[(rg * 4 + 2) * (C::VROW / 2)];
      const unsigned v3 = col[(rg * 4 + 3) * (C::VROW / 2)];
      u32x2_t a;
      a[0] = v0 | (v1 << 16);
      a[1] = v2 | (v3 << 16);
      oacc[db] = mfma_16x16x16(a, pb, oacc[db] * alpha);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Walk the split's pages, the next ATTN_DECODE_PREFETCH pages' loads issued
  // ahead; the register buffers rotate by unrolling, so they are never
  // indexed at run time.
  int vi = v_begin;
#if ATTN_DECODE_PREFETCH == 1
  u32x4_t ka[C::VCH], va[C::VCH], kb[C::VCH], vb[C::VCH];
  if (vi < v_end) load_page(page_of(vi), ka, va);
  while (vi < v_end) {
    if (vi + 1 < v_end) load_page(page_of(vi + 1), kb, vb);
    consume(page_of(vi), ka, va);
    if (++vi >= v_end) break;
    if (vi + 1 < v_end) load_page(page_of(vi + 1), ka, va);
    consume(page_of(vi), kb, vb);
    ++vi;
  }
#else
  u32x4_t ka[C::VCH], va[C::VCH], kb[C::VCH], vb[C::VCH], kc[C::VCH], vc[C::VCH];
  if (vi < v_end) load_page(page_of(vi), ka, va);
  if (vi + 1 < v_end) load_page(page_of(vi + 1), kb, vb);
  while (vi < v_end) {
    if (vi + 2 < v_end) load_page(page_of(vi + 2), kc, vc);
    consume(page_of(vi), ka, va);
    if (++vi >= v_end) break;
    if (vi + 2 < v_end) load_page(page_of(vi + 2), ka, va);
    consume(page_of(vi), kb, vb);
    if (++vi >= v_end) break;
    if (vi + 2 < v_end) load_page(page_of(vi + 2), kb, vb);
    consume(page_of(vi), kc, vc);
    ++vi;
  }
#endif

  // the row groups each summed 4 of the 16 slots of every page
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- this wave's partial for (b, head, split) ------------------------------------
  if (head_ok) {
    const long long slot = ((long long)b * p.Hq + h) * S + split;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      *(f32x4_t*)(p.ws_o + slot * D + db * 16 + rg * 4) = oacc[db];
    if (rg == 0) {
      p.ws_ml[slot * 2 + 0] = m_run;
      p.ws_ml[slot * 2 + 1] = l_run;
    }
  }
}

// Merge the split partials of one (sequence, query head): M = max_s m_s,
// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s; zero when no split saw a key.
// One 256-thread work-group per (sequence, head): the split weights are
// computed once, in parallel; then 256/D groups of D threads each sum every
// (256/D)-th split for one output dim, and the group sums are added in a fixed
// order (so the result does not depend on timing).
constexpr int MERGE_MAX_SPLITS = 1024;
constexpr int MERGE_THREADS = 256;
template <int D>
__global__ __launch_bounds__(MERGE_THREADS) void decode_merge_kernel(DecodeParams p) {
  constexpr int G = MERGE_THREADS / D;  // split groups
  __shared__ float wts[MERGE_MAX_SPLITS];
  __shared__ float red[MERGE_THREADS / 64];
  __shared__ float part[G][D];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int S = p.num_splits;
  const float* ml = p.ws_ml + (long long)bh * S * 2;
  const float* po = p.ws_o + (long long)bh * S * D;

  // a learned sink logit is one more partial: m = s_h, l = 1, O = 0
  const float sink = p.sinks ? p.sinks[bh % p.Hq] * 1.4426950408889634f : kNegInf;
  float M = kNegInf;
  for (int s = tid; s < S; s += MERGE_THREADS) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wv] = M;
  __syncthreads();
  M = fmaxf(red[0], sink);
#pragma unroll
  for (int i = 1; i < MERGE_THREADS / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();

  float den = 0.f;
  for (int s = tid; s < S; s += MERGE_THREADS) {
    const float w = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml[2 * s] - M);
    wts[s] = w;
    den += w * ml[2 * s + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  if (lane == 0) red[wv] = den;
  __syncthreads();
  den = (p.sinks && M != kNegInf) ? __builtin_amdgcn_exp2f(sink - M) : 0.f;
#pragma unroll
  for (int i = 0; i < MERGE_THREADS / 64; ++i) den += red[i];

  const int d = tid % D, grp = tid / D;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int s = grp;
  for (; s + 3 * G < S; s += 4 * G) {
    a0 += wts[s] * po[(long long)s * D + d];
    a1 += wts[s + G] * po[(long long)(s + G) * D + d];
    a2 += wts[s + 2 * G] * po[(long long)(s + 2 * G) * D + d];
    a3 += wts[s + 3 * G] * po[(long long)(s + 3 * G) * D + d];
  }
  for (; s < S; s += G) a0 += wts[s] * po[(long long)s * D + d];
  part[grp][d] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (grp == 0) {
    float num = part[0][d];
#pragma unroll
    for (int i = 1; i < G; ++i) num += part[i][d];
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
    ((__bf16*)p.o)[(long long)bh * D + d] = (__bf16)(num * inv);
  }
}

// Copy token rows out of the page pool through the block table (test aid).
__global__ void gather_kernel(const unsigned char* __restrict__ pages, const int32_t* __restrict__ table,
                              const int32_t* __restrict__ seq_lens, unsigned char* __restrict__ out,
                              int Hkv, int D, int max_pages_per_seq, int max_len, int elem_bytes) {
  const int b = blockIdx.y;
  const int t = blockIdx.x;
  const int L = min(seq_lens[b], max_len);
  if (t >= L) return;
  const int phys = table[(long long)b * max_pages_per_seq + t / PAGE];
  const long long row_bytes = (long long)Hkv * D * elem_bytes;
  const unsigned char* src = pages + kv_row_offset(phys, t % PAGE, 0, Hkv, D) * elem_bytes;
  unsigned char* dst = out + ((long long)b * max_len + t) * row_bytes;
  for (long long i = threadIdx.x * 4; i < row_bytes; i += blockDim.x * 4)
    *(unsigned*)(dst + i) = *(const unsigned*)(src + i);
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const int g = p.Hq / p.Hkv;
  const int HG = (g + 15) / 16;
  const long long units = (long long)p.Hkv * HG;
  const long long total = (long long)p.B * ((units + NWU - 1) / NWU) * p.num_splits;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)total), dim3(NWU * 64), 0, stream, p, HG);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(MERGE_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int auto_decode_splits(int B, int Hkv, int max_pages_per_seq) {
  // One round of work-groups: B * ceil(Hkv / 8) * S work-groups of 8 waves
  // close to (not above) 256, the compute units of an MI355X, each split
  // holding at least 4 pages. Measured on the long-context and batched decode
  // workloads and on the 8192-token window: a round of exactly the CU count
  // beats two rounds, and counts that leave CUs with one work-group more than
  // others run up to 30% slower. A constant, not a device query, keeps the
  // choice (and so the summation order) a function of the arguments only.
  constexpr long long kTargetWorkGroups = 256;
  const long long wgs = (long long)B * ((Hkv + NWU - 1) / NWU);
  long long s = kTargetWorkGroups / wgs;
  const long long cap = max(1, max_pages_per_seq / 4);
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream) {
  if (d == 128) return launch_decode_d<128>(p, stream);
  if (d == 64) return launch_decode_d<64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gather(const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                         void* out, int B, int Hkv, int d, int page_size, int max_pages_per_seq,
                         int max_len, int elem_bytes, hipStream_t stream) {
  (void)page_size;
  hipLaunchKernelGGL(gather_kernel, dim3(max_len, B), dim3(64), 0, stream,
                     (const unsigned char*)pages, block_table, seq_lens, (unsigned char*)out, Hkv, d,
                     max_pages_per_seq, max_len, elem_bytes);
  return hipGetLastError();
}

}  // namespace attn
