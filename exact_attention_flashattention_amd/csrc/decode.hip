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
// goal is bytes in flight, not arithmetic):
//  * One work-group = 4 waves = one (sequence, KV head, group of <= 16 query
//    heads, split). Wave w of the group takes pages first+w, first+w+4, ...
//    so the K/V of each page are read once and shared by all query heads of
//    the GQA group.
//  * Scores for a page are S^T (16 slots x 16 heads) = K q^T with
//    v_mfma_f32_16x16x32_bf16; the K operand is loaded straight from HBM in
//    the MFMA layout (16-byte loads). Unused head columns carry q = 0.
//  * V is staged through a per-wave LDS region and read back transposed for
//    O^T (d x heads) += V^T P^T with v_mfma_f32_16x16x16_bf16; slots past the
//    end of the sequence are written as zeros so that a NaN left in an unused
//    slot cannot reach the output (0 * NaN would).
//  * The next page's K and V loads are issued before the current page is
//    consumed (one page of prefetch per wave, 16 waves per CU).
//  * The 4 wave partials are combined in LDS into one partial per split; the
//    split boundaries depend only on logical page numbers, so the result is
//    independent of where the pages sit in the pool.
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
constexpr int NWD = 4;  // waves per work-group

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
  static constexpr int COMB = NWD * 16 * (D + 2) * 4;  // combine area
  static constexpr int LDS = (NWD * VPAGE > COMB) ? NWD * VPAGE : COMB;
};

template <int D>
__global__ __launch_bounds__(NWD * 64) void decode_split_kernel(DecodeParams p, int HG) {
  using C = DCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS];

  const int S = p.num_splits;
  int w = blockIdx.x;
  const int split = w % S;
  w /= S;
  const int hgrp = w % HG;
  w /= HG;
  const int kvh = w % p.Hkv;
  const int b = w / p.Hkv;

  const int g = p.Hq / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15;   // head column (B operand, S^T and O^T columns)
  const int rg = lane >> 4;  // row group: key slots rg*4..rg*4+3 of S^T, dims of O^T
  const int head_local = hgrp * 16 + j;
  const bool head_ok = head_local < g;
  const int h = kvh * g + head_local;

  const int L = p.seq_lens[b];
  const int np = (L + PAGE - 1) / PAGE;
  const int pps = (np + S - 1) / S;
  const int pg_begin = min(np, split * pps);
  const int pg_end = min(np, pg_begin + pps);

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
  u32x4_t kreg[C::KS], vreg[C::VCH];
  auto load_page = [&](int pg, u32x4_t (&kr)[C::KS], u32x4_t (&vr)[C::VCH]) {
    const int phys = table[pg];
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      kr[s] = *(const u32x4_t*)(kp + kv_row_offset(phys, j, kvh, p.Hkv, D) + s * 32 + rg * 8);
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = lane + 64 * i;
      const int slot = ch / (D / 8), dch = ch - slot * (D / 8);
      vr[i] = *(const u32x4_t*)(vp + kv_row_offset(phys, slot, kvh, p.Hkv, D) + dch * 8);
    }
  };

  int pg = pg_begin + wave;
  if (pg < pg_end) load_page(pg, kreg, vreg);
  for (; pg < pg_end; pg += NWD) {
    u32x4_t kn[C::KS], vn[C::VCH];
    const bool more = pg + NWD < pg_end;
    if (more) load_page(pg + NWD, kn, vn);

    const int valid = min(PAGE, L - pg * PAGE);  // slots of this page that hold tokens
    // stage V (zeros in unused slots)
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ch = lane + 64 * i;
      const int slot = ch / (D / 8), dch = ch - slot * (D / 8);
      const u32x4_t val = slot < valid ? vreg[i] : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t*)(vst + slot * C::VROW + dch * 16) = val;
    }

    // S^T = K q^T : lane holds slots rg*4 + e for head j
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) sacc = mfma_16x16x32(kreg[s], qreg[s], sacc);

    float sv[4];
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = rg * 4 + e;
      sv[e] = slot < valid ? sacc[e] * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    u32x2_t pb;
    float rs;
    {
      const float p0 = __builtin_amdgcn_exp2f(sv[0] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(sv[1] - m_use);
      const float p2 = __builtin_amdgcn_exp2f(sv[2] - m_use);
      const float p3 = __builtin_amdgcn_exp2f(sv[3] - m_use);
      pb[0] = pack_bf16x2(p0, p1);
      pb[1] = pack_bf16x2(p2, p3);
      rs = __builtin_bit_cast(float, pb[0] << 16) + __builtin_bit_cast(float, pb[0] & 0xffff0000u) +
           __builtin_bit_cast(float, pb[1] << 16) + __builtin_bit_cast(float, pb[1] & 0xffff0000u);
    }
    l_run = l_run * alpha + rs;  // partial over this lane's 4 slots; summed over row groups at the end

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

    if (more) {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) kreg[s] = kn[s];
#pragma unroll
      for (int i = 0; i < C::VCH; ++i) vreg[i] = vn[i];
    }
  }

  // the row groups each summed 4 of the 16 slots of every page
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- combine the NWD wave partials of this split ---------------------------------
  __syncthreads();  // every wave is done with its V staging area
  float* comb = (float*)lds;                 // [NWD][16][D] unnormalised outputs
  float* comb_ml = comb + NWD * 16 * D;      // [NWD][16][2]
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) comb[(wave * 16 + j) * D + db * 16 + rg * 4 + e] = oacc[db][e];
  if (rg == 0) {
    comb_ml[(wave * 16 + j) * 2 + 0] = m_run;
    comb_ml[(wave * 16 + j) * 2 + 1] = l_run;
  }
  __syncthreads();

  const int nheads = min(16, g - hgrp * 16);
  for (int idx = tid; idx < nheads * D; idx += NWD * 64) {
    const int hj = idx / D, d = idx - hj * D;
    float M = kNegInf;
#pragma unroll
    for (int wv = 0; wv < NWD; ++wv) M = fmaxf(M, comb_ml[(wv * 16 + hj) * 2]);
    const float M_use = (M == kNegInf) ? 0.f : M;
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWD; ++wv) {
      const float sc = __builtin_amdgcn_exp2f(comb_ml[(wv * 16 + hj) * 2] - M_use);
      acc += sc * comb[(wv * 16 + hj) * D + d];
      lsum += sc * comb_ml[(wv * 16 + hj) * 2 + 1];
    }
    const int hh = kvh * g + hgrp * 16 + hj;
    const long long slot = ((long long)b * p.Hq + hh) * S + split;
    p.ws_o[slot * D + d] = acc;
    if (d == 0) {
      p.ws_ml[slot * 2 + 0] = M;
      p.ws_ml[slot * 2 + 1] = lsum;
    }
  }
}

// Merge the split partials of one (sequence, query head): M = max_s m_s,
// o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s; zero when no split saw a key.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const int S = p.num_splits;
  const float* ml = p.ws_ml + (long long)bh * S * 2;
  const float* po = p.ws_o + (long long)bh * S * D;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float out = 0.f;
  if (M != kNegInf) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < S; ++s) {
      const float sc = __builtin_amdgcn_exp2f(ml[2 * s] - M);
      num += sc * po[(long long)s * D + d];
      den += sc * ml[2 * s + 1];
    }
    out = num / den;
  }
  ((__bf16*)p.o)[(long long)bh * D + d] = (__bf16)out;
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
  const long long total = (long long)p.B * p.Hkv * HG * p.num_splits;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)total), dim3(NWD * 64), 0, stream, p, HG);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int auto_decode_splits(int B, int Hkv, int max_pages_per_seq) {
  const long long pairs = (long long)B * Hkv;
  long long s = (1024 + pairs - 1) / pairs;
  const long long cap = max(1, max_pages_per_seq / 8);
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
