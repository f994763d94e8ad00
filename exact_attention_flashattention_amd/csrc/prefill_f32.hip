// Causal GQA prefill in fp32 (fp32 inputs, fp32 arithmetic, fp32 output).
//
// Same operator and same streaming recurrence as the bf16 MFMA kernel (the SDPA
// definition of "Module 5. Modern Attention Mechanisms", sections 4 and 6,
// computed with the online softmax of the "FlashAttention" section of the
// "inference-attention" page), but in plain fp32 vector arithmetic: one lane
// per query row, key/value tiles of BN keys staged in LDS and read as
// broadcasts. This path exists for fp32 callers and small problems; it makes
// no use of the matrix cores.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int D, int BN>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillParams p) {
  __shared__ float k_lds[BN][D];
  __shared__ float v_lds[BN][D];
  const int lane = threadIdx.x;
  const int qtile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = p.Hq / p.Hkv;
  const int kvh = h / g;
  const int N = p.N;
  const int qi = qtile * 64 + lane;
  const bool valid = qi < N;

  const float* __restrict__ qg = (const float*)p.q + b * p.q_sb + h * p.q_sh;
  const float* __restrict__ kg = (const float*)p.k + b * p.k_sb + kvh * p.k_sh;
  const float* __restrict__ vg = (const float*)p.v + b * p.k_sb + kvh * p.k_sh;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = valid ? qg[(long long)qi * p.q_sn + e] : 0.f;
    o[e] = 0.f;
  }
  float m = kNegInf, l = 0.f;

  const int q_last = min(qtile * 64 + 63, N - 1);
  const int n_keys = p.causal ? q_last + 1 : N;
  for (int k0 = 0; k0 < n_keys; k0 += BN) {
    __syncthreads();
    for (int idx = lane; idx < BN * D; idx += 64) {
      const int r = idx / D, e = idx - r * D;
      const int key = k0 + r;
      k_lds[r][e] = key < N ? kg[(long long)key * p.k_sn + e] : 0.f;
      v_lds[r][e] = key < N ? vg[(long long)key * p.k_sn + e] : 0.f;
    }
    __syncthreads();
    float s[BN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc = fmaf(q[e], k_lds[j][e], acc);
      const int key = k0 + j;
      const bool vis = key < N && (!p.causal || key <= qi);
      s[j] = vis ? acc * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pj = exp2f(s[j] - m_use);
      rs += pj;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(pj, v_lds[j][e], o[e]);
    }
    l = l * alpha + rs;
  }

  if (valid) {
    float* __restrict__ og = (float*)p.o + b * p.o_sb + h * p.o_sh + (long long)qi * p.o_sn;
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) og[e] = o[e] * inv;
    if (p.lse) p.lse[((long long)b * p.Hq + h) * N + qi] = (m + log2f(l)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream) {
  const dim3 grid((p.N + 63) / 64, p.Hq, p.B);
  if (d == 64)
    hipLaunchKernelGGL((prefill_f32_kernel<64, 32>), grid, dim3(64), 0, stream, p);
  else if (d == 128)
    hipLaunchKernelGGL((prefill_f32_kernel<128, 16>), grid, dim3(64), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace attn
