// Internal interface between the C-ABI shim (attn_abi.hip) and the kernel
// launchers. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// One prefill problem. Strides are in elements; v shares k's strides.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // optional [B, Hq, N] natural-log LSE
  int B, N, Hq, Hkv;
  long long q_sb, q_sn, q_sh;
  long long k_sb, k_sn, k_sh;
  long long o_sb, o_sn, o_sh;
  float scale_log2;  // scale * log2(e): scores are carried in base-2 units
  int causal;
  // Paged variant only: q/o rows of sequence b are cu_q[b] .. cu_q[b+1]-1
  // (strides q_sn/q_sh, o_sn/o_sh; q_sb, o_sb, k_sb unused), k/v are page
  // pools [pages, 16, Hkv, d] with row stride k_sn = Hkv*d and head stride
  // k_sh = d, and sequence b holds seq_lens[b] keys.
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int max_pages_per_seq;
  int total_q;  // lse layout [Hq, total_q]
  // Variants (causal only): window W > 0 keeps keys with 0 <= p_q - p_k < W,
  // plus the first n_sink positions; sinks (fp32 [Hq] or null) is a learned
  // logit per query head with zero value.
  int window;
  int n_sink;
  const float* sinks;
};

// One decode problem (bf16 pages, page_size 16).
struct DecodeParams {
  const void* q;        // [B, Hq, d]
  const void* k_pages;  // [num_pages, 16, Hkv, d]
  const void* v_pages;
  const int32_t* block_table;  // [B, max_pages_per_seq]
  const int32_t* seq_lens;     // [B]
  void* o;                     // [B, Hq, d]
  float* ws_ml;                // [B, Hq, splits, 2]   (m in base-2 units, l)
  float* ws_o;                 // [B, Hq, splits, d]   unnormalised partial outputs
  int B, Hq, Hkv, max_pages_per_seq, num_splits;
  float scale_log2;
  // Variants: window W > 0 keeps tokens t >= L - W plus t < n_sink; sinks
  // (fp32 [Hq] or null) is a learned logit per query head with zero value.
  int window;
  int n_sink;
  const float* sinks;
};

// Backward of the prefill (bf16). q, o, dout, dq share q's strides; k, v,
// dk, dv share k's. lse is the forward's [B, Hq, N] natural-log LSE; dvec and
// lse2 are workspace arrays [B, Hq, Npad] (Npad = N rounded up to 64).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  float* lse2;
  int B, N, Npad, Hq, Hkv;
  long long q_sb, q_sn, q_sh;
  long long k_sb, k_sn, k_sh;
  float scale;
  float scale_log2;
  int causal;
};

// Absorbed-MLA decode: q [B, Hq, 576], pool [pages, 16, 576] (latent 512 then
// rotary key 64), o [B, Hq, 512]; workspace as for decode with d = 512.
struct MlaParams {
  const void* q;
  const void* kv_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* ws_ml;  // [B, Hq, splits, 2]
  float* ws_o;   // [B, Hq, splits, 512]
  int B, Hq, max_pages_per_seq, num_splits;
  float scale_log2;
};

hipError_t launch_decode_mla(const MlaParams& p, hipStream_t stream);
int mla_auto_splits(int B, int Hq, int max_pages_per_seq);

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_pp(const PrefillParams& p, int d, int n_rows, bool paged, hipStream_t stream);
hipError_t launch_backward(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_prefill_paged(const PrefillParams& p, int d, int max_q_len, hipStream_t stream);
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* cu_new,
                            const int32_t* start_pos, int B, int Hkv, int d,
                            int max_pages_per_seq, int max_new, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t stream);
hipError_t launch_gather(const void* pages, const int32_t* block_table,
                         const int32_t* seq_lens, void* out, int B, int Hkv, int d,
                         int page_size, int max_pages_per_seq, int max_len,
                         int elem_bytes, hipStream_t stream);

// Split count chosen when the caller passes 0: one round of work-groups (about
// 256 of them, the CU count), with at least 4 pages per split.
int auto_decode_splits(int B, int Hkv, int max_pages_per_seq);

}  // namespace attn
