// C-ABI entry points: argument validation on the host, then kernel launches.
// Every check happens before anything is enqueued, so an error status means
// no kernel ran and no output was touched.
#include "../../include/attn.h"
#include "attn_internal.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

namespace {

constexpr long long kMaxElems = 1LL << 40;  // sanity bound on any one tensor

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_heads(int Hq, int Hkv) {
  if (Hq < 1 || Hkv < 1) return ATTN_ERR_SHAPE;
  if (Hq % Hkv) return ATTN_ERR_GQA;
  return ATTN_OK;
}

// A variant: window >= 0, n_sink >= 0 only with a window, a window only when
// causal, the sink array 4-byte aligned.
int check_variant(const attn_variant* v, int causal) {
  if (!v) return ATTN_OK;
  if (v->window < 0 || v->n_sink < 0) return ATTN_ERR_SHAPE;
  if (v->n_sink > 0 && v->window == 0) return ATTN_ERR_SHAPE;
  if (v->window > 0 && !causal) return ATTN_ERR_SHAPE;
  if (v->sinks && (reinterpret_cast<uintptr_t>(v->sinks) & 3u)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

bool has_variant(const attn_variant* v) { return v && (v->window > 0 || v->sinks); }

void set_variant(attn::PrefillParams& p, const attn_variant* v) {
  p.window = v ? v->window : 0;
  p.n_sink = v && v->window > 0 ? v->n_sink : 0;
  p.sinks = v ? v->sinks : nullptr;
}

// ---- fixed scratch of attn_decode_noalloc ----------------------------------------
// The split partials of attn_decode_noalloc live in this array instead of a
// caller-supplied workspace. Each GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` is only a stand-in for the
// symbol: its device address is taken once per device with
// hipGetSymbolAddress and kept in scratch_ptr, which is what kernels receive.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream); ATTN_ERR_LAUNCH if the runtime refuses.
int device_scratch(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return ATTN_ERR_LAUNCH;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    // the symbol's address is per device: take it with that device current
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return ATTN_ERR_LAUNCH;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: invalid size or scale";
    case ATTN_ERR_GQA: return "ATTN_ERR_GQA: Hq is not a multiple of Hkv";
    case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM: head dimension must be 64 or 128";
    case ATTN_ERR_DTYPE: return "ATTN_ERR_DTYPE: unsupported element type";
    case ATTN_ERR_LAYOUT: return "ATTN_ERR_LAYOUT: unsupported layout";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace too small";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: kernel launch failed";
    case ATTN_ERR_PAGE: return "ATTN_ERR_PAGE: page_size must be 16";
    case ATTN_ERR_SCRATCH: return "ATTN_ERR_SCRATCH: the call needs more than the fixed scratch of attn_decode_noalloc";
    default: return "unknown attn status";
  }
}

int attn_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int N, int Hq, int Hkv, int d, float scale, int causal,
                    int dtype, int layout, const attn_variant* variant, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || N < 1) return ATTN_ERR_SHAPE;
  int st = check_heads(Hq, Hkv);
  if (st) return st;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (layout != ATTN_BNHD && layout != ATTN_BHND) return ATTN_ERR_LAYOUT;
  if (!isfinite(scale)) return ATTN_ERR_SHAPE;
  if ((long long)B * N * Hq * d > kMaxElems) return ATTN_ERR_SHAPE;
  if ((long long)Hkv * d >= (1 << 24)) return ATTN_ERR_SHAPE;  // key row offsets in a tile fit 32 bits
  if (dtype == ATTN_F32 && (Hq > 65535 || B > 65535)) return ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  st = check_variant(variant, causal);
  if (st) return st;
  if (has_variant(variant) && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;

  attn::PrefillParams p = {};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv;
  const long long D = d;
  if (layout == ATTN_BNHD) {
    p.q_sb = (long long)N * Hq * D; p.q_sn = Hq * D; p.q_sh = D;
    p.k_sb = (long long)N * Hkv * D; p.k_sn = Hkv * D; p.k_sh = D;
  } else {
    p.q_sb = (long long)Hq * N * D; p.q_sn = D; p.q_sh = (long long)N * D;
    p.k_sb = (long long)Hkv * N * D; p.k_sn = D; p.k_sh = (long long)N * D;
  }
  p.o_sb = p.q_sb; p.o_sn = p.q_sn; p.o_sh = p.q_sh;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  set_variant(p, variant);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(p, d, s)
                                          : attn::launch_prefill_f32(p, d, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 int B, int N, int Hq, int Hkv, int d, float scale, int causal, void* stream) {
  return attn_prefill_ex(q, k, v, o, nullptr, B, N, Hq, Hkv, d, scale, causal, ATTN_BF16,
                         ATTN_BNHD, nullptr, stream);
}

int attn_decode_num_splits(int B, int Hkv, int max_pages_per_seq, int num_splits) {
  if (B < 1 || Hkv < 1 || max_pages_per_seq < 1 || num_splits < 0) return ATTN_ERR_SHAPE;
  if (num_splits > 0) {
    int s = num_splits < max_pages_per_seq ? num_splits : max_pages_per_seq;
    return s < 1024 ? s : 1024;  // the merge keeps one weight per split on chip
  }
  return attn::auto_decode_splits(B, Hkv, max_pages_per_seq);
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int d, int max_pages_per_seq,
                                  int num_splits) {
  if (check_heads(Hq, Hkv) || (d != 64 && d != 128)) return 0;
  const int S = attn_decode_num_splits(B, Hkv, max_pages_per_seq, num_splits);
  if (S < 1) return 0;
  return (size_t)B * Hq * S * (d + 2) * sizeof(float);
}

// Validation and launch shared by attn_decode_ex and attn_decode_noalloc.
// With fixed_scratch the workspace is the library's own array: its size
// limit replaces workspace_bytes, and its device address is taken only once
// every argument has passed.
static int decode_enqueue(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens, void* o,
                          int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                          int num_pages, float scale, int num_splits, int dtype,
                          const attn_variant* variant, void* workspace, size_t workspace_bytes,
                          bool fixed_scratch, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o) return ATTN_ERR_NULL;
  if (!fixed_scratch && !workspace) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (B < 1 || max_pages_per_seq < 1 || num_pages < 1 || num_splits < 0) return ATTN_ERR_SHAPE;
  int st = check_heads(Hq, Hkv);
  if (st) return st;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_PAGE;
  if (!isfinite(scale)) return ATTN_ERR_SHAPE;
  if ((long long)max_pages_per_seq * page_size > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)num_pages * page_size * Hkv * d > kMaxElems) return ATTN_ERR_SHAPE;
  if ((long long)B * max_pages_per_seq > kMaxElems) return ATTN_ERR_SHAPE;
  // with a window the automatic split count is taken over the pages a query
  // can see (never more than without it, so the workspace size still fits)
  int split_pages = max_pages_per_seq;
  if (variant && variant->window > 0) {
    const long long vis = ((long long)variant->window + 15) / 16 + 1 + ((long long)variant->n_sink + 15) / 16;
    if (vis < split_pages) split_pages = (int)vis;
  }
  const int S = num_splits > 0 ? attn_decode_num_splits(B, Hkv, max_pages_per_seq, num_splits)
                               : attn_decode_num_splits(B, Hkv, split_pages, 0);
  const size_t need = attn_decode_workspace_size(B, Hq, Hkv, d, max_pages_per_seq, num_splits);
  if (fixed_scratch) {
    if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
  } else if (workspace_bytes < need) {
    return ATTN_ERR_WORKSPACE;
  }
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
      (!fixed_scratch && !aligned16(workspace)) || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return ATTN_ERR_ALIGN;
  st = check_variant(variant, 1);
  if (st) return st;
  if (fixed_scratch) {
    st = device_scratch(reinterpret_cast<hipStream_t>(stream), &workspace);
    if (st) return st;
  }

  attn::DecodeParams p = {};
  p.q = q; p.k_pages = k_pages; p.v_pages = v_pages;
  p.block_table = block_table; p.seq_lens = seq_lens; p.o = o;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + (size_t)B * Hq * S * d;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.max_pages_per_seq = max_pages_per_seq;
  p.num_splits = S;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.window = variant ? variant->window : 0;
  p.n_sink = variant && variant->window > 0 ? variant->n_sink : 0;
  p.sinks = variant ? variant->sinks : nullptr;
  const hipError_t e = attn::launch_decode(p, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_ex(const void* q, const void* k_pages, const void* v_pages,
                   const int32_t* block_table, const int32_t* seq_lens, void* o,
                   int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                   int num_pages, float scale, int num_splits, int dtype,
                   const attn_variant* variant, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return decode_enqueue(q, k_pages, v_pages, block_table, seq_lens, o, B, Hq, Hkv, d, page_size,
                        max_pages_per_seq, num_pages, scale, num_splits, dtype, variant, workspace,
                        workspace_bytes, false, stream);
}

int attn_decode(const void* q, const void* k_pages, const void* v_pages,
                const int32_t* block_table, const int32_t* seq_lens, void* o,
                int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                int num_pages, float scale, int num_splits, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_enqueue(q, k_pages, v_pages, block_table, seq_lens, o, B, Hq, Hkv, d, page_size,
                        max_pages_per_seq, num_pages, scale, num_splits, dtype, nullptr, workspace,
                        workspace_bytes, false, stream);
}

int attn_decode_noalloc(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens, void* o,
                        int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                        int num_pages, float scale, int num_splits, int dtype, void* stream) {
  return decode_enqueue(q, k_pages, v_pages, block_table, seq_lens, o, B, Hq, Hkv, d, page_size,
                        max_pages_per_seq, num_pages, scale, num_splits, dtype, nullptr, nullptr, 0,
                        true, stream);
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                   const int32_t* block_table, const int32_t* cu_new, const int32_t* start_pos,
                   int B, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages,
                   int total_new, int max_new, void* stream) {
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !cu_new || !start_pos)
    return ATTN_ERR_NULL;
  if (B < 1 || B > 65535 || Hkv < 1 || max_pages_per_seq < 1 || num_pages < 1 || total_new < 0 ||
      max_new < 0)
    return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_PAGE;
  if ((long long)total_new * Hkv * d > kMaxElems || (long long)num_pages * page_size * Hkv * d > kMaxElems ||
      (long long)max_pages_per_seq * page_size > 0x7fffffffLL)
    return ATTN_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(cu_new) & 3u) ||
      (reinterpret_cast<uintptr_t>(start_pos) & 3u))
    return ATTN_ERR_ALIGN;
  if (total_new == 0 || max_new == 0) return ATTN_OK;  // nothing to write
  const hipError_t e = attn::launch_kv_append(k_new, v_new, k_pages, v_pages, block_table, cu_new,
                                              start_pos, B, Hkv, d, max_pages_per_seq, max_new,
                                              reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* cu_q, const int32_t* seq_lens,
                       void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                       int max_pages_per_seq, int num_pages, int total_q, int max_q_len,
                       float scale, const attn_variant* variant, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !cu_q || !seq_lens || !o) return ATTN_ERR_NULL;
  if (B < 1 || max_pages_per_seq < 1 || num_pages < 1 || total_q < 0 || max_q_len < 0)
    return ATTN_ERR_SHAPE;
  int st = check_heads(Hq, Hkv);
  if (st) return st;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_PAGE;
  if (!isfinite(scale)) return ATTN_ERR_SHAPE;
  if ((long long)total_q * Hq * d > kMaxElems || (long long)num_pages * page_size * Hkv * d > kMaxElems ||
      (long long)Hkv * d > (1 << 20) || (long long)max_pages_per_seq * page_size > 0x7fffffffLL ||
      (long long)B * max_pages_per_seq > kMaxElems)
    return ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(cu_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGN;
  st = check_variant(variant, 1);
  if (st) return st;
  if (total_q == 0 || max_q_len == 0) return ATTN_OK;  // no query rows

  attn::PrefillParams p = {};
  p.q = q; p.k = k_pages; p.v = v_pages; p.o = o; p.lse = lse;
  p.B = B; p.N = max_q_len; p.Hq = Hq; p.Hkv = Hkv;
  p.q_sn = (long long)Hq * d; p.q_sh = d;
  p.o_sn = p.q_sn; p.o_sh = p.q_sh;
  p.k_sn = (long long)Hkv * d; p.k_sh = d;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = 1;
  p.cu_q = cu_q; p.seq_lens = seq_lens; p.block_table = block_table;
  p.max_pages_per_seq = max_pages_per_seq;
  p.total_q = total_q;
  set_variant(p, variant);
  const hipError_t e = attn::launch_prefill_paged(p, d, max_q_len, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_backward_workspace_size(int B, int N, int Hq) {
  if (B < 1 || N < 1 || Hq < 1) return 0;
  const long long npad = ((long long)N + 63) / 64 * 64;
  return (size_t)(2LL * B * Hq * npad * 4);
}

int attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int N, int Hq, int Hkv, int d,
                  float scale, int causal, int layout, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return ATTN_ERR_NULL;
  if (B < 1 || N < 1) return ATTN_ERR_SHAPE;
  int st = check_heads(Hq, Hkv);
  if (st) return st;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (layout != ATTN_BNHD && layout != ATTN_BHND) return ATTN_ERR_LAYOUT;
  if (!isfinite(scale)) return ATTN_ERR_SHAPE;
  if ((long long)B * N * Hq * d > kMaxElems) return ATTN_ERR_SHAPE;
  if ((long long)Hq * d >= (1 << 24)) return ATTN_ERR_SHAPE;  // row offsets in a tile fit 32 bits
  const size_t need = attn_backward_workspace_size(B, N, Hq);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return ATTN_ERR_ALIGN;

  attn::BwdParams p = {};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.B = B; p.N = N; p.Npad = (N + 63) / 64 * 64; p.Hq = Hq; p.Hkv = Hkv;
  p.dvec = static_cast<float*>(workspace);
  p.lse2 = p.dvec + (size_t)B * Hq * p.Npad;
  const long long D = d;
  if (layout == ATTN_BNHD) {
    p.q_sb = (long long)N * Hq * D; p.q_sn = Hq * D; p.q_sh = D;
    p.k_sb = (long long)N * Hkv * D; p.k_sn = Hkv * D; p.k_sh = D;
  } else {
    p.q_sb = (long long)Hq * N * D; p.q_sn = D; p.q_sh = (long long)N * D;
    p.k_sb = (long long)Hkv * N * D; p.k_sn = D; p.k_sh = (long long)N * D;
  }
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  const hipError_t e = attn::launch_backward(p, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_mla_num_splits(int B, int Hq, int max_pages_per_seq, int num_splits) {
  if (B < 1 || Hq < 1 || max_pages_per_seq < 1 || num_splits < 0) return ATTN_ERR_SHAPE;
  const int cap = max_pages_per_seq < 1024 ? max_pages_per_seq : 1024;
  int s = num_splits > 0 ? num_splits : attn::mla_auto_splits(B, Hq, max_pages_per_seq);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

size_t attn_decode_mla_workspace_size(int B, int Hq, int max_pages_per_seq, int num_splits) {
  const int S = attn_decode_mla_num_splits(B, Hq, max_pages_per_seq, num_splits);
  if (S < 1 || Hq % 16) return 0;
  return (size_t)B * Hq * S * (512 + 2) * 4;
}

int attn_decode_mla(const void* q, const void* kv_pages, const int32_t* block_table, const int32_t* seq_lens,
                    void* o, int B, int Hq, int d_c, int d_r, int page_size, int max_pages_per_seq,
                    int num_pages, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!q || !kv_pages || !block_table || !seq_lens || !o || !workspace) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || max_pages_per_seq < 1 || num_pages < 1 || num_splits < 0) return ATTN_ERR_SHAPE;
  if (Hq % 16) return ATTN_ERR_SHAPE;
  if (d_c != 512 || d_r != 64) return ATTN_ERR_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_PAGE;
  if (!isfinite(scale)) return ATTN_ERR_SHAPE;
  if ((long long)max_pages_per_seq * page_size > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if ((long long)num_pages * page_size * 576 > kMaxElems || (long long)B * max_pages_per_seq > kMaxElems)
    return ATTN_ERR_SHAPE;
  const int S = attn_decode_mla_num_splits(B, Hq, max_pages_per_seq, num_splits);
  if (workspace_bytes < attn_decode_mla_workspace_size(B, Hq, max_pages_per_seq, num_splits))
    return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(kv_pages) || !aligned16(o) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return ATTN_ERR_ALIGN;
  attn::MlaParams p = {};
  p.q = q; p.kv_pages = kv_pages; p.block_table = block_table; p.seq_lens = seq_lens; p.o = o;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + (size_t)B * Hq * S * 512;
  p.B = B; p.Hq = Hq; p.max_pages_per_seq = max_pages_per_seq; p.num_splits = S;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = attn::launch_decode_mla(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_gather_pages(const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                      void* out, int B, int Hkv, int d, int page_size, int max_pages_per_seq,
                      int num_pages, int max_len, int elem_bytes, void* stream) {
  if (!pages || !block_table || !seq_lens || !out) return ATTN_ERR_NULL;
  if (B < 1 || B > 65535 || Hkv < 1 || d < 1 || max_pages_per_seq < 1 || num_pages < 1 ||
      max_len < 1)
    return ATTN_ERR_SHAPE;
  if (page_size != 16) return ATTN_ERR_PAGE;
  if (elem_bytes != 2 && elem_bytes != 4) return ATTN_ERR_DTYPE;
  if (((long long)Hkv * d * elem_bytes) % 4) return ATTN_ERR_SHAPE;
  if (!aligned16(pages) || !aligned16(out)) return ATTN_ERR_ALIGN;
  const hipError_t e = attn::launch_gather(pages, block_table, seq_lens, out, B, Hkv, d, page_size,
                                           max_pages_per_seq, max_len, elem_bytes,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
