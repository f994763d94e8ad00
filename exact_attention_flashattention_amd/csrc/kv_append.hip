// KV append: new tokens' keys and values into the paged cache.
//
// Token t of sequence b lives at (block_table[b, t / 16], t % 16) of the pool
// [pages, 16, Hkv, d] ("Module 09: Efficient Attention", section "Paged
// Attention: The KV Cache as Virtual Memory", subsection "Code: A Paged KV
// Cache from Scratch"); a chunk of c_b new tokens starting at position
// start_pos[b] is written there before the chunk's queries attend to it.
//
// Pure data movement, bound by HBM: each thread moves one 16-byte piece of a
// token row (Hkv * d bf16 values), so consecutive threads read and write
// consecutive bytes of a row; grid.y is the sequence.
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kPage = 16;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint4* __restrict__ k_pages,
    uint4* __restrict__ v_pages, const int32_t* __restrict__ table, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ start_pos, int pieces_per_row, int max_pages_per_seq, int max_new) {
  const int b = blockIdx.y;
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int r = (int)(idx / pieces_per_row);  // new-token index within the sequence
  const int piece = (int)(idx - (long long)r * pieces_per_row);
  const int r0 = cu_new[b];
  const int n = min(cu_new[b + 1] - r0, max_new);
  if (r >= n) return;
  const int t = start_pos[b] + r;  // cache position of the token
  const int page = table[(long long)b * max_pages_per_seq + t / kPage];
  const long long dst = ((long long)page * kPage + (t % kPage)) * pieces_per_row + piece;
  const long long src = (long long)(r0 + r) * pieces_per_row + piece;
  k_pages[dst] = k_new[src];
  v_pages[dst] = v_new[src];
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                            const int32_t* block_table, const int32_t* cu_new,
                            const int32_t* start_pos, int B, int Hkv, int d,
                            int max_pages_per_seq, int max_new, hipStream_t stream) {
  const int pieces = Hkv * d / 8;  // 16-byte pieces per token row
  const long long blocks = ((long long)max_new * pieces + kThreads - 1) / kThreads;
  if (blocks <= 0 || blocks > 0x7fffffffLL || B > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks, (unsigned)B), dim3(kThreads), 0, stream,
                     (const uint4*)k_new, (const uint4*)v_new, (uint4*)k_pages, (uint4*)v_pages,
                     block_table, cu_new, start_pos, pieces, max_pages_per_seq, max_new);
  return hipGetLastError();
}

}  // namespace attn
