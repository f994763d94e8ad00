/*
 * attn.h - exact scaled-dot-product attention for AMD MI355X (gfx950 / CDNA4).
 *
 * Two entry points compute softmax(Q K^T * scale + M) V exactly, in the
 * FlashAttention style (key tiles, online softmax, no N x N matrix in memory):
 *
 *   attn_prefill / attn_prefill_ex : causal (or full) self-attention over a
 *       whole sequence, grouped-query heads (MHA, GQA and MQA by one Hkv dial).
 *   attn_decode : one new query token per sequence against a KV cache stored in
 *       fixed-size pages addressed through a block table, split along the
 *       context and merged by log-sum-exp.
 *   attn_backward : the gradients of the prefill with respect to q, k and v.
 *   attn_decode_mla : decode for multi-head latent attention with absorbed
 *       projections (one shared 576-wide latent row per token).
 *   attn_prefill_paged : a chunk of new queries per sequence against the same
 *       paged cache, each row seeing every key up to its own position (the
 *       attention half of chunked prefill); attn_kv_append writes the chunk's
 *       keys and values into the pages first.
 *
 * Definitions follow these pages (cited by title and section):
 *   [SDPA]  "Module 5. Modern Attention Mechanisms" (vladkulikov.com), section 4
 *           "SDPA, masks, and the square-root scale" (the operator, the additive
 *           0/-inf mask, causality p_k <= p_q, the empty-row policy) and
 *           section 6 "GQA is a grouping invariant" (query head h reads KV head
 *           floor(h / (Hq/Hkv)); Hq must be a multiple of Hkv).
 *   [FA]    "inference-attention" (brunomaga.github.io), section "FlashAttention"
 *           (running max m, running sum l, unnormalised O rescaled by e^(m-m'),
 *           output O / l; tiles entirely above the diagonal are skipped) and
 *           section "FlashDecoding" (the cached keys and values are cut into
 *           ranges along the sequence; each range gives an unnormalised
 *           partial output with its own max and sum, and one more pass merges
 *           the partials after bringing them to a common max).
 *   [PAGED] "Module 09: Efficient Attention" (learnllm.pages.dev), section "Paged
 *           Attention: The KV Cache as Virtual Memory", subsection "Code: A
 *           Paged KV Cache from Scratch": pool (num_blocks, block_size,
 *           num_kv_heads, head_dim); token t of a sequence is at
 *           (block_table[t / block_size], t % block_size).
 *   [KV]    "USAAIO Lesson 90" (naruhodotutoring.com), KV-cache worked example:
 *           a decode step appends its own K/V, then its query attends over
 *           every cached key including itself.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory, keeps no pointer after the call returns and
 *     has no global state, with one exception: the fixed per-device scratch
 *     array of attn_decode_noalloc (see there). Calls are thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). The
 *     call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising. Errors inside kernels (a
 *     device fault) surface at the caller's next synchronisation.
 *   - On any non-zero status nothing has been enqueued and no output has been
 *     written. No C++ exception crosses this interface.
 *   - Every tensor pointer must be 16-byte aligned and dense (no padding
 *     between rows) in the layout stated.
 *   - bf16 is the bfloat16 storage format (1 sign, 8 exponent, 7 mantissa
 *     bits). Products are accumulated in fp32; outputs are rounded to
 *     nearest-even once.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (0 = success, negative = error). */
enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,       /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,      /* a size is <= 0 (or < 0 where 0 is allowed), a size
                                 product overflows, or scale is not finite */
    ATTN_ERR_GQA = -3,        /* Hq is not a multiple of Hkv */
    ATTN_ERR_HEAD_DIM = -4,   /* d is not 64 or 128 */
    ATTN_ERR_DTYPE = -5,      /* unsupported dtype code */
    ATTN_ERR_LAYOUT = -6,     /* unsupported layout code */
    ATTN_ERR_WORKSPACE = -7,  /* workspace_bytes below the size the call needs
                                 (a NULL workspace is ATTN_ERR_NULL) */
    ATTN_ERR_ALIGN = -8,      /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_LAUNCH = -9,     /* the HIP runtime refused a launch */
    ATTN_ERR_PAGE = -10,      /* page_size is not 16 */
    ATTN_ERR_SCRATCH = -11    /* attn_decode_noalloc: the call needs more
                                 scratch than ATTN_NOALLOC_SCRATCH_BYTES */
};

/* Element types. */
enum { ATTN_F32 = 0, ATTN_BF16 = 1 };

/* Prefill layouts for q, k, v and o (the head axis holds Hq heads for q and o,
 * Hkv heads for k and v):
 *   ATTN_BNHD : [B, N, H, d]  token-major (row (b, n) holds all heads)
 *   ATTN_BHND : [B, H, N, d]  head-major                                   */
enum { ATTN_BNHD = 0, ATTN_BHND = 1 };

/*
 * attn_variant - optional changes to the causal mask and the softmax, shared
 * by attn_prefill_ex, attn_prefill_paged and attn_decode_ex (NULL = none).
 *
 * window: 0, or W > 0: a key is visible to a query only if 0 <= p_q - p_k < W
 *         (the window includes the query's own position) [SDPA] sections 4
 *         and 9. Tiles outside every row's window are not visited.
 * n_sink: 0, or S > 0 together with a window: the keys at positions 0..S-1
 *         stay visible to every later query (StreamingLLM's initial-token
 *         anchors, [SDPA] section 10).
 * sinks:  NULL, or a device fp32 [Hq] array: a learned logit s_h per query
 *         head, an extra score column that takes part in the softmax and
 *         contributes no value ([SDPA] section 10):
 *           o = sum_j e^(s_j - m) v_j / (sum_j e^(s_j - m) + e^(s_h - m)),
 *         with m the row max over the visible scores and s_h. The lse output
 *         includes the e^(s_h) term.
 * The window and the initial-token anchors need causal attention.
 */
typedef struct attn_variant {
  int window;
  int n_sink;
  const float* sinks;
} attn_variant;

/*
 * attn_prefill - causal GQA attention over whole sequences, bf16, [B, N, H, d].
 *
 * q: [B, N, Hq, d] bf16;  k, v: [B, N, Hkv, d] bf16;  o: [B, N, Hq, d] bf16 (out).
 * For batch b, query head h and query position i:
 *   o[b,i,h,:] = sum_j P_ij v[b,j,kv,:],  P_i = softmax_j(scale * q[b,i,h,:].k[b,j,kv,:] + M_ij)
 * with kv = floor(h / (Hq/Hkv)) [SDPA section 6] and M_ij = 0 if (causal == 0 or
 * j <= i) else -inf [SDPA section 4]. Queries and keys share the origin
 * (N_q = N_k = N), so every row has at least one visible key. Requires
 * B, N, Hq, Hkv >= 1, d in {64, 128}, finite scale (1/sqrt(d) is the usual
 * choice). Equivalent to attn_prefill_ex(..., lse = NULL, ATTN_BF16, ATTN_BNHD).
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 int B, int N, int Hq, int Hkv, int d, float scale, int causal,
                 void* stream);

/*
 * attn_prefill_ex - as attn_prefill, with the element type, the layout and an
 * optional log-sum-exp output made explicit.
 *
 * dtype:  ATTN_BF16 (bf16 in, fp32 accumulation, bf16 out, MFMA path) or
 *         ATTN_F32 (fp32 in, fp32 arithmetic, fp32 out).
 * layout: ATTN_BNHD or ATTN_BHND, applied to q, k, v and o alike.
 * lse:    NULL, or fp32 [B, Hq, N] (out): the natural logarithm of each row's
 *         softmax denominator, max_j s_ij + ln(sum_j e^(s_ij - max)), where
 *         s_ij = scale * q_i . k_j over the visible keys.
 * variant: NULL, or window / initial tokens / sink logits (attn_variant);
 *         any variant needs dtype ATTN_BF16, and a window needs causal != 0.
 */
int attn_prefill_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int N, int Hq, int Hkv, int d, float scale, int causal,
                    int dtype, int layout, const attn_variant* variant, void* stream);

/*
 * attn_decode_num_splits - the number of context splits attn_decode uses.
 *
 * num_splits > 0 is returned clamped to [1, min(max_pages_per_seq, 1024)]; 0 asks
 * for the automatic choice, which depends only on the arguments given here
 * (not on the device), so that a result can be reproduced exactly. Returns
 * a negative status for invalid sizes.
 */
int attn_decode_num_splits(int B, int Hkv, int max_pages_per_seq, int num_splits);

/*
 * attn_decode_workspace_size - bytes of fp32 scratch attn_decode needs:
 * B*Hq*S*(d + 2)*4, with S = attn_decode_num_splits(B, Hkv, max_pages_per_seq,
 * num_splits). It takes Hkv and max_pages_per_seq besides (B, Hq, d,
 * num_splits) because the automatic split count (num_splits = 0) is a
 * function of them. Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int d, int max_pages_per_seq,
                                  int num_splits);

/*
 * attn_decode - one query token per sequence against a paged KV cache, bf16.
 *
 * q:           [B, Hq, d] bf16, the query of the newest token of each sequence.
 * k_pages,
 * v_pages:     [num_pages, page_size, Hkv, d] bf16, the physical page pool
 *              [PAGED]; a page holds page_size consecutive tokens of one
 *              sequence, every KV head.
 * block_table: int32 [B, max_pages_per_seq] (device). Entry p of row b is the
 *              physical page holding tokens p*page_size .. p*page_size +
 *              page_size - 1 of sequence b. Entries past a sequence's last page
 *              are never read.
 * seq_lens:    int32 [B] (device), tokens cached per sequence, including the
 *              newest token (its K/V already written) [KV].
 * o:           [B, Hq, d] bf16 (out).
 * For sequence b with L = seq_lens[b] and query head h:
 *   o[b,h,:] = sum_{t<L} P_t v_t,  P = softmax_t(scale * q[b,h,:].k_t),
 * with k_t = k_pages[block_table[b, t/page_size], t%page_size, kv, :] (and v_t
 * alike), kv = floor(h / (Hq/Hkv)). A sequence with L == 0 has no visible key
 * and gets o[b] = 0 (the zero-output policy of [SDPA] section 4).
 * The context of each sequence is cut into num_splits contiguous ranges of
 * logical pages; each range yields a partial (max, sum, unnormalised output)
 * in `workspace`, and a second kernel merges them by log-sum-exp [FA,
 * FlashDecoding]. The split boundaries depend only on L and num_splits, so the
 * result does not depend on where the pages sit in the pool: a permuted block
 * table gives output bit-identical to the identity table.
 *
 * dtype:       element type of q, the pools and o. ATTN_BF16 is the one
 *              supported (bf16 in, fp32 accumulation, bf16 out, the widening
 *              policy of [SDPA] section 4); any other code returns
 *              ATTN_ERR_DTYPE.
 * workspace:   caller-owned device memory of at least
 *              attn_decode_workspace_size(B, Hq, Hkv, d, max_pages_per_seq,
 *              num_splits) bytes. It is needed for every split count (the
 *              merge pass also runs for one split), so NULL returns
 *              ATTN_ERR_NULL and a smaller size ATTN_ERR_WORKSPACE. Calls
 *              that overlap in time must not share one.
 *
 * Preconditions checked on the device side only by the caller:
 *   0 <= seq_lens[b] <= max_pages_per_seq * page_size, and every table entry
 *   that is read lies in [0, num_pages). Violations read out of bounds.
 * Requires page_size == 16, d in {64, 128}, Hq a multiple of Hkv.
 */
int attn_decode(const void* q, const void* k_pages, const void* v_pages,
                const int32_t* block_table, const int32_t* seq_lens, void* o,
                int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                int num_pages, float scale, int num_splits, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and results as attn_decode
 * with the same arguments, but the split partials go to a scratch array of
 * ATTN_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on each GPU it
 * runs on, from the first call on that GPU until the process ends. The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller still owns q, the pools, the table, seq_lens and o.
 *
 * Returns ATTN_ERR_SCRATCH when attn_decode_workspace_size(B, Hq, Hkv, d,
 * max_pages_per_seq, num_splits) exceeds ATTN_NOALLOC_SCRATCH_BYTES (the
 * long-context and batched decode shapes of the benchmarks need 8.5 MB and
 * 4.3 MB), otherwise the statuses of attn_decode. The array is found on the
 * device `stream` belongs to (the current device for the null stream).
 * Every partial the merge reads is written by the same call first, so the
 * array needs no clearing between calls. All calls on one GPU share its
 * array: calls that overlap in time on one GPU (two streams, two threads)
 * race on it and must be ordered by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_noalloc(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens, void* o,
                        int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                        int num_pages, float scale, int num_splits, int dtype, void* stream);

/*
 * attn_kv_append - write the keys and values of new tokens into the paged
 * cache, the append step of [PAGED] (token t of sequence b goes to page
 * block_table[b, t / page_size], slot t % page_size) [KV].
 *
 * k_new, v_new: [T, Hkv, d] bf16, the new tokens of all sequences packed row
 *               after row; sequence b owns rows cu_new[b] .. cu_new[b+1]-1.
 * k_pages,
 * v_pages:      [num_pages, page_size, Hkv, d] bf16 (in/out); only the slots
 *               of the new tokens are written, every other byte is left as is.
 * block_table:  int32 [B, max_pages_per_seq] (device), as for attn_decode.
 * cu_new:       int32 [B + 1] (device), non-decreasing, cu_new[0] = 0,
 *               cu_new[B] = T.
 * start_pos:    int32 [B] (device), position of sequence b's first new token
 *               (the number of tokens cached before the append).
 * total_new:    T, the rows of k_new and v_new (host).
 * max_new:      an upper bound on cu_new[b+1] - cu_new[b] (host); rows beyond
 *               it are not written.
 * Preconditions checked on the device side only by the caller:
 *   start_pos[b] + (cu_new[b+1] - cu_new[b]) <= max_pages_per_seq * page_size,
 *   and every table entry that is written through lies in [0, num_pages).
 * Requires page_size == 16 and d in {64, 128}. Pure data movement: the pool
 * afterwards holds the new rows bit for bit.
 */
int attn_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                   const int32_t* block_table, const int32_t* cu_new, const int32_t* start_pos,
                   int B, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages,
                   int total_new, int max_new, void* stream);

/*
 * attn_prefill_paged - a chunk of new queries per sequence against a paged
 * KV cache that already holds the sequence's earlier tokens and the chunk's
 * own K/V (write those first with attn_kv_append): the attention half of a
 * chunked prefill ("Module 09: Efficient Attention", section "Chunked
 * Prefill: Bounding the Stall"). bf16 in, fp32 accumulation, bf16 out.
 *
 * q:           [T, Hq, d] bf16, the chunks of all sequences packed row after
 *              row; sequence b owns rows cu_q[b] .. cu_q[b+1]-1 (c_b rows).
 * k_pages,
 * v_pages:     [num_pages, page_size, Hkv, d] bf16, as for attn_decode.
 * block_table: int32 [B, max_pages_per_seq] (device).
 * cu_q:        int32 [B + 1] (device), non-decreasing, cu_q[0] = 0, cu_q[B] = T.
 * seq_lens:    int32 [B] (device), L_b: tokens cached for sequence b
 *              including its chunk, so the chunk sits at positions
 *              P_b = L_b - c_b .. L_b - 1.
 * o:           [T, Hq, d] bf16 (out).
 * lse:         NULL, or fp32 [Hq, T] (out), natural-log softmax denominator
 *              of each row, as for attn_prefill_ex.
 * total_q:     T, the rows of q and o (host); it fixes the lse layout.
 * max_q_len:   an upper bound on every c_b (host); it sizes the launch.
 * variant:     NULL, or window / initial tokens / sink logits (attn_variant),
 *              with positions counted from the start of the sequence.
 * Row i of sequence b, query head h, sees the keys at positions 0 .. P_b + i
 * (causality compares token positions [SDPA] section 4; after a prefix of P
 * tokens row i is at position P + i):
 *   o[cu_q[b]+i, h, :] = sum_{t <= P_b+i} softmax_t(scale * q.k_t) v_t,
 * with k_t, v_t read through the block table [PAGED] and kv = floor(h / g).
 * With P_b = 0 this is the causal prefill of the chunk alone.
 * Preconditions checked on the device side only by the caller:
 *   c_b <= L_b <= max_pages_per_seq * page_size, c_b <= max_q_len, and every
 *   table entry that is read lies in [0, num_pages). A sequence with
 *   c_b > L_b (violating the first) gets zeros for the rows that see no key.
 * Requires page_size == 16, d in {64, 128}, Hq a multiple of Hkv.
 */
int attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* cu_q, const int32_t* seq_lens,
                       void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                       int max_pages_per_seq, int num_pages, int total_q, int max_q_len,
                       float scale, const attn_variant* variant, void* stream);

/*
 * attn_decode_ex - attn_decode with a variant (NULL = none, the same as
 * attn_decode): with a window W the query at position L-1 sees the tokens
 * t >= L - W and t < n_sink, and only the pages holding them are read (the
 * splits cut those pages); a sink logit joins the merge as one more partial
 * with max s_h, sum 1 and zero output [SDPA] section 10. The workspace size
 * is that of attn_decode for the same arguments; with num_splits = 0 and a
 * window, the automatic split count is attn_decode_num_splits taken with
 * max_pages_per_seq replaced by the pages a window can touch,
 * min(max_pages_per_seq, ceil(W/16) + 1 + ceil(n_sink/16)) (page_size 16).
 */
int attn_decode_ex(const void* q, const void* k_pages, const void* v_pages,
                   const int32_t* block_table, const int32_t* seq_lens, void* o,
                   int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                   int num_pages, float scale, int num_splits, int dtype,
                   const attn_variant* variant, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * attn_backward_workspace_size - bytes of fp32 scratch attn_backward needs:
 * two [B, Hq, Npad] arrays, Npad = N rounded up to a multiple of 64.
 * Returns 0 for invalid sizes.
 */
size_t attn_backward_workspace_size(int B, int N, int Hq);

/*
 * attn_backward - gradients of attn_prefill_ex's output with respect to q, k
 * and v, bf16 in and out, fp32 accumulation. S and P are recomputed tile by
 * tile from the forward's log-sum-exp instead of being stored ("inference-
 * attention", section "FlashAttention"):
 *   dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
 *   dQ = scale * dS K, dK = scale * dS^T Q,
 * where dK, dV of a KV head sum over its g query heads (GQA, [SDPA] section 6).
 *
 * q, o, dout, dq: [B, N, Hq, d] (layout ATTN_BNHD) or [B, Hq, N, d] (ATTN_BHND);
 * k, v, dk, dv:   the same layout with Hkv heads.
 * o, lse:         the forward's output and its fp32 [B, Hq, N] natural-log LSE
 *                 (attn_prefill_ex with the same q, k, v, scale, causal).
 * dq, dk, dv:     outputs, fully overwritten (no accumulation into them).
 * workspace:      caller-owned device memory of at least
 *                 attn_backward_workspace_size(B, N, Hq) bytes (NULL returns
 *                 ATTN_ERR_NULL); calls that overlap in time must not share one.
 * Requires d in {64, 128} and Hq a multiple of Hkv. Deterministic: every
 * gradient element is reduced in a fixed order (no atomics).
 */
int attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int N, int Hq, int Hkv, int d,
                  float scale, int causal, int layout, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * attn_decode_mla_num_splits / attn_decode_mla_workspace_size - split count
 * (clamped to [1, min(max_pages_per_seq, 1024)]; 0 = automatic, a function of
 * the arguments only) and fp32 scratch bytes, B*Hq*splits*(512 + 2)*4, of
 * attn_decode_mla. The workspace size is 0 for invalid sizes.
 */
int attn_decode_mla_num_splits(int B, int Hq, int max_pages_per_seq, int num_splits);
size_t attn_decode_mla_workspace_size(int B, int Hq, int max_pages_per_seq, int num_splits);

/*
 * attn_decode_mla - one decode step of multi-head latent attention with the
 * up-projections absorbed ("inference-attention", section "DeepSeek
 * Multi-head Latent Attention"): each cached token is one row
 * [c_t ; k^R_t] = [latent (d_c = 512) ; rotary key (d_r = 64)] shared by all
 * query heads, i.e. multi-query attention with d_k = 576 and d_v = 512 whose
 * values are the latent columns of the same rows. bf16 in and out.
 *
 * q:          [B, Hq, 576] bf16, head h's absorbed query [W_UK,h^T q^C_h ; q^R_h].
 * kv_pages:   [num_pages, page_size, 576] bf16, the page pool of latent rows [PAGED].
 * block_table, seq_lens: as for attn_decode (the query is the newest token,
 *             already cached; L = 0 gives zeros).
 * o:          [B, Hq, 512] bf16 (out): sum_t softmax_t(scale * q_h . row_t) row_t[0:512]
 *             (W_UV is applied by the caller).
 * scale:      the score scale of the heads the latent stands for, usually
 *             1/sqrt(d_head + d_r).
 * Requires d_c == 512, d_r == 64, Hq a multiple of 16, page_size == 16 and
 * workspace_bytes >= attn_decode_mla_workspace_size(...) (a NULL workspace
 * returns ATTN_ERR_NULL). Preconditions on
 * device data as for attn_decode. The split boundaries depend only on L and
 * the split count, so a permuted table gives bit-identical output.
 */
int attn_decode_mla(const void* q, const void* kv_pages, const int32_t* block_table, const int32_t* seq_lens,
                    void* o, int B, int Hq, int d_c, int d_r, int page_size, int max_pages_per_seq,
                    int num_pages, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_gather_pages - materialise the logical cache of each sequence from the
 * page pool, with the same address computation attn_decode uses [PAGED].
 *
 * pages: [num_pages, page_size, Hkv, d] of elem_bytes-sized elements (2 or 4);
 * out:   [B, max_len, Hkv, d] (out); row t of sequence b receives token t for
 *        t < min(seq_lens[b], max_len); other rows are left untouched.
 * A test aid: it moves bytes only, so its result is bit-exact.
 */
int attn_gather_pages(const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                      void* out, int B, int Hkv, int d, int page_size, int max_pages_per_seq,
                      int num_pages, int max_len, int elem_bytes, void* stream);

/* attn_status_string - a static, human-readable name for a status code. */
const char* attn_status_string(int status);

/* attn_version - library version, major*10000 + minor*100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
