/*
 * lvq.h -- C ABI of liblvq: decode attention read directly from a
 * sub-2-bit quantized KV cache on AMD Instinct MI355X (gfx950).
 *
 * Two cache formats share one engine:
 *
 *  - LoopVQ ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
 *    Transformers", Cheong & Yoo).  Each (loop block, layer, head, channel
 *    group) has a codebook of K = 256 codewords of G coordinates; one 8-bit
 *    index covers c = G/T_c channels at each of T_c consecutive loop steps
 *    ("method steps", step 1).  Sinks and the recent window stay bf16 at
 *    every loop step; older tokens live as indices in 8-token pages (step 4,
 *    Figure 5).  Loop step t rebuilds pre-RoPE keys and values through its own
 *    slice B_t of each codeword, rotates keys by their positions, and attends;
 *    index pages and bf16 tokens are attended separately and merged exactly
 *    through logsumexp (step 5, Figure 5; background "SGLang and
 *    Flash-Decoding").
 *
 *  - KIVI ("KIVI 完全拆解" walkthrough of KIVI): 2-bit asymmetric uniform
 *    quantization q = clamp(round(x/s + z), 0, 3), x_hat = s (q - z) with
 *    fp16 s and z ("definitions" section); keys per channel over groups of
 *    32 tokens, values per token over groups of 32 channels, the newest
 *    tokens kept fp16 in a residual window of R = 128 ("core design").
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller, unless a
 *    parameter says "host".  The library never allocates, frees or
 *    synchronizes; callers size buffers with the *_workspace queries.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *  - Arguments are validated before anything is launched.  On failure the
 *    call returns a non-zero lvq_status, launches nothing, and
 *    lvq_last_error() returns a message (thread-local) describing it.
 *  - LVQ_ERR_HIP is returned if the launch itself fails (hipGetLastError).
 *  - Device-side contents (lengths, page ids) are trusted: the caller
 *    guarantees page ids < the pool's page count and lengths <= the
 *    max_len it passes.
 *  - Calls that write the same buffers must not overlap across streams.
 *  - Element types: bf16 and fp16 arrays are passed as void* holding 16-bit
 *    IEEE-style bf16 / binary16 values.
 */
#ifndef LVQ_H
#define LVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LVQ_API __attribute__((visibility("default")))

typedef enum {
    LVQ_OK = 0,
    LVQ_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent geometry */
    LVQ_ERR_UNSUPPORTED = 2,  /* a shape this build has no kernel for */
    LVQ_ERR_WORKSPACE = 3,    /* workspace smaller than the *_workspace query */
    LVQ_ERR_HIP = 4           /* the HIP runtime reported an error */
} lvq_status;

typedef enum { LVQ_BF16 = 0, LVQ_FP32 = 1 } lvq_dtype;

/* Thread-local description of the last failure of a call on this thread. */
LVQ_API const char* lvq_last_error(void);

/* ------------------------------------------------------------------------ */
/* LoopVQ geometry                                                          */
/* ------------------------------------------------------------------------ */

/*
 * D       head dimension (128 supported)
 * T       loop steps; T_c must divide T and G ("method steps", step 1)
 * Tc      loop steps that share one index row
 * G       codeword dimension (at most 32); c = G/Tc channels per codeword
 *         per step (c = 4 or 8 supported); NG = D/c index groups per token
 *         and step
 * K       codewords per codebook (256: 8-bit indices)
 * page    tokens per index page (8)
 * sink    leading tokens kept bf16 (8)
 * window  recent-window length W; a request of length L keeps
 *         n_pages = max(0, (L - sink - W) / page) index pages covering
 *         positions [sink, sink + page*n_pages) and bf16 tokens elsewhere,
 *         so the recent part holds W .. W+page-1 tokens (step 4, Figure 5)
 * H       KV heads (multi-head: one query head per KV head)
 * cb_dtype  element type of codebooks and slices (LVQ_BF16 or LVQ_FP32)
 *
 * Memory layouts (row-major, innermost last):
 *  codebooks  [NB=T/Tc][H][2 (0=K,1=V)][NG][K][G]          cb_dtype
 *  slices     [T][H][2][NG][K][c]   slice[t][h][kv][g][r][i] =
 *             codebooks[t/Tc][h][kv][g][r][i*Tc + t%Tc]       cb_dtype
 *  pool       [P][NB][H][2][page][NG] uint8 index pages; one physical page
 *             holds 8 tokens of one request for every block and head.  Rows
 *             are permuted by the index-token number tau (counted from the
 *             first paged position), t = tau & 15:
 *             - a value row is XOR-rotated: byte m holds group m ^ t;
 *             - a key row of 16 groups (c = 8): byte j holds group P(j) ^ t,
 *               P the bit permutation (j3 j2 j1 j0) -> (j1 j3 j2 j0), so
 *               dword k holds groups {2k, 2k+1, 2k+8, 2k+9} ^ t: two pairs of
 *               RoPE-partner groups (channels i and i + 64);
 *             - a key row of 32 groups (c = 4) is in group order.
 *             The permutations let the 16 lanes of one LDS phase of the
 *             attention kernels read or update 16 distinct groups (hence
 *             16 distinct banks) while each lane keeps whole index dwords.
 *  page_table [B][pt_stride] int32, logical page -> physical page; attention
 *             reads only the entries of a request's own index pages, which
 *             must name pages of the pool (other entries may hold anything)
 *  window     [B][T][H][Wcap][D] bf16, Wcap = sink + W + page; pre-RoPE
 *             K (and separately V) of every loop step; position p < sink sits
 *             in slot p, position p >= sink in slot sink + (p - sink) % (W + page)
 *  rope       cos, sin fp32 [rope_len][D/2]: cos/sin(p * base^(-2i/D))
 *  rope_f16   packed fp16 copy for the index-page kernels (D = 128), 384
 *             halves (768 bytes) per position in two parts: part A
 *             [rope_len][32 chunks][8 halves], where chunk m < 16 of position
 *             p holds cos of frequencies 4m..4m+3, then sin of the same four,
 *             and chunk 16 + m the same with the sines negated; then part B
 *             [16 chunks][rope_len][8 halves], chunks m < 16 again, chunk-major
 *             (part A serves kernels whose lanes take one position's chunks
 *             together, part B kernels whose lanes hold consecutive positions)
 */
typedef struct {
    int32_t D, T, Tc, G, K, page, sink, window, H, cb_dtype;
} lvq_geom;

/*
 * Cut the per-step codebook slices B_t out of the full codebooks, once at
 * load time ("method steps", step 5; Figure 3).  Layouts above.
 */
LVQ_API lvq_status lvq_slice_codebooks(const lvq_geom* g, const void* codebooks, void* slices,
                               hipStream_t stream);

/*
 * RoPE table: cos_out[p][i] = fp32(cos(p * base^(-2i/D))), same for sin,
 * for p < len, i < D/2; angles and the functions are evaluated in fp64 and
 * rounded once (background "RoPE": keys are rotated by their position after
 * reconstruction, with a precomputed table).  The rotation pairs channel i
 * with channel i + D/2 (rotate-half form).
 */
LVQ_API lvq_status lvq_rope_table(int32_t len, int32_t D, double base, float* cos_out, float* sin_out,
                          hipStream_t stream);

/*
 * The packed fp16 RoPE table (layout rope_f16 above): each cos/sin is
 * evaluated in fp64 and rounded once to binary16.  D must be 128.  out holds
 * len * 768 bytes.  The index-page pass forms its scores from it in packed
 * half precision (q turned back by the key's angle, dotted with the key in
 * fp32 accumulation).
 */
LVQ_API lvq_status lvq_rope_table_f16(int32_t len, int32_t D, double base, void* out, hipStream_t stream);

/*
 * Channel permutation P of the cached keys and values (LoopVQ page,
 * "technical novelty", system level: combined with TaSQ, LoopVQ optimises a
 * channel permutation P jointly with the grouping).  perm (host, D int32):
 * stored channel j holds original channel perm[j].  The library serves a
 * permutation that maps RoPE pairs to RoPE pairs in its rotate-half pairing:
 * perm[j] < D/2 and perm[j + D/2] == perm[j] + D/2 for every j < D/2.  The
 * caller then passes permuted keys and values to lvq_encode / the window,
 * the permuted query q'[j] = q[perm[j]], and RoPE tables whose frequency
 * column j is frequency perm[j] (lvq_rope_table_perm); attention output
 * channel j is original value channel perm[j].  The scores are unchanged:
 * the pair (j, j + D/2) rotates by the angle of original pair perm[j].
 * Returns LVQ_OK for such a permutation; LVQ_ERR_UNSUPPORTED for any other
 * permutation, with a message saying so when it puts both channels of a
 * RoPE pair in one index group (the form the kernels cannot serve: they
 * rotate group x against group x + NG/2); LVQ_ERR_INVALID_ARG when perm is
 * NULL or not a permutation of 0 .. D-1.  Host only: touches no device.
 */
LVQ_API lvq_status lvq_channel_perm_check(const lvq_geom* g, const int32_t* perm);

/*
 * lvq_rope_table and (f16_out != NULL) lvq_rope_table_f16 for a channel
 * permutation that lvq_channel_perm_check accepts: frequency column j
 * holds frequency perm[j] (cos/sin of p * base^(-2 perm[j] / D)).  cos_out
 * and sin_out are both given or both NULL; the packed table needs D = 128.
 * Errors as lvq_channel_perm_check, then as the two table calls.
 */
LVQ_API lvq_status lvq_rope_table_perm(const lvq_geom* g, const int32_t* perm, int32_t len, double base,
                                       float* cos_out, float* sin_out, void* f16_out, hipStream_t stream);

/*
 * Encode index pages of loop block `block` ("method steps", step 4; Figure 5):
 * for each request b and each logical page lp in
 * [first_page[b], first_page[b] + n_pages[b]), the 8 tokens of the page are
 * coupled across the block's T_c loop steps and each coupled sub-vector is
 * replaced by the index of its nearest codeword, argmin_r ||z - e_r||^2, and
 * written to pool page page_table[b*pt_stride + lp] at [block][h][kv].
 * bf16 codebooks with G a multiple of 8 and T_c in {1, 2, 4, 8}: the
 * scores come from a bf16 matrix-core contraction with fp32 sums,
 * argmax_r (z . e_r - ||e_r||^2 / 2); where a token's best two scores lie
 * within twice the fp32 error bound of a score, its nearest codeword is
 * taken again from fp64 direct differences over all codewords, so every
 * pick is the exact nearest codeword, the lowest index among equal
 * distances.  fp32 codebooks and the other bf16 shapes: an exact fp64 scan,
 * lowest index on ties.
 * The same call serves prefill (many pages) and decode (the oldest window
 * page, every 8 generated tokens).
 *
 *  x_k, x_v      bf16 pre-RoPE keys / values (either may be NULL to skip).
 *                Element (b, h, token j, step m, d) is read from
 *                x + b*x_strides[0] + h*x_strides[1] + (x_tok0[b] + j)*x_strides[2]
 *                  + m*x_strides[3] + d          (strides in elements),
 *                where m in [0, Tc) is the step inside the block and j counts
 *                tokens from the first encoded page (j = 8*(lp - first_page[b]) + i).
 *  x_tok0        device int64 [B] token-row offsets, or NULL for all zero.
 *  codebooks     full codebooks (layout above).
 *  first_page, n_pages   device int32 [B].
 *  max_pages     host: an upper bound of n_pages[b] over the batch (grid size).
 */
LVQ_API lvq_status lvq_encode(const lvq_geom* g, int32_t block,
                      const void* x_k, const void* x_v, const int64_t x_strides[4],
                      const int64_t* x_tok0, const void* codebooks,
                      uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                      const int32_t* first_page, const int32_t* n_pages,
                      int32_t B, int32_t max_pages, hipStream_t stream);

/*
 * One Lloyd step of Fisher-weighted k-means for the codebooks of loop block `block` (the LoopVQ page:
 * background "Fisher-weighted k-means" and "method steps" step 2, the codebook initialisation of Eq. 3).
 * The assignment is the encoder's: call lvq_encode on the calibration pages with the current codebooks
 * first (a scalar weight per sub-vector scales all of its distances alike, so the nearest codeword does
 * not depend on it).  Then each coupled vector z of those pages, weight w, adds w*z and w to the sums of
 * the codeword its page holds, and every codeword of block `block` becomes sum(w z) / sum(w), rounded
 * once to the codebook dtype (nearest-even); a codeword whose weight sum is not positive keeps its value.
 * The sums are exact fixed-point integers per (head, K|V, group): each product w*z is rounded to a
 * multiple of 2^-e with N * max|w z| * 2^e < 2^51 (N the samples of the call), likewise w, so the result
 * does not depend on the order of the adds and is reproducible bit for bit.  A weight below about
 * 2^-52 * N times the largest one can round to zero.  A NaN or infinite weight or coordinate turns the
 * whole codebook of its (head, K|V, group) into NaN.  No workspace.  Requires G <= 32.
 *
 *  x_k, x_v, x_strides, x_tok0, page_table, pt_stride, first_page, n_pages, B, max_pages: as for
 *            lvq_encode (the same pages it encoded); either of x_k / x_v may be NULL to skip K or V.
 *  w_k, w_v  fp32 weights (>= 0) of the key / value sub-vectors: the weight of group g of token row
 *            `row` (x_tok0[b] + j, as for x) of request b, head h is
 *            w[b*w_strides[0] + h*w_strides[1] + row*w_strides[2] + g] (strides in elements); required
 *            with the matching x.
 *  codebooks the full codebooks (layout above), updated in place for block `block` only.
 * Errors: LVQ_ERR_INVALID_ARG for a bad block, sizes or NULL pointers, LVQ_ERR_UNSUPPORTED for G > 32.
 */
LVQ_API lvq_status lvq_codebook_update(const lvq_geom* g, int32_t block, const void* x_k, const void* x_v,
                                       const int64_t x_strides[4], const int64_t* x_tok0, const float* w_k,
                                       const float* w_v, const int64_t w_strides[3], void* codebooks,
                                       const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                       const int32_t* first_page, const int32_t* n_pages, int32_t B,
                                       int32_t max_pages, hipStream_t stream);

/*
 * Bytes of workspace lvq_decode_attn needs for B requests of length at most
 * max_len with the given split count (0 = the library's choice); 0 for
 * invalid arguments.  With bf16 codebooks this counts the room for a packed
 * fp16 RoPE table of the positions below max_len (768 B each), which a call
 * given rope_f16 does not use.
 */
LVQ_API size_t lvq_decode_attn_workspace(const lvq_geom* g, int32_t B, int32_t max_len, int32_t num_splits);

/*
 * Decode attention of loop step `step` (0-based) for B requests (step 5,
 * Figure 5): out[b][h] = softmax(sm_scale * q . RoPE(k_p)) V over positions
 * p in [0, seq_len[b]), where keys and values of paged positions are rebuilt
 * from their indices through the step's codebook slice, and sink/recent
 * positions come from the window buffers; keys are rotated at their absolute
 * position.  The index pages are attended in `num_splits` splits per request
 * (Flash-Decoding); a second kernel attends the bf16 window and merges its
 * partial with the splits' exactly through logsumexp.  With bf16 codebooks
 * one workgroup scores the tokens of a split for four requests (two when
 * c = 4), sharing the codebook slice and the RoPE table loads, then turns the
 * scores into softmax weights and accumulates them per (group, codeword) of
 * the value indices; a split then holds at most 1536 index tokens (192
 * pages), so a request holds at most 1024 * 192 index pages (longer
 * contexts: LVQ_ERR_UNSUPPORTED).
 *
 *  q          bf16 [B][H][D], already rotated at position seq_len[b] - 1.
 *  seq_len    device int32 [B], 1 <= seq_len[b] <= max_len <= rope_len.
 *  order      device int32 [B] or NULL: the grouping of requests into
 *             workgroups, which take consecutive entries (four at a time,
 *             two when c = 4); NULL means order[i] = i.  It must hold each
 *             request once (lvq_request_order below writes one sorted by
 *             length, which keeps a workgroup's requests of similar length
 *             and so saves work on ragged batches); an entry outside [0, B)
 *             leaves its slot empty and that request unattended (its output
 *             is then undefined), never an out-of-bounds access.  The output
 *             does not depend on the grouping.
 *  k_scales   device fp16 [physical page][T][8] or NULL: the key scale stream
 *             of TaSQ+LoopVQ (LoopVQ page, limitations note: an extra fp16
 *             key scale of about 0.008 bit per element, read as one per index
 *             token and loop step, shared by the heads).  Index token i of
 *             physical page p is scored with its reconstructed key times
 *             k_scales[(p*T + step)*8 + i]; bf16 window tokens are not scaled.
 *             One page of scales per pool page.  The transform that
 *             produces the scales is not part of this library: lvq_encode
 *             takes keys already divided by their scale.
 *  slices     slices of ALL steps (layout above); the call reads step `step`.
 *             bf16 slice entries must lie within the binary16 range
 *             (|x| <= 65504): the index-page pass converts the step's key
 *             slice to fp16 (exact for |x| >= 2^-14, absolute error below
 *             2^-25 under that).
 *  rope_cos, rope_sin  fp32 tables (lvq_rope_table), rope_len rows each.
 *  rope_f16   packed fp16 table (lvq_rope_table_f16) with the same rope_len,
 *             or NULL: with bf16 codebooks the call then builds the table
 *             for positions below max_len from rope_cos / rope_sin in the
 *             workspace (each fp32 value rounded once to binary16; one more
 *             small launch per call).  Ignored for fp32 codebooks.
 *  out        fp32 [B][H][D];  lse_out fp32 [B][H] or NULL.
 *  ws         device workspace of at least lvq_decode_attn_workspace() bytes
 *             (which counts the room for a packed table; a call given
 *             rope_f16 needs that much less), 256-byte aligned
 *             (LVQ_ERR_INVALID_ARG otherwise); contents need no
 *             initialisation and are scratch after the call.
 *  num_splits 0 lets the library choose; otherwise
 *             1..1024, and with bf16 codebooks large enough that a split
 *             holds at most 192 index pages:
 *             ceil(ceil(max_pages / num_splits) / 8) * 8 <= 192,
 *             max_pages = (max_len - sink - window) / 8 (LVQ_ERR_INVALID_ARG).
 */
LVQ_API lvq_status lvq_decode_attn(const lvq_geom* g, int32_t step, const void* q,
                           const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                           const int32_t* seq_len, int32_t max_len, const int32_t* order,
                           const void* k_scales, const void* win_k, const void* win_v,
                           const void* slices, const float* rope_cos, const float* rope_sin,
                           const void* rope_f16, int32_t rope_len, float sm_scale, float* out, float* lse_out,
                           void* ws, size_t ws_bytes, int32_t num_splits, int32_t B,
                           hipStream_t stream);

/*
 * lvq_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as lvq_decode_attn, without ws / ws_bytes: the
 * workspace is a device array the library holds, LVQ_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, kept until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's copy of the array.
 * Errors: those of lvq_decode_attn, and LVQ_ERR_WORKSPACE when
 * lvq_decode_attn_workspace(g, B, max_len, num_splits) exceeds
 * LVQ_NOALLOC_SCRATCH_BYTES (nothing is launched).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (several streams or host threads at once) race and must not be issued.
 */
#define LVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
LVQ_API lvq_status lvq_decode_attn_noalloc(const lvq_geom* g, int32_t step, const void* q,
                                           const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                           const int32_t* seq_len, int32_t max_len, const int32_t* order,
                                           const void* k_scales, const void* win_k, const void* win_v,
                                           const void* slices, const float* rope_cos, const float* rope_sin,
                                           const void* rope_f16, int32_t rope_len, float sm_scale, float* out,
                                           float* lse_out, int32_t num_splits, int32_t B, hipStream_t stream);

/*
 * Append one generated token to the bf16 window of loop step `step` (the LoopVQ page, Figure 5: each new
 * token's pre-RoPE K and V of every loop step enter the recent window; after every 8 generated tokens
 * the window's oldest page is encoded into the pool with lvq_encode, reading the window through its
 * strides, and leaves it).  For each request b the token is position p = min(seq_len[b], max_len) - 1,
 * i.e. seq_len already counts it (nothing is written when p < 0); it goes to window slot p for
 * p < sink, else sink + (p - sink) mod (window + page) of win_k / win_v [B][T][H][sink+window+page][D].
 *  k_new, v_new  bf16 [B][H][D] pre-RoPE (either may be NULL to skip), 16-byte aligned.
 * Errors: LVQ_ERR_INVALID_ARG for a bad step, B < 0, max_len < 1, NULL or misaligned buffers.
 */
LVQ_API lvq_status lvq_window_append(const lvq_geom* g, int32_t step, const void* k_new, const void* v_new,
                                     void* win_k, void* win_v, const int32_t* seq_len, int32_t max_len,
                                     int32_t B, hipStream_t stream);

/* The split count lvq_decode_attn runs for num_splits = 0 (0 on bad arguments). */
LVQ_API int32_t lvq_decode_attn_splits(const lvq_geom* g, int32_t B, int32_t max_len);

/*
 * A request order for ragged batches: order[k] = the request of rank k when
 * the batch is sorted by length min(max(seq_len[b], 0), max_len), longest
 * first, equal lengths by index (a permutation of 0 .. B-1; equal lengths
 * give the identity).  Batches of more than 4096 requests, or max_len of
 * 2^20 or more, get the identity.  One kernel launch; within a decode step
 * every layer and loop step can use the same order.
 *  seq_len  device int32 [B];  order  device int32 [B], written.
 * Errors: LVQ_ERR_INVALID_ARG for B < 0, max_len < 1 or NULL pointers.
 */
LVQ_API lvq_status lvq_request_order(const int32_t* seq_len, int32_t B, int32_t max_len, int32_t* order,
                                     hipStream_t stream);

/*
 * Debug check of what the attention and encode kernels take on trust (they
 * clamp lengths to max_len but dereference page ids as given): for every
 * request b, each of its index pages lp < n_pages(min(max(seq_len[b], 0),
 * max_len)), n_pages(L) = max(0, floor((L - sink - window) / page)), must name
 * a physical page in [0, n_pool_pages).  Writes bad (device int32 [3]):
 * bad[0] = the number of offending page-table entries, bad[1] = the lowest
 * request holding one (-1 if none), bad[2] = the number of requests whose
 * seq_len lies outside [0, max_len] (the kernels clamp those; reported for
 * information).  Reads only those page-table entries; one kernel launch of
 * one workgroup, meant for debug builds and tests (the caller reads bad).
 *  page_table [B][pt_stride] int32, seq_len [B] int32 (device).
 * Errors: LVQ_ERR_INVALID_ARG for B < 0, max_len < 1, n_pool_pages < 1,
 * pt_stride below the page count of max_len, or NULL pointers.
 */
LVQ_API lvq_status lvq_check_pages(const lvq_geom* g, const int32_t* page_table, int32_t pt_stride,
                                   const int32_t* seq_len, int32_t max_len, int32_t n_pool_pages, int32_t B,
                                   int32_t* bad, hipStream_t stream);

/*
 * The two partial passes lvq_decode_attn is made of, callable on their own
 * (Figure 5 of the LoopVQ page: one kernel attends the index pages, another
 * the bf16 pages, and their outputs are merged).  Both write normalised
 * partials part_o fp32 [B*H][S_tot][D] and their logsumexp part_lse fp32
 * [B*H][S_tot]; splitk_lse_merge(part_o, part_lse, B*H, S_tot, D, ...) then
 * gives the attention output.  Rows are (request b, head h) -> b*H + h.
 *
 * lvq_quant_partial: the index pages of each request are cut into
 *   num_splits ranges of ceil(max_pages / num_splits) pages and split s writes
 *   slot s; an empty range writes part_o = 0, part_lse = -inf.
 *   S_tot >= num_splits.  Splits cover ceil(ceil(max_pages / num_splits) / 8) * 8
 *   pages each (later ones may be empty; with bf16 codebooks at most 192, as
 *   for lvq_decode_attn).  ws is 256-byte aligned device scratch of at least
 *   lvq_quant_partial_workspace(g, B, max_len) bytes: the query rows repacked
 *   as fp16 (pre-scaled by sm_scale * log2 e), 256 B per (request, head),
 *   then, with bf16 codebooks, room for the packed RoPE table of positions
 *   below max_len (768 B each; used only when rope_f16 is NULL).
 * lvq_window_partial: the sink and recent bf16 tokens of step `step`, written
 *   to slot `slot` (< S_tot).  Never empty for seq_len >= 1.
 * Other arguments as for lvq_decode_attn.
 */
LVQ_API lvq_status lvq_quant_partial(const lvq_geom* g, int32_t step, const void* q,
                                     const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                     const int32_t* seq_len, int32_t max_len, const int32_t* order,
                                     const void* k_scales, const void* slices,
                                     const float* rope_cos, const float* rope_sin, const void* rope_f16,
                                     int32_t rope_len, float sm_scale, float* part_o, float* part_lse,
                                     int32_t num_splits,
                                     int32_t S_tot, void* ws, size_t ws_bytes, int32_t B, hipStream_t stream);
LVQ_API size_t lvq_quant_partial_workspace(const lvq_geom* g, int32_t B, int32_t max_len);
LVQ_API lvq_status lvq_window_partial(const lvq_geom* g, int32_t step, const void* q,
                                      const int32_t* seq_len, int32_t max_len,
                                      const void* win_k, const void* win_v,
                                      const float* rope_cos, const float* rope_sin, int32_t rope_len,
                                      float sm_scale, float* part_o, float* part_lse, int32_t slot,
                                      int32_t S_tot, int32_t B, hipStream_t stream);

/*
 * Exact merge of split partials (background "SGLang and Flash-Decoding"):
 *   lse[n] = M + ln sum_s exp(part_lse[n][s] - M),  M = max_s part_lse[n][s]
 *   out[n] = sum_s exp(part_lse[n][s] - lse[n]) * part_o[n][s]
 * Splits with part_lse = -inf contribute nothing; a row whose splits are all
 * empty gets out = 0, lse = -inf.
 *  part_o fp32 [n][S][D], part_lse fp32 [n][S], out fp32 [n][D], lse_out [n] or NULL.
 */
LVQ_API lvq_status splitk_lse_merge(const float* part_o, const float* part_lse, int32_t n, int32_t S,
                            int32_t D, float* out, float* lse_out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* KIVI                                                                     */
/* ------------------------------------------------------------------------ */

/*
 * D      head dimension (128 supported)     H      KV heads
 * bits   key code width: 2 or 4 (KIVI page, "definitions": 2^b - 1 levels;
 *        4 bits is its KIVI-4 variant)
 * group  32 (tokens per key group, channels per value group)
 * R      residual length (a multiple of group)
 * cap    token capacity per request (a multiple of group)
 * v_bits value code width: 2 or 4, or 0 for the keys' width (mixed widths)
 * Hq     query heads (grouped-query attention: Hq / H query heads share each
 *        KV head, query head j uses KV head j / (Hq / H)); 0 means H.  Hq / H
 *        must divide 32.
 */
typedef struct {
    int32_t D, H, bits, group, R, cap, v_bits, Hq;
} kivi_geom;

/*
 * Cache of B requests, all device pointers (b = the side's code width, kb for
 * keys, vb for values):
 *  k_codes  uint8 [B][H][cap][D*kb/8] key codes, token-major; channel d of a
 *                                    token sits in byte d*kb/8 at bits
 *                                    kb*(d % (8/kb))
 *  k_scale, k_zero  fp16 [B][H][cap/group][D]   per (32-token group, channel)
 *  v_codes  uint8 [B][H][cap][D*vb/8] value codes, same packing
 *  v_scale, v_zero  fp16 [B][H][cap][D/group]   per (token, 32-channel group)
 *  k_res, v_res     fp16 [B][H][R+group][D]     residual rings: position p in slot p % (R+group)
 *  len, n_kq, n_vq  int32 [B]        tokens held; keys [0, n_kq) and values
 *                                    [0, n_vq) are quantized, the rest fp16
 */
typedef struct {
    uint8_t* k_codes; void* k_scale; void* k_zero;
    uint8_t* v_codes; void* v_scale; void* v_zero;
    void* k_res; void* v_res;
    int32_t* len; int32_t* n_kq; int32_t* n_vq;
} kivi_cache;

/*
 * Append n_new tokens per request ("core design", pseudo-code):
 *  - prefill (n_new >= 1, cache empty: len[b] == 0 for all b): keys
 *    [0, group*floor((n_new-R)/group)) are quantized per channel, values
 *    [0, n_new-R) per token, the rest kept fp16;
 *  - decode (n_new == 1, cache non-empty): the token goes to the residuals;
 *    then, if the key residual holds R or more rows, its oldest R rows are
 *    quantized (R/group whole groups) and dropped; if the value residual holds
 *    more than R rows, the rows beyond the newest R are quantized.
 * Codes, s and z follow q = clamp(rint(fl32(fl32(x/s) + z)), 0, 2^b - 1) with
 * s = fp16(fl32(fl32(max - min)/(2^b - 1))) (1 if that is 0) and z = fp16(fl32(-min/s)),
 * each step IEEE binary32 round-to-nearest-even.
 *  k_new, v_new  fp16 (H KV heads); element (b, h, j, d) at b*new_strides[0] + h*new_strides[1]
 *                + j*new_strides[2] + d   (strides in elements, host array).
 *  prefill       host flag: 1 = prefill, 0 = decode.
 */
LVQ_API lvq_status kivi_append(const kivi_geom* g, const void* k_new, const void* v_new,
                       const int64_t new_strides[3], int32_t n_new, int32_t prefill,
                       const kivi_cache* c, int32_t B, hipStream_t stream);

LVQ_API size_t kivi_decode_attn_workspace(const kivi_geom* g, int32_t B, int32_t max_len, int32_t num_splits);

/*
 * Decode attention over the quantized and fp16 segments with ONE softmax over
 * all logits ("core design", segment attention; "engineering": the segments
 * must share the normaliser).  Keys are used as stored (post-RoPE in KIVI).
 *  q  fp16 [B][Hq][D];  out fp32 [B][Hq][D];  lse_out fp32 [B][Hq] or NULL
 *  (Hq = H when the geometry's Hq is 0).  Query head j attends over KV head
 *  j / (Hq / H).
 *  max_len (host) bounds len[b]; num_splits 0 = the library's choice, else
 *  the number of splits of each request's tokens.  The splits share only the
 *  key groups quantized on both sides and one more workgroup per (request,
 *  KV head) takes the rest (the fp16 residual rows, a partial group);
 *  kivi_decode_attn_workspace counts num_splits + 1 partial slots.  A
 *  request holding no tokens gets out = 0, lse = -inf.
 *  Numerics: with up to 16 query heads per KV head the scores take each
 *  query element times its channel's key scale as an fp16 product (held
 *  exactly as a rounding plus its remainder), so |q[d] * s_k[d]| must stay
 *  within the fp16 range (65504); the value sums take p * s_v in fp16.
 *  Everything is accumulated in fp32.
 */
LVQ_API lvq_status kivi_decode_attn(const kivi_geom* g, const void* q, const kivi_cache* c, int32_t max_len,
                            float sm_scale, float* out, float* lse_out, void* ws, size_t ws_bytes,
                            int32_t num_splits, int32_t B, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LVQ_H */
