/*
 * mla_attn.h - C ABI of the causal multi-head latent attention (MLA) core
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (Kimi K2 pages, "Similarities" page, section "Query-key
 * similarity", and "Weighted sum of values" page): for every batch b, head h
 * and new query i < T, with S = past_len + T keys,
 *
 *   s[i,j] = sum_{d<128} q_nope[b,h,i,d] * k_nope[b,h,j,d]
 *          + sum_{d<64}  q_pe[b,h,i,d]   * k_pe[b,0,j,d]
 *   z[i,j] = softmax_scale * s[i,j]  + (0 if j <= past_len + i else -inf)
 *   p[i,:] = softmax(z[i,:])                   (fp32)
 *   out[b,h,i,:] = sum_j p[i,j] * v[b,h,j,:]   (bf16 result)
 *
 * The rotary key k_pe is one tensor shared by all heads (the "Scale scores"
 * section: the joint key-value down-projection emits a single rotary key);
 * queries sit at absolute positions past_len + i ("Causal mask" page,
 * "Construct causal mask": positions are numbered from the cached length and
 * the 4D causal mask is built with it). Head dims are fixed by the released
 * config ("Embedded state" page, config.json): 128 non-rotary, 64 rotary and
 * 128 value dims per head. Dropout is the identity (p = 0.0, inference).
 *
 * Conventions shared by every entry point:
 *  - All tensors are bf16, contiguous, row-major, in device memory owned by
 *    the caller. Shapes: q_nope [B,H,T,128], q_pe [B,H,T,64],
 *    k_nope [B,H,S,128], k_pe [B,1,S,64], v [B,H,S,128], out [B,H,T,128].
 *    (Exceptions, stated where they apply: lengths and block tables are
 *    int32, masks are bytes, the rotary table is fp32.)
 *  - Every non-empty tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *    work on it and return without synchronising; ordering against other
 *    work is the caller's job. The library never allocates or frees memory.
 *  - All argument checks run on the host before any HIP call; a failing
 *    call returns a status and enqueues nothing. No exceptions cross the ABI.
 *    mla_last_error() gives a thread-local description of the last failure.
 *  - B == 0, H == 0 or T == 0 is a valid empty call: it returns MLA_OK
 *    (the rotary calls state their own empty cases).
 *  - softmax_scale is taken as a 32-bit float and may be any finite value,
 *    zero and negative included (the pages multiply the scores by it without
 *    stating its value); the kernels fold softmax_scale * log2(e) into their
 *    exponent, so |softmax_scale| must stay at most FLT_MAX / log2(e)
 *    (about 2.36e38). NaN, infinities and larger magnitudes are
 *    MLA_ERR_SCALE. A zero scale weights every visible key equally.
 */
#ifndef MLA_ATTN_H_
#define MLA_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_QK_NOPE_HEAD_DIM 128
#define MLA_QK_ROPE_HEAD_DIM 64
#define MLA_V_HEAD_DIM 128

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a pointer to a non-empty tensor is NULL */
  MLA_ERR_SHAPE = 2,     /* negative size, S != past_len + T, or size beyond the launch limits */
  MLA_ERR_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
  MLA_ERR_SCALE = 4,     /* softmax_scale is NaN or infinite, or softmax_scale * log2(e)
                            overflows fp32 (or a RoPE parameter is out of range) */
  MLA_ERR_WORKSPACE = 5, /* decode workspace missing or smaller than required */
  MLA_ERR_DEVICE = 6     /* the HIP runtime reported an error at launch */
} mla_status;

/*
 * Causal MLA attention for T new queries against S = past_len + T keys
 * (prefill, chunked prefill on top of a cache of past_len keys, or any T).
 * Shape contract mirrors the attention-core excerpt ("Similarities" page):
 * the scores must be (B,H,T,kv_seq_len) and the mask (B,1,T,kv_seq_len) with
 * kv_seq_len = past_len + T; a mismatch is MLA_ERR_SHAPE (ValueError there).
 * The causal mask is generated from indices and never read from memory.
 * S is at most 8,388,607 (the key rows of a (b, h) slice are addressed
 * through a 32-bit byte range); longer sequences are MLA_ERR_SHAPE.
 */
mla_status mla_attn_prefill(const void* q_nope, const void* q_pe,
                            const void* k_nope, const void* k_pe,
                            const void* v, void* out,
                            int32_t B, int32_t H, int32_t T, int32_t S,
                            int32_t past_len, float softmax_scale,
                            void* stream);

/*
 * Bytes of device workspace mla_attn_prefill_ws needs for (B, H, T, S); 0
 * when one workgroup per query tile already fills the GPU. A pure function of
 * its arguments.
 */
size_t mla_attn_prefill_workspace_bytes(int32_t B, int32_t H, int32_t T, int32_t S);

/*
 * mla_attn_prefill with a workspace: the same result (up to the order of
 * rounding). When B*H*ceil(T/128) workgroups would leave the GPU part-empty
 * (fewer than 512: it holds two per CU), the keys each query tile sees are
 * split into near-equal ranges of whole 32-key tiles (as many ranges as
 * 512-key pieces of S, at most 16, and no more than fill the GPU); each
 * range's workgroup writes an fp32 partial (unnormalised output, max and
 * sum per query) to the workspace, and a second kernel merges the partials by
 * log-sum-exp into out. Otherwise it is exactly mla_attn_prefill.
 * workspace: caller-owned device scratch of at least
 * mla_attn_prefill_workspace_bytes(B, H, T, S) bytes, 16-byte aligned (may
 * be NULL when that is 0); contents on entry do not matter. Calls that may
 * run at the same time must not share a workspace. Errors as for
 * mla_attn_prefill, plus MLA_ERR_WORKSPACE.
 */
mla_status mla_attn_prefill_ws(const void* q_nope, const void* q_pe,
                               const void* k_nope, const void* k_pe,
                               const void* v, void* out,
                               void* workspace, size_t workspace_bytes,
                               int32_t B, int32_t H, int32_t T, int32_t S, int32_t past_len,
                               float softmax_scale, void* stream);

/*
 * Prefill of a padded batch whose sequences differ in length. The "Causal
 * mask" page ("Construct causal mask") numbers positions from each cached
 * length and passes the caller's 2D padding mask (1 keeps a position, 0 pads
 * it) with that length to the 4D mask builder. Here both the queries and the
 * keys of each sequence are right-padded: sequence b has Tb = q_lens[b] new
 * queries, rows [0, Tb) of its max_q_len query rows, over Pb = past_lens[b]
 * cached keys; its keys are rows [0, Pb + Tb) of its max_kv_len key rows, and
 * its query i (at position Pb + i) sees keys 0 .. Pb + i, as mla_attn_prefill
 * with T = Tb, past_len = Pb on that sequence alone.
 *
 *   q_nope [B, H, max_q_len, 128], q_pe [B, H, max_q_len, 64]      bf16
 *   k_nope [B, H, max_kv_len, 128], k_pe [B, 1, max_kv_len, 64],
 *   v      [B, H, max_kv_len, 128]                                   bf16
 *   q_lens, past_lens  [B] int32 in device memory, 4-byte aligned; read by
 *                      the kernel only (the host never looks at them), so a
 *                      captured graph can replay the call with new lengths
 *   out    [B, H, max_q_len, 128]                                     bf16
 *
 * Padded query rows (i >= Tb) are written as 0: they attend to nothing. Padded
 * rows of the inputs are never read. On the device Tb is clamped to
 * [0, max_q_len] and Pb to [0, max_kv_len - Tb], so no row outside the slices
 * is read whatever the arrays hold. max_q_len > max_kv_len is MLA_ERR_SHAPE
 * (a sequence's own keys follow its cache); max_kv_len is at most 8,388,607.
 * B == 0, H == 0 or max_q_len == 0 is a valid empty call. Other errors as for
 * mla_attn_prefill. One kernel is enqueued on `stream`.
 */
mla_status mla_attn_prefill_varlen(const void* q_nope, const void* q_pe,
                                   const void* k_nope, const void* k_pe,
                                   const void* v, const int32_t* q_lens,
                                   const int32_t* past_lens, void* out,
                                   int32_t B, int32_t H, int32_t max_q_len,
                                   int32_t max_kv_len, float softmax_scale, void* stream);

/*
 * mla_attn_prefill under the caller's 2D padding mask. The "Causal mask"
 * page ("Construct causal mask") hands the caller's 2D attention mask (1 keeps
 * a position, 0 pads it) with the cached length to the 4D mask builder; the
 * two combine, so key j is visible to query i of sequence b iff
 * j <= past_len + i and attn_mask[b * S + j] != 0. This covers left padding
 * (leading zeros), right padding and any other pattern.
 *
 *   attn_mask  [B, S] uint8 in device memory (S = past_len + T: every key,
 *              cached and new), nonzero keeps; no alignment needed
 *   other tensors and errors as for mla_attn_prefill (attn_mask NULL is
 *   MLA_ERR_NULL)
 *
 * A query with no visible key (a position inside left padding, say) has no
 * defined softmax; its output row is 0. Hidden keys get weight exactly 0;
 * their rows must hold finite values, as every input must (a NaN or infinite
 * value row would still meet its zero weight in the value contraction; a
 * non-finite key row is harmless). One kernel is enqueued on `stream` (no
 * key-range splits).
 */
mla_status mla_attn_prefill_masked(const void* q_nope, const void* q_pe,
                                   const void* k_nope, const void* k_pe,
                                   const void* v, const uint8_t* attn_mask, void* out,
                                   int32_t B, int32_t H, int32_t T, int32_t S,
                                   int32_t past_len, float softmax_scale, void* stream);

/*
 * Bytes of device workspace mla_attn_decode needs for (B, H, S). A pure
 * function of its arguments (no device query); 0 means no workspace is
 * needed. Returns 0 for negative sizes.
 */
size_t mla_attn_decode_workspace_bytes(int32_t B, int32_t H, int32_t S);

/*
 * Decode: one new query per sequence (T = 1) against S = past_len + 1 keys;
 * the same result as mla_attn_prefill with T = 1 (the pages run one code path
 * for both, the "Similarities" page showing decode with p = 1000, S = 1001).
 * Shapes as above with T = 1.
 *
 * When B*H is too small to fill the GPU, the key range of each (b, h) is
 * split across workgroups whose fp32 partial results (o, max, sum) are merged
 * by log-sum-exp: inside the same kernel when all splits of a (b, h) land on
 * one XCD (the last workgroup to finish merges), otherwise by a combine kernel
 * enqueued right after on the same stream.
 * workspace: caller-owned device scratch of at least
 * mla_attn_decode_workspace_bytes(B, H, S) bytes (may be NULL when that is 0),
 * 16-byte aligned. Its contents on entry do not matter and are overwritten.
 * Calls that may run at the same time must not share a workspace.
 */
mla_status mla_attn_decode(const void* q_nope, const void* q_pe,
                           const void* k_nope, const void* k_pe,
                           const void* v, void* out,
                           void* workspace, size_t workspace_bytes,
                           int32_t B, int32_t H, int32_t S, int32_t past_len,
                           float softmax_scale, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * mla_attn_decode without a workspace argument. The split partials and
 * completion flags live in a library-owned array of
 * MLA_DECODE_NOALLOC_SCRATCH_BYTES bytes on each device (reserved with the
 * library's code on that device, kept until the process ends); the call
 * allocates nothing. Every shape mla_attn_decode accepts fits (its workspace
 * never exceeds 410,112 bytes); a plan larger than the array would be
 * MLA_ERR_WORKSPACE. All calls on one device share that array: calls that
 * can overlap on one device (on different streams, or graphs replayed
 * concurrently) race, and the caller must order them. The array's contents
 * on entry do not matter (each call's completion flags carry the call's tag
 * and the merging workgroup clears them). Arguments, result and other errors
 * as for mla_attn_decode.
 */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES (512u * 1024u)
mla_status mla_attn_decode_noalloc(const void* q_nope, const void* q_pe,
                                   const void* k_nope, const void* k_pe,
                                   const void* v, void* out,
                                   int32_t B, int32_t H, int32_t S, int32_t past_len,
                                   float softmax_scale, void* stream);

/*
 * mla_attn_decode under the caller's 2D padding mask ("Causal mask" page,
 * "Construct causal mask"): the new query of sequence b sees key j iff
 * attn_mask[b * S + j] != 0 (the causal mask hides no key from the last
 * position). attn_mask is [B, S] uint8 in device memory, nonzero keeps, no
 * alignment needed; NULL is MLA_ERR_NULL. A sequence with no visible key
 * gives a zero row; hidden keys do not reach the output whatever their rows
 * hold (from the second 128-key trip of a workgroup on, their rows are not
 * even fetched). Padding differs by sequence, so the keys are split as in
 * mla_attn_decode_varlen: workspace of at least
 * mla_attn_decode_varlen_workspace_bytes(B, H, S) bytes, 16-byte aligned
 * (may be NULL when that is 0). Shapes and other errors as for
 * mla_attn_decode.
 */
mla_status mla_attn_decode_masked(const void* q_nope, const void* q_pe,
                                  const void* k_nope, const void* k_pe,
                                  const void* v, const uint8_t* attn_mask, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t B, int32_t H, int32_t S, int32_t past_len,
                                  float softmax_scale, void* stream);

/*
 * Bytes of device workspace mla_attn_decode_varlen needs for (B, H,
 * max_seq_len); 0 when no split is needed. A pure function of its arguments.
 */
size_t mla_attn_decode_varlen_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len);

/*
 * Decode over a preallocated, right-padded key-value cache with a length per
 * sequence. The "Causal mask" page ("Construct causal mask") hands a 2D
 * padding mask (1 keeps a position, 0 pads it) with the cached length to the
 * 4D mask builder, and the "Similarities" page ("Query-key similarity")
 * appends each new key and value to the cache before the new query attends.
 * Here sequence b's keys are rows [0, seq_lens[b]) of its cache slices, which
 * is the 2D mask [1]*len + [0]*(cache_len - len): right padding. The new
 * query of sequence b sees all of its keys (the new token's own key is its
 * last one); rows past seq_lens[b] are never read.
 *
 *   q_nope        [B, H, 1, 128]        bf16
 *   q_pe          [B, H, 1, 64]         bf16 (post-RoPE)
 *   k_nope_cache  [B, H, cache_len, 128] bf16
 *   k_pe_cache    [B, 1, cache_len, 64]  bf16 (shared rotary key, post-RoPE)
 *   v_cache       [B, H, cache_len, 128] bf16
 *   seq_lens      [B] int32 in device memory, 4-byte aligned; read by the
 *                 kernel (the host never looks at it), so a graph can capture
 *                 the call and the lengths change between replays
 *   out           [B, H, 1, 128]        bf16
 *
 * max_seq_len (0 <= max_seq_len <= cache_len, else MLA_ERR_SHAPE) bounds the
 * lengths: each seq_lens[b] is clamped to [0, max_seq_len] on the device, so
 * no row at or past max_seq_len is read whatever the array holds; the split
 * plan and the workspace size follow max_seq_len. A sequence whose length is
 * 0 has no visible key; its output is 0 (the convention for a fully masked
 * row, where the softmax is undefined). The cache pointers may be NULL only
 * when cache_len is 0.
 *
 * workspace: caller-owned device scratch of at least
 * mla_attn_decode_varlen_workspace_bytes(B, H, max_seq_len) bytes, 16-byte
 * aligned (may be NULL when that is 0); contents on entry do not matter.
 * Calls that may run at the same time must not share a workspace. Other
 * errors as for mla_attn_decode. One kernel (two for some shapes), as
 * mla_attn_decode, enqueued on `stream`.
 */
mla_status mla_attn_decode_varlen(const void* q_nope, const void* q_pe,
                                  const void* k_nope_cache, const void* k_pe_cache,
                                  const void* v_cache, const int32_t* seq_lens,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  int32_t B, int32_t H, int32_t cache_len,
                                  int32_t max_seq_len, float softmax_scale, void* stream);

/*
 * Bytes of device workspace mla_attn_decode_paged needs for (B, H,
 * max_seq_len); 0 when no split is needed. A pure function of its arguments.
 */
size_t mla_attn_decode_paged_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len);

/*
 * Decode over a paged key-value cache, optionally appending the new token.
 * The pages keep one growing cache per layer and append each new key and
 * value to it before the new query attends ("Similarities" page, "Query-key
 * similarity"); here the cache is stored in fixed blocks named by a table.
 * Sequence b's key j is row j % block_size of block block_table[b * max_blocks
 * + j / block_size]:
 *
 *   k_nope_pages  [num_blocks, H, block_size, 128]  bf16
 *   k_pe_pages    [num_blocks, block_size, 64]      bf16 (shared rotary key)
 *   v_pages       [num_blocks, H, block_size, 128]  bf16
 *   block_table   [B, max_blocks] int32, device memory, 4-byte aligned
 *   seq_lens      [B] int32, device memory: keys of sequence b after the call
 *   q_nope [B, H, 1, 128], q_pe [B, H, 1, 64], out [B, H, 1, 128]  bf16
 *
 * block_size is a positive multiple of 32 (else MLA_ERR_SHAPE); max_seq_len
 * <= max_blocks * block_size (else MLA_ERR_SHAPE) bounds every length, each
 * clamped on the device to [0, max_seq_len]; block ids read from the table
 * are clamped on the device to [0, num_blocks). Rows past a sequence's length
 * are never read; a sequence of length 0 gives a zero row.
 *
 * Append: k_nope_new [B, H, 1, 128], k_pe_new [B, 1, 1, 64], v_new
 * [B, H, 1, 128] (all three, or all NULL: MLA_ERR_NULL otherwise). When given,
 * the new token is key seq_lens[b] - 1 of sequence b: the call attends to it
 * from these tensors and writes them into that slot of the pages (each head's
 * rows by that head's workgroup, the shared rotary row once), so the pages
 * hold the appended token when the call completes. The slot's block must
 * belong to sequence b alone. Without them the pages are only read.
 *
 * workspace: at least mla_attn_decode_paged_workspace_bytes(B, H,
 * max_seq_len) bytes, 16-byte aligned (may be NULL when that is 0); contents
 * on entry do not matter. Calls that may run at the same time must not share
 * a workspace. The host reads neither the table nor the lengths, so a graph
 * can capture the call and both change between replays. Other errors as for
 * mla_attn_decode.
 */
mla_status mla_attn_decode_paged(const void* q_nope, const void* q_pe,
                                 void* k_nope_pages, void* k_pe_pages, void* v_pages,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const void* k_nope_new, const void* k_pe_new,
                                 const void* v_new, void* out,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t B, int32_t H, int32_t num_blocks, int32_t block_size,
                                 int32_t max_blocks, int32_t max_seq_len, float softmax_scale,
                                 void* stream);

/*
 * Bytes of device workspace mla_attn_decode_latent needs for (B, H, S); a pure
 * function of its arguments (never 0 for a non-empty call).
 */
size_t mla_attn_decode_latent_workspace_bytes(int32_t B, int32_t H, int32_t S);

/*
 * Decode over the compressed key-value cache. The "Similarities" page's
 * module ("Scale scores") keeps, per token, a latent of kv_lora_rank = 512
 * dims (after its RMSNorm) plus the one shared rotary key, and kv_b_proj
 * (no bias) expands the latent into each head's 128 non-rotary key dims and
 * 128 value dims. This call returns what mla_attn_decode would return on
 * those expanded keys and values, without expanding them: kv_b_proj's key
 * half is folded into the query and its value half is applied to the
 * attention-weighted latent.
 *
 *   q_nope  [B, H, 1, 128]  bf16      q_pe [B, H, 1, 64] bf16 (post-RoPE)
 *   c_kv    [B, S, 512]     bf16      normalised latent of every key
 *   k_pe    [B, 1, S, 64]   bf16      shared rotary key (post-RoPE)
 *   w_kv_b  [H*256, 512]    bf16      kv_b_proj.weight as stored ([out, in]);
 *                                     rows 256h..256h+127 give head h's key,
 *                                     rows 256h+128..256h+255 its value
 *   out     [B, H, 1, 128]  bf16
 *   S = past_len + 1, at most 2,097,151; H at most 64 (else MLA_ERR_SHAPE).
 *
 * workspace: caller-owned device scratch of at least
 * mla_attn_decode_latent_workspace_bytes(B, H, S) bytes, 16-byte aligned;
 * contents on entry do not matter. Calls that may run at the same time must
 * not share a workspace. Errors as for mla_attn_decode. Three kernels are
 * enqueued on `stream`: absorb (kv_b_proj's key half into the query),
 * attention over key splits (each split's latent output kept in the
 * workspace, rounded to bf16, with its fp32 max and sum), and the merge of
 * the splits followed by the value half of kv_b_proj.
 */
mla_status mla_attn_decode_latent(const void* q_nope, const void* q_pe,
                                  const void* c_kv, const void* k_pe,
                                  const void* w_kv_b, void* out,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t B, int32_t H, int32_t S, int32_t past_len,
                                  float softmax_scale, void* stream);

/*
 * Rotary prologue (YaRN-scaled RoPE on the 64 rotary dims). The
 * "Similarities" page ("Query-key similarity") rotates the new tokens' q_pe
 * and k_pe with a cos/sin table built for kv_seq_len positions and picked by
 * position, before they join the non-rotary parts; the attention calls above
 * take q_pe and k_pe after this rotation. The released configuration
 * ("Embedded state" page, config.json) gives rope_theta 50000 and a "yarn"
 * rope_scaling: factor 32, original_max_position_embeddings 4096,
 * beta_fast = beta_slow = 1, mscale = mscale_all_dim = 1. The pages print
 * neither the rotation nor the YaRN formula; this library takes them as
 * published: pair i = dims (2i, 2i+1) turns by pos * w_i' (RoPE, Su et al.),
 * (x, y) -> (x cos - y sin, x sin + y cos), with w_i = theta^(-2i/64) and,
 * when factor != 1, w_i' = g_i w_i + (1 - g_i) w_i / factor where g_i is
 * YaRN's ramp (Peng et al.) over the turns r_i = L w_i / (2 pi) that pair i
 * makes within L = original_max_position: 1 for r_i >= beta_fast, 0 for
 * r_i < beta_slow, (r_i - beta_slow) / (beta_fast - beta_slow) between.
 * YaRN's logit temperature (mscale) is not part of the table: it belongs to
 * softmax_scale.
 */

/* Bytes of the table for positions 0..max_pos-1 (256 per position); 0 for
 * max_pos <= 0 or beyond 16,777,216. A pure function of its argument. */
size_t mla_rope_table_bytes(int32_t max_pos);

/*
 * Fill table [max_pos, 32, 2] fp32 with (cos, sin) of pos * w_i' for every
 * position pos < max_pos and pair i < 32 (angle, cosine and sine computed in
 * fp64, stored rounded to fp32). table: device memory, 16-byte aligned, at
 * least mla_rope_table_bytes(max_pos) bytes. Errors: MLA_ERR_SHAPE for
 * max_pos outside [0, 16,777,216] or original_max_position <= 0;
 * MLA_ERR_SCALE unless theta > 1, factor >= 1 and both betas are finite;
 * MLA_ERR_NULL / MLA_ERR_ALIGN for the table. max_pos == 0 is a no-op.
 */
mla_status mla_rope_table(void* table, int32_t max_pos, double theta, double factor,
                          int32_t original_max_position, double beta_fast, double beta_slow,
                          void* stream);

/*
 * Rotate x [B, R, T, 64] bf16 in place: R = H for the new queries' q_pe, or
 * R = 1 for the new keys' shared k_pe (before they are appended to a cache).
 * Row t of sequence b sits at position past_len + t, or past_lens[b] + t when
 * past_lens ([B] int32, device memory, 4-byte aligned) is given; positions
 * read from past_lens are clamped on the device into [0, max_pos), so the
 * table must cover every position. The rotation runs in fp32 on the bf16
 * inputs and the fp32 table; results are rounded to nearest even bf16.
 * Errors: MLA_ERR_SHAPE for negative sizes, for past_len + T > max_pos
 * (without past_lens), max_pos == 0 with rows to rotate, or more than
 * 2^31 - 1 rows; MLA_ERR_NULL / MLA_ERR_ALIGN for x (16-byte) and the table
 * (16-byte). B, R or T == 0 is a no-op. The host reads no device memory, so
 * a graph can capture the call and past_lens can change between replays.
 */
mla_status mla_rope_apply(void* x, const int32_t* past_lens, const void* table, int32_t max_pos,
                          int32_t B, int32_t R, int32_t T, int32_t past_len, void* stream);

/*
 * The pages' one call for both rotary parts: q_pe [B, H, T, 64] and the new
 * keys' k_pe [B, 1, T, 64] (both bf16, 16-byte aligned) rotated in place, in
 * one launch, at the positions mla_rope_apply uses. Errors as for
 * mla_rope_apply (the row limit counts B * (H + 1) * T rows); B == 0 or
 * T == 0 is a no-op (with H == 0 only the key rows turn).
 */
mla_status mla_rope_apply_qk(void* q_pe, void* k_pe, const int32_t* past_lens, const void* table,
                             int32_t max_pos, int32_t B, int32_t H, int32_t T, int32_t past_len,
                             void* stream);

/*
 * mla_attn_decode with the rotary prologue fused in: q_pe is the new query's
 * rotary part before rotation, and the kernel turns it at position past_len
 * (the new token's, the last key) with rope_table [rope_max_pos, 32, 2]
 * (filled by mla_rope_table; device memory, 16-byte aligned) before scoring;
 * the rotated query stays in fp32. k_pe holds cached keys already rotated at
 * their positions, as the pages' cache stores them. Errors as for
 * mla_attn_decode, plus MLA_ERR_NULL / MLA_ERR_ALIGN for rope_table and
 * MLA_ERR_SHAPE when rope_max_pos <= past_len (or beyond 16,777,216).
 */
mla_status mla_attn_decode_rope(const void* q_nope, const void* q_pe, const void* k_nope,
                                const void* k_pe, const void* v, const void* rope_table,
                                int32_t rope_max_pos, void* out, void* workspace,
                                size_t workspace_bytes, int32_t B, int32_t H, int32_t S,
                                int32_t past_len, float softmax_scale, void* stream);

/*
 * mla_attn_decode_varlen with the rotary prologue fused in: q_pe is the new
 * query's rotary part before rotation; sequence b's query turns at position
 * seq_lens[b] - 1 (its last key; lengths clamped on the device as for
 * mla_attn_decode_varlen). The cache holds keys already rotated at their
 * positions. rope_table as for mla_attn_decode_rope, covering positions up
 * to max_seq_len - 1 and holding at least one row (rope_max_pos >=
 * max(max_seq_len, 1), else MLA_ERR_SHAPE). Other errors as for
 * mla_attn_decode_varlen.
 */
mla_status mla_attn_decode_varlen_rope(const void* q_nope, const void* q_pe,
                                       const void* k_nope_cache, const void* k_pe_cache,
                                       const void* v_cache, const int32_t* seq_lens,
                                       const void* rope_table, int32_t rope_max_pos, void* out,
                                       void* workspace, size_t workspace_bytes, int32_t B,
                                       int32_t H, int32_t cache_len, int32_t max_seq_len,
                                       float softmax_scale, void* stream);

/*
 * mla_attn_decode_paged with the rotary prologue fused in: q_pe and, when the
 * call appends the new token, k_pe_new are rotary parts before rotation.
 * Sequence b's new token sits at position seq_lens[b] - 1 (clamped into the
 * table on the device); the kernel turns the query there, and turns the new
 * key there, rounds it to bf16 and both attends to it and stores it in its
 * slot, so later calls read the same rotated key. rope_table as for
 * mla_attn_decode_rope, covering positions up to max_seq_len - 1 and
 * holding at least one row (rope_max_pos >= max(max_seq_len, 1), else
 * MLA_ERR_SHAPE). Other errors as for mla_attn_decode_paged.
 */
mla_status mla_attn_decode_paged_rope(const void* q_nope, const void* q_pe, void* k_nope_pages,
                                      void* k_pe_pages, void* v_pages, const int32_t* block_table,
                                      const int32_t* seq_lens, const void* k_nope_new,
                                      const void* k_pe_new, const void* v_new,
                                      const void* rope_table, int32_t rope_max_pos, void* out,
                                      void* workspace, size_t workspace_bytes, int32_t B,
                                      int32_t H, int32_t num_blocks, int32_t block_size,
                                      int32_t max_blocks, int32_t max_seq_len,
                                      float softmax_scale, void* stream);

/* Static name of a status code ("MLA_OK", ...); "unknown status" otherwise. */
const char* mla_status_string(mla_status s);

/* Thread-local message for the last failing call on this thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ATTN_H_ */
