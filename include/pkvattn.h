/*
 * pkvattn: causal grouped-query attention over a KV cache on MI355X (gfx950).
 *
 * Operations, one entry point each:
 *   attn_prefill        multi-token causal prefill, contiguous or paged K/V
 *   attn_prefill_varlen ragged batch of prefill chunks over one shared cache
 *   attn_decode_contig  single-token decode over a contiguous cache
 *   attn_decode_paged   single-token decode over a block-table paged cache
 *   attn_decode_*_ext   the same with a layer's arms (window, softcap, ALiBi,
 *                       sinks, V width)
 *   mla_decode_latent   absorbed multi-head latent attention decode
 *   mla_decode_latent_paged   the same over a paged latent pool
 *   mla_absorb_q, mla_up_proj the per-head projections around it
 *   kv_append           push of new K/V rows into a cache or pool
 *   mla_append_latent   push of an MLA latent row, k_rot rotated once
 *
 * What is computed (kopitiam-runtime 0.2.4, src/attention.rs, module doc
 * "Grouped-query attention" and "Causal masking", fns repeat_kv_heads,
 * causal_mask, attention_forward):
 *   query head h reads KV head h / (n_heads / n_kv_heads); the query at
 *   row i sits at absolute position position_offset + i and attends to keys
 *   j = 0 .. position_offset + i (and j < seq_kv);
 *   o[i,h,:] = sum_j softmax_j(attention_scale * q[i,h,:] . k[j,h/G,:]) v[j,h/G,:].
 * attention_scale is the whole logit multiplier (kopitiam uses 1/sqrt(head_dim);
 * frink-models 0.31.0 src/mla/mod.rs passes the scale explicitly).
 * Decode is push-then-attend (frink-models 0.38.0 src/decoder/attn_block.rs,
 * push_and_attend_row): the caller has already written this step's K/V, and
 * the query of sequence b sits at position seq_lens[b] - 1.
 *
 * Conventions shared by every entry point:
 *  - dtype is a pkva_dtype code. Inputs and outputs use it; accumulation and
 *    softmax are always fp32. bf16 outputs are rounded to nearest even.
 *  - All tensors are dense, row-major, token-major, in DEVICE memory, owned by
 *    the caller. Index arrays (block_table, seq_lens) are device int32.
 *    The library never allocates, frees or synchronises; work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns as
 *    soon as it is enqueued.
 *  - Host-side validation runs before any HIP call. On a non-zero return
 *    nothing was enqueued. Return codes:
 *      PKVA_OK           enqueued
 *      PKVA_EINVAL       a required pointer is NULL, a size is out of range,
 *                        n_kv_heads does not divide n_heads, the scale is not
 *                        finite or is negative, ...
 *      PKVA_EUNSUPPORTED dtype code unknown, or (dtype, head size) combination
 *                        not built (see each entry point)
 *      PKVA_EWORKSPACE   workspace NULL or smaller than the *_workspace_size call
 *      PKVA_EHIP         the kernel launch failed
 *      PKVA_ESCRATCH     (attn_decode_paged_noalloc only) the sizes need more
 *                        than the library's fixed scratch array holds
 *  - Device-side data errors never cause an out-of-bounds access: a sequence
 *    whose seq_lens entry is outside [1, max_seq_len], or whose block table
 *    names a block outside [0, num_blocks) among the blocks it needs, gets
 *    NaN in every output element of that sequence (prefill: of the affected
 *    query rows' heads).
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs on every call, and attn_decode_contig and attn_decode_paged give
 *    bitwise-identical outputs for the same cache rows (frink-models 0.38.0
 *    src/decoder/attn_block.rs, doc of push_and_attend_row: paging changes
 *    where rows live and nothing else).
 *  - The library's only global state is a per-device cache of launch facts
 *    (compute units, resident workgroups) and the scratch array of
 *    attn_decode_paged_noalloc; calls are thread-safe. Calls that share a
 *    workspace must be ordered on one stream.
 */
#ifndef PKVATTN_H
#define PKVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKVA_F32 = 0, PKVA_BF16 = 1 } pkva_dtype;

enum {
  PKVA_OK = 0,
  PKVA_EINVAL = 1,
  PKVA_EUNSUPPORTED = 2,
  PKVA_EWORKSPACE = 3,
  PKVA_EHIP = 4,
  PKVA_ESCRATCH = 5
};

/* A static, human-readable name for a return code ("unknown status" otherwise). */
const char* pkva_status_string(int status);

/* The library's version string, e.g. "pkvattn 0.1.0 gfx950". */
const char* pkva_version(void);

/*
 * attn_prefill: causal GQA for a batch of sequences that share seq_q, seq_kv
 * and position_offset (kopitiam-runtime 0.2.4 src/attention.rs,
 * attention_forward and causal_mask; the same mask serves a prompt prefill,
 * position_offset == 0, and a chunk after cached tokens).
 *
 *   q  [batch, seq_q, n_heads, head_dim]              (dtype)
 *   o  [batch, seq_q, n_heads, head_dim]              (dtype, written)
 *   Contiguous K/V (block_table == NULL):
 *     k, v  [batch, kv_capacity, n_kv_heads, head_dim], rows 0..seq_kv-1 used;
 *     requires seq_kv <= kv_capacity. max_blocks_per_seq, block_size and
 *     num_blocks are ignored.
 *   Paged K/V (block_table != NULL):
 *     k, v  pools [num_blocks, block_size, n_kv_heads, head_dim];
 *     block_table [batch, max_blocks_per_seq] int32; token t of sequence b is
 *     row t % block_size of block block_table[b][t / block_size];
 *     requires block_size a power of two and
 *     seq_kv <= max_blocks_per_seq * block_size. kv_capacity is ignored.
 *   Row i of q sits at absolute position position_offset + i and sees keys
 *   0 .. min(position_offset + i, seq_kv - 1). Key 0 is always visible.
 *   Requires batch, n_heads, n_kv_heads, seq_q, seq_kv >= 1,
 *   n_heads % n_kv_heads == 0, position_offset >= 0.
 *   Built: (PKVA_F32, head_dim 16), (PKVA_BF16, head_dim 128); others return
 *   PKVA_EUNSUPPORTED.
 */
int attn_prefill(int dtype, const void* q, const void* k, const void* v, void* o,
                 int batch, int n_heads, int n_kv_heads, int head_dim,
                 int seq_q, int seq_kv, int position_offset, float attention_scale,
                 const int32_t* block_table, int max_blocks_per_seq, int block_size,
                 int num_blocks, int kv_capacity, void* stream);

/*
 * attn_prefill_varlen: causal GQA prefill of a ragged batch, every sequence
 * with its own chunk length and history, over one shared cache (the batched
 * and paged multi-sequence caller: frink-models 0.38.0
 * src/decoder/attn_block.rs, KvStep::Batched and KvStep::Paged, "one
 * sequence of a multi-sequence batch"; the mask is kopitiam-runtime 0.2.4
 * src/attention.rs, causal_mask, per sequence).
 *
 *   q, o  [total_q, n_heads, head_dim] (dtype): the chunks' query rows packed
 *         in sequence order.
 *   cu_seqlens_q [batch + 1] int32, device: sequence b owns rows
 *         cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (its chunk length n_b may
 *         be 0); 0 <= cu_seqlens_q[b] <= cu_seqlens_q[b+1] <= total_q.
 *   seq_kv [batch] int32, device: keys of sequence b, its chunk's rows
 *         already pushed as the last n_b of them; row i sits at position
 *         seq_kv[b] - n_b + i and sees keys 0 .. that position.
 *   max_seq_q: host bound on every n_b (sizes the launch).
 *   k, v: pools [num_blocks, block_size, n_kv_heads, head_dim] with
 *         block_table [batch, max_blocks_per_seq] (as attn_prefill), or
 *         contiguous [batch, kv_capacity, n_kv_heads, head_dim] when
 *         block_table is NULL.
 *   Device-side bad data never causes an out-of-bounds access: a sequence
 *   whose rows leave [0, total_q) is skipped (its rows are not written); one
 *   with seq_kv[b] < n_b, seq_kv[b] beyond the cache, n_b > max_seq_q or a
 *   needed block id outside the pool gets NaN rows.
 *   For equal chunk lengths and histories the result is bitwise that of
 *   attn_prefill. Built: as attn_prefill.
 */
int attn_prefill_varlen(int dtype, const void* q, const void* k, const void* v, void* o,
                        int batch, int n_heads, int n_kv_heads, int head_dim,
                        const int32_t* cu_seqlens_q, const int32_t* seq_kv, int total_q,
                        int max_seq_q, float attention_scale, const int32_t* block_table,
                        int max_blocks_per_seq, int block_size, int num_blocks, int kv_capacity,
                        void* stream);

/*
 * Bytes of device workspace attn_decode_contig / attn_decode_paged need for
 * these sizes (the split-K partial results). Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_size(int batch, int n_heads, int n_kv_heads, int head_dim,
                                  int max_seq_len);

/*
 * attn_decode_contig: one query token per sequence over a contiguous cache
 * (frink-models 0.38.0 src/decoder/attn_block.rs, push_and_attend_row,
 * contiguous arm: push this row, then attend over every row the sequence
 * holds).
 *
 *   q        [batch, n_heads, head_dim]                  (dtype)
 *   k_cache, v_cache [batch, kv_capacity, n_kv_heads, head_dim] (dtype)
 *   o        [batch, n_heads, head_dim]                  (dtype, written)
 *   seq_lens [batch] int32, device: keys 0..seq_lens[b]-1 of sequence b,
 *            including the query's own (already appended) key.
 *   max_seq_len: host upper bound on every seq_lens[b]; sizes the launch.
 *            Requires 1 <= max_seq_len <= kv_capacity.
 *   workspace: device memory of at least attn_decode_workspace_size(...)
 *            bytes, contents irrelevant on entry, clobbered on return.
 *   Built: (PKVA_F32, 16), (PKVA_BF16, 128), with n_heads / n_kv_heads <= 8;
 *            a larger group returns PKVA_EUNSUPPORTED.
 */
int attn_decode_contig(int dtype, const void* q, const void* k_cache, const void* v_cache,
                       void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                       const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                       float attention_scale, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * attn_decode_paged: one query token per sequence over a block-table paged
 * cache shared across sequences (frink-models 0.38.0
 * src/decoder/attn_block.rs, push_and_attend_row, paged arm: attend through
 * the sequence's block_table over seq_len keys).
 *
 *   q        [batch, n_heads, head_dim]                          (dtype)
 *   k_pool, v_pool [num_blocks, block_size, n_kv_heads, head_dim] (dtype)
 *   o        [batch, n_heads, head_dim]                          (dtype, written)
 *   block_table [batch, max_blocks_per_seq] int32, device; token t of
 *            sequence b is row t % block_size of block block_table[b][t / block_size].
 *            Entries past the sequence's last needed block are never read.
 *   seq_lens, max_seq_len, workspace: as attn_decode_contig; requires
 *            max_seq_len <= max_blocks_per_seq * block_size and block_size a
 *            power of two.
 *   For the same rows, the result is bitwise identical to attn_decode_contig.
 *   Built: as attn_decode_contig.
 */
int attn_decode_paged(int dtype, const void* q, const void* k_pool, const void* v_pool,
                      void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      int num_blocks, const int32_t* seq_lens, int max_seq_len,
                      float attention_scale, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * The optional arms of one attention layer (frink-models 0.38.0
 * src/decoder/attn_block.rs, push_and_attend_row: one kernel serves plain,
 * windowed, softcapped and sink-bearing layers, with ALiBi slopes, at the
 * cache's own key and value widths). The page names them; the readings are
 * their usual definitions. For the query at position p and key j <= p:
 *   window > 0      only keys with p - window < j <= p are visible; 0: all
 *   softcap > 0     logit x = attention_scale * q.k becomes
 *                   softcap * tanh(x / softcap); 0: off
 *   alibi_slopes    device float [n_heads] or NULL: head h adds
 *                   alibi_slopes[h] * (j - p) to its logits (after softcap)
 *   sinks           device float [n_heads] or NULL: head h's softmax also
 *                   counts exp(sinks[h]), a logit with no value, so its key
 *                   weights sum to less than one
 *   v_head_dim      width of the V rows and of o; 0 means head_dim (the K
 *                   and q width)
 */
typedef struct pkva_arms {
  int window;
  float softcap;
  const float* alibi_slopes;
  const float* sinks;
  int v_head_dim;
} pkva_arms;

/*
 * attn_decode_contig_ext / attn_decode_paged_ext: attn_decode_contig /
 * attn_decode_paged with the arms above (arms must not be NULL; all arms off
 * gives the plain result up to rounding). Layouts as the plain calls, with
 * V rows [.., n_kv_heads, v_head_dim] and o [batch, n_heads, v_head_dim];
 * the workspace is attn_decode_workspace_size(batch, n_heads, n_kv_heads,
 * v_head_dim, max_seq_len). For the same rows and arms the two give
 * bitwise-identical results.
 *   Built: (PKVA_BF16, head_dim 128 or 192, v_head_dim 128),
 *          (PKVA_F32, 16, 16); group sizes as the plain calls.
 *   PKVA_EINVAL also for a negative window or v_head_dim, or a softcap that
 *   is negative or not finite.
 */
int attn_decode_contig_ext(int dtype, const void* q, const void* k_cache, const void* v_cache,
                           void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                           const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                           float attention_scale, const pkva_arms* arms, void* workspace,
                           size_t workspace_bytes, void* stream);
int attn_decode_paged_ext(int dtype, const void* q, const void* k_pool, const void* v_pool,
                          void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                          const int32_t* block_table, int max_blocks_per_seq, int block_size,
                          int num_blocks, const int32_t* seq_lens, int max_seq_len,
                          float attention_scale, const pkva_arms* arms, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc: attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, layouts, validation and
 * results (bitwise) as attn_decode_paged, without the workspace arguments:
 * the split partials live in a fixed device array inside the library
 * (64 MiB, one copy per device that runs the library, held until the
 * process ends). The call allocates nothing. It needs
 * attn_decode_workspace_size(batch, n_heads, n_kv_heads, head_dim,
 * max_seq_len) <= 64 MiB (e.g. the 64-sequence, 32-head, D=128, 8192-token
 * workload takes 35 MB) and returns PKVA_ESCRATCH otherwise. Every call on a
 * device shares that device's array: calls that overlap on one device (two
 * streams, two threads) race and must be ordered by the caller. The first
 * call on a device looks up the array's device address (a HIP call that
 * enqueues nothing); the call uses the current device, which must be the
 * device of `stream`.
 */
int attn_decode_paged_noalloc(int dtype, const void* q, const void* k_pool, const void* v_pool,
                              void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                              const int32_t* block_table, int max_blocks_per_seq, int block_size,
                              int num_blocks, const int32_t* seq_lens, int max_seq_len,
                              float attention_scale, void* stream);

/*
 * mla_decode_latent_paged: mla_decode_latent over a block-table paged latent
 * pool (the latent cache of frink-models 0.31.0 src/mla/mod.rs,
 * MlaKvB::Split, "[seq, kv_lora_rank + qk_rope]", laid out in pages as the
 * K/V pools of attn_decode_paged).
 *
 *   latent_pool [num_blocks, block_size, kv_lora_rank + qk_rope_head_dim];
 *   block_table [batch, max_blocks_per_seq] int32 device; token t of
 *   sequence b is row t % block_size of block block_table[b][t / block_size].
 *   block_size a power of two; max_seq_len <= max_blocks_per_seq *
 *   block_size. A sequence with a needed block id outside [0, num_blocks)
 *   gets NaN rows. Other arguments, workspace and results as
 *   mla_decode_latent (bitwise equal for the same rows).
 */
int mla_decode_latent_paged(int dtype, const void* q_abs, const void* latent_pool, void* o_lat,
                            int batch, int n_heads, int kv_lora_rank, int qk_rope_head_dim,
                            const int32_t* block_table, int max_blocks_per_seq, int block_size,
                            int num_blocks, const int32_t* seq_lens, int max_seq_len,
                            float attention_scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * mla_absorb_q: the absorbed query of frink-models 0.31.0 src/mla/mod.rs,
 * absorbed_attention: q_abs[b, h] = [k_b[h] . q_nope[b, h] | q_rot[b, h]],
 * with one weight matrix per head in the absorb direction (MlaKvB::Split
 * doc: k_b[h] is [kv_lora_rank, qk_nope]).
 *   q      [batch, n_heads, qk_nope_head_dim + qk_rope_head_dim] (nope first)
 *   k_b    [n_heads, kv_lora_rank, qk_nope_head_dim]
 *   q_abs  [batch, n_heads, kv_lora_rank + qk_rope_head_dim] (written)
 *   bf16 only, fp32 accumulation, output rounded to nearest even. Built for
 *   qk_nope_head_dim % 16 == 0, kv_lora_rank % 32 == 0,
 *   qk_rope_head_dim % 8 == 0 (else PKVA_EUNSUPPORTED); pointers 16-byte
 *   aligned (else PKVA_EINVAL).
 */
int mla_absorb_q(int dtype, const void* q, const void* k_b, void* q_abs, int batch, int n_heads,
                 int qk_nope_head_dim, int qk_rope_head_dim, int kv_lora_rank, void* stream);

/*
 * mla_up_proj: the per-head value up-projection after the latent attention
 * (absorbed_attention's last loop): out[b, h] = v_b[h] . o_lat[b, h], with
 * v_b[h] [v_head_dim, kv_lora_rank] (MlaKvB::Split doc).
 *   o_lat  [batch, n_heads, kv_lora_rank]
 *   v_b    [n_heads, v_head_dim, kv_lora_rank]
 *   out    [batch, n_heads, v_head_dim] (written)
 *   bf16 only, fp32 accumulation. Built for kv_lora_rank % 16 == 0,
 *   v_head_dim % 32 == 0; pointers 16-byte aligned.
 */
int mla_up_proj(int dtype, const void* o_lat, const void* v_b, void* out, int batch, int n_heads,
                int kv_lora_rank, int v_head_dim, void* stream);

/*
 * kv_append: the push of push-then-attend. Writes n_new K and V rows per
 * sequence into a contiguous cache or a block-table pool, before an
 * attention call reads them (frink-models 0.38.0 src/decoder/attn_block.rs,
 * push_and_attend_row: the row is pushed to whichever backing, then
 * attended; kopitiam-runtime 0.2.4 src/attention.rs, attention_forward
 * appends to the cache before scoring).
 *
 *   k_new, v_new [batch, n_new, n_kv_heads, head_dim]   (dtype)
 *   positions [batch] int32, device: rows sequence b holds before the push;
 *            row i becomes token positions[b] + i.
 *   Contiguous (block_table == NULL): k_cache, v_cache
 *            [batch, kv_capacity, n_kv_heads, head_dim]; token t of b is row
 *            (b, t). max_blocks_per_seq, block_size, num_blocks are ignored.
 *   Paged (block_table != NULL): pools [num_blocks, block_size, n_kv_heads,
 *            head_dim], block_table [batch, max_blocks_per_seq] int32 device;
 *            token t of b is row t % block_size of block
 *            block_table[b][t / block_size] (the caller reserves the blocks
 *            first). block_size a power of two; kv_capacity is ignored.
 *   The rows are copied bit for bit; any dtype code and head size. A row
 *   whose target lies outside the cache (negative position, past kv_capacity
 *   or the table, or a block id outside [0, num_blocks)) is not written.
 *   Afterwards the attention calls take seq_lens[b] = positions[b] + n_new.
 */
int kv_append(int dtype, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              int batch, int n_kv_heads, int head_dim, int n_new, const int32_t* positions,
              const int32_t* block_table, int max_blocks_per_seq, int block_size, int num_blocks,
              int kv_capacity, void* stream);

/*
 * mla_append_latent: the push of one MLA latent row per sequence
 * (frink-models 0.31.0 src/mla/mod.rs, mla_forward_token and
 * absorbed_attention): the row [c | rope(k_rot)] of width
 * kv_lora_rank + qk_rope_head_dim, where k_rot, shared by every head, is
 * rotated once at the row's position with the interleaved convention (module
 * doc point 2, rotate_pe): pair (x[2i], x[2i+1]) turns by
 * position * rope_theta^(-2i / qk_rope_head_dim). rope_theta <= 0 stores
 * k_rot as given (the rope-free configuration, module doc point 1).
 *
 *   c_new     [batch, kv_lora_rank]        (dtype), copied bit for bit
 *   k_rot_new [batch, qk_rope_head_dim]    (dtype), not yet rotated; the
 *             rotation runs in double precision and is rounded once
 *             (nearest even) to the dtype
 *   positions [batch] int32, device: the row becomes token positions[b]
 *   latent: contiguous [batch, kv_capacity, R + P] (block_table == NULL) or a
 *           pool [num_blocks, block_size, R + P] with block_table as in
 *           kv_append. Out-of-cache targets are not written.
 *   qk_rope_head_dim must be even (0 allowed); rope_theta finite.
 */
int mla_append_latent(int dtype, const void* c_new, const void* k_rot_new, void* latent,
                      int batch, int kv_lora_rank, int qk_rope_head_dim,
                      const int32_t* positions, float rope_theta, const int32_t* block_table,
                      int max_blocks_per_seq, int block_size, int num_blocks, int kv_capacity,
                      void* stream);

/*
 * Bytes of device workspace mla_decode_latent needs. Returns 0 for invalid sizes.
 */
size_t mla_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int max_seq_len);

/*
 * mla_decode_latent: absorbed multi-head latent attention decode
 * (frink-models 0.31.0 src/mla/mod.rs, absorbed_attention and the MlaKvB
 * doc): multi-query attention in which every head's key is the whole cached
 * latent row [c | k_rot] (width kv_lora_rank + qk_rope_head_dim) and its
 * value is the row's first kv_lora_rank entries.
 *
 *   q_abs   [batch, n_heads, kv_lora_rank + qk_rope_head_dim] (dtype): per head
 *           the absorbed nope part (kv_lora_rank) then the rotated rope part.
 *   latent  [batch, kv_capacity, kv_lora_rank + qk_rope_head_dim] (dtype).
 *   o_lat   [batch, n_heads, kv_lora_rank] (dtype, written): the softmax-weighted
 *           latent, before the per-head value up-projection.
 *   seq_lens, max_seq_len: as attn_decode_contig (the latent row of the
 *           current token is already appended).
 *   workspace: device memory of at least mla_decode_workspace_size(...) bytes,
 *           16-byte aligned, owned by the caller, contents overwritten; may be
 *           null when that size is 0 (the batch fills the GPU without
 *           splitting the context). With a split context each piece leaves
 *           its output divided by its own softmax sum in bf16 plus its max
 *           and sum in fp32, and a second kernel merges the pieces.
 *   Built: PKVA_BF16 with kv_lora_rank 512, qk_rope_head_dim 64, n_heads
 *           from 1 to 128 or a multiple of 128. A workgroup always serves 128
 *           heads, so a smaller head count costs about what 128 heads cost.
 */
int mla_decode_latent(int dtype, const void* q_abs, const void* latent, void* o_lat,
                      int batch, int n_heads, int kv_lora_rank, int qk_rope_head_dim,
                      const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                      float attention_scale, void* workspace, size_t workspace_bytes,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKVATTN_H */
