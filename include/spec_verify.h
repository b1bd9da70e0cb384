/*
 * spec_verify.h -- C ABI of the speculative-decoding verification step on
 * AMD Instinct MI355X (gfx950).
 *
 * The verification step scores the D drafted tokens of each sequence plus one
 * bonus position in a single target pass, then keeps the drafts up to the first
 * one the target disagrees with.  The calls:
 *
 *   spec_kv_append     writes the K/V rows of the new positions into the paged
 *                      cache (e4m3 caches: quantize on write) and grows the
 *                      lengths; the step before attention.
 *   spec_verify_attn   attention of the R = D + 1 new positions of every
 *                      sequence over its paged KV cache (GQA: G = H_q / H_kv
 *                      query heads share one KV head, so G * R query rows read
 *                      each KV head), with an online softmax and a split-K
 *                      merge for long contexts.
 *   spec_accept        per-row argmax of the target logits, first-mismatch
 *                      prefix against the drafts, acceptance length and the
 *                      committed KV length.
 *   spec_verify_attn_tree, spec_accept_tree, spec_kv_commit_tree
 *                      the same steps for a tree of drafts instead of a chain, and
 *                      the move of the accepted nodes' K/V behind the root.
 *   spec_accept_sampled  the same for sampled decoding: lossless stochastic
 *                      acceptance of the drafts and a draw of the next token.
 *   spec_draft_signals confidence and entropy of the draft's distribution and
 *                      the draft length for the next step.
 *
 * Where the operations are defined (the pages this library implements):
 *   - one target pass over the drafted positions plus the bonus position, and
 *     the acceptance rule: "GPU and LLM", chapter 5 (animemo.app), section
 *     "Speculative decoding (2): verify in one pass"; NVIDIA co-design summary
 *     (papanda925.com), section "Basic structure of speculative decoding"
 *     (draft length D, acceptance length AL in 1 .. 1 + D);
 *   - the running max / running sum softmax: "GPU and LLM" ch. 5, section
 *     "Online softmax: carry the max and the sum";
 *   - grouped KV heads: "GPU and LLM" ch. 5, section "GQA";
 *   - 16-token KV blocks behind a block table: "GPU and LLM" ch. 5, section
 *     "PagedAttention (2)";
 *   - FP8 KV storage with scaling factors: novita.ai blog "Revolutionizing LLM
 *     inference: speculative decoding and low-precision quantization",
 *     sections "Proprietary FP8 quantization scheme" and "KVCache quantization".
 *
 * General rules for every call:
 *   - All tensor arguments are device pointers to dense row-major arrays that
 *     the caller allocates and owns.  The library never allocates, frees or
 *     synchronizes, keeps no state between calls and is safe to call from
 *     several host threads.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *     Outputs are valid once that stream has been synchronized.
 *   - Every argument check the host can make (NULL pointers, sizes, shapes,
 *     alignment, support, workspace size) happens before anything is launched;
 *     a failed check returns an error code, launches nothing and records a
 *     message retrievable with sv_last_error() on the calling thread.
 *   - Data on the device is not checked (it would need a synchronization).
 *     The preconditions are stated per call; breaking them gives unspecified
 *     output values but never an access outside the buffers described here.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_INVALID = 1,     /* a pointer, size, shape or alignment argument is invalid */
  SV_ERR_WORKSPACE = 2,   /* the workspace is missing or smaller than required */
  SV_ERR_UNSUPPORTED = 3, /* well formed, but not a supported configuration */
  SV_ERR_LAUNCH = 4       /* the HIP runtime reported an error for a launch */
} sv_status;

typedef enum sv_kv_dtype {
  SV_KV_BF16 = 0,         /* bfloat16 K and V */
  SV_KV_FP8_E4M3 = 1      /* OCP e4m3 codes, one fp32 scale per (block, KV head) */
} sv_kv_dtype;

/* Shape and options of one spec_verify_attn call.  Sizes are element counts. */
typedef struct sv_attn_params {
  int32_t batch;              /* B >= 1 sequences */
  int32_t draft_len;          /* D in [0, 63]; R = D + 1 query positions per sequence */
  int32_t num_q_heads;        /* H_q >= 1 */
  int32_t num_kv_heads;       /* H_kv >= 1, divides H_q; G = H_q / H_kv */
  int32_t head_dim;           /* hd: 64 or 128 */
  int32_t block_size;         /* tokens per KV block: must be 16 */
  int32_t max_blocks_per_seq; /* columns of block_table, >= ceil(max_kv_len / 16) */
  int32_t num_blocks;         /* physical blocks in each cache, >= 1 */
  int32_t max_kv_len;         /* upper bound on every kv_lens[b], >= R; sizes the
                                 launch grid and the workspace on the host */
  int32_t kv_dtype;           /* an sv_kv_dtype */
  float sm_scale;             /* softmax scale applied to q.k, > 0 (usually 1/sqrt(hd)) */
  int32_t split_tokens;       /* keys per split-K partition: 0 = chosen by the
                                 library, else a positive multiple of 64 */
} sv_attn_params;

/*
 * Bytes of device workspace spec_verify_attn needs for `p`.  May be 0.
 * Returns SV_ERR_INVALID / SV_ERR_UNSUPPORTED for parameters spec_verify_attn
 * would reject.
 */
sv_status spec_verify_attn_workspace_size(const sv_attn_params* p, size_t* bytes);

/*
 * Attention of the R = D + 1 newest positions of every sequence.
 *
 * For sequence b with L_b = kv_lens[b] keys (the context plus the R new
 * positions, whose K and V are already in the cache), position i in 0..D,
 * query head h and its KV head kvh = h / G:
 *     s_t = sm_scale * q[b][i][h] . K_b[t][kvh]         for t = 0 .. L_b - R + i
 *     out[b][i][h] = sum_t softmax(s)_t * V_b[t][kvh]
 * computed with a running max and running sum over key tiles; key ranges of
 * `split_tokens` keys are processed independently and merged with the same
 * rescaling rule.  Accumulation is fp32; out is rounded to bf16 (nearest even).
 *
 *   q            [B][R][H_q][hd] bf16.                                16-byte aligned.
 *   k_cache      bf16: [num_blocks][H_kv][hd/8][16][8]  (16-byte vectors of 8
 *                      dims per token: element (blk, kvh, token slot s, dim d)
 *                      is at ((blk*H_kv + kvh)*hd/8 + d/8)*128 + s*8 + d%8)
 *                e4m3: [num_blocks][H_kv][hd/16][16][16] (uint8 codes; element
 *                      at ((blk*H_kv + kvh)*hd/16 + d/16)*256 + s*16 + d%16).
 *                                                                 16-byte aligned.
 *   v_cache      [num_blocks][H_kv][hd][16]: element (blk, kvh, s, d) is at
 *                ((blk*H_kv + kvh)*hd + d)*16 + s; bf16 or uint8 e4m3 codes.
 *                                                                 16-byte aligned.
 *   k_scale,     [num_blocks][H_kv] fp32: the value of an e4m3 code is
 *   v_scale      decode(code) * scale[blk][kvh].  Required for e4m3, must be
 *                NULL for bf16.
 *   block_table  [B][max_blocks_per_seq] int32: token t of sequence b is in
 *                physical block block_table[b][t / 16], slot t % 16.
 *   kv_lens      [B] int32, L_b.
 *   out          [B][R][H_q][hd] bf16, written.  16-byte aligned; must not
 *                overlap any input.
 *   workspace    device memory of at least spec_verify_attn_workspace_size()
 *                bytes (may be NULL when that size is 0), 256-byte aligned;
 *                contents on entry are ignored.
 *
 * Size limits (SV_ERR_UNSUPPORTED beyond them): B*R*H_q*hd < 2^31 elements;
 * H_kv*hd*32 < 2^31 (bytes of one physical block of a bf16 cache, all KV
 * heads); num_blocks*H_kv < 2^32 (entries of a scale array); for B <= 2048,
 * B*H_kv*U*ceil(max_kv_len/32) < 2^31 (32-key tiles of the whole batch), with
 * M = G*R rows per KV head and U its row units: ceil(M/256) for a bf16 cache
 * with M > 128, M != 256 and M mod 256 either 0 or above 128, else
 * ceil(M/128).
 *
 * Device preconditions: R <= kv_lens[b] <= max_kv_len; block_table[b][j] in
 * [0, num_blocks) for j < ceil(kv_lens[b] / 16).  The other entries of the
 * table (all B x max_blocks_per_seq of which must be readable) may hold
 * anything: they may be read, clamped into [0, num_blocks), but what they
 * point at only meets keys past kv_lens[b], which never reach the output.
 * K and V slots past kv_lens[b] may hold anything, NaN included.
 */
sv_status spec_verify_attn(const sv_attn_params* p, const void* q, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* kv_lens, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tree verification: attention of R = D + 1 draft-tree nodes instead of a chain
 * of drafts.  The pages' drafter proposes several candidates per position and
 * the target scores them grouped in one pass (novita.ai blog, section
 * "Implementation": candidate generation and batch verification); the tree
 * layout below is this library's.
 *
 * Node j of sequence b is new position j: its K and V are at token
 * L_b - R + j of the cache (node 0 is the last committed token, the root) and
 * its query is q[b][j].  Node i sees every context key (t < L_b - R) and the
 * nodes set in tree_mask[b][i]: bit j set iff node j is node i or one of its
 * ancestors.  Everything else is as for spec_verify_attn (same parameters,
 * layouts, workspace size and preconditions); a chain tree, mask[i] =
 * 2^(i+1) - 1, gives spec_verify_attn's result.
 *
 *   tree_mask  [B][R] uint64, 8-byte aligned.  Precondition: bit i of
 *              tree_mask[b][i] is set and no bit above i is set (nodes in
 *              topological order, parents before children); bits at or above R
 *              are ignored.
 * Errors: as spec_verify_attn; SV_ERR_INVALID for a NULL or misaligned
 * tree_mask.
 */
sv_status spec_verify_attn_tree(const sv_attn_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_table, const int32_t* kv_lens,
                                const uint64_t* tree_mask, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Bytes of device workspace spec_accept needs for (batch, draft_len, vocab). */
sv_status spec_accept_workspace_size(int32_t batch, int32_t draft_len, int32_t vocab,
                                     size_t* bytes);

/*
 * Greedy acceptance.
 *
 * For sequence b and row j in 0..D (row j is the target's prediction after
 * input position j; row D is the bonus position):
 *     target_tokens[b][j] = lowest v with logits[b][j][v] = max_v logits[b][j][v]
 *                           (fp32 compares, so -0 == +0; all -inf -> 0)
 *     n  = first j < D with draft[b][j] != target_tokens[b][j], else D
 *     accept_len[b]  = n + 1                                  (1 .. 1 + D)
 *     out_tokens[b]  = draft[b][0..n) , target_tokens[b][n] , -1 padding
 *     kv_lens_out[b] = kv_lens_in[b] - (1 + D) + accept_len[b]
 *
 *   logits         [B][1+D][V] fp32; 16-byte aligned.  Finite or -inf (NaN
 *                  gives unspecified tokens).
 *   draft          [B][D] int32 (may be NULL when D = 0).  Ids outside [0, V)
 *                  are allowed and never match.
 *   target_tokens  [B][1+D] int32, written.
 *   accept_len     [B] int32, written.
 *   out_tokens     [B][1+D] int32, written.
 *   kv_lens_in     [B] int32, read.
 *   kv_lens_out    [B] int32, written; may be the same pointer as kv_lens_in
 *                  (in-place commit).
 *   workspace      at least spec_accept_workspace_size() bytes, 256-byte aligned;
 *                  contents on entry are ignored.
 */
sv_status spec_accept(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                      const int32_t* draft, int32_t* target_tokens, int32_t* accept_len,
                      int32_t* out_tokens, const int32_t* kv_lens_in, int32_t* kv_lens_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_accept without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus the workspace), results and
 * errors as spec_accept, same kernels.  The per-chunk results live in a fixed
 * device array of the library instead of a workspace: 4 MiB on each GPU it
 * runs on, held until the process ends, its address looked up once per device
 * on the first call there.  The call allocates nothing and calls no allocating
 * routine; every call overwrites the entries it reads, so nothing is cleared
 * between calls.  Every call on a GPU uses that GPU's one array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and give
 * unspecified results.
 * Limit: batch * (1 + draft_len) * ceil(vocab / 4096) * 8 bytes <= 4 MiB
 * (e.g. 512 rows of a 128256-token vocabulary use 128 KiB); SV_ERR_UNSUPPORTED
 * beyond it.
 */
sv_status spec_accept_noalloc(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                              const int32_t* draft, int32_t* target_tokens, int32_t* accept_len,
                              int32_t* out_tokens, const int32_t* kv_lens_in,
                              int32_t* kv_lens_out, void* stream);

/*
 * Greedy acceptance over a draft tree (the nodes scored by spec_verify_attn_tree).
 *
 * For sequence b with R = D + 1 nodes (node 0 = the root, the last committed
 * token; parents[b][j] < j for j >= 1):
 *     target_tokens[b][j] = argmax of logits[b][j] (lowest index on ties, as in
 *                           spec_accept): the target's token after node j
 *     walk from the root: while the current node i has a child c with
 *         tokens[b][c] == target_tokens[b][i], step to the lowest such c
 *     accept_path[b] = the nodes walked, root first, -1 padding
 *     accept_len[b]  = their number (1 .. 1 + tree depth)
 *     out_tokens[b]  = tokens of the walked nodes after the root, then the
 *                      target token of the last one, -1 padding
 *     kv_lens_out[b] = kv_lens_in[b] - (1 + D) + accept_len[b]
 * The accepted nodes' K/V rows are at new positions accept_path[b][1..]; the
 * committed length counts them as positions 1 .. accept_len - 1 after the root,
 * where the caller moves them (for a chain tree they are already in place).
 *
 *   logits      [B][1+D][V] fp32, 16-byte aligned (as spec_accept).
 *   tokens      [B][1+D] int32: the draft token of each node (entry 0 unused).
 *   parents     [B][1+D] int32: each node's parent (entry 0 unused); a parent
 *               outside [0, j) simply never lets node j be walked to.
 *               tokens and parents may be NULL when draft_len = 0.
 *   accept_path [B][1+D] int32, written.
 *   target_tokens, accept_len, out_tokens, kv_lens_in, kv_lens_out and the
 *   workspace (spec_accept_workspace_size bytes) as for spec_accept.
 */
sv_status spec_accept_tree(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                           const int32_t* tokens, const int32_t* parents, int32_t* target_tokens,
                           int32_t* accept_len, int32_t* out_tokens, int32_t* accept_path,
                           const int32_t* kv_lens_in, int32_t* kv_lens_out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of device workspace spec_accept_sampled needs for (batch, draft_len, vocab). */
sv_status spec_accept_sampled_workspace_size(int32_t batch, int32_t draft_len, int32_t vocab,
                                             size_t* bytes);

/*
 * Stochastic (lossless) acceptance: the emitted tokens follow the target's own
 * distribution ("GPU and LLM" ch. 5, section "Speculative decoding (2)"), by the
 * rule of the paper the pages cite there (Leviathan et al.).
 *
 * For sequence b, with p_j = softmax(target_logits[b][j] / temperature) for j in
 * 0..D and q_j = softmax(draft_logits[b][j] / temperature) for j < D:
 *     draft j is kept iff  u_accept[b][j] * q_j(d_j) < p_j(d_j)   (d_j = draft[b][j])
 *     n = first j < D whose draft is not kept, else D
 *     the emitted token is drawn with u = u_sample[b] from
 *         max(0, p_n - q_n)   when n < D (p_n itself if that is zero everywhere),
 *         p_D                 when n = D;
 *     drawing from weights w: the first v whose running sum of w exceeds u * sum(w)
 *     accept_len[b]  = n + 1
 *     out_tokens[b]  = draft[b][0..n) , emitted token , -1 padding
 *     kv_lens_out[b] = kv_lens_in[b] - (1 + D) + accept_len[b]
 * The GPU evaluates p and q from fp32 exponentials with fp64 sums; a decision
 * whose margin lies within that rounding (about 1e-6 relative) may differ from
 * an exact evaluation.
 *
 *   temperature    > 0, finite.
 *   target_logits  [B][1+D][V] fp32, 16-byte aligned.  Finite or -inf, at least
 *                  one finite value per row.
 *   draft_logits   [B][D][V] fp32, 16-byte aligned: the draft model's logits the
 *                  drafts were drawn from (same conditions; NULL when D = 0).
 *   draft          [B][D] int32 (NULL when D = 0); ids are clamped into [0, V)
 *                  for the keep test and copied unchanged into out_tokens.
 *   u_accept       [B][D] fp32 uniforms in [0, 1) (NULL when D = 0).
 *   u_sample       [B] fp32 uniforms in [0, 1).
 *   accept_len, out_tokens, kv_lens_in, kv_lens_out as for spec_accept
 *                  (kv_lens_out may alias kv_lens_in).
 *   workspace      at least spec_accept_sampled_workspace_size() bytes,
 *                  256-byte aligned.
 * Errors: SV_ERR_INVALID for shapes, temperature, NULL or misaligned pointers;
 * SV_ERR_UNSUPPORTED when batch * (1 + 2 draft_len) > 65535; SV_ERR_WORKSPACE.
 */
sv_status spec_accept_sampled(int32_t batch, int32_t draft_len, int32_t vocab, float temperature,
                              const float* target_logits, const float* draft_logits,
                              const int32_t* draft, const float* u_accept, const float* u_sample,
                              int32_t* accept_len, int32_t* out_tokens, const int32_t* kv_lens_in,
                              int32_t* kv_lens_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Shape of one spec_kv_append call.  Sizes are element counts. */
typedef struct sv_append_params {
  int32_t batch;              /* B >= 1 sequences */
  int32_t num_new;            /* R >= 1 rows appended per sequence (1 + D at a
                                 verification step), <= 16 * max_blocks_per_seq */
  int32_t num_kv_heads;       /* H_kv >= 1 */
  int32_t head_dim;           /* hd: 64 or 128 */
  int32_t block_size;         /* tokens per KV block: must be 16 */
  int32_t max_blocks_per_seq; /* columns of block_table, 16 * max_blocks_per_seq < 2^31 */
  int32_t num_blocks;         /* physical blocks in each cache, >= 1 */
  int32_t kv_dtype;           /* an sv_kv_dtype */
} sv_append_params;

/*
 * KV append: the step before spec_verify_attn.  The K and V rows of the R new
 * positions of every sequence are written into its paged cache at token
 * positions c_b .. c_b + R - 1, c_b = kv_lens_in[b] (the committed length), and
 * kv_lens_out[b] = c_b + R, the L_b spec_verify_attn takes.  Rejected drafts need
 * no undo here: spec_accept lowers the length, and the next append writes over
 * the slots past it.  Paged blocks: "GPU and LLM" ch. 5, section "PagedAttention
 * (2)"; FP8 KV with scaling factors, updated as the cache grows: novita.ai blog,
 * sections "Proprietary FP8 quantization scheme" and "KVCache quantization".
 *
 * bf16 caches: the rows are stored as given.
 * e4m3 caches, per (physical block, KV head), for K and V separately, with
 * a = slots of the block held before the call and amax_new = the largest
 * |value| appended to the block:
 *   - a = 0 (the block starts here): scale = amax_new / 448 (1 if amax_new = 0);
 *   - a > 0, amax_new <= fp32(max_held |decode(code)| * scale): scale and held
 *     codes stay;
 *   - otherwise scale = amax_new / 448 and every held code is re-encoded from
 *     fp32(decode(code) * old scale).
 *   A value x is stored as e4m3(fp32(x / scale)): the nearest e4m3 value, ties to
 *   the even code, magnitudes of 448 and above saturated to 448, sign bit of the
 *   quotient.  Slots other than those written, and the scales of blocks not
 *   written, keep their bytes.
 *
 *   k_new, v_new   [B][R][H_kv][hd] bf16, finite.                  16-byte aligned.
 *   k_cache, v_cache, k_scale, v_scale, block_table: layouts as for
 *                  spec_verify_attn (scales required for e4m3, NULL for bf16);
 *                  caches 16-byte aligned.  Read and written.
 *   kv_lens_in     [B] int32, c_b.
 *   kv_lens_out    [B] int32, written c_b + R; may be the same pointer as
 *                  kv_lens_in.
 *
 * Device preconditions: 0 <= c_b <= 16 * max_blocks_per_seq - R;
 * block_table[b][j] in [0, num_blocks) for the blocks j = c_b / 16 ..
 * (c_b + R - 1) / 16, and no physical block written by this call appears in
 * two of those places; the held slots of a block whose scale is in use hold
 * finite codes.  A length outside its range is clamped (giving kv_lens_out =
 * clamped length + R) and table entries are clamped into [0, num_blocks), so
 * no access leaves the buffers.
 * Errors: SV_ERR_INVALID for shapes, NULL or misaligned pointers, scales given
 * for bf16 or missing for e4m3; SV_ERR_UNSUPPORTED for head_dim or block_size.
 */
sv_status spec_kv_append(const sv_append_params* p, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* block_table, const int32_t* kv_lens_in,
                         int32_t* kv_lens_out, void* stream);

/*
 * Tree commit: the KV step after spec_accept_tree.  With kv_lens[b] already
 * committed to L_b - R + AL (spec_accept_tree's kv_lens_out), the rows of the
 * accepted nodes after the root, k_new/v_new[b][accept_path[b][k]] for k = 1 ..
 * AL - 1, are appended right behind the root, at token positions kv_lens[b] -
 * (AL - 1) + (k - 1), by spec_kv_append's rule (e4m3 scales included); AL is
 * the number of entries of accept_path[b] before its first -1.  kv_lens is not
 * written.  For a chain tree the rows are rewritten in place.  Tree layout:
 * see spec_verify_attn_tree.
 *
 *   p            as for spec_kv_append, num_new = R = 1 + D (<= 64) nodes.
 *   k_new, v_new [B][R][H_kv][hd] bf16: the step's node rows (those given to
 *                spec_kv_append before the attention).
 *   accept_path  [B][R] int32 from spec_accept_tree, 4-byte aligned.
 *   kv_lens      [B] int32, the committed lengths; read only.
 *   caches, scales, block_table: as for spec_kv_append.
 * Errors: as spec_kv_append; SV_ERR_INVALID for a NULL accept_path or R > 64.
 */
sv_status spec_kv_commit_tree(const sv_append_params* p, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_table, const int32_t* accept_path,
                              const int32_t* kv_lens, void* stream);

/* Bytes of device workspace spec_draft_signals needs for (rows, vocab). */
sv_status spec_draft_signals_workspace_size(int32_t rows, int32_t vocab, size_t* bytes);

/*
 * Draft-side signals and the next draft length.  The confidence (largest
 * probability) and entropy of the draft model's next-token distribution predict
 * how many drafts the target accepts (SpecKV summary, arXiv 2605.02888, section
 * "Technical core"); the next draft length maximises expected tokens per unit
 * time with the expected-token formula of "GPU and LLM" ch. 5, section
 * "Speculative decoding (2)", and the drafting cost of the NVIDIA co-design
 * summary, guidelines 3 and 4.
 *
 * For row r, p = softmax(draft_logits[r] / temperature):
 *     confidence[r] = max_v p_v
 *     entropy[r]    = -sum_v p_v ln p_v            (nats)
 *     next_draft_len[r] = the D in the candidates maximising
 *         f(D) = E(a, D) / (1 + rho D),  E(a, D) = sum_{i=0..D} a^i,  a = min(confidence[r], 1)
 *     (ties to the shorter D).  Candidates: 0 .. max_draft_len; with
 *     group_size G > 0, a D with G (1 + D) > 128 only if G (1 + D) is a multiple
 *     of 128 (whole 128-row attention tiles).  f is evaluated in fp64 from the
 *     returned fp32 confidence, in this order and without fused operations:
 *     P_0 = 1, P_{D+1} = P_D * a; E = D + 1 if a == 1 else (1 - P_{D+1}) / (1 - a);
 *     cost = 1 + (rho * D); f = E / cost.
 * The GPU sums fp32 exponentials in fp64: confidence and entropy are within
 * about 1e-6 relative of exact values.
 *
 *   draft_logits    [rows][V] fp32, 16-byte aligned.  Finite or -inf, at least
 *                   one finite value per row.
 *   confidence,     [rows] fp32, written.
 *   entropy
 *   next_draft_len  [rows] int32, written; may be NULL (signals only).
 *   max_draft_len   in [0, 63];  rho >= 0 (draft cost per drafted token relative
 *                   to one target pass);  group_size G in [0, 1024], 0 = no tile rule.
 *   workspace       at least spec_draft_signals_workspace_size() bytes,
 *                   256-byte aligned.
 * Errors: SV_ERR_INVALID for rows outside [1, 65535], vocab < 1, temperature,
 * max_draft_len, rho or group_size out of range, a (group_size, max_draft_len)
 * pair for which no D in [0, max_draft_len] passes the tile rule (G > 128, not
 * a multiple of 128, and no multiple of 128 among G (1 + D)), NULL or
 * misaligned pointers; SV_ERR_WORKSPACE.
 */
sv_status spec_draft_signals(int32_t rows, int32_t vocab, float temperature,
                             const float* draft_logits, float* confidence, float* entropy,
                             int32_t* next_draft_len, int32_t max_draft_len, float rho,
                             int32_t group_size, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Static description of a status code. */
const char* sv_status_string(sv_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* sv_last_error(void);

/* SV_ABI_VERSION of the built library. */
int32_t sv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
