/*
 * ev.h -- C ABI of the draft-tree verification step on AMD MI355X (gfx950).
 *
 * Speculative decoding (kongchang.com English article, section "Technical Background"): a small
 * draft model proposes tokens, the target model checks all of them in ONE parallel forward pass,
 * keeps the prefix that agrees with its own choice and then contributes one token of its own;
 * EAGLE-2's dynamic draft tree lets that one pass cover several candidate paths.  This library
 * is the target-side hot path of that check for one attention layer at temperature 0 (greedy;
 * aiposthub.com analysis, "paper Table 2"), in four calls:
 *
 *   ev_tree_attention   tree-masked GQA attention of every tree node over its sequence's KV
 *                       prefix plus its own ancestors (and itself)
 *   ev_node_argmax      the target's greedy token for every tree node (row argmax of logits)
 *   ev_greedy_accept    the longest accepted root-to-node path per sequence, its bonus token
 *                       and the tokens the round emits (ev_sampled_accept: the same at
 *                       temperature > 0, from per-node draws)
 *   ev_compact_kv       in-place move of the accepted nodes' K/V rows right after the prefix,
 *                       so the next round sees prefix + accepted tokens contiguously (the pages
 *                       name per-sequence acceptance lengths under continuous batching as the
 *                       main integration difficulty: same article, "Current Limitation")
 *
 * plus variants of the same operations: ev_tree_attention_window (a sliding window over the
 * prefix, as in the drafter's layers), ev_tree_attention_paged and ev_compact_kv_paged (KV
 * held in a paged pool through a per-sequence block table), and ev_node_sample (the per-node
 * draw of sampled verification at temperature > 0, in place of the argmax).
 * ev_select_accept_compact (and its _paged form) runs the last three steps -- the per-node
 * token, acceptance and compaction -- as one call of two launches, with results identical to
 * the separate calls.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the library allocates
 *     nothing and keeps no per-call state between calls (a small per-device cache of device
 *     properties aside).  Calls are asynchronous on `stream` and never synchronize.
 *   - Host-visible argument problems return an ev_status synchronously and launch nothing.
 *   - Problems that live in device data (a malformed tree, a token outside the vocabulary, a
 *     slot range outside the cache) are OR-ed into `*err_flag` (nullable device int32, never
 *     cleared by the library) with the EV_DATA_* bits; the affected sequence is skipped.
 *   - Trees: per sequence b, N_b nodes in topological order, node 0 the root (the token decided
 *     last round, always accepted), parent[node_start[b] + 0] == -1 and
 *     0 <= parent[node_start[b] + i] < i for i >= 1 (LOCAL indices).  1 <= N_b <= max_nodes
 *     <= EV_MAX_NODES.
 *   - KV cache: [total_slots][num_kv_heads][head_dim], contiguous.  Sequence b's prefix sits in
 *     slots kv_start[b] .. kv_start[b]+prefix_len[b]-1 and the K/V of its tree node i have
 *     already been written to slot kv_start[b] + prefix_len[b] + i.
 *   - Q and the attention output: [total_nodes][num_q_heads][head_dim]; q head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 *   - Base pointers of q, k_cache, v_cache, out and logits must be 16-byte aligned.
 */
#ifndef EV_H_
#define EV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EV_OK = 0,
    EV_ERR_NULL = 1,      /* a required pointer is NULL */
    EV_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes */
    EV_ERR_DTYPE = 3,     /* unsupported element type */
    EV_ERR_ALIGN = 4,     /* a base pointer, stride or row size breaks the alignment rules */
    EV_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the matching *_workspace_size() */
    EV_ERR_DEVICE = 6,    /* the current device is not gfx950 */
    EV_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed */
} ev_status;

typedef enum { EV_BF16 = 0, EV_F32 = 1 } ev_dtype;

/* Bits OR-ed into *err_flag for problems found in device data. */
#define EV_DATA_BAD_PARENT 1 /* parent[0] != -1 or parent[i] outside [0, i) */
#define EV_DATA_BAD_NODES 2  /* N_b = node_start[b+1] - node_start[b] outside [1, max_nodes] */
#define EV_DATA_BAD_TOKEN 4  /* a compared draft token or a target token outside [0, vocab) */
#define EV_DATA_BAD_SLOTS 8  /* kv_start / prefix_len negative, slots past total_slots, or pages
                               outside the block table or the pool */
#define EV_DATA_BAD_PATH 16  /* accepted path not strictly increasing from node 0, or too long */

#define EV_MAX_NODES 64
#define EV_MAX_BATCH 2048

/* Human-readable name of a status code (static string). */
const char *ev_status_string(ev_status status);

/* ---------------------------------------------------------------------------------------------
 * ev_tree_attention
 *
 * For every sequence b, tree node i and q head h (KV head g = h / (Hq/Hkv)):
 *   visible slots  S(i) = { s0 + t : 0 <= t < L }  U  { s0 + L + j : j ancestor of i or j == i }
 *   out[i,h]       = sum_{s in S(i)} softmax_s( sm_scale * <q[i,h], k[s,g]> ) * v[s,g]
 *   lse[i,h]       = natural-log log-sum-exp of the scaled scores
 * with s0 = kv_start[b], L = prefix_len[b] (L = 0 allowed).  A node never sees its siblings,
 * its descendants or other branches.  Arithmetic: bf16 operands on the matrix cores (fp32
 * inputs are rounded to bf16 first), fp32 accumulation and softmax, probabilities rounded to
 * bf16 for the value product; out has the input element type.
 *
 *   q, k_cache, v_cache   dtype elements, layouts above (read only)
 *   out                   [total_nodes][num_q_heads][head_dim], written for valid sequences
 *   lse                   [total_nodes][num_q_heads] fp32, nullable
 *   node_start            int32 [batch+1], node_start[0] == 0, node_start[batch] == total_nodes
 *   parent                int32 [total_nodes], local parent indices (see the tree rules)
 *   kv_start, prefix_len  int32 [batch]
 *   max_nodes             upper bound of N_b, 1..EV_MAX_NODES
 *   total_slots           slots in the cache (bounds check)
 *   head_dim              64 or 128;  num_q_heads % num_kv_heads == 0
 *   sm_scale              finite and > 0 (EV_ERR_SHAPE otherwise)
 *   workspace             >= ev_tree_attention_workspace_size(...) bytes of device memory; no
 *                         initialisation needed (every call writes what it later reads).  It
 *                         holds the partial results of sequences split over workgroups, which a
 *                         second launch on the same stream combines.  Calls that share one
 *                         workspace must be ordered (same stream).
 * Data errors (EV_DATA_BAD_PARENT / _NODES / _SLOTS): the sequence's rows are not written.
 * -------------------------------------------------------------------------------------------*/
size_t ev_tree_attention_workspace_size(int32_t batch, int32_t max_nodes, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim);

ev_status ev_tree_attention(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                            const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                            const int32_t *prefix_len, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                            int64_t total_slots, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            ev_dtype dtype, float sm_scale, void *workspace, size_t workspace_bytes,
                            int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_tree_attention_strided
 *
 * ev_tree_attention over K/V caches with caller-given element strides: cache row (slot s, KV head
 * g) starts at element s * kv_slot_stride + g * kv_head_stride of k_cache / v_cache (head_dim
 * contiguous elements).  ev_tree_attention is the case kv_slot_stride = num_kv_heads * head_dim,
 * kv_head_stride = head_dim ([slot][kv_head][dim]); kv_slot_stride = head_dim, kv_head_stride =
 * total_slots * head_dim is the head-major cache [kv_head][slot][dim], whose rows of one KV head
 * are contiguous and stream faster (a unit reads whole runs of its own head's rows).  Every other
 * argument, the arithmetic, the workspace and the error behaviour are those of ev_tree_attention;
 * results are bit-identical to ev_tree_attention on the same values in its layout.
 *   kv_slot_stride   >= 1;  kv_head_stride >= 0;  both times the element size must be multiples
 *                    of 16 bytes (EV_ERR_ALIGN) and kv_slot_stride * element size <= 2^26
 *                    (EV_ERR_SHAPE).  The caches must hold (total_slots - 1) * kv_slot_stride +
 *                    (num_kv_heads - 1) * kv_head_stride + head_dim elements.
 * A head-major cache is compacted by ev_compact_kv (or the fused call) with num_layers = KV heads
 * per layer, layer_stride_bytes = total_slots * head_dim * element size and num_kv_heads = 1.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_tree_attention_strided(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                                    const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                    const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
                                    int32_t max_nodes, int64_t total_slots, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int64_t kv_slot_stride,
                                    int64_t kv_head_stride, ev_dtype dtype, float sm_scale, void *workspace,
                                    size_t workspace_bytes, int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_tree_attention_window
 *
 * ev_tree_attention with a sliding window over the prefix: the EAGLE-4 drafter's layers attend
 * only to the most recent stretch of an append-only cache, which keeps long documents cheap
 * (aiposthub.com analysis, section "EAGLE-4 是什麼？先看推測解碼為什麼能變快"; arex-research.com
 * release note, section "投机树多大，由实测成本决定").  Read here as: the last `window` prefix
 * tokens stay visible, every tree ancestor (and the node itself) stays visible whatever the
 * window, i.e. with Lf = prefix_len[b] and L = min(Lf, window)
 *   S(i) = { kv_start[b] + Lf - L + t : 0 <= t < L }  U  { kv_start[b] + Lf + j : j anc. of i or i }
 * All other arguments, layouts, arithmetic and error behaviour are those of ev_tree_attention,
 * and the same workspace size applies.  window >= 1 (EV_ERR_SHAPE otherwise); window >= Lf
 * gives ev_tree_attention's result for that sequence.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_tree_attention_window(const void *q, const void *k_cache, const void *v_cache, void *out,
                                   float *lse, const int32_t *node_start, const int32_t *parent,
                                   const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                                   int32_t total_nodes, int32_t max_nodes, int64_t total_slots,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype,
                                   float sm_scale, int32_t window, void *workspace, size_t workspace_bytes,
                                   int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_tree_attention_paged
 *
 * ev_tree_attention (optionally windowed) over a paged KV pool, the cache layout of the
 * PagedAttention serving engines the verification kernel has to live in (kongchang.com English
 * article, section "Current Limitation: Only Qwen3.8-27B Supported"; arex-research.com release
 * note, section "eagle-harness 是插件，不改引擎本体", on tree verification in vLLM needing an
 * unquantized KV cache).  Token t of sequence b (prefix tokens t < Lf = prefix_len[b], then tree
 * node i at t = Lf + i) lives in pool row
 *     row(b, t) = block_table[b * bt_stride + t / page_size] * page_size + t % page_size
 * and the visible set of node i is { row(b, t) : Lf - L <= t < Lf } U { row(b, Lf + j) : j
 * ancestor of i or j == i } with L = Lf (window == 0) or min(Lf, window).
 *
 *   k_pages, v_pages   bf16 [num_pages][page_size][num_kv_heads][head_dim] (read only)
 *   block_table        int32 [batch][bt_stride]; entries 0 .. (Lf + N_b - 1) / page_size of row
 *                      b are read, the rest are ignored
 *   page_size          a power of two, 16 .. 65536;  bt_stride >= 1;  num_pages >= 0
 *   window             0: no window;  >= 1: sliding window as in ev_tree_attention_window
 * q, out, lse, node_start, parent, prefix_len, the sizes, sm_scale, workspace and err_flag are as
 * in ev_tree_attention (same workspace size); kv_start does not exist here.  dtype must be
 * EV_BF16 (EV_ERR_DTYPE otherwise).  Data errors: N_b outside [1, max_nodes] or a bad parent
 * (EV_DATA_BAD_NODES / _PARENT) and Lf < 0 or (Lf + N_b - 1) / page_size >= bt_stride
 * (EV_DATA_BAD_SLOTS) leave the sequence's rows unwritten as in ev_tree_attention; a block-table
 * entry outside [0, num_pages) that the sequence reads raises EV_DATA_BAD_SLOTS while its rows
 * are computed (their values are then unspecified: page 0 stands in, no load leaves the pool).
 * -------------------------------------------------------------------------------------------*/
ev_status ev_tree_attention_paged(const void *q, const void *k_pages, const void *v_pages, void *out, float *lse,
                                  const int32_t *node_start, const int32_t *parent, const int32_t *block_table,
                                  int32_t bt_stride, int32_t page_size, const int32_t *prefix_len, int32_t batch,
                                  int32_t total_nodes, int32_t max_nodes, int32_t num_pages, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype, float sm_scale,
                                  int32_t window, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_tree_attention_noalloc
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): ev_tree_attention with the same arguments, results
 * and errors, minus the workspace, which is a static device array inside the library of
 * 42,606,592 bytes (the largest workspace any supported shape needs, so every shape that
 * ev_tree_attention accepts is accepted; a shape needing more would return EV_ERR_WORKSPACE).
 * Each GPU the library runs on holds its own copy of that array from the first call on that
 * device until the process ends.  The call allocates nothing and frees nothing.  All calls on
 * one GPU share its copy: calls ordered on one stream are safe, calls that overlap on one GPU
 * (other streams, other host threads) race on it and give wrong results.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_tree_attention_noalloc(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                                    const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                    const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
                                    int32_t max_nodes, int64_t total_slots, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype, float sm_scale,
                                    int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_node_argmax
 *
 * target_token[r] = the LOWEST index v in [0, vocab) holding the maximum of logits row r (the
 * target's greedy token at temperature 0).  +0 and -0 compare equal; a NaN ranks above every
 * number, so a row's first NaN wins.  max_value[r] (nullable, fp32) receives that maximum.
 *
 *   logits       dtype elements, row r starts at logits + r * row_stride (elements);
 *                row_stride >= vocab and row_stride * element size must be a multiple of 16 B
 *   workspace    >= ev_node_argmax_workspace_size(num_rows, vocab) bytes (may be 0 bytes, then
 *                NULL is fine), zeroed once before first use, left reusable by every call.
 * -------------------------------------------------------------------------------------------*/
size_t ev_node_argmax_workspace_size(int32_t num_rows, int32_t vocab);

ev_status ev_node_argmax(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t num_rows, int32_t vocab,
                         int32_t *target_token, float *max_value, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_node_sample
 *
 * Sampled verification (temperature T > 0; the pages report T = 1 results: aiposthub.com
 * analysis, section "它和 DFlash 2、DSpark 比，贏在哪個條件？"; arex-research.com release note,
 * section "论文口径与推文口径").  target_token[r] = one draw from softmax(logits[r] / T):
 *     y = argmax_v  fma(z_v, c, -log2(-log2(u_v))),   c = log2(e) / T
 * (Gumbel-max in base 2), fp32 scores, largest score wins, lowest index on ties, a NaN logit
 * above every number.  u_v = ((w >> 9) + 1/2) * 2^-23 with w the 32-bit word of element v from
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) under the 64-bit key seed (low word first)
 * and the 128-bit counter (v / 4, r, low word of offset, high word of offset): output word k
 * gives element 4j + k.  Use a fresh (seed, offset) per call (e.g. offset = decoding round) for
 * fresh noise.
 * Fed to ev_sampled_accept as target_token, the draws make the accept step speculative
 * sampling along the tree with the drafted children as point proposals: a sequence descends
 * into the lowest-index child holding its node's draw and otherwise stops with the draw as
 * bonus, which keeps the target's sampling distribution (release note, opening section).  (Not
 * ev_greedy_accept: its deepest-path choice among siblings holding the same token would pick
 * between independent draws by their outcomes.)  The log2 is the hardware's
 * (about 1 ulp), so a draw can differ from an exact evaluation only where two scores of the row
 * agree to a few ulps.
 *
 *   logits, dtype, row_stride, num_rows, vocab   as in ev_node_argmax
 *   temperature    finite, > 0, with log2(e) / temperature finite in fp32 (EV_ERR_SHAPE otherwise)
 *   workspace      >= ev_node_argmax_workspace_size(num_rows, vocab) bytes, zeroed once before
 *                  first use and left reusable (the same buffer may serve both calls)
 * -------------------------------------------------------------------------------------------*/
ev_status ev_node_sample(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t num_rows, int32_t vocab,
                         float temperature, uint64_t seed, uint64_t offset, int32_t *target_token, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_greedy_accept
 *
 * Per sequence b (one wavefront each): accepted(0) = true and, for i >= 1,
 * accepted(i) = accepted(parent(i)) and draft_token[i] == target_token[parent(i)].
 * i* = the accepted node of greatest depth, lowest index among equal depths.
 *   accept_len[b]      depth(i*) + 1  (root included = tokens emitted this round)
 *   accept_path[b, :]  the ancestors of i* root first (local indices), then -1 padding
 *   bonus_token[b]     target_token[i*]  (the target's own token after the accepted path)
 *   out_tokens[b, :]   draft tokens of accept_path[1..len-1], then the bonus, then -1 padding
 * The root's draft token is never compared.  node_start/parent/draft_token/target_token are as in
 * ev_tree_attention (total_nodes entries); all arrays int32; the [B, max_nodes] outputs are
 * row-major.  Data errors (EV_DATA_BAD_PARENT / _NODES / _TOKEN): accept_len = 0, bonus = -1,
 * path and tokens all -1 for that sequence.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_greedy_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft_token,
                           const int32_t *target_token, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                           int32_t vocab,
                           int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token, int32_t *out_tokens,
                           int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_sampled_accept
 *
 * Acceptance of sampled verification (temperature > 0; the pages report T = 1 results --
 * aiposthub.com analysis, section "它和 DFlash 2、DSpark 比，贏在哪個條件？" -- and say that
 * verification keeps the target model's output distribution: kongchang.com English article,
 * "Technical Background"; arex-research.com release note, opening section).  target_token[i] is
 * node i's draw from the target (ev_node_sample).  Drafted children are point proposals, and
 * speculative sampling tries a node's children in index order against its draw, so:
 *   accepted(0) = true;  for i >= 1, accepted(i) = accepted(parent(i)) and
 *   draft_token[i] == target_token[parent(i)] and no sibling j < i has draft_token[j] ==
 *   draft_token[i]
 * The accepted nodes form one root path (the walk into the lowest-index child holding each
 * node's draw); i* is its last node.  Outputs, arguments, layouts and data errors are those of
 * ev_greedy_accept; on trees whose siblings hold distinct tokens both calls give the same result.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_sampled_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft_token,
                            const int32_t *target_token, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                            int32_t vocab, int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                            int32_t *out_tokens, int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_compact_kv
 *
 * In place, for every layer l, KV head and 0 <= d < len = accept_len[b]:
 *   slot s0+L+d of layer l  <-  the bytes slot s0+L+path[d] held BEFORE the call
 * (s0 = kv_start[b], L = prefix_len[b], path = accept_path[b, :]); every other byte is left
 * unchanged (slots L+len .. L+N-1 keep stale rows).  new_len[b] = L + len.  A sequence with
 * len <= 0 is left alone and gets new_len = L.  The path must start at 0 and strictly
 * increase (ev_greedy_accept guarantees it), which makes the move safe in place.
 *
 *   k_cache, v_cache     layer l's cache starts at base + l * layer_stride_bytes; each layer
 *                        is [total_slots][num_kv_heads][head_dim] of elem_bytes (2 or 4)
 *                        elements; one slot's row (num_kv_heads*head_dim*elem_bytes bytes) and
 *                        layer_stride_bytes must be multiples of 16, base pointers 16-aligned
 *   new_len              int32 [batch]; must not alias prefix_len
 * Data errors (EV_DATA_BAD_PATH / _SLOTS): that sequence is left alone, new_len = L.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_compact_kv(void *k_cache, void *v_cache, int32_t elem_bytes, int32_t num_layers,
                        int64_t layer_stride_bytes, const int32_t *kv_start, const int32_t *prefix_len,
                        const int32_t *accept_len, const int32_t *accept_path, int32_t batch, int32_t max_nodes,
                        int64_t total_slots, int32_t num_kv_heads, int32_t head_dim, int32_t *new_len,
                        int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_compact_kv_paged
 *
 * ev_compact_kv through a block table (the per-sequence acceptance lengths of continuous
 * batching over a paged pool: kongchang.com English article, "Current Limitation: Only
 * Qwen3.8-27B Supported").  In place, for every layer l and 0 <= d < len = accept_len[b]:
 *   row(b, L + d) of layer l  <-  the bytes row(b, L + path[d]) held BEFORE the call
 * with row(b, t) = block_table[b * bt_stride + t / page_size] * page_size + t % page_size and
 * L = prefix_len[b].  The pages a sequence uses must be distinct (so distinct tokens are
 * distinct rows; the in-place move relies on it).  new_len[b] = L + len (L when len <= 0).
 *
 *   k_pages, v_pages     layer l starts at base + l * layer_stride_bytes and is
 *                        [num_pages][page_size][num_kv_heads][head_dim] of elem_bytes (2 or 4)
 *                        elements, alignment rules as in ev_compact_kv
 *   block_table          int32 [batch][bt_stride];  page_size >= 1 (any);  num_pages >= 0
 * Data errors: a bad path (EV_DATA_BAD_PATH) as in ev_compact_kv; L < 0,
 * (L + path[len-1]) / page_size >= bt_stride or a source or destination page outside
 * [0, num_pages) raise EV_DATA_BAD_SLOTS; such a sequence is left alone with new_len = L.
 * -------------------------------------------------------------------------------------------*/
ev_status ev_compact_kv_paged(void *k_pages, void *v_pages, int32_t elem_bytes, int32_t num_layers,
                              int64_t layer_stride_bytes, const int32_t *block_table, int32_t bt_stride,
                              int32_t page_size, const int32_t *prefix_len, const int32_t *accept_len,
                              const int32_t *accept_path, int32_t batch, int32_t max_nodes, int32_t num_pages,
                              int32_t num_kv_heads, int32_t head_dim, int32_t *new_len, int32_t *err_flag,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_select_accept_compact
 *
 * ev_node_argmax then ev_greedy_accept (temperature == 0), or ev_node_sample then
 * ev_sampled_accept (temperature > 0), then ev_compact_kv of the accepted paths: the per-node
 * target token, the
 * accept rule and the KV move of one verification round (kongchang.com English article,
 * "Technical Background"), in two launches instead of three and without the arrival counting
 * that the standalone argmax needs.  The first launch streams the logits and leaves every row
 * piece's winner in the workspace; the second, one workgroup per (sequence, layer), finishes
 * its rows' tokens, applies the accept rule and moves the layer's accepted K/V rows.  Every
 * output is bit-identical to the three separate calls on the same inputs:
 *
 *   target_token   [total_nodes]  as ev_node_argmax / ev_node_sample (no max_value output)
 *   accept_len, accept_path, bonus_token, out_tokens   as ev_greedy_accept / ev_sampled_accept
 *   K/V caches, new_len                                as ev_compact_kv
 *
 *   logits, dtype, row_stride, vocab   as ev_node_argmax, num_rows = total_nodes
 *   temperature    0 for the argmax; otherwise finite and > 0 with log2(e)/temperature finite
 *                  in fp32 (EV_ERR_SHAPE otherwise); seed, offset as ev_node_sample (unused at 0)
 *   node_start, parent, draft_token, batch, total_nodes, max_nodes   as ev_greedy_accept
 *   k_cache ... head_dim, new_len                                    as ev_compact_kv
 *   workspace      >= ev_select_workspace_size(total_nodes, vocab) bytes, 8-byte aligned (NULL
 *                  when that size is 0); fully rewritten by each call, needs no zeroing
 * Every argument is checked before the first launch.  Data errors are reported as by the
 * separate calls (a sequence whose tree or tokens are bad gets accept_len 0 and its KV is left
 * alone with new_len = L).
 * -------------------------------------------------------------------------------------------*/
size_t ev_select_workspace_size(int32_t num_rows, int32_t vocab);

ev_status ev_select_accept_compact(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t vocab,
                                   float temperature, uint64_t seed, uint64_t offset, const int32_t *node_start,
                                   const int32_t *parent, const int32_t *draft_token, int32_t batch,
                                   int32_t total_nodes, int32_t max_nodes, void *k_cache, void *v_cache,
                                   int32_t elem_bytes, int32_t num_layers, int64_t layer_stride_bytes,
                                   const int32_t *kv_start, const int32_t *prefix_len, int64_t total_slots,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t *target_token,
                                   int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                                   int32_t *out_tokens, int32_t *new_len, void *workspace, size_t workspace_bytes,
                                   int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_select_accept_compact_paged
 *
 * ev_select_accept_compact with the K/V in a paged pool: the compaction is ev_compact_kv_paged
 * (k_pages, v_pages, block_table, bt_stride, page_size, num_pages as there).
 * -------------------------------------------------------------------------------------------*/
ev_status ev_select_accept_compact_paged(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t vocab,
                                         float temperature, uint64_t seed, uint64_t offset,
                                         const int32_t *node_start, const int32_t *parent,
                                         const int32_t *draft_token, int32_t batch, int32_t total_nodes,
                                         int32_t max_nodes, void *k_pages, void *v_pages, int32_t elem_bytes,
                                         int32_t num_layers, int64_t layer_stride_bytes, const int32_t *block_table,
                                         int32_t bt_stride, int32_t page_size, const int32_t *prefix_len,
                                         int32_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t *target_token, int32_t *accept_len, int32_t *accept_path,
                                         int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len,
                                         void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_verify_step
 *
 * The whole verification step of one tree (kongchang.com English article, "Technical
 * Background": one target pass scores every node, the accepted path is kept and its K/V moved):
 * ev_tree_attention_strided, then ev_select_accept_compact, as one call: every argument of both
 * is checked before the first launch, then the attention, the merge of split units, the per-node
 * selection pass and the acceptance/compaction launch run in that order on `stream`.  When the
 * attention splits units over workgroups and head_dim is 128, the selection pass's row pieces run
 * as workgroups of the merge launch (the two read and write disjoint data), which saves a launch
 * and lets the logits stream while the merge combines: three launches instead of four.  Every
 * output is bit-identical to the two separate calls on the same inputs:
 *
 *   out, lse                                          as ev_tree_attention_strided
 *   target_token, accept_len, accept_path, bonus_token, out_tokens, K/V caches, new_len
 *                                                     as ev_select_accept_compact
 *
 *   q ... sm_scale   as ev_tree_attention_strided (the caches are read through kv_slot_stride /
 *                    kv_head_stride, then compacted in place, so they are not const here)
 *   logits ... draft_token   as ev_select_accept_compact (logits_dtype is its dtype)
 *   num_layers, layer_stride_bytes, compact_kv_heads, compact_head_dim
 *                    the compaction's view of the same caches, as ev_select_accept_compact's
 *                    num_layers, layer_stride_bytes, num_kv_heads, head_dim (elem_bytes is the
 *                    attention dtype's size): [slots][Hkv][D] caches are 1 layer of Hkv heads;
 *                    head-major [Hkv][slots][D] caches are Hkv layers of 1 head, layer stride
 *                    slots * D * elem_bytes
 *   workspace        >= ev_verify_step_workspace_size(...) bytes, 256-byte aligned
 *                    (EV_ERR_ALIGN), for this call only: the selection pieces
 *                    (ev_select_workspace_size(total_nodes, vocab) bytes), then the attention
 *                    workspace.
 *                    No initial contents are needed; calls that share a workspace must not
 *                    overlap.
 * Every argument is checked before the first launch (nothing runs on an error).  Data errors
 * are reported as by the separate calls.
 * -------------------------------------------------------------------------------------------*/
size_t ev_verify_step_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t vocab);

ev_status ev_verify_step(const void *q, void *k_cache, void *v_cache, void *out, float *lse,
                         const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                         const int32_t *prefix_len, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                         int64_t total_slots, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int64_t kv_slot_stride, int64_t kv_head_stride, ev_dtype dtype, float sm_scale,
                         const void *logits, ev_dtype logits_dtype, int64_t row_stride, int32_t vocab,
                         float temperature, uint64_t seed, uint64_t offset, const int32_t *draft_token,
                         int32_t num_layers, int64_t layer_stride_bytes, int32_t compact_kv_heads,
                         int32_t compact_head_dim, int32_t *target_token, int32_t *accept_len,
                         int32_t *accept_path, int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len,
                         void *workspace, size_t workspace_bytes, int32_t *err_flag, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ev_stream_read
 *
 * Measurement helper, not part of the verification step: reads every byte of a device buffer
 * once, with non-temporal 16-byte loads over the whole GPU, and discards the data.  Its rate on a
 * buffer far larger than the 256 MB Infinity Cache is the streaming-read ceiling that the
 * attention's K/V read rate is reported against, besides the 8 TB/s HBM peak.
 *
 *   src     device buffer, 16-byte aligned (EV_ERR_ALIGN), read only
 *   bytes   > 0 and a multiple of 16 (EV_ERR_SHAPE)
 *   sink    device uint32; written only in the (practically impossible) case that the XOR of all
 *           data equals 0x9E3779B9, which keeps the loads from being removed
 * -------------------------------------------------------------------------------------------*/
ev_status ev_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EV_H_ */
