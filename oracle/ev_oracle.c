/*
 * ev_oracle.c -- CPU oracle of the draft-tree verification step (TEST INFRASTRUCTURE).
 *
 * Plain, slow loops in double precision.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library; the GPU library never
 * links it and shares no code or header with it.
 *
 * What is computed follows the descriptions of speculative decoding on the pages
 * (kongchang.com EN article, "Technical Background": the target model checks all drafted
 * tokens in one parallel forward pass, keeps the prefix that agrees with it and adds one
 * token of its own after the first rejected position; EAGLE-2's dynamic draft tree lets one
 * verification cover several candidate paths), at temperature 0 (aiposthub.com analysis,
 * "paper Table 2", greedy T=0 results), plus the four-step decomposition named for this
 * verification step: tree-masked GQA attention, per-node argmax, greedy longest-path
 * acceptance, KV compaction.  Readings where the pages are silent:
 *   - node 0 is the root (the previous round's decided token), always accepted;
 *   - nodes are in topological order: parent[0] == -1 and 0 <= parent[i] < i;
 *   - a node sees the whole prefix plus its ancestors INCLUDING itself;
 *   - q head h reads KV head h / (Hq / Hkv);
 *   - argmax ties go to the lowest index, +0 == -0, NaN ranks above everything
 *     (first NaN wins);
 *   - the accepted node is the deepest accepted node, lowest index on equal depth;
 *   - sliding windows keep the last W prefix tokens; paged caches map token t through a
 *     block table (page t / P, row t % P);
 *   - sampled verification (T > 0, reported at temperature 1 in aiposthub.com analysis, "它和
 *     DFlash 2、DSpark 比，贏在哪個條件？", and arex-research.com, "论文口径与推文口径"): drafted
 *     children are point proposals, so speculative sampling along the tree is a per-node draw
 *     from softmax(z / T) and a walk from the root that enters the LOWEST-INDEX child holding
 *     the current node's draw and stops with the draw as bonus when no child holds it (see the
 *     sampled section below for the draw, its generator and why a repeated sibling token is
 *     never entered).
 *
 * Fixed-size work arrays hold at most ORACLE_MAX_NODES tree nodes; larger trees are reported as
 * a node-count error (bit 2) instead of being processed.
 *
 * Parity pins: every function here is checked in tests against an independent formulation
 * (brute force / library routines / closed forms / hand-built cases); none is unpinned.
 *
 * Data-error bits (per sequence) mirror the GPU library's: 1 bad parent array,
 * 2 node count outside [1, max_nodes], 4 token outside [0, vocab), 8 slot range outside the
 * cache, 16 malformed accepted path.  A sequence with an error is skipped.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_F32 = 1 };
enum { ORACLE_MAX_NODES = 1024 }; /* capacity of the per-tree work arrays below */

/* Element `idx` of a bf16 (raw bits) or fp32 array, widened exactly to double. */
static double elem(const void *base, int dtype, size_t idx) {
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Tree rule: parent[0] == -1 and 0 <= parent[i] < i; 1 <= n <= max_nodes (and n within the
   work arrays' capacity). */
int32_t oracle_tree_errors(const int32_t *parent, int32_t n, int32_t max_nodes) {
    int32_t err = 0;
    if (n < 1 || n > max_nodes || n > ORACLE_MAX_NODES) return 2;
    if (parent[0] != -1) err |= 1;
    for (int32_t i = 1; i < n; ++i)
        if (parent[i] < 0 || parent[i] >= i) err |= 1;
    return err;
}

/* Ancestors of node i including i itself, written root first (increasing depth).
   Returns how many there are, i.e. depth(i) + 1; -1 when i is outside [0, ORACLE_MAX_NODES) or
   the chain breaks the topological rule (a parent index not below its child's), which would
   otherwise loop or overrun the work array. */
int32_t oracle_ancestor_path(const int32_t *parent, int32_t i, int32_t *path) {
    int32_t rev[ORACLE_MAX_NODES];
    int32_t n = 0;
    if (i < 0 || i >= ORACLE_MAX_NODES) return -1;
    for (int32_t j = i; j >= 0; j = parent[j]) {
        if (j > 0 && parent[j] >= j) return -1;
        rev[n++] = j;
    }
    for (int32_t t = 0; t < n; ++t) path[t] = rev[n - 1 - t];
    return n;
}

/* Cache row of logical token t of sequence b (token t = prefix position t; tree node j sits at
   t = L + j).  Contiguous caches: row kv_start[b] + t.  Paged caches (block_table != NULL):
   page block_table[b * bt_stride + t / page_size], row t % page_size inside it. */
static int64_t token_slot(const int32_t *kv_start, const int32_t *block_table, int32_t bt_stride,
                          int32_t page_size, int32_t b, int64_t t) {
    if (block_table)
        return (int64_t)block_table[(int64_t)b * bt_stride + t / page_size] * page_size + t % page_size;
    return (int64_t)kv_start[b] + t;
}

/* First prefix token a query sees: the last `window` tokens only when a window is set. */
static int32_t first_visible(int32_t L, int32_t window) { return (window > 0 && L > window) ? L - window : 0; }

static int32_t seq_layout_errors(const int32_t *kv_start, const int32_t *prefix_len, const int32_t *block_table,
                                 int32_t bt_stride, int32_t page_size, int32_t window, int32_t b, int32_t n,
                                 int64_t total_slots) {
    if (prefix_len[b] < 0) return 8;
    if (!block_table) {
        if (kv_start[b] < 0) return 8;
        if ((int64_t)kv_start[b] + prefix_len[b] + n > total_slots) return 8;
        return 0;
    }
    /* every page the visible tokens and the tree use must exist */
    const int64_t t_end = (int64_t)prefix_len[b] + n;
    if ((t_end + page_size - 1) / page_size > bt_stride) return 8;
    for (int64_t t = first_visible(prefix_len[b], window); t < t_end; ++t) {
        const int32_t pg = block_table[(int64_t)b * bt_stride + t / page_size];
        if (pg < 0 || (int64_t)pg * page_size >= total_slots) return 8;
    }
    return 0;
}

/* Per-sequence validity for attention: tree rule and slot range. */
static void attention_errors(const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                             const int32_t *prefix_len, const int32_t *block_table, int32_t bt_stride,
                             int32_t page_size, int32_t window, int32_t batch, int32_t max_nodes,
                             int64_t total_slots, int32_t *seq_err) {
    for (int32_t b = 0; b < batch; ++b) {
        int32_t n = node_start[b + 1] - node_start[b];
        int32_t e = oracle_tree_errors(parent + node_start[b], n, max_nodes);
        if (!(e & 2))
            e |= seq_layout_errors(kv_start, prefix_len, block_table, bt_stride, page_size, window, b, n, total_slots);
        seq_err[b] = e;
    }
}

void oracle_attention_errors(const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                             const int32_t *prefix_len, int32_t batch, int32_t max_nodes,
                             int64_t total_slots, int32_t *seq_err) {
    attention_errors(node_start, parent, kv_start, prefix_len, NULL, 0, 0, 0, batch, max_nodes, total_slots,
                     seq_err);
}

/* Attention of one (sequence b, local node i, q head h) row.
   Visible keys: the prefix tokens t0 <= t < L (t0 = 0, or L - window with a sliding window of the
   drafter's kind), then the tree tokens L + j for every j in anc(i), each at its cache row
   (token_slot).  scores = sm_scale * <q, k>;  out = sum_t e^{s_t - m} v_t / sum_t e^{s_t - m};
   lse = m + ln sum_t e^{s_t - m}. */
static void attention_row(const void *q, const void *k, const void *v, int dtype, const int32_t *node_start,
                          const int32_t *parent, const int32_t *kv_start, const int32_t *prefix_len,
                          const int32_t *bt, int32_t bt_stride, int32_t page, int32_t window,
                          int32_t b, int32_t i, int32_t h, int32_t hq, int32_t hkv, int32_t d,
                          double sm_scale, double *out, double *lse, double *scratch, int64_t *slots) {
    const int32_t G = hq / hkv;
    const int32_t g = h / G;
    const int32_t L = prefix_len[b];
    const int32_t t0 = first_visible(L, window);
    const int32_t *par = parent + node_start[b];
    int32_t path[ORACLE_MAX_NODES];
    int32_t np = oracle_ancestor_path(par, i, path);
    int64_t nvis = 0;
    for (int32_t t = t0; t < L; ++t) slots[nvis++] = token_slot(kv_start, bt, bt_stride, page, b, t);
    for (int32_t t = 0; t < np; ++t) slots[nvis++] = token_slot(kv_start, bt, bt_stride, page, b, L + path[t]);

    const size_t qrow = ((size_t)(node_start[b] + i) * hq + h) * d;
    double m = -INFINITY;
    for (int64_t t = 0; t < nvis; ++t) {
        const size_t krow = ((size_t)slots[t] * hkv + g) * d;
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += elem(q, dtype, qrow + c) * elem(k, dtype, krow + c);
        scratch[t] = sm_scale * dot;
        if (scratch[t] > m) m = scratch[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < nvis; ++t) {
        scratch[t] = exp(scratch[t] - m);
        sum += scratch[t];
    }
    for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t t = 0; t < nvis; ++t) {
        const size_t vrow = ((size_t)slots[t] * hkv + g) * d;
        for (int32_t c = 0; c < d; ++c) out[c] += scratch[t] * elem(v, dtype, vrow + c);
    }
    for (int32_t c = 0; c < d; ++c) out[c] /= sum;
    *lse = m + log(sum);
}

/* A list of rows: rows[2r] = global node index, rows[2r+1] = q head.  out [nrows, d], lse [nrows].
   Rows of sequences with data errors are left untouched.  block_table == NULL: contiguous caches
   (kv_start used); else paged caches of page_size rows per page (kv_start unused); total_slots =
   rows of the cache.  window > 0: the sliding window. */
void oracle_tree_attention_rows_ex(const void *q, const void *k, const void *v, int32_t dtype,
                                   const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                   const int32_t *prefix_len, const int32_t *block_table, int32_t bt_stride,
                                   int32_t page_size, int32_t window, int32_t batch, int32_t max_nodes,
                                   int64_t total_slots, int32_t hq, int32_t hkv, int32_t d, double sm_scale,
                                   const int32_t *rows, int64_t nrows, double *out, double *lse) {
    int32_t *seq_err = (int32_t *)calloc(batch > 0 ? batch : 1, sizeof(int32_t));
    attention_errors(node_start, parent, kv_start, prefix_len, block_table, bt_stride, page_size, window, batch,
                     max_nodes, total_slots, seq_err);
    int32_t maxvis = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int32_t n = node_start[b + 1] - node_start[b];
        if (prefix_len[b] + n > maxvis) maxvis = prefix_len[b] + n;
    }
#pragma omp parallel
    {
        double *scratch = (double *)malloc(sizeof(double) * (maxvis + 1));
        int64_t *slots = (int64_t *)malloc(sizeof(int64_t) * (maxvis + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int32_t node = rows[2 * r], h = rows[2 * r + 1];
            int32_t b = 0;
            while (b + 1 <= batch && node_start[b + 1] <= node) ++b;
            if (seq_err[b]) continue;
            attention_row(q, k, v, dtype, node_start, parent, kv_start, prefix_len, block_table, bt_stride,
                          page_size, window, b, node - node_start[b], h, hq, hkv, d, sm_scale,
                          out + (size_t)r * d, lse + r, scratch, slots);
        }
        free(scratch);
        free(slots);
    }
    free(seq_err);
}

void oracle_tree_attention_rows(const void *q, const void *k, const void *v, int32_t dtype,
                                const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                const int32_t *prefix_len, int32_t batch, int32_t max_nodes,
                                int64_t total_slots, int32_t hq, int32_t hkv, int32_t d, double sm_scale,
                                const int32_t *rows, int64_t nrows, double *out, double *lse) {
    oracle_tree_attention_rows_ex(q, k, v, dtype, node_start, parent, kv_start, prefix_len, NULL, 0, 0, 0, batch,
                                  max_nodes, total_slots, hq, hkv, d, sm_scale, rows, nrows, out, lse);
}

/* Every row: out [total_nodes, hq, d], lse [total_nodes, hq]. */
void oracle_tree_attention_ex(const void *q, const void *k, const void *v, int32_t dtype,
                              const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                              const int32_t *prefix_len, const int32_t *block_table, int32_t bt_stride,
                              int32_t page_size, int32_t window, int32_t batch, int32_t max_nodes,
                              int64_t total_slots, int32_t hq, int32_t hkv, int32_t d, double sm_scale, double *out,
                              double *lse, int32_t *seq_err) {
    attention_errors(node_start, parent, kv_start, prefix_len, block_table, bt_stride, page_size, window, batch,
                     max_nodes, total_slots, seq_err);
    const int64_t total = (int64_t)node_start[batch] * hq;
    int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * 2 * (total > 0 ? total : 1));
    for (int64_t r = 0; r < total; ++r) {
        rows[2 * r] = (int32_t)(r / hq);
        rows[2 * r + 1] = (int32_t)(r % hq);
    }
    oracle_tree_attention_rows_ex(q, k, v, dtype, node_start, parent, kv_start, prefix_len, block_table, bt_stride,
                                  page_size, window, batch, max_nodes, total_slots, hq, hkv, d, sm_scale, rows,
                                  total, out, lse);
    free(rows);
}

void oracle_tree_attention(const void *q, const void *k, const void *v, int32_t dtype,
                           const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                           const int32_t *prefix_len, int32_t batch, int32_t max_nodes, int64_t total_slots,
                           int32_t hq, int32_t hkv, int32_t d, double sm_scale, double *out, double *lse,
                           int32_t *seq_err) {
    oracle_tree_attention_ex(q, k, v, dtype, node_start, parent, kv_start, prefix_len, NULL, 0, 0, 0, batch,
                             max_nodes, total_slots, hq, hkv, d, sm_scale, out, lse, seq_err);
}

/* Greedy target token of every logits row: the lowest index holding the row maximum.
   +0 and -0 are equal; a NaN ranks above every number, so the first NaN wins. */
void oracle_node_argmax(const void *logits, int32_t dtype, int64_t row_stride, int32_t num_rows,
                        int32_t vocab, int32_t *target, double *max_value) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int32_t r = 0; r < num_rows; ++r) {
        const size_t base = (size_t)r * row_stride;
        int32_t best = 0;
        double bv = elem(logits, dtype, base);
        if (!isnan(bv)) {
            for (int32_t t = 1; t < vocab; ++t) {
                double x = elem(logits, dtype, base + t);
                if (isnan(x)) { best = t; bv = x; break; }
                if (x > bv) { best = t; bv = x; }
            }
        }
        target[r] = best;
        if (max_value) max_value[r] = bv;
    }
}

/* ---- Sampled verification (temperature T > 0) ----
   Reading: a drafted child is a point proposal for its parent's next token (the dynamic tree
   expands the drafter's best tokens).  Speculative sampling with point proposals tries a node's
   children in index order, accepting child token x with the residual target probability of x
   and removing x from the residual when it is rejected; the bonus token is then drawn from what
   is left.  A token already rejected has residual probability 0, so a later sibling holding the
   same token is never accepted.  The result has the law of one draw y from the target
   distribution at the node, with the walk descending into the LOWEST-INDEX child whose token is
   y and stopping with bonus y when no child holds it (the target's output distribution is kept:
   the token emitted after reaching a node is that node's draw).  So the sampled step is a
   per-node draw followed by that walk (oracle_sampled_accept).  Choosing among several children
   holding y by what lies below them (the deepest-path rule of the greedy case) would select
   between independent draws by their outcomes and change the emitted law.

   The draw is the Gumbel-max rule in base 2: with u_v uniform in (0, 1),
       y = argmax_v  z_v * log2(e) / T  -  log2(-log2(u_v)),
   which equals argmax_v (z_v / T + g_v) / ln 2 + const with g_v = -ln(-ln u_v) standard Gumbel
   noise, hence y ~ softmax(z / T).  The uniforms come from Philox4x32-10 (Salmon, Moraes, Dror
   and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11: ten rounds of two 32x32->64
   multiplications by 0xD2511F53 and 0xCD9E8D57, the key bumped by 0x9E3779B9 and 0xBB67AE85
   between rounds): 64-bit key = seed (low word first), 128-bit counter = (v / 4, row, low word of
   offset, high word of offset); output word k gives element 4j + k; a 32-bit word w maps to
   u = ((w >> 9) + 1/2) * 2^-23 (exact in fp32, strictly inside (0, 1)).
   The decision is taken in fp32 as the library computes it: c = (float)(log2(e) / T) rounded
   from double, s_v = fmaf(z_v, c, -log2f(-log2f(u_v))); largest s wins, lowest index on ties, a
   NaN score (NaN logit) above every number. */
static void philox_round(uint32_t x[4], const uint32_t k[2]) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x[2];
    const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x[1] ^ k[0];
    const uint32_t y1 = (uint32_t)p1;
    const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x[3] ^ k[1];
    const uint32_t y3 = (uint32_t)p0;
    x[0] = y0; x[1] = y1; x[2] = y2; x[3] = y3;
}

void oracle_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out) {
    uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) { k[0] += 0x9E3779B9u; k[1] += 0xBB67AE85u; }
        philox_round(x, k);
    }
    for (int i = 0; i < 4; ++i) out[i] = x[i];
}

float oracle_sample_uniform(uint64_t seed, uint64_t offset, int64_t row, int64_t v) {
    const uint32_t ctr[4] = {(uint32_t)(v / 4), (uint32_t)row, (uint32_t)offset, (uint32_t)(offset >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const uint32_t word = out[v % 4];
    return ((float)(word >> 9) + 0.5f) * 0x1p-23f;
}

static float sample_c(float temperature) { return (float)(1.4426950408889634 / (double)temperature); }

static float score_of(float z, float c, float u) { return fmaf(z, c, -log2f(-log2f(u))); }

/* Score of element v of row `row` with logit z (the quantity the draw maximises). */
float oracle_sample_score(float z, float temperature, uint64_t seed, uint64_t offset, int64_t row, int64_t v) {
    return score_of(z, sample_c(temperature), oracle_sample_uniform(seed, offset, row, v));
}

void oracle_node_sample(const void *logits, int32_t dtype, int64_t row_stride, int32_t num_rows, int32_t vocab,
                        float temperature, uint64_t seed, uint64_t offset, int32_t *token, float *score) {
    const float c = sample_c(temperature);
#pragma omp parallel for schedule(dynamic, 4)
    for (int32_t r = 0; r < num_rows; ++r) {
        const size_t base = (size_t)r * row_stride;
        int32_t best = -1;
        float bs = 0.f;
        for (int32_t v = 0; v < vocab; ++v) {
            const float z = (float)elem(logits, dtype, base + v);
            const float s = score_of(z, c, oracle_sample_uniform(seed, offset, r, v));
            if (isnan(s)) { best = v; bs = s; break; }
            if (best < 0 || s > bs) { best = v; bs = s; }
        }
        token[r] = best;
        if (score) score[r] = bs;
    }
}

/* Per-sequence checks shared by both acceptance rules: the tree rule, then (for a well-sized tree)
   every target token and every compared draft token inside [0, vocab).  Outputs are reset to
   "nothing accepted" (padding -1, len 0, bonus -1) first. */
static int32_t accept_prologue(const int32_t *parent, const int32_t *draft, const int32_t *target, int32_t s,
                               int32_t n, int32_t max_nodes, int32_t vocab, int32_t *path, int32_t *outt,
                               int32_t *len, int32_t *bonus) {
    for (int32_t t = 0; t < max_nodes; ++t) path[t] = outt[t] = -1;
    *len = 0;
    *bonus = -1;
    int32_t err = oracle_tree_errors(parent + s, n, max_nodes);
    if (!(err & 2)) {
        for (int32_t i = 0; i < n; ++i) {
            if (target[s + i] < 0 || target[s + i] >= vocab) err |= 4;
            if (i > 0 && (draft[s + i] < 0 || draft[s + i] >= vocab)) err |= 4;
        }
    }
    return err;
}

/* The round's outputs once the last accepted node `best` is known: path = anc(best) root first,
   len = depth(best) + 1, bonus = target[best], out_tokens = drafts of path[1..len-1], bonus. */
static void accept_emit(const int32_t *parent, const int32_t *draft, const int32_t *target, int32_t s,
                        int32_t best, int32_t *path, int32_t *outt, int32_t *len, int32_t *bonus) {
    const int32_t np = oracle_ancestor_path(parent + s, best, path);
    *len = np;
    *bonus = target[s + best];
    for (int32_t t = 1; t < np; ++t) outt[t - 1] = draft[s + path[t]];
    outt[np - 1] = *bonus;
}

/* Greedy acceptance per sequence (temperature 0).
   accepted(0) = true; for i >= 1 in index order accepted(i) = accepted(parent(i)) and
   draft[i] == target[parent(i)].  The chosen node i* maximises (depth, -index) over accepted
   nodes; the path is anc(i*) root first; len = depth(i*) + 1; bonus = target[i*];
   out_tokens = draft of path[1..len-1] followed by the bonus.  Padding is -1.  (At T = 0 the
   target tokens are fixed, so taking the deepest of several accepted siblings that hold the same
   token emits more tokens and changes no token's value.) */
void oracle_greedy_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft,
                          const int32_t *target, int32_t batch, int32_t max_nodes, int32_t vocab,
                          int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                          int32_t *out_tokens, int32_t *seq_err) {
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t s = node_start[b];
        const int32_t n = node_start[b + 1] - s;
        int32_t *path = accept_path + (size_t)b * max_nodes;
        int32_t *outt = out_tokens + (size_t)b * max_nodes;
        const int32_t err = accept_prologue(parent, draft, target, s, n, max_nodes, vocab, path, outt,
                                            &accept_len[b], &bonus_token[b]);
        seq_err[b] = err;
        if (err) continue;
        char acc[ORACLE_MAX_NODES];
        int32_t depth[ORACLE_MAX_NODES];
        acc[0] = 1;
        depth[0] = 0;
        int32_t best = 0;
        for (int32_t i = 1; i < n; ++i) {
            const int32_t p = parent[s + i];
            depth[i] = depth[p] + 1;
            acc[i] = acc[p] && draft[s + i] == target[s + p];
            if (acc[i] && depth[i] > depth[best]) best = i; /* equal depth keeps the lower index */
        }
        accept_emit(parent, draft, target, s, best, path, outt, &accept_len[b], &bonus_token[b]);
    }
}

/* Sampled acceptance per sequence (temperature > 0; target[i] is node i's draw).
   The walk starts at the root; at node x it enters the lowest-index child c of x with
   draft[c] == target[x], and stops at x when there is none.  The node where it stops is the
   last accepted one: path, len, bonus and out_tokens follow from it as in the greedy rule.
   Arguments, checks and padding are those of oracle_greedy_accept. */
void oracle_sampled_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft,
                           const int32_t *target, int32_t batch, int32_t max_nodes, int32_t vocab,
                           int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                           int32_t *out_tokens, int32_t *seq_err) {
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t s = node_start[b];
        const int32_t n = node_start[b + 1] - s;
        int32_t *path = accept_path + (size_t)b * max_nodes;
        int32_t *outt = out_tokens + (size_t)b * max_nodes;
        const int32_t err = accept_prologue(parent, draft, target, s, n, max_nodes, vocab, path, outt,
                                            &accept_len[b], &bonus_token[b]);
        seq_err[b] = err;
        if (err) continue;
        int32_t x = 0;
        for (;;) {
            int32_t next = -1;
            for (int32_t c = x + 1; c < n; ++c) {
                if (parent[s + c] == x && draft[s + c] == target[s + x]) {
                    next = c;
                    break; /* the first child holding the draw; later siblings are never tried */
                }
            }
            if (next < 0) break;
            x = next;
        }
        accept_emit(parent, draft, target, s, x, path, outt, &accept_len[b], &bonus_token[b]);
    }
}

/* KV compaction, out of place: k_out/v_out start as copies of k_in/v_in; then for every layer,
   KV head and 0 <= d < len, slot s0+L+d of the output takes slot s0+L+path[d] of the INPUT.
   new_len = L + len.  A sequence with len <= 0 is left alone (new_len = L). */
void oracle_compact_kv(const void *k_in, const void *v_in, void *k_out, void *v_out, int32_t elem_bytes,
                       int32_t num_layers, int64_t layer_stride_bytes, const int32_t *kv_start,
                       const int32_t *prefix_len, const int32_t *accept_len, const int32_t *accept_path,
                       int32_t batch, int32_t max_nodes, int64_t total_slots, int32_t hkv, int32_t d,
                       int32_t *new_len, int32_t *seq_err) {
    const size_t bytes = (size_t)num_layers * (size_t)layer_stride_bytes;
    memcpy(k_out, k_in, bytes);
    memcpy(v_out, v_in, bytes);
    const size_t row = (size_t)hkv * d * elem_bytes; /* one slot: all KV heads */
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t len = accept_len[b];
        const int32_t *path = accept_path + (size_t)b * max_nodes;
        int32_t err = 0;
        new_len[b] = prefix_len[b];
        if (len <= 0) { seq_err[b] = 0; continue; }
        if (len > max_nodes || path[0] != 0) err |= 16;
        for (int32_t t = 1; t < len && !err; ++t)
            if (path[t] <= path[t - 1]) err |= 16;
        if (!err && (kv_start[b] < 0 || prefix_len[b] < 0 ||
                     (int64_t)kv_start[b] + prefix_len[b] + path[len - 1] >= total_slots))
            err |= 8;
        seq_err[b] = err;
        if (err) continue;
        const int64_t base = (int64_t)kv_start[b] + prefix_len[b];
        for (int32_t l = 0; l < num_layers; ++l) {
            const size_t lo = (size_t)l * layer_stride_bytes;
            for (int32_t t = 0; t < len; ++t) {
                const size_t dst = lo + (size_t)(base + t) * row;
                const size_t src = lo + (size_t)(base + path[t]) * row;
                memcpy((char *)k_out + dst, (const char *)k_in + src, row);
                memcpy((char *)v_out + dst, (const char *)v_in + src, row);
            }
        }
        new_len[b] = prefix_len[b] + len;
    }
}

/* Paged KV compaction, out of place: caches [layers][total_rows][hkv][d] where a sequence's token
   t sits at page block_table[b * bt_stride + t / page_size], row t % page_size; for every layer and
   0 <= d < len, token L + d of the output takes token L + path[d] of the INPUT (the pages may
   differ).  new_len = L + len.  A sequence with len <= 0 is left alone (new_len = L). */
void oracle_compact_kv_paged(const void *k_in, const void *v_in, void *k_out, void *v_out, int32_t elem_bytes,
                             int32_t num_layers, int64_t layer_stride_bytes, const int32_t *block_table,
                             int32_t bt_stride, int32_t page_size, const int32_t *prefix_len,
                             const int32_t *accept_len, const int32_t *accept_path, int32_t batch,
                             int32_t max_nodes, int64_t total_rows, int32_t hkv, int32_t d, int32_t *new_len,
                             int32_t *seq_err) {
    const size_t bytes = (size_t)num_layers * (size_t)layer_stride_bytes;
    memcpy(k_out, k_in, bytes);
    memcpy(v_out, v_in, bytes);
    const size_t row = (size_t)hkv * d * elem_bytes; /* one token: all KV heads */
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t len = accept_len[b];
        const int32_t *path = accept_path + (size_t)b * max_nodes;
        int32_t err = 0;
        new_len[b] = prefix_len[b];
        if (len <= 0) { seq_err[b] = 0; continue; }
        if (len > max_nodes || path[0] != 0) err |= 16;
        for (int32_t t = 1; t < len && !err; ++t)
            if (path[t] <= path[t - 1]) err |= 16;
        if (!err && prefix_len[b] < 0) err |= 8;
        if (!err && ((int64_t)prefix_len[b] + path[len - 1]) / page_size >= bt_stride) err |= 8;
        for (int32_t t = 0; t < len && !err; ++t) {
            const int64_t tok[2] = {(int64_t)prefix_len[b] + t, (int64_t)prefix_len[b] + path[t]};
            for (int u = 0; u < 2; ++u) {
                const int32_t pg = block_table[(int64_t)b * bt_stride + tok[u] / page_size];
                if (pg < 0 || (int64_t)pg * page_size >= total_rows) err |= 8;
            }
        }
        seq_err[b] = err;
        if (err) continue;
        const int64_t L = prefix_len[b];
        for (int32_t l = 0; l < num_layers; ++l) {
            const size_t lo = (size_t)l * layer_stride_bytes;
            for (int32_t t = 0; t < len; ++t) {
                const size_t dst = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + t) * row;
                const size_t src = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + path[t]) * row;
                memcpy((char *)k_out + dst, (const char *)k_in + src, row);
                memcpy((char *)v_out + dst, (const char *)v_in + src, row);
            }
        }
        new_len[b] = (int32_t)(L + len);
    }
}
