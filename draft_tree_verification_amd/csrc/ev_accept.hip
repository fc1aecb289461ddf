// ev_accept.hip -- greedy longest-accepted-path selection and in-place KV compaction (gfx950).
//
// Acceptance follows the verification rule on the pages (kongchang.com English article,
// "Technical Background"): the target keeps the drafted prefix that agrees with its own greedy
// choices and adds one token of its own after it; with a draft tree several root-to-node paths
// are candidates at once.  A node is accepted when its parent is accepted and its draft token
// equals the parent's greedy target token; the deepest accepted node wins (lowest index on equal
// depth) and its target token is the bonus.  Per-sequence acceptance lengths differ inside one
// batch (same article, "Current Limitation"), so compaction moves each sequence's accepted rows
// right after its own prefix.
//
// Sampled verification (temperature > 0; the pages report T = 1 results and state that
// verification keeps the target's output distribution) takes each node's draw as its target
// token, and a child is accepted only if no lower-index sibling holds the same drafted token:
// speculative sampling tries the children in order against the node's draw, so a repeated token
// is never tried twice.  The accepted nodes are then one root path -- the walk that enters the
// first child holding the draw -- and its last node ends the round.
//
// One wavefront per sequence, lane i = tree node i (trees have at most 64 nodes).
#include <cmath>

#include "ev_internal.h"

namespace {

struct AcceptArgs {
    const int32_t *node_start, *parent, *draft, *target;
    int32_t batch, total_nodes, max_nodes, vocab;
    int32_t *accept_len, *accept_path, *bonus, *out_tokens, *err_flag;
};

// Acceptance of one sequence by one wave, lane i = node i of n, from each lane's parent, draft
// token and target token.
struct LaneAccept {
    int err;    // EV_DATA_* bits found (the same in every lane); nothing is accepted then
    int len;    // nodes on the accepted path, root included
    int bonus;  // target token of the deepest accepted node
    int depth;  // this lane's depth when its node is on the accepted path, else -1
};

// sampled: the first-child rule of sampled verification (a child repeating a lower-index
// sibling's drafted token is never accepted); otherwise the greedy rule.  n is wave-uniform.
__device__ LaneAccept accept_lanes(int lane, int n, int err, int par, int tgt, int dft, int vocab, bool sampled) {
    if (!err && lane < n) {
        if (lane == 0 ? par != -1 : (par < 0 || par >= lane)) err |= EV_DATA_BAD_PARENT;
        if (tgt < 0 || tgt >= vocab) err |= EV_DATA_BAD_TOKEN;
        if (lane > 0 && (dft < 0 || dft >= vocab)) err |= EV_DATA_BAD_TOKEN;
    }
    // OR of the error bits over the wave
    for (int o = 32; o > 0; o >>= 1) err |= __shfl_xor(err, o, 64);
    LaneAccept r{err, 0, -1, -1};
    if (err) return r;
    // an edge agrees when the child's draft token is the parent's greedy token
    const int tpar = __shfl(tgt, par >= 0 ? par : 0, 64);
    bool agree = lane < n && (lane == 0 || dft == tpar);
    if (sampled) {
        // a lower-index sibling with the same drafted token takes precedence (scalar reads of
        // every node's parent and token, one node per step)
        bool repeat = false;
        for (int j = 1; j < n; ++j) {
            const int pj = __builtin_amdgcn_readlane(par, j);
            const int dj = __builtin_amdgcn_readlane(dft, j);
            repeat |= j < lane && pj == par && dj == dft;
        }
        agree = agree && !repeat;
    }
    // accepted(i) = every edge on the root path agrees; depth(i) = edges on it; anc = bitmask
    bool acc = agree;
    int depth = 0;
    uint64_t anc = lane < n ? (1ull << lane) : 0ull;
    int j = lane < n ? par : -1;
    while (__any(j >= 0)) {
        const int jj = j >= 0 ? j : 0;
        const bool ag = __shfl(static_cast<int>(agree), jj, 64) != 0;
        const int pj = __shfl(par, jj, 64);
        if (j >= 0) {
            acc = acc && ag;
            ++depth;
            anc |= 1ull << j;
            j = pj;
        }
    }
    // deepest accepted node, lowest index on equal depth: maximise (depth << 8) | (255 - index)
    int key = (lane < n && acc) ? (depth << 8) | (255 - lane) : -1;
    for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
    const int best = 255 - (key & 255);
    r.len = (key >> 8) + 1;
    const uint32_t mlo = __shfl(static_cast<uint32_t>(anc), best, 64);
    const uint32_t mhi = __shfl(static_cast<uint32_t>(anc >> 32), best, 64);
    const uint64_t on_path = (static_cast<uint64_t>(mhi) << 32) | mlo;
    r.bonus = __shfl(tgt, best, 64);
    r.depth = (lane < n && ((on_path >> lane) & 1ull)) ? depth : -1;
    return r;
}

// The acceptance outputs of sequence b; each position is written by exactly one lane: the
// on-path node of that depth, or lane d past the path.
__device__ void write_accept(const AcceptArgs &a, int b, int lane, const LaneAccept &r, int dft) {
    int32_t *path = a.accept_path + static_cast<size_t>(b) * a.max_nodes;
    int32_t *outt = a.out_tokens + static_cast<size_t>(b) * a.max_nodes;
    if (r.err) {
        if (lane == 0) {
            ev::flag_error(a.err_flag, r.err);
            a.accept_len[b] = 0;
            a.bonus[b] = -1;
        }
        for (int i = lane; i < a.max_nodes; i += 64) path[i] = outt[i] = -1;
        return;
    }
    if (r.depth >= 0) {
        path[r.depth] = lane;
        if (lane > 0) outt[r.depth - 1] = dft;
    }
    if (lane >= r.len && lane < a.max_nodes) path[lane] = outt[lane] = -1;
    if (lane == 0) {
        outt[r.len - 1] = r.bonus;
        a.accept_len[b] = r.len;
        a.bonus[b] = r.bonus;
    }
}

// The sequence's node range (bad ranges flag EV_DATA_BAD_NODES).
__device__ __forceinline__ int node_range(const AcceptArgs &a, int b, int &ns0, int &n) {
    ns0 = a.node_start[b];
    const int ns1 = a.node_start[b + 1];
    n = ns1 - ns0;
    return (ns0 < 0 || ns1 > a.total_nodes || n < 1 || n > a.max_nodes) ? EV_DATA_BAD_NODES : 0;
}

template <bool SAMPLED>
__global__ __launch_bounds__(64) void accept_kernel(const AcceptArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int ns0, n;
    const int err = node_range(a, b, ns0, n);
    int par = -1, tgt = 0, dft = 0;
    if (!err && lane < n) {
        par = a.parent[ns0 + lane];
        tgt = a.target[ns0 + lane];
        dft = a.draft[ns0 + lane];
    }
    write_accept(a, b, lane, accept_lanes(lane, n, err, par, tgt, dft, a.vocab, SAMPLED), dft);
}

// Fused step: the per-piece winners of the selection pass and where the row tokens go.
struct SelectArgs {
    AcceptArgs acc;                      // target: unused (the tokens come from the pieces)
    const unsigned long long *pieces;    // [rows][splits]: (order key << 32) | ~index
    int32_t splits;
    int32_t sampled;                     // the pieces are draws (temperature > 0): first-child rule
    int32_t *target_out;                 // [rows] the finished tokens
};

struct CompactArgs {
    unsigned char *k, *v;
    int64_t layer_stride;
    const int32_t *kv_start, *prefix_len, *accept_len, *accept_path;
    const int32_t *block_table;       // paged caches (else NULL): [batch][bt_stride] pool pages
    int32_t bt_stride, page_size;
    int32_t batch, max_nodes, row16;  // row16: 16-byte chunks per slot row
    int64_t total_slots, row_bytes;   // paged: total_slots = pool pages * page_size
    int32_t *new_len, *err_flag;
};

constexpr int kCompactThreads = 256;
constexpr int kBatchRows = 8;

// Block (b, layer).  Rows move in increasing d; a destination token L+d can only be the source
// of some d' <= d (path[d'] >= d' since the path strictly increases from 0), so every source is
// read before anything overwrites it even though each thread streams its own columns
// independently.  With a block table the same holds row by row as long as the sequence's pages
// are distinct (tokens then map to distinct rows).
//
// Fused step (FUSED): wave 0 first finishes the sequence's target tokens from the selection
// pass's pieces (maximum of the packed words), runs the acceptance rule, and hands the accepted
// path to the other waves through LDS; the layer-0 workgroup writes the tokens and the
// acceptance outputs.  Every layer's workgroup repeats the (small) acceptance work instead of
// waiting for another workgroup.
template <bool FUSED>
__global__ __launch_bounds__(kCompactThreads) void compact_kv_kernel(const CompactArgs a, const SelectArgs sel) {
    const int b = blockIdx.x;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    __shared__ int64_t s_src[EV_MAX_NODES], s_dst[EV_MAX_NODES];
    __shared__ int s_path[FUSED ? EV_MAX_NODES : 1];
    __shared__ int s_len;
    const int L = a.prefix_len[b];
    const int s0 = a.block_table ? 0 : a.kv_start[b];  // loaded up front, used after the path is known
    int len, err = 0, p = 0, last = 0;
    if constexpr (FUSED) {
        if (tid < 64) {
            const AcceptArgs &x = sel.acc;
            int ns0, n;
            const int err0 = node_range(x, b, ns0, n);
            int par = -1, tgt = 0, dft = 0;
            if (!err0 && tid < n) {
                const int row = ns0 + tid;
                par = x.parent[row];
                dft = x.draft[row];
                // the row's pieces in groups of sixteen independent loads, one round trip for
                // vocabularies up to 16 pieces (indices clamped to the last piece: a repeat does
                // not change a maximum)
                const unsigned long long *pc = sel.pieces + static_cast<size_t>(row) * sel.splits;
                unsigned long long w = 0;
                for (int k0 = 0; k0 < sel.splits; k0 += 16) {
                    unsigned long long x[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) x[k] = pc[min(k0 + k, sel.splits - 1)];
#pragma unroll
                    for (int k = 0; k < 16; ++k) w = x[k] > w ? x[k] : w;
                }
                tgt = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(w & 0xFFFFFFFFu));
                if (layer == 0) sel.target_out[row] = tgt;
            }
            const LaneAccept r = accept_lanes(tid, n, err0, par, tgt, dft, x.vocab, sel.sampled != 0);
            if (layer == 0) write_accept(x, b, tid, r, dft);
            if (r.depth >= 0) s_path[r.depth] = tid;
            if (tid == 0) s_len = r.err ? 0 : r.len;
        }
        __syncthreads();
        len = s_len;
        if (tid < len) p = s_path[tid];
        if (len > 0) last = s_path[len - 1];
    } else {
        len = a.accept_len[b];
        if (len > 0) {
            if (len > a.max_nodes) err = EV_DATA_BAD_PATH;
            if (!err && tid < len) {
                p = a.accept_path[static_cast<size_t>(b) * a.max_nodes + tid];
                const int prev = tid ? a.accept_path[static_cast<size_t>(b) * a.max_nodes + tid - 1] : -1;
                if (tid == 0 ? p != 0 : p <= prev) err = EV_DATA_BAD_PATH;
            }
        }
        err = __syncthreads_or(err) ? EV_DATA_BAD_PATH : 0;
        if (len > 0 && !err) last = a.accept_path[static_cast<size_t>(b) * a.max_nodes + len - 1];
    }
    if (len > 0 && !err) {
        if (!a.block_table) {
            if (s0 < 0 || L < 0 || static_cast<int64_t>(s0) + L + last >= a.total_slots) err = EV_DATA_BAD_SLOTS;
            else if (tid < len) {
                s_src[tid] = static_cast<int64_t>(s0) + L + p;
                s_dst[tid] = static_cast<int64_t>(s0) + L + tid;
            }
        } else if (L < 0 || (static_cast<int64_t>(L) + last) / a.page_size >= a.bt_stride) {
            err = EV_DATA_BAD_SLOTS;
        } else {
            int bad = 0;
            if (tid < len) {
                const int32_t *bt = a.block_table + static_cast<size_t>(b) * a.bt_stride;
                const int64_t num_pages = a.total_slots / a.page_size;
                const int64_t ts = static_cast<int64_t>(L) + p, td = static_cast<int64_t>(L) + tid;
                const int ps = bt[ts / a.page_size], pd = bt[td / a.page_size];
                bad = ps < 0 || ps >= num_pages || pd < 0 || pd >= num_pages;
                s_src[tid] = static_cast<int64_t>(ps) * a.page_size + ts % a.page_size;
                s_dst[tid] = static_cast<int64_t>(pd) * a.page_size + td % a.page_size;
            }
            err = __syncthreads_or(bad) ? EV_DATA_BAD_SLOTS : 0;
        }
    }
    if (layer == 0 && tid == 0) {
        a.new_len[b] = (len > 0 && !err) ? L + len : L;
        ev::flag_error(a.err_flag, err);
    }
    if (len <= 1 || err) return;
    __syncthreads();  // the row indices are in LDS
    const int64_t base = static_cast<int64_t>(layer) * a.layer_stride;
    for (int c = tid; c < 2 * a.row16; c += kCompactThreads) {
        unsigned char *buf = (c < a.row16 ? a.k : a.v) + base + static_cast<int64_t>(c % a.row16) * 16;
        for (int d0 = 1; d0 < len; d0 += kBatchRows) {
            u32x4_t rows[kBatchRows];
#pragma unroll
            for (int i = 0; i < kBatchRows; ++i) {
                const int d = d0 + i;
                if (d < len && s_src[d] != s_dst[d]) rows[i] = ev::ld16(buf + s_src[d] * a.row_bytes);
            }
#pragma unroll
            for (int i = 0; i < kBatchRows; ++i) {
                const int d = d0 + i;
                if (d < len && s_src[d] != s_dst[d])
                    *reinterpret_cast<u32x4_t *>(buf + s_dst[d] * a.row_bytes) = rows[i];
            }
        }
    }
}

}  // namespace

namespace {
ev_status launch_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft_token,
                        const int32_t *target_token, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                        int32_t vocab, int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token,
                        int32_t *out_tokens, int32_t *err_flag, bool sampled, hipStream_t stream) {
    if (!node_start || !parent || !draft_token || !target_token || !accept_len || !accept_path || !bonus_token ||
        !out_tokens)
        return EV_ERR_NULL;
    if (batch < 0 || total_nodes < 0 || max_nodes < 1 || max_nodes > EV_MAX_NODES || vocab < 1) return EV_ERR_SHAPE;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (batch == 0) return EV_OK;
    AcceptArgs args{node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes, vocab,
                    accept_len, accept_path, bonus_token, out_tokens, err_flag};
    if (sampled) hipLaunchKernelGGL(accept_kernel<true>, dim3(batch), dim3(64), 0, stream, args);
    else hipLaunchKernelGGL(accept_kernel<false>, dim3(batch), dim3(64), 0, stream, args);
    return ev::launch_status();
}
}  // namespace

extern "C" ev_status ev_greedy_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft_token,
                                      const int32_t *target_token, int32_t batch, int32_t total_nodes,
                                      int32_t max_nodes, int32_t vocab, int32_t *accept_len, int32_t *accept_path,
                                      int32_t *bonus_token, int32_t *out_tokens, int32_t *err_flag,
                                      hipStream_t stream) {
    return launch_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes, vocab,
                         accept_len, accept_path, bonus_token, out_tokens, err_flag, false, stream);
}

extern "C" ev_status ev_sampled_accept(const int32_t *node_start, const int32_t *parent, const int32_t *draft_token,
                                       const int32_t *target_token, int32_t batch, int32_t total_nodes,
                                       int32_t max_nodes, int32_t vocab, int32_t *accept_len, int32_t *accept_path,
                                       int32_t *bonus_token, int32_t *out_tokens, int32_t *err_flag,
                                       hipStream_t stream) {
    return launch_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes, vocab,
                         accept_len, accept_path, bonus_token, out_tokens, err_flag, true, stream);
}

namespace {
// Checks of the compaction's arguments; fills the kernel arguments.
ev_status compact_args(void *k_cache, void *v_cache, int32_t elem_bytes, int32_t num_layers,
                       int64_t layer_stride_bytes, const int32_t *kv_start, const int32_t *block_table,
                       int32_t bt_stride, int32_t page_size, const int32_t *prefix_len, const int32_t *accept_len,
                       const int32_t *accept_path, int32_t batch, int32_t max_nodes, int64_t total_slots,
                       int32_t num_kv_heads, int32_t head_dim, int32_t *new_len, int32_t *err_flag, bool fused,
                       CompactArgs &args) {
    if (!k_cache || !v_cache || !prefix_len || (!fused && (!accept_len || !accept_path)) || !new_len ||
        (block_table ? false : !kv_start))
        return EV_ERR_NULL;
    if (batch < 0 || num_layers < 1 || max_nodes < 1 || max_nodes > EV_MAX_NODES || total_slots < 0 ||
        num_kv_heads < 1 || head_dim < 1)
        return EV_ERR_SHAPE;
    if (elem_bytes != 2 && elem_bytes != 4) return EV_ERR_DTYPE;
    const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes;
    if (layer_stride_bytes < total_slots * row_bytes) return EV_ERR_SHAPE;
    if (!ev::aligned16(k_cache) || !ev::aligned16(v_cache) || row_bytes % 16 || layer_stride_bytes % 16)
        return EV_ERR_ALIGN;
    if (new_len == prefix_len) return EV_ERR_SHAPE;
    args.k = static_cast<unsigned char *>(k_cache);
    args.v = static_cast<unsigned char *>(v_cache);
    args.layer_stride = layer_stride_bytes;
    args.kv_start = kv_start;
    args.prefix_len = prefix_len;
    args.accept_len = accept_len;
    args.accept_path = accept_path;
    args.block_table = block_table;
    args.bt_stride = bt_stride;
    args.page_size = page_size;
    args.batch = batch;
    args.max_nodes = max_nodes;
    args.row16 = static_cast<int32_t>(row_bytes / 16);
    args.total_slots = total_slots;
    args.row_bytes = row_bytes;
    args.new_len = new_len;
    args.err_flag = err_flag;
    return EV_OK;
}

ev_status launch_compact(void *k_cache, void *v_cache, int32_t elem_bytes, int32_t num_layers,
                         int64_t layer_stride_bytes, const int32_t *kv_start, const int32_t *block_table,
                         int32_t bt_stride, int32_t page_size, const int32_t *prefix_len, const int32_t *accept_len,
                         const int32_t *accept_path, int32_t batch, int32_t max_nodes, int64_t total_slots,
                         int32_t num_kv_heads, int32_t head_dim, int32_t *new_len, int32_t *err_flag,
                         hipStream_t stream) {
    CompactArgs args;
    const ev_status st = compact_args(k_cache, v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start,
                                      block_table, bt_stride, page_size, prefix_len, accept_len, accept_path, batch,
                                      max_nodes, total_slots, num_kv_heads, head_dim, new_len, err_flag, false, args);
    if (st != EV_OK) return st;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (batch == 0) return EV_OK;
    hipLaunchKernelGGL(compact_kv_kernel<false>, dim3(batch, num_layers), dim3(kCompactThreads), 0, stream, args,
                       SelectArgs{});
    return ev::launch_status();
}

size_t select_bytes(int32_t rows, int32_t vocab) {
    if (rows <= 0 || vocab < 1) return 0;
    const size_t b = static_cast<size_t>(rows) * ev::select_splits(rows, vocab) * 8;
    return (b + 255) / 256 * 256;
}

// The fused step: every argument is checked before the first launch; then the selection pass
// (pieces into the workspace) and the fused compaction launch, which finishes the row tokens,
// accepts and compacts.
ev_status select_accept_compact(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t vocab,
                                float temperature, uint64_t seed, uint64_t offset, const int32_t *node_start,
                                const int32_t *parent, const int32_t *draft_token, int32_t batch,
                                int32_t total_nodes, int32_t max_nodes, void *k_cache, void *v_cache,
                                int32_t elem_bytes, int32_t num_layers, int64_t layer_stride_bytes,
                                const int32_t *kv_start, const int32_t *block_table, int32_t bt_stride,
                                int32_t page_size, const int32_t *prefix_len, int64_t total_slots,
                                int32_t num_kv_heads, int32_t head_dim, int32_t *target_token, int32_t *accept_len,
                                int32_t *accept_path, int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len,
                                void *workspace, size_t workspace_bytes, int32_t *err_flag, hipStream_t stream,
                                bool validate_only = false, bool selection_launched = false) {
    if (!logits || !node_start || !parent || !draft_token || !target_token || !accept_len || !accept_path ||
        !bonus_token || !out_tokens)
        return EV_ERR_NULL;
    if (batch < 0 || total_nodes < 0 || max_nodes < 1 || max_nodes > EV_MAX_NODES || vocab < 1 || row_stride < vocab)
        return EV_ERR_SHAPE;
    if (!std::isfinite(temperature) || temperature < 0.f) return EV_ERR_SHAPE;
    // (the draw's scale log2(e)/T must be a finite float)
    if (temperature > 0.f && !std::isfinite(static_cast<float>(1.4426950408889634 / static_cast<double>(temperature))))
        return EV_ERR_SHAPE;
    if (dtype != EV_BF16 && dtype != EV_F32) return EV_ERR_DTYPE;
    const int esz = dtype == EV_BF16 ? 2 : 4;
    if (!ev::aligned16(logits) || (row_stride * esz) % 16) return EV_ERR_ALIGN;
    const size_t need = select_bytes(total_nodes, vocab);
    if (need && (!workspace || workspace_bytes < need)) return EV_ERR_WORKSPACE;
    if (need && (reinterpret_cast<uintptr_t>(workspace) & 7u)) return EV_ERR_ALIGN;
    CompactArgs cargs;
    ev_status st = compact_args(k_cache, v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start, block_table,
                                bt_stride, page_size, prefix_len, nullptr, nullptr, batch, max_nodes, total_slots,
                                num_kv_heads, head_dim, new_len, err_flag, true, cargs);
    if (st != EV_OK) return st;
    if (validate_only) return EV_OK;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (batch == 0) return EV_OK;
    SelectArgs sel{};
    sel.acc = AcceptArgs{node_start, parent, draft_token, nullptr, batch, total_nodes, max_nodes, vocab,
                         accept_len, accept_path, bonus_token, out_tokens, err_flag};
    sel.pieces = static_cast<const unsigned long long *>(workspace);
    sel.splits = total_nodes > 0 ? ev::select_splits(total_nodes, vocab) : 1;
    sel.target_out = target_token;
    sel.sampled = temperature > 0.f;
    if (total_nodes > 0 && !selection_launched) {
        st = ev::launch_select_pieces(logits, dtype, row_stride, total_nodes, vocab, temperature, seed, offset,
                                      static_cast<unsigned long long *>(workspace), stream);
        if (st != EV_OK) return st;
    }
    hipLaunchKernelGGL(compact_kv_kernel<true>, dim3(batch, num_layers), dim3(kCompactThreads), 0, stream, cargs, sel);
    return ev::launch_status();
}
}  // namespace

extern "C" ev_status ev_compact_kv(void *k_cache, void *v_cache, int32_t elem_bytes, int32_t num_layers,
                                   int64_t layer_stride_bytes, const int32_t *kv_start, const int32_t *prefix_len,
                                   const int32_t *accept_len, const int32_t *accept_path, int32_t batch,
                                   int32_t max_nodes, int64_t total_slots, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t *new_len, int32_t *err_flag, hipStream_t stream) {
    return launch_compact(k_cache, v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start, nullptr, 0, 0,
                          prefix_len, accept_len, accept_path, batch, max_nodes, total_slots, num_kv_heads, head_dim,
                          new_len, err_flag, stream);
}

extern "C" ev_status ev_compact_kv_paged(void *k_pages, void *v_pages, int32_t elem_bytes, int32_t num_layers,
                                         int64_t layer_stride_bytes, const int32_t *block_table, int32_t bt_stride,
                                         int32_t page_size, const int32_t *prefix_len, const int32_t *accept_len,
                                         const int32_t *accept_path, int32_t batch, int32_t max_nodes,
                                         int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, int32_t *new_len,
                                         int32_t *err_flag, hipStream_t stream) {
    if (!block_table) return EV_ERR_NULL;
    if (page_size < 1 || bt_stride < 1 || num_pages < 0) return EV_ERR_SHAPE;
    return launch_compact(k_pages, v_pages, elem_bytes, num_layers, layer_stride_bytes, nullptr, block_table,
                          bt_stride, page_size, prefix_len, accept_len, accept_path, batch, max_nodes,
                          static_cast<int64_t>(num_pages) * page_size, num_kv_heads, head_dim, new_len, err_flag,
                          stream);
}

extern "C" size_t ev_select_workspace_size(int32_t num_rows, int32_t vocab) { return select_bytes(num_rows, vocab); }

extern "C" ev_status ev_select_accept_compact(
    const void *logits, ev_dtype dtype, int64_t row_stride, int32_t vocab, float temperature, uint64_t seed,
    uint64_t offset, const int32_t *node_start, const int32_t *parent, const int32_t *draft_token, int32_t batch,
    int32_t total_nodes, int32_t max_nodes, void *k_cache, void *v_cache, int32_t elem_bytes, int32_t num_layers,
    int64_t layer_stride_bytes, const int32_t *kv_start, const int32_t *prefix_len, int64_t total_slots,
    int32_t num_kv_heads, int32_t head_dim, int32_t *target_token, int32_t *accept_len, int32_t *accept_path,
    int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len, void *workspace, size_t workspace_bytes,
    int32_t *err_flag, hipStream_t stream) {
    return select_accept_compact(logits, dtype, row_stride, vocab, temperature, seed, offset, node_start, parent,
                                 draft_token, batch, total_nodes, max_nodes, k_cache, v_cache, elem_bytes, num_layers,
                                 layer_stride_bytes, kv_start, nullptr, 0, 0, prefix_len, total_slots, num_kv_heads,
                                 head_dim, target_token, accept_len, accept_path, bonus_token, out_tokens, new_len,
                                 workspace, workspace_bytes, err_flag, stream);
}

extern "C" ev_status ev_select_accept_compact_paged(
    const void *logits, ev_dtype dtype, int64_t row_stride, int32_t vocab, float temperature, uint64_t seed,
    uint64_t offset, const int32_t *node_start, const int32_t *parent, const int32_t *draft_token, int32_t batch,
    int32_t total_nodes, int32_t max_nodes, void *k_pages, void *v_pages, int32_t elem_bytes, int32_t num_layers,
    int64_t layer_stride_bytes, const int32_t *block_table, int32_t bt_stride, int32_t page_size,
    const int32_t *prefix_len, int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, int32_t *target_token,
    int32_t *accept_len, int32_t *accept_path, int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len,
    void *workspace, size_t workspace_bytes, int32_t *err_flag, hipStream_t stream) {
    if (!block_table) return EV_ERR_NULL;
    if (page_size < 1 || bt_stride < 1 || num_pages < 0) return EV_ERR_SHAPE;
    return select_accept_compact(logits, dtype, row_stride, vocab, temperature, seed, offset, node_start, parent,
                                 draft_token, batch, total_nodes, max_nodes, k_pages, v_pages, elem_bytes, num_layers,
                                 layer_stride_bytes, nullptr, block_table, bt_stride, page_size, prefix_len,
                                 static_cast<int64_t>(num_pages) * page_size, num_kv_heads, head_dim, target_token,
                                 accept_len, accept_path, bonus_token, out_tokens, new_len, workspace,
                                 workspace_bytes, err_flag, stream);
}

// ---------------------------------------------------------------------------------------------
// The whole verification step as one call: the attention (and the merge of split units), the
// selection pass, then acceptance and compaction, in that order on the caller's stream, after
// every argument of all of them has been checked.  Workspace: the selection pieces (a multiple
// of 256 bytes), then the attention workspace.
extern "C" size_t ev_verify_step_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                int32_t vocab) {
    if (total_nodes < 0 || vocab < 1) return 0;
    const size_t attn = ev_tree_attention_workspace_size(batch, max_nodes, num_q_heads, num_kv_heads, head_dim);
    if (!attn) return 0;
    return select_bytes(total_nodes, vocab) + attn;
}

extern "C" ev_status ev_verify_step(
    const void *q, void *k_cache, void *v_cache, void *out, float *lse, const int32_t *node_start,
    const int32_t *parent, const int32_t *kv_start, const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
    int32_t max_nodes, int64_t total_slots, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int64_t kv_slot_stride, int64_t kv_head_stride, ev_dtype dtype, float sm_scale, const void *logits,
    ev_dtype logits_dtype, int64_t row_stride, int32_t vocab, float temperature, uint64_t seed, uint64_t offset,
    const int32_t *draft_token, int32_t num_layers, int64_t layer_stride_bytes, int32_t compact_kv_heads,
    int32_t compact_head_dim, int32_t *target_token, int32_t *accept_len, int32_t *accept_path,
    int32_t *bonus_token, int32_t *out_tokens, int32_t *new_len, void *workspace, size_t workspace_bytes,
    int32_t *err_flag, hipStream_t stream) {
    if (!workspace) return EV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return EV_ERR_ALIGN;
    if (total_nodes < 0 || vocab < 1) return EV_ERR_SHAPE;
    const size_t need = ev_verify_step_workspace_size(batch, total_nodes, max_nodes, num_q_heads, num_kv_heads,
                                                      head_dim, vocab);
    if (!need) return EV_ERR_SHAPE;
    if (workspace_bytes < need) return EV_ERR_WORKSPACE;
    const size_t sel = select_bytes(total_nodes, vocab);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int32_t elem_bytes = dtype == EV_F32 ? 4 : 2;
    // the selection/acceptance/compaction arguments first (no device call), then the attention
    // launcher checks its own before its first launch and runs the selection pass with it (beside
    // the merge of split units when there is a merge at head_dim 128), then the acceptance and
    // compaction launch
    ev_status st = select_accept_compact(logits, logits_dtype, row_stride, vocab, temperature, seed, offset,
                                         node_start, parent, draft_token, batch, total_nodes, max_nodes, k_cache,
                                         v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start, nullptr, 0, 0,
                                         prefix_len, total_slots, compact_kv_heads, compact_head_dim, target_token,
                                         accept_len, accept_path, bonus_token, out_tokens, new_len, ws, sel, err_flag,
                                         stream, true);
    if (st != EV_OK) return st;
    ev::AttentionCall attn{};
    attn.q = q;
    attn.k_cache = k_cache;
    attn.v_cache = v_cache;
    attn.out = out;
    attn.lse = lse;
    attn.node_start = node_start;
    attn.parent = parent;
    attn.kv_start = kv_start;
    attn.prefix_len = prefix_len;
    attn.batch = batch;
    attn.total_nodes = total_nodes;
    attn.max_nodes = max_nodes;
    attn.total_slots = total_slots;
    attn.num_q_heads = num_q_heads;
    attn.num_kv_heads = num_kv_heads;
    attn.head_dim = head_dim;
    attn.slot_stride = kv_slot_stride;
    attn.head_stride = kv_head_stride;
    attn.dtype = dtype;
    attn.sm_scale = sm_scale;
    attn.workspace = ws + sel;
    attn.workspace_bytes = workspace_bytes - sel;
    attn.err_flag = err_flag;
    const ev::SelectJob job{logits, logits_dtype, row_stride, total_nodes, vocab, temperature, seed, offset,
                            reinterpret_cast<unsigned long long *>(ws)};
    st = ev::launch_attention_step(attn, &job, stream);
    if (st != EV_OK) return st;
    return select_accept_compact(logits, logits_dtype, row_stride, vocab, temperature, seed, offset, node_start,
                                 parent, draft_token, batch, total_nodes, max_nodes, k_cache, v_cache, elem_bytes,
                                 num_layers, layer_stride_bytes, kv_start, nullptr, 0, 0, prefix_len, total_slots,
                                 compact_kv_heads, compact_head_dim, target_token, accept_len, accept_path,
                                 bonus_token, out_tokens, new_len, ws, sel, err_flag, stream, false, true);
}
