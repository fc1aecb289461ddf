// ev_argmax.hip -- per-node greedy target token (row argmax over the vocabulary) for gfx950.
//
// At temperature 0 the target's own choice at every tree node is the argmax of its logits row
// (aiposthub.com analysis, "paper Table 2": greedy T=0 verification); the accept step compares
// each child's draft token with it.  The result must be bit-exact, so the total order is fixed:
// larger value first, lower index on ties, +0 == -0, any NaN above every number.
//
// HBM-bound streaming: each thread reads 16 bytes per load, eight loads in flight.  Values are
// mapped to order-preserving unsigned keys (sign-magnitude -> offset binary, both zeros to the
// same key); for bf16 the key transform and the per-load maximum run on packed 16-bit integer
// ops, and a round of eight loads searches an index only when its maximum beats the running best,
// and then only in the first load that holds it, so ties keep the earliest index for free.  Rows with few rows in the
// batch are split across workgroups; the pieces meet through a 64-bit atomicMax on
// (key << 32 | ~index) and the last-arriving workgroup writes the token.  In the fused step
// (ev_select_accept_compact) each piece instead stores its (key << 32 | ~index) word, and the
// acceptance launch that follows takes the maximum over a row's pieces: no atomics, no arrival
// counting, nothing to reset.
#include <cmath>

#include "ev_select.h"

namespace {

using namespace ev::sel;

template <bool F32IN>
__global__ __launch_bounds__(kThreads) void node_argmax_kernel(const ArgmaxArgs a) {
    argmax_piece<F32IN>(a, static_cast<int>(blockIdx.x));
}

template <bool F32IN>
__global__ __launch_bounds__(kThreads) void node_sample_kernel(const ArgmaxArgs a) {
    sample_piece<F32IN>(a, static_cast<int>(blockIdx.x));
}

struct ArgmaxPlan {
    int splits, seg;
    size_t bytes;
};

ArgmaxPlan make_plan(int32_t rows, int32_t vocab) {
    ArgmaxPlan p{};
    int splits = rows >= kTargetBlocks ? 1 : (kTargetBlocks + rows - 1) / rows;
    const int max_by_len = (vocab + kSplitQuanta * kSegQuantum - 1) / (kSplitQuanta * kSegQuantum);
    if (splits > max_by_len) splits = max_by_len;
    if (splits < 1) splits = 1;
    int seg = (vocab + splits - 1) / splits;
    seg = ((seg + kSegQuantum - 1) / kSegQuantum) * kSegQuantum;
    splits = (vocab + seg - 1) / seg;
    p.splits = splits;
    p.seg = seg;
    p.bytes = splits > 1 ? ((static_cast<size_t>(rows) * 12 + 255) / 256) * 256 : 0;
    return p;
}

}  // namespace

namespace ev {

int select_splits(int32_t rows, int32_t vocab) { return make_plan(rows, vocab).splits; }

void select_plan(int32_t rows, int32_t vocab, int32_t &splits, int32_t &seg) {
    const ArgmaxPlan p = make_plan(rows, vocab);
    splits = p.splits;
    seg = p.seg;
}

ev_status launch_select_pieces(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t rows, int32_t vocab,
                               float temperature, uint64_t seed, uint64_t offset, unsigned long long *pieces,
                               hipStream_t stream) {
    const ArgmaxPlan plan = make_plan(rows, vocab);
    ArgmaxArgs args{};
    args.logits = logits;
    args.row_stride = row_stride;
    args.rows = rows;
    args.vocab = vocab;
    args.splits = plan.splits;
    args.seg = plan.seg;
    args.pieces = pieces;
    const dim3 grid(static_cast<unsigned>(rows) * plan.splits);
    if (temperature > 0.f) {
        args.c = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
        args.seed = seed;
        args.offset = offset;
        if (dtype == EV_BF16)
            hipLaunchKernelGGL(node_sample_kernel<false>, grid, dim3(kThreads), 0, stream, args);
        else
            hipLaunchKernelGGL(node_sample_kernel<true>, grid, dim3(kThreads), 0, stream, args);
    } else if (dtype == EV_BF16) {
        hipLaunchKernelGGL(node_argmax_kernel<false>, grid, dim3(kThreads), 0, stream, args);
    } else {
        hipLaunchKernelGGL(node_argmax_kernel<true>, grid, dim3(kThreads), 0, stream, args);
    }
    return launch_status();
}

}  // namespace ev

extern "C" size_t ev_node_argmax_workspace_size(int32_t num_rows, int32_t vocab) {
    if (num_rows < 0 || vocab < 1) return 0;
    return make_plan(num_rows, vocab).bytes;
}

extern "C" ev_status ev_node_argmax(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t num_rows,
                                    int32_t vocab, int32_t *target_token, float *max_value, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (!logits || !target_token) return EV_ERR_NULL;
    if (num_rows < 0 || vocab < 1 || row_stride < vocab) return EV_ERR_SHAPE;
    if (dtype != EV_BF16 && dtype != EV_F32) return EV_ERR_DTYPE;
    const int esz = dtype == EV_BF16 ? 2 : 4;
    if (!ev::aligned16(logits) || (row_stride * esz) % 16) return EV_ERR_ALIGN;
    const ArgmaxPlan plan = make_plan(num_rows, vocab);
    if (plan.bytes && (!workspace || workspace_bytes < plan.bytes)) return EV_ERR_WORKSPACE;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (num_rows == 0) return EV_OK;
    ArgmaxArgs args{};
    args.logits = logits;
    args.row_stride = row_stride;
    args.rows = num_rows;
    args.vocab = vocab;
    args.splits = plan.splits;
    args.seg = plan.seg;
    args.target = target_token;
    args.max_value = max_value;
    args.keys = static_cast<unsigned long long *>(workspace);
    args.counters = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(workspace) +
                                                static_cast<size_t>(num_rows) * 8);
    const dim3 grid(static_cast<unsigned>(num_rows) * plan.splits);
    if (dtype == EV_BF16)
        hipLaunchKernelGGL(node_argmax_kernel<false>, grid, dim3(kThreads), 0, stream, args);
    else
        hipLaunchKernelGGL(node_argmax_kernel<true>, grid, dim3(kThreads), 0, stream, args);
    return ev::launch_status();
}

extern "C" ev_status ev_node_sample(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t num_rows,
                                    int32_t vocab, float temperature, uint64_t seed, uint64_t offset,
                                    int32_t *target_token, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (!logits || !target_token) return EV_ERR_NULL;
    if (num_rows < 0 || vocab < 1 || row_stride < vocab) return EV_ERR_SHAPE;
    if (!std::isfinite(temperature) || !(temperature > 0.f)) return EV_ERR_SHAPE;
    const float c = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
    if (!std::isfinite(c)) return EV_ERR_SHAPE;
    if (dtype != EV_BF16 && dtype != EV_F32) return EV_ERR_DTYPE;
    const int esz = dtype == EV_BF16 ? 2 : 4;
    if (!ev::aligned16(logits) || (row_stride * esz) % 16) return EV_ERR_ALIGN;
    const ArgmaxPlan plan = make_plan(num_rows, vocab);
    if (plan.bytes && (!workspace || workspace_bytes < plan.bytes)) return EV_ERR_WORKSPACE;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (num_rows == 0) return EV_OK;
    ArgmaxArgs args{};
    args.logits = logits;
    args.row_stride = row_stride;
    args.rows = num_rows;
    args.vocab = vocab;
    args.splits = plan.splits;
    args.seg = plan.seg;
    args.target = target_token;
    args.max_value = nullptr;
    args.keys = static_cast<unsigned long long *>(workspace);
    args.counters = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(workspace) +
                                                static_cast<size_t>(num_rows) * 8);
    args.c = c;
    args.seed = seed;
    args.offset = offset;
    const dim3 grid(static_cast<unsigned>(num_rows) * plan.splits);
    if (dtype == EV_BF16)
        hipLaunchKernelGGL(node_sample_kernel<false>, grid, dim3(kThreads), 0, stream, args);
    else
        hipLaunchKernelGGL(node_sample_kernel<true>, grid, dim3(kThreads), 0, stream, args);
    return ev::launch_status();
}
