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

#include "ev_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;                        // elements per thread per load group
constexpr int kSegQuantum = kThreads * kChunk;   // segment lengths are multiples of this
constexpr int kTargetBlocks = 2048;
constexpr int kSplitQuanta = 8;                  // a split of few rows: 8 quanta, one load batch per thread

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short ss2 __attribute__((ext_vector_type(2)));

struct ArgmaxArgs {
    const void *logits;
    int64_t row_stride;
    int32_t rows, vocab, splits, seg;
    int32_t *target;
    float *max_value;
    unsigned long long *keys;  // [rows] (only when splits > 1)
    int32_t *counters;         // [rows]
    unsigned long long *pieces;  // [rows][splits] each piece's winner (fused step), else NULL
    float c;                   // sampling: log2(e) / temperature
    uint64_t seed, offset;     // sampling: Philox key
};

// Order-preserving key of a bf16 value (16 bits, in a uint32): +-0 -> 0x8000, NaN -> 0xFFFF.
__device__ __forceinline__ uint32_t key_bf16(uint32_t h) {
    const uint32_t mag = h & 0x7FFFu;
    if (mag > 0x7F80u) return 0xFFFFu;
    return (h & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
}
// Order-preserving key of an fp32 value: +-0 -> 0x80000000, NaN -> 0xFFFFFFFF.
__device__ __forceinline__ uint32_t key_f32(uint32_t u) {
    const uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return 0xFFFFFFFFu;
    return (u & 0x80000000u) ? 0x80000000u - mag : 0x80000000u + mag;
}
__device__ __forceinline__ float value_of_key(uint32_t key, bool f32) {
    if (f32) {
        if (key == 0xFFFFFFFFu) return __builtin_nanf("");
        const uint32_t bits = key >= 0x80000000u ? key - 0x80000000u : (0x80000000u - key) | 0x80000000u;
        return __builtin_bit_cast(float, bits);
    }
    if (key == 0xFFFFu) return __builtin_nanf("");
    const uint32_t h = key >= 0x8000u ? key - 0x8000u : (0x8000u - key) | 0x8000u;
    return __builtin_bit_cast(float, h << 16);
}

// Keys of two packed bf16 values without NaN handling (the caller checks for NaN separately).
__device__ __forceinline__ us2 keys2(uint32_t w) {
    const us2 h = __builtin_bit_cast(us2, w);
    const us2 mag = h & static_cast<unsigned short>(0x7FFF);
    const us2 smask = __builtin_bit_cast(us2, __builtin_bit_cast(ss2, h) >> static_cast<short>(15));
    return ((mag ^ smask) - smask) + static_cast<unsigned short>(0x8000);
}

// Largest key of the eight bf16 values in one 16-byte load, 0xFFFF when any of them is a NaN.
__device__ __forceinline__ uint32_t load_max_key(u32x4_t w) {
    const us2 k0 = keys2(w[0]), k1 = keys2(w[1]), k2 = keys2(w[2]), k3 = keys2(w[3]);
    const us2 km = __builtin_elementwise_max(__builtin_elementwise_max(k0, k1), __builtin_elementwise_max(k2, k3));
    const us2 mags = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(us2, w[0] & 0x7FFF7FFFu), __builtin_bit_cast(us2, w[1] & 0x7FFF7FFFu)),
        __builtin_elementwise_max(__builtin_bit_cast(us2, w[2] & 0x7FFF7FFFu), __builtin_bit_cast(us2, w[3] & 0x7FFF7FFFu)));
    const bool has_nan = mags[0] > 0x7F80u || mags[1] > 0x7F80u;
    return has_nan ? 0xFFFFu : (km[0] > km[1] ? km[0] : km[1]);
}

__device__ __forceinline__ unsigned long long pack(uint32_t key, int32_t idx) {
    return (static_cast<unsigned long long>(key) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

// Wave-wide unsigned maximum: DPP row shifts (an inclusive scan within each 16-lane row; lanes
// shifted in from outside the row read 0, the identity) and the four rows' last lanes.
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, false)));
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, false)));
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, false)));
    x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, false)));
    const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
    const uint32_t r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
    return max(max(r0, r1), max(r2, r3));
}

// The workgroup's best (key, lowest index) for `row`, then across the row's split workgroups;
// the row's token (and the maximum, if asked for) is written once.  Workgroup-uniform call.
__device__ __forceinline__ void finish_row(const ArgmaxArgs &a, int row, uint32_t best, int32_t bidx, bool f32) {
    const int tid = threadIdx.x;
    // wave reduction of (key, lowest index): the largest key, then the lowest index among the
    // lanes that hold it (register-only DPP steps, no LDS permutes)
    const uint32_t kmax = wave_umax(best);
    const uint32_t imin = ~wave_umax(~(best == kmax ? static_cast<uint32_t>(bidx) : 0xFFFFFFFFu));
    unsigned long long p = kmax ? pack(kmax, static_cast<int32_t>(imin)) : 0ull;
    __shared__ unsigned long long s_red[kThreads / 64];
    if ((tid & 63) == 0) s_red[tid >> 6] = p;
    __syncthreads();
    if (tid != 0) return;
    for (int w = 1; w < kThreads / 64; ++w) p = s_red[w] > p ? s_red[w] : p;

    if (a.pieces) {  // the acceptance launch combines the row's pieces
        a.pieces[static_cast<size_t>(row) * a.splits + blockIdx.x % a.splits] = p;
        return;
    }
    if (a.splits > 1) {
        // all three are device-coherent atomics on the same path: the max lands before this
        // workgroup's arrival is counted, and the last arriver's exchange sees every max
        __hip_atomic_fetch_max(a.keys + row, p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ev::vm_wait();
        const int old = ev::atomic_add_agent(a.counters + row, 1);
        if (old != a.splits - 1) return;
        p = __hip_atomic_exchange(a.keys + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.counters + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t key = static_cast<uint32_t>(p >> 32);
    a.target[row] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(p & 0xFFFFFFFFu));
    if (a.max_value) a.max_value[row] = value_of_key(key, f32);
}

template <bool F32IN>
__global__ __launch_bounds__(kThreads) void node_argmax_kernel(const ArgmaxArgs a) {
    const int row = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
    const int v0 = split * a.seg;
    const int v1 = min(a.vocab, v0 + a.seg);
    const int tid = threadIdx.x;
    uint32_t best = 0;           // keys are >= 0x80 for every real value, so 0 means "none"
    int32_t bidx = 0x7FFFFFFF;

    if constexpr (!F32IN) {
        const uint16_t *rp = static_cast<const uint16_t *>(a.logits) + static_cast<int64_t>(row) * a.row_stride;
        int base = v0 + tid * kChunk;
        auto consume = [&](u32x4_t w, int at) {
            const us2 k0 = keys2(w[0]), k1 = keys2(w[1]), k2 = keys2(w[2]), k3 = keys2(w[3]);
            const us2 km = __builtin_elementwise_max(__builtin_elementwise_max(k0, k1), __builtin_elementwise_max(k2, k3));
            const us2 mags = __builtin_elementwise_max(
                __builtin_elementwise_max(__builtin_bit_cast(us2, w[0] & 0x7FFF7FFFu),
                                          __builtin_bit_cast(us2, w[1] & 0x7FFF7FFFu)),
                __builtin_elementwise_max(__builtin_bit_cast(us2, w[2] & 0x7FFF7FFFu),
                                          __builtin_bit_cast(us2, w[3] & 0x7FFF7FFFu)));
            const uint32_t kmax = km[0] > km[1] ? km[0] : km[1];
            const bool has_nan = mags[0] > 0x7F80u || mags[1] > 0x7F80u;
            if (kmax > best || has_nan) {
                // exact scan of these eight values in index order
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t h = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                    const uint32_t k = key_bf16(h);
                    if (k > best) { best = k; bidx = at + e; }
                }
            }
        };
        // main body: eight 16-byte loads in flight per thread (a split of 8 quanta is one round trip).
        // Each load's maximum key comes from the packed keys (0xFFFF when the load holds a NaN);
        // only when the round's maximum beats the running best is a single load -- the first
        // one holding that maximum -- scanned value by value for its lowest index.  (A wave runs
        // a per-lane scan whenever any of its lanes needs one, so scanning per load would run
        // nearly every load's scan in the first rounds.)
        for (; base + 7 * kSegQuantum + kChunk <= v1; base += 8 * kSegQuantum) {
            u32x4_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = ev::ld16_stream(rp + base + k * kSegQuantum);
            uint32_t km[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) km[k] = load_max_key(w[k]);
            uint32_t rk = km[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) rk = km[k] > rk ? km[k] : rk;
            if (rk > best) {
                u32x4_t x = w[7];
                int at = base + 7 * kSegQuantum;
#pragma unroll
                for (int k = 6; k >= 0; --k) {
                    if (km[k] == rk) {
                        x = w[k];
                        at = base + k * kSegQuantum;
                    }
                }
                int first = at + 7;
#pragma unroll
                for (int e = 6; e >= 0; --e) {
                    const uint32_t h = (e & 1) ? (x[e >> 1] >> 16) : (x[e >> 1] & 0xFFFFu);
                    if (key_bf16(h) == rk) first = at + e;
                }
                best = rk;
                bidx = first;
            }
        }
        for (; base + 3 * kSegQuantum + kChunk <= v1; base += 4 * kSegQuantum) {
            u32x4_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = ev::ld16_stream(rp + base + k * kSegQuantum);
#pragma unroll
            for (int k = 0; k < 4; ++k) consume(w[k], base + k * kSegQuantum);
        }
        for (; base + kChunk <= v1; base += kSegQuantum) consume(ev::ld16_stream(rp + base), base);
        if (base < v1) {  // ragged end of the row: element by element
            for (int e = base; e < v1; ++e) {
                const uint32_t k = key_bf16(rp[e]);
                if (k > best) { best = k; bidx = e; }
            }
        }
    } else {
        const float *rp = static_cast<const float *>(a.logits) + static_cast<int64_t>(row) * a.row_stride;
        int base = v0 + tid * kChunk;
        auto consume = [&](u32x4_t x, u32x4_t y, int at) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t k = key_f32(e < 4 ? x[e] : y[e - 4]);
                if (k > best) { best = k; bidx = at + e; }
            }
        };
        for (; base + kChunk <= v1; base += kSegQuantum)
            consume(ev::ld16_stream(rp + base), ev::ld16_stream(rp + base + 4), base);
        if (base < v1) {
            for (int e = base; e < v1; ++e) {
                const uint32_t k = key_f32(__builtin_bit_cast(uint32_t, rp[e]));
                if (k > best) { best = k; bidx = e; }
            }
        }
    }

    finish_row(a, row, best, bidx, F32IN);
}

// ---------------------------------------------------------------------------------------------
// Sampled draw per row (temperature T > 0): y = argmax_v  z_v * c - log2(-log2(u_v)),
// c = log2(e) / T, the Gumbel-max rule in base 2, so y ~ softmax(z / T).  Each draw feeds the same
// greedy acceptance rule as the argmax: with drafted children taken as point proposals, a walk
// that descends into the child holding the node's draw is speculative sampling along the tree
// (the target's sampling distribution is kept; arex-research.com release note, opening section).
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) keyed by (seed, offset) on the
// counter (v / 8, row, 0, 0); output k feeds elements 8j + 2k (low word) and 8j + 2k + 1 (high
// word); word w -> u = ((w >> 9) + 1/2) * 2^-23.  One Philox block per thread per 16-byte load of
// eight bf16 logits.  The scores are fp32: the logit times c fused with the noise subtraction.
// Bound by the ALU (about 30 integer ops of Philox and two hardware log2 per element), not HBM.
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint64_t lo0 = kPhiloxM0 * x[0], hi0 = __umul64hi(kPhiloxM0, x[0]);
        const uint64_t lo1 = kPhiloxM1 * x[2], hi1 = __umul64hi(kPhiloxM1, x[2]);
        const uint64_t y0 = hi1 ^ x[1] ^ k0, y2 = hi0 ^ x[3] ^ k1;
        x[0] = y0;
        x[1] = lo1;
        x[2] = y2;
        x[3] = lo0;
    }
}

// Score of one element from its logit and its 32-bit random word.
__device__ __forceinline__ float sample_score(float z, uint32_t word, float c) {
    const float u = (static_cast<float>(word >> 9) + 0.5f) * 0x1p-23f;  // exact: 24 significant bits
    const float e = -__builtin_amdgcn_logf(u);                          // -log2(u) > 0
    return __builtin_fmaf(z, c, -__builtin_amdgcn_logf(e));
}

template <bool F32IN>
__global__ __launch_bounds__(kThreads) void node_sample_kernel(const ArgmaxArgs a) {
    const int row = blockIdx.x / a.splits, split = blockIdx.x % a.splits;
    const int v0 = split * a.seg;
    const int v1 = min(a.vocab, v0 + a.seg);
    const int tid = threadIdx.x;
    uint32_t best = 0;
    int32_t bidx = 0x7FFFFFFF;
    const float c = a.c;
    auto take = [&](float z, uint32_t word, int idx) {
        const uint32_t k = key_f32(__builtin_bit_cast(uint32_t, sample_score(z, word, c)));
        if (k > best) { best = k; bidx = idx; }
    };
    auto block = [&](int j, uint32_t (&w)[8]) {
        uint64_t x[4] = {static_cast<uint64_t>(j), static_cast<uint64_t>(row), 0ull, 0ull};
        philox4x64_10(x, a.seed, a.offset);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[2 * k] = static_cast<uint32_t>(x[k]);
            w[2 * k + 1] = static_cast<uint32_t>(x[k] >> 32);
        }
    };
    const unsigned char *rp = static_cast<const unsigned char *>(a.logits) +
                              static_cast<int64_t>(row) * a.row_stride * (F32IN ? 4 : 2);
    int base = v0 + tid * kChunk;
    // two 16-byte loads (bf16) or four (fp32) ahead of the ALU work of each group of eight
    for (; base + kSegQuantum + kChunk <= v1; base += 2 * kSegQuantum) {
        float z[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int at = base + h * kSegQuantum;
            if constexpr (F32IN) {
                const f32x4_t p = ev::ld16f_stream(reinterpret_cast<const float *>(rp) + at);
                const f32x4_t q = ev::ld16f_stream(reinterpret_cast<const float *>(rp) + at + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { z[h][e] = p[e]; z[h][e + 4] = q[e]; }
            } else {
                const u32x4_t p = ev::ld16_stream(reinterpret_cast<const uint16_t *>(rp) + at);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[h][2 * e] = __builtin_bit_cast(float, p[e] << 16);
                    z[h][2 * e + 1] = __builtin_bit_cast(float, p[e] & 0xFFFF0000u);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int at = base + h * kSegQuantum;
            uint32_t w[8];
            block(at >> 3, w);
#pragma unroll
            for (int e = 0; e < 8; ++e) take(z[h][e], w[e], at + e);
        }
    }
    for (; base + kChunk <= v1; base += kSegQuantum) {
        uint32_t w[8];
        block(base >> 3, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float z = F32IN ? reinterpret_cast<const float *>(rp)[base + e]
                                  : __builtin_bit_cast(float, static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(rp)[base + e]) << 16);
            take(z, w[e], base + e);
        }
    }
    if (base < v1) {  // ragged end of the row (fewer than eight elements): one block for all of them
        uint32_t w[8];
        block(base >> 3, w);
        for (int e = base; e < v1; ++e) {
            const float z = F32IN ? reinterpret_cast<const float *>(rp)[e]
                                  : __builtin_bit_cast(float, static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(rp)[e]) << 16);
            take(z, w[e - base], e);
        }
    }
    finish_row(a, row, best, bidx, F32IN);
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
