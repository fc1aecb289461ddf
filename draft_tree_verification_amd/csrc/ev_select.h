// ev_select.h -- the per-node selection pass of gfx950 (row argmax at temperature 0, the sampled
// draw at temperature > 0), one row piece per 256-thread workgroup: device code shared by the
// selection kernels (ev_argmax.hip) and by the whole-step call's launch that runs the selection
// pieces beside the merge of split attention units (ev_attention.hip).  The algorithms and their
// orders are described in ev_argmax.hip.
#pragma once

#include "ev_internal.h"

namespace ev {
namespace sel {

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
    uint64_t seed, offset;     // sampling: Philox key (seed) and counter words 2-3 (offset)
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
__device__ __forceinline__ void finish_row(const ArgmaxArgs &a, int row, uint32_t best, int32_t bidx, bool f32,
                                           int piece) {
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
        a.pieces[static_cast<size_t>(row) * a.splits + static_cast<unsigned>(piece) % static_cast<unsigned>(a.splits)] = p;
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
__device__ __forceinline__ void argmax_piece(const ArgmaxArgs &a, int piece) {
    const unsigned up = static_cast<unsigned>(piece), us = static_cast<unsigned>(a.splits);
    const int row = static_cast<int>(up / us), split = static_cast<int>(up % us);
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

    finish_row(a, row, best, bidx, F32IN, piece);
}

// ---------------------------------------------------------------------------------------------
// Sampled draw per row (temperature T > 0): y = argmax_v  z_v * c - log2(-log2(u_v)),
// c = log2(e) / T, the Gumbel-max rule in base 2, so y ~ softmax(z / T).  Each draw feeds the same
// greedy acceptance rule as the argmax: with drafted children taken as point proposals, a walk
// that descends into the child holding the node's draw is speculative sampling along the tree
// (the target's sampling distribution is kept; arex-research.com release note, opening section).
// Uniforms: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) under the 64-bit key seed (low word
// first) on the 128-bit counter (v / 4, row, low and high words of offset); output word k feeds
// element 4j + k; word w -> u = ((w >> 9) + 1/2) * 2^-23.  Two Philox blocks per thread per
// 16-byte load of eight bf16 logits.  The scores are fp32: the logit times c fused with the noise
// subtraction.  Bound by the ALU (Philox's 32x32->64 products run on v_mad_u64_u32, five per
// element, and two hardware log2 per element), not HBM.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * x[0];  // one v_mad_u64_u32 each
        const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * x[2];
        // three-way XORs in one v_bitop3_b32 each (truth table 0x96)
        const uint32_t y0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), x[1], k0, 0x96);
        const uint32_t y2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), x[3], k1, 0x96);
        x[0] = y0;
        x[1] = static_cast<uint32_t>(p1);
        x[2] = y2;
        x[3] = static_cast<uint32_t>(p0);
    }
}

// Score of one element from its logit and its 32-bit random word.  The uniform is built from its
// bits: 0x3F800000 | (w >> 9) is 1 + (w >> 9) * 2^-23, and subtracting 1 - 2^-24 is exact
// (Sterbenz), giving ((w >> 9) + 1/2) * 2^-23 in two operations.
__device__ __forceinline__ float sample_score(float z, uint32_t word, float c) {
    const float u = __builtin_bit_cast(float, __builtin_amdgcn_alignbit(0x7Fu, word, 9u)) - 0x1.fffffep-1f;
    const float e = -__builtin_amdgcn_logf(u);                          // -log2(u) > 0
    return __builtin_fmaf(z, c, -__builtin_amdgcn_logf(e));
}

template <bool F32IN>
__device__ __forceinline__ void sample_piece(const ArgmaxArgs &a, int piece) {
    const unsigned up = static_cast<unsigned>(piece), us = static_cast<unsigned>(a.splits);
    const int row = static_cast<int>(up / us), split = static_cast<int>(up % us);
    const int v0 = split * a.seg;
    const int v1 = min(a.vocab, v0 + a.seg);
    const int tid = threadIdx.x;
    const float c = a.c;
    // The thread's best score and its index.  Scores are compared as floats: a score is NaN only
    // where its logit is NaN (u lies strictly inside (0, 1) and c is finite and positive), so a
    // load whose eight logits hold no NaN takes the plain strict comparison (earliest index on
    // ties, +0 == -0), and only a load holding a NaN takes the NaN-aware one (a NaN above every
    // number, the first NaN kept).  Starting from -inf at the thread's first index covers a
    // thread whose every score is -inf.
    float bs = -__builtin_inff();
    int32_t bidx = v0 + tid * kChunk < v1 ? v0 + tid * kChunk : 0x7FFFFFFF;
    auto take_plain = [&](float z, uint32_t word, int idx) {
        const float sc = sample_score(z, word, c);
        if (sc > bs) { bs = sc; bidx = idx; }
    };
    auto take_nan = [&](float z, uint32_t word, int idx) {
        const float sc = sample_score(z, word, c);
        if (sc > bs || (__builtin_isnan(sc) && !__builtin_isnan(bs))) { bs = sc; bidx = idx; }
    };
    auto take8 = [&](const float (&z)[8], const uint32_t (&w)[8], int at) {
        // NaN if a logit is NaN (or if +inf and -inf meet: then the exact path runs needlessly)
        const float zs = ((z[0] + z[1]) + (z[2] + z[3])) + ((z[4] + z[5]) + (z[6] + z[7]));
        if (__builtin_isnan(zs)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) take_nan(z[e], w[e], at + e);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) take_plain(z[e], w[e], at + e);
        }
    };
    // the eight words of elements 8j .. 8j + 7: Philox blocks 2j and 2j + 1
    const uint32_t klo = static_cast<uint32_t>(a.seed), khi = static_cast<uint32_t>(a.seed >> 32);
    const uint32_t olo = static_cast<uint32_t>(a.offset), ohi = static_cast<uint32_t>(a.offset >> 32);
    auto block = [&](int j, uint32_t (&w)[8]) {
        uint32_t x[4] = {static_cast<uint32_t>(2 * j), static_cast<uint32_t>(row), olo, ohi};
        uint32_t y[4] = {static_cast<uint32_t>(2 * j + 1), static_cast<uint32_t>(row), olo, ohi};
        philox4x32_10(x, klo, khi);
        philox4x32_10(y, klo, khi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[k] = x[k];
            w[4 + k] = y[k];
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
            take8(z[h], w, at);
        }
    }
    for (; base + kChunk <= v1; base += kSegQuantum) {
        uint32_t w[8];
        block(base >> 3, w);
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            z[e] = F32IN ? reinterpret_cast<const float *>(rp)[base + e]
                         : __builtin_bit_cast(float, static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(rp)[base + e]) << 16);
        take8(z, w, base);
    }
    if (base < v1) {  // ragged end of the row (fewer than eight elements): one block for all of them
        uint32_t w[8];
        block(base >> 3, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // (unrolled: the words stay in registers)
            if (base + e < v1) {
                const float z = F32IN ? reinterpret_cast<const float *>(rp)[base + e]
                                      : __builtin_bit_cast(float, static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(rp)[base + e]) << 16);
                take_nan(z, w[e], base + e);
            }
        }
    }
    const uint32_t best = bidx == 0x7FFFFFFF ? 0u : key_f32(__builtin_bit_cast(uint32_t, bs));
    finish_row(a, row, best, bidx, F32IN, piece);
}

}  // namespace sel
}  // namespace ev
