// ev_attention.hip -- tree-masked GQA verification attention for gfx950 (MI355X).
//
// What it computes: for every draft-tree node i of sequence b and q head h, softmax attention
// over the sequence's KV prefix plus the tree slots of i's ancestors and i itself (the target's
// single parallel verification forward over the whole draft tree: kongchang.com English
// article, "Technical Background"; EAGLE-2's dynamic tree covers several candidate paths in one
// verification).  The KV cache is bf16 and never quantised (arex-research.com release note,
// plugin section: tree verification needs an unquantised KV cache).
//
// How (one launch, no second merge kernel):
//   * Work unit = (sequence, row group, KV head).  A unit's rows are all (node, q-head-in-group)
//     pairs of that KV head -- up to 80 rows -- so every K/V byte is read from HBM exactly once
//     and shared by all N*G rows (the arithmetic intensity is N*G flop per byte).
//   * Stream-K split: each unit's keys are cut into 32-key steps; all steps of all units are laid
//     end to end and the grid's workgroups take equal contiguous ranges (ragged prefix lengths
//     cost nothing in balance).  Workgroup ranges are mapped XCD-major so the pieces of one unit
//     mostly land on one XCD's L2.
//   * Inside a workgroup the four waves take steps round-robin (split-K across waves).  Per step
//     a wave loads 32 keys of K straight into MFMA A-operand registers (16-byte loads, 256-byte
//     rows), computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (Q staged once per piece in
//     LDS), applies the ancestor mask only on steps that reach the tree slots, runs the online
//     softmax in fp32 with exp2, and accumulates O^T = V^T P^T.  V is transposed through a
//     wave-private LDS tile; the score layout already matches P^T's operand layout, so P needs
//     no shuffle and the output rows sit on the same lanes as the softmax state.
//   * The four waves merge through LDS in a fixed order; a unit covered by one workgroup is
//     written directly, otherwise each piece writes (m, l, O) partials and the last-arriving
//     workgroup of the unit merges them in workgroup order (deterministic).
#include <cmath>
#include <mutex>

#include "ev_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;          // keys per wave step (the K extent of one 16x16x32 MFMA)
constexpr int kMaxGrid = 512;      // workgroups per launch (bounds the partial-result slots)
constexpr int kMaxRowTiles = 5;    // 16-row tiles per unit: at most 80 rows
constexpr int kVtPitch = 72;       // bytes per row of a wave's V^T tile (32 keys + pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    float *lse;
    const int32_t *node_start;
    const int32_t *parent;
    const int32_t *kv_start;
    const int32_t *prefix_len;
    int64_t total_slots;
    int32_t batch, total_nodes, max_nodes, hq, hkv, group, row_groups;
    float scale_log2;  // sm_scale * log2(e): scores live in the base-2 domain
    int32_t *counters; // [batch * row_groups * hkv] arrival counters
    float *part;       // [2 * kMaxGrid] partial-result slots
    int32_t *err_flag;
};

template <int D, int RT>
struct Layout {
    static constexpr int R = RT * 16;
    static constexpr int QP = D + 8;     // bf16 per staged Q row (pad breaks bank aliasing)
    static constexpr int OP = D + 4;     // floats per row of a merge buffer
    static constexpr int kScan = EV_MAX_BATCH * 8;
    static constexpr int kMisc = 64;
    static constexpr int kQ = R * QP * 2;
    static constexpr int kVt = kWaves * D * kVtPitch;
    static constexpr int kMerge = 2 * R * OP * 4 + 2 * kWaves * R * 4;
    static constexpr int kBody = (kQ + kVt) > kMerge ? (kQ + kVt) : kMerge;
    static constexpr int kTotal = kScan + kMisc + kBody;
    static constexpr size_t kSlotFloats = (size_t)R * D + 2 * R;  // O [R][D], then m [R], l [R]
};

__device__ __forceinline__ int64_t shfl_up_i64(int64_t x, int o) {
    const int lo = __shfl_up(static_cast<int>(x & 0xFFFFFFFF), o, 64);
    const int hi = __shfl_up(static_cast<int>(x >> 32), o, 64);
    return (static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo);
}

// Workgroup (logical index) whose step range contains step x: the largest w with
// floor(w*S/P) <= x.
__device__ __forceinline__ int wg_of(int64_t x, int64_t S, int P) {
    return static_cast<int>(((x + 1) * P - 1) / S);
}

template <int D, int RT, bool F32IN>
__global__ __launch_bounds__(kThreads, 1) void tree_attention_kernel(const AttnArgs a) {
    using Lay = Layout<D, RT>;
    constexpr int R = Lay::R;
    constexpr int QP = Lay::QP;
    constexpr int OP = Lay::OP;
    constexpr int KS = D / 32;          // k-steps of the QK^T contraction
    constexpr int DT = D / 16;          // 16-wide d tiles of O^T
    constexpr int CPR = D / 8;          // 8-element chunks per K/V row
    constexpr int KG = 64 / CPR;        // key rows covered by one V load instruction
    constexpr int NQ = kStep / (4 * KG);  // quads of 4 keys per lane per step
    static_assert(NQ >= 1, "V load mapping");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kTotal];
    int64_t *s_cum = reinterpret_cast<int64_t *>(smem);
    int64_t *s_wsum = reinterpret_cast<int64_t *>(smem + Lay::kScan);  // [kWaves]
    int32_t *s_flag = reinterpret_cast<int32_t *>(smem + Lay::kScan + 32);
    unsigned char *body = smem + Lay::kScan + Lay::kMisc;
    uint16_t *s_q = reinterpret_cast<uint16_t *>(body);
    float *s_oa = reinterpret_cast<float *>(body);
    float *s_ob = s_oa + R * OP;
    float *s_mw = s_ob + R * OP;
    float *s_lw = s_mw + kWaves * R;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;
    const int lq = lane >> 4;
    unsigned char *s_vt = body + Lay::kQ + wave * D * kVtPitch;
    const int G = a.group;

    // ---- schedule: per-sequence step counts and their inclusive scan (identical in every WG)
    int64_t carry = 0;
    for (int b0 = 0; b0 < a.batch; b0 += kThreads) {
        const int b = b0 + tid;
        int64_t work = 0;
        if (b < a.batch) {
            const int ns0 = a.node_start[b], ns1 = a.node_start[b + 1];
            const int n = ns1 - ns0;
            const int L = a.prefix_len[b], s0 = a.kv_start[b];
            int err = 0;
            if (ns0 < 0 || ns1 > a.total_nodes || n < 1 || n > a.max_nodes)
                err = EV_DATA_BAD_NODES;
            else if (L < 0 || s0 < 0 || static_cast<int64_t>(s0) + L + n > a.total_slots)
                err = EV_DATA_BAD_SLOTS;
            if (err) {
                if (blockIdx.x == 0) ev::flag_error(a.err_flag, err);
            } else {
                work = static_cast<int64_t>(a.hkv) * ((n * G + R - 1) / R) * ((L + n + kStep - 1) / kStep);
            }
        }
        int64_t x = work;
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t y = shfl_up_i64(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_wsum[wave] = x;
        __syncthreads();
        int64_t wbase = 0, tot = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) wbase += s_wsum[w];
            tot += s_wsum[w];
        }
        if (b < a.batch) s_cum[b] = carry + wbase + x;
        carry += tot;
        __syncthreads();
    }
    const int64_t S = carry;
    const int P = gridDim.x;
    const int wl = (P % 8 == 0) ? (blockIdx.x % 8) * (P / 8) + blockIdx.x / 8 : blockIdx.x;
    const int64_t begin = S * wl / P, end = S * (wl + 1) / P;

    for (int64_t pos = begin; pos < end;) {
        // ---- locate the unit that holds step `pos`
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] > pos) hi = mid; else lo = mid + 1;
        }
        const int b = lo;
        const int64_t seq_base = b ? s_cum[b - 1] : 0;
        const int ns0 = a.node_start[b];
        const int n = a.node_start[b + 1] - ns0;
        const int L = a.prefix_len[b];
        const int64_t s0 = a.kv_start[b];
        const int steps = (L + n + kStep - 1) / kStep;
        const int ui = static_cast<int>((pos - seq_base) / steps);
        const int rg = ui / a.hkv, g = ui % a.hkv;
        const int64_t ustart = seq_base + static_cast<int64_t>(ui) * steps, uend = ustart + steps;
        const int64_t pend = end < uend ? end : uend;
        const int st0 = static_cast<int>(pos - ustart), st1 = static_cast<int>(pend - ustart);
        pos = pend;

        // ---- tree: validity and ancestor masks (every wave derives the same values)
        int par = -1;
        bool ok = true;
        if (lane < n) {
            par = a.parent[ns0 + lane];
            ok = lane == 0 ? par == -1 : (par >= 0 && par < lane);
        }
        if (__any(!ok)) {
            if (tid == 0) ev::flag_error(a.err_flag, EV_DATA_BAD_PARENT);
            continue;  // uniform across the workgroup: every wave read the same parents
        }
        uint64_t anc = lane < n ? (1ull << lane) : 0ull;
        int j = lane < n ? par : -1;
        while (__any(j >= 0)) {
            if (j >= 0) anc |= 1ull << j;
            const int pj = __shfl(par, j >= 0 ? j : 0, 64);
            j = j >= 0 ? pj : -1;
        }
        const int nrows = n * G;
        uint64_t rmask[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row = rg * R + 16 * t + lr;
            const int node = row < nrows ? row / G : 0;
            const uint32_t mlo = __shfl(static_cast<uint32_t>(anc), node, 64);
            const uint32_t mhi = __shfl(static_cast<uint32_t>(anc >> 32), node, 64);
            rmask[t] = row < nrows ? ((static_cast<uint64_t>(mhi) << 32) | mlo) : 0ull;
        }

        // ---- stage this unit's Q rows (bf16) in LDS
        __syncthreads();
        for (int c = tid; c < R * CPR; c += kThreads) {
            const int r = c / CPR, ch = c % CPR;
            const int row = rg * R + r;
            u32x4_t val = {0u, 0u, 0u, 0u};
            if (row < nrows) {
                const int node = row / G, h = g * G + row % G;
                const size_t off = (static_cast<size_t>(ns0 + node) * a.hq + h) * D + ch * 8;
                if constexpr (F32IN) {
                    const float *qp = static_cast<const float *>(a.q) + off;
                    val = ev::f32x8_to_bf16x8(ev::ld16f(qp), ev::ld16f(qp + 4));
                } else {
                    val = ev::ld16(static_cast<const uint16_t *>(a.q) + off);
                }
            }
            *reinterpret_cast<u32x4_t *>(s_q + r * QP + ch * 8) = val;
        }
        __syncthreads();

        // ---- this wave's steps
        const int kv_end = L + n;  // unit-relative key positions below this exist
        const size_t slot_stride = static_cast<size_t>(a.hkv) * D;  // elements between slots
        const size_t head_off = static_cast<size_t>(s0) * slot_stride + static_cast<size_t>(g) * D;
        const int vc = lane % CPR, vkg = lane / CPR;

        f32x4_t o[RT][DT];
        float m_run[RT], l_run[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            m_run[t] = -INFINITY;
            l_run[t] = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        auto load_step = [&](int st, u32x4_t (&kd)[2][KS], u32x4_t (&vd)[NQ][4]) {
            const int kb = st * kStep;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int p = kb + 16 * u + lr;
                const size_t base = head_off + static_cast<size_t>(p) * slot_stride + 8 * lq;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    u32x4_t val = {0u, 0u, 0u, 0u};
                    if (p < kv_end) {
                        if constexpr (F32IN) {
                            const float *kp = static_cast<const float *>(a.k) + base + 32 * s;
                            val = ev::f32x8_to_bf16x8(ev::ld16f_stream(kp), ev::ld16f_stream(kp + 4));
                        } else {
                            val = ev::ld16_stream(static_cast<const uint16_t *>(a.k) + base + 32 * s);
                        }
                    }
                    kd[u][s] = val;
                }
            }
#pragma unroll
            for (int qd = 0; qd < NQ; ++qd) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int p = kb + 4 * (vkg + KG * qd) + jj;
                    u32x4_t val = {0u, 0u, 0u, 0u};
                    if (p < kv_end) {
                        const size_t off = head_off + static_cast<size_t>(p) * slot_stride + 8 * vc;
                        if constexpr (F32IN) {
                            const float *vp = static_cast<const float *>(a.v) + off;
                            val = ev::f32x8_to_bf16x8(ev::ld16f_stream(vp), ev::ld16f_stream(vp + 4));
                        } else {
                            val = ev::ld16_stream(static_cast<const uint16_t *>(a.v) + off);
                        }
                    }
                    vd[qd][jj] = val;
                }
            }
        };

        int st = st0 + wave;
        u32x4_t kr[2][KS], vr[NQ][4];
        if (st < st1) load_step(st, kr, vr);
        for (; st < st1; st += kWaves) {
            u32x4_t kn[2][KS], vn[NQ][4];
            const bool more = st + kWaves < st1;
            if (more) load_step(st + kWaves, kn, vn);

            // V^T tile: row d holds this step's 32 keys of column d (4 keys per 8-byte write)
#pragma unroll
            for (int qd = 0; qd < NQ; ++qd) {
                const int kq = 4 * (vkg + KG * qd);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t w0 = __builtin_amdgcn_perm(vr[qd][1][e >> 1], vr[qd][0][e >> 1], sel);
                    const uint32_t w1 = __builtin_amdgcn_perm(vr[qd][3][e >> 1], vr[qd][2][e >> 1], sel);
                    *reinterpret_cast<u32x2_t *>(s_vt + (8 * vc + e) * kVtPitch + 2 * kq) = u32x2_t{w0, w1};
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

            // S^T = K Q^T : sc[u][t] holds keys 16u + 4*lq + r for row 16t + lr
            f32x4_t sc[2][RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                bf16x8_t qop[KS];
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    qop[s] = *reinterpret_cast<const bf16x8_t *>(s_q + (16 * t + lr) * QP + 32 * s + 8 * lq);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, kr[u][s]), qop[s], acc, 0, 0, 0);
                    sc[u][t] = acc * a.scale_log2;
                }
            }
            const int kb = st * kStep;
            if (kb + kStep > L) {  // this step reaches the tree slots or the unit's end
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = kb + 16 * u + 4 * lq + r;
#pragma unroll
                        for (int t = 0; t < RT; ++t) {
                            const bool vis = p < L || (p < kv_end && ((rmask[t] >> (p - L)) & 1ull));
                            if (!vis) sc[u][t][r] = -INFINITY;
                        }
                    }
                }
            }

            // online softmax (fp32); P rounded to bf16 and laid out as the P^T operand
            bf16x8_t pop[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                float mx = fmaxf(fmaxf(fmaxf(sc[0][t][0], sc[0][t][1]), fmaxf(sc[0][t][2], sc[0][t][3])),
                                 fmaxf(fmaxf(sc[1][t][0], sc[1][t][1]), fmaxf(sc[1][t][2], sc[1][t][3])));
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[t], mx);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_use);
                u32x4_t pw;
                float psum = 0.f;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const uint32_t w = ev::pack_bf16x2(__builtin_amdgcn_exp2f(sc[u][t][2 * h2] - m_use),
                                                           __builtin_amdgcn_exp2f(sc[u][t][2 * h2 + 1] - m_use));
                        psum += ev::bf_lo(w) + ev::bf_hi(w);
                        pw[2 * u + h2] = w;
                    }
                }
                pop[t] = __builtin_bit_cast(bf16x8_t, pw);
                l_run[t] = l_run[t] * alpha + psum;
                if (__any(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
                }
                m_run[t] = m_new;
            }

            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const unsigned char *vrow = s_vt + (16 * dt + lr) * kVtPitch + 8 * lq;
                const u32x2_t v0 = *reinterpret_cast<const u32x2_t *>(vrow);
                const u32x2_t v1 = *reinterpret_cast<const u32x2_t *>(vrow + 32);
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, u32x4_t{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], o[t][dt], 0, 0, 0);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

            if (more) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int s = 0; s < KS; ++s) kr[u][s] = kn[u][s];
#pragma unroll
                for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) vr[qd][jj] = vn[qd][jj];
            }
        }

        // ---- per-row sums over the four lanes that share a row
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            l_run[t] += __shfl_xor(l_run[t], 16, 64);
            l_run[t] += __shfl_xor(l_run[t], 32, 64);
        }

        // ---- merge the four waves (fixed order: (w0 + w2) + (w1 + w3))
        __syncthreads();
        if (lq == 0) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                s_mw[wave * R + 16 * t + lr] = m_run[t];
                s_lw[wave * R + 16 * t + lr] = l_run[t];
            }
        }
        __syncthreads();
        float m_tot[RT], l_tot[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int row = 16 * t + lr;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_mw[w * R + row]);
            const float Mu = M == -INFINITY ? 0.f : M;
            float lt = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) lt += s_lw[w * R + row] * __builtin_amdgcn_exp2f(s_mw[w * R + row] - Mu);
            const float c = __builtin_amdgcn_exp2f(m_run[t] - Mu);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[t][dt] *= c;
            m_tot[t] = M;
            l_tot[t] = lt;
        }
        auto store_o = [&](float *buf) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<f32x4_t *>(buf + (16 * t + lr) * OP + 16 * dt + 4 * lq) = o[t][dt];
        };
        auto add_o = [&](const float *buf) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[t][dt] += *reinterpret_cast<const f32x4_t *>(buf + (16 * t + lr) * OP + 16 * dt + 4 * lq);
        };
        __syncthreads();
        if (wave == 2) store_o(s_oa);
        if (wave == 3) store_o(s_ob);
        __syncthreads();
        if (wave == 0) add_o(s_oa);
        if (wave == 1) add_o(s_ob);
        __syncthreads();
        if (wave == 1) store_o(s_oa);
        __syncthreads();
        if (wave == 0) add_o(s_oa);

        // ---- output
        const bool whole = ustart >= begin && uend <= end;
        if (whole) {
            if (wave == 0) {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const int row = rg * R + 16 * t + lr;
                    if (row >= nrows) continue;
                    const int node = row / G, h = g * G + row % G;
                    const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
                    const float inv = 1.f / l_tot[t];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const f32x4_t val = o[t][dt] * inv;
                        const size_t off = orow * D + 16 * dt + 4 * lq;
                        if constexpr (F32IN) {
                            *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + off) = val;
                        } else {
                            *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + off) =
                                u32x2_t{ev::pack_bf16x2(val[0], val[1]), ev::pack_bf16x2(val[2], val[3])};
                        }
                    }
                    if (a.lse && lq == 0) a.lse[orow] = (m_tot[t] + __log2f(l_tot[t])) * kLn2;
                }
            }
            continue;
        }

        // ---- split unit: publish this piece's partial, the last arriver merges all pieces
        const int w1 = wg_of(ustart, S, P), w2 = wg_of(uend - 1, S, P);
        float *slot = a.part + static_cast<size_t>(wl == w1 ? 2 * wl + 1 : 2 * wl) * Lay::kSlotFloats;
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<f32x4_t *>(slot + (16 * t + lr) * D + 16 * dt + 4 * lq) = o[t][dt];
                if (lq == 0) {
                    slot[R * D + 16 * t + lr] = m_tot[t];
                    slot[R * D + R + 16 * t + lr] = l_tot[t];
                }
            }
        }
        __threadfence();
        __syncthreads();
        int32_t *counter = a.counters + (static_cast<size_t>(b) * a.row_groups + rg) * a.hkv + g;
        if (tid == 0) {
            int pieces = 0;
            for (int w = w1; w <= w2; ++w) pieces += (S * w / P) < (S * (w + 1) / P);
            const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            s_flag[0] = old == pieces - 1;
        }
        __syncthreads();
        if (!s_flag[0]) continue;
        __threadfence();
        for (int e = tid; e < R * D; e += kThreads) {
            const int r = e / D, dc = e % D;
            const int row = rg * R + r;
            if (row >= nrows) continue;
            float M = -INFINITY;
            for (int w = w1; w <= w2; ++w) {
                if (!((S * w / P) < (S * (w + 1) / P))) continue;
                const float *ps = a.part + static_cast<size_t>(w == w1 ? 2 * w + 1 : 2 * w) * Lay::kSlotFloats;
                M = fmaxf(M, ps[R * D + r]);
            }
            const float Mu = M == -INFINITY ? 0.f : M;
            float acc = 0.f, lt = 0.f;
            for (int w = w1; w <= w2; ++w) {
                if (!((S * w / P) < (S * (w + 1) / P))) continue;
                const float *ps = a.part + static_cast<size_t>(w == w1 ? 2 * w + 1 : 2 * w) * Lay::kSlotFloats;
                const float f = __builtin_amdgcn_exp2f(ps[R * D + r] - Mu);
                acc += f * ps[r * D + dc];
                lt += f * ps[R * D + R + r];
            }
            const int node = row / G, h = g * G + row % G;
            const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
            const float val = acc / lt;
            if constexpr (F32IN) {
                static_cast<float *>(a.out)[orow * D + dc] = val;
            } else {
                static_cast<uint16_t *>(a.out)[orow * D + dc] = static_cast<uint16_t>(ev::f2bf_bits(val));
            }
            if (a.lse && dc == 0) a.lse[orow] = (M + __log2f(lt)) * kLn2;
        }
        if (tid == 0) *counter = 0;
    }
}

// ---------------------------------------------------------------------------------------------
struct Plan {
    int RT, R, RG;
    size_t slot_floats;
    size_t counters_bytes;
    size_t bytes;
};

Plan make_plan(int32_t batch, int32_t max_nodes, int32_t hq, int32_t hkv, int32_t head_dim) {
    Plan p{};
    const int G = hq / hkv;
    const int rows = max_nodes * G;
    p.RT = rows >= 16 * kMaxRowTiles ? kMaxRowTiles : (rows + 15) / 16;
    p.R = 16 * p.RT;
    p.RG = (rows + p.R - 1) / p.R;
    p.slot_floats = static_cast<size_t>(p.R) * head_dim + 2 * p.R;
    p.counters_bytes = ((static_cast<size_t>(batch) * p.RG * hkv * 4 + 255) / 256) * 256;
    p.bytes = p.counters_bytes + 2 * static_cast<size_t>(kMaxGrid) * p.slot_floats * 4;
    return p;
}

using KernelFn = void (*)(AttnArgs);

template <int D, bool F32IN>
KernelFn pick_rt(int rt) {
    switch (rt) {
        case 1: return tree_attention_kernel<D, 1, F32IN>;
        case 2: return tree_attention_kernel<D, 2, F32IN>;
        case 3: return tree_attention_kernel<D, 3, F32IN>;
        case 4: return tree_attention_kernel<D, 4, F32IN>;
        default: return tree_attention_kernel<D, 5, F32IN>;
    }
}

KernelFn pick_kernel(int head_dim, int rt, bool f32) {
    if (head_dim == 64) return f32 ? pick_rt<64, true>(rt) : pick_rt<64, false>(rt);
    return f32 ? pick_rt<128, true>(rt) : pick_rt<128, false>(rt);
}

// Resident workgroups per CU for a kernel variant, cached per (device, variant).
int blocks_per_cu(KernelFn fn, int variant) {
    static std::mutex mu;
    static int cache[16][32] = {};
    const int dev = ev::current_device();
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 16) return 1;
    int &c = cache[dev][variant];
    if (c == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(fn), kThreads, 0) !=
                hipSuccess || n < 1)
            n = 1;
        c = n;
    }
    return c;
}

}  // namespace

extern "C" size_t ev_tree_attention_workspace_size(int32_t batch, int32_t max_nodes, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim) {
    if (batch < 0 || batch > EV_MAX_BATCH || max_nodes < 1 || max_nodes > EV_MAX_NODES || num_q_heads < 1 ||
        num_kv_heads < 1 || num_q_heads % num_kv_heads || (head_dim != 64 && head_dim != 128))
        return 0;
    return make_plan(batch, max_nodes, num_q_heads, num_kv_heads, head_dim).bytes;
}

extern "C" ev_status ev_tree_attention(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                                       const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                       const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
                                       int32_t max_nodes, int64_t total_slots, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype, float sm_scale,
                                       void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                       hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !out || !node_start || !parent || !kv_start || !prefix_len)
        return EV_ERR_NULL;
    if (batch < 0 || batch > EV_MAX_BATCH || total_nodes < 0 || max_nodes < 1 || max_nodes > EV_MAX_NODES ||
        total_slots < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
        (head_dim != 64 && head_dim != 128) || !std::isfinite(sm_scale))
        return EV_ERR_SHAPE;
    if (dtype != EV_BF16 && dtype != EV_F32) return EV_ERR_DTYPE;
    if (!ev::aligned16(q) || !ev::aligned16(k_cache) || !ev::aligned16(v_cache) || !ev::aligned16(out))
        return EV_ERR_ALIGN;
    const Plan plan = make_plan(batch, max_nodes, num_q_heads, num_kv_heads, head_dim);
    if (!workspace || workspace_bytes < plan.bytes) return EV_ERR_WORKSPACE;
    if (!ev::aligned16(workspace)) return EV_ERR_ALIGN;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (batch == 0 || total_nodes == 0) return EV_OK;

    const bool f32 = dtype == EV_F32;
    KernelFn fn = pick_kernel(head_dim, plan.RT, f32);
    const int variant = (head_dim == 64 ? 0 : 16) + (f32 ? 8 : 0) + plan.RT;
    const int resident = ev::device_cu_count() * blocks_per_cu(fn, variant);
    // Upper bound of the step count: every sequence's keys fit in the cache.
    const int64_t max_steps = static_cast<int64_t>(num_kv_heads) * plan.RG * (total_slots / kStep + 2 * batch);
    int64_t grid = resident;
    if (grid > kMaxGrid) grid = kMaxGrid;
    const int64_t want = (max_steps + kWaves - 1) / kWaves;  // at least a step per wave
    if (grid > want) grid = want;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;

    AttnArgs args;
    args.q = q;
    args.k = k_cache;
    args.v = v_cache;
    args.out = out;
    args.lse = lse;
    args.node_start = node_start;
    args.parent = parent;
    args.kv_start = kv_start;
    args.prefix_len = prefix_len;
    args.total_slots = total_slots;
    args.batch = batch;
    args.total_nodes = total_nodes;
    args.max_nodes = max_nodes;
    args.hq = num_q_heads;
    args.hkv = num_kv_heads;
    args.group = num_q_heads / num_kv_heads;
    args.row_groups = plan.RG;
    args.scale_log2 = sm_scale * kLog2e;
    args.counters = static_cast<int32_t *>(workspace);
    args.part = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + plan.counters_bytes);
    args.err_flag = err_flag;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, args);
    return ev::launch_status();
}
