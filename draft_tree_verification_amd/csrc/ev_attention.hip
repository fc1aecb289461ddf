// ev_attention.hip -- tree-masked GQA verification attention for gfx950 (MI355X).
//
// What it computes: for every draft-tree node i of sequence b and q head h, softmax attention
// over the sequence's KV prefix plus the tree slots of i's ancestors and i itself (the target's
// single parallel verification forward over the whole draft tree: kongchang.com English
// article, "Technical Background"; EAGLE-2's dynamic tree covers several candidate paths in one
// verification).  The KV cache is bf16 and never quantised (arex-research.com release note,
// plugin section: tree verification needs an unquantised KV cache).
//
// How (two launches on one stream: the attention kernel, then the merge of split units):
//   * Work unit = (sequence, row group, KV head).  A unit's rows are all (node, q-head-in-group)
//     pairs of that KV head -- up to 80 rows -- so every K/V byte is read from HBM exactly once
//     and shared by all N*G rows (the arithmetic intensity is N*G flop per byte).
//   * Each unit's keys are cut into stages (64 keys for 80-row units, 32 keys otherwise) and a
//     workgroup takes a range of stages.  When the units fit the grid the split is unit-aligned
//     (each workgroup one near-equal piece of one unit); otherwise all stages are laid end to end
//     and the workgroups take equal contiguous ranges (stream-K), mapped XCD-major so the pieces
//     of one unit mostly land on one XCD.
//   * bf16 inputs stream HBM -> LDS with direct 16-byte loads (global_load_lds_dwordx4), several
//     stages in flight, no register staging.  K and V rows keep their natural layout with the
//     16-byte chunks XOR-swizzled per row: K operand reads are ds_read_b128 and the V^T operand
//     comes from ds_read_b64_tr_b16 transpose reads, both bank-conflict free.  fp32 inputs go
//     through registers (converted to bf16) into a padded K tile and a transposed V tile.
//   * Four waves per workgroup.  In the row-tile kernels wave w owns 16-row tile w; 80-row bf16
//     units run the key-split kernel below, where every wave covers all 80 rows for its own
//     16-key quarter of each stage.  S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 and O^T =
//     V^T P^T on the 16x16x32 or 16x16x16 form; the online softmax is fp32 base-2 with the scale
//     folded into the exponent's FMA; the ancestor mask is applied only on stages that reach the
//     tree slots.  The score layout already matches P^T's operand layout, so P needs no shuffle.
//   * A unit covered by one workgroup is written directly; otherwise each piece publishes its
//     (m, l, O) partial and the unit's first piece records the unit in a table, and the merge
//     launch (whose launch boundary makes the partials visible) combines each unit's pieces in
//     piece order: deterministic, no atomics, no L2 flushes.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "ev_internal.h"
#include "ev_select.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxGrid = 512;      // workgroups per launch (bounds the partial-result slots)
constexpr int kMaxRowTiles = 5;    // 16-row tiles per unit: at most 80 rows
constexpr int kStages = 4;         // LDS stage buffers of the bf16 path: three stages in flight
constexpr float kLog2e = 1.4426950408889634f;
// Cache policy of the K/V global->LDS loads: nt (streaming; every K/V byte is read once).  On
// MI355X this pattern streams at ~6.5 TB/s with it and ~5.8 TB/s with the default policy.
constexpr int kKvLoadPolicy = 2;
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
    int64_t kv_slot_stride, kv_head_stride;  // elements between a K/V cache's slots / KV heads
    int32_t batch, total_nodes, max_nodes, hq, hkv, group, row_groups;
    int32_t window;    // > 0: only the last `window` prefix tokens are visible (sliding window)
    const int32_t *block_table;  // paged caches (else NULL): [batch][bt_stride] pool page of each
                                 // run of 2^page_shift tokens; row = page * 2^page_shift + offset
    int32_t bt_stride, page_shift, num_pages;
    float scale_log2;  // sm_scale * log2(e) > 0: scores live in the base-2 domain
    int4 *table;       // [grid] per logical workgroup: {pieces, first node, nodes, unit index} of the
                       // split unit whose first piece it holds (pieces = 0: none)
    float *part;       // [2 * kMaxGrid] partial-result slots
    int32_t *err_flag;
};

template <int D, int RT, bool F32IN>
struct Layout {
    static constexpr bool X5 = RT == 5;             // four full tiles + one split by keys
    static constexpr int KST = X5 ? 64 : 32;        // keys per stage
    static constexpr int R = RT * 16;
    static constexpr int kScan = EV_MAX_BATCH * 4;  // int32 inclusive scan of per-sequence stages
    static constexpr int kMisc = 32;                // wave sums of the schedule scan
    // fp32 inputs: two register-staged buffers (K row-major padded, V transposed)
    static constexpr int KP = 2 * D + 16;
    static constexpr int VTP = 2 * KST + 8;
    static constexpr int kK = KST * KP;
    static constexpr int kVt = D * VTP;
    // bf16 inputs: kStages buffers filled straight from HBM (K then V, rows XOR-swizzled)
    static constexpr int kRowB = 2 * D;
    static constexpr int kTensorB = KST * kRowB;
    static constexpr int kStageBytes = F32IN ? kK + kVt : 2 * kTensorB;
    static constexpr int kBuffers = F32IN ? 2 : kStages;
    static constexpr int kTotal = kScan + kMisc + kBuffers * kStageBytes;
    static constexpr size_t kSlotFloats = (size_t)R * D + 2 * R;  // O [R][D], then m [R], l [R]
    static_assert(!X5 || 4 * 16 * (D + 4) * 4 + 2 * 64 * 4 <= kBuffers * kStageBytes, "tile-4 merge space");
};

template <int N>
__device__ __forceinline__ void vm_wait_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence (ordering is explicit: counted vmcnt waits before it).
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Byte address of a shared-memory pointer in the LDS aperture.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    typedef const __attribute__((address_space(3))) unsigned char *lds_cptr;
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cptr)p));
}

// All V^T operand reads of one stage: x[dt][j] = ds_read_b64_tr_b16 at addr[dt] + j * 16 rows.
// One asm block that waits for its own reads before it ends, so every output register holds its
// value when the block is left.  Issued through the builtin instead, these reads get a
// conservative wait for all outstanding global-to-LDS loads in front of them (the compiler
// cannot tell that they touch another stage buffer), which would drain the stage pipeline.
// Outputs are early-clobber: a read may land while later reads still need their address.
#define EV_TR(o, a, off) "ds_read_b64_tr_b16 %" #o ", %" #a " offset:" #off "\n\t"
#define EV_O(i) "=&v"(x[(i) / NJ][(i) % NJ])
template <int D, int KC> struct TrRead;
template <> struct TrRead<128, 2> {  // 16-row step 4096 bytes, 4 reads per d tile
    static constexpr int NJ = 4;
    __device__ static __forceinline__ void run(u32x2_t (&x)[8][4], const uint32_t (&a)[8]) {
        asm volatile(EV_TR(0, 32, 0) EV_TR(1, 32, 4096) EV_TR(2, 32, 8192) EV_TR(3, 32, 12288)
                     EV_TR(4, 33, 0) EV_TR(5, 33, 4096) EV_TR(6, 33, 8192) EV_TR(7, 33, 12288)
                     EV_TR(8, 34, 0) EV_TR(9, 34, 4096) EV_TR(10, 34, 8192) EV_TR(11, 34, 12288)
                     EV_TR(12, 35, 0) EV_TR(13, 35, 4096) EV_TR(14, 35, 8192) EV_TR(15, 35, 12288)
                     EV_TR(16, 36, 0) EV_TR(17, 36, 4096) EV_TR(18, 36, 8192) EV_TR(19, 36, 12288)
                     EV_TR(20, 37, 0) EV_TR(21, 37, 4096) EV_TR(22, 37, 8192) EV_TR(23, 37, 12288)
                     EV_TR(24, 38, 0) EV_TR(25, 38, 4096) EV_TR(26, 38, 8192) EV_TR(27, 38, 12288)
                     EV_TR(28, 39, 0) EV_TR(29, 39, 4096) EV_TR(30, 39, 8192) EV_TR(31, 39, 12288)
                     "s_waitcnt lgkmcnt(0)"
                     : EV_O(0), EV_O(1), EV_O(2), EV_O(3), EV_O(4), EV_O(5), EV_O(6), EV_O(7), EV_O(8),
                       EV_O(9), EV_O(10), EV_O(11), EV_O(12), EV_O(13), EV_O(14), EV_O(15), EV_O(16),
                       EV_O(17), EV_O(18), EV_O(19), EV_O(20), EV_O(21), EV_O(22), EV_O(23), EV_O(24),
                       EV_O(25), EV_O(26), EV_O(27), EV_O(28), EV_O(29), EV_O(30), EV_O(31)
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                     : "memory");
    }
};
template <> struct TrRead<128, 1> {  // 2 reads per d tile
    static constexpr int NJ = 2;
    __device__ static __forceinline__ void run(u32x2_t (&x)[8][2], const uint32_t (&a)[8]) {
        asm volatile(EV_TR(0, 16, 0) EV_TR(1, 16, 4096) EV_TR(2, 17, 0) EV_TR(3, 17, 4096)
                     EV_TR(4, 18, 0) EV_TR(5, 18, 4096) EV_TR(6, 19, 0) EV_TR(7, 19, 4096)
                     EV_TR(8, 20, 0) EV_TR(9, 20, 4096) EV_TR(10, 21, 0) EV_TR(11, 21, 4096)
                     EV_TR(12, 22, 0) EV_TR(13, 22, 4096) EV_TR(14, 23, 0) EV_TR(15, 23, 4096)
                     "s_waitcnt lgkmcnt(0)"
                     : EV_O(0), EV_O(1), EV_O(2), EV_O(3), EV_O(4), EV_O(5), EV_O(6), EV_O(7), EV_O(8),
                       EV_O(9), EV_O(10), EV_O(11), EV_O(12), EV_O(13), EV_O(14), EV_O(15)
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                     : "memory");
    }
};
template <> struct TrRead<64, 2> {  // 16-row step 2048 bytes
    static constexpr int NJ = 4;
    __device__ static __forceinline__ void run(u32x2_t (&x)[4][4], const uint32_t (&a)[4]) {
        asm volatile(EV_TR(0, 16, 0) EV_TR(1, 16, 2048) EV_TR(2, 16, 4096) EV_TR(3, 16, 6144)
                     EV_TR(4, 17, 0) EV_TR(5, 17, 2048) EV_TR(6, 17, 4096) EV_TR(7, 17, 6144)
                     EV_TR(8, 18, 0) EV_TR(9, 18, 2048) EV_TR(10, 18, 4096) EV_TR(11, 18, 6144)
                     EV_TR(12, 19, 0) EV_TR(13, 19, 2048) EV_TR(14, 19, 4096) EV_TR(15, 19, 6144)
                     "s_waitcnt lgkmcnt(0)"
                     : EV_O(0), EV_O(1), EV_O(2), EV_O(3), EV_O(4), EV_O(5), EV_O(6), EV_O(7), EV_O(8),
                       EV_O(9), EV_O(10), EV_O(11), EV_O(12), EV_O(13), EV_O(14), EV_O(15)
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};
template <> struct TrRead<64, 1> {
    static constexpr int NJ = 2;
    __device__ static __forceinline__ void run(u32x2_t (&x)[4][2], const uint32_t (&a)[4]) {
        asm volatile(EV_TR(0, 8, 0) EV_TR(1, 8, 2048) EV_TR(2, 9, 0) EV_TR(3, 9, 2048)
                     EV_TR(4, 10, 0) EV_TR(5, 10, 2048) EV_TR(6, 11, 0) EV_TR(7, 11, 2048)
                     "s_waitcnt lgkmcnt(0)"
                     : EV_O(0), EV_O(1), EV_O(2), EV_O(3), EV_O(4), EV_O(5), EV_O(6), EV_O(7)
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};
#undef EV_O
#undef EV_TR
typedef __attribute__((address_space(3))) void lds_void_t;

// Workgroup (logical index) whose stage range contains stage x: the largest w with
// floor(w*S/P) <= x.
__device__ __forceinline__ int wg_of(int64_t x, int64_t S, int P) {
    return static_cast<int>(((x + 1) * P - 1) / S);
}

// The visible prefix of sequence b: its last `window` tokens when a window is set (the
// drafter's sliding window over its append-only cache), else all of it.  L is the visible
// length and s0 the position of its first token: a cache slot (contiguous caches; the tree
// slots follow at s0 + L) or a token index within the sequence (paged caches).
template <bool PG>
__device__ __forceinline__ void visible_prefix(const AttnArgs &a, int b, int &L, int64_t &s0) {
    const int Lf = a.prefix_len[b];
    L = (a.window > 0 && Lf > a.window) ? a.window : Lf;
    s0 = (PG ? 0 : static_cast<int64_t>(a.kv_start[b])) + (Lf - L);
}

using const_i32_t = const __attribute__((address_space(4))) int32_t;

// Paged caches: the first pool row of the page that holds token `tok` of the block-table row
// `bt` (uniform arguments: one scalar load).  A page outside the pool raises EV_DATA_BAD_SLOTS
// and page 0 is read instead, so no load leaves the pool.
__device__ __forceinline__ int64_t page_row(const AttnArgs &a, const int32_t *bt, int tok) {
    int pg = ((const_i32_t *)bt)[tok >> a.page_shift];
    if (static_cast<unsigned>(pg) >= static_cast<unsigned>(a.num_pages)) {
        ev::flag_error(a.err_flag, EV_DATA_BAD_SLOTS);
        pg = 0;
    }
    return static_cast<int64_t>(pg) << a.page_shift;
}

// Partial-result slot of piece `piece` of the split unit whose first piece is held by logical
// workgroup w1: a workgroup holds at most two split pieces, the last piece of a unit begun
// earlier (slot 2w) and the first piece of a unit that continues past it (slot 2w + 1).
__device__ __forceinline__ float *slot_of_piece(float *part, int w1, int piece, int slot_floats) {
    const int w = w1 + piece;
    return part + static_cast<size_t>(piece == 0 ? 2 * w + 1 : 2 * w) * slot_floats;
}

// Batches of at most kAlignedMaxBatch sequences also keep each sequence's stages per unit and
// unit count in s_cum[kSeqStages + b] and s_cum[kSeqUnits + b] (for the unit-aligned split).
constexpr int kAlignedMaxBatch = 64;
constexpr int kSeqStages = EV_MAX_BATCH / 2;
constexpr int kSeqUnits = EV_MAX_BATCH / 2 + kAlignedMaxBatch;

// Per-sequence stage counts of the whole batch and their inclusive scan into s_cum (identical
// in every workgroup); returns the total stage count.  Sequences with bad geometry get no stages
// and raise their error bit once.  The scan runs in 64 bits: a batch whose total reaches 2^31
// stages (only possible when sequences share slot ranges, which the host's bound from
// total_slots does not see) raises EV_DATA_BAD_SLOTS and gets no stages at all, so the 32-bit
// prefix sums in s_cum never wrap.
template <int R, int KST>
__device__ __forceinline__ int64_t schedule_scan(const AttnArgs &a, int32_t *s_cum, int64_t *s_misc) {
    constexpr int NT = kThreads;
    constexpr int NW = kWaves;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = a.group;
    int64_t carry = 0;
    for (int b0 = 0; b0 < a.batch; b0 += NT) {
        const int b = b0 + tid;
        int64_t work = 0;
        if (b < a.batch) {
            const int ns0 = a.node_start[b], ns1 = a.node_start[b + 1];
            const int n = ns1 - ns0;
            const int L = a.prefix_len[b], s0 = a.block_table ? 0 : a.kv_start[b];
            int err = 0;
            if (ns0 < 0 || ns1 > a.total_nodes || n < 1 || n > a.max_nodes)
                err = EV_DATA_BAD_NODES;
            else if (a.block_table ? (L < 0 || ((static_cast<int64_t>(L) + n - 1) >> a.page_shift) >= a.bt_stride)
                                   : (L < 0 || s0 < 0 || static_cast<int64_t>(s0) + L + n > a.total_slots))
                err = EV_DATA_BAD_SLOTS;
            int st = 0, units = 0;
            if (err) {
                if (blockIdx.x == 0) ev::flag_error(a.err_flag, err);
            } else {
                const int Lv = (a.window > 0 && L > a.window) ? a.window : L;
                st = static_cast<int>((static_cast<int64_t>(Lv) + n + KST - 1) / KST);
                units = a.hkv * ((n * G + R - 1) / R);
                work = static_cast<int64_t>(units) * st;
            }
            if (a.batch <= kAlignedMaxBatch) {
                s_cum[kSeqStages + b] = st;
                s_cum[kSeqUnits + b] = units;
            }
        }
        int64_t x = work;
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_misc[wave] = x;
        __syncthreads();
        int64_t wbase = 0, tot = 0;
        for (int w = 0; w < NW; ++w) {
            if (w < wave) wbase += s_misc[w];
            tot += s_misc[w];
        }
        if (b < a.batch) s_cum[b] = static_cast<int32_t>(min(carry + wbase + x, static_cast<int64_t>(INT32_MAX)));
        carry += tot;
        __syncthreads();
    }
    if (carry > INT32_MAX) {
        if (blockIdx.x == 0 && tid == 0) ev::flag_error(a.err_flag, EV_DATA_BAD_SLOTS);
        return 0;
    }
    return carry;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive prefix over each 16-lane row with DPP row shifts (lanes shifted in from outside the
// row read 0), then across the four rows through their last lanes; `total` = the wave's sum.
// All values non-negative, so the same steps give a row-wise running maximum with op = max.
template <bool MAX>
__device__ __forceinline__ int wave_scan(int x, int &total) {
    auto op = [](int u, int v) { return MAX ? max(u, v) : u + v; };
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
    const int row = (threadIdx.x & 63) >> 4;
    if (row > 0) x = op(x, r0);
    if (row > 1) x = op(x, r1);
    if (row > 2) x = op(x, r2);
    total = op(op(r0, r1), op(r2, r3));
    return x;
}
__device__ __forceinline__ int wave_sum(int x) {
    int t;
    wave_scan<false>(x, t);
    return t;
}

// The stage range of one logical workgroup.
struct PieceMap {
    int64_t begin, end;  // its stages in the batch's stage order
    int P;               // logical workgroups with work
    int k;               // unit-aligned split: pieces of this workgroup's unit (0: contiguous split)
    int w1;              // unit-aligned split: logical workgroup of the unit's first piece
};

// Two ways to cut the batch's stages into per-workgroup ranges.
//  * Unit-aligned (at most `grid` units, at most kAlignedMaxBatch sequences): unit u gets
//    k_u = ceil(stages_u / C) pieces of near-equal length, C the smallest cap whose pieces fit the
//    grid; each workgroup holds exactly one piece of one unit, so none restarts its load pipeline
//    on a second unit, and the workgroups in use spread over all XCDs (logical = hardware index).
//  * Contiguous (otherwise): equal ranges of the whole stage order; a range may cover the end of
//    one unit and the start of the next (XCD-major logical order).
// Every wave computes the map itself (lane = sequence), from the per-sequence counts in LDS.
__device__ __forceinline__ PieceMap map_pieces(const AttnArgs &a, const int32_t *s_cum, int64_t S, int grid,
                                               int &wl) {
    PieceMap m{};
    m.k = -1;
    const int lane = threadIdx.x & 63;
    if (S > 0 && a.batch <= kAlignedMaxBatch) {
        const int st = lane < a.batch ? s_cum[kSeqStages + lane] : 0;
        const int units = lane < a.batch ? s_cum[kSeqUnits + lane] : 0;
        const int utot = wave_sum(units);
        if (utot > 0 && utot <= grid) {
            // C >= S / grid; C = max st_b fits (one piece per unit), and so does any C with
            // S / C + utot <= grid (each unit rounds up by less than one piece)
            int hi;
            wave_scan<true>(st, hi);
            int lo = static_cast<int>((S + grid - 1) / grid);
            if (utot < grid) hi = min(hi, static_cast<int>((S + grid - utot - 1) / (grid - utot)));
            lo = max(1, min(lo, hi));
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (wave_sum(units * ((st + mid - 1) / mid)) <= grid) hi = mid; else lo = mid + 1;
            }
            const int k = (st + lo - 1) / lo;
            const int wk = units * k;
            int P;
            const int W = wave_scan<false>(wk, P) - wk;  // exclusive prefix
            const int wb = blockIdx.x;
            if (wb >= P) {
                m.k = 0;
                m.P = P;
                wl = wb;
            } else {
                const uint64_t hit = __ballot(wk > 0 && W <= wb);
                const int bs = hit ? 63 - __builtin_clzll(hit) : 0;
                const int Wb = __builtin_amdgcn_readlane(W, bs), kb = __builtin_amdgcn_readlane(k, bs);
                const int stb = __builtin_amdgcn_readlane(st, bs);
                const int r = wb - Wb;
                if (hit && kb > 0 && r >= 0) {
                    const int ui = r / kb, j = r % kb;
                    const int64_t ustart = (bs ? s_cum[bs - 1] : 0) + static_cast<int64_t>(ui) * stb;
                    m.begin = ustart + static_cast<int64_t>(stb) * j / kb;
                    m.end = ustart + static_cast<int64_t>(stb) * (j + 1) / kb;
                    m.k = kb;
                    m.w1 = Wb + ui * kb;
                    m.P = P;
                    wl = wb;
                    // a map that fails these checks falls back to the contiguous split
                    if (!(P <= grid && m.begin >= 0 && m.begin < m.end && m.end <= S)) m.k = -1;
                }
            }
        }
    }
    if (m.k < 0) {
        m.k = 0;
        wl = (grid % 8 == 0) ? (blockIdx.x % 8) * (grid / 8) + blockIdx.x / 8 : blockIdx.x;
        m.P = static_cast<int>(S < grid ? S : grid);  // never more than stages: every range non-empty
        m.begin = m.P ? S * wl / m.P : 0;              // (no stages: no workgroup has work)
        m.end = m.P ? S * (wl + 1) / m.P : 0;
    }
    // uniform values: scalar registers and scalar branches in the piece loop
    m.begin = uniform64(m.begin);
    m.end = uniform64(m.end);
    m.P = __builtin_amdgcn_readfirstlane(m.P);
    m.k = __builtin_amdgcn_readfirstlane(m.k);
    m.w1 = __builtin_amdgcn_readfirstlane(m.w1);
    wl = __builtin_amdgcn_readfirstlane(wl);
    return m;
}

template <int D, int RT, bool F32IN, bool PG>
__device__ __forceinline__ void attention_body(const AttnArgs &a) {
    static_assert(!(PG && F32IN), "paged caches hold bf16");
    using Lay = Layout<D, RT, F32IN>;
    constexpr bool X5 = Lay::X5;
    constexpr int KST = Lay::KST;
    constexpr int U = KST / 16;                // 16-key sub-tiles per stage
    constexpr int KC = KST / 32;               // 32-key halves per stage (PV MFMA extent)
    constexpr int NW = kWaves;
    constexpr int NT = kThreads;
    constexpr int R = Lay::R;
    constexpr int KS = D / 32;                 // k-steps of the QK^T contraction
    constexpr int DT = D / 16;                 // 16-wide d tiles of O^T
    constexpr int CPR = D / 8;                 // 8-element chunks per K/V row
    constexpr int NTL = X5 ? 2 : 1;            // register tiles per wave: own tile (+ tile 4's quarter)

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kTotal];
    int32_t *s_cum = reinterpret_cast<int32_t *>(smem);
    int64_t *s_misc = reinterpret_cast<int64_t *>(smem + Lay::kScan);
    unsigned char *stage_buf = smem + Lay::kScan + Lay::kMisc;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The wave index must be visibly uniform: every wave-dependent choice below (which tiles a
    // wave owns, which key quarter it takes) then compiles to a scalar branch.  Under an
    // EXEC-masked branch the compiler may drop the skip jump around a short block, and an MFMA
    // in such a block still writes its accumulator when no lane is active.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15;
    const int lq = lane >> 4;
    const int G = a.group;
    const float c2 = a.scale_log2;

    const int64_t S = schedule_scan<R, KST>(a, s_cum, s_misc);
    const int grid = gridDim.x;
    int wl;
    const PieceMap pm = map_pieces(a, s_cum, S, grid, wl);
    const int P = pm.P;
    if (tid == 0) a.table[wl] = int4{0, 0, 0, 0};  // no split unit starts here (until one does)
    if (wl >= P) return;
    const int64_t begin = pm.begin, end = pm.end;

    for (int64_t pos = begin; pos < end;) {
        // ---- locate the unit that holds stage `pos`
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] > pos) hi = mid; else lo = mid + 1;
        }
        const int b = lo;
        const int64_t seq_base = b ? s_cum[b - 1] : 0;
        const int ns0 = a.node_start[b];
        const int n = a.node_start[b + 1] - ns0;
        int L;
        int64_t s0;
        visible_prefix<PG>(a, b, L, s0);
        const int stages = (L + n + KST - 1) / KST;
        const int ui = static_cast<int>((pos - seq_base) / stages);
        const int rg = ui / a.hkv, g = ui % a.hkv;
        const int64_t ustart = seq_base + static_cast<int64_t>(ui) * stages, uend = ustart + stages;
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

        // ---- this wave's tiles (slot 0: tile `wave`; slot 1: tile 4 when X5): Q^T operands in
        // registers, ancestor masks, softmax state
        const bool have_main = wave < RT;
        uint64_t rmask[NTL];
        bf16x8_t qop[NTL][KS];
        f32x4_t o[NTL][DT];
        float m_run[NTL], l_run[NTL];
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            const int t = tt == 0 ? wave : 4;
            const int row = rg * R + 16 * t + lr;
            const bool live = t < RT && row < nrows;
            const int node = live ? row / G : 0;
            const uint32_t mlo = __shfl(static_cast<uint32_t>(anc), node, 64);
            const uint32_t mhi = __shfl(static_cast<uint32_t>(anc >> 32), node, 64);
            rmask[tt] = live ? ((static_cast<uint64_t>(mhi) << 32) | mlo) : 0ull;
            const int h = g * G + (live ? row % G : 0);
            const size_t qoff = (static_cast<size_t>(ns0 + node) * a.hq + h) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4_t val = {0u, 0u, 0u, 0u};
                if (live) {
                    if constexpr (F32IN) {
                        const float *qp = static_cast<const float *>(a.q) + qoff + 32 * s + 8 * lq;
                        val = ev::f32x8_to_bf16x8(ev::ld16f(qp), ev::ld16f(qp + 4));
                    } else {
                        val = ev::ld16(static_cast<const uint16_t *>(a.q) + qoff + 32 * s + 8 * lq);
                    }
                }
                qop[tt][s] = __builtin_bit_cast(bf16x8_t, val);
            }
            m_run[tt] = -INFINITY;
            l_run[tt] = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[tt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        const int kv_end = L + n;  // unit-relative key positions below this exist
        const size_t slot_stride = static_cast<size_t>(a.kv_slot_stride);  // elements between slots
        // paged caches: rows are found per load through the block table, s0 is a token index
        const size_t head_off = (PG ? 0 : static_cast<size_t>(s0) * slot_stride) + static_cast<size_t>(g) * a.kv_head_stride;
        const int32_t *bt = nullptr;
        if constexpr (PG) bt = a.block_table + static_cast<size_t>(__builtin_amdgcn_readfirstlane(b)) * a.bt_stride;

        // Online-softmax update of tile slot tt from raw scores (masked entries are -inf): the
        // running max moves to the stage's max (scaled), the exponent folds the scale into one
        // FMA, the state rescales only when some row's max moved.  emit(p_of) lets the caller pack
        // the probabilities where it needs them.
        auto softmax_update = [&](int tt, float mx_raw, auto &&emit) {
            mx_raw = fmaxf(mx_raw, __shfl_xor(mx_raw, 16, 64));
            mx_raw = fmaxf(mx_raw, __shfl_xor(mx_raw, 32, 64));
            const float m_new = fmaxf(m_run[tt], mx_raw * c2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[tt] - m_use);
            float psum = 0.f;
            emit([&](float s) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c2, -m_use));
                psum += p;
                return p;
            });
            l_run[tt] = l_run[tt] * alpha + psum;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[tt][dt] *= alpha;
            }
            m_run[tt] = m_new;
        };
        auto mask_scores = [&](int tt, int kb, int key0, f32x4_t &sc) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = kb + key0 + 4 * lq + r;
                const bool vis = p < L || (p < kv_end && ((rmask[tt] >> (p - L)) & 1ull));
                if (!vis) sc[r] = -INFINITY;
            }
        };

        // One stage of this wave's tiles, given the K operand reader and the V^T operand filler.
        // vop[kc][dt] holds the operand for keys (32kc + 4*lq + 0..3, then 32kc + 16 + 4*lq + 0..3).
        auto compute_stage = [&](int kb, auto kop_at, auto vload) {
            if constexpr (!X5) {
                if (!have_main) return;  // a wave without a tile of this unit
            }
            // every operand read of the stage is issued before the first MFMA needs one: the V^T
            // reads complete under the QK^T MFMAs and the softmax
            bf16x8_t kop[U][KS];
            u32x4_t vop[KC][DT];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int s = 0; s < KS; ++s) kop[u][s] = kop_at(u, s);
            vload(vop);
            // S^T = K Q^T : sc[u] holds raw scores of keys 16u + 4*lq + r for row 16t + lr
            f32x4_t sc[U], scx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                if (have_main) {
#pragma unroll
                    for (int s = 0; s < KS; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u][s], qop[0][s], acc, 0, 0, 0);
                }
                sc[u] = acc;
                if constexpr (X5) {
                    if (u == wave) {
#pragma unroll
                        for (int s = 0; s < KS; ++s)
                            scx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u][s], qop[1][s], scx, 0, 0, 0);
                    }
                }
            }
            const bool edge = kb + KST > L;  // the stage reaches the tree slots or the unit's end
            u32x4_t pw[KC];
            uint32_t pwx[2] = {0u, 0u};
            if (have_main) {
                if (edge) {
#pragma unroll
                    for (int u = 0; u < U; ++u) mask_scores(0, kb, 16 * u, sc[u]);
                }
                float mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    mx = fmaxf(mx, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
                softmax_update(0, mx, [&](auto &&p_of) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
                            pw[u >> 1][2 * (u & 1) + h2] =
                                ev::pack_bf16x2(p_of(sc[u][2 * h2]), p_of(sc[u][2 * h2 + 1]));
                    }
                });
            }
            if constexpr (X5) {
                if (edge) mask_scores(1, kb, 16 * wave, scx);
                const float mx = fmaxf(fmaxf(scx[0], scx[1]), fmaxf(scx[2], scx[3]));
                softmax_update(1, mx, [&](auto &&p_of) {
                    pwx[0] = ev::pack_bf16x2(p_of(scx[0]), p_of(scx[1]));
                    pwx[1] = ev::pack_bf16x2(p_of(scx[2]), p_of(scx[3]));
                });
            }
            // O^T += V^T P^T per 32-key half (the quarter tile uses the matching 16-key half of
            // the same V^T operand with a 16x16x16 MFMA)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw[kc]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x4_t vv = vop[kc][dt];
                    if (have_main)
                        o[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pop,
                                                                           o[0][dt], 0, 0, 0);
                    if constexpr (X5) {
                        if (kc == (wave >> 1)) {
                            const u32x2_t half = (wave & 1) ? u32x2_t{vv[2], vv[3]} : u32x2_t{vv[0], vv[1]};
                            o[1][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                __builtin_bit_cast(v4i16_t, half), __builtin_bit_cast(v4i16_t, u32x2_t{pwx[0], pwx[1]}),
                                o[1][dt], 0, 0, 0);
                        }
                    }
                }
            }
        };

        if constexpr (F32IN) {
            // fp32 inputs: global -> registers (one stage ahead) -> bf16 in LDS
            constexpr int KP = Lay::KP;
            constexpr int VTP = Lay::VTP;
            constexpr int KLD = (KST * CPR + NT - 1) / NT;        // K chunks per thread per stage
            constexpr int VLD = (KST / 4 * CPR + NT - 1) / NT;    // V key-quads per thread
            u32x4_t kreg[KLD][2], vreg[VLD][4][2];
            auto load_stage = [&](int st) {
                const int kb = st * KST;
#pragma unroll
                for (int i = 0; i < KLD; ++i) {
                    const int id = tid + NT * i;
                    const int key = id / CPR, c = id % CPR;
                    const int p = kb + key;
                    const bool ok_ld = id < KST * CPR && p < kv_end;
                    const float *src = static_cast<const float *>(a.k) + head_off +
                                       static_cast<size_t>(ok_ld ? p : 0) * slot_stride + 8 * c;
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        kreg[i][e] = ok_ld ? __builtin_bit_cast(u32x4_t, ev::ld16f_stream(src + 4 * e))
                                           : u32x4_t{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < VLD; ++i) {
                    const int id = tid + NT * i;
                    const int c = id % CPR, kq = 4 * (id / CPR);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int p = kb + kq + jj;
                        const bool ok_ld = id < KST / 4 * CPR && p < kv_end;
                        const float *src = static_cast<const float *>(a.v) + head_off +
                                           static_cast<size_t>(ok_ld ? p : 0) * slot_stride + 8 * c;
#pragma unroll
                        for (int e = 0; e < 2; ++e)
                            vreg[i][jj][e] = ok_ld ? __builtin_bit_cast(u32x4_t, ev::ld16f_stream(src + 4 * e))
                                                   : u32x4_t{0u, 0u, 0u, 0u};
                    }
                }
            };
            auto to_bf16 = [&](const u32x4_t (&x)[2]) -> u32x4_t {
                return ev::f32x8_to_bf16x8(__builtin_bit_cast(f32x4_t, x[0]), __builtin_bit_cast(f32x4_t, x[1]));
            };
            auto store_stage = [&](unsigned char *buf) {
#pragma unroll
                for (int i = 0; i < KLD; ++i) {
                    const int id = tid + NT * i;
                    if (id < KST * CPR) {
                        const int key = id / CPR, c = id % CPR;
                        *reinterpret_cast<u32x4_t *>(buf + key * KP + 16 * c) = to_bf16(kreg[i]);
                    }
                }
                unsigned char *vt = buf + Lay::kK;
#pragma unroll
                for (int i = 0; i < VLD; ++i) {
                    const int id = tid + NT * i;
                    if (id < KST / 4 * CPR) {
                        const int c = id % CPR, kq = 4 * (id / CPR);
                        const u32x4_t v0 = to_bf16(vreg[i][0]), v1 = to_bf16(vreg[i][1]);
                        const u32x4_t v2 = to_bf16(vreg[i][2]), v3 = to_bf16(vreg[i][3]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                            const uint32_t w0 = __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], sel);
                            const uint32_t w1 = __builtin_amdgcn_perm(v3[e >> 1], v2[e >> 1], sel);
                            *reinterpret_cast<u32x2_t *>(vt + (8 * c + e) * VTP + 2 * kq) = u32x2_t{w0, w1};
                        }
                    }
                }
            };
            __syncthreads();  // the previous piece is done with both stage buffers
            load_stage(st0);
            store_stage(stage_buf);
            __syncthreads();
            for (int st = st0; st < st1; ++st) {
                unsigned char *cur = stage_buf + ((st - st0) & 1) * Lay::kStageBytes;
                unsigned char *nxt = stage_buf + ((st - st0 + 1) & 1) * Lay::kStageBytes;
                const bool more = st + 1 < st1;
                if (more) load_stage(st + 1);
                const unsigned char *vt = cur + Lay::kK;
                compute_stage(
                    st * KST,
                    [&](int u, int s) {
                        return *reinterpret_cast<const bf16x8_t *>(cur + (16 * u + lr) * KP + 2 * (32 * s + 8 * lq));
                    },
                    [&](u32x4_t (&vop)[KC][DT]) {
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                            for (int dt = 0; dt < DT; ++dt) {
                                const unsigned char *vrow = vt + (16 * dt + lr) * VTP + 2 * (32 * kc + 4 * lq);
                                const u32x2_t v0 = *reinterpret_cast<const u32x2_t *>(vrow);
                                const u32x2_t v1 = *reinterpret_cast<const u32x2_t *>(vrow + 32);
                                vop[kc][dt] = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
                            }
                    });
                if (more) store_stage(nxt);
                __syncthreads();
            }
        } else {
            // bf16 inputs: HBM -> LDS with direct 16-byte loads, kStages - 1 stages in flight and
            // no register staging.  K and V rows keep their natural layout; within a row the
            // 16-byte chunks are XOR-swizzled per row so both the K operand reads (16 rows, one
            // chunk each) and the V transpose reads (8 rows, two chunks each, per half-wave)
            // spread over all LDS banks.
            constexpr int ROWB = Lay::kRowB;
            constexpr int TB = Lay::kTensorB;
            constexpr int RPI = 1024 / ROWB;                    // rows per 1-KB wave load
            constexpr int INSTR = 2 * TB / 1024;                // wave loads per stage (K and V)
            constexpr int PERL = INSTR / NW;                    // loads per wave per stage
            constexpr int SWZ = 16 / CPR;                       // rows per 256-byte bank cycle
            static_assert(INSTR % (2 * NW) == 0, "loader split");
            static_assert(PERL * (kStages - 2) < 64, "vmcnt range");
            const uint16_t *kbase = static_cast<const uint16_t *>(a.k) + head_off;
            const uint16_t *vbase = static_cast<const uint16_t *>(a.v) + head_off;
            auto fk = [](int r) { return (r / SWZ) & (CPR - 1); };
            auto fv = [](int r) { return 2 * ((r / SWZ) & (CPR / 2 - 1)); };
            auto issue = [&](int st, int bi) {
                unsigned char *buf = stage_buf + bi * Lay::kStageBytes;
#pragma unroll
                for (int i = 0; i < PERL; ++i) {
                    const int ins = wave * PERL + i;
                    const bool isv = ins >= INSTR / 2;            // uniform per wave
                    const int local = isv ? ins - INSTR / 2 : ins;
                    const int row = local * RPI + lane / CPR;
                    const int p = lane % CPR;
                    const int kp = st * KST + row;
                    const int c = p ^ (isv ? fv(row) : fk(row));
                    const uint16_t *src;
                    if constexpr (PG) {
                        // this load's RPI rows span at most two pages (pages hold >= 16 tokens);
                        // rows past the unit read its last row
                        const int kl = kv_end - 1, kf = st * KST + local * RPI;
                        const int t0 = static_cast<int>(s0) + min(kf, kl);
                        const int t1 = static_cast<int>(s0) + min(kf + RPI - 1, kl);
                        const int64_t r0 = page_row(a, bt, __builtin_amdgcn_readfirstlane(t0));
                        const int64_t r1 = page_row(a, bt, __builtin_amdgcn_readfirstlane(t1));
                        const int t = static_cast<int>(s0) + min(kp, kl);
                        const int64_t r = ((t >> a.page_shift) == (t0 >> a.page_shift) ? r0 : r1) +
                                          (t & ((1 << a.page_shift) - 1));
                        src = (isv ? vbase : kbase) + static_cast<size_t>(r) * slot_stride + 8 * c;
                    } else {
                        const int kpc = kp < kv_end ? kp : 0;      // rows past the unit: any finite row
                        src = (isv ? vbase : kbase) + static_cast<size_t>(kpc) * slot_stride + 8 * c;
                    }
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf + (isv ? TB : 0) + local * 1024), 16, 0, kKvLoadPolicy);
                }
            };
            __syncthreads();  // the previous piece is done with the stage buffers
            const int nst = st1 - st0;
            for (int i = 0; i < kStages - 1 && i < nst; ++i) issue(st0 + i, i);
            for (int i = 0; i < nst; ++i) {
                const int later = min(kStages - 2, nst - 1 - i);   // stages issued after this one
                if (later >= 2) vm_wait_n<2 * PERL>();
                else if (later == 1) vm_wait_n<PERL>();
                else vm_wait_n<0>();
                // Stage i is in LDS and every wave is done with stage i - 1.  A bare barrier: the
                // fence of __syncthreads would drain the loads still in flight for later stages.
                bare_barrier();
                if (i + kStages - 1 < nst) issue(st0 + i + kStages - 1, (i + kStages - 1) % kStages);
                const unsigned char *cur = stage_buf + (i % kStages) * Lay::kStageBytes;
                compute_stage(
                    (st0 + i) * KST,
                    [&](int u, int s) {
                        const int row = 16 * u + lr;
                        return *reinterpret_cast<const bf16x8_t *>(cur + row * ROWB + 16 * ((4 * s + lq) ^ fk(row)));
                    },
                    [&](u32x4_t (&vop)[KC][DT]) {
                        // Lane address of d tile dt for keys 4*lq + lr/4 (+16, +32, +48: the same
                        // swizzle, so those are immediate offsets).  The swizzle term is even, so
                        // (2dt + b) ^ fv = 2 (dt ^ fv/2) + b.
                        const int r0 = 4 * lq + (lr >> 2);
                        const uint32_t row_addr = lds_addr(cur + TB) + r0 * ROWB + 16 * ((lr & 3) >> 1) + 8 * (lr & 1);
                        uint32_t addr[DT];
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) addr[dt] = row_addr + 32 * (dt ^ (fv(r0) >> 1));
                        u32x2_t x[DT][2 * KC];
                        TrRead<D, KC>::run(x, addr);
#pragma unroll
                        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                            for (int dt = 0; dt < DT; ++dt)
                                vop[kc][dt] = u32x4_t{x[dt][2 * kc][0], x[dt][2 * kc][1], x[dt][2 * kc + 1][0],
                                                      x[dt][2 * kc + 1][1]};
                    });
            }
            __syncthreads();  // every wave is done with the stage buffers
        }

        // ---- per-row sums over the four lanes that share a row
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            l_run[tt] += __shfl_xor(l_run[tt], 16, 64);
            l_run[tt] += __shfl_xor(l_run[tt], 32, 64);
        }

        // ---- tile 4: merge the four key-quarter states into wave 0 (fixed order)
        if constexpr (X5) {
            float *xo = reinterpret_cast<float *>(stage_buf);   // [4][16][D + 4]
            float *xm = xo + 4 * 16 * (D + 4);                  // [4][16]
            float *xl = xm + 64;                                // [4][16]
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4_t *>(xo + (wave * 16 + lr) * (D + 4) + 16 * dt + 4 * lq) = o[1][dt];
            if (lq == 0) {
                xm[wave * 16 + lr] = m_run[1];
                xl[wave * 16 + lr] = l_run[1];
            }
            __syncthreads();
            if (wave == 0) {
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, xm[w * 16 + lr]);
                const float Mu = M == -INFINITY ? 0.f : M;
                float lt = 0.f;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[1][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float f = __builtin_amdgcn_exp2f(xm[w * 16 + lr] - Mu);
                    lt += f * xl[w * 16 + lr];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        o[1][dt] += f * *reinterpret_cast<const f32x4_t *>(xo + (w * 16 + lr) * (D + 4) + 16 * dt + 4 * lq);
                }
                m_run[1] = M;
                l_run[1] = lt;
            }
            __syncthreads();
        }
        // tiles this wave finally holds: slot 0 (tile `wave`), slot 1 (tile 4, wave 0 only)
        auto tile_of = [&](int tt) { return tt == 0 ? (have_main ? wave : -1) : (wave == 0 ? 4 : -1); };

        // ---- output
        const bool whole = ustart >= begin && uend <= end;
        if (whole) {
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int t = tile_of(tt);
                const int row = rg * R + 16 * t + lr;
                if (t < 0 || row >= nrows) continue;
                const int node = row / G, h = g * G + row % G;
                const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
                const float inv = 1.f / l_run[tt];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const f32x4_t val = o[tt][dt] * inv;
                    const size_t off = orow * D + 16 * dt + 4 * lq;
                    if constexpr (F32IN) {
                        *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + off) = val;
                    } else {
                        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + off) =
                            u32x2_t{ev::pack_bf16x2(val[0], val[1]), ev::pack_bf16x2(val[2], val[3])};
                    }
                }
                if (a.lse && lq == 0) a.lse[orow] = (m_run[tt] + __log2f(l_run[tt])) * kLn2;
            }
            continue;
        }

        // ---- split unit: publish this piece's partial (m, l, unnormalised O); the merge launch
        // combines the unit's pieces
        const int w1 = pm.k ? pm.w1 : wg_of(ustart, S, P);
        {
            float *slot = slot_of_piece(a.part, w1, wl - w1, Lay::kSlotFloats);
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int t = tile_of(tt);
                if (t < 0) continue;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<f32x4_t *>(slot + (16 * t + lr) * D + 16 * dt + 4 * lq) = o[tt][dt];
                if (lq == 0) {
                    slot[R * D + 16 * t + lr] = m_run[tt];
                    slot[R * D + R + 16 * t + lr] = l_run[tt];
                }
            }
        }
        if (wl == w1 && tid == 0) a.table[wl] = int4{pm.k ? pm.k : wg_of(uend - 1, S, P) - w1 + 1, ns0, n, ui};
    }
}

// Up to four row tiles: 32-key stages, two workgroups per CU.
template <int D, int RT, bool F32IN, bool PG>
__global__ __launch_bounds__(kThreads, 2) void tree_attention_kernel(const AttnArgs a) {
    attention_body<D, RT, F32IN, PG>(a);
}
// 80-row units: 64-key stages, one workgroup per CU (each wave holds 1.25 tiles).
template <int D, bool F32IN>
__global__ __launch_bounds__(kThreads, 1) void tree_attention_kernel5(const AttnArgs a) {
    attention_body<D, 5, F32IN, false>(a);
}

// ---------------------------------------------------------------------------------------------
// 80-row units with bf16 inputs: key-split waves with private load pipelines.
//
// Every wave covers all five 16-row tiles (all N*G rows of the unit) for its own 16-key quarter
// of each 64-key stage, so each K/V byte is read from LDS once (not once per row tile), and the
// wave alone loads, reads and refills its quarter's LDS buffers: no workgroup barrier inside the
// stage loop, and a buffer is refilled as soon as its operands are in registers, which keeps
// about four stages in flight per wave.  The softmax keeps a running maximum per row and rescales
// only when a new score exceeds it by more than 2^8 (in the exponent's base-2 domain), so the
// cross-lane maximum is taken rarely; probabilities stay below 2^8 and lose nothing in bf16's
// relative precision.  The four wave states meet through LDS at the end of each piece, each wave
// finalising a quarter of the d columns.

template <int D>
struct LayKS {
    static constexpr int R = 80;
    static constexpr int RT = 5;
    static constexpr int KST = 64;                        // keys per stage, 16 per wave
    static constexpr int ROWB = 2 * D;                    // bytes per K/V row
    static constexpr int SUB = 16 * ROWB;                 // one wave's 16 K (or V) rows
    static constexpr int WBUF = 2 * SUB;                  // K rows then V rows
    static constexpr int NB = 4;                          // buffers per wave
    static constexpr int kScan = 4 * EV_MAX_BATCH;
    static constexpr int kMisc = 32;
    static constexpr int kPar = kWaves * 4 * EV_MAX_NODES;  // each wave's copy of the parents
    static constexpr int kQ = R * ROWB;                   // the unit's Q rows (bf16, swizzled like K)
    static constexpr int kBufs = kWaves * NB * WBUF;
    static constexpr int kTotal = kScan + kMisc + kPar + kQ + kBufs;
    static_assert(kTotal <= 160 * 1024, "LDS");
    static constexpr int DTW = D / 16 / kWaves;           // d tiles each wave finalises
    static constexpr int XO = kWaves * (D / 16 - DTW) * RT * 64 * 16;  // merge exchange bytes
    static_assert(XO + 2 * kWaves * R * 4 <= kBufs, "merge exchange space");
};

// One asm block per stage and wave: the K operand reads (ds_read_b128) and the V^T operand
// transpose reads (ds_read_b64_tr_b16), waiting for all of them before the block ends.
#define EV_RK(o, a) "ds_read_b128 %" #o ", %" #a "\n\t"
#define EV_RV(o, a) "ds_read_b64_tr_b16 %" #o ", %" #a "\n\t"
template <int D> struct ReadKV;
template <> struct ReadKV<128> {
    __device__ static __forceinline__ void run(u32x4_t (&k)[4], u32x2_t (&v)[8], const uint32_t (&ka)[4],
                                               const uint32_t (&va)[8]) {
        asm volatile(EV_RK(0, 12) EV_RK(1, 13) EV_RK(2, 14) EV_RK(3, 15)
                     EV_RV(4, 16) EV_RV(5, 17) EV_RV(6, 18) EV_RV(7, 19)
                     EV_RV(8, 20) EV_RV(9, 21) EV_RV(10, 22) EV_RV(11, 23)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
                       "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
                     : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
                       "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
                     : "memory");
    }
};
template <> struct ReadKV<64> {
    __device__ static __forceinline__ void run(u32x4_t (&k)[2], u32x2_t (&v)[4], const uint32_t (&ka)[2],
                                               const uint32_t (&va)[4]) {
        asm volatile(EV_RK(0, 6) EV_RK(1, 7) EV_RV(2, 8) EV_RV(3, 9) EV_RV(4, 10) EV_RV(5, 11)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                     : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
                     : "memory");
    }
};
#undef EV_RK
#undef EV_RV

// The Q^T operands of all five row tiles from the staged Q rows: q[t][s] at a[s] + t * 16 rows.
#define EV_RQ(o, a, off) "ds_read_b128 %" #o ", %" #a " offset:" #off "\n\t"
template <int D> struct ReadQ;
template <> struct ReadQ<128> {  // 16 rows = 4096 bytes
    __device__ static __forceinline__ void run(bf16x8_t (&q)[5][4], const uint32_t (&a)[4]) {
        asm volatile(EV_RQ(0, 20, 0) EV_RQ(1, 21, 0) EV_RQ(2, 22, 0) EV_RQ(3, 23, 0)
                     EV_RQ(4, 20, 4096) EV_RQ(5, 21, 4096) EV_RQ(6, 22, 4096) EV_RQ(7, 23, 4096)
                     EV_RQ(8, 20, 8192) EV_RQ(9, 21, 8192) EV_RQ(10, 22, 8192) EV_RQ(11, 23, 8192)
                     EV_RQ(12, 20, 12288) EV_RQ(13, 21, 12288) EV_RQ(14, 22, 12288) EV_RQ(15, 23, 12288)
                     EV_RQ(16, 20, 16384) EV_RQ(17, 21, 16384) EV_RQ(18, 22, 16384) EV_RQ(19, 23, 16384)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(q[0][0]), "=&v"(q[0][1]), "=&v"(q[0][2]), "=&v"(q[0][3]), "=&v"(q[1][0]),
                       "=&v"(q[1][1]), "=&v"(q[1][2]), "=&v"(q[1][3]), "=&v"(q[2][0]), "=&v"(q[2][1]),
                       "=&v"(q[2][2]), "=&v"(q[2][3]), "=&v"(q[3][0]), "=&v"(q[3][1]), "=&v"(q[3][2]),
                       "=&v"(q[3][3]), "=&v"(q[4][0]), "=&v"(q[4][1]), "=&v"(q[4][2]), "=&v"(q[4][3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};
template <> struct ReadQ<64> {  // 16 rows = 2048 bytes
    __device__ static __forceinline__ void run(bf16x8_t (&q)[5][2], const uint32_t (&a)[2]) {
        asm volatile(EV_RQ(0, 10, 0) EV_RQ(1, 11, 0) EV_RQ(2, 10, 2048) EV_RQ(3, 11, 2048)
                     EV_RQ(4, 10, 4096) EV_RQ(5, 11, 4096) EV_RQ(6, 10, 6144) EV_RQ(7, 11, 6144)
                     EV_RQ(8, 10, 8192) EV_RQ(9, 11, 8192)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(q[0][0]), "=&v"(q[0][1]), "=&v"(q[1][0]), "=&v"(q[1][1]), "=&v"(q[2][0]),
                       "=&v"(q[2][1]), "=&v"(q[3][0]), "=&v"(q[3][1]), "=&v"(q[4][0]), "=&v"(q[4][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    }
};
#undef EV_RQ

constexpr float kRescaleSlack = 8.f;  // log2 of the largest probability allowed before a rescale

template <int D, bool PG>
__device__ __forceinline__ void attention_ks_body(const AttnArgs &a) {
    using Lay = LayKS<D>;
    constexpr int R = Lay::R;
    constexpr int RT = Lay::RT;
    constexpr int KST = Lay::KST;
    constexpr int NW = kWaves;
    constexpr int KS = D / 32;                 // k-steps of the QK^T contraction
    constexpr int DT = D / 16;                 // 16-wide d tiles of O^T
    constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
    constexpr int ROWB = Lay::ROWB;
    constexpr int SUB = Lay::SUB;
    constexpr int WBUF = Lay::WBUF;
    constexpr int NB = Lay::NB;
    constexpr int RPI = 1024 / ROWB;           // rows per 1-KB wave load
    constexpr int PERK = 16 / RPI;             // wave loads per 16-row block
    constexpr int PERW = 2 * PERK;             // wave loads per stage (K and V)
    constexpr int SWZ = 16 / CPR;              // rows per 256-byte bank cycle
    constexpr int DTW = Lay::DTW;
    static_assert(PERW * (NB - 1) < 64, "vmcnt range");
    static_assert(NB % 2 == 0, "the ring is consumed and refilled two stages at a time");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::kTotal];
    int32_t *s_cum = reinterpret_cast<int32_t *>(smem);
    int64_t *s_misc = reinterpret_cast<int64_t *>(smem + Lay::kScan);
    unsigned char *pbufs = smem + Lay::kScan + Lay::kMisc;               // [wave][64] int32 parents
    unsigned char *qbuf = pbufs + Lay::kPar;                             // [80 rows][D] bf16
    unsigned char *bufs = qbuf + Lay::kQ;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches only
    const int G = a.group;
    const float c2 = a.scale_log2;

    const int64_t S = schedule_scan<R, KST>(a, s_cum, s_misc);
    const int grid = gridDim.x;
    int wl;
    const PieceMap pm = map_pieces(a, s_cum, S, grid, wl);
    const int P = pm.P;
    if (tid == 0) a.table[wl] = int4{0, 0, 0, 0};  // no split unit starts here (until one does)
    if (wl >= P) return;
    const int64_t begin = pm.begin, end = pm.end;

    // Chunks are XOR-swizzled per row (same rule as the other bf16 path): K row r keeps global
    // chunk c at slot c ^ fk(r), V row r at slot c ^ fv(r); rows are local to a 16-row block.
    auto fk = [](int r) { return (r / SWZ) & (CPR - 1); };
    auto fv = [](int r) { return 2 * ((r / SWZ) & (CPR / 2 - 1)); };
    unsigned char *wbuf = bufs + wave * NB * WBUF;        // this wave's private buffers

    for (int64_t pos = begin; pos < end;) {
        // Lane-derived values are recomputed for every piece: kept live across the whole kernel
        // they crowd the registers of the stage loop out and come back through scratch.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int lr = lane & 15;
        const int lq = lane >> 4;
        // ---- locate the unit that holds stage `pos`
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] > pos) hi = mid; else lo = mid + 1;
        }
        const int b = lo;
        const int64_t seq_base = b ? s_cum[b - 1] : 0;
        const int ns0 = a.node_start[b];
        const int n = a.node_start[b + 1] - ns0;
        int L;
        int64_t s0;
        visible_prefix<PG>(a, b, L, s0);
        const int stages = (L + n + KST - 1) / KST;
        const int ui = static_cast<int>((pos - seq_base) / stages);
        const int rg = ui / a.hkv, g = ui % a.hkv;
        const int64_t ustart = seq_base + static_cast<int64_t>(ui) * stages, uend = ustart + stages;
        const int64_t pend = end < uend ? end : uend;
        const int st0 = static_cast<int>(pos - ustart), st1 = static_cast<int>(pend - ustart);
        pos = pend;

        const int nrows = n * G;
        const int kv_end = L + n;
        const int nst = st1 - st0;
        const size_t slot_stride = static_cast<size_t>(a.kv_slot_stride);  // elements between slots
        // paged caches: rows are found per block through the block table, s0 is a token index
        const size_t head_off = (PG ? 0 : static_cast<size_t>(s0) * slot_stride) + static_cast<size_t>(g) * a.kv_head_stride;
        const uint16_t *kbase = static_cast<const uint16_t *>(a.k) + head_off;
        const uint16_t *vbase = static_cast<const uint16_t *>(a.v) + head_off;
        const int32_t *bt = nullptr;
        if constexpr (PG) bt = a.block_table + static_cast<size_t>(__builtin_amdgcn_readfirstlane(b)) * a.bt_stride;

        // lane offsets of the operand reads inside one buffer: K operand step s = row lr, chunk
        // 4s + lq; V^T operand d tile dt = rows 4lq + lr/4, chunk 2dt + (lr&3)/2, half lr&1
        const uint32_t wbuf_lds = lds_addr(wbuf);
        uint32_t koff[KS], voff[DT];
#pragma unroll
        for (int s = 0; s < KS; ++s) koff[s] = lr * ROWB + 16 * ((4 * s + lq) ^ fk(lr));
        {
            const int r0 = 4 * lq + (lr >> 2);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                voff[dt] = SUB + r0 * ROWB + 32 * (dt ^ (fv(r0) >> 1)) + 16 * ((lr & 3) >> 1) + 8 * (lr & 1);
        }
        // this wave's quarter of stage st (keys st*64 + 16*wave + 0..15) into buffer bi: a uniform
        // block address plus loop-invariant lane offsets; rows past the unit (only in the block
        // that crosses its end) read row 0 instead, a finite row that the mask removes
        const uint32_t slot_bytes = static_cast<uint32_t>(slot_stride) * 2;
        uint32_t doff[PERW];
#pragma unroll
        for (int i = 0; i < PERW; ++i) {
            const bool isv = i >= PERK;
            const int row = (isv ? i - PERK : i) * RPI + lane / CPR;
            doff[i] = row * slot_bytes + 16 * ((lane % CPR) ^ (isv ? fv(row) : fk(row)));
        }
        const char *kb8 = reinterpret_cast<const char *>(kbase);
        const char *vb8 = reinterpret_cast<const char *>(vbase);
        auto issue = [&](int st, int bi) {
            unsigned char *buf = wbuf + bi * WBUF;
            const int kp0 = st * KST + 16 * wave;
            if constexpr (PG) {
                // the block's tokens (rows past the unit read its last row) span at most two pages
                const int kl = kv_end - 1;
                const int t0 = __builtin_amdgcn_readfirstlane(static_cast<int>(s0) + min(kp0, kl));
                const int t1 = __builtin_amdgcn_readfirstlane(static_cast<int>(s0) + min(kp0 + 15, kl));
                const int sh = a.page_shift;
                const int64_t r0 = page_row(a, bt, t0);
                if (kp0 + 16 <= kv_end && (t0 >> sh) == (t1 >> sh)) {
                    // one page: a uniform block address plus the invariant lane offsets
                    const size_t boff = static_cast<size_t>(r0 + (t0 & ((1 << sh) - 1))) * slot_bytes;
#pragma unroll
                    for (int i = 0; i < PERW; ++i) {
                        const bool isv = i >= PERK;
                        const char *src = (isv ? vb8 : kb8) + boff + doff[i];
                        __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf + (isv ? SUB : 0) + (isv ? i - PERK : i) * 1024),
                                                         16, 0, kKvLoadPolicy);
                    }
                } else {
                    const int64_t r1 = page_row(a, bt, t1);
#pragma unroll
                    for (int i = 0; i < PERW; ++i) {
                        const bool isv = i >= PERK;
                        const int local = isv ? i - PERK : i;
                        const int row = local * RPI + lane / CPR;
                        const int c = (lane % CPR) ^ (isv ? fv(row) : fk(row));
                        const int t = static_cast<int>(s0) + min(kp0 + row, kl);
                        const int64_t r = ((t >> sh) == (t0 >> sh) ? r0 : r1) + (t & ((1 << sh) - 1));
                        const char *src = (isv ? vb8 : kb8) + static_cast<size_t>(r) * slot_bytes + 16 * c;
                        __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf + (isv ? SUB : 0) + local * 1024), 16, 0, kKvLoadPolicy);
                    }
                }
            } else if (kp0 + 16 <= kv_end) {
                const size_t boff = static_cast<size_t>(kp0) * slot_bytes;
#pragma unroll
                for (int i = 0; i < PERW; ++i) {
                    const bool isv = i >= PERK;
                    const char *src = (isv ? vb8 : kb8) + boff + doff[i];
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf + (isv ? SUB : 0) + (isv ? i - PERK : i) * 1024),
                                                     16, 0, kKvLoadPolicy);
                }
            } else {
#pragma unroll
                for (int i = 0; i < PERW; ++i) {
                    const bool isv = i >= PERK;
                    const int local = isv ? i - PERK : i;
                    const int row = local * RPI + lane / CPR;
                    const int c = (lane % CPR) ^ (isv ? fv(row) : fk(row));
                    const int kp = kp0 + row;
                    const int kpc = kp < kv_end ? kp : 0;
                    const char *src = (isv ? vb8 : kb8) + static_cast<size_t>(kpc) * slot_bytes + 16 * c;
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(buf + (isv ? SUB : 0) + local * 1024), 16, 0, kKvLoadPolicy);
                }
            }
        };

        // ---- the piece's loads, all global -> LDS (no register loads to wait for): this wave's
        // copy of the parents, its share of the unit's Q rows (rows past the unit read a real
        // row: their results are never written), then its first NB stages (indices clamped into
        // the piece, so the count is fixed).  Waiting for the first stage covers the rest.
        // Every wave is done with the previous piece's buffers and Q rows first.  (The builtin wait
        // costs nothing here -- the unit's geometry loads above are complete -- but it tells the
        // compiler that no earlier load is pending, so it adds no wait among the loads below.)
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        bare_barrier();
        unsigned char *pbuf = pbufs + wave * 4 * EV_MAX_NODES;
        __builtin_amdgcn_global_load_lds(a.parent + ns0 + min(lane, n - 1), (lds_void_t *)pbuf, 4, 0, 0);
        {
            constexpr int NQ = Lay::kQ / 1024;                   // 1-KB wave loads of Q rows
#pragma unroll
            for (int k0 = 0; k0 < NQ; k0 += NW) {
                const int k = k0 + wave;
                if (k < NQ) {
                    const int r = k * RPI + lane / CPR;            // row within the unit
                    const int c = (lane % CPR) ^ fk(r);
                    const int row = rg * R + r;
                    const bool live = row < nrows;
                    const int node = live ? row / G : 0;
                    const int h = g * G + (live ? row % G : 0);
                    const uint16_t *src = static_cast<const uint16_t *>(a.q) +
                                          (static_cast<size_t>(ns0 + node) * a.hq + h) * D + 8 * c;
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(qbuf + k * 1024), 16, 0, 0);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) issue(st0 + min(i, nst - 1), i);
        vm_wait_n<(NB - 1) * PERW>();
        bare_barrier();  // every wave's share of the Q rows has landed
        int par;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(par) : "v"(lds_addr(pbuf) + 4 * lane) : "memory");
        if (lane >= n) par = -1;
        // the Q^T operands are read from the staged Q rows once per pair of blocks (held for the
        // whole piece they would crowd the pair's operands out of the registers)
        uint32_t qa[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) qa[s] = lds_addr(qbuf) + koff[s];
        // ---- tree: validity and ancestor masks, while the loads are in flight
        const bool ok = lane >= n || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
        if (__any(!ok)) {
            if (tid == 0) ev::flag_error(a.err_flag, EV_DATA_BAD_PARENT);
            vm_wait_n<0>();
            continue;  // uniform across the workgroup: every wave read the same parents
        }
        uint64_t anc = lane < n ? (1ull << lane) : 0ull;
        int j = lane < n ? par : -1;
        while (__any(j >= 0)) {
            if (j >= 0) anc |= 1ull << j;
            const int pj = __shfl(par, j >= 0 ? j : 0, 64);
            j = j >= 0 ? pj : -1;
        }
        f32x4_t o[RT][DT];
        float m_run[RT], l_run[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            m_run[t] = -INFINITY;
            l_run[t] = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        // The wave takes its 16-key blocks two at a time (block a of stage i, block b of stage
        // i + 1).  Scores are S^T = K Q^T per block; the value product runs over both blocks' 32
        // keys on v_mfma_f32_16x16x32_bf16 (half the instructions of two 16-key products).  Its k
        // slots 8q + e (lane group q = lane / 16) hold keys 4q + e of block a for e < 4 and keys
        // 4q + e - 4 of block b for e >= 4: exactly the four score rows each lane holds in both
        // score tiles and the four keys each V^T transpose read returns, so no value moves between
        // lanes.  A missing block b (odd stage count) enters with zero probabilities against a
        // copy of block a's values.
        auto accumulate = [&](const f32x4_t (&sa)[RT], const f32x4_t (&sb)[RT], const u32x2_t (&vqa)[DT],
                              const u32x2_t (&vqb)[DT]) {
            u32x4_t pw[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const float mu = m_run[t] == -INFINITY ? 0.f : m_run[t];
                const float a0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][0], c2, -mu));
                const float a1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][1], c2, -mu));
                const float a2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][2], c2, -mu));
                const float a3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][3], c2, -mu));
                const float b0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[t][0], c2, -mu));
                const float b1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[t][1], c2, -mu));
                const float b2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[t][2], c2, -mu));
                const float b3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[t][3], c2, -mu));
                l_run[t] += ((a0 + a1) + (a2 + a3)) + ((b0 + b1) + (b2 + b3));
                pw[t] = u32x4_t{ev::pack_bf16x2(a0, a1), ev::pack_bf16x2(a2, a3), ev::pack_bf16x2(b0, b1),
                                ev::pack_bf16x2(b2, b3)};
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, u32x4_t{vqa[dt][0], vqa[dt][1], vqb[dt][0], vqb[dt][1]});
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, __builtin_bit_cast(bf16x8_t, pw[t]), o[t][dt],
                                                                       0, 0, 0);
            }
        };
        // scores of one block of 16 keys starting at unit-relative key kb: S^T = K Q^T, then the
        // ancestor mask where the block reaches the tree slots
        auto scores = [&](f32x4_t (&sc)[RT], const u32x4_t (&kq)[KS], const bf16x8_t (&qop)[RT][KS], int kb) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[s2]), qop[t][s2], acc,
                                                                  0, 0, 0);
                sc[t] = acc;
            }
            if (kb + 16 > L) {  // the block reaches the tree slots or the unit's end
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    // ancestor mask of this lane's row (rows past the unit see nothing)
                    const int row = rg * R + 16 * t + lr;
                    const int node = row < nrows ? row / G : 0;
                    const uint32_t mlo = __shfl(static_cast<uint32_t>(anc), node, 64);
                    const uint32_t mhi = __shfl(static_cast<uint32_t>(anc >> 32), node, 64);
                    const uint64_t rmask = row < nrows ? ((static_cast<uint64_t>(mhi) << 32) | mlo) : 0ull;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = kb + 4 * lq + r;
                        const bool vis = p < L || (p < kv_end && ((rmask >> (p - L)) & 1ull));
                        if (!vis) sc[t][r] = -INFINITY;
                    }
                }
            }
        };

        // The hot loop never touches the accumulators outside the MFMAs (they stay in the matrix
        // registers); a pair whose scores need new maxima leaves it, and the rescale runs below.
        int i = 0;
        for (;;) {
            f32x4_t sa[RT], sb[RT];
            float mloc[RT];
            u32x2_t vqa[DT], vqb[DT];
            bool rescale = false;
            for (; i < nst; i += 2) {
                const bool two = i + 1 < nst;
                // this wave's stages issued after the pair: the ring holds NB stages, refilled two
                // at a time
                const int later = min(nst, i + NB) - min(nst, i + 2);
                if (later >= 2) vm_wait_n<2 * PERW>();
                else if (later == 1) vm_wait_n<PERW>();
                else vm_wait_n<0>();
                // block a's operands, its refill and its scores, then block b's (one block's K
                // operands live at a time); sa[t] / sb[t] hold raw scores of keys kb + 4*lq + r
                // for row 16t + lr, kb the block's unit-relative first key
                bf16x8_t qop[RT][KS];
                ReadQ<D>::run(qop, qa);
                {
                    u32x4_t kq[KS];
                    const uint32_t base = wbuf_lds + (i % NB) * WBUF;
                    uint32_t ka[KS], va[DT];
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) ka[s2] = base + koff[s2];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) va[dt] = base + voff[dt];
                    ReadKV<D>::run(kq, vqa, ka, va);
                    if (i + NB < nst) issue(st0 + i + NB, i % NB);  // the buffer's operands are in registers
                    scores(sa, kq, qop, (st0 + i) * KST + 16 * wave);
                }
                if (two) {
                    u32x4_t kq[KS];
                    const uint32_t base = wbuf_lds + ((i + 1) % NB) * WBUF;
                    uint32_t ka[KS], va[DT];
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) ka[s2] = base + koff[s2];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) va[dt] = base + voff[dt];
                    ReadKV<D>::run(kq, vqb, ka, va);
                    if (i + 1 + NB < nst) issue(st0 + i + 1 + NB, (i + 1) % NB);
                    scores(sb, kq, qop, (st0 + i + 1) * KST + 16 * wave);
                } else {
#pragma unroll
                    for (int t = 0; t < RT; ++t) sb[t] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) vqb[dt] = vqa[dt];
                }
                // running maxima move only when a score exceeds them by more than the slack
                bool need = false;
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    mloc[t] = fmaxf(fmaxf(fmaxf(sa[t][0], sa[t][1]), fmaxf(sa[t][2], sa[t][3])),
                                    fmaxf(fmaxf(sb[t][0], sb[t][1]), fmaxf(sb[t][2], sb[t][3])));
                    need |= mloc[t] * c2 > m_run[t] + kRescaleSlack;
                }
                if (__any(need)) {
                    rescale = true;
                    break;
                }
                accumulate(sa, sb, vqa, vqb);
            }
            if (!rescale) break;
            // new maxima for the pair at i: rescale the states, then finish the pair
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                float mx = mloc[t];
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[t], mx * c2);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[t] - m_new);
                if (__any(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
                }
                l_run[t] *= alpha;
                m_run[t] = m_new;
            }
            accumulate(sa, sb, vqa, vqb);
            i += 2;
        }

        // ---- row sums over the four lanes that share a row
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            l_run[t] += __shfl_xor(l_run[t], 16, 64);
            l_run[t] += __shfl_xor(l_run[t], 32, 64);
        }

        // ---- the four wave states meet in LDS; wave w finalises d tiles [w*DTW, (w+1)*DTW)
        f32x4_t *xo = reinterpret_cast<f32x4_t *>(bufs);                       // [src][dt'][t][lane]
        float *xm = reinterpret_cast<float *>(bufs + Lay::XO);                 // [src][R]
        float *xl = xm + NW * R;                                               // [src][R]
        __syncthreads();  // every wave is done with its stage buffers
        {
            int jj = 0;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (dt / DTW == wave) continue;
#pragma unroll
                for (int t = 0; t < RT; ++t) xo[((wave * (DT - DTW) + jj) * RT + t) * 64 + lane] = o[t][dt];
                ++jj;
            }
            if (lq == 0) {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    xm[wave * R + 16 * t + lr] = m_run[t];
                    xl[wave * R + 16 * t + lr] = l_run[t];
                }
            }
        }
        __syncthreads();
        float fac[NW][RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            float ms[NW], M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                ms[w] = xm[w * R + 16 * t + lr];
                M = fmaxf(M, ms[w]);
            }
            const float Mu = M == -INFINITY ? 0.f : M;
            float lt = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                fac[w][t] = __builtin_amdgcn_exp2f(ms[w] - Mu);
                lt += fac[w][t] * xl[w * R + 16 * t + lr];
            }
            m_run[t] = M;
            l_run[t] = lt;
        }
        // (one instantiation per wave keeps every register index a compile-time constant)
        f32x4_t fin[RT][DTW];
        auto finalise = [&](auto wc) {
            constexpr int W = decltype(wc)::value;
#pragma unroll
            for (int k = 0; k < DTW; ++k) {
                const int dt = W * DTW + k;
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        f32x4_t x;
                        if (w == W) {
                            x = o[t][dt];
                        } else {
                            const int jw = dt < w * DTW ? dt : dt - DTW;  // dt's index among w's exported tiles
                            x = xo[((w * (DT - DTW) + jw) * RT + t) * 64 + lane];
                        }
                        acc += fac[w][t] * x;
                    }
                    fin[t][k] = acc;
                }
            }
        };
        switch (wave) {
            case 0: finalise(std::integral_constant<int, 0>{}); break;
            case 1: finalise(std::integral_constant<int, 1>{}); break;
            case 2: finalise(std::integral_constant<int, 2>{}); break;
            default: finalise(std::integral_constant<int, 3>{}); break;
        }

        // ---- output
        const bool whole = ustart >= begin && uend <= end;
        if (whole) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const int row = rg * R + 16 * t + lr;
                if (row >= nrows) continue;
                const int node = row / G, h = g * G + row % G;
                const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
                const float inv = 1.f / l_run[t];
#pragma unroll
                for (int k = 0; k < DTW; ++k) {
                    const f32x4_t val = fin[t][k] * inv;
                    const size_t off = orow * D + 16 * (wave * DTW + k) + 4 * lq;
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + off) =
                        u32x2_t{ev::pack_bf16x2(val[0], val[1]), ev::pack_bf16x2(val[2], val[3])};
                }
                if (a.lse && wave == 0 && lq == 0) a.lse[orow] = (m_run[t] + __log2f(l_run[t])) * kLn2;
            }
            continue;
        }
        // split unit: publish this piece's partial; the merge launch combines the unit's pieces
        const int w1 = pm.k ? pm.w1 : wg_of(ustart, S, P);
        {
            float *slot = slot_of_piece(a.part, w1, wl - w1, R * D + 2 * R);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
#pragma unroll
                for (int k = 0; k < DTW; ++k)
                    *reinterpret_cast<f32x4_t *>(slot + (16 * t + lr) * D + 16 * (wave * DTW + k) + 4 * lq) = fin[t][k];
                if (wave == 0 && lq == 0) {
                    slot[R * D + 16 * t + lr] = m_run[t];
                    slot[R * D + R + 16 * t + lr] = l_run[t];
                }
            }
        }
        if (wl == w1 && tid == 0) a.table[wl] = int4{pm.k ? pm.k : wg_of(uend - 1, S, P) - w1 + 1, ns0, n, ui};
    }
}

template <int D, bool PG>
__global__ __launch_bounds__(kThreads, 1) void tree_attention_kernel_ks(const AttnArgs a) {
    attention_ks_body<D, PG>(a);
}

// ---------------------------------------------------------------------------------------------
// Merge of split units (second launch; the launch boundary makes the published partials visible).
// A resident grid: every block compacts the table's split units (their entries, in LDS, so no
// item re-reads the table), then the blocks stride
// over the work items (unit, row tile, half of the d columns).  An item combines the unit's
// pieces: M = max_i m_i, O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i, summed in the fixed
// chunked piece order below (deterministic), 16 rows x D/8 threads with one float4 of O each.
constexpr int kMergeBlocks = 512;
// Summation order of a unit's pieces in every merge: consecutive chunks of kMergeChunk pieces,
// each summed in piece order from zero, and the chunk sums added in chunk order to a total that
// starts at zero.  Units of at most kMergeChunk pieces are one chunk (a plain sum in piece order);
// larger units may then be merged chunk-parallel (merge_item_split) with the same bits.
constexpr int kMergeChunk = 8;

template <int D, int BATCH, bool F32OUT>
__device__ __forceinline__ void merge_item(const AttnArgs &a, int R, int w1, int4 e, int t, int half, bool given,
                                           float Mg) {
    constexpr int CT = D / 8;                  // threads per row (float4 chunks per half row)
    const int rr = threadIdx.x / CT, c = threadIdx.x % CT;
    const int npieces = e.x, ns0 = e.y, n = e.z, ui = e.w;
    const int rg = ui / a.hkv, g = ui % a.hkv;
    const int G = a.group;
    const int r = 16 * t + rr;                 // row within the unit (every slot has R rows)
    const int d0 = half * (D / 2) + 4 * c;
    const int slot_floats = R * D + 2 * R;
    // The maximum over all the unit's pieces comes first: from the loads of the one round when a
    // round holds every piece, else (given) from a pass over the pieces' maxima before the call.
    // The sums then run in the chunked piece order (kMergeChunk) under that one scale, so the
    // result has the same bits for any round size.  (A chunk sum is never -0: it starts at +0.)
    static_assert(BATCH < kMergeChunk ? kMergeChunk % BATCH == 0 : BATCH % kMergeChunk == 0, "chunk-aligned rounds");
    float M = given ? Mg : -INFINITY, l = 0.f, lc = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, cacc = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < npieces; i0 += BATCH) {
        const float *slot[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) slot[k] = slot_of_piece(a.part, w1, i0 + k < npieces ? i0 + k : i0, slot_floats);
        f32x4_t x[BATCH];
        float mi[BATCH], li[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            x[k] = *reinterpret_cast<const f32x4_t *>(slot[k] + r * D + d0);
            mi[k] = slot[k][R * D + r];
            li[k] = slot[k][R * D + R + r];
        }
        // (an empty asm that takes every loaded value: no use of one moves above a later load)
#pragma unroll
        for (int k = 0; k < BATCH; ++k) asm volatile("" : "+v"(x[k]), "+v"(mi[k]), "+v"(li[k]));
        if (!given) {
#pragma unroll
            for (int k = 0; k < BATCH; ++k) M = fmaxf(M, i0 + k < npieces ? mi[k] : -INFINITY);
        }
        const float mu = M == -INFINITY ? 0.f : M;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const float f = i0 + k < npieces ? __builtin_amdgcn_exp2f(mi[k] - mu) : 0.f;
            cacc += f * x[k];
            lc += f * li[k];
            if (BATCH >= kMergeChunk && k % kMergeChunk == kMergeChunk - 1) {
                acc += cacc;
                l += lc;
                cacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                lc = 0.f;
            }
        }
        if (BATCH < kMergeChunk && (i0 + BATCH) % kMergeChunk == 0) {
            acc += cacc;
            l += lc;
            cacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            lc = 0.f;
        }
    }
    acc += cacc;  // the last, partial chunk (adds +0 when there is none)
    l += lc;
    const int row = rg * R + r;
    if (row >= n * G) return;                  // rows past the unit's nodes
    const int node = row / G, h = g * G + row % G;
    const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
    const f32x4_t val = acc * (1.f / l);
    if constexpr (F32OUT) {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + orow * D + d0) = val;
    } else {
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + orow * D + d0) =
            u32x2_t{ev::pack_bf16x2(val[0], val[1]), ev::pack_bf16x2(val[2], val[3])};
    }
    if (a.lse && half == 0 && c == 0) a.lse[orow] = (M + __log2f(l)) * kLn2;
}

// One merge item of a unit of more than kMergeChunk pieces, chunk-parallel: 8 rows and 32 columns
// (one 128-byte line of every fp32 row) of the unit's output, on a block of 256 threads; item col
// (0..7) of row tile t holds rows 16t + 8 (col / 4) .. + 7 and columns 32 (col % 4) .. + 31.  Wave
// w sums chunks w, w + 4, ... (thread: row lane / 8, four columns); the block adds the chunk
// sums in chunk order through LDS, four chunks per round.  Same bits as merge_item (the same scale, the same chunk
// sums, the same order of their addition), in one or two round trips for units of up to
// 4 * kMergeChunk pieces instead of a pass over the maxima and a round per four pieces.
template <bool F32OUT>
__device__ __forceinline__ void merge_item_split(const AttnArgs &a, int R, int w1, int4 e, int t, int col) {
    constexpr int D = 128;
    constexpr int CH = kMergeChunk;
    __shared__ f32x4_t s_acc[kWaves][64];
    __shared__ float s_l[kWaves][8], s_m[kWaves][8];
    const int tid = threadIdx.x, j = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: piece addresses in scalar registers
    const int rr = j >> 3, c = j & 7;
    const int npieces = e.x, ns0 = e.y, n = e.z, ui = e.w;
    const int nch = (npieces + CH - 1) / CH;
    const int r = 16 * t + 8 * (col >> 2) + rr;
    const int d0 = 32 * (col & 3) + 4 * c;
    const int slot_floats = R * D + 2 * R;
    auto piece = [&](int p) { return slot_of_piece(a.part, w1, p < npieces ? p : npieces - 1, slot_floats); };
    // the maximum of row r over every piece (this wave's chunks, then the four waves' maxima)
    auto exchange_max = [&](float mw) {
        if (c == 0) s_m[wave][rr] = mw;
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][rr]);
        return M;
    };
    // the chunk sums of one round (chunks c0 .. c0 + 3) in chunk order onto wave 0's total
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    auto add_round = [&](int c0, bool mine, const f32x4_t &cacc, float lc) {
        if (mine) {
            s_acc[wave][j] = cacc;
            if (c == 0) s_l[wave][rr] = lc;
        }
        __syncthreads();
        if (wave == 0) {
            const int nw = min(kWaves, nch - c0);
            for (int w = 0; w < nw; ++w) {
                acc += s_acc[w][j];
                l += s_l[w][rr];
            }
        }
        __syncthreads();
    };
    float M;
    if (nch <= kWaves) {
        // each wave holds at most one chunk: all its loads in one round trip
        const bool mine = wave < nch;
        f32x4_t x[CH];
        float mi[CH], li[CH];
        float mw = -INFINITY;
        if (mine) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const float *sl = piece(wave * CH + k);
                x[k] = *reinterpret_cast<const f32x4_t *>(sl + r * D + d0);
                mi[k] = sl[R * D + r];
                li[k] = sl[R * D + R + r];
            }
#pragma unroll
            for (int k = 0; k < CH; ++k) mw = fmaxf(mw, wave * CH + k < npieces ? mi[k] : -INFINITY);
        }
        M = exchange_max(mw);
        const float mu = M == -INFINITY ? 0.f : M;
        f32x4_t cacc = {0.f, 0.f, 0.f, 0.f};
        float lc = 0.f;
        if (mine) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const float f = wave * CH + k < npieces ? __builtin_amdgcn_exp2f(mi[k] - mu) : 0.f;
                cacc += f * x[k];
                lc += f * li[k];
            }
        }
        add_round(0, mine, cacc, lc);
    } else {
        float mw = -INFINITY;
        for (int ch = wave; ch < nch; ch += kWaves) {
            float m8[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) m8[k] = piece(ch * CH + k)[R * D + r];
#pragma unroll
            for (int k = 0; k < CH; ++k) mw = fmaxf(mw, ch * CH + k < npieces ? m8[k] : -INFINITY);
        }
        M = exchange_max(mw);
        const float mu = M == -INFINITY ? 0.f : M;
        for (int c0 = 0; c0 < nch; c0 += kWaves) {
            const int ch = c0 + wave;
            const bool mine = ch < nch;
            f32x4_t cacc = {0.f, 0.f, 0.f, 0.f};
            float lc = 0.f;
            if (mine) {
                // the chunk in two halves (fewer registers; the sum still runs in piece order)
#pragma unroll
                for (int h0 = 0; h0 < CH; h0 += CH / 2) {
                    f32x4_t x[CH / 2];
                    float mi[CH / 2], li[CH / 2];
#pragma unroll
                    for (int k = 0; k < CH / 2; ++k) {
                        const float *sl = piece(ch * CH + h0 + k);
                        x[k] = *reinterpret_cast<const f32x4_t *>(sl + r * D + d0);
                        mi[k] = sl[R * D + r];
                        li[k] = sl[R * D + R + r];
                    }
#pragma unroll
                    for (int k = 0; k < CH / 2; ++k) {
                        const float f = ch * CH + h0 + k < npieces ? __builtin_amdgcn_exp2f(mi[k] - mu) : 0.f;
                        cacc += f * x[k];
                        lc += f * li[k];
                    }
                }
            }
            add_round(c0, mine, cacc, lc);
        }
    }
    if (wave != 0) return;
    const int rg = ui / a.hkv, g = ui % a.hkv;
    const int G = a.group;
    const int row = rg * R + r;
    if (row >= n * G) return;  // rows past the unit's nodes
    const int node = row / G, h = g * G + row % G;
    const size_t orow = static_cast<size_t>(ns0 + node) * a.hq + h;
    const f32x4_t val = acc * (1.f / l);
    if constexpr (F32OUT) {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + orow * D + d0) = val;
    } else {
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + orow * D + d0) =
            u32x2_t{ev::pack_bf16x2(val[0], val[1]), ev::pack_bf16x2(val[2], val[3])};
    }
    if (a.lse && (col & 3) == 0 && c == 0) a.lse[orow] = (M + __log2f(l)) * kLn2;
}

// The maximum of row 16t + threadIdx.x / (D / 8) of a unit over all its pieces (for units of
// more pieces than one round loads), sixteen independent loads at a time.
template <int D>
__device__ __forceinline__ float unit_row_max(const AttnArgs &a, int R, int w1, int npieces, int t) {
    const int r = 16 * t + static_cast<int>(threadIdx.x) / (D / 8);
    const int slot_floats = R * D + 2 * R;
    float M = -INFINITY;
    for (int i0 = 0; i0 < npieces; i0 += 16) {
        float mi[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) mi[k] = slot_of_piece(a.part, w1, i0 + k < npieces ? i0 + k : i0, slot_floats)[R * D + r];
#pragma unroll
        for (int k = 0; k < 16; ++k) M = fmaxf(M, i0 + k < npieces ? mi[k] : -INFINITY);
    }
    return M;
}

// The merge items of blocks mb, mb + nb, mb + 2 nb, ...  MAXB (4 or 32) caps the pieces loaded
// in one round (fewer registers; a unit of more pieces takes several rounds).  SPLIT (head_dim
// 128, 256 threads): when some unit has more than kMergeChunk pieces, every unit is merged in
// items of 8 rows x 32 columns by merge_item_split instead.
template <int D, bool F32OUT, int MAXB, bool SPLIT>
__device__ __forceinline__ void merge_blocks(const AttnArgs &a, int R, int RT, int entries, int mb, int nb) {
    constexpr int NT = 2 * D;
    static_assert(!SPLIT || D == 128, "chunk-parallel items: head_dim 128, 256 threads");
    __shared__ int s_idx[kMaxGrid];
    __shared__ int4 s_ent[kMaxGrid];
    __shared__ int s_cnt[NT / 64 + 1];
    __shared__ int s_maxk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if constexpr (SPLIT) {
        if (tid == 0) s_maxk = 0;
        __syncthreads();
    }
    // compact the table's split units (same order in every block)
    int base = 0;
    for (int e0 = 0; e0 < entries; e0 += NT) {
        const int e = e0 + tid;
        const int4 v = e < entries ? a.table[e] : int4{0, 0, 0, 0};
        const bool act = v.x > 0;
        if (SPLIT && act) atomicMax(&s_maxk, v.x);
        const uint64_t bal = __ballot(act);
        const int before = __popcll(bal & ((1ull << lane) - 1));
        if (lane == 0) s_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += s_cnt[w];
        if (act) {
            s_idx[off + before] = e;
            s_ent[off + before] = v;
        }
        int tot = 0;
        for (int w = 0; w < NT / 64; ++w) tot += s_cnt[w];
        base += tot;
        __syncthreads();
    }
    if (SPLIT && s_maxk > kMergeChunk) {  // (read after the compaction's last barrier)
        const int sitems = base * RT * (D / 16);
        for (int it = mb; it < sitems; it += nb) {
            const int u = it / (RT * (D / 16)), t = (it / (D / 16)) % RT, col = it % (D / 16);
            // (the item's unit is uniform: its table entry goes to scalar registers)
            const int4 eu = s_ent[u];
            const int4 es = int4{__builtin_amdgcn_readfirstlane(eu.x), __builtin_amdgcn_readfirstlane(eu.y),
                                 __builtin_amdgcn_readfirstlane(eu.z), __builtin_amdgcn_readfirstlane(eu.w)};
            merge_item_split<F32OUT>(a, R, __builtin_amdgcn_readfirstlane(s_idx[u]), es, t, col);
        }
        return;
    }
    const int items = base * RT * 2;
    for (int it = mb; it < items; it += nb) {
        const int u = it / (RT * 2), t = (it / 2) % RT, half = it % 2;
        const int w1 = s_idx[u];
        const int4 e = s_ent[u];
        // round size: every piece in one round when MAXB allows, else MAXB pieces per round after
        // a pass over the pieces' maxima
        const bool given = e.x > MAXB;
        const float Mg = given ? unit_row_max<D>(a, R, w1, e.x, t) : 0.f;
        if (e.x <= 2) merge_item<D, 2, F32OUT>(a, R, w1, e, t, half, false, Mg);
        else if (e.x <= 4 || MAXB == 4) merge_item<D, 4, F32OUT>(a, R, w1, e, t, half, given, Mg);
        else if (e.x <= 8) merge_item<D, 8, F32OUT>(a, R, w1, e, t, half, false, Mg);
        else if (e.x <= 16) merge_item<D, 16, F32OUT>(a, R, w1, e, t, half, false, Mg);
        else merge_item<D, 32, F32OUT>(a, R, w1, e, t, half, given, Mg);
    }
}

// SPLIT: the form with chunk-parallel items, launched for batches of few units (each then split
// into many pieces); both forms give the same bits, the plain one is faster where no unit needs it.
template <int D, bool F32OUT, bool SPLIT>
__global__ __launch_bounds__(2 * D, 2) void tree_attention_merge_kernel(const AttnArgs a, int R, int RT, int entries) {
    merge_blocks<D, F32OUT, 32, SPLIT>(a, R, RT, entries, static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
}

// The whole-step call's second launch at head_dim 128: the merge of the split units (the first
// kMergeBlocks blocks, dispatched first: some take two items in a row) beside the selection
// pass's row pieces (the blocks after them, one piece each; sel_mode 1 argmax of bf16 logits, 2
// of fp32 logits, 3 / 4 the sampled draw).  The two read disjoint data and write disjoint
// outputs; one launch lets the selection stream while the merge combines, instead of after it.
// Merge rounds load at most 4 pieces (registers for a full occupancy of the selection blocks).
template <bool F32OUT, bool SPLIT>
__global__ __launch_bounds__(256, 8) void tree_attention_merge_select_kernel(const AttnArgs a, const ev::sel::ArgmaxArgs s,
                                                                          int sel_pieces, int sel_mode, int R, int RT,
                                                                          int entries) {
    const int b = static_cast<int>(blockIdx.x);
    if (b >= kMergeBlocks) {
        const int pc = b - kMergeBlocks;
        switch (sel_mode) {
            case 1: ev::sel::argmax_piece<false>(s, pc); break;
            case 2: ev::sel::argmax_piece<true>(s, pc); break;
            case 3: ev::sel::sample_piece<false>(s, pc); break;
            default: ev::sel::sample_piece<true>(s, pc); break;
        }
        return;
    }
    merge_blocks<128, F32OUT, 4, SPLIT>(a, R, RT, entries, b, kMergeBlocks);
}

// ---------------------------------------------------------------------------------------------
struct Plan {
    int RT, R, RG;
    size_t slot_floats;
    size_t table_bytes;
    size_t bytes;
};

// Largest workspace any supported shape needs: the table plus 2 * kMaxGrid slots of 80-row,
// 128-wide partials (the plan below depends on the row tile and head_dim, never on the batch):
// 42,606,592 bytes.
constexpr size_t kMaxWorkspaceBytes =
    static_cast<size_t>(kMaxGrid) * sizeof(int4) +
    2 * static_cast<size_t>(kMaxGrid) * (static_cast<size_t>(16 * kMaxRowTiles) * 128 + 2 * 16 * kMaxRowTiles) * 4;
static_assert(kMaxWorkspaceBytes == 42606592, "the header states this size");

Plan make_plan(int32_t batch, int32_t max_nodes, int32_t hq, int32_t hkv, int32_t head_dim) {
    Plan p{};
    const int G = hq / hkv;
    const int rows = max_nodes * G;
    p.RT = rows >= 16 * kMaxRowTiles ? kMaxRowTiles : (rows + 15) / 16;
    p.R = 16 * p.RT;
    p.RG = (rows + p.R - 1) / p.R;
    p.slot_floats = static_cast<size_t>(p.R) * head_dim + 2 * p.R;
    p.table_bytes = static_cast<size_t>(kMaxGrid) * sizeof(int4);
    p.bytes = p.table_bytes + 2 * static_cast<size_t>(kMaxGrid) * p.slot_floats * 4;
    return p;
}

using KernelFn = void (*)(AttnArgs);

template <int D, bool F32IN, bool PG>
KernelFn pick_rt(int rt) {
    switch (rt) {
        case 1: return tree_attention_kernel<D, 1, F32IN, PG>;
        case 2: return tree_attention_kernel<D, 2, F32IN, PG>;
        case 3: return tree_attention_kernel<D, 3, F32IN, PG>;
        case 4: return tree_attention_kernel<D, 4, F32IN, PG>;
        default: return tree_attention_kernel5<D, F32IN>;  // fp32 only: bf16 80-row units go key-split
    }
}

KernelFn pick_kernel(int head_dim, int rt, bool f32, bool pg) {
    if (rt == kMaxRowTiles && !f32) {
        if (head_dim == 64) return pg ? tree_attention_kernel_ks<64, true> : tree_attention_kernel_ks<64, false>;
        return pg ? tree_attention_kernel_ks<128, true> : tree_attention_kernel_ks<128, false>;
    }
    if (pg) return head_dim == 64 ? pick_rt<64, false, true>(rt) : pick_rt<128, false, true>(rt);
    if (head_dim == 64) return f32 ? pick_rt<64, true, false>(rt) : pick_rt<64, false, false>(rt);
    return f32 ? pick_rt<128, true, false>(rt) : pick_rt<128, false, false>(rt);
}

// Resident workgroups per CU for a kernel variant, cached per (device, variant).
int blocks_per_cu(KernelFn fn, int variant) {
    static std::mutex mu;
    static int cache[16][64] = {};
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

// ---------------------------------------------------------------------------------------------
// Allocation-free form of ev_tree_attention.  Its workspace is this file-scope device array: one
// copy per GPU the library runs on, held until the process ends.  In host code the array's name
// stands for a host-side shadow, not a device address, so the device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that pointer reaches the
// kernels.  Every call on a GPU shares its copy: calls that overlap on one GPU (different
// streams, or other host threads) race on it; calls ordered on one stream do not.  The attention
// launches write every part of the workspace they later read, so nothing needs clearing.
static __device__ __align__(256) unsigned char scratch[kMaxWorkspaceBytes];  // 42,606,592 bytes

namespace {
constexpr int kScratchDevices = 16;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];

ev_status scratch_of_current_device(void **ptr) {
    const int dev = ev::current_device();
    if (dev < 0 || dev >= kScratchDevices) return EV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return EV_OK;
}
}  // namespace

namespace {
ev_status launch_attention(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                           const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                           const int32_t *prefix_len, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                           int64_t total_slots, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           ev_dtype dtype, float sm_scale, int32_t window, const int32_t *block_table,
                           int32_t bt_stride, int32_t page_size, void *workspace, size_t workspace_bytes,
                           int32_t *err_flag, hipStream_t stream, bool use_scratch = false,
                           int64_t slot_stride = 0, int64_t head_stride = -1, const ev::SelectJob *job = nullptr,
                           bool validate_only = false) {
    const bool pg = page_size > 0;  // paged caches: total_slots = pool pages * page_size
    // K/V element strides: [slot][kv_head][dim] unless the caller gives its own
    if (slot_stride == 0 && head_stride == -1) {
        slot_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
        head_stride = head_dim;
    }
    if (!q || !k_cache || !v_cache || !out || !node_start || !parent || !prefix_len || (pg ? !block_table : !kv_start))
        return EV_ERR_NULL;
    if (batch < 0 || batch > EV_MAX_BATCH || total_nodes < 0 || max_nodes < 1 || max_nodes > EV_MAX_NODES ||
        total_slots < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
        (head_dim != 64 && head_dim != 128) || !std::isfinite(sm_scale) || !(sm_scale > 0.f) || window < 0)
        return EV_ERR_SHAPE;
    if (dtype != EV_BF16 && dtype != EV_F32) return EV_ERR_DTYPE;
    if (pg && dtype != EV_BF16) return EV_ERR_DTYPE;
    if (!ev::aligned16(q) || !ev::aligned16(k_cache) || !ev::aligned16(v_cache) || !ev::aligned16(out))
        return EV_ERR_ALIGN;
    // strides: one slot's rows must stay under 2^26 bytes apart (32-bit lane offsets over 16 rows)
    // and every row must start on 16 bytes
    const int64_t esz = dtype == EV_F32 ? 4 : 2;
    if (slot_stride < 1 || head_stride < 0 || slot_stride * esz > (int64_t(1) << 26)) return EV_ERR_SHAPE;
    if ((slot_stride * esz) % 16 || (head_stride * esz) % 16) return EV_ERR_ALIGN;
    const Plan plan = make_plan(batch, max_nodes, num_q_heads, num_kv_heads, head_dim);
    if (use_scratch) {
        if (plan.bytes > kMaxWorkspaceBytes) return EV_ERR_WORKSPACE;  // beyond the static scratch
    } else {
        if (!workspace || workspace_bytes < plan.bytes) return EV_ERR_WORKSPACE;
        if (!ev::aligned16(workspace)) return EV_ERR_ALIGN;
    }
    // stage counts are 32-bit in the kernel (32-key stages bound them from above); token indices
    // of paged sequences are 32-bit
    const int64_t max_tokens = pg ? static_cast<int64_t>(bt_stride) * page_size * batch : total_slots;
    const int64_t max_stages = static_cast<int64_t>(num_kv_heads) * plan.RG * (max_tokens / 32 + 2 * batch);
    if (max_stages >= (int64_t(1) << 31)) return EV_ERR_SHAPE;
    if (pg && static_cast<int64_t>(bt_stride) * page_size >= (int64_t(1) << 31)) return EV_ERR_SHAPE;
    if (validate_only) return EV_OK;
    const ev_status dev = ev::check_device();
    if (dev != EV_OK) return dev;
    if (use_scratch) {  // this device's copy of the static scratch (no allocation)
        const ev_status st = scratch_of_current_device(&workspace);
        if (st != EV_OK) return st;
    }
    if (batch == 0 || total_nodes == 0) return EV_OK;

    const bool f32 = dtype == EV_F32;
    KernelFn fn = pick_kernel(head_dim, plan.RT, f32, pg);
    const int variant = (head_dim == 64 ? 0 : 16) + (f32 ? 8 : 0) + plan.RT + (pg ? 32 : 0);
    const int resident = ev::device_cu_count() * blocks_per_cu(fn, variant);
    int64_t grid = resident;
    if (grid > kMaxGrid) grid = kMaxGrid;
    const int64_t want = (max_stages + 1) / 2;  // about two stages per workgroup at least
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
    args.kv_slot_stride = slot_stride;
    args.kv_head_stride = head_stride;
    args.batch = batch;
    args.total_nodes = total_nodes;
    args.max_nodes = max_nodes;
    args.hq = num_q_heads;
    args.hkv = num_kv_heads;
    args.group = num_q_heads / num_kv_heads;
    args.row_groups = plan.RG;
    args.window = window;
    args.block_table = pg ? block_table : nullptr;
    args.bt_stride = bt_stride;
    args.page_shift = pg ? __builtin_ctz(static_cast<unsigned>(page_size)) : 0;
    args.num_pages = pg ? static_cast<int32_t>(total_slots / page_size) : 0;
    args.scale_log2 = sm_scale * kLog2e;
    args.table = static_cast<int4 *>(workspace);
    args.part = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + plan.table_bytes);
    args.err_flag = err_flag;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, args);
    // Merge launches with chunk-parallel items (head_dim 128) when the batch has so few units that
    // each is cut into many pieces: at most grid / kMergeChunk units.  (Both forms give the same
    // bits; the choice only picks the faster code for the batch's shape.)
    const bool split_items = head_dim == 128 &&
                             static_cast<int64_t>(batch) * num_kv_heads * plan.RG * kMergeChunk <= grid;
    // whole-step calls: the selection pass shares the merge launch when there is one at head_dim
    // 128, and is launched after the attention otherwise
    const bool sel = job && job->rows > 0;
    if (sel && grid > 1 && head_dim == 128) {
        ev::sel::ArgmaxArgs sa{};
        int32_t splits = 0, seg = 0;
        ev::select_plan(job->rows, job->vocab, splits, seg);
        sa.logits = job->logits;
        sa.row_stride = job->row_stride;
        sa.rows = job->rows;
        sa.vocab = job->vocab;
        sa.splits = splits;
        sa.seg = seg;
        sa.pieces = job->pieces;
        const bool sampled = job->temperature > 0.f;
        if (sampled) {
            sa.c = static_cast<float>(1.4426950408889634 / static_cast<double>(job->temperature));
            sa.seed = job->seed;
            sa.offset = job->offset;
        }
        const int pieces = job->rows * splits;
        const int mode = (sampled ? 3 : 1) + (job->dtype == EV_F32 ? 1 : 0);
        const dim3 fgrid(static_cast<unsigned>(pieces + kMergeBlocks));
        const int g32 = static_cast<int>(grid);
        if (split_items) {
            if (f32) hipLaunchKernelGGL((tree_attention_merge_select_kernel<true, true>), fgrid, dim3(256), 0, stream, args, sa, pieces, mode, plan.R, plan.RT, g32);
            else hipLaunchKernelGGL((tree_attention_merge_select_kernel<false, true>), fgrid, dim3(256), 0, stream, args, sa, pieces, mode, plan.R, plan.RT, g32);
        } else {
            if (f32) hipLaunchKernelGGL((tree_attention_merge_select_kernel<true, false>), fgrid, dim3(256), 0, stream, args, sa, pieces, mode, plan.R, plan.RT, g32);
            else hipLaunchKernelGGL((tree_attention_merge_select_kernel<false, false>), fgrid, dim3(256), 0, stream, args, sa, pieces, mode, plan.R, plan.RT, g32);
        }
        return ev::launch_status();
    }
    if (grid > 1) {  // units split over workgroups: combine their pieces
        const dim3 mgrid(static_cast<unsigned>(kMergeBlocks));
        const int g32 = static_cast<int>(grid);
        if (head_dim == 64) {
            if (f32) hipLaunchKernelGGL((tree_attention_merge_kernel<64, true, false>), mgrid, dim3(128), 0, stream, args, plan.R, plan.RT, g32);
            else hipLaunchKernelGGL((tree_attention_merge_kernel<64, false, false>), mgrid, dim3(128), 0, stream, args, plan.R, plan.RT, g32);
        } else if (split_items) {
            if (f32) hipLaunchKernelGGL((tree_attention_merge_kernel<128, true, true>), mgrid, dim3(256), 0, stream, args, plan.R, plan.RT, g32);
            else hipLaunchKernelGGL((tree_attention_merge_kernel<128, false, true>), mgrid, dim3(256), 0, stream, args, plan.R, plan.RT, g32);
        } else {
            if (f32) hipLaunchKernelGGL((tree_attention_merge_kernel<128, true, false>), mgrid, dim3(256), 0, stream, args, plan.R, plan.RT, g32);
            else hipLaunchKernelGGL((tree_attention_merge_kernel<128, false, false>), mgrid, dim3(256), 0, stream, args, plan.R, plan.RT, g32);
        }
    }
    if (sel) {
        const ev_status st = ev::launch_select_pieces(job->logits, job->dtype, job->row_stride, job->rows, job->vocab,
                                                      job->temperature, job->seed, job->offset, job->pieces, stream);
        if (st != EV_OK) return st;
    }
    return ev::launch_status();
}
}  // namespace

namespace ev {
ev_status launch_attention_step(const AttentionCall &c, const SelectJob *job, hipStream_t stream, bool validate_only) {
    return launch_attention(c.q, c.k_cache, c.v_cache, c.out, c.lse, c.node_start, c.parent, c.kv_start, c.prefix_len,
                            c.batch, c.total_nodes, c.max_nodes, c.total_slots, c.num_q_heads, c.num_kv_heads,
                            c.head_dim, c.dtype, c.sm_scale, 0, nullptr, 0, 0, c.workspace, c.workspace_bytes,
                            c.err_flag, stream, false, c.slot_stride, c.head_stride, job, validate_only);
}
}  // namespace ev

extern "C" ev_status ev_tree_attention(const void *q, const void *k_cache, const void *v_cache, void *out, float *lse,
                                       const int32_t *node_start, const int32_t *parent, const int32_t *kv_start,
                                       const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
                                       int32_t max_nodes, int64_t total_slots, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype, float sm_scale,
                                       void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                       hipStream_t stream) {
    return launch_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                            total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                            sm_scale, 0, nullptr, 0, 0, workspace, workspace_bytes, err_flag, stream);
}

extern "C" ev_status ev_tree_attention_noalloc(const void *q, const void *k_cache, const void *v_cache, void *out,
                                               float *lse, const int32_t *node_start, const int32_t *parent,
                                               const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                                               int32_t total_nodes, int32_t max_nodes, int64_t total_slots,
                                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                               ev_dtype dtype, float sm_scale, int32_t *err_flag,
                                               hipStream_t stream) {
    return launch_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                            total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                            sm_scale, 0, nullptr, 0, 0, nullptr, 0, err_flag, stream, true);
}

extern "C" ev_status ev_tree_attention_strided(const void *q, const void *k_cache, const void *v_cache, void *out,
                                               float *lse, const int32_t *node_start, const int32_t *parent,
                                               const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                                               int32_t total_nodes, int32_t max_nodes, int64_t total_slots,
                                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                               int64_t kv_slot_stride, int64_t kv_head_stride, ev_dtype dtype,
                                               float sm_scale, void *workspace, size_t workspace_bytes,
                                               int32_t *err_flag, hipStream_t stream) {
    if (kv_slot_stride < 1 || kv_head_stride < 0) return EV_ERR_SHAPE;
    return launch_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                            total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                            sm_scale, 0, nullptr, 0, 0, workspace, workspace_bytes, err_flag, stream, false,
                            kv_slot_stride, kv_head_stride);
}

extern "C" ev_status ev_tree_attention_window(const void *q, const void *k_cache, const void *v_cache, void *out,
                                              float *lse, const int32_t *node_start, const int32_t *parent,
                                              const int32_t *kv_start, const int32_t *prefix_len, int32_t batch,
                                              int32_t total_nodes, int32_t max_nodes, int64_t total_slots,
                                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                              ev_dtype dtype, float sm_scale, int32_t window, void *workspace,
                                              size_t workspace_bytes, int32_t *err_flag, hipStream_t stream) {
    if (window < 1) return EV_ERR_SHAPE;
    return launch_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                            total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                            sm_scale, window, nullptr, 0, 0, workspace, workspace_bytes, err_flag, stream);
}

extern "C" ev_status ev_tree_attention_paged(const void *q, const void *k_pages, const void *v_pages, void *out,
                                             float *lse, const int32_t *node_start, const int32_t *parent,
                                             const int32_t *block_table, int32_t bt_stride, int32_t page_size,
                                             const int32_t *prefix_len, int32_t batch, int32_t total_nodes,
                                             int32_t max_nodes, int32_t num_pages, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, ev_dtype dtype, float sm_scale,
                                             int32_t window, void *workspace, size_t workspace_bytes,
                                             int32_t *err_flag, hipStream_t stream) {
    if (page_size < 16 || page_size > 65536 || (page_size & (page_size - 1)) || bt_stride < 1 || num_pages < 0)
        return EV_ERR_SHAPE;
    return launch_attention(q, k_pages, v_pages, out, lse, node_start, parent, nullptr, prefix_len, batch,
                            total_nodes, max_nodes, static_cast<int64_t>(num_pages) * page_size, num_q_heads,
                            num_kv_heads, head_dim, dtype, sm_scale, window, block_table, bt_stride, page_size,
                            workspace, workspace_bytes, err_flag, stream);
}
