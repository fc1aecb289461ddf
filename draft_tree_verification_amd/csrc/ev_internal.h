// ev_internal.h -- helpers shared by the gfx950 kernels of the verification-step library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ev.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));

namespace ev {

// ---------------------------------------------------------------- host side
ev_status check_device();         // current device must be gfx950
int device_cu_count();            // compute units of the current device (cached per device)
int current_device();
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline ev_status launch_status() { return hipGetLastError() == hipSuccess ? EV_OK : EV_ERR_HIP; }

// The per-node selection pass of the fused step (ev_argmax.hip): argmax (temperature 0) or the
// sampled draw of every row, each row cut into select_splits() pieces whose winners, packed as
// (order key << 32 | ~index), go to pieces[row * splits + piece].  Arguments already validated.
int select_splits(int32_t rows, int32_t vocab);
ev_status launch_select_pieces(const void *logits, ev_dtype dtype, int64_t row_stride, int32_t rows, int32_t vocab,
                               float temperature, uint64_t seed, uint64_t offset, unsigned long long *pieces,
                               hipStream_t stream);
void select_plan(int32_t rows, int32_t vocab, int32_t &splits, int32_t &seg);

// The whole-step call (ev_verify_step): its attention arguments, as ev_tree_attention_strided
// takes them, and its selection pass, which the attention launcher runs beside the merge of
// split units when it can (one launch) and launches after the attention otherwise.
struct AttentionCall {
    const void *q, *k_cache, *v_cache;
    void *out;
    float *lse;
    const int32_t *node_start, *parent, *kv_start, *prefix_len;
    int32_t batch, total_nodes, max_nodes;
    int64_t total_slots;
    int32_t num_q_heads, num_kv_heads, head_dim;
    int64_t slot_stride, head_stride;
    ev_dtype dtype;
    float sm_scale;
    void *workspace;
    size_t workspace_bytes;
    int32_t *err_flag;
};
struct SelectJob {
    const void *logits;
    ev_dtype dtype;
    int64_t row_stride;
    int32_t rows, vocab;
    float temperature;
    uint64_t seed, offset;
    unsigned long long *pieces;  // [rows * select_splits(rows, vocab)]
};
// Checks every attention argument before its first launch (nothing is launched on an error);
// with validate_only, returns after the checks (no device call).  job: the selection pass to run
// with it (arguments already checked), or NULL.
ev_status launch_attention_step(const AttentionCall &c, const SelectJob *job, hipStream_t stream,
                                bool validate_only = false);

// ---------------------------------------------------------------- device side
__device__ __forceinline__ u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }

// Streaming 16-byte load: data read exactly once, so keep it out of the caches' way.
__device__ __forceinline__ u32x4_t ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one dword, low half first: one
// v_cvt_pk_bf16_f32.  (Built from a bf16x2 vector: element-wise bit_casts out of u32x4
// vectors were mis-translated by the compiler, converting only the first element.)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f2bf_bits(float x) { return pack_bf16x2(x, 0.f) & 0xFFFFu; }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ f32x4_t ld16f(const float *p) { return *reinterpret_cast<const f32x4_t *>(p); }
__device__ __forceinline__ f32x4_t ld16f_stream(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
}

// Eight fp32 values (two 16-byte loads) -> eight bf16 in four dwords.
__device__ __forceinline__ u32x4_t f32x8_to_bf16x8(f32x4_t a, f32x4_t b) {
    return u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                   pack_bf16x2(b[2], b[3])};
}

// Cross-workgroup publication without L2 flushes.  Agent-scope relaxed atomic stores/loads are
// sc1 accesses (coherent across the XCDs' separate L2s); a writer drains them with vm_wait()
// before its arrival counter's atomic, and the reader issues its sc1 loads after observing
// the counter, so no buffer_wbl2 / buffer_inv is needed.
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (Whole-vector bit casts only: casting single elements out of vectors was mis-translated.)
__device__ __forceinline__ void st_agent4(float *p, f32x4_t v) {
    const u64x2_t w = __builtin_bit_cast(u64x2_t, v);
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    __hip_atomic_store(q, w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4_t ld_agent4(const float *p) {
    uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<float *>(p));
    const u64x2_t w = {__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
    return __builtin_bit_cast(f32x4_t, w);
}
__device__ __forceinline__ int atomic_add_agent(int32_t *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ void flag_error(int32_t *err_flag, int32_t bits) {
    if (err_flag && bits) atomicOr(err_flag, bits);
}

}  // namespace ev
