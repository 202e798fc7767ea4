// Shared helpers of the tav HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tav.h"

namespace tav {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kBlock = 16;     // tokens per paged KV block
constexpr int kMaxNodes = 256; // largest supported tree

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ inline void raise_flag(uint32_t *flags, uint32_t bit)
{
    if (flags)
        atomicOr(flags, bit);
}

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device (0 if there is no usable device).
int device_cu_count();

// Workgroups of `kernel` with `threads` threads one CU of the current device
// holds at once (0 on failure).
int kernel_occupancy(const void *kernel, int threads);

// The KV commit that the walk's workgroups can do themselves right after each
// sequence is decided (null k_tree: none): path row t of sequence b to token
// position prefix_len[b] + t, as kv_commit_path does.
struct CommitArgs {
    const uint16_t *k_tree, *v_tree;
    const int32_t *block_table, *prefix_len;
    uint16_t *k_cache, *v_cache;
    int32_t *commit_slots, *new_prefix_len;
    int32_t num_blocks, max_blocks, Hkv, D;
};

// The launch behind spec_verify_sample and its variants: host checks, plan,
// workspace check, one kernel launch. wor: the without-replacement sibling
// rule; p_rows/q_rows/child_pq non-NULL: the probe variant; commit non-NULL:
// the walk also commits the accepted path (its arguments already checked).
tav_status sv_launch(const float *target_logits, const float *draft_logits,
                     const int32_t *parent, const int32_t *token, int32_t B, int32_t N, int32_t V,
                     double temperature, uint64_t seed, uint64_t offset, int32_t *path,
                     int32_t *n_accepted, int32_t *out_tokens, void *workspace, size_t ws_bytes,
                     uint32_t *dev_flags, void *stream, bool wor, double *p_rows,
                     double *q_rows, double *child_pq, const CommitArgs *commit = nullptr);

} // namespace tav
