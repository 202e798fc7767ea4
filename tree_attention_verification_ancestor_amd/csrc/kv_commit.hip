// kv_commit_path: copy the accepted path's K/V rows into the paged cache.
//
// Only the accepted root-to-node path survives verification; everything else
// the tree produced is dropped and the sequence continues from the accepted
// length (radar-34b blog §5, KV-cache management; jisaku.com glossary,
// KV-cache section on pruning and rollback).
//
// Path row t of sequence b goes to token position prefix_len[b] + t. K blocks
// are token-major ([blk][h][16][D]): a row is one contiguous D-vector. V
// blocks are feature-major ([blk][h][D][16]): a row is D values 32 bytes
// apart. One thread moves 8 features (16 bytes) of one (b, t, kv head) row.

#include "common.h"

namespace tav {
namespace {

template <int D>
__global__ __launch_bounds__(256) void kv_commit_kernel(
    const uint16_t *__restrict__ k_tree, const uint16_t *__restrict__ v_tree,
    const int32_t *__restrict__ path, const int32_t *__restrict__ n_accepted, int32_t num_blocks,
    const int32_t *__restrict__ block_table, int32_t max_blocks,
    const int32_t *__restrict__ prefix_len, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int32_t N, int32_t Hkv, int32_t *__restrict__ commit_slots,
    int32_t *__restrict__ new_prefix_len, uint32_t *flags)
{
    constexpr int CPR = D / 8; // 16-byte chunks per row
    const int b = blockIdx.y;
    // this thread's first work item's path entry (t0 < N always)
    const int64_t it0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int t0 = (int)std::min<int64_t>(it0 / ((int64_t)CPR * Hkv), N - 1);
    const int32_t node0 = path[(int64_t)b * N + t0];
    const int32_t m = n_accepted[b];
    const int32_t L = prefix_len[b];
    const bool m_ok = m >= 0 && m < N;

    // Slot bookkeeping: one thread per path entry.
    if (blockIdx.x == 0) {
        for (int t = threadIdx.x; t < N; t += blockDim.x) {
            int32_t slot = -1;
            if (m_ok && t <= m) {
                const int64_t pos = (int64_t)L + t;
                const int64_t lb = pos / kBlock;
                if (L >= 0 && lb < max_blocks) {
                    const int32_t blk = block_table[(int64_t)b * max_blocks + lb];
                    if (blk >= 0 && blk < num_blocks)
                        slot = blk * kBlock + (int32_t)(pos % kBlock);
                }
            }
            commit_slots[(int64_t)b * N + t] = slot;
        }
        if (threadIdx.x == 0) {
            new_prefix_len[b] = m_ok ? L + m + 1 : L;
            if (!m_ok)
                raise_flag(flags, TAV_FLAG_BAD_PARENT);
        }
    }
    if (!m_ok || L < 0)
        return;

    // Row copies: work item = (t, kv head, chunk). The launch covers every
    // t < N, so each thread reads its path entry alongside n_accepted and
    // prefix_len instead of after them.
    const int64_t items = (int64_t)(m + 1) * Hkv * CPR;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(it % CPR);
        const int h = (int)((it / CPR) % Hkv);
        const int t = (int)(it / ((int64_t)CPR * Hkv));
        const int32_t node = t == t0 ? node0 : path[(int64_t)b * N + t];
        if (node < 0 || node >= N) {
            raise_flag(flags, TAV_FLAG_BAD_PARENT);
            continue;
        }
        const int64_t pos = (int64_t)L + t;
        const int64_t lb = pos / kBlock;
        if (lb >= max_blocks) {
            raise_flag(flags, TAV_FLAG_CAPACITY);
            continue;
        }
        const int32_t blk = block_table[(int64_t)b * max_blocks + lb];
        if (blk < 0 || blk >= num_blocks) {
            raise_flag(flags, TAV_FLAG_BAD_BLOCK);
            continue;
        }
        const int s = (int)(pos % kBlock);
        const int64_t src = (((int64_t)b * N + node) * Hkv + h) * D + c * 8;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(k_tree + src);
        *reinterpret_cast<u32x4 *>(k_cache + (((int64_t)blk * Hkv + h) * kBlock + s) * D + c * 8) = kv;
        const u32x4 vv = *reinterpret_cast<const u32x4 *>(v_tree + src);
        uint16_t *vdst = v_cache + (((int64_t)blk * Hkv + h) * D + c * 8) * kBlock + s;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vdst[e * kBlock] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
}


// ---------------------------------------------------------------------------
// kv_commit_inplace: zero-copy rollback. The tree's rows were written at
// positions prefix_len[b] + i (node i); after verification position L + t
// takes node path[t]'s row for t <= m, the length becomes L + m + 1 and the
// positions past it are abandoned (radar-34b blog §5: branching and rollback
// through block-table operations, no copy; jisaku.com glossary, KV-cache
// section: prune what is off the accepted path, roll back to the right
// position). Only rows whose node index differs from their path position
// move, so a chain accepted from the root moves nothing.
//
// One workgroup per (KV head, sequence): no other workgroup touches its
// bytes. A destination can be an earlier step's source (path[t'] = t for some
// t' < t), so every moving row is read into registers first and written
// after a barrier.
constexpr int kInplaceThreads = 512;

template <int D>
__global__ __launch_bounds__(kInplaceThreads) void kv_commit_inplace_kernel(
    const int32_t *__restrict__ path, const int32_t *__restrict__ n_accepted, int32_t num_blocks,
    const int32_t *__restrict__ block_table, int32_t max_blocks,
    const int32_t *__restrict__ prefix_len, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int32_t N, int32_t Hkv, int32_t *__restrict__ commit_slots,
    int32_t *__restrict__ new_prefix_len, uint32_t *flags)
{
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    constexpr int kItems = (kMaxNodes * CPR + kInplaceThreads - 1) / kInplaceThreads;
    const int h = blockIdx.x, b = blockIdx.y;
    const int32_t m = n_accepted[b];
    const int32_t L = prefix_len[b];
    const bool m_ok = m >= 0 && m < N;
    const bool cap_ok = L >= 0 && ((int64_t)L + N - 1) / kBlock < max_blocks;
    const int32_t *bt = block_table + (int64_t)b * max_blocks;
    // physical block of position pos, or -1 if the entry is out of range
    auto block_of = [&](int64_t pos) __attribute__((always_inline)) {
        const int32_t blk = bt[pos / kBlock];
        return (blk >= 0 && blk < num_blocks) ? blk : -1;
    };

    if (h == 0) {
        for (int t = threadIdx.x; t < N; t += blockDim.x) {
            int32_t slot = -1;
            if (m_ok && cap_ok && t <= m) {
                const int64_t pos = (int64_t)L + t;
                const int32_t blk = block_of(pos);
                if (blk >= 0)
                    slot = blk * kBlock + (int32_t)(pos % kBlock);
            }
            commit_slots[(int64_t)b * N + t] = slot;
        }
        if (threadIdx.x == 0) {
            new_prefix_len[b] = m_ok ? L + m + 1 : L;
            if (!m_ok)
                raise_flag(flags, TAV_FLAG_BAD_PARENT);
            if (!cap_ok)
                raise_flag(flags, TAV_FLAG_CAPACITY);
        }
    }
    if (!m_ok || !cap_ok)
        return;

    // phase 1: read every moving row chunk (item = (t, chunk c))
    u32x4 kreg[kItems], vreg[kItems];
    int32_t dst_blk[kItems];
    int dst_s[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        dst_blk[i] = -1;
        const int it = threadIdx.x + i * kInplaceThreads;
        const int t = it / CPR, c = it % CPR;
        if (t > m)
            continue;
        const int32_t node = path[(int64_t)b * N + t];
        if (node < 0 || node >= N) {
            raise_flag(flags, TAV_FLAG_BAD_PARENT);
            continue;
        }
        if (node == t)
            continue;   // already in place
        const int64_t src = (int64_t)L + node, dst = (int64_t)L + t;
        const int32_t sb = block_of(src), db = block_of(dst);
        if (sb < 0 || db < 0) {
            raise_flag(flags, TAV_FLAG_BAD_BLOCK);
            continue;
        }
        const int ss = (int)(src % kBlock);
        kreg[i] = *reinterpret_cast<const u32x4 *>(
            k_cache + (((int64_t)sb * Hkv + h) * kBlock + ss) * D + c * 8);
        const uint16_t *vs = v_cache + (((int64_t)sb * Hkv + h) * D + c * 8) * kBlock + ss;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)vs[(2 * e) * kBlock] | ((uint32_t)vs[(2 * e + 1) * kBlock] << 16);
        vreg[i] = u32x4{w[0], w[1], w[2], w[3]};
        dst_blk[i] = db;
        dst_s[i] = (int)(dst % kBlock);
    }
    __syncthreads();   // every source read before any destination is written
    // phase 2: write them at their path positions
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        if (dst_blk[i] < 0)
            continue;
        const int it = threadIdx.x + i * kInplaceThreads;
        const int c = it % CPR;
        const int32_t db = dst_blk[i];
        const int ds = dst_s[i];
        *reinterpret_cast<u32x4 *>(k_cache + (((int64_t)db * Hkv + h) * kBlock + ds) * D + c * 8) = kreg[i];
        uint16_t *vd = v_cache + (((int64_t)db * Hkv + h) * D + c * 8) * kBlock + ds;
        const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vd[e * kBlock] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
}

} // namespace
} // namespace tav

extern "C" tav_status kv_commit_path(const uint16_t *k_tree, const uint16_t *v_tree,
                                     const int32_t *path, const int32_t *n_accepted,
                                     int32_t num_blocks, const int32_t *block_table,
                                     int32_t max_blocks, const int32_t *prefix_len,
                                     uint16_t *k_cache, uint16_t *v_cache, int32_t B, int32_t N,
                                     int32_t Hkv, int32_t D, int32_t block_size,
                                     int32_t *commit_slots, int32_t *new_prefix_len,
                                     uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!k_tree || !v_tree || !path || !n_accepted || !block_table || !prefix_len || !k_cache ||
        !v_cache || !commit_slots || !new_prefix_len)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1)
        return TAV_ERR_ARG;
    if (block_size != kBlock || (D != 64 && D != 128) || N > kMaxNodes)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 2))
        return TAV_ERR_ARG;
    // Enough blocks per sequence to spread the longest path's rows.
    const int64_t items = (int64_t)N * Hkv * (D / 8);
    const int gx = (int)std::min<int64_t>(ceil_div(items, 256), 64);
    dim3 grid(gx, B);
    if (D == 128)
        hipLaunchKernelGGL(kv_commit_kernel<128>, grid, dim3(256), 0, as_stream(stream), k_tree,
                           v_tree, path, n_accepted, num_blocks, block_table, max_blocks,
                           prefix_len, k_cache, v_cache, N, Hkv, commit_slots, new_prefix_len,
                           dev_flags);
    else
        hipLaunchKernelGGL(kv_commit_kernel<64>, grid, dim3(256), 0, as_stream(stream), k_tree,
                           v_tree, path, n_accepted, num_blocks, block_table, max_blocks,
                           prefix_len, k_cache, v_cache, N, Hkv, commit_slots, new_prefix_len,
                           dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}

extern "C" tav_status kv_commit_inplace(const int32_t *path, const int32_t *n_accepted,
                                        int32_t num_blocks, const int32_t *block_table,
                                        int32_t max_blocks, const int32_t *prefix_len,
                                        uint16_t *k_cache, uint16_t *v_cache, int32_t B, int32_t N,
                                        int32_t Hkv, int32_t D, int32_t block_size,
                                        int32_t *commit_slots, int32_t *new_prefix_len,
                                        uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!path || !n_accepted || !block_table || !prefix_len || !k_cache || !v_cache ||
        !commit_slots || !new_prefix_len)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1)
        return TAV_ERR_ARG;
    if (block_size != kBlock || (D != 64 && D != 128) || N > kMaxNodes || B > 65535 ||
        Hkv > (1 << 30))
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 2))
        return TAV_ERR_ARG;
    dim3 grid(Hkv, B);
    if (D == 128)
        hipLaunchKernelGGL(kv_commit_inplace_kernel<128>, grid, dim3(kInplaceThreads), 0,
                           as_stream(stream), path, n_accepted, num_blocks, block_table,
                           max_blocks, prefix_len, k_cache, v_cache, N, Hkv, commit_slots,
                           new_prefix_len, dev_flags);
    else
        hipLaunchKernelGGL(kv_commit_inplace_kernel<64>, grid, dim3(kInplaceThreads), 0,
                           as_stream(stream), path, n_accepted, num_blocks, block_table,
                           max_blocks, prefix_len, k_cache, v_cache, N, Hkv, commit_slots,
                           new_prefix_len, dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}
