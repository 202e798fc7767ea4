// tree_attn_verify: GQA flash-decoding tree attention over a paged prefix.
//
// Every candidate node attends to the whole committed prefix plus the tree
// nodes on its own root-to-node path (jisaku.com glossary, tree-attention
// section; radar-34b blog §3). All candidates are scored in one pass (LLM
// Primer ch. 9, §9.1). The prefix comes from a paged cache through a block
// table (radar-34b blog §5).
//
// Work decomposition. For one sequence b and KV head kvh, the N*G query rows
// (node i, head g of the group) share every key and value, so a workgroup
// takes a block of 32*NW of those rows and one split of the prefix; the K/V
// tiles it stages in LDS are read by all its rows (the tree's queries are the
// M of a small dense contraction, which is what makes MFMA pay here).
//
// Per 64-key tile and wave (32 query rows):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = the wave's
//                 Q^T held in registers. The accumulator gives each lane one
//                 query column and 16 keys of each 32-key tile.
//   softmax       online, per lane; the running max is only moved when a tile
//                 exceeds it by more than 2^8 in probability, so the O rescale
//                 is rare; exp2 with the scale folded into one FMA.
//   O^T += V^T P^T  v_mfma_f32_32x32x16_f16. P^T is the S^T accumulator
//                 itself: the key order inside each 32-key tile is permuted
//                 (rows 4..7 and 8..11 of the tile swapped, and so on) so that
//                 each lane's 16 accumulator values are exactly the 8+8
//                 consecutive keys the PV B operand needs. V^T comes from
//                 feature-major V blocks, so its A operand is one 16-byte LDS
//                 read. This contraction runs in fp16, not bf16: bf16 V
//                 converts to fp16 exactly (within fp16's range) while staging,
//                 and fp16 keeps 11 significant bits of each weight where bf16
//                 keeps 8, which the output tolerance needs when attention
//                 falls on a few keys. Weights carry a 2^7 bias so small ones
//                 stay clear of fp16 subnormals; the bias cancels in O/l.
// Tiles are double-buffered in LDS. Prefix tiles move from HBM straight into
// LDS (global_load_lds_dwordx4: 16 bytes per lane, no staging registers), a
// whole tile ahead of the MFMAs that use them; one pass per tile then turns the
// tile's V from bf16 into fp16 in place and zeroes keys past the prefix. The
// few tree tiles go through registers (their V rows need a transpose). Splits
// of the prefix write unnormalised partials (O, max, sum) that a combine
// kernel merges with log-sum-exp; the last split also takes the tree tiles
// (keys masked by the ancestor bitmask).

#include <algorithm>

#include "common.h"

namespace tav {
namespace {

constexpr int kKT = 64;              // keys per tile
constexpr int kMaxSplitBlocks = 2048; // block-table entries one split stages in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWeightBias = 7.0f;  // log2 of the bias on the fp16 weights

template <int D, int NW, int CT>
struct Cfg {
    static constexpr int kThreads = NW * 64;
    static constexpr int kWaveRows = CT * 32;            // query rows per wave
    static constexpr int kRows = NW * kWaveRows;         // query rows per workgroup
    static constexpr int kKSteps = D / 16;
    static constexpr int kDTiles = D / 32;
    static constexpr int kCpr = D / 8;                   // 16-byte chunks per row
    static constexpr int kKRow = D * 2;                  // K row in LDS (16-byte chunks swizzled)
    static constexpr int kKTileBytes = kKT * kKRow;
    static constexpr int kVTileBytes = kKT * D * 2;
    static constexpr int kBufBytes = kKTileBytes + kVTileBytes;
    static constexpr int kChunks = kKT * kCpr;           // 16-byte chunks per K (or V) tile
    static constexpr int kLoadsPerWave = kChunks / 64 / NW;   // direct loads per wave per K (or V) tile
    static constexpr int kChPerThread = kChunks / kThreads;
    static_assert(kChunks % kThreads == 0, "tile chunks must split evenly");
    static_assert(kLoadsPerWave * 64 * NW == kChunks, "direct loads must split evenly");
};

struct AttnArgs {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len;
    const uint64_t *mask;
    float *out, *part_o, *part_ml;
    uint32_t *flags;
    int32_t num_blocks, max_blocks, max_prefix_len;
    int32_t B, N, Hq, Hkv, G, NG, W;
    int32_t RB, S, KS;       // row blocks, splits, KV streams (B*Hkv*S)
    float c;                 // scale * log2(e)
    float th;                // lazy-rescale threshold in raw score units (8 / c)
};

// Row r of a 32-row MFMA tile holds key perm(r): bits 2 and 3 of r swapped.
__device__ __forceinline__ int perm32(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS byte offset of chunk cc (8 features) of MFMA row `row` of a K tile.
// Row 32t + r holds key 32t + perm32(r), so lane r of a wave reads row r. The
// chunk position within a row is XOR-swizzled by k_swz(row) so the lanes that
// one LDS cycle serves (8 or 16 for a 16-byte read) hit distinct bank groups:
// 256-byte rows (D = 128) use the row's low four bits; 128-byte rows (D = 64)
// pair up (rows r and r+2 share banks), so bit 3 breaks the tie of rows 8
// apart.
template <int D>
__device__ __forceinline__ int k_swz(int row)
{
    return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

template <int D>
__device__ __forceinline__ int k_off_row(int row, int cc)
{
    return row * (D * 2) + ((cc ^ k_swz<D>(row)) << 4);
}

// The same for key k of the tile.
template <int D>
__device__ __forceinline__ int k_off(int k, int cc)
{
    return k_off_row<D>((k & ~31) | perm32(k & 31), cc);
}

// One direct HBM -> LDS load: lane l's 16 bytes at base + off land at LDS
// byte address lds_addr + 16 l (lds_addr is the same for the whole wave).
// Issued as inline assembly: the compiler then neither makes later LDS reads
// of the other tile buffer wait for it nor reasons about what it writes; the
// code that reads the destination waits for it explicitly with
// lds_loads_landed().
__device__ __forceinline__ void load_lds16(const void *base, uint32_t off, uint32_t lds_addr)
{
    const char *src = static_cast<const char *>(base) + off;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}

// LDS byte address of a __shared__ object (folded at compile time).
#define TAV_LDS_ADDR(obj) ((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(obj))

// Every direct load this workgroup issued has landed in LDS and is visible to
// all its waves.
__device__ __forceinline__ void lds_loads_landed()
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Two bf16 values (low, high half of w) to two fp16 values, round to nearest.
// Exact while |v| < 65520; larger magnitudes become infinite.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w)
{
    const f32x2 f = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// LDS byte offset of keys [8*hh, 8*hh+8) of feature d in 16-key block bi of a
// V tile. A feature's two halves share 32 bytes; which half comes first
// flips with bits 2 and 3 of d, so the 8 or 16 consecutive features one LDS
// cycle serves land in distinct bank groups.
__device__ __forceinline__ int v_slot(int d, int hh) { return hh ^ ((d >> 2) & 1) ^ ((d >> 3) & 1); }

template <int D>
__device__ __forceinline__ int v_off(int bi, int d, int hh)
{
    return bi * (D * 32) + d * 32 + (v_slot(d, hh) << 4);
}

template <int D, int NW, int CT>
__global__ __launch_bounds__(NW * 64, 2) void tree_attn_kernel(AttnArgs a)
{
    using C = Cfg<D, NW, CT>;
    // Two tile buffers as separate objects: with the loop unrolled by two,
    // every access names its buffer statically, so the compiler can tell the
    // next tile's direct loads from the current tile's LDS reads and does not
    // make the reads wait for those loads.
    __shared__ __attribute__((aligned(16))) char lds_a[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) char lds_b[C::kBufBytes];
    __shared__ __attribute__((aligned(16))) int32_t s_bt[kMaxSplitBlocks];   // this split's physical block ids

    // ---- which (sequence, kv head, split, row block) ------------------------
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int rb = slot % a.RB;
    const int ks = (slot / a.RB) * 8 + xcd;     // row blocks of one KV stream share an XCD
    if (ks >= a.KS)
        return;
    const int s = ks % a.S;
    const int bh = ks / a.S;
    const int b = bh / a.Hkv;
    const int kvh = bh % a.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: SGPR arithmetic
    const int col = lane & 31;      // query column of this lane within a 32-row tile
    const int hh = lane >> 5;       // which half of the K dimension this lane feeds

    int L = a.prefix_len[b];
    if (L < 0 || L > a.max_prefix_len || L > a.max_blocks * kBlock) {
        if (tid == 0)
            raise_flag(a.flags, TAV_FLAG_CAPACITY);
        L = std::max(0, std::min(L, std::min(a.max_prefix_len, a.max_blocks * kBlock)));
    }
    const int Tb = (L + kKT - 1) / kKT;
    const int t_begin = (int)((int64_t)s * Tb / a.S);
    const int t_end = (int)((int64_t)(s + 1) * Tb / a.S);
    const int n_pre = t_end - t_begin;
    const int n_tree = (s == a.S - 1) ? (a.N + kKT - 1) / kKT : 0;
    const int n_tiles = n_pre + n_tree;
    // The split's block-table slice, validated once: later tiles look block
    // ids up in LDS instead of waiting on a dependent global load per tile.
    {
        const int32_t *bt = a.block_table + (int64_t)b * a.max_blocks;
        const int nb = std::min(n_pre * (kKT / kBlock), (L + kBlock - 1) / kBlock - t_begin * (kKT / kBlock));
        for (int i = tid; i < nb; i += C::kThreads) {
            int32_t blk = bt[t_begin * (kKT / kBlock) + i];
            if (blk < 0 || blk >= a.num_blocks) {
                raise_flag(a.flags, TAV_FLAG_BAD_BLOCK);
                blk = -1;
            }
            s_bt[i] = blk;
        }
    }
    const int blk0 = t_begin * (kKT / kBlock);

    // ---- this lane's query rows: one per 32-row column tile --------------------
    int node[CT], head[CT];
    bool row_ok[CT];
    bf16x8 qf[CT][C::kKSteps];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const int row = rb * C::kRows + wave * C::kWaveRows + 32 * c + col;
        row_ok[c] = row < a.NG;
        node[c] = row_ok[c] ? row / a.G : 0;
        head[c] = kvh * a.G + (row_ok[c] ? row % a.G : 0);
        const uint16_t *qrow = a.q + (((int64_t)b * a.N + node[c]) * a.Hq + head[c]) * D;
#pragma unroll
        for (int k = 0; k < C::kKSteps; ++k) {
            u32x4 v = {0, 0, 0, 0};
            if (row_ok[c])
                v = *reinterpret_cast<const u32x4 *>(qrow + 16 * k + 8 * hh);
            qf[c][k] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- staging -----------------------------------------------------------
    // Prefix tile: each wave issues kLoadsPerWave direct loads for K and as
    // many for V; load j fills LDS chunks [64j, 64j+64) of the tile in lane
    // order. The chunks of one load always come from a single 16-key paged
    // block (4 or 8 whole MFMA rows of K, whose keys differ only in their low
    // bits; or 64 feature halves of one V block), so the block's address is a
    // wave-uniform base and each lane adds a byte offset below 4 KB. A block
    // past the prefix or a bad block reads the cache's first block instead;
    // those keys' scores are masked and their V entries zeroed later.
    auto issue_prefix_tile = [&](int it, uint32_t kl) __attribute__((always_inline)) {
        const uint32_t vl = kl + C::kKTileBytes;
        const int p0 = (t_begin + it) * kKT;
        // the tile's four block ids in one 16-byte LDS read (tiles start on a
        // multiple of four blocks); entries past the prefix are never used
        const u32x4 ids = *reinterpret_cast<const u32x4 *>(&s_bt[it * (kKT / kBlock)]);
        const uint32_t idv[4] = {ids.x, ids.y, ids.z, ids.w};
        uint64_t kb[4], vb[4];   // uniform block base addresses
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int blk = (int)__builtin_amdgcn_readfirstlane(idv[bb]);
            const bool ok = p0 + bb * kBlock < L && blk >= 0;
            const int64_t e = ok ? ((int64_t)blk * a.Hkv + kvh) * (kBlock * D) : 0;
            kb[bb] = (uint64_t)(uintptr_t)(a.k_cache + e);
            vb[bb] = (uint64_t)(uintptr_t)(a.v_cache + e);
        }
        auto pick = [&](const uint64_t (&t)[4], int bb) __attribute__((always_inline)) -> const void * {
            return (const void *)(uintptr_t)(bb == 0 ? t[0] : bb == 1 ? t[1] : bb == 2 ? t[2] : t[3]);
        };
#pragma unroll
        for (int i = 0; i < C::kLoadsPerWave; ++i) {
            const int j = wave + i * NW;
            const int row0 = j * 64 / C::kCpr;                   // first MFMA row of this load
            const int bb = ((row0 & ~31) | perm32(row0 & 31)) >> 4;
            const int q = j * 64 + lane;
            const int row = q / C::kCpr, pos = q % C::kCpr;
            const int cc = pos ^ k_swz<D>(row);
            const int key = (row & ~31) | perm32(row & 31);
            const uint32_t off = (uint32_t)(((key & 15) * D + cc * 8) * 2);
            load_lds16(pick(kb, bb), off, kl + j * 1024u);
        }
#pragma unroll
        for (int i = 0; i < C::kLoadsPerWave; ++i) {
            const int j = wave + i * NW;
            const int bb = j * 64 / (2 * D);
            const int q = j * 64 + lane;
            const int rem = q % (2 * D);
            const int d = rem >> 1, pos = rem & 1;
            const int h2 = v_slot(d, pos);   // v_slot is its own inverse in hh
            const uint32_t off = (uint32_t)((d * kBlock + h2 * 8) * 2);
            load_lds16(pick(vb, bb), off, vl + j * 1024u);
        }
    };

    // bf16 -> fp16 of a landed prefix tile's V, in place; keys past the prefix
    // become zero (unused cache slots may hold anything).
    auto convert_prefix_v = [&](int it, char *buf) __attribute__((always_inline)) {
        char *vl = buf + C::kKTileBytes;
        const int p0 = (t_begin + it) * kKT;
#pragma unroll
        for (int r = 0; r < C::kChPerThread; ++r) {
            const int q = tid + r * C::kThreads;
            u32x4 *pv = reinterpret_cast<u32x4 *>(vl + q * 16);
            const u32x4 v = *pv;
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
            const int bi = q / (2 * D), rem = q % (2 * D);
            const int d = rem >> 1, pos = rem & 1;
            const int h2 = v_slot(d, pos);   // v_slot is its own inverse in hh
            const int valid = L - (p0 + bi * 16 + h2 * 8);
            if (valid < 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (e >= valid)
                        w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            }
            u32x4 h;
            h.x = bf16x2_to_f16x2(w[0]);
            h.y = bf16x2_to_f16x2(w[1]);
            h.z = bf16x2_to_f16x2(w[2]);
            h.w = bf16x2_to_f16x2(w[3]);
            *pv = h;
        }
    };

    // Tree tile: through registers. K rows go to their MFMA rows; V rows are
    // feature-contiguous, so 8 features of a key are scattered (as fp16).
    auto stage_tree_tile = [&](int it, char *kl) __attribute__((always_inline)) {
        char *vl = kl + C::kKTileBytes;
        const int j0 = (it - n_pre) * kKT;
#pragma unroll 1   // keeps one chunk's registers live
        for (int r = 0; r < C::kChPerThread; ++r) {
            const int ci = tid + r * C::kThreads;
            const int k = ci / C::kCpr, cc = ci % C::kCpr;
            const int j = j0 + k;
            u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (j < a.N) {
                const int64_t src = (((int64_t)b * a.N + j) * a.Hkv + kvh) * D + cc * 8;
                kv = *reinterpret_cast<const u32x4 *>(a.k_tree + src);
                vv = *reinterpret_cast<const u32x4 *>(a.v_tree + src);
            }
            *reinterpret_cast<u32x4 *>(kl + k_off<D>(k, cc)) = kv;
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
            const int bi = k >> 4, kb = k & 15;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const uint32_t h = bf16x2_to_f16x2(w[e >> 1]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int d = cc * 8 + e + u;
                    *reinterpret_cast<uint16_t *>(vl + v_off<D>(bi, d, kb >> 3) + (kb & 7) * 2) =
                        (uint16_t)(h >> (u * 16));
                }
            }
        }
    };

    // ---- accumulators --------------------------------------------------------
    f32x16 oacc[C::kDTiles][CT];
#pragma unroll
    for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                oacc[m][c][e] = 0.f;
    float m_used[CT];   // raw-score max the exponentials are taken against
    float lsum[CT];     // this lane's share of the softmax denominator
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        m_used[c] = -INFINITY;
        lsum[c] = 0.f;
    }
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    __syncthreads();   // s_bt ready
    if (n_tiles > 0) {
        if (n_pre > 0)
            issue_prefix_tile(0, TAV_LDS_ADDR(lds_a));
        else
            stage_tree_tile(0, lds_a);
    }
    lds_loads_landed();
    if (n_pre > 0) {
        convert_prefix_v(0, lds_a);
        __syncthreads();
    }

    // One tile: compute on `cur` while the next tile streams into `nxt`.
    auto tile_step = [&](int it, char *cur, char *nxt, uint32_t nxt_addr) __attribute__((always_inline)) {
        if (it + 1 < n_pre)
            issue_prefix_tile(it + 1, nxt_addr);

        const char *kl = cur;
        const char *vl = kl + C::kKTileBytes;

        // S^T = K Q^T for two 32-key tiles and every column tile; each K
        // fragment read from LDS feeds CT MFMAs
        f32x16 sacc[2][CT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sacc[t][c][e] = 0.f;
#pragma unroll
        for (int k = 0; k < C::kKSteps; ++k) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 av =
                    *reinterpret_cast<const bf16x8 *>(kl + k_off_row<D>(32 * t + col, 2 * k + hh));
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    sacc[t][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[c][k], sacc[t][c], 0, 0, 0);
            }
            // keep at most two k-steps of K fragments in flight (registers)
            if (k & 1)
                __builtin_amdgcn_sched_barrier(0);
        }

        // masks: ragged prefix tail, or ancestor bits of the tree tile
        // Accumulator entry (t, 4i+j) is key 32t + 16(i>>1) + 8hh + 4(i&1) + j;
        // the lane-dependent 8hh is taken out once so the rest are constants.
        if (it >= n_pre) {
            const int tt = it - n_pre;
            const int nlim = a.N - tt * kKT - 8 * hh;   // keys at or past it are not nodes
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                uint64_t mw = 1;
                if (row_ok[c])
                    mw = a.mask[((int64_t)b * a.N + node[c]) * a.W + tt];
                mw >>= 8 * hh;
                const uint32_t mlo = (uint32_t)mw, mhi = (uint32_t)(mw >> 32);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int kr = 16 * (i >> 1) + 4 * (i & 1) + j;   // < 32
                            const uint32_t word = t ? mhi : mlo;
                            const bool ok = (32 * t + kr < nlim) && ((word >> kr) & 1u);
                            if (!ok)
                                sacc[t][c][4 * i + j] = -INFINITY;
                        }
            }
        } else {
            const int p0 = (t_begin + it) * kKT;
            if (p0 + kKT > L) {
                const int plim = L - p0 - 8 * hh;
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int kr = 32 * t + 16 * (i >> 1) + 4 * (i & 1) + j;
                                if (kr >= plim)
                                    sacc[t][c][4 * i + j] = -INFINITY;
                            }
            }
        }

        // online softmax with lazy rescaling, per column tile
        f16x8 pb[CT][2][2];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            float mt = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    mt = fmaxf(mt, sacc[t][c][e]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const bool need = mt > m_used[c] + a.th;
            if (__any(need)) {
                const float mnew = need ? mt : m_used[c];
                const float alpha =
                    (m_used[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_used[c] - mnew) * a.c);
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        oacc[m][c][e] *= alpha;
                lsum[c] *= alpha;
                m_used[c] = mnew;
            }
            // weights 2^(s*c - m*c + 7): at most 2^15 after the lazy threshold
            const float moff = (m_used[c] == -INFINITY) ? 0.f : m_used[c] * a.c - kWeightBias;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[t][c][8 * h2 + e], a.c, -moff));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[t][c][8 * h2 + e + 1], a.c, -moff));
                        const f32x2 pf = {p0, p1};
                        const f16x2 pk = __builtin_convertvector(pf, f16x2);
                        pb[c][t][h2][e] = pk[0];
                        pb[c][t][h2][e + 1] = pk[1];
                        lsum[c] = __builtin_amdgcn_fdot2(pk, ones, lsum[c], false);
                    }
                }
        }

        // O^T += V^T P^T; each V fragment read from LDS feeds CT MFMAs
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m) {
                    const f16x8 av =
                        *reinterpret_cast<const f16x8 *>(vl + v_off<D>(2 * t + h2, 32 * m + col, hh));
#pragma unroll
                    for (int c = 0; c < CT; ++c)
                        oacc[m][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[c][t][h2], oacc[m][c], 0, 0, 0);
                    if (m & 1)
                        __builtin_amdgcn_sched_barrier(0);
                }

        if (it + 1 < n_tiles) {
            if (it + 1 >= n_pre)
                stage_tree_tile(it + 1, nxt);
            lds_loads_landed();
            if (it + 1 < n_pre) {
                convert_prefix_v(it + 1, nxt);
                __syncthreads();
            }
        }
    };
    for (int it = 0; it < n_tiles; it += 2) {
        tile_step(it, lds_a, lds_b, TAV_LDS_ADDR(lds_b));
        if (it + 1 < n_tiles)
            tile_step(it + 1, lds_b, lds_a, TAV_LDS_ADDR(lds_a));
    }

    // ---- write the result or the split's partial ------------------------------
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const float ltot = lsum[c] + __shfl_xor(lsum[c], 32);
        if (!row_ok[c])
            continue;
        if (a.S == 1) {
            const float inv = 1.0f / ltot;
            float *orow = a.out + (((int64_t)b * a.N + node[c]) * a.Hq + head[c]) * D;
            bool finite = true;
#pragma unroll
            for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 v = {oacc[m][c][4 * i] * inv, oacc[m][c][4 * i + 1] * inv,
                                     oacc[m][c][4 * i + 2] * inv, oacc[m][c][4 * i + 3] * inv};
                    finite &= __builtin_isfinite(v.x) && __builtin_isfinite(v.y) &&
                              __builtin_isfinite(v.z) && __builtin_isfinite(v.w);
                    *reinterpret_cast<f32x4 *>(orow + 32 * m + 8 * i + 4 * hh) = v;
                }
            if (!finite)
                raise_flag(a.flags, TAV_FLAG_ATTN_RANGE);
        } else {
            const int64_t P = ((int64_t)bh * a.RB + rb) * a.S + s;
            const int rloc = wave * C::kWaveRows + 32 * c + col;
            float *po = a.part_o + (P * C::kRows + rloc) * D;
#pragma unroll
            for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 v = {oacc[m][c][4 * i], oacc[m][c][4 * i + 1], oacc[m][c][4 * i + 2],
                                     oacc[m][c][4 * i + 3]};
                    *reinterpret_cast<f32x4 *>(po + 32 * m + 8 * i + 4 * hh) = v;
                }
            if (hh == 0) {
                float *pml = a.part_ml + (P * C::kRows + rloc) * 2;
                pml[0] = (m_used[c] == -INFINITY) ? -INFINITY : m_used[c] * a.c;
                pml[1] = ltot;
            }
        }
    }
}

// Merge split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(AttnArgs a, int rows_per_block)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int dq = (int)(idx % (D / 4));
    const int64_t rr = idx / (D / 4);              // (bh, rb, rloc)
    const int rloc = (int)(rr % rows_per_block);
    const int64_t brb = rr / rows_per_block;
    const int rb = (int)(brb % a.RB);
    const int64_t bh = brb / a.RB;
    if (bh >= (int64_t)a.B * a.Hkv)
        return;
    const int row = rb * rows_per_block + rloc;
    if (row >= a.NG)
        return;
    const int b = (int)(bh / a.Hkv), kvh = (int)(bh % a.Hkv);
    const int node = row / a.G, head = kvh * a.G + row % a.G;
    const int64_t P0 = ((int64_t)bh * a.RB + rb) * a.S;
    float M = -INFINITY;
    for (int s = 0; s < a.S; ++s)
        M = fmaxf(M, a.part_ml[((P0 + s) * rows_per_block + rloc) * 2]);
    float lsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.S; ++s) {
        const int64_t pr = (P0 + s) * rows_per_block + rloc;
        const float ms = a.part_ml[pr * 2];
        if (ms == -INFINITY)
            continue;
        const float w = __builtin_amdgcn_exp2f(ms - M);
        lsum += w * a.part_ml[pr * 2 + 1];
        const f32x4 v = *reinterpret_cast<const f32x4 *>(a.part_o + pr * D + dq * 4);
        o += w * v;
    }
    const float inv = 1.0f / lsum;
    const f32x4 r = o * inv;
    if (!(__builtin_isfinite(r.x) && __builtin_isfinite(r.y) && __builtin_isfinite(r.z) &&
          __builtin_isfinite(r.w)))
        raise_flag(a.flags, TAV_FLAG_ATTN_RANGE);
    *reinterpret_cast<f32x4 *>(a.out + (((int64_t)b * a.N + node) * a.Hq + head) * D + dq * 4) = r;
}

struct AttnPlan {
    int NW, CT, rows, RB, S, KS;
    int64_t grid;
    size_t part_o_bytes, part_ml_bytes, ws_bytes;
};

size_t round_up(size_t v, size_t al) { return (v + al - 1) / al * al; }

constexpr int kMinTilesPerSplit = 4;   // below this, partials cost more than the split gains

template <int D>
const void *kernel_for(int NW, int CT)
{
    (void)CT;
    switch (NW) {
    case 8:
        return reinterpret_cast<const void *>(tree_attn_kernel<D, 8, 1>);
    case 4:
        return reinterpret_cast<const void *>(tree_attn_kernel<D, 4, 1>);
    case 2:
        return reinterpret_cast<const void *>(tree_attn_kernel<D, 2, 1>);
    default:
        return reinterpret_cast<const void *>(tree_attn_kernel<D, 1, 1>);
    }
}

// Work decomposition for a shape: rows per wave (32*CT), waves per workgroup
// (NW), row blocks (RB) and prefix splits (S), enough workgroups to fill the
// device once.
bool attn_plan(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_prefix_len,
               AttnPlan &p)
{
    const int G = Hq / Hkv;
    const int NG = N * G;
    // 32 query rows per wave, up to 4 waves per workgroup; two workgroups
    // share a CU so one's softmax overlaps the other's MFMAs
    p.CT = 1;
    p.NW = NG > 128 ? 8 : NG > 64 ? 4 : NG > 32 ? 2 : 1;
    p.rows = 32 * p.CT * p.NW;
    p.RB = (int)ceil_div(NG, p.rows);
    const int cus = device_cu_count();
    if (cus <= 0)
        return false;
    int per_cu = 0;
    const void *fn = D == 128 ? kernel_for<128>(p.NW, p.CT) : kernel_for<64>(p.NW, p.CT);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, p.NW * 64, 0) != hipSuccess ||
        per_cu <= 0)
        return false;
    const int64_t base = (int64_t)B * Hkv * p.RB;
    const int64_t target = (int64_t)cus * per_cu;
    const int64_t tiles = std::max<int64_t>(1, ceil_div(max_prefix_len, kKT));
    int64_t S = ceil_div(target, base);
    S = std::max<int64_t>(1, std::min<int64_t>(S, tiles / kMinTilesPerSplit));
    // a split's block-table slice must fit its LDS copy
    const int64_t max_tiles_per_split = kMaxSplitBlocks / (kKT / kBlock);
    S = std::max<int64_t>(S, ceil_div(tiles, max_tiles_per_split));
    p.S = (int)S;
    p.KS = (int)((int64_t)B * Hkv * p.S);
    p.grid = ceil_div(p.KS, 8) * 8 * p.RB;
    if (p.S > 1) {
        p.part_o_bytes = (size_t)B * Hkv * p.RB * p.S * p.rows * D * sizeof(float);
        p.part_ml_bytes = (size_t)B * Hkv * p.RB * p.S * p.rows * 2 * sizeof(float);
    } else {
        p.part_o_bytes = p.part_ml_bytes = 0;
    }
    p.ws_bytes = p.S > 1 ? round_up(p.part_o_bytes, 256) + round_up(p.part_ml_bytes, 256) : 0;
    return true;
}

bool attn_shape_ok(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t max_prefix_len)
{
    return B >= 1 && N >= 1 && N <= kMaxNodes && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 &&
           (D == 64 || D == 128) && (int64_t)(Hq / Hkv) * N <= 4096 && max_prefix_len >= 0;
}

template <int D, int NW, int CT>
hipError_t launch_main(const AttnPlan &p, const AttnArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((tree_attn_kernel<D, NW, CT>), dim3((unsigned)p.grid), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const AttnPlan &p, const AttnArgs &a, hipStream_t s)
{
    switch (p.NW) {
    case 8:
        return launch_main<D, 8, 1>(p, a, s);
    case 4:
        return launch_main<D, 4, 1>(p, a, s);
    case 2:
        return launch_main<D, 2, 1>(p, a, s);
    default:
        return launch_main<D, 1, 1>(p, a, s);
    }
}

} // namespace
} // namespace tav

extern "C" size_t tree_attn_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t max_prefix_len)
{
    using namespace tav;
    if (!attn_shape_ok(B, N, Hq, Hkv, D, max_prefix_len))
        return 0;
    AttnPlan p;
    if (!attn_plan(B, N, Hq, Hkv, D, max_prefix_len, p))
        return 0;
    return p.ws_bytes;
}

extern "C" tav_status tree_attn_verify(const uint16_t *q, const uint16_t *k_tree,
                                       const uint16_t *v_tree, const uint16_t *k_cache,
                                       const uint16_t *v_cache, int32_t num_blocks,
                                       const int32_t *block_table, int32_t max_blocks,
                                       const int32_t *prefix_len, int32_t max_prefix_len,
                                       const uint64_t *mask, int32_t B, int32_t N, int32_t Hq,
                                       int32_t Hkv, int32_t D, int32_t block_size, float scale,
                                       float *out, void *workspace, size_t ws_bytes,
                                       uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!q || !k_tree || !v_tree || !k_cache || !v_cache || !block_table || !prefix_len ||
        !mask || !out)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1 ||
        max_prefix_len < 0 || !(scale > 0.0f) || !(scale < INFINITY))
        return TAV_ERR_ARG;
    if (!attn_shape_ok(B, N, Hq, Hkv, D, max_prefix_len) || block_size != kBlock)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(mask, 8) || !aligned(out, 16) || !aligned(block_table, 4) ||
        !aligned(prefix_len, 4))
        return TAV_ERR_ARG;
    AttnPlan p;
    if (!attn_plan(B, N, Hq, Hkv, D, max_prefix_len, p))
        return TAV_ERR_LAUNCH;
    if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes || !aligned(workspace, 256)))
        return TAV_ERR_WORKSPACE;

    AttnArgs a;
    a.q = q;
    a.k_tree = k_tree;
    a.v_tree = v_tree;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.prefix_len = prefix_len;
    a.mask = mask;
    a.out = out;
    a.part_o = p.S > 1 ? static_cast<float *>(workspace) : nullptr;
    a.part_ml = p.S > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                     round_up(p.part_o_bytes, 256))
                        : nullptr;
    a.flags = dev_flags;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.max_prefix_len = max_prefix_len;
    a.B = B;
    a.N = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.NG = N * a.G;
    a.W = (int32_t)ceil_div(N, 64);
    a.RB = p.RB;
    a.S = p.S;
    a.KS = p.KS;
    a.c = scale * kLog2e;
    a.th = 8.0f / a.c;

    hipStream_t s = as_stream(stream);
    hipError_t err = D == 128 ? launch_main_d<128>(p, a, s) : launch_main_d<64>(p, a, s);
    if (err != hipSuccess)
        return TAV_ERR_LAUNCH;
    if (p.S > 1) {
        const int64_t threads = (int64_t)B * Hkv * p.RB * p.rows * (D / 4);
        const unsigned blocks = (unsigned)ceil_div(threads, 256);
        if (D == 128)
            hipLaunchKernelGGL(tree_attn_combine_kernel<128>, dim3(blocks), dim3(256), 0, s, a, p.rows);
        else
            hipLaunchKernelGGL(tree_attn_combine_kernel<64>, dim3(blocks), dim3(256), 0, s, a, p.rows);
        if (hipGetLastError() != hipSuccess)
            return TAV_ERR_LAUNCH;
    }
    return TAV_OK;
}
