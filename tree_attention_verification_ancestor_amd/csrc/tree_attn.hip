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
// Tiles are double-buffered in LDS; the next tile's global loads are issued
// before the current tile's MFMAs. Splits of the prefix write unnormalised
// partials (O, max, sum) that a combine kernel merges with log-sum-exp; the
// last split also takes the tree tiles (keys masked by the ancestor bitmask).

#include <algorithm>

#include "common.h"

namespace tav {
namespace {

constexpr int kKT = 64;              // keys per tile
constexpr int kMaxSplitBlocks = 2048; // block-table entries one split stages in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWeightBias = 7.0f;  // log2 of the bias on the fp16 weights

template <int D, int NW>
struct Cfg {
    static constexpr int kThreads = NW * 64;
    static constexpr int kRows = NW * 32;
    static constexpr int kKSteps = D / 16;
    static constexpr int kDTiles = D / 32;
    static constexpr int kCpr = D / 8;                   // 16-byte chunks per row
    static constexpr int kKRow = D * 2 + 16;             // padded K row in LDS
    static constexpr int kKTileBytes = kKT * kKRow;
    static constexpr int kVTileBytes = kKT * D * 2;
    static constexpr int kBufBytes = kKTileBytes + kVTileBytes;
    static constexpr int kChunks = kKT * kCpr;           // 16-byte chunks per tile
    static constexpr int kChPerThread = kChunks / kThreads;
    // Below this many chunks per thread the next tile is prefetched into
    // registers during the current tile's MFMAs; above it, staged directly.
    static constexpr bool kPrefetch = kChPerThread <= 4;
    static_assert(kChunks % kThreads == 0, "tile chunks must split evenly");
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

// LDS byte offset of chunk cc (8 features) of key k in a K tile. Keys are
// stored in MFMA-row order (row 32t + r holds key 32t + perm32(r)), so lane r
// of a wave reads row r, and rows are padded by 16 bytes so the 8 lanes of a
// 128-byte LDS access hit 8 different bank groups.
template <int D>
__device__ __forceinline__ int k_off(int k, int cc)
{
    return ((k & ~31) | perm32(k & 31)) * (D * 2 + 16) + (cc << 4);
}

// Two bf16 values (low, high half of w) to two fp16 values, round to nearest.
// Exact while |v| < 65520; larger magnitudes become infinite.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w)
{
    const f32x2 f = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// LDS byte offset of keys [8*hh, 8*hh+8) of feature d in 16-key block bi of a V tile.
template <int D>
__device__ __forceinline__ int v_off(int bi, int d, int hh)
{
    return bi * (D * 32) + d * 32 + ((hh ^ ((d >> 2) & 1)) << 4);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void tree_attn_kernel(AttnArgs a)
{
    using C = Cfg<D, NW>;
    __shared__ __attribute__((aligned(16))) char lds[2 * C::kBufBytes];
    __shared__ int32_t s_bt[kMaxSplitBlocks];   // this split's physical block ids

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
    const int wave = tid >> 6;
    const int col = lane & 31;      // query column of this lane
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

    // ---- this lane's query row ---------------------------------------------
    const int row = rb * C::kRows + wave * 32 + col;
    const bool row_ok = row < a.NG;
    const int node = row_ok ? row / a.G : 0;
    const int head = kvh * a.G + (row_ok ? row % a.G : 0);
    bf16x8 qf[C::kKSteps];
    {
        const uint16_t *qrow = a.q + (((int64_t)b * a.N + node) * a.Hq + head) * D;
#pragma unroll
        for (int k = 0; k < C::kKSteps; ++k) {
            u32x4 v = {0, 0, 0, 0};
            if (row_ok)
                v = *reinterpret_cast<const u32x4 *>(qrow + 16 * k + 8 * hh);
            qf[k] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- staging of one tile into registers, then LDS ------------------------
    u32x4 kreg[C::kChPerThread], vreg[C::kChPerThread];

    auto load_tile = [&](int it) {
        if (it < n_pre) {
            const int p0 = (t_begin + it) * kKT;
#pragma unroll
            for (int r = 0; r < C::kChPerThread; ++r) {
                const int ci = tid + r * C::kThreads;
                // K: key k, chunk cc
                {
                    const int k = ci / C::kCpr, cc = ci % C::kCpr;
                    const int pos = p0 + k;
                    u32x4 v = {0, 0, 0, 0};
                    if (pos < L) {
                        const int blk = s_bt[(pos >> 4) - blk0];
                        if (blk >= 0)
                            v = *reinterpret_cast<const u32x4 *>(
                                a.k_cache + (((int64_t)blk * a.Hkv + kvh) * kBlock + (pos & 15)) * D + cc * 8);
                    }
                    kreg[r] = v;
                }
                // V: block bi, feature d, key half h2
                {
                    const int bi = ci / (2 * D), rem = ci % (2 * D);
                    const int d = rem >> 1, h2 = rem & 1;
                    const int pos0 = p0 + bi * 16 + h2 * 8;
                    u32x4 v = {0, 0, 0, 0};
                    if (pos0 < L) {
                        const int blk = s_bt[(pos0 >> 4) - blk0];
                        if (blk >= 0) {
                            v = *reinterpret_cast<const u32x4 *>(
                                a.v_cache + (((int64_t)blk * a.Hkv + kvh) * D + d) * kBlock + h2 * 8);
                            const int valid = L - pos0;   // keys past the prefix read as zero
                            if (valid < 8) {
                                uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    if (e >= valid)
                                        w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                                v = u32x4{w[0], w[1], w[2], w[3]};
                            }
                        }
                    }
                    vreg[r] = v;
                }
            }
        } else {
            const int j0 = (it - n_pre) * kKT;
#pragma unroll
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
                kreg[r] = kv;
                vreg[r] = vv;
            }
        }
    };

    auto store_tile = [&](int it, int buf) {
        char *kl = lds + buf * C::kBufBytes;
        char *vl = kl + C::kKTileBytes;
        const bool tree = it >= n_pre;
#pragma unroll
        for (int r = 0; r < C::kChPerThread; ++r) {
            const int ci = tid + r * C::kThreads;
            const int k = ci / C::kCpr, cc = ci % C::kCpr;
            *reinterpret_cast<u32x4 *>(kl + k_off<D>(k, cc)) = kreg[r];
            const uint32_t w[4] = {vreg[r].x, vreg[r].y, vreg[r].z, vreg[r].w};
            if (!tree) {
                const int bi = ci / (2 * D), rem = ci % (2 * D);
                u32x4 h;
                h.x = bf16x2_to_f16x2(w[0]);
                h.y = bf16x2_to_f16x2(w[1]);
                h.z = bf16x2_to_f16x2(w[2]);
                h.w = bf16x2_to_f16x2(w[3]);
                *reinterpret_cast<u32x4 *>(vl + v_off<D>(bi, rem >> 1, rem & 1)) = h;
            } else {
                // tree V rows are feature-contiguous: scatter 8 features of key k
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
        }
    };

    // ---- accumulators --------------------------------------------------------
    f32x16 oacc[C::kDTiles];
#pragma unroll
    for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            oacc[m][e] = 0.f;
    float m_used = -INFINITY;   // raw-score max the exponentials are taken against
    float lsum = 0.f;           // this lane's share of the softmax denominator
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    __syncthreads();   // s_bt ready
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        if (C::kPrefetch && it + 1 < n_tiles)
            load_tile(it + 1);

        const char *kl = lds + buf * C::kBufBytes;
        const char *vl = kl + C::kKTileBytes;

        // S^T = K Q^T for two 32-key tiles
        f32x16 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[t][e] = 0.f;
        const char *krd = kl + col * C::kKRow + hh * 16;   // this lane's MFMA row
#pragma unroll
        for (int k = 0; k < C::kKSteps; ++k) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 av =
                    *reinterpret_cast<const bf16x8 *>(krd + t * 32 * C::kKRow + k * 32);
                sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[k], sacc[t], 0, 0, 0);
            }
        }

        // masks: ragged prefix tail, or ancestor bits of the tree tile
        // Accumulator entry (t, 4i+j) is key 32t + 16(i>>1) + 8hh + 4(i&1) + j;
        // the lane-dependent 8hh is taken out once so the rest are constants.
        if (it >= n_pre) {
            const int tt = it - n_pre;
            uint64_t mw = 1;
            if (row_ok)
                mw = a.mask[((int64_t)b * a.N + node) * a.W + tt];
            mw >>= 8 * hh;
            const uint32_t mlo = (uint32_t)mw, mhi = (uint32_t)(mw >> 32);
            const int nlim = a.N - tt * kKT - 8 * hh;   // keys at or past it are not nodes
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
                            sacc[t][4 * i + j] = -INFINITY;
                    }
        } else {
            const int p0 = (t_begin + it) * kKT;
            if (p0 + kKT > L) {
                const int plim = L - p0 - 8 * hh;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int kr = 32 * t + 16 * (i >> 1) + 4 * (i & 1) + j;
                            if (kr >= plim)
                                sacc[t][4 * i + j] = -INFINITY;
                        }
            }
        }

        // online softmax with lazy rescaling
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                mt = fmaxf(mt, sacc[t][e]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool need = mt > m_used + a.th;
        if (__any(need)) {
            const float mnew = need ? mt : m_used;
            const float alpha =
                (m_used == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_used - mnew) * a.c);
#pragma unroll
            for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[m][e] *= alpha;
            lsum *= alpha;
            m_used = mnew;
        }
        // weights 2^(s*c - m*c + 7): at most 2^15 after the lazy threshold
        const float moff = (m_used == -INFINITY) ? 0.f : m_used * a.c - kWeightBias;

        f16x8 pb[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * h2 + e], a.c, -moff));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * h2 + e + 1], a.c, -moff));
                    const f32x2 pf = {p0, p1};
                    const f16x2 pk = __builtin_convertvector(pf, f16x2);
                    pb[t][h2][e] = pk[0];
                    pb[t][h2][e + 1] = pk[1];
                    lsum = __builtin_amdgcn_fdot2(pk, ones, lsum, false);
                }
            }

        // O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m) {
                    const f16x8 av =
                        *reinterpret_cast<const f16x8 *>(vl + v_off<D>(2 * t + h2, 32 * m + col, hh));
                    oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[t][h2], oacc[m], 0, 0, 0);
                }

        if (it + 1 < n_tiles) {
            if (!C::kPrefetch)
                load_tile(it + 1);
            store_tile(it + 1, buf ^ 1);
        }
        __syncthreads();
    }

    // ---- write the result or the split's partial ------------------------------
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!row_ok)
        return;
    if (a.S == 1) {
        const float inv = 1.0f / ltot;
        float *orow = a.out + (((int64_t)b * a.N + node) * a.Hq + head) * D;
        bool finite = true;
#pragma unroll
        for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = {oacc[m][4 * i] * inv, oacc[m][4 * i + 1] * inv,
                                 oacc[m][4 * i + 2] * inv, oacc[m][4 * i + 3] * inv};
                finite &= __builtin_isfinite(v.x) && __builtin_isfinite(v.y) &&
                          __builtin_isfinite(v.z) && __builtin_isfinite(v.w);
                *reinterpret_cast<f32x4 *>(orow + 32 * m + 8 * i + 4 * hh) = v;
            }
        if (!finite)
            raise_flag(a.flags, TAV_FLAG_ATTN_RANGE);
    } else {
        const int64_t P = ((int64_t)bh * a.RB + rb) * a.S + s;
        const int rloc = wave * 32 + col;
        float *po = a.part_o + (P * C::kRows + rloc) * D;
#pragma unroll
        for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = {oacc[m][4 * i], oacc[m][4 * i + 1], oacc[m][4 * i + 2],
                                 oacc[m][4 * i + 3]};
                *reinterpret_cast<f32x4 *>(po + 32 * m + 8 * i + 4 * hh) = v;
            }
        if (hh == 0) {
            float *pml = a.part_ml + (P * C::kRows + rloc) * 2;
            pml[0] = (m_used == -INFINITY) ? -INFINITY : m_used * a.c;
            pml[1] = ltot;
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
    int NW, rows, RB, S, KS;
    int64_t grid;
    size_t part_o_bytes, part_ml_bytes, ws_bytes;
};

size_t round_up(size_t v, size_t al) { return (v + al - 1) / al * al; }

bool attn_plan(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_prefix_len,
               AttnPlan &p)
{
    (void)D;
    const int G = Hq / Hkv;
    const int NG = N * G;
    p.NW = NG > 128 ? 8 : NG > 64 ? 4 : NG > 32 ? 2 : 1;
    p.rows = 32 * p.NW;
    p.RB = (int)ceil_div(NG, p.rows);
    const int cus = device_cu_count();
    if (cus <= 0)
        return false;
    const int64_t base = (int64_t)B * Hkv * p.RB;
    const int64_t per_cu = std::max(1, 8 / p.NW);          // resident workgroups per CU
    const int64_t target = (int64_t)cus * per_cu;
    const int64_t tiles = std::max<int64_t>(1, ceil_div(max_prefix_len, kKT));
    int64_t S = ceil_div(target, base);
    S = std::max<int64_t>(1, std::min<int64_t>(S, tiles));
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

template <int D, int NW>
hipError_t launch_main(const AttnPlan &p, const AttnArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((tree_attn_kernel<D, NW>), dim3((unsigned)p.grid), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const AttnPlan &p, const AttnArgs &a, hipStream_t s)
{
    switch (p.NW) {
    case 1:
        return launch_main<D, 1>(p, a, s);
    case 2:
        return launch_main<D, 2>(p, a, s);
    case 4:
        return launch_main<D, 4>(p, a, s);
    default:
        return launch_main<D, 8>(p, a, s);
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
