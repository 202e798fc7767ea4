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
// takes a block of 32*NW of those rows and one split of the key tiles; the K/V
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
// Staging. V tiles sit in a ring of five LDS slots and K tiles in a ring of
// one slot more than the tiles in flight: an 8-wave workgroup fills two tiles
// ahead (three K slots; its lagging waves read V up to two tiles behind),
// smaller D = 128 workgroups, which wait on memory more than on arithmetic,
// three (four K slots; their V is read one tile behind). Prefix tiles move from HBM straight into LDS
// (global_load_lds_dwordx4: 16 bytes per lane, no staging registers), with
// the block table resolved once per split into head-block indices in LDS;
// in an 8-wave workgroup the four waves with the shorter chain of work per
// tile issue every load (an issuing wave stalls until the CU's load path
// takes each one). Each tile's V is turned from bf16 into fp16 in place,
// one 16-byte chunk at a time between the S MFMAs, keys past the prefix
// zeroed. The few tree tiles go through registers (their V rows need a
// transpose). One barrier per tile.
// Operand reads. The S and P.V MFMAs take their LDS operands from reads
// issued four MFMAs ahead into separate registers, held in that order by a
// scheduling fence after each MFMA.
// Small row counts. Up to 128 query rows per (sequence, KV head) a
// workgroup takes 128 rows (four row waves) in two wave sets over the same
// rows: set h takes keys [32h, 32h + 32) of every tile (half the S and P.V
// MFMAs and half the softmax each), and at the end the upper set's
// (O, max, sum) merge into the lower set's through LDS, as two splits
// would. A tile's chain of work per wave is then half as long, and eight
// waves (two per SIMD) work on it.
// Overlap. A wave's work per tile is an MFMA phase (S) and a phase that
// mixes vector ALU work and MFMAs: the softmax of the tile spread between the
// P.V MFMAs of the tile before. In an 8-wave workgroup the two waves that
// share a SIMD run these in opposite order, one a tile behind the other.
// The key tiles of a (sequence, KV head) are its prefix tiles and then its
// tree tiles (keys masked by the ancestor bitmask), split evenly. Two splits
// of a (sequence, KV head, row block) merge inside the launch: each counts
// its arrival on a counter in the workspace, the first writes its
// unnormalised partial (O, max, sum) and counts itself done, and the second
// waits for that, merges it with its own registers in split order
// (log-sum-exp), writes the result and clears the counters. With more
// splits every split writes its partial and a combine kernel merges them
// (the last split's serial reads of many partials cost more than a kernel).

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace tav {
namespace {

constexpr int kKT = 64;              // keys per tile
constexpr uint32_t kMergeSpinLimit = 1u << 20;   // polls before the merge's wait gives up
constexpr int kMaxSplitBlocks = 2048; // block-table entries one split stages in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWeightBias = 7.0f;  // log2 of the bias on the fp16 weights

template <int D, int NW, int KSP = 1>
struct Cfg {
    static constexpr int kThreads = NW * KSP * 64;
    static constexpr int kRows = NW * 32;                // query rows per workgroup (32 per row wave)
    static constexpr int kKSteps = D / 16;
    static constexpr int kDTiles = D / 32;
    static constexpr int kCpr = D / 8;                   // 16-byte chunks per row
    static constexpr int kKRow = D * 2;                  // K row in LDS (16-byte chunks swizzled)
    static constexpr int kKTileBytes = kKT * kKRow;
    static constexpr int kVTileBytes = kKT * D * 2;
    static constexpr int kBufBytes = kKTileBytes + kVTileBytes;
    static constexpr int kChunks = kKT * kCpr;           // 16-byte chunks per K (or V) tile
    static constexpr int kChPerThread = kChunks / kThreads;
    static_assert(kChunks % kThreads == 0, "tile chunks must split evenly");
};

struct AttnArgs {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *block_table, *prefix_len;
    const uint64_t *mask;    // [B][N][W] ancestor bits, or NULL: built from parent
    const int32_t *parent;   // [B][N] when mask is NULL
    uint64_t *mask_out;      // optional copies of the built mask and depths
    int32_t *depth_out;
    float *out, *part_o, *part_ml;
    uint32_t *counters;      // [B * Hkv * RB][2]: arrived, done (zero between calls)
    int32_t merge;           // S == 2: the splits merge inside the launch
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

// One direct HBM -> LDS load: lane l's 16 bytes at base + voff land at LDS
// byte address lds_addr + 16 l (base and lds_addr are the same for the whole
// wave). Issued as inline assembly: the compiler then neither makes later LDS
// reads wait for it nor reasons about what it writes; the code that reads
// the destination waits for it explicitly (wait_vmem, then a barrier).
__device__ __forceinline__ void load_lds16(const void *base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_addr)
                 : "memory", "m0");
}

// LDS byte address of a __shared__ object (folded at compile time).
#define TAV_LDS_ADDR(obj) ((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(obj))

// An LDS location by byte address.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T *lds_at(uint32_t addr)
{
    return reinterpret_cast<__attribute__((address_space(3))) T *>((uintptr_t)addr);
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

// s_waitcnt with only the vector-memory count set: wait until at most N of
// this wave's vector memory operations are outstanding (they complete in
// issue order).
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// sched_group_barrier instruction classes
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;

template <int D, int NW, int KSP = 1>
__global__ __launch_bounds__(NW * KSP * 64) void tree_attn_kernel(AttnArgs a)
{
    using C = Cfg<D, NW, KSP>;
    static_assert(KSP == 1 || (KSP == 2 && NW <= 4), "keys split between two wave sets");
    // Which waves issue the direct tile loads. A wave stalls at each one until
    // the CU's load path takes it (about 14 cycles per kilobyte, every wave of
    // the CU in one queue), so with 8 waves the four whose work per tile is
    // the shorter chain (see "Overlap") issue them all and the other four none.
    constexpr int kIssuers = NW == 8 ? NW / 2 : NW * KSP;
    constexpr int LPW = C::kChunks / 64 / kIssuers;   // loads per issuing wave per K (or V) tile
    static_assert(LPW * 64 * kIssuers == C::kChunks, "direct loads must split evenly");
    constexpr int KTB = C::kKTileBytes, VTB = C::kVTileBytes;
    // Tiles in flight: tile t + kAhead streams in during step t. Tile t's K
    // is read in step t only, its V in step t+1 (or t+2 for the lagging
    // waves of an 8-wave workgroup), so K needs kAhead + 1 slots and V
    // kAhead + 2 (+ 1 with lagging waves): 3 and 5 at depth 2 with lagging
    // waves, 4 and 5 at depth 3 without. Depth 3 fits the LDS for D = 128
    // below 8 waves (157 KB); for D = 64 it would cost the second workgroup
    // per CU.
    constexpr int kAhead = (D == 128 && NW < 8) ? 3 : 2;
    constexpr int kKSlots = kAhead + 1, kVSlots = 5;
    static_assert(kVSlots >= kAhead + (NW == 8 ? 3 : 2), "V ring too short for the pipeline");
    __shared__ __attribute__((aligned(16))) char s_k[kKSlots * KTB];
    __shared__ __attribute__((aligned(16))) char s_v[kVSlots * VTB];
    // this split's cache blocks as head-block indices (block * Hkv + kvh)
    __shared__ __attribute__((aligned(16))) uint32_t s_bt[kMaxSplitBlocks];
    // ancestor bits of this workgroup's nodes built from parent[] (when no
    // mask is passed in), and the parent row they are built from
    __shared__ uint64_t s_mask[C::kRows][kMaxNodes / 64];
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int s_last;   // this split arrived last at its unit

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
    // With KSP = 2 the workgroup's waves form two sets over the same query
    // rows (row wave rw), set `half` taking keys [32 half, 32 half + 32) of
    // every tile; the two online softmaxes merge at the end.
    const int rw = wave % NW;
    const int half = wave / NW;
    const int col = lane & 31;      // query column of this lane
    const int hh = lane >> 5;       // which half of the K dimension this lane feeds

    int L = a.prefix_len[b];
    if (L < 0 || L > a.max_prefix_len || L > a.max_blocks * kBlock) {
        if (tid == 0)
            raise_flag(a.flags, TAV_FLAG_CAPACITY);
        L = std::max(0, std::min(L, std::min(a.max_prefix_len, a.max_blocks * kBlock)));
    }
    // The unit's tiles are its Tb prefix tiles and then its tree tiles; split
    // s takes [s U / S, (s + 1) U / S) of them, so the tree tiles count in the
    // balance of the splits.
    const int Tb = (L + kKT - 1) / kKT;
    const int Ub = Tb + (a.N + kKT - 1) / kKT;
    const int u0 = (int)((int64_t)s * Ub / a.S), u1 = (int)((int64_t)(s + 1) * Ub / a.S);
    const int t_begin = std::min(u0, Tb);
    const int t_end = std::min(u1, Tb);
    // The plan keeps every split's slice within its LDS copy; a launch that
    // broke that rule would index past it, so that split computes nothing
    // (and still takes its part in the merge).
    const bool oversize = (t_end - t_begin) * (kKT / kBlock) > kMaxSplitBlocks;
    if (oversize && tid == 0)
        raise_flag(a.flags, TAV_FLAG_CAPACITY);
    const int n_pre = oversize ? 0 : t_end - t_begin;
    const int tt0 = std::max(u0, Tb) - Tb;               // first tree tile of the split
    const int n_tree = oversize ? 0 : std::max(0, u1 - std::max(u0, Tb));
    const int n_tiles = n_pre + n_tree;
    // The split's block-table slice, validated once. Entries past the prefix
    // (and bad ones, which also raise a flag) name block 0 of this head, a
    // valid address whose keys are masked and whose V entries are zeroed.
    {
        const int32_t *bt = a.block_table + (int64_t)b * a.max_blocks;
        const int nbt = n_pre * (kKT / kBlock);
        const int nvalid = (L + kBlock - 1) / kBlock - t_begin * (kKT / kBlock);
        for (int i = tid; i < nbt; i += C::kThreads) {
            uint32_t hb = (uint32_t)kvh;
            if (i < nvalid) {
                const int32_t blk = bt[t_begin * (kKT / kBlock) + i];
                if (blk < 0 || blk >= a.num_blocks)
                    raise_flag(a.flags, TAV_FLAG_BAD_BLOCK);
                else
                    hb = (uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh;
            }
            s_bt[i] = hb;
        }
    }

    // ---- this lane's query row, and the first word of its ancestor mask ------
    const int row = rb * C::kRows + rw * 32 + col;
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
    const bool built = a.mask == nullptr;
    // The workgroup of (sequence, KV head 0, split 0, row block 0) also
    // checks the tree and writes the built mask out, if asked to.
    const bool lead_mask = built && kvh == 0 && s == 0 && rb == 0;
    const bool need_mask = built && (n_tree > 0 || lead_mask);
    const uint64_t mrow0 =
        (!built && n_tree > 0 && row_ok) ? a.mask[((int64_t)b * a.N + node) * a.W + tt0] : 1;
    if (need_mask)
        for (int i = tid; i < a.N; i += C::kThreads)
            s_par[i] = a.parent[(int64_t)b * a.N + i];
    // Wait for these loads here, before any tile load is in flight. The
    // compiler does not see the direct tile loads (inline assembly), so a
    // register load it still counts as outstanding inside the tile loop would
    // make it wait for every vector memory operation, prefetched tiles
    // included, at the first use.
    wait_vmem<0>();

    // ---- direct-load descriptors, fixed for the whole kernel ------------------
    // Load j of a tile fills LDS chunks [64j, 64j+64) in lane order; issuing
    // wave w issues loads j = w + i*kIssuers. The chunks of one load always come from a
    // single 16-key cache block (4 or 8 whole MFMA rows of K, whose keys differ
    // only in their low bits; or 64 feature halves of one V block): the
    // block's address is a wave-uniform base and each lane adds a byte offset
    // below 4 KB.
    const bool issuer = wave < kIssuers;
    int kbb[LPW], vbb[LPW];          // which of the tile's four blocks
    uint32_t koff[LPW], voff[LPW];   // this lane's byte offset inside it
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int j = wave % kIssuers + i * kIssuers;
        const int row0 = j * 64 / C::kCpr;   // first MFMA row of this load
        kbb[i] = ((row0 & ~31) | perm32(row0 & 31)) >> 4;
        const int q = j * 64 + lane;
        const int r = q / C::kCpr, pos = q % C::kCpr;
        const int cc = pos ^ k_swz<D>(r);
        const int key = (r & ~31) | perm32(r & 31);
        koff[i] = (uint32_t)(((key & 15) * D + cc * 8) * 2);
        vbb[i] = j * 64 / (2 * D);
        const int rem = q % (2 * D);
        const int d = rem >> 1, hpos = rem & 1;
        const int h2 = v_slot(d, hpos);   // v_slot is its own inverse in hh
        voff[i] = (uint32_t)((d * kBlock + h2 * 8) * 2);
    }
    const uint32_t k_lds = TAV_LDS_ADDR(s_k), v_lds = TAV_LDS_ADDR(s_v);

    // ---- staging -----------------------------------------------------------
    // The head-block indices a prefix tile's loads need, read from LDS ahead
    // of the barrier that precedes the loads.
    struct TileIds {
        uint32_t k[LPW], v[LPW];
    };
    auto read_ids = [&](int it) __attribute__((always_inline)) {
        TileIds ids;
        const int e0 = it * (kKT / kBlock);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            ids.k[i] = s_bt[e0 + kbb[i]];
            ids.v[i] = s_bt[e0 + vbb[i]];
        }
        return ids;
    };
    auto issue_prefix_tile = [&](const TileIds &ids, uint32_t kdst, uint32_t vdst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const uint32_t hb = __builtin_amdgcn_readfirstlane(ids.k[i]);
            load_lds16(a.k_cache + (uint64_t)hb * (kBlock * D), koff[i], kdst + (wave + i * kIssuers) * 1024u);
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const uint32_t hb = __builtin_amdgcn_readfirstlane(ids.v[i]);
            load_lds16(a.v_cache + (uint64_t)hb * (kBlock * D), voff[i], vdst + (wave + i * kIssuers) * 1024u);
        }
    };

    // bf16 -> fp16 of a landed prefix tile's V, in place, in two halves so
    // the S MFMAs can run between them (the compiler cannot tell the V writes
    // from the K reads apart). `masked`: the tile ends past the prefix, whose
    // keys become zero (unused cache slots may hold anything).
    auto convert_load = [&](uint32_t vaddr, u32x4 (&cv)[C::kChPerThread]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < C::kChPerThread; ++r)
            cv[r] = *lds_at<u32x4>(vaddr + (tid + r * C::kThreads) * 16);
    };
    auto convert_store_chunk = [&](int it, uint32_t vaddr, const u32x4 &c, int r, bool masked)
                                   __attribute__((always_inline)) {
        const int p0 = (t_begin + it) * kKT;
        {
            const int q = tid + r * C::kThreads;
            uint32_t w[4] = {c.x, c.y, c.z, c.w};
            if (masked) {
                const int bi = q / (2 * D), rem = q % (2 * D);
                const int d = rem >> 1, hpos = rem & 1;
                const int valid = L - (p0 + bi * 16 + v_slot(d, hpos) * 8);
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
            *lds_at<u32x4>(vaddr + q * 16) = h;
        }
    };
    auto convert_store = [&](int it, uint32_t vaddr, u32x4 (&cv)[C::kChPerThread], bool masked)
                             __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < C::kChPerThread; ++r)
            convert_store_chunk(it, vaddr, cv[r], r, masked);
    };

    // Tree tile: through registers. K rows go to their MFMA rows; V rows are
    // feature-contiguous, so 8 features of a key are scattered (as fp16).
    auto stage_tree_tile = [&](int it, char *kl, char *vl) __attribute__((always_inline)) {
        const int j0 = (it - n_pre + tt0) * kKT;
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

    // S^T = K Q^T for the two 32-key halves of a tile (MFMA: A = K rows from
    // LDS, B = this wave's Q^T in registers). K fragment k of row 32t + col
    // sits at col*2D + ((2k ^ x) << 4) + t*64D with x = hh ^ k_swz(col): a
    // per-lane offset for each k, and a constant for t.
    //
    // Fragment reads run kDepth MFMAs ahead of their use, each into its own
    // registers, and a scheduling fence after every MFMA keeps that order: left
    // free, the scheduler pulls each read down next to its MFMA (fewer live
    // registers), and every MFMA then waits out a full LDS round trip. MFMA j
    // takes k = j/2 and half t = j%2, so consecutive MFMAs feed different
    // accumulators. `between(j)` runs after MFMA j (vector work to hide).
    uint32_t kfrag[C::kKSteps];
#pragma unroll
    for (int k = 0; k < C::kKSteps; ++k)
        kfrag[k] = (uint32_t)(col * (2 * D) + (((2 * k) ^ hh ^ k_swz<D>(col)) << 4));
    constexpr int kDepth = 4;
    // halves of a tile's keys per wave: both, or (KSP = 2) the wave's own,
    // kept in sacc[0] / pb[0]
    constexpr int kT = 2 / KSP;
    constexpr int kQkN = kT * C::kKSteps;
    static_assert(kQkN >= kDepth, "read pipeline deeper than the MFMA sequence");
    // MFMA j of a tile: key half t = j & 1 (or the wave's), K step j >> 1 (or j)
    auto kfrag_of = [&](int j) __attribute__((always_inline)) {
        if constexpr (KSP == 1)
            return kfrag[j >> 1] + (uint32_t)((j & 1) * (64 * D));
        else
            return kfrag[j];
    };
    auto qk = [&](uint32_t kaddr, f32x16 (&sacc)[2], auto &&between) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[t][e] = 0.f;
        if constexpr (KSP == 2)
            kaddr += (uint32_t)(half * (64 * D));
        bf16x8 kb[kDepth];
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            kb[j] = *lds_at<bf16x8>(kaddr + kfrag_of(j));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kQkN; ++j) {
            constexpr int kTShift = KSP == 1 ? 1 : 0;
            const int t = KSP == 1 ? (j & 1) : 0;
            sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[j % kDepth], qf[j >> kTShift], sacc[t], 0, 0, 0);
            if (j + kDepth < kQkN) {
                const int n = j + kDepth;
                kb[j % kDepth] = *lds_at<bf16x8>(kaddr + kfrag_of(n));
            }
            between(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto no_work = [](int) __attribute__((always_inline)) {};

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

    // Keys a tile may not see get score -inf: keys past the prefix in the
    // last prefix tile of a split, and in tree tiles the keys that are not
    // ancestors of this lane's node (or are not nodes). Accumulator entry
    // (t, 4i+j) is key 32t + 16(i>>1) + 8hh + 4(i&1) + j.
    auto apply_mask = [&](int it, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
        uint64_t mw;   // bit k: key k of the tile is visible
        int lim;       // keys at or past it are not keys
        if (it >= n_pre) {
            const int tt = it - n_pre + tt0;
            mw = 1;    // a padding row sees key 0 only
            if (row_ok)
                mw = built ? s_mask[node - rb * C::kRows / a.G][tt]
                           : tt == tt0 ? mrow0 : a.mask[((int64_t)b * a.N + node) * a.W + tt];
            lim = a.N - tt * kKT;
        } else {
            mw = ~0ull;
            lim = L - (t_begin + it) * kKT;
        }
        mw >>= 8 * hh;
        lim -= 8 * hh;
        const uint32_t mlo = (uint32_t)mw, mhi = (uint32_t)(mw >> 32);
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kr = 16 * (i >> 1) + 4 * (i & 1) + j;   // < 32
                    const int th = KSP == 1 ? t : half;                  // the key half
                    const uint32_t word = th ? mhi : mlo;
                    const bool ok = (32 * th + kr < lim) && ((word >> kr) & 1u);
                    if (!ok)
                        sacc[t][4 * i + j] = -INFINITY;
                }
    };

    // Online softmax of one tile's scores, without branches: the running max
    // only moves when the tile exceeds it by more than 2^8 in probability
    // (then alpha < 1 rescales what was accumulated before), and the weights
    // 2^(s*c - m*c + 7), at most 2^15, go to pb as fp16.
    auto softmax = [&](f32x16 (&sacc)[2], f16x8 (&pb)[2][2], float &alpha) __attribute__((always_inline)) {
        // (NaN-propagating maximum: no canonicalising of the MFMA results; a
        // NaN score leaves the max alone and surfaces in the output check)
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int e = 0; e < 16; e += 2)
                mt = __builtin_elementwise_maximum(mt, __builtin_elementwise_maximum(sacc[t][e], sacc[t][e + 1]));
        {   // the other half of the wave holds the same column's other keys
            const uint32_t u = __builtin_bit_cast(uint32_t, mt);
            const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            const uint32_t u0 = sw[0];
            const uint32_t u1 = sw[1];
            mt = __builtin_elementwise_maximum(__builtin_bit_cast(float, u0), __builtin_bit_cast(float, u1));
        }
        const bool need = mt > m_used + a.th;
        const float mnew = need ? mt : m_used;
        // m_used = -inf gives exp2(-inf) = 0: nothing accumulated yet
        alpha = need ? __builtin_amdgcn_exp2f((m_used - mnew) * a.c) : 1.0f;
        m_used = mnew;
        lsum *= alpha;
        const float moff = (m_used == -INFINITY) ? 0.f : m_used * a.c - kWeightBias;
        if constexpr (KSP == 2) {   // the other half's weights: none
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pb[1][h2][e] = (_Float16)0.0f;
        }
#pragma unroll
        for (int t = 0; t < kT; ++t)
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
    };

    // O^T += V^T P^T for one tile (MFMA: A = V^T from the fp16 V tile at LDS
    // byte address vaddr, B = the weights). Feature d = 32m + col of block bi
    // sits at v_off(bi, d, hh) = bi*32D + 1024m + v_off(0, col, hh): one
    // per-lane base register and constant offsets that fit the LDS
    // instruction's offset field. MFMA j takes block bi = j / kDTiles (weights
    // pb[bi/2][bi%2]) and feature tile m = j % kDTiles. The same read pipeline
    // as the scores; pv_begin issues the first kDepth reads, so a caller can
    // put vector work between them and the MFMAs.
    constexpr int kPvN = 2 * kT * C::kDTiles;
    static_assert(kPvN >= kDepth, "read pipeline deeper than the MFMA sequence");
    struct VReads {
        uint32_t base;
        f16x8 vb[kDepth];
    };
    auto pv_begin = [&](uint32_t vaddr) __attribute__((always_inline)) {
        VReads r;
        r.base = vaddr + (uint32_t)v_off<D>(0, col, hh);
        if constexpr (KSP == 2)   // this wave's key half: 16-key blocks 2 half, 2 half + 1
            r.base += (uint32_t)(half * 2 * (D * 32));
        asm("" : "+v"(r.base));   // keep the sum in one register
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            r.vb[j] = *lds_at<f16x8>(r.base + (uint32_t)((j / C::kDTiles) * (D * 32) + (j % C::kDTiles) * 1024));
        return r;
    };
    // kValuPerMfma > 0: no fences; instead the scheduler is asked for MFMA j,
    // then the read of fragment j + kDepth, then up to kValuPerMfma vector
    // instructions from the same region (the caller's independent vector work
    // written before this call), so that work issues while the MFMAs run.
    constexpr int kValuPerMfma = 10;
    auto pv_finish = [&](const f16x8 (&pb)[2][2], VReads &r, auto interleave) __attribute__((always_inline)) {
        constexpr bool kMix = decltype(interleave)::value;
        if constexpr (!kMix)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kPvN; ++j) {
            const int bi = j / C::kDTiles, m = j % C::kDTiles;
            oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(r.vb[j % kDepth], pb[bi >> 1][bi & 1], oacc[m], 0, 0, 0);
            if (j + kDepth < kPvN) {
                const int n = j + kDepth;
                r.vb[j % kDepth] =
                    *lds_at<f16x8>(r.base + (uint32_t)((n / C::kDTiles) * (D * 32) + (n % C::kDTiles) * 1024));
            }
            if constexpr (!kMix)
                __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kMix) {
#pragma unroll
            for (int j = 0; j < kPvN; ++j) {
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 2);
                if (j + kDepth < kPvN)
                    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 2);
                __builtin_amdgcn_sched_group_barrier(kSgValu, kValuPerMfma, 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto pv = [&](const f16x8 (&pb)[2][2], uint32_t vaddr) __attribute__((always_inline)) {
        VReads r = pv_begin(vaddr);
        pv_finish(pb, r, std::false_type{});
    };

    // ---- the tile pipeline ---------------------------------------------------
    // Tile t's K sits in K slot t % kKSlots and its V in V slot t % 5; both
    // are filled kAhead steps ahead, by direct loads (prefix tiles) or
    // through registers (tree tiles). Every step starts by waiting for tile t
    // (the later tiles' loads may stay in flight) and passing the step's only
    // barrier, after which every wave is done with tile t-1's K and tile
    // t-3's V (t-2's without lagging waves); it then fills tile t + kAhead
    // into those slots. Per tile a wave has an MFMA phase
    //   Q(t): S = K Q^T (and tile t's V turned into fp16 meanwhile)
    // and a phase that is mostly vector ALU work:
    //   R(t): the softmax of tile t, with P.V of the tile before on the
    //         matrix cores in between.
    // The two waves that share a SIMD (waves w and w+4 of an 8-wave
    // workgroup) run them in opposite order: one runs Q(t) R(t) in step t,
    // the other R(t-1) Q(t), carrying S across the barrier. Each one's
    // vector work then overlaps the other's MFMAs. A rescale of O (rare)
    // waits for the P.V before it through the register dependency.
    const bool lag = NW == 8 && wave >= NW / 2;
    auto fill = [&](int t, const TileIds &ids) __attribute__((always_inline)) {
        const int kslot = t % kKSlots, vslot = t % kVSlots;
        if (t < n_pre) {
            if (issuer)
                issue_prefix_tile(ids, k_lds + kslot * KTB, v_lds + vslot * VTB);
        }
        else if (t < n_tiles)
            stage_tree_tile(t, s_k + kslot * KTB, s_v + vslot * VTB);
    };
    // "tiles -2 and -1" (V slots 3 and 4) contribute nothing: zero weights
    // times zero V
    for (int q = tid; q < 2 * VTB / 16; q += C::kThreads)
        *lds_at<u32x4>(v_lds + 3 * VTB + q * 16) = u32x4{0, 0, 0, 0};
    __syncthreads();   // s_bt (and s_par) written by all threads before any wave reads it
    if (need_mask) {
        // Node i's bits: climb from i to the root setting one bit per node
        // met (parent[i] < i, so each climb ends); the same rule and flag as
        // tree_mask_build. Read only at the tree tiles, several barriers on.
        // this workgroup's nodes: those of rows [rb R, rb R + R), R = kRows
        const int node_lo = rb * C::kRows / a.G;
        const int node_hi = std::min(a.N, (rb * C::kRows + C::kRows - 1) / a.G + 1);
        for (int i = lead_mask ? tid : node_lo + tid; i < (lead_mask ? a.N : node_hi);
             i += C::kThreads) {
            uint64_t words[kMaxNodes / 64] = {0, 0, 0, 0};
            bool bad = (i == 0) ? (s_par[0] != -1) : (s_par[i] < 0 || s_par[i] >= i);
            int dep = 0, j = i;
            while (!bad) {
                words[j >> 6] |= 1ull << (j & 63);
                if (j == 0)
                    break;
                const int pj = s_par[j];
                if (pj < 0 || pj >= j) {
                    bad = true;
                    break;
                }
                j = pj;
                ++dep;
            }
            if (i >= node_lo && i < node_hi)
#pragma unroll
                for (int w = 0; w < kMaxNodes / 64; ++w)
                    s_mask[i - node_lo][w] = words[w];
            if (lead_mask) {
                if (bad)
                    raise_flag(a.flags, TAV_FLAG_BAD_PARENT);
                if (a.mask_out)
                    for (int w = 0; w < a.W; ++w)
                        a.mask_out[((int64_t)b * a.N + i) * a.W + w] = words[w];
                if (a.depth_out)
                    a.depth_out[(int64_t)b * a.N + i] = dep;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
        fill(t, read_ids(t));

    f16x8 pb_prev[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pb_prev[t][h2][e] = (_Float16)0.0f;
    f32x16 sacc[2];   // the lagging wave's "tile -1" scores: all masked
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            sacc[t][e] = -INFINITY;

    // Q(it): scores of tile it into sacc.
    auto phase_q = [&](int it, uint32_t kcur, uint32_t vcur) __attribute__((always_inline)) {
        if (it < n_pre && (t_begin + it + 1) * kKT <= L) {
            // a whole prefix tile: its V conversion runs between the S MFMAs,
            // chunk r after MFMA (2r + 1) * kQkN / (2 * chunks), in [0, kQkN)
            u32x4 cv[C::kChPerThread];
            convert_load(vcur, cv);
            qk(kcur, sacc, [&](int j) __attribute__((always_inline)) {
#pragma unroll
                for (int r = 0; r < C::kChPerThread; ++r)
                    if (j == (2 * r + 1) * kQkN / (2 * C::kChPerThread))
                        convert_store_chunk(it, vcur, cv[r], r, false);
            });
        } else {
            if (it < n_pre) {
                u32x4 cv[C::kChPerThread];
                convert_load(vcur, cv);
                convert_store(it, vcur, cv, true);
            }
            qk(kcur, sacc, no_work);
            apply_mask(it, sacc);
        }
    };
    // R: P.V of the tile whose weights are in pb_prev (its fp16 V at vprev),
    // then the softmax of sacc into pb_prev.
    auto phase_r = [&](uint32_t vprev) __attribute__((always_inline)) {
        f16x8 pb[2][2];
        float alpha;
        // The first V reads, then P.V of the tile before with the softmax of
        // this tile (independent of it) spread between its MFMAs. The V reads
        // run ahead of their MFMAs, so the waits for them rarely hold up the
        // vector work behind them (a wave issues in order).
        VReads vr = pv_begin(vprev);
        __builtin_amdgcn_sched_barrier(0);
        softmax(sacc, pb, alpha);
        pv_finish(pb_prev, vr, std::true_type{});
        // every weight computed before the branch (the compiler would sink them)
        asm volatile("" ::"v"(pb[0][0]), "v"(pb[0][1]), "v"(pb[1][0]), "v"(pb[1][1]), "v"(lsum));
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[m][e] *= alpha;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                pb_prev[t][h2] = pb[t][h2];
    };

    // one loop per phase order, so each gets its own register allocation
    // (every wave passes the same number of barriers)
    auto run = [&](auto lag_c) __attribute__((always_inline)) {
        constexpr bool kLag = decltype(lag_c)::value;
        int kslot = 0, vslot = 0;   // tile it's slots
        auto vslot_back = [&](int n) __attribute__((always_inline)) {
            const int v = vslot - n;
            return v < 0 ? v + kVSlots : v;
        };
        for (int it = 0; it < n_tiles; ++it) {
            TileIds ids{};
            if (issuer && it + kAhead < n_pre)
                ids = read_ids(it + kAhead);
            // tile it's loads done; those of the prefix tiles after it (up to
            // kAhead - 1, issued later) may stay in flight. Counts beyond the
            // counter's range wait longer.
            if (kAhead == 3 && it + 2 < n_pre)
                wait_vmem<(4 * LPW < 64 ? 4 * LPW : 63)>();
            else if (it + 1 < n_pre)
                wait_vmem<(2 * LPW < 64 ? 2 * LPW : 63)>();
            else
                wait_vmem<0>();
            __syncthreads();
            fill(it + kAhead, ids);

            const uint32_t kcur = k_lds + kslot * KTB;
            const uint32_t vcur = v_lds + vslot * VTB;
            if (!kLag) {
                phase_q(it, kcur, vcur);
                phase_r(v_lds + vslot_back(1) * VTB);
            } else {
                phase_r(v_lds + vslot_back(2) * VTB);
                phase_q(it, kcur, vcur);
            }
            kslot = kslot == kKSlots - 1 ? 0 : kslot + 1;
            vslot = vslot == kVSlots - 1 ? 0 : vslot + 1;
        }
        if (n_tiles > 0) {
            if (kLag)
                phase_r(v_lds + vslot_back(2) * VTB);   // softmax of the last tile
            __syncthreads();             // the last tile's fp16 V is visible
            pv(pb_prev, v_lds + vslot_back(1) * VTB);
        }
    };
    if (lag)
        run(std::true_type{});
    else
        run(std::false_type{});

    // Two wave sets over the same rows: the upper key half's waves leave
    // their (O, running max, sum share) in LDS (the V ring, no longer read)
    // and the lower half's merge them into theirs, as two splits merge.
    if constexpr (KSP == 2) {
        constexpr int kOW = 16 * C::kDTiles;   // O values per lane
        static_assert(NW * (kOW + 2) * 64 * 4 <= kVSlots * VTB, "merge area inside the V ring");
        float *s_po = reinterpret_cast<float *>(s_v);
        float *s_pml = s_po + NW * kOW * 64;
        __syncthreads();   // every wave is past its last read of the ring
        if (half == 1) {
#pragma unroll
            for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s_po[(rw * kOW + 16 * m + e) * 64 + lane] = oacc[m][e];
            s_pml[(2 * rw) * 64 + lane] = m_used;
            s_pml[(2 * rw + 1) * 64 + lane] = lsum;
        }
        __syncthreads();
        if (half == 0) {
            const float m1 = s_pml[(2 * rw) * 64 + lane], l1 = s_pml[(2 * rw + 1) * 64 + lane];
            const float M = fmaxf(m_used, m1);
            if (M != -INFINITY) {
                const float w0 = m_used == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_used - M) * a.c);
                const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * a.c);
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        oacc[m][e] = oacc[m][e] * w0 + s_po[(rw * kOW + 16 * m + e) * 64 + lane] * w1;
                lsum = lsum * w0 + l1 * w1;
                m_used = M;
            }
        }
    }
    // the lower key half's waves (all waves when KSP = 1) own the output
    const bool out_ok = row_ok && half == 0;

    // ---- write the result, or leave a partial, or merge the splits -------------
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float mrow = (m_used == -INFINITY) ? -INFINITY : m_used * a.c;   // log2 units
    auto write_out = [&](const f32x16 (&o)[C::kDTiles], float inv) __attribute__((always_inline)) {
        float *orow = a.out + (((int64_t)b * a.N + node) * a.Hq + head) * D;
        bool finite = true;
#pragma unroll
        for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = {o[m][4 * i] * inv, o[m][4 * i + 1] * inv, o[m][4 * i + 2] * inv,
                                 o[m][4 * i + 3] * inv};
                finite &= __builtin_isfinite(v.x) && __builtin_isfinite(v.y) &&
                          __builtin_isfinite(v.z) && __builtin_isfinite(v.w);
                *reinterpret_cast<f32x4 *>(orow + 32 * m + 8 * i + 4 * hh) = v;
            }
        if (!finite)
            raise_flag(a.flags, TAV_FLAG_ATTN_RANGE);
    };
    if (a.S == 1) {
        if (out_ok)
            write_out(oacc, 1.0f / ltot);
        return;
    }
    const int64_t unit = (int64_t)bh * a.RB + rb;
    const int rloc = rw * 32 + col;
    const int64_t P0 = unit * a.S;
    auto write_partial = [&]() __attribute__((always_inline)) {
        float *po = a.part_o + ((P0 + s) * C::kRows + rloc) * D;
#pragma unroll
        for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = {oacc[m][4 * i], oacc[m][4 * i + 1], oacc[m][4 * i + 2],
                                 oacc[m][4 * i + 3]};
                *reinterpret_cast<f32x4 *>(po + 32 * m + 8 * i + 4 * hh) = v;
            }
        if (hh == 0)
            *reinterpret_cast<f32x2 *>(a.part_ml + ((P0 + s) * C::kRows + rloc) * 2) = f32x2{mrow, ltot};
    };
    if (!a.merge) {
        // more than two splits: every split leaves its partial for the
        // combine kernel
        if (out_ok)
            write_partial();
        return;
    }
    uint32_t *arrived = a.counters + 2 * unit, *done = arrived + 1;
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(a.S - 1);
    __syncthreads();
    // A split leaves its partial with ordinary stores and one write-back of
    // its XCD's L2 before it counts itself done; the merging split reads the
    // partials with agent-scope atomic loads (64 bits each), which are
    // coherent across XCDs at the memory side, so its L2 is not invalidated
    // (that would also drop the K/V tiles the other row block of its XCD is
    // reading).
    auto unpack = [](uint64_t w) __attribute__((always_inline)) {
        return f32x2{__builtin_bit_cast(float, (uint32_t)w), __builtin_bit_cast(float, (uint32_t)(w >> 32))};
    };
    if (!s_last) {
        if (out_ok)
            write_partial();
        wait_vmem<0>();   // this wave's stores are in the L2
        __syncthreads();
        if (tid == 0) {
            // the L2's dirty lines, the partial among them, written back to
            // memory before the count
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    // The last split: the others arrived before it and are past their tile
    // loops, so they finish their partials without waiting on anything; the
    // wait is bounded all the same.
    if (tid == 0) {
        uint32_t polls = 0;
        while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               (uint32_t)(a.S - 1)) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kMergeSpinLimit) {
                raise_flag(a.flags, TAV_FLAG_SYNC_TIMEOUT);
                break;
            }
        }
    }
    __syncthreads();
    if (out_ok) {
        // out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s in split order
        // (a split that saw no key has m_s = -inf and is skipped)
        auto ml_of = [&](int s2) __attribute__((always_inline)) {
            return s2 == s ? f32x2{mrow, ltot}
                           : unpack(__hip_atomic_load(reinterpret_cast<const uint64_t *>(a.part_ml) +
                                                          (P0 + s2) * C::kRows + rloc,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        };
        float M = -INFINITY;
        for (int s2 = 0; s2 < a.S; ++s2)
            M = fmaxf(M, ml_of(s2).x);
        f32x16 acc[C::kDTiles];
#pragma unroll
        for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[m][e] = 0.f;
        float lw = 0.f;
        for (int s2 = 0; s2 < a.S; ++s2) {
            const f32x2 ml = ml_of(s2);
            if (ml.x == -INFINITY)
                continue;
            const float w = __builtin_amdgcn_exp2f(ml.x - M);
            lw += w * ml.y;
            if (s2 == s) {
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[m][e] += w * oacc[m][e];
            } else {
                const uint64_t *po =
                    reinterpret_cast<const uint64_t *>(a.part_o + ((P0 + s2) * C::kRows + rloc) * D);
#pragma unroll
                for (int m = 0; m < C::kDTiles; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = 32 * m + 8 * i + 4 * hh;
                        const f32x2 v0 = unpack(__hip_atomic_load(po + f / 2, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT));
                        const f32x2 v1 = unpack(__hip_atomic_load(po + f / 2 + 1, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT));
                        acc[m][4 * i] += w * v0.x;
                        acc[m][4 * i + 1] += w * v0.y;
                        acc[m][4 * i + 2] += w * v1.x;
                        acc[m][4 * i + 3] += w * v1.y;
                    }
            }
        }
        write_out(acc, 1.0f / lw);
    }
    // leave the counters as the call found them
    if (tid == 0) {
        __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    // The (max, sum) pair and O chunk of up to kCombineBatch splits are
    // requested before any is used, so the loads overlap instead of waiting
    // on one another: every split count the planner makes for a batch of one
    // (up to 16) is a single round trip to memory. A split that saw no key
    // has max -inf, O = 0 and sum 0; it is skipped.
    constexpr int kCombineBatch = 16;
    f32x2 ml[kCombineBatch];
    f32x4 v[kCombineBatch];
    auto load_batch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            if (s0 + k < a.S) {
                const int64_t pr = (P0 + s0 + k) * rows_per_block + rloc;
                ml[k] = *reinterpret_cast<const f32x2 *>(a.part_ml + pr * 2);
                v[k] = *reinterpret_cast<const f32x4 *>(a.part_o + pr * D + dq * 4);
            }
        }
    };
    load_batch(0);
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
        if (k < a.S)
            M = fmaxf(M, ml[k].x);
    for (int s = kCombineBatch; s < a.S; ++s)
        M = fmaxf(M, a.part_ml[((P0 + s) * rows_per_block + rloc) * 2]);
    float lsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.S; s0 += kCombineBatch) {
        if (s0 > 0)
            load_batch(s0);
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            if (s0 + k < a.S && ml[k].x != -INFINITY) {
                const float w = __builtin_amdgcn_exp2f(ml[k].x - M);
                lsum += w * ml[k].y;
                o += w * v[k];
            }
        }
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
    bool merge;   // the two splits merge inside the launch
    int64_t grid;
    size_t counter_bytes, part_o_bytes, part_ml_bytes, ws_bytes;
};

size_t round_up(size_t v, size_t al) { return (v + al - 1) / al * al; }

// Splits of a prefix: at least kMinTilesPerSplit tiles each and at most
// kMaxSplits of them (where the block-table bound below allows). Measured at
// batch one (8B-shaped 64-node trees over 4096 tokens, 16-node trees over
// 2048): 16 splits beat both 8 and 32, each split's fixed cost (Q, the
// first tiles' latency, its partial) against the tiles it shares out.
constexpr int kMinTilesPerSplit = 2;
constexpr int kMaxSplits = 16;

template <int D>
const void *kernel_for(int NW)
{
    return NW == 8 ? reinterpret_cast<const void *>(tree_attn_kernel<D, 8>)
                   : reinterpret_cast<const void *>(tree_attn_kernel<D, 4, 2>);
}

// Wave sets per workgroup: up to 128 query rows per (sequence, KV head) a
// workgroup takes 128 rows (four row waves, padding rows included) and
// splits the keys of every tile between two sets of them, eight waves, two
// per SIMD (a tile's chain of work per wave is about the same length at any
// row count, so more waves per CU is what shortens the launch).
constexpr int ksp_for(int NW)
{
    return NW == 8 ? 1 : 2;
}

int waves_for(int32_t N, int32_t Hq, int32_t Hkv)
{
    const int NG = N * (Hq / Hkv);
    return NG > 128 ? 8 : 4;   // see ksp_for
}

// The decomposition with NW row waves per workgroup (32 query rows each): row
// blocks (RB) and prefix splits (S), enough workgroups to fill a device of
// `cus` compute units holding `per_cu` workgroups each once.
void attn_plan_nw(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                  int32_t max_prefix_len, int cus, int per_cu, int NW, AttnPlan &p)
{
    const int G = Hq / Hkv;
    const int NG = N * G;
    p.NW = NW;
    p.rows = 32 * p.NW;
    p.RB = (int)ceil_div(NG, p.rows);
    const int64_t base = (int64_t)B * Hkv * p.RB;
    const int64_t target = (int64_t)cus * per_cu;
    const int64_t tiles = std::max<int64_t>(1, ceil_div(max_prefix_len, kKT));
    int64_t S = ceil_div(target, base);
    S = std::max<int64_t>(1, std::min<int64_t>({S, tiles / kMinTilesPerSplit, (int64_t)kMaxSplits}));
    // A split's block-table slice must fit its LDS copy. Split s takes units
    // [s U / S, (s + 1) U / S) of the U = prefix tiles + tree tiles, so it
    // can hold up to ceil(U / S) prefix tiles: the bound counts every unit.
    const int64_t max_tiles_per_split = kMaxSplitBlocks / (kKT / kBlock);
    const int64_t units = tiles + ceil_div(N, kKT);
    S = std::max<int64_t>(S, ceil_div(units, max_tiles_per_split));
    p.S = (int)S;
    p.KS = (int)((int64_t)B * Hkv * p.S);
    p.grid = ceil_div(p.KS, 8) * 8 * p.RB;
    p.merge = p.S == 2;
    if (p.S > 1) {
        p.counter_bytes = p.merge ? (size_t)B * Hkv * p.RB * 2 * sizeof(uint32_t) : 0;
        p.part_o_bytes = (size_t)B * Hkv * p.RB * p.S * p.rows * D * sizeof(float);
        p.part_ml_bytes = (size_t)B * Hkv * p.RB * p.S * p.rows * 2 * sizeof(float);
    } else {
        p.counter_bytes = p.part_o_bytes = p.part_ml_bytes = 0;
    }
    p.ws_bytes = p.S > 1 ? round_up(p.counter_bytes, 256) + round_up(p.part_o_bytes, 256) +
                               round_up(p.part_ml_bytes, 256)
                         : 0;
}

// Work decomposition for a shape. Pure arithmetic (no device call), so it can
// be checked on the host. Above 128 query rows per (sequence, KV head) the
// 8-row-wave form, unless its plan is dominated by splits, where the 4-row-
// wave form with its two key sets makes twice the row blocks and so needs
// half the splits (each split's fp32 partial is written and read back once
// more): at most 256 rows, when the 8-row-wave form cannot fill the device
// or needs 8 splits or more to fill it; above, only when filling it takes
// the split cap.
// Measured side by side: the 8B-shaped batch one 32.3 -> 27.4 us, batch 4
// 48.0 -> 44.8 us; the 70B-shaped batch one 42.0 -> 39.9 us and one KV head
// of its batch 8 43.3 -> 42.2 us; but the 70B-shaped batch 2 (8 splits, 512
// rows) 57.3 against 58.7 us, and the 8B-shaped batch 8 and 32, where the
// 8-row-wave form fills the device with few splits, 66.0 against 68.5 and
// 156 against 191 us, so these keep it.
void attn_plan_for(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t max_prefix_len, int cus, int per_cu, AttnPlan &p)
{
    attn_plan_nw(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu, waves_for(N, Hq, Hkv), p);
    if (p.NW != 8)
        return;
    // the splits filling the device would take, before the caps and the
    // block-table bound (which long prefixes raise on a full device too)
    const int64_t NG = (int64_t)N * (Hq / Hkv);
    const int64_t S_fill = ceil_div((int64_t)cus * per_cu, (int64_t)B * Hkv * p.RB);
    const bool try4 = NG <= 256 ? (p.grid < (int64_t)cus * per_cu || S_fill >= 8)
                                : S_fill >= kMaxSplits;
    if (try4) {
        AttnPlan q;
        attn_plan_nw(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu, 4, q);
        if (q.grid > p.grid || q.S < p.S)
            p = q;
    }
}

// The same for the current device.
bool attn_plan(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_prefix_len,
               AttnPlan &p)
{
    const int cus = device_cu_count();
    if (cus <= 0)
        return false;
    const int NW = waves_for(N, Hq, Hkv);
    const void *fn = D == 128 ? kernel_for<128>(NW) : kernel_for<64>(NW);
    const int per_cu = kernel_occupancy(fn, NW * ksp_for(NW) * 64);
    if (per_cu <= 0)
        return false;
    attn_plan_for(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu, p);
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
    constexpr int KSP = ksp_for(NW);
    hipLaunchKernelGGL((tree_attn_kernel<D, NW, KSP>), dim3((unsigned)p.grid), dim3(NW * KSP * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const AttnPlan &p, const AttnArgs &a, hipStream_t s)
{
    return p.NW == 8 ? launch_main<D, 8>(p, a, s) : launch_main<D, 4>(p, a, s);
}

} // namespace
} // namespace tav

extern "C" tav_status tav_attn_plan(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_prefix_len, int32_t cus, int32_t per_cu,
                                    int32_t *plan)
{
    using namespace tav;
    if (!plan || cus < 1 || per_cu < 1)
        return TAV_ERR_ARG;
    if (!attn_shape_ok(B, N, Hq, Hkv, D, max_prefix_len))
        return TAV_ERR_UNSUPPORTED;
    AttnPlan p;
    attn_plan_for(B, N, Hq, Hkv, D, max_prefix_len, cus, per_cu, p);
    // the largest prefix-tile count of any split, over every prefix length up
    // to max_prefix_len (longer prefixes give every split at least as many)
    const int64_t Tb = ceil_div(max_prefix_len, kKT);
    const int64_t Ub = Tb + ceil_div(N, kKT);
    int64_t most = 0;
    for (int64_t s = 0; s < p.S; ++s) {
        const int64_t u0 = s * Ub / p.S, u1 = (s + 1) * Ub / p.S;
        most = std::max(most, std::min(u1, Tb) - std::min(u0, Tb));
    }
    plan[0] = p.NW * ksp_for(p.NW);
    plan[1] = p.RB;
    plan[2] = p.S;
    plan[3] = (int32_t)(most * (kKT / kBlock));
    plan[4] = kMaxSplitBlocks;
    return TAV_OK;
}

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

namespace tav {
namespace {

// The launch behind tree_attn_verify and tree_attn_verify_tree: exactly one
// of mask and parent is non-NULL.
tav_status attn_launch(const uint16_t *q, const uint16_t *k_tree, const uint16_t *v_tree,
                       const uint16_t *k_cache, const uint16_t *v_cache, int32_t num_blocks,
                       const int32_t *block_table, int32_t max_blocks, const int32_t *prefix_len,
                       int32_t max_prefix_len, const uint64_t *mask, const int32_t *parent,
                       uint64_t *mask_out, int32_t *depth_out, int32_t B, int32_t N, int32_t Hq,
                       int32_t Hkv, int32_t D, int32_t block_size, float scale, float *out,
                       void *workspace, size_t ws_bytes, uint32_t *dev_flags, void *stream)
{
    if (!q || !k_tree || !v_tree || !k_cache || !v_cache || !block_table || !prefix_len ||
        (!mask && !parent) || !out)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1 ||
        max_prefix_len < 0 || !(scale > 0.0f) || !(scale < INFINITY))
        return TAV_ERR_ARG;
    if (!attn_shape_ok(B, N, Hq, Hkv, D, max_prefix_len) || block_size != kBlock ||
        (int64_t)num_blocks * Hkv > (int64_t)UINT32_MAX)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || (mask && !aligned(mask, 8)) || (parent && !aligned(parent, 4)) ||
        (mask_out && !aligned(mask_out, 8)) || (depth_out && !aligned(depth_out, 4)) ||
        !aligned(out, 16) || !aligned(block_table, 4) || !aligned(prefix_len, 4))
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
    a.parent = parent;
    a.mask_out = mask_out;
    a.depth_out = depth_out;
    a.out = out;
    // workspace: the merge counters, then the partials O and (max, sum)
    char *ws = static_cast<char *>(workspace);
    a.counters = p.merge ? reinterpret_cast<uint32_t *>(ws) : nullptr;
    a.merge = p.merge ? 1 : 0;
    a.part_o = p.S > 1 ? reinterpret_cast<float *>(ws + round_up(p.counter_bytes, 256)) : nullptr;
    a.part_ml = p.S > 1 ? reinterpret_cast<float *>(ws + round_up(p.counter_bytes, 256) +
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
    if (p.S > 1 && !p.merge) {
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

} // namespace
} // namespace tav

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
    if (!mask)
        return TAV_ERR_ARG;
    return tav::attn_launch(q, k_tree, v_tree, k_cache, v_cache, num_blocks, block_table,
                            max_blocks, prefix_len, max_prefix_len, mask, nullptr, nullptr,
                            nullptr, B, N, Hq, Hkv, D, block_size, scale, out, workspace,
                            ws_bytes, dev_flags, stream);
}

extern "C" tav_status tree_attn_verify_tree(const uint16_t *q, const uint16_t *k_tree,
                                            const uint16_t *v_tree, const uint16_t *k_cache,
                                            const uint16_t *v_cache, int32_t num_blocks,
                                            const int32_t *block_table, int32_t max_blocks,
                                            const int32_t *prefix_len, int32_t max_prefix_len,
                                            const int32_t *parent, uint64_t *mask_out,
                                            int32_t *depth_out, int32_t B, int32_t N,
                                            int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t block_size, float scale, float *out,
                                            void *workspace, size_t ws_bytes,
                                            uint32_t *dev_flags, void *stream)
{
    if (!parent)
        return TAV_ERR_ARG;
    return tav::attn_launch(q, k_tree, v_tree, k_cache, v_cache, num_blocks, block_table,
                            max_blocks, prefix_len, max_prefix_len, nullptr, parent, mask_out,
                            depth_out, B, N, Hq, Hkv, D, block_size, scale, out, workspace,
                            ws_bytes, dev_flags, stream);
}
