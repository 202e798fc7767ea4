// spec_verify_sample: target/draft softmax over the vocabulary and the
// root-down rejection-sampling walk, in float64 arithmetic except the
// per-token exponentials of the vocabulary-wide sums (see "exp." below).
//
// The rule (radar-34b blog §2, rejection-sampling acceptance condition): a
// draft x drawn from q is kept with probability min(1, p(x)/q(x)); on a
// rejection the next draw comes from the normalised positive part of p - q.
// One target pass yields a distribution at every node plus one more, so a
// fully accepted path still emits a bonus token (LLM Primer ch. 9, §9.1).
// Nodes are decided from the root down, depth first (jisaku.com glossary,
// SpecInfer). Children are tried in ascending node index against the running
// residual; uniforms come from Philox (philox.h).
//
// Layout of the work. A "group" of wpg workgroups owns one sequence at a
// time; workgroup r of the group owns vocabulary entries
// [r*chunk, (r+1)*chunk) and keeps them in registers (8 or 16 per thread,
// 512 threads; at large batches 16 in registers and 12 more in LDS), so
// every pass over a row after the first stays on the CU.
// The walk is serial; for each visited node u the group
//   1. takes its chunk of target row u (and draft row u if u has children)
//      and the logits of u's children's tokens; each wave reduces a local
//      (max, sum exp) per row with DPP, wave 0 merges the waves' pairs and
//      exchanges the chunk's pair with the group (one group sync), then
//      merges the wpg pairs in member order, so every workgroup holds
//      bit-identical normalisers and per-chunk masses. Wave 0 also takes
//      p(x) and q(x) of every child's token (one lane per child);
//   2. tests the children in order against the running residual, from those
//      values and the node's Philox uniforms (all computed once per
//      sequence), the same instructions in every workgroup, so every
//      workgroup takes the same decision. Meanwhile the rows of u's first
//      child, the likeliest next node, are already being fetched, so a walk
//      down first children never waits on memory;
//   3. after each rejection exchanges the chunk sums of max(0, p_res - q)
//      (one group sync), which give the new normaliser and the new chunk
//      masses, and updates its registers;
//   4. if it stops at u, every workgroup already holds the chunk masses of
//      the final distribution; the one workgroup whose prefix interval holds
//      r * total scans its chunk, so the draw costs no further sync.
//
// Group sync. Each workgroup owns a 64-byte mailbox slot per parity: up to
// eight 64-bit words, each carrying the sync's generation in its high half
// and 32 bits of payload in its low half (fp32 maxima as they are, fp64 sums
// split in two). Words are written and read with agent-scope 64-bit atomics,
// which are single-copy atomic and stay coherent across XCDs at the memory
// side, so no cache is flushed or invalidated and no write has to be
// acknowledged before another: wave 0 polls a member's words (one lane per
// member) until every one carries the current generation. Two parities
// suffice: a member can only reuse a slot after every member has arrived at
// the sync in between, i.e. after everyone has read it. The grid never
// exceeds what the device holds resident at once (from the occupancy query),
// and every wait is bounded: on expiry the kernel raises
// TAV_FLAG_SYNC_TIMEOUT and the workgroup stops, so every wave exits even on
// a device shared with other work. The last workgroup to finish clears every
// slot, so each call leaves the workspace as it found it (zero-filled).
//
// exp. The stats pass takes one exponential per vocabulary entry and row,
// which makes it bound by the vector ALUs; those are fp32 (y = x/T - m to
// one rounding, then v_exp_f32) and are summed in fp64, so the entries that
// carry a sum are within a few 1e-7. The rebasing of partial sums to the
// row's maximum and p and q at a child's token use exp_bulk (an fp32 head and
// an fp64 tail, 1e-7 relative): a decision can then differ from one taken in
// exact arithmetic only for a draw within a few 1e-7 of its boundary. exp_f64,
// a table-free fp64 routine within one ulp, serves tav_target_probs.

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "philox.h"


namespace tav {
namespace {

constexpr int kSvThreads = 512;
constexpr int kSvWaves = kSvThreads / 64;
constexpr int kSvEpt = 8;                       // vocabulary entries per thread
constexpr int kSvChunk = kSvThreads * kSvEpt;   // per workgroup
constexpr int kMaxWpg = kSvThreads;             // workgroups per sequence (one slot per thread)
constexpr int64_t kMaxVocab = (int64_t)1 << 21;
constexpr uint32_t kSpinLimit = 1u << 20;       // polls before a wait gives up
constexpr int kSlotWords = 8;                   // 64-byte slot of tagged 64-bit words
constexpr size_t kHeaderBytes = 256;            // exit counter

static_assert(kMaxVocab <= (int64_t)kSvChunk * kMaxWpg, "vocabulary limit");

struct SvArgs {
    const float *tl;
    const float *dl;
    const int32_t *parent;
    const int32_t *token;
    int32_t B, N, V;
    double T;
    uint64_t seed, offset;
    int32_t *path;
    int32_t *n_acc;
    int32_t *out_tok;
    uint32_t *done;   // exit counter
    uint64_t *box;    // [ngroups][2][wpg][kSlotWords]
    uint32_t *flags;
    int32_t wpg, ngroups, chunk;
    int32_t vec4;     // rows can be read 16 bytes at a time (V % 4 == 0, aligned logits)
    // probe outputs (kProbe): the softmax rows the walk holds at each visited
    // node, and p, q of each tested child's token as the walk decides with them
    double *p_rows;   // [B][N][V]
    double *q_rows;   // [B][N][V]
    double *child_pq; // [B][N][2]
    CommitArgs cm;
};

// ---------------------------------------------------------------------------
// exp in float64 without a table: x = n ln2 + r with |r| <= ln2/2 (ln 2 in
// two parts, so n*hi is exact), e^r - 1 = r + r^2 (1/2! + r/3! + ... +
// r^11/13!) with the bracket evaluated by Estrin's scheme (a short dependency
// chain), then 2^n (1 + (e^r - 1)). The truncation error is below 5e-18;
// the result is within one ulp (checked on the CPU against a 40-digit
// reference over 45000 arguments).

__device__ __forceinline__ double exp_f64(double x)
{
    if (x < -746.0)
        return 0.0;   // below the smallest subnormal (also x = -inf)
    constexpr double kLog2e = 0x1.71547652b82fep+0;
    constexpr double kLn2Hi = 0x1.62e42fee00000p-1;
    constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;
    constexpr double kRound = 0x1.8p52;
    x = fmin(x, 709.0);
    const double nd = (x * kLog2e + kRound) - kRound;   // nearest integer to x/ln2
    const int n = (int)nd;
    double r = fma(-nd, kLn2Hi, x);
    r = fma(-nd, kLn2Lo, r);
    const double r2 = r * r, r4 = r2 * r2, r8 = r4 * r4;
    const double a0 = fma(1.0 / 6.0, r, 1.0 / 2.0);
    const double a1 = fma(1.0 / 120.0, r, 1.0 / 24.0);
    const double a2 = fma(1.0 / 5040.0, r, 1.0 / 720.0);
    const double a3 = fma(1.0 / 362880.0, r, 1.0 / 40320.0);
    const double a4 = fma(1.0 / 39916800.0, r, 1.0 / 3628800.0);
    const double a5 = fma(1.0 / 6227020800.0, r, 1.0 / 479001600.0);
    const double b0 = fma(a1, r2, a0), b1 = fma(a3, r2, a2), b2 = fma(a5, r2, a4);
    const double q = fma(b2, r8, fma(b1, r4, b0));
    return ldexp(1.0 + fma(r2, q, r), n);
}

// The vocabulary-wide terms exp(y), y <= 0: 2^t with t = y log2(e) split into
// an fp32 head (v_exp_f32, under one fp32 ulp) and an fp64 tail, 2^tl taken to
// first order. Within 1e-7 relative (8.2e-8 measured over [-80, 0]); terms
// below 2^-126 of the row's maximum flush to zero. Sums and decisions stay in
// fp64, so a decision can differ from an all-fp64 one only for a draw within
// about 1e-7 of its boundary.
__device__ __forceinline__ double exp_bulk(double y)
{
    constexpr double kLog2e = 0x1.71547652b82fep+0;
    constexpr double kLn2 = 0x1.62e42fefa39efp-1;
    const double t = y * kLog2e;
    const float th = (float)t;
    const double tl = t - (double)th;
    const float e = __builtin_amdgcn_exp2f(th);
    return y < -745.0 ? 0.0 : (double)e * fma(tl, kLn2, 1.0);
}

// ---------------------------------------------------------------------------
// Reductions. Within a wave: DPP butterflies inside each 16-lane row, then
// the four row totals read out and combined in a fixed order, so every lane
// holds the same bits. Across the workgroup: the waves' totals in index order.

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF,
                                                              false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                              0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double lane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<kQuadSwap1>(v);
    v += dpp_f64<kQuadSwap2>(v);
    v += dpp_f64<kRowHalfMirror>(v);
    v += dpp_f64<kRowMirror>(v);
    return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
}

__device__ __forceinline__ double wave_max(double v)
{
    v = fmax(v, dpp_f64<kQuadSwap1>(v));
    v = fmax(v, dpp_f64<kQuadSwap2>(v));
    v = fmax(v, dpp_f64<kRowHalfMirror>(v));
    v = fmax(v, dpp_f64<kRowMirror>(v));
    return fmax(fmax(lane_f64(v, 0), lane_f64(v, 16)), fmax(lane_f64(v, 32), lane_f64(v, 48)));
}

// The same for fp32 values (32-bit DPP: half the moves of the fp64 form),
// with the IEEE maximum, which propagates NaN: a NaN anywhere in the wave is
// the result.
__device__ __forceinline__ float fmax_nan(float a, float b)
{
    return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float wave_max_f32(float v)
{
    v = fmax_nan(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kQuadSwap1, 0xF, 0xF, false)));
    v = fmax_nan(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kQuadSwap2, 0xF, 0xF, false)));
    v = fmax_nan(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kRowHalfMirror, 0xF, 0xF, false)));
    v = fmax_nan(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kRowMirror, 0xF, 0xF, false)));
    const int u = __builtin_bit_cast(int, v);
    return fmax_nan(fmax_nan(__builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0)),
                             __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16))),
                    fmax_nan(__builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32)),
                             __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48))));
}

// Inclusive prefix sums over the wave in a fixed order: a Hillis-Steele
// scan inside each 16-lane row (DPP row shifts), then the rows' totals
// carried across in row order. Every caller with the same inputs gets the
// same bits, and lane 63 holds the total.
__device__ __forceinline__ double wave_scan_incl(double v)
{
    v += dpp_f64<0x111>(v);   // row_shr:1 (0 where the row has no lane below)
    v += dpp_f64<0x112>(v);   // row_shr:2
    v += dpp_f64<0x114>(v);   // row_shr:4
    v += dpp_f64<0x118>(v);   // row_shr:8
    const double c1 = lane_f64(v, 15);
    const double c2 = c1 + lane_f64(v, 31);
    const double c3 = c2 + lane_f64(v, 47);
    const int row = (int)(threadIdx.x & 63) >> 4;
    return row == 0 ? v : v + (row == 1 ? c1 : row == 2 ? c2 : c3);
}

// The value of the lane below (0 in lane 0): DPP wave_shr:1.
__device__ __forceinline__ double wave_shift_up1(double v)
{
    return dpp_f64<0x138>(v);
}

// Workgroup-wide reductions of two values at once; every thread gets the
// results. `red` holds 2 * kSvWaves doubles.
__device__ void block_sum2(double &a, double &b, double *red)
{
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[wave] = a;
        red[kSvWaves + wave] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int w = 0; w < kSvWaves; ++w) {
        a += red[w];
        b += red[kSvWaves + w];
    }
}

__device__ void block_max2(double &a, double &b, double *red)
{
    a = wave_max(a);
    b = wave_max(b);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[wave] = a;
        red[kSvWaves + wave] = b;
    }
    __syncthreads();
    a = -INFINITY;
    b = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSvWaves; ++w) {
        a = fmax(a, red[w]);
        b = fmax(b, red[kSvWaves + w]);
    }
}

// ---------------------------------------------------------------------------
// Group sync.

__device__ __forceinline__ uint64_t tag_word(uint32_t gen, uint32_t payload)
{
    return ((uint64_t)gen << 32) | payload;
}

// Wave 0 only. Lanes 0..NW-1 publish word i = mine (lane i's payload) in
// this workgroup's slot for generation `gen`; then lane l polls members l,
// l+64, ... and keeps member l's payloads in w0[0..NW) (registers) and
// member m's for m >= 64 in got[m][0..NW) (LDS, read back by the same lane).
// Returns false on a timeout (every lane).
template <int NW>
__device__ bool wave0_exchange(uint64_t *box, int wpg, int rank, uint32_t gen, uint32_t mine,
                               uint32_t (*got)[kSlotWords], uint32_t (&w0)[NW])
{
    const int lane = threadIdx.x & 63;
    uint64_t *base = box + (size_t)(gen & 1u) * wpg * kSlotWords;
    if (lane < NW)
        __hip_atomic_store(base + (size_t)rank * kSlotWords + lane, tag_word(gen, mine),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    for (int m = lane; m < wpg && ok; m += 64) {
        uint64_t *slot = base + (size_t)m * kSlotWords;
        uint32_t polls = 0;
        for (;;) {
            uint64_t word[NW];
#pragma unroll
            for (int i = 0; i < NW; ++i)
                word[i] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool all = true;
#pragma unroll
            for (int i = 0; i < NW; ++i)
                all &= (uint32_t)(word[i] >> 32) == gen;
            if (all) {
#pragma unroll
                for (int i = 0; i < NW; ++i) {
                    if (m == lane)
                        w0[i] = (uint32_t)word[i];
                    else
                        got[m][i] = (uint32_t)word[i];
                }
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kSpinLimit) {
                ok = false;
                break;
            }
        }
    }
    return !__any(!ok);
}

__device__ __forceinline__ uint32_t f32_bits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bits_f32(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t f64_hi(double v)
{
    return (uint32_t)(__builtin_bit_cast(uint64_t, v) >> 32);
}
__device__ __forceinline__ uint32_t f64_lo(double v) { return (uint32_t)__builtin_bit_cast(uint64_t, v); }
__device__ __forceinline__ double bits_f64(uint32_t hi, uint32_t lo)
{
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------

// The group's share of sequence b's KV commit: path rows 0..m (s_path, in
// LDS) to positions prefix_len[b] + t, work items (row, KV head, 16-byte
// chunk) spread over the group's members; member 0 writes the slots and the
// new length. Bad entries raise the flags kv_commit_path raises.
__device__ void commit_path_rows(const CommitArgs &c, int b, int N, int m, const int32_t *s_path,
                                 int rank, int wpg, int tid, uint32_t *flags)
{
    const int32_t L = c.prefix_len[b];
    const int64_t rowbase = (int64_t)b * N;
    if (rank == 0) {
        for (int t = tid; t < N; t += kSvThreads) {
            int32_t slot = -1;
            if (t <= m) {
                const int64_t pos = (int64_t)L + t;
                const int64_t lb = pos / kBlock;
                if (L >= 0 && lb < c.max_blocks) {
                    const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + lb];
                    if (blk >= 0 && blk < c.num_blocks)
                        slot = blk * kBlock + (int32_t)(pos % kBlock);
                }
            }
            c.commit_slots[rowbase + t] = slot;
        }
        if (tid == 0)
            c.new_prefix_len[b] = L + m + 1;
    }
    if (L < 0)
        return;
    const int cpr = c.D / 8;
    const int64_t items = (int64_t)(m + 1) * c.Hkv * cpr;
    for (int64_t it = (int64_t)rank * kSvThreads + tid; it < items; it += (int64_t)wpg * kSvThreads) {
        const int ch = (int)(it % cpr);
        const int h = (int)((it / cpr) % c.Hkv);
        const int t = (int)(it / ((int64_t)cpr * c.Hkv));
        const int32_t node = s_path[t];
        const int64_t pos = (int64_t)L + t;
        const int64_t lb = pos / kBlock;
        if (lb >= c.max_blocks) {
            raise_flag(flags, TAV_FLAG_CAPACITY);
            continue;
        }
        const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + lb];
        if (blk < 0 || blk >= c.num_blocks) {
            raise_flag(flags, TAV_FLAG_BAD_BLOCK);
            continue;
        }
        const int sl = (int)(pos % kBlock);
        const int64_t src = ((rowbase + node) * c.Hkv + h) * c.D + ch * 8;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(c.k_tree + src);
        *reinterpret_cast<u32x4 *>(c.k_cache + (((int64_t)blk * c.Hkv + h) * kBlock + sl) * c.D + ch * 8) = kv;
        const u32x4 vv = *reinterpret_cast<const u32x4 *>(c.v_tree + src);
        uint16_t *vdst = c.v_cache + (((int64_t)blk * c.Hkv + h) * c.D + ch * 8) * kBlock + sl;
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vdst[e * kBlock] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
}

// kWor selects the sibling rule: false, every child of u is tested with q_u
// (siblings drawn independently from q_u); true, a rejected child's token
// leaves q_u, the rest renormalised, before the next sibling is tried
// (siblings drawn from q_u without replacement). kProbe also writes, at each
// visited node, the normalised p and q the walk holds in registers and the
// p, q of its children's tokens that the child tests read; nothing else
// changes.
//
// E is the number of vocabulary entries each thread holds (a workgroup holds
// 512 E), so a sequence's group has ceil(V / 512 E) members: fewer, larger
// members let more sequences walk at once when the batch is large. Each entry
// keeps only its two fp32 exponentials (target and draft, relative to its
// wave's maximum); the fp64 values the walk decides with (p, q and the
// residual after k rejections at the current node) are formed from them
// when needed, by the same operations in the same order every time, so they
// are the same bits whenever they are formed.
// One direct HBM -> LDS load: lane l's 16 bytes at base + voff land at LDS
// byte address lds_addr + 16 l (base and lds_addr the same for the whole
// wave). Inline assembly, so the compiler neither makes later LDS accesses
// wait for it nor reasons about what it writes: a reader of the destination
// first waits with sv_wait_loads.
__device__ __forceinline__ void sv_load_lds16(const void *base, uint32_t voff, uint32_t lds_addr)
{
    // (both are the same in every lane; the compiler cannot always tell)
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(bs), "s"(ls)
                 : "memory", "m0");
}

// Every vector memory load of the wave complete (its LDS writes included).
__device__ __forceinline__ void sv_wait_loads()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// This wave's LDS accesses complete.
__device__ __forceinline__ void sv_wait_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t sv_lds_addr(T *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)p;
}

template <int E, bool kWor, bool kProbe = false>
__global__ __launch_bounds__(kSvThreads) void spec_verify_kernel(SvArgs a)
{
    static_assert(E % 4 == 0, "whole 16-byte runs");
    // Entries e < ER are held in registers. With E > 16 the other EL per
    // thread keep their exponentials in LDS, in two buffers: one holds the
    // current node's, the other takes the logits of the node fetched ahead
    // (direct HBM -> LDS loads) while the current node is decided. Thread
    // tid only ever touches its own slots, so no barrier guards them.
    constexpr int ER = E > 16 ? 16 : E;
    constexpr int EL = E - ER;
    constexpr int kLRuns = EL / 4;
    __shared__ f32x4 s_lx[EL ? 2 : 1][EL ? kLRuns : 1][2][EL ? kSvThreads : 1];
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_path[kMaxNodes];   // accepted path, for the fused commit
    __shared__ int32_t s_first[kMaxNodes];
    __shared__ int32_t s_next[kMaxNodes];
    constexpr int kKidWords = kMaxNodes / 64;
    __shared__ unsigned long long s_kids[kMaxNodes][kKidWords];   // children of each node, as bits
    __shared__ int32_t s_tok[kMaxNodes];
    __shared__ float s_tx[kMaxNodes];     // target logit of child c's token in its parent's row
    __shared__ float s_dx[kMaxNodes];     // draft logit of the same
    __shared__ double s_red[2 * kSvWaves];
    __shared__ double s_wq[4 * kSvWaves];   // per wave: raw max t, sum t, raw max q, sum q
    __shared__ double s_norm[4];            // Mp, Zp, Mq, Zq of the whole row
    __shared__ double s_uacc[kMaxNodes];    // node i's acceptance uniform
    __shared__ double s_ures[kMaxNodes];    // node i's resampling uniform
    __shared__ double s_px[kMaxNodes];      // p and q of child c's token at its parent
    __shared__ double s_qx[kMaxNodes];
    __shared__ int s_sync_ok;
    __shared__ uint32_t s_words[kMaxWpg][kSlotWords];   // the group's payloads, as wave 0 received them
    __shared__ double s_mass[kMaxWpg];    // mass of every member's chunk in the current distribution
    __shared__ double s_zhist[kMaxNodes]; // residual normalisers after each rejection at u
    // without replacement: after j rejections at u, q_j = q * s_qs[j] off the
    // removed tokens (s_qs[0] = 1 is implied); s_rtok[j] = token rejected at step j
    __shared__ double s_qs[kWor ? kMaxNodes + 1 : 1];
    __shared__ int32_t s_rtok[kWor ? kMaxNodes : 1];
    __shared__ double s_slot[E * kSvWaves];
    __shared__ double s_hit_off;
    __shared__ int s_bad;
    __shared__ int s_found;
    __shared__ int s_last_live;
    __shared__ int s_hit;
    __shared__ int s_owner;   // the member whose interval holds the draw
    __shared__ int s_is_last;

    const int g = blockIdx.x % a.ngroups;
    const int rank = blockIdx.x / a.ngroups;
    const int tid = threadIdx.x;
    const int N = a.N;
    const int wpg = a.wpg;
    const int64_t base = (int64_t)rank * a.chunk;
    const int64_t lim = std::min<int64_t>((int64_t)a.V, base + a.chunk);
    // This thread's entries of the chunk: run h (of two) holds tokens
    // base + h * 4 * 512 + 4 tid + j, j < 4, read as one 16-byte load where
    // the row allows it (the chunk is a multiple of 4 tokens).
    constexpr int kRun = 4 * kSvThreads;
    // (token ids fit 32 bits: V <= 2^21)
    const int32_t base32 = (int32_t)base;
    auto tok = [&](int e) __attribute__((always_inline)) {
        return base32 + (e >> 2) * kRun + 4 * tid + (e & 3);
    };
    auto load_row = [&](const float *row, float (&v)[ER]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < ER / 4; ++h) {
            const int64_t i0 = base + (int64_t)h * kRun + 4 * tid;
            if (a.vec4 && i0 + 3 < lim) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(row + i0);
                v[4 * h] = x.x;
                v[4 * h + 1] = x.y;
                v[4 * h + 2] = x.z;
                v[4 * h + 3] = x.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[4 * h + j] = i0 + j < lim ? row[i0 + j] : -INFINITY;
            }
        }
    };
    auto no_row = [&](float (&v)[ER]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < ER; ++e)
            v[e] = -INFINITY;
    };
    // The LDS entries' runs of a node's target row (and draft row, if the
    // node has children) into buffer `buf`: run hl holds tokens
    // base + (ER / 4 + hl) * kRun + 4 tid + j. Tokens past the chunk are
    // masked where they are read; a run past the row reads the row's first
    // run instead, so no address leaves the row. Rows that are not 16-byte
    // aligned go through registers.
    const int wave_s = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t lim32 = (int32_t)lim;
    // how many of run h's four tokens lie in the chunk (32-bit arithmetic)
    auto run_valid = [&](int h) __attribute__((always_inline)) {
        return std::min(4, std::max(0, lim32 - (base32 + h * kRun + 4 * tid)));
    };
    auto stage_rows = [&](int buf, const float *trow, const float *drow,
                          bool kids) __attribute__((always_inline)) {
        if constexpr (EL > 0) {
            sv_wait_lds();   // this thread's earlier accesses of the buffer are done
#pragma unroll
            for (int hl = 0; hl < kLRuns; ++hl) {
                const int32_t i0 = base32 + (ER / 4 + hl) * kRun + 4 * tid;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    if (r == 1 && !kids)
                        break;
                    const float *row = r ? drow : trow;
                    if (a.vec4) {
                        const uint32_t voff = i0 < a.V ? (uint32_t)(4 * i0) : 0u;
                        sv_load_lds16(row, voff, sv_lds_addr(&s_lx[buf][hl][r][64 * wave_s]));
                    } else {
                        const int nv = run_valid(ER / 4 + hl);
                        f32x4 x;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            x[j] = j < nv ? row[i0 + j] : -INFINITY;
                        s_lx[buf][hl][r][tid] = x;
                    }
                }
            }
        }
    };
    uint64_t *box = a.box + (size_t)g * 2 * wpg * kSlotWords;
    const double invT = 1.0 / a.T;
    // The reference maxima that the vocabulary-wide sums are taken against
    // are fp32 products fl(m * invT32), the same values in every rebase, so
    // the sums stay consistent with each other (and exact in m for T = 1).
    const float invT32 = (float)invT;
    constexpr float kLog2eF = 0x1.715476p+0f;
    uint32_t gen = 0;
    bool alive = true;
    int lb = 0;   // the LDS buffer of the current node's entries

    for (int b = g; b < a.B && alive; b += a.ngroups) {
        const int64_t rowbase = (int64_t)b * N;
        // ---- the root's rows first: the walk starts there --------------------
        // Rows of the likeliest next node, fetched a level ahead into
        // registers (while the current node is decided) when they fit: with
        // up to 16 entries per thread. Larger E reads each node's rows when
        // it reaches it.
        constexpr bool kPrefetch = ER <= 16;
        constexpr int PE = kPrefetch ? ER : 4;
        int pf_node = kPrefetch ? 0 : -1;
        float pf_t[PE], pf_d[PE];
        float pf_tx = 0.f, pf_dx = 0.f;   // logits of child `tid` of pf_node, if any
        if constexpr (kPrefetch) {
            if constexpr (EL > 0) {
                sv_wait_loads();   // no fetch-ahead of the last sequence still lands there
                stage_rows(lb ^ 1, a.tl + rowbase * a.V, a.dl + rowbase * a.V, true);
            }
            load_row(a.tl + rowbase * a.V, pf_t);
            load_row(a.dl + rowbase * a.V, pf_d);
        }
        // ---- tree structure in LDS, validated ------------------------------
        // Each node's children as a bitmask (bit c of word c / 64), so first
        // child and next sibling are find-first-set operations; meanwhile the
        // upper half of the workgroup draws every node's uniforms (indexed by
        // node, not walk order).
        __syncthreads();
        // node `tid`'s parent and token, and its token's logits in the
        // parent's rows while the walk is at that parent (wave 0 reads them
        // from these registers for nodes below 64)
        int my_par = -2, my_tok = 0;
        float my_tx = 0.f, my_dx = 0.f;
        if (tid == 0) {
            s_bad = 0;
            s_path[0] = 0;
        }
        if (tid < N) {
            my_par = a.parent[rowbase + tid];
            my_tok = a.token[rowbase + tid];
            s_par[tid] = my_par;
            s_tok[tid] = my_tok;
#pragma unroll
            for (int w = 0; w < kKidWords; ++w)
                s_kids[tid][w] = 0ull;
            if (kPrefetch && tid >= 1 && my_par == 0 && my_tok >= 0 && my_tok < a.V) {
                pf_tx = a.tl[rowbase * a.V + my_tok];
                pf_dx = a.dl[rowbase * a.V + my_tok];
            }
        } else if (tid >= kSvThreads / 2 && tid - kSvThreads / 2 < N) {
            const int i = tid - kSvThreads / 2;
            const NodeUniforms r = node_uniforms(a.seed, a.offset, b, i);
            s_uacc[i] = r.acc;
            s_ures[i] = r.res;
        }
        __syncthreads();
        if (tid < N) {
            const bool bad_p = tid == 0 ? my_par != -1 : (my_par < 0 || my_par >= tid);
            if (bad_p)
                atomicOr(&s_bad, 1);
            if (tid > 0 && (my_tok < 0 || my_tok >= a.V))
                atomicOr(&s_bad, 2);
            if (tid >= 1 && !bad_p)
                atomicOr(&s_kids[my_par][tid >> 6], 1ull << (tid & 63));
        }
        __syncthreads();
        if (tid < N) {
            int first = -1, next = -1;
#pragma unroll
            for (int w = 0; w < kKidWords; ++w) {
                const uint64_t m = s_kids[tid][w];
                if (first < 0 && m != 0ull)
                    first = 64 * w + __builtin_ctzll(m);
            }
            if (tid >= 1 && my_par >= 0 && my_par < tid) {
#pragma unroll
                for (int w = 0; w < kKidWords; ++w) {
                    uint64_t m = w >= (tid >> 6) ? s_kids[my_par][w] : 0ull;
                    if (w == (tid >> 6))
                        m &= ~((2ull << (tid & 63)) - 1ull);   // siblings after tid
                    if (next < 0 && m != 0ull)
                        next = 64 * w + __builtin_ctzll(m);
                }
            }
            s_first[tid] = first;
            s_next[tid] = next;
        }
        __syncthreads();

        const bool lead = rank == 0 && tid == 0;
        int nacc = 0;
        bool failed = s_bad != 0;
        if (failed && lead)
            raise_flag(a.flags, (s_bad & 1 ? TAV_FLAG_BAD_PARENT : 0u) |
                                    (s_bad & 2 ? TAV_FLAG_BAD_TOKEN : 0u));

        int u = 0;
        while (!failed) {
            const float *trow = a.tl + (rowbase + u) * a.V;
            const float *drow = a.dl + (rowbase + u) * a.V;
            const bool has_kids = s_first[u] >= 0;

            // ---- 1. local (max, sum exp) of target and draft rows ------------
            float tf[ER], df[ER];
            if (pf_node == u) {
#pragma unroll
                for (int e = 0; e < ER; ++e) {
                    tf[e] = pf_t[e % PE];
                    df[e] = has_kids ? pf_d[e % PE] : -INFINITY;
                }
                if (my_par == u) {
                    s_tx[tid] = my_tx = pf_tx;
                    s_dx[tid] = my_dx = pf_dx;
                }
                lb ^= 1;   // its LDS entries were fetched into the other buffer
            } else {
                // (the current buffer's entries belong to a node left behind)
                stage_rows(lb, trow, drow, has_kids);
                load_row(trow, tf);
                if (has_kids)
                    load_row(drow, df);
                else
                    no_row(df);
                if (my_par == u) {
                    const int x = s_tok[tid];
                    s_tx[tid] = my_tx = trow[x];
                    s_dx[tid] = my_dx = drow[x];
                }
            }
            if constexpr (EL > 0)
                sv_wait_loads();
            // Maxima of the raw fp32 logits (exact; x -> x/T is monotone) and
            // sums of exp relative to them, per wave (DPP, no barrier). The
            // maxima propagate NaN, so a NaN logit makes the wave's maximum,
            // every exponential against it and the row's sum NaN.
            const int lane = tid & 63, wave = tid >> 6;
            float mt_l = -INFINITY, mq_l = -INFINITY;
#pragma unroll
            for (int e = 0; e < ER; e += 2) {
                mt_l = fmax_nan(mt_l, fmax_nan(tf[e], tf[e + 1]));
                mq_l = fmax_nan(mq_l, fmax_nan(df[e], df[e + 1]));
            }
            // an LDS entry's logit, -inf past the chunk (and for the draft
            // row of a node without children)
            auto lds_logit = [&](const f32x4 &x, int hl, int j, bool row_ok)
                __attribute__((always_inline)) {
                return row_ok && j < run_valid(ER / 4 + hl) ? x[j] : -INFINITY;
            };
#pragma unroll
            for (int hl = 0; hl < kLRuns; ++hl) {
                const f32x4 xt = s_lx[lb][hl][0][tid], xd = s_lx[lb][hl][1][tid];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mt_l = fmax_nan(mt_l, lds_logit(xt, hl, j, true));
                    mq_l = fmax_nan(mq_l, lds_logit(xd, hl, j, has_kids));
                }
            }
            const float wmt = wave_max_f32(mt_l), wmq = wave_max_f32(mq_l);
            const float wts32 = wmt * invT32, wqs32 = wmq * invT32;
            const double wts = wts32, wqs = wqs32;
            // e^(x/T - wts) per entry in fp32: y to one rounding, then
            // v_exp_f32 (under one ulp); summed in fp64. An entry's relative
            // error is about |y| 2^-24, so the entries that carry the sum
            // (|y| of a few units) are within a few 1e-7.
            float ep[ER], eq[ER];
            double zt = 0.0, zq = 0.0;
#pragma unroll
            for (int e = 0; e < ER; ++e) {
                ep[e] = (wmt == -INFINITY) ? 0.0f
                                           : __builtin_amdgcn_exp2f(fmaf(tf[e], invT32, -wts32) * kLog2eF);
                eq[e] = (wmq == -INFINITY) ? 0.0f
                                           : __builtin_amdgcn_exp2f(fmaf(df[e], invT32, -wqs32) * kLog2eF);
                zt += (double)ep[e];
                zq += (double)eq[e];
            }
            // the LDS entries' exponentials replace their logits in place
#pragma unroll
            for (int hl = 0; hl < kLRuns; ++hl) {
                const f32x4 xt = s_lx[lb][hl][0][tid], xd = s_lx[lb][hl][1][tid];
                f32x4 et, eqv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = lds_logit(xt, hl, j, true), d = lds_logit(xd, hl, j, has_kids);
                    et[j] = (wmt == -INFINITY) ? 0.0f
                                               : __builtin_amdgcn_exp2f(fmaf(t, invT32, -wts32) * kLog2eF);
                    eqv[j] = (wmq == -INFINITY) ? 0.0f
                                                : __builtin_amdgcn_exp2f(fmaf(d, invT32, -wqs32) * kLog2eF);
                    zt += (double)et[j];
                    zq += (double)eqv[j];
                }
                s_lx[lb][hl][0][tid] = et;
                s_lx[lb][hl][1][tid] = eqv;
            }
            // Entry e's exponentials. With E > 8 a register entry passes
            // through an empty asm statement at each use so that the compiler
            // forms the fp64 products there instead of hoisting all of them
            // out of the loops (which would hold them in 4E registers); with
            // E = 8 they fit, and are hoisted.
            auto fresh = [](float v) __attribute__((always_inline)) {
                if constexpr (E > 8)
                    asm volatile("" : "+v"(v));
                return v;
            };
            auto ep_of = [&](int e) __attribute__((always_inline)) -> float {
                if (e < ER)
                    return fresh(ep[e < ER ? e : 0]);
                return s_lx[lb][(e - ER) >> 2][0][tid][e & 3];
            };
            auto eq_of = [&](int e) __attribute__((always_inline)) -> float {
                if (e < ER)
                    return fresh(eq[e < ER ? e : 0]);
                return s_lx[lb][(e - ER) >> 2][1][tid][e & 3];
            };
            zt = wave_sum(zt);
            zq = wave_sum(zq);
            if (lane == 0) {
                s_wq[4 * wave + 0] = (double)wmt;
                s_wq[4 * wave + 1] = zt;
                s_wq[4 * wave + 2] = (double)wmq;
                s_wq[4 * wave + 3] = zq;
            }

            // the first child's rows and its children's logits, for the next level
            if (kPrefetch && has_kids) {
                const int c1 = s_first[u];
                pf_node = c1;
                const float *t1 = a.tl + (rowbase + c1) * a.V;
                const float *d1 = a.dl + (rowbase + c1) * a.V;
                const bool c1_kids = s_first[c1] >= 0;
                if constexpr (kPrefetch) {
                    stage_rows(lb ^ 1, t1, d1, c1_kids);
                    load_row(t1, pf_t);
                    if (c1_kids)
                        load_row(d1, pf_d);
                    else
                        no_row(pf_d);
                }
                if (tid < N && s_par[tid] == c1) {
                    const int x = s_tok[tid];
                    pf_tx = t1[x];
                    pf_dx = d1[x];
                }
            }
            __syncthreads();   // s_wq (and s_tx, s_dx) visible

            // Wave 0: the chunk's (max, sum) from its waves' in wave order,
            // exchanged with the group, and the members' pairs merged in
            // member order, so every workgroup of the group holds the same
            // bits. Then one barrier hands the results to the other waves.
            if (wave == 0) {
                const bool wl = lane < kSvWaves;
                const double m_w = wl ? s_wq[4 * lane + 0] : -INFINITY;
                const double z_w = wl ? s_wq[4 * lane + 1] : 0.0;
                const double mq_w = wl ? s_wq[4 * lane + 2] : -INFINITY;
                const double zq_w = wl ? s_wq[4 * lane + 3] : 0.0;
                const float mt_raw = wave_max_f32((float)m_w), mq_raw = wave_max_f32((float)mq_w);
                // a NaN sum travels through; an empty wave adds nothing
                const double zt_c =
                    wave_sum(m_w == -INFINITY ? (z_w != z_w ? z_w : 0.0)
                                              : z_w * exp_bulk((double)((float)m_w * invT32) - (double)(mt_raw * invT32)));
                const double zq_c =
                    wave_sum(mq_w == -INFINITY ? 0.0
                                               : zq_w * exp_bulk((double)((float)mq_w * invT32) - (double)(mq_raw * invT32)));
                const uint32_t mine6[6] = {f32_bits(mt_raw), f64_hi(zt_c), f64_lo(zt_c),
                                           f32_bits(mq_raw), f64_hi(zq_c), f64_lo(zq_c)};
                uint32_t mine = 0;
#pragma unroll
                for (int i = 0; i < 6; ++i)
                    if (lane == i)
                        mine = mine6[i];
                bool ok = true;
                uint32_t w6[6] = {0, 0, 0, 0, 0, 0};   // member `lane`'s payloads
                if (wpg == 1) {
#pragma unroll
                    for (int i = 0; i < 6; ++i)
                        w6[i] = mine6[i];
                } else {
                    ok = wave0_exchange<6>(box, wpg, rank, ++gen, mine, s_words, w6);
                }
                auto word6 = [&](int m, int i) __attribute__((always_inline)) {
                    return m == lane ? w6[i] : s_words[m][i];
                };
                // member maxima first, then the rebased sums, in member order
                float Mp32 = -INFINITY, Mq32 = -INFINITY;
                for (int m = lane; m < wpg; m += 64) {
                    Mp32 = fmaxf(Mp32, bits_f32(word6(m, 0)) * invT32);
                    Mq32 = fmaxf(Mq32, bits_f32(word6(m, 3)) * invT32);
                }
                const double Mp = wave_max_f32(Mp32), Mq = wave_max_f32(Mq32);
                // e^(x/T - M) of the children's tokens (one lane per child)
                // first: they need only the maxima, so their long fp64
                // chains overlap the sums' reductions
                // child c = lane + 64 k; for k = 0 its logits are this lane's
                double ex_p[kMaxNodes / 64], ex_q[kMaxNodes / 64];
#pragma unroll
                for (int k = 0; k < kMaxNodes / 64; ++k) {
                    const int c = lane + 64 * k;
                    ex_p[k] = ex_q[k] = 0.0;
                    if (k == 0 ? my_par == u : (c < N && s_par[c] == u)) {
                        const float tx = k == 0 ? my_tx : s_tx[c], dx = k == 0 ? my_dx : s_dx[c];
                        ex_p[k] = exp_bulk((double)tx * invT - Mp);
                        ex_q[k] = exp_bulk((double)dx * invT - Mq);
                    }
                }
                double Zp = 0.0, Zq = 0.0, zm0 = 0.0;
                for (int m = lane; m < wpg; m += 64) {
                    const double mk = (double)(bits_f32(word6(m, 0)) * invT32);
                    const double zk = bits_f64(word6(m, 1), word6(m, 2));
                    const double zm = (mk == -INFINITY) ? (zk != zk ? zk : 0.0) : zk * exp_bulk(mk - Mp);
                    if (m == lane)
                        zm0 = zm;
                    else
                        s_mass[m] = zm;   // divided by Zp below
                    Zp += zm;
                    const double mqk = (double)(bits_f32(word6(m, 3)) * invT32);
                    const double zqk = bits_f64(word6(m, 4), word6(m, 5));
                    Zq += (mqk == -INFINITY) ? 0.0 : zqk * exp_bulk(mqk - Mq);
                }
                Zp = wave_sum(Zp);
                Zq = wave_sum(Zq);
                const double inv_zp = 1.0 / Zp, inv_zq = 1.0 / Zq;
                if (lane < wpg)
                    s_mass[lane] = zm0 * inv_zp;
                for (int m = lane + 64; m < wpg; m += 64)
                    s_mass[m] *= inv_zp;
                if (lane == 0) {
                    s_norm[0] = Mp;
                    s_norm[1] = Zp;
                    s_norm[2] = Mq;
                    s_norm[3] = Zq;
                    s_sync_ok = ok;
                }
                // p and q of every child's token, one lane per child
#pragma unroll
                for (int k = 0; k < kMaxNodes / 64; ++k) {
                    const int c = lane + 64 * k;
                    if (k == 0 ? my_par == u : (c < N && s_par[c] == u)) {
                        s_px[c] = ex_p[k] * inv_zp;
                        s_qx[c] = ex_q[k] * inv_zq;
                    }
                }
            }
            __syncthreads();   // s_norm, s_mass visible
            if (!s_sync_ok) {
                if (tid == 0)
                    raise_flag(a.flags, TAV_FLAG_SYNC_TIMEOUT);
                alive = false;
                break;
            }
            const double Mp = s_norm[0], Zp = s_norm[1], Mq = s_norm[2], Zq = s_norm[3];
            const bool bad_p = !(Zp > 0.0) || Mp == -INFINITY || __builtin_isinf(Mp) ||
                               __builtin_isnan(Zp) || __builtin_isinf(Zp);
            const bool bad_q = has_kids && (!(Zq > 0.0) || Mq == -INFINITY ||
                                            __builtin_isinf(Mq) || __builtin_isinf(Zq));
            if (bad_p || bad_q) {
                if (lead)
                    raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
                failed = true;
                break;
            }
            if constexpr (kProbe) {
                // the same arithmetic as the rebase before a rejection below
                const double sp = (wmt == -INFINITY) ? 0.0 : exp_bulk(wts - Mp) * (1.0 / Zp);
                const double sq = (wmq == -INFINITY) ? 0.0 : exp_bulk(wqs - Mq) * (1.0 / Zq);
                double *prow = a.p_rows + (rowbase + u) * a.V;
                double *qrow = a.q_rows + (rowbase + u) * a.V;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int64_t t = tok(e);
                    if (t < lim) {
                        prow[t] = (double)ep_of(e) * sp;
                        if (has_kids)
                            qrow[t] = (double)eq_of(e) * sq;
                    }
                }
                if (rank == 0 && tid < N && s_par[tid] == u) {
                    a.child_pq[2 * (rowbase + tid)] = s_px[tid];
                    a.child_pq[2 * (rowbase + tid) + 1] = s_qx[tid];
                }
            }
            // ---- 2./3. children in ascending order against the running residual
            // Child c, tried after k rejections at u: its token's p under the
            // residual after those k rejections, against r * q.
            auto accepts = [&](int c, int k) __attribute__((always_inline)) {
                const double qx = s_qx[c];
                double prx = s_px[c];
                if constexpr (kWor) {
                    // q_j(x) after j removals; zero once x itself was removed
                    const int x = s_tok[c];
                    bool gone = false;
                    for (int j = 0; j < k; ++j) {
                        const double qj = gone ? 0.0 : (j == 0 ? qx : qx * s_qs[j]);
                        const double zj = s_zhist[j];
                        if (zj > 0.0) {
                            const double d = prx - qj;
                            prx = (d > 0.0 ? d : 0.0) / zj;
                        }
                        gone |= s_rtok[j] == x;
                    }
                    const double qk = gone ? 0.0 : (k == 0 ? qx : qx * s_qs[k]);
                    return s_uacc[c] * qk < prx;
                } else {
                    for (int j = 0; j < k; ++j) {
                        const double zj = s_zhist[j];
                        if (zj > 0.0) {
                            const double d = prx - qx;
                            prx = (d > 0.0 ? d : 0.0) / zj;
                        }
                    }
                    return s_uacc[c] * qx < prx;
                }
            };
            auto accept = [&](int c) __attribute__((always_inline)) {
                if (lead) {
                    a.out_tok[rowbase + nacc] = s_tok[c];
                    a.path[rowbase + nacc + 1] = c;
                }
                if (tid == 0)
                    s_path[nacc + 1] = c;
                ++nacc;
                u = c;
            };
            int c = s_first[u];
            if (c >= 0 && accepts(c, 0)) {
                accept(c);
                continue;   // the first child needs only the normalisers
            }
            // A rejection or the final draw follows. This chunk's p and q are
            // its exponentials rebased from the wave's max and normalised:
            // p(e) = ep[e] sp, q(e) = eq[e] sq. After k rejections at u the
            // target is the residual chain res_k(e): res_0 = p(e) and, for
            // j < k, res_{j+1} = max(0, res_j - q_j(e)) / Z_j when Z_j > 0
            // (else unchanged), Z_j the residual mass of round j; q_j = q
            // (independent siblings) or, without replacement, q(e) s_j off
            // the tokens removed before round j (s_0 = 1).
            const double sp = (wmt == -INFINITY) ? 0.0 : exp_bulk(wts - Mp) * (1.0 / Zp);
            const double sq = (wmq == -INFINITY) ? 0.0 : exp_bulk(wqs - Mq) * (1.0 / Zq);
            // round at which entry e's token left the draft (without
            // replacement), kMaxNodes if it has not
            auto removed_at = [&](int e, int k_now) __attribute__((always_inline)) {
                int at = kMaxNodes;
                if constexpr (kWor) {
                    const int64_t t = tok(e);
                    for (int j = 0; j < k_now; ++j)
                        if (s_rtok[j] == t && at == kMaxNodes)
                            at = j;
                }
                return at;
            };
            auto q_at = [&](int e, int j, int gone) __attribute__((always_inline)) {
                const double q = (double)eq_of(e) * sq;
                if constexpr (kWor)
                    return j > gone ? 0.0 : q * (j == 0 ? 1.0 : s_qs[j]);
                else
                    return q;
            };
            auto residual = [&](int e, int k_now) __attribute__((always_inline)) {
                double r = (double)ep_of(e) * sp;
                const int gone = removed_at(e, k_now);
                for (int j = 0; j < k_now; ++j) {
                    const double zj = s_zhist[j];
                    if (zj > 0.0) {
                        const double d = r - q_at(e, j, gone);
                        r = (d > 0.0 ? d : 0.0) * (1.0 / zj);
                    }
                }
                return r;
            };
            // With E <= 8, p and q (then the residual) are held in fp64 registers
            // and updated in place after each rejection, the same operations
            // on the same values as the chain above, without re-forming it.
            constexpr bool kHold = E <= 8;
            double pr_h[kHold ? E : 1], qv_h[kHold ? E : 1];
            double sk = 1.0;   // held, without replacement: q_k = qv_h sk
            if constexpr (kHold) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    pr_h[e] = (double)ep[e] * sp;
                    qv_h[e] = (double)eq[e] * sq;
                }
            }
            auto cur_res = [&](int e, int k_now) __attribute__((always_inline)) {
                if constexpr (kHold)
                    return pr_h[e];
                else
                    return residual(e, k_now);
            };
            int k = 0;
            bool accepted = false;
            while (c >= 0) {
                // rejected: the chunk's residual mass, per wave, then in wave
                // 0 exchanged with the group and summed in member order
                double rsum = 0.0, qrem = 0.0;
                // without replacement, this thread's entry of the rejected
                // token, if it holds it: its q leaves the remaining mass now
                // and its register after the residual pass
                int ex = -1;
                if constexpr (kWor) {
                    const int64_t off = (int64_t)s_tok[c] - base;
                    if (off >= 0 && off < lim - base && (int)((off % kRun) >> 2) == tid)
                        ex = (int)((off / kRun) * 4 + (off & 3));
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if constexpr (kHold) {
                        const double d = pr_h[e] - (kWor ? qv_h[e] * sk : qv_h[e]);
                        rsum += d > 0.0 ? d : 0.0;
                        if constexpr (kWor)
                            qrem += e == ex ? 0.0 : qv_h[e];
                    } else {
                        const int gone = removed_at(e, k);
                        const double d = residual(e, k) - q_at(e, k, gone);
                        rsum += d > 0.0 ? d : 0.0;
                        if constexpr (kWor)
                            qrem += (e == ex || gone < k) ? 0.0 : (double)eq_of(e) * sq;
                    }
                }
                rsum = wave_sum(rsum);
                if constexpr (kWor)
                    qrem = wave_sum(qrem);
                // (wave 0 read s_wq before the last barrier)
                if (lane == 0) {
                    s_wq[wave] = rsum;
                    if constexpr (kWor)
                        s_wq[kSvWaves + wave] = qrem;
                }
                __syncthreads();
                if (wave == 0) {
                    constexpr int kNW = kWor ? 4 : 2;
                    const double sc = wave_sum(lane < kSvWaves ? s_wq[lane] : 0.0);
                    double sqr = 0.0;
                    if constexpr (kWor)
                        sqr = wave_sum(lane < kSvWaves ? s_wq[kSvWaves + lane] : 0.0);
                    const uint32_t mine = lane == 0   ? f64_hi(sc)
                                          : lane == 1 ? f64_lo(sc)
                                          : lane == 2 ? f64_hi(sqr)
                                          : lane == 3 ? f64_lo(sqr)
                                                      : 0u;
                    bool ok = true;
                    uint32_t wv[kNW];   // member `lane`'s payloads
                    wv[0] = f64_hi(sc);
                    wv[1] = f64_lo(sc);
                    if constexpr (kWor) {
                        wv[2] = f64_hi(sqr);
                        wv[3] = f64_lo(sqr);
                    }
                    if (wpg > 1)
                        ok = wave0_exchange<kNW>(box, wpg, rank, ++gen, mine, s_words, wv);
                    auto wordn = [&](int m, int i) __attribute__((always_inline)) {
                        return m == lane ? wv[i] : s_words[m][i];
                    };
                    double Zr = 0.0, Qr = 0.0;
                    for (int m = lane; m < wpg; m += 64) {
                        Zr += bits_f64(wordn(m, 0), wordn(m, 1));
                        if constexpr (kWor)
                            Qr += bits_f64(wordn(m, 2), wordn(m, 3));
                    }
                    Zr = wave_sum(Zr);
                    if constexpr (kWor)
                        Qr = wave_sum(Qr);
                    if (Zr > 0.0) {
                        for (int m = lane; m < wpg; m += 64)
                            s_mass[m] = bits_f64(wordn(m, 0), wordn(m, 1)) / Zr;
                    }
                    if (lane == 0) {
                        s_zhist[k] = Zr;
                        if constexpr (kWor) {
                            // no draft mass left: every later q is zero
                            s_qs[k + 1] = Qr > 0.0 ? 1.0 / Qr : 0.0;
                            s_rtok[k] = s_tok[c];
                        }
                        s_sync_ok = ok;
                    }
                }
                __syncthreads();   // s_zhist, s_mass (and s_qs, s_rtok) visible
                if (!s_sync_ok) {
                    if (tid == 0)
                        raise_flag(a.flags, TAV_FLAG_SYNC_TIMEOUT);
                    alive = false;
                    break;
                }
                if constexpr (kHold) {
                    const double Z = s_zhist[k];
                    if (Z > 0.0) {
                        const double inv = 1.0 / Z;
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const double d = pr_h[e] - (kWor ? qv_h[e] * sk : qv_h[e]);
                            pr_h[e] = (d > 0.0 ? d : 0.0) * inv;
                        }
                    }
                    if constexpr (kWor) {
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            if (e == ex)
                                qv_h[e] = 0.0;
                        sk = s_qs[k + 1];
                    }
                }
                ++k;
                c = s_next[c];
                if (c >= 0 && accepts(c, k)) {
                    accept(c);
                    accepted = true;
                    break;
                }
            }
            if (!alive)
                break;
            if (accepted)
                continue;

            // ---- 4. inverse-CDF draw from the final distribution at u ---------
            // Member w's interval starts at lo_w, the exclusive prefix sum of
            // the members' masses in member order (a wave scan per 64
            // members, carried across; the same bits in every workgroup),
            // and the draw belongs to the last member with mass whose
            // interval starts at or before it. A member without mass owns
            // nothing, not even the ulp-wide interval the scan's differently
            // associated sums can leave it.
            if (wave == 0) {
                int owner = -1;
                double total = 0.0, target = 0.0;
                if (wpg <= 64) {
                    const double m = lane < wpg ? s_mass[lane] : 0.0;
                    const double inc = wave_scan_incl(m);
                    total = lane_f64(inc, 63);
                    target = s_ures[u] * total;
                    const double lo = wave_shift_up1(inc);
                    const uint64_t at = __ballot(m > 0.0 && lo <= target);
                    if (at) {
                        owner = 63 - (int)__builtin_clzll(at);
                        if (lane == owner)
                            s_red[0] = lo;
                    }
                } else {
                    for (int w0 = 0; w0 < wpg; w0 += 64)
                        total = total + lane_f64(wave_scan_incl(w0 + lane < wpg ? s_mass[w0 + lane] : 0.0), 63);
                    target = s_ures[u] * total;
                    double carry = 0.0;
                    for (int w0 = 0; w0 < wpg; w0 += 64) {
                        const double m = w0 + lane < wpg ? s_mass[w0 + lane] : 0.0;
                        const double inc = wave_scan_incl(m);
                        const double lo = carry + wave_shift_up1(inc);
                        const uint64_t at = __ballot(m > 0.0 && lo <= target);
                        if (at) {
                            owner = w0 + 63 - (int)__builtin_clzll(at);
                            if (w0 + lane == owner)
                                s_red[0] = lo;
                        }
                        carry = carry + lane_f64(inc, 63);
                    }
                }
                if (lane == 0) {
                    s_red[1] = total;
                    s_red[2] = target;
                    s_owner = owner;
                    s_found = -1;
                    s_last_live = -1;
                    s_hit = -1;
                }
            }
            __syncthreads();
            const double before = s_red[0], total = s_red[1], target = s_red[2];
            const int owner = s_owner;
            __syncthreads();
            if (!(total > 0.0)) {
                if (lead)
                    raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
                failed = true;
                break;
            }
            if (rank == owner) {
                // Token order is (run h, wave, lane, entry j). Totals of every
                // (run, wave) slot first (a wave scan's last value); then the
                // slots scanned in that order, the wave holding the target
                // scans its lanes' run sums the same way, and the lane its
                // four entries.
                const int lane = tid & 63, wave = tid >> 6;
                auto run_sum = [&](int h) __attribute__((always_inline)) {
                    return ((cur_res(4 * h, k) + cur_res(4 * h + 1, k)) + cur_res(4 * h + 2, k)) +
                           cur_res(4 * h + 3, k);
                };
#pragma unroll
                for (int h = 0; h < E / 4; ++h) {
                    const double t = lane_f64(wave_scan_incl(run_sum(h)), 63);
                    if (lane == 0)
                        s_slot[h * kSvWaves + wave] = t;
                }
                __syncthreads();
                if (wave == 0) {
                    constexpr int kSlots = (E / 4) * kSvWaves;
                    static_assert(kSlots <= 64, "one lane per slot");
                    const double sl = lane < kSlots ? s_slot[lane] : 0.0;
                    const double inc = wave_scan_incl(sl);
                    const double lo = before + wave_shift_up1(inc), hi = before + inc;
                    const uint64_t hits = __ballot(sl > 0.0 && lo <= target && target < hi);
                    const int first = hits ? (int)__builtin_ctzll(hits) : -1;
                    if (lane == 0)
                        s_hit = first;
                    if (lane == first)
                        s_hit_off = lo;
                }
                __syncthreads();
                const int hit = s_hit;
                if (hit >= 0 && wave == hit % kSvWaves) {
                    const int h_hit = hit / kSvWaves;
                    double v = 0.0, pe[4];
#pragma unroll
                    for (int h = 0; h < E / 4; ++h)
                        if (h == h_hit) {
                            v = run_sum(h);
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                pe[j] = cur_res(4 * h + j, k);
                        }
                    const double incl = wave_scan_incl(v);
                    const double lo = s_hit_off + wave_shift_up1(incl), hi = s_hit_off + incl;
                    const int64_t i0 = base + (int64_t)h_hit * kRun + 4 * tid;
                    if (v > 0.0) {
                        int last = -1, found = -1;
                        double r = lo;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const double nx = r + pe[j];
                            if (pe[j] > 0.0) {
                                last = j;
                                if (found < 0 && r <= target && target < nx)
                                    found = j;
                            }
                            r = nx;
                        }
                        atomicMax(&s_last_live, (int)(i0 + last));
                        // at most one lane's run holds the target; rounding
                        // between its sum and its entries' running sum gives
                        // the run's last live entry
                        if (lo <= target && target < hi)
                            s_found = (int)(i0 + (found >= 0 ? found : last));
                    }
                }
                // rounding left the target past the chunk's summed slots: the
                // chunk's last live token takes it
                if (hit < 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (cur_res(e, k) > 0.0)
                            atomicMax(&s_last_live, (int)tok(e));
                }
                __syncthreads();
                if (tid == 0)
                    a.out_tok[rowbase + nacc] = s_found >= 0 ? s_found : s_last_live;
            }
            break;
        }

        // ---- outputs owned by the group leader ------------------------------
        if (failed || !alive) {
            if (lead) {
                for (int i = 0; i < N; ++i) {
                    a.path[rowbase + i] = i == 0 ? 0 : -1;
                    a.out_tok[rowbase + i] = -1;
                }
                a.n_acc[b] = 0;
            }
        } else if (rank == 0) {
            // the padding past the emitted entries, which the walk never wrote
            for (int i = nacc + 1 + tid; i < N; i += kSvThreads) {
                a.path[rowbase + i] = -1;
                a.out_tok[rowbase + i] = -1;
            }
            if (lead) {
                a.path[rowbase] = 0;
                a.n_acc[b] = nacc;
            }
        }
        if (a.cm.k_tree) {
            __syncthreads();   // s_path complete
            commit_path_rows(a.cm, b, N, (failed || !alive) ? 0 : nacc, s_path, rank, wpg, tid,
                             a.flags);
        }
    }

    // ---- exit: the last workgroup out clears every mailbox word -------------
    // Each workgroup counts itself out only after its last poll, so the last
    // one knows no slot is still being read. (No fetch-ahead into LDS may
    // outlive the workgroup.)
    if constexpr (EL > 0)
        sv_wait_loads();
    __syncthreads();
    if (tid == 0) {
        const uint32_t out =
            __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_is_last = out == gridDim.x - 1;
    }
    __syncthreads();
    if (s_is_last) {
        const int64_t words = (int64_t)a.ngroups * 2 * wpg * kSlotWords;
        for (int64_t i = tid; i < words; i += kSvThreads)
            __hip_atomic_store(a.box + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0)
            __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Greedy verification (temperature 0). The target's choice at a node is the
// argmax of its target row, the lowest token id among equal maxima; the first
// child (ascending node index) carrying it is accepted, otherwise the choice
// is emitted and the walk stops (LLM Primer ch. 9, §9.1: the longest prefix
// matching the target's own choice, then the target's choice). No draft row
// and no uniform is read.
//
// Same group layout as spec_verify_kernel: workgroup r of a group owns
// vocabulary entries [r*chunk, (r+1)*chunk) of the node's target row. Each
// thread reduces its entries to a 64-bit key, the value's order-preserving
// bits above the complement of the token id, so the largest key is the
// largest value at its lowest token; waves reduce keys with DPP, wave 0
// merges the waves' keys and exchanges its workgroup's key (and a NaN flag)
// through the mailbox, and every workgroup takes the largest key of the
// group, so all hold the same choice. The first child's row is fetched
// while the current node is decided.

// Order-preserving map of a float that is not NaN to 32 bits (-0 as +0).
__device__ __forceinline__ uint32_t ordered_bits(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o)
{
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF,
                                                              false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The largest key of the wave, in every lane (0 is the identity).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    v = max_u64(v, dpp_u64<kQuadSwap1>(v));
    v = max_u64(v, dpp_u64<kQuadSwap2>(v));
    v = max_u64(v, dpp_u64<kRowHalfMirror>(v));
    v = max_u64(v, dpp_u64<kRowMirror>(v));
    return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)), max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

__global__ __launch_bounds__(kSvThreads) void spec_verify_greedy_kernel(SvArgs a)
{
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_path[kMaxNodes];   // accepted path, for the fused commit
    __shared__ int32_t s_first[kMaxNodes];
    __shared__ int32_t s_next[kMaxNodes];
    __shared__ int32_t s_tok[kMaxNodes];
    constexpr int kKidWords = kMaxNodes / 64;
    __shared__ unsigned long long s_kids[kMaxNodes][kKidWords];   // children of each node, as bits
    __shared__ uint64_t s_key[kSvWaves];
    __shared__ uint32_t s_words[kMaxWpg][kSlotWords];   // the group's payloads, as wave 0 received them
    __shared__ int s_wnan[kSvWaves];   // a wave saw a NaN logit
    __shared__ uint64_t s_choice;      // the group's largest key
    __shared__ int s_gnan;             // a NaN anywhere in the row
    __shared__ int s_sync_ok;
    __shared__ int s_bad;
    __shared__ int s_is_last;

    const int g = blockIdx.x % a.ngroups;
    const int rank = blockIdx.x / a.ngroups;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int N = a.N;
    const int wpg = a.wpg;
    const int64_t base = (int64_t)rank * a.chunk;
    const int64_t lim = std::min<int64_t>((int64_t)a.V, base + a.chunk);
    // entries of the chunk as in spec_verify_kernel: run h holds tokens
    // base + h * 4 * 512 + 4 tid + j, j < 4
    constexpr int kRun = 4 * kSvThreads;
    auto load_row = [&](const float *row, float (&v)[kSvEpt]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < kSvEpt / 4; ++h) {
            const int64_t i0 = base + (int64_t)h * kRun + 4 * tid;
            if (a.vec4 && i0 + 3 < lim) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(row + i0);
                v[4 * h] = x.x;
                v[4 * h + 1] = x.y;
                v[4 * h + 2] = x.z;
                v[4 * h + 3] = x.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[4 * h + j] = i0 + j < lim ? row[i0 + j] : -INFINITY;
            }
        }
    };
    uint64_t *box = a.box + (size_t)g * 2 * wpg * kSlotWords;
    uint32_t gen = 0;
    bool alive = true;

    for (int b = g; b < a.B && alive; b += a.ngroups) {
        const int64_t rowbase = (int64_t)b * N;
        // the root's row first: the walk starts there
        int pf_node = 0;
        float pf[kSvEpt];
        load_row(a.tl + rowbase * a.V, pf);
        // ---- tree structure in LDS, validated (children as bitmasks) --------
        __syncthreads();
        int my_par = -2, my_tok = 0;
        if (tid == 0) {
            s_bad = 0;
            s_path[0] = 0;
        }
        if (tid < N) {
            my_par = a.parent[rowbase + tid];
            my_tok = a.token[rowbase + tid];
            s_par[tid] = my_par;
            s_tok[tid] = my_tok;
#pragma unroll
            for (int w = 0; w < kKidWords; ++w)
                s_kids[tid][w] = 0ull;
        }
        __syncthreads();
        if (tid < N) {
            const bool bad_p = tid == 0 ? my_par != -1 : (my_par < 0 || my_par >= tid);
            if (bad_p)
                atomicOr(&s_bad, 1);
            if (tid > 0 && (my_tok < 0 || my_tok >= a.V))
                atomicOr(&s_bad, 2);
            if (tid >= 1 && !bad_p)
                atomicOr(&s_kids[my_par][tid >> 6], 1ull << (tid & 63));
        }
        __syncthreads();
        if (tid < N) {
            int first = -1, next = -1;
#pragma unroll
            for (int w = 0; w < kKidWords; ++w) {
                const uint64_t m = s_kids[tid][w];
                if (first < 0 && m != 0ull)
                    first = 64 * w + __builtin_ctzll(m);
            }
            if (tid >= 1 && my_par >= 0 && my_par < tid) {
#pragma unroll
                for (int w = 0; w < kKidWords; ++w) {
                    uint64_t m = w >= (tid >> 6) ? s_kids[my_par][w] : 0ull;
                    if (w == (tid >> 6))
                        m &= ~((2ull << (tid & 63)) - 1ull);   // siblings after tid
                    if (next < 0 && m != 0ull)
                        next = 64 * w + __builtin_ctzll(m);
                }
            }
            s_first[tid] = first;
            s_next[tid] = next;
        }
        __syncthreads();

        const bool lead = rank == 0 && tid == 0;
        int nacc = 0;
        bool failed = s_bad != 0;
        if (failed && lead)
            raise_flag(a.flags, (s_bad & 1 ? TAV_FLAG_BAD_PARENT : 0u) |
                                    (s_bad & 2 ? TAV_FLAG_BAD_TOKEN : 0u));

        int u = 0;
        while (!failed) {
            float tf[kSvEpt];
            if (pf_node == u) {
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e)
                    tf[e] = pf[e];
            } else {
                load_row(a.tl + (rowbase + u) * a.V, tf);
            }
            // this thread's key: its largest entry at its lowest token
            bool nan_seen = false;
            uint64_t key = 0;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e) {
                nan_seen |= __builtin_isnan(tf[e]);
                const int64_t t = base + (int64_t)(e >> 2) * kRun + 4 * tid + (e & 3);
                const uint64_t k = __builtin_isnan(tf[e]) || t >= lim
                                       ? 0ull
                                       : ((uint64_t)ordered_bits(tf[e]) << 32) | (0xFFFFFFFFu - (uint32_t)t);
                key = max_u64(key, k);
            }
            key = wave_max_key(key);
            const bool wave_nan = __any(nan_seen);
            if (lane == 0) {
                s_key[wave] = key;
                s_wnan[wave] = wave_nan;
            }
            // the first child's row, for the next level
            const int c1 = s_first[u];
            if (c1 >= 0) {
                pf_node = c1;
                load_row(a.tl + (rowbase + c1) * a.V, pf);
            }
            __syncthreads();   // s_key, s_wnan visible
            if (wave == 0) {
                const uint64_t wk = wave_max_key(lane < kSvWaves ? s_key[lane] : 0ull);
                const bool wn = __any(lane < kSvWaves && s_wnan[lane] != 0);
                const uint32_t mine3[3] = {(uint32_t)(wk >> 32), (uint32_t)wk, (uint32_t)wn};
                uint32_t mine = 0;
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    if (lane == i)
                        mine = mine3[i];
                bool ok = true;
                uint32_t w3[3] = {0, 0, 0};   // member `lane`'s payloads
                if (wpg == 1) {
#pragma unroll
                    for (int i = 0; i < 3; ++i)
                        w3[i] = mine3[i];
                } else {
                    ok = wave0_exchange<3>(box, wpg, rank, ++gen, mine, s_words, w3);
                }
                uint64_t gk = 0;
                bool gnan = false;
                for (int m = lane; m < wpg; m += 64) {
                    const uint32_t hi = m == lane ? w3[0] : s_words[m][0];
                    const uint32_t lo = m == lane ? w3[1] : s_words[m][1];
                    const uint32_t nn = m == lane ? w3[2] : s_words[m][2];
                    gk = max_u64(gk, ((uint64_t)hi << 32) | lo);
                    gnan |= nn != 0;
                }
                gk = wave_max_key(gk);
                gnan = __any(gnan);
                if (lane == 0) {
                    s_choice = gk;
                    s_gnan = gnan;
                    s_sync_ok = ok;
                }
            }
            __syncthreads();   // s_choice, s_gnan, s_sync_ok visible
            if (!s_sync_ok) {
                if (tid == 0)
                    raise_flag(a.flags, TAV_FLAG_SYNC_TIMEOUT);
                alive = false;
                break;
            }
            const uint64_t ck = s_choice;
            const float cv = from_ordered_bits((uint32_t)(ck >> 32));
            if (s_gnan || ck == 0ull || !__builtin_isfinite(cv)) {
                if (lead)
                    raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
                failed = true;
                break;
            }
            const int x = (int)(0xFFFFFFFFu - (uint32_t)ck);
            int c = s_first[u];
            while (c >= 0 && s_tok[c] != x)
                c = s_next[c];
            if (lead)
                a.out_tok[rowbase + nacc] = x;
            if (c < 0)
                break;   // the target's choice is emitted; the walk stops
            if (lead)
                a.path[rowbase + nacc + 1] = c;
            if (tid == 0)
                s_path[nacc + 1] = c;
            ++nacc;
            u = c;
        }

        // ---- outputs owned by the group's first workgroup ----------------------
        if (failed || !alive) {
            if (lead) {
                for (int i = 0; i < N; ++i) {
                    a.path[rowbase + i] = i == 0 ? 0 : -1;
                    a.out_tok[rowbase + i] = -1;
                }
                a.n_acc[b] = 0;
            }
        } else if (rank == 0) {
            for (int i = nacc + 1 + tid; i < N; i += kSvThreads) {
                a.path[rowbase + i] = -1;
                a.out_tok[rowbase + i] = -1;
            }
            if (lead) {
                a.path[rowbase] = 0;
                a.n_acc[b] = nacc;
            }
        }
        if (a.cm.k_tree) {
            __syncthreads();   // s_path complete
            commit_path_rows(a.cm, b, N, (failed || !alive) ? 0 : nacc, s_path, rank, wpg, tid,
                             a.flags);
        }
    }

    // ---- exit: the last workgroup out clears every mailbox word -------------
    __syncthreads();
    if (tid == 0) {
        const uint32_t out =
            __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_is_last = out == gridDim.x - 1;
    }
    __syncthreads();
    if (s_is_last) {
        const int64_t words = (int64_t)a.ngroups * 2 * wpg * kSlotWords;
        for (int64_t i = tid; i < words; i += kSvThreads)
            __hip_atomic_store(a.box + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0)
            __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

struct SvPlan {
    int E;                // vocabulary entries per thread
    int wpg, ngroups, chunk;
    size_t box_bytes;
};

// Workgroups of the sampling kernels with E entries per thread the device
// holds at once (every variant that may run with that E: the group syncs
// wait on each other, so a grid must be resident); 0 on failure.
template <int E>
int64_t sampling_resident(int cus)
{
    const int a = kernel_occupancy(reinterpret_cast<const void *>(spec_verify_kernel<E, false>),
                                   kSvThreads);
    const int b = kernel_occupancy(reinterpret_cast<const void *>(spec_verify_kernel<E, true>),
                                   kSvThreads);
    const int c = kernel_occupancy(
        reinterpret_cast<const void *>(spec_verify_kernel<E, false, true>), kSvThreads);
    return (int64_t)std::min(std::min(a, b), c) * cus;
}

// A group of ceil(V / 512 E) workgroups per sequence, as many groups as the
// device holds at once (at most B), each walking its sequences in turn. The
// sampling walk takes the E of 4, 8, 16 and 28 (16 in registers and 12 in
// LDS) with the least cost, sequences per group times a weight per E, the
// smallest E among equals (more members share each row: at batches up to 4
// over a 128256-token vocabulary, 63 workgroups of 4 entries per thread,
// 2-5 % faster than 32 of 8 at batch one); greedy verification keeps E = 8.
// A sequence costs about the same with 4, 8 or 16
// entries per thread (the group syncs set a level's time) and about 1.5
// times that with 28 (measured at batches 64 and 128 over a 128256-token
// vocabulary: 42-45 against 63-65 us per sequence), so 28 pays only where
// it cuts the sequences per group by more than a third. (More than 16 in
// registers would need more than a resident 512-thread workgroup has; the
// two LDS buffers of 12 entries take 96 KB.)
// The same from the workgroups a device holds at once for each layout
// (resident[i] for E = 4, 8, 16, 28, then greedy verification): pure
// arithmetic, so it can be checked on the host.
bool sv_plan_for(int32_t B, int32_t V, bool greedy, const int64_t (&resident)[5], SvPlan &p)
{
    auto fit = [&](int E, int64_t res, SvPlan &q) {
        q.E = E;
        q.wpg = (int)ceil_div(V, (int64_t)kSvThreads * E);
        if (res <= 0 || q.wpg > res || q.wpg > kMaxWpg)
            return false;
        q.chunk = (int)(ceil_div(ceil_div(V, q.wpg), 4) * 4);   // whole 16-byte runs
        q.ngroups = (int)std::min<int64_t>(B, res / q.wpg);
        q.box_bytes = (size_t)q.ngroups * 2 * q.wpg * kSlotWords * sizeof(uint64_t);
        return true;
    };
    if (greedy)
        return fit(kSvEpt, resident[4], p);
    const int Es[4] = {4, 8, 16, 28};
    const int64_t weight[4] = {2, 2, 2, 3};
    bool found = false;
    int64_t best = 0;
    for (int i = 0; i < 4; ++i) {
        SvPlan q;
        if (!fit(Es[i], resident[i], q))
            continue;
        const int64_t cost = ceil_div(B, q.ngroups) * weight[i];
        if (!found || cost < best) {
            p = q;
            best = cost;
            found = true;
        }
    }
    return found;
}

bool sv_plan(int32_t B, int32_t V, bool greedy, SvPlan &p)
{
    const int cus = device_cu_count();
    if (cus <= 0)
        return false;
    int64_t res[5] = {0, 0, 0, 0, 0};
    if (greedy) {
        res[4] = (int64_t)kernel_occupancy(reinterpret_cast<const void *>(spec_verify_greedy_kernel),
                                           kSvThreads) * cus;
    } else {
        res[0] = sampling_resident<4>(cus);
        res[1] = sampling_resident<8>(cus);
        res[2] = sampling_resident<16>(cus);
        res[3] = sampling_resident<28>(cus);
    }
    return sv_plan_for(B, V, greedy, res, p);
}

// Workspace for either mode of spec_verify_sample (0 if neither plan fits).
size_t sv_workspace(int32_t B, int32_t V)
{
    SvPlan s, g;
    if (!sv_plan(B, V, false, s) || !sv_plan(B, V, true, g))
        return 0;
    return kHeaderBytes + std::max(s.box_bytes, g.box_bytes);
}

// ---------------------------------------------------------------------------
// Diagnostics: the uniforms and the device softmax, exposed for checking.

__global__ void philox_uniforms_kernel(uint64_t seed, uint64_t offset, int32_t B, int32_t N,
                                       float *u)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * N)
        return;
    const NodeUniforms r = node_uniforms(seed, offset, i / N, i % N);
    u[2 * i] = (float)r.acc;
    u[2 * i + 1] = (float)r.res;
}

// One row per workgroup, with the sampler's scaling, maximum and exp.
__global__ __launch_bounds__(kSvThreads) void target_probs_kernel(const float *logits,
                                                                  int32_t V, double T,
                                                                  double *p, uint32_t *flags)
{
    __shared__ double red[2 * kSvWaves];
    const float *row = logits + (int64_t)blockIdx.x * V;
    double *out = p + (int64_t)blockIdx.x * V;
    const double invT = 1.0 / T;
    double m = -INFINITY, unused = -INFINITY;
    bool nan_seen = false;
    for (int x = threadIdx.x; x < V; x += kSvThreads) {
        nan_seen |= __builtin_isnan(row[x]);
        m = fmax(m, (double)row[x]);
    }
    block_max2(m, unused, red);
    const double ms = (double)(float)m * invT;
    double z = 0.0, unused2 = 0.0;
    for (int x = threadIdx.x; x < V; x += kSvThreads)
        z += exp_f64((double)row[x] * invT - ms);
    block_sum2(z, unused2, red);
    if (__syncthreads_or(nan_seen) || m == -INFINITY || __builtin_isinf(m)) {
        if (threadIdx.x == 0)
            raise_flag(flags, TAV_FLAG_NONFINITE_LOGITS);
        return;
    }
    for (int x = threadIdx.x; x < V; x += kSvThreads)
        out[x] = exp_f64((double)row[x] * invT - ms) / z;
}

} // namespace
} // namespace tav

extern "C" tav_status tav_sampler_plan(int32_t B, int32_t V, int32_t greedy, int32_t *plan)
{
    using namespace tav;
    if (!plan || B < 1 || V < 1 || greedy < 0 || greedy > 1)
        return TAV_ERR_ARG;
    if (V > kMaxVocab)
        return TAV_ERR_UNSUPPORTED;
    SvPlan p;
    if (!sv_plan(B, V, greedy == 1, p))
        return TAV_ERR_LAUNCH;
    plan[0] = p.E;
    plan[1] = p.wpg;
    plan[2] = p.ngroups;
    plan[3] = p.chunk;
    return TAV_OK;
}

extern "C" tav_status tav_sampler_plan_for(int32_t B, int32_t V, int32_t greedy, int32_t cus,
                                           const int32_t *per_cu, int32_t *plan)
{
    using namespace tav;
    if (!plan || !per_cu || B < 1 || V < 1 || greedy < 0 || greedy > 1 || cus < 1)
        return TAV_ERR_ARG;
    for (int i = 0; i < 5; ++i)
        if (per_cu[i] < 0)
            return TAV_ERR_ARG;
    if (V > kMaxVocab)
        return TAV_ERR_UNSUPPORTED;
    int64_t res[5];
    for (int i = 0; i < 5; ++i)
        res[i] = (int64_t)per_cu[i] * cus;
    SvPlan p;
    if (!sv_plan_for(B, V, greedy == 1, res, p))
        return TAV_ERR_LAUNCH;
    plan[0] = p.E;
    plan[1] = p.wpg;
    plan[2] = p.ngroups;
    plan[3] = p.chunk;
    return TAV_OK;
}

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t N, int32_t V)
{
    using namespace tav;
    if (B < 1 || N < 1 || N > kMaxNodes || V < 1 || V > kMaxVocab)
        return 0;
    return sv_workspace(B, V);
}

namespace tav {

tav_status sv_launch(const float *target_logits, const float *draft_logits,
                     const int32_t *parent, const int32_t *token, int32_t B, int32_t N, int32_t V,
                     double temperature, uint64_t seed, uint64_t offset, int32_t *path,
                     int32_t *n_accepted, int32_t *out_tokens, void *workspace, size_t ws_bytes,
                     uint32_t *dev_flags, void *stream, bool wor, double *p_rows,
                     double *q_rows, double *child_pq, const CommitArgs *commit)
{
    using namespace tav;
    // temperature 0 selects greedy verification, which reads no draft row
    const bool greedy = temperature == 0.0;
    if (!target_logits || (!draft_logits && !greedy) || !parent || !token || !path ||
        !n_accepted || !out_tokens)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || V < 1 || !(temperature >= 0.0) || !(temperature < INFINITY))
        return TAV_ERR_ARG;
    if (N > kMaxNodes || V > kMaxVocab)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(target_logits, 4) || (!greedy && !aligned(draft_logits, 4)))
        return TAV_ERR_ARG;
    SvPlan p;
    if (!sv_plan(B, V, greedy, p))
        return TAV_ERR_LAUNCH;
    const size_t need = kHeaderBytes + p.box_bytes;
    if (!workspace || ws_bytes < need || !aligned(workspace, 256))
        return TAV_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    SvArgs a;
    a.tl = target_logits;
    a.dl = draft_logits;
    a.parent = parent;
    a.token = token;
    a.B = B;
    a.N = N;
    a.V = V;
    a.T = temperature;
    a.seed = seed;
    a.offset = offset;
    a.path = path;
    a.n_acc = n_accepted;
    a.out_tok = out_tokens;
    a.done = reinterpret_cast<uint32_t *>(ws);
    a.box = reinterpret_cast<uint64_t *>(ws + kHeaderBytes);
    a.flags = dev_flags;
    a.wpg = p.wpg;
    a.ngroups = p.ngroups;
    a.chunk = p.chunk;
    a.vec4 = V % 4 == 0 && aligned(target_logits, 16) && (greedy || aligned(draft_logits, 16));
    a.p_rows = p_rows;
    a.q_rows = q_rows;
    a.child_pq = child_pq;
    a.cm = commit ? *commit : CommitArgs{};
    const bool probe = p_rows != nullptr;
    const dim3 grid(p.wpg * p.ngroups), block(kSvThreads);
    hipStream_t st = as_stream(stream);
    auto sampling = [&](auto e_c) {
        constexpr int E = decltype(e_c)::value;
        if (probe)
            hipLaunchKernelGGL((spec_verify_kernel<E, false, true>), grid, block, 0, st, a);
        else if (wor)
            hipLaunchKernelGGL((spec_verify_kernel<E, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((spec_verify_kernel<E, false>), grid, block, 0, st, a);
    };
    if (greedy)
        hipLaunchKernelGGL(spec_verify_greedy_kernel, grid, block, 0, st, a);
    else if (p.E == 4)
        sampling(std::integral_constant<int, 4>{});
    else if (p.E == 8)
        sampling(std::integral_constant<int, 8>{});
    else if (p.E == 16)
        sampling(std::integral_constant<int, 16>{});
    else
        sampling(std::integral_constant<int, 28>{});
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}

} // namespace tav

extern "C" tav_status spec_verify_sample(const float *target_logits, const float *draft_logits,
                                         const int32_t *parent, const int32_t *token, int32_t B,
                                         int32_t N, int32_t V, double temperature, uint64_t seed,
                                         uint64_t offset, int32_t *path, int32_t *n_accepted,
                                         int32_t *out_tokens, void *workspace, size_t ws_bytes,
                                         uint32_t *dev_flags, void *stream)
{
    return tav::sv_launch(target_logits, draft_logits, parent, token, B, N, V, temperature, seed,
                     offset, path, n_accepted, out_tokens, workspace, ws_bytes, dev_flags, stream,
                     false, nullptr, nullptr, nullptr);
}

extern "C" tav_status spec_verify_sample_wor(const float *target_logits,
                                             const float *draft_logits, const int32_t *parent,
                                             const int32_t *token, int32_t B, int32_t N,
                                             int32_t V, double temperature, uint64_t seed,
                                             uint64_t offset, int32_t *path, int32_t *n_accepted,
                                             int32_t *out_tokens, void *workspace,
                                             size_t ws_bytes, uint32_t *dev_flags, void *stream)
{
    return tav::sv_launch(target_logits, draft_logits, parent, token, B, N, V, temperature, seed,
                     offset, path, n_accepted, out_tokens, workspace, ws_bytes, dev_flags, stream,
                     true, nullptr, nullptr, nullptr);
}

extern "C" tav_status spec_verify_sample_commit(
    const float *target_logits, const float *draft_logits, const int32_t *parent,
    const int32_t *token, int32_t B, int32_t N, int32_t V, double temperature, uint64_t seed,
    uint64_t offset, int32_t without_replacement, int32_t *path, int32_t *n_accepted,
    int32_t *out_tokens, const uint16_t *k_tree, const uint16_t *v_tree, int32_t num_blocks,
    const int32_t *block_table, int32_t max_blocks, const int32_t *prefix_len, uint16_t *k_cache,
    uint16_t *v_cache, int32_t Hkv, int32_t D, int32_t block_size, int32_t *commit_slots,
    int32_t *new_prefix_len, void *workspace, size_t ws_bytes, uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    // kv_commit_path's checks, then the walk's (in sv_launch)
    if (!k_tree || !v_tree || !block_table || !prefix_len || !k_cache || !v_cache ||
        !commit_slots || !new_prefix_len)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1 ||
        (without_replacement != 0 && without_replacement != 1))
        return TAV_ERR_ARG;
    if (block_size != kBlock || (D != 64 && D != 128) || N > kMaxNodes)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 2))
        return TAV_ERR_ARG;
    CommitArgs c;
    c.k_tree = k_tree;
    c.v_tree = v_tree;
    c.block_table = block_table;
    c.prefix_len = prefix_len;
    c.k_cache = k_cache;
    c.v_cache = v_cache;
    c.commit_slots = commit_slots;
    c.new_prefix_len = new_prefix_len;
    c.num_blocks = num_blocks;
    c.max_blocks = max_blocks;
    c.Hkv = Hkv;
    c.D = D;
    return sv_launch(target_logits, draft_logits, parent, token, B, N, V, temperature, seed,
                     offset, path, n_accepted, out_tokens, workspace, ws_bytes, dev_flags, stream,
                     without_replacement != 0, nullptr, nullptr, nullptr, &c);
}

extern "C" tav_status spec_verify_sample_probe(
    const float *target_logits, const float *draft_logits, const int32_t *parent,
    const int32_t *token, int32_t B, int32_t N, int32_t V, double temperature, uint64_t seed,
    uint64_t offset, int32_t *path, int32_t *n_accepted, int32_t *out_tokens, double *p_rows,
    double *q_rows, double *child_pq, void *workspace, size_t ws_bytes, uint32_t *dev_flags,
    void *stream)
{
    using namespace tav;
    if (!p_rows || !q_rows || !child_pq || !aligned(p_rows, 8) || !aligned(q_rows, 8) ||
        !aligned(child_pq, 8) || !(temperature > 0.0))
        return TAV_ERR_ARG;
    return tav::sv_launch(target_logits, draft_logits, parent, token, B, N, V, temperature, seed,
                     offset, path, n_accepted, out_tokens, workspace, ws_bytes, dev_flags, stream,
                     false, p_rows, q_rows, child_pq);
}

extern "C" tav_status tav_philox_uniforms(uint64_t seed, uint64_t offset, int32_t B, int32_t N,
                                          float *u, void *stream)
{
    using namespace tav;
    if (!u || B < 1 || N < 1)
        return TAV_ERR_ARG;
    const int64_t n = (int64_t)B * N;
    hipLaunchKernelGGL(philox_uniforms_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0,
                       as_stream(stream), seed, offset, B, N, u);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}

extern "C" tav_status tav_target_probs(const float *logits, int64_t rows, int32_t V,
                                       double temperature, double *p, uint32_t *dev_flags,
                                       void *stream)
{
    using namespace tav;
    if (!logits || !p || rows < 1 || V < 1 || !(temperature > 0.0) || !(temperature < INFINITY))
        return TAV_ERR_ARG;
    if (rows > (1ll << 31) - 1)
        return TAV_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(target_probs_kernel, dim3((unsigned)rows), dim3(kSvThreads), 0,
                       as_stream(stream), logits, V, temperature, p, dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}
