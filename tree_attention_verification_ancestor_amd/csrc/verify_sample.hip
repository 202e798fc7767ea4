// spec_verify_sample: target/draft softmax over the vocabulary and the
// root-down rejection-sampling walk, all in float64.
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
// [r*chunk, (r+1)*chunk) and keeps them in registers (8 per thread, 512
// threads), so every pass over a row after the first is register-resident.
// The walk is serial; for each visited node u the group
//   1. takes its chunk of target row u (and draft row u if u has children)
//      and the logits of u's children's tokens, reduces a local
//      (max, sum exp) per row and exchanges it (one group sync). Every
//      workgroup merges the wpg pairs in the same order, so all hold
//      bit-identical normalisers and per-chunk masses;
//   2. tests the children in order. p(x), q(x) and the residual at x are
//      recomputed from the logits at x with the same instructions in every
//      workgroup, so every workgroup takes the same decision. Meanwhile the
//      rows of u's first child, the likeliest next node, are already being
//      fetched, so a walk down first children never waits on memory;
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
// acknowledged before another: a reader polls a member's words (one lane per
// member) until every one carries the current generation. Two parities
// suffice: a member can only reuse a slot after every member has arrived at
// the sync in between, i.e. after everyone has read it. The grid never
// exceeds what the device holds resident at once (from the occupancy query),
// and every wait is bounded: on expiry the kernel raises
// TAV_FLAG_SYNC_TIMEOUT and the workgroup stops, so every wave exits even on
// a device shared with other work. The last workgroup to finish clears every
// slot, so each call leaves the workspace as it found it (zero-filled).
//
// exp. Every exponential is exp_f64 below: a 64-entry table of 2^(j/64) and
// a degree-6 polynomial on |r| <= ln2/128 (a few ulp), about a third of the
// instructions of the general-purpose routine, which matters because the
// stats pass takes one exp per vocabulary entry and row.

#include <algorithm>

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
};

// ---------------------------------------------------------------------------
// exp in float64: x = (n/64) ln2 + r, exp(x) = 2^(n>>6) * 2^((n&63)/64) * e^r.

struct ExpTable {
    double t[64];   // 2^(j/64)
};

__device__ __forceinline__ double exp_f64(double x, const ExpTable &T)
{
    if (x < -746.0)
        return 0.0;   // below the smallest subnormal (also x = -inf); NaN falls through
    constexpr double kScale = 0x1.71547652b82fep+6;        // 64 / ln 2
    constexpr double kLn2Hi = 0x1.62e42fee00000p-1 / 64.0;  // ln 2 / 64, high part (exact n*hi)
    constexpr double kLn2Lo = 0x1.a39ef35793c76p-33 / 64.0; // ln 2 / 64, low part
    constexpr double kRound = 0x1.8p52;
    x = fmin(x, 709.0);
    const double nd = (x * kScale + kRound) - kRound;        // nearest integer to 64x/ln2
    const int n = (int)nd;
    double r = fma(-nd, kLn2Hi, x);
    r = fma(-nd, kLn2Lo, r);
    // e^r - 1 = r + r^2 (1/2 + r (1/6 + r (1/24 + r (1/120 + r/720))))
    double p = fma(r, 1.0 / 720.0, 1.0 / 120.0);
    p = fma(r, p, 1.0 / 24.0);
    p = fma(r, p, 1.0 / 6.0);
    p = fma(r, p, 0.5);
    p = fma(r * r, p, r);
    const double t = T.t[n & 63];
    return ldexp(fma(t, p, t), n >> 6);
}

__device__ void exp_table_init(ExpTable &T)
{
    if (threadIdx.x < 64)
        T.t[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
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

// Sum over the wave in lane order (an inclusive scan's last value).
__device__ __forceinline__ double wave_sum_ordered(double v)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(v, o);
        if ((threadIdx.x & 63) >= o)
            v += y;
    }
    return __shfl(v, 63);
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

// Threads 0..NW-1 publish word i = mine[i] (32 payload bits) in this
// workgroup's slot for generation `gen`; on return (true) thread t < wpg holds
// member t's payloads in got[0..NW). A group of one workgroup exchanges
// nothing. Returns false on a timeout.
template <int NW>
__device__ bool group_sync(uint64_t *box, int wpg, int rank, uint32_t gen,
                           const uint32_t (&mine)[NW], uint32_t (&got)[NW], uint32_t *flags)
{
    if (wpg == 1) {
#pragma unroll
        for (int i = 0; i < NW; ++i)
            got[i] = mine[i];
        return true;
    }
    uint64_t *base = box + (size_t)(gen & 1u) * wpg * kSlotWords;
    __syncthreads();
    if (threadIdx.x < NW) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            if ((int)threadIdx.x == i)
                v = mine[i];
        __hip_atomic_store(base + (size_t)rank * kSlotWords + threadIdx.x, tag_word(gen, v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NW; ++i)
        got[i] = 0u;
    if ((int)threadIdx.x < wpg) {
        uint64_t *slot = base + (size_t)threadIdx.x * kSlotWords;
        uint32_t polls = 0;
        for (;;) {
            uint64_t word[NW];
#pragma unroll
            for (int i = 0; i < NW; ++i)
                word[i] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool all = true;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                all &= (uint32_t)(word[i] >> 32) == gen;
                got[i] = (uint32_t)word[i];
            }
            if (all)
                break;
            __builtin_amdgcn_s_sleep(1);
            if (++polls > kSpinLimit) {
                ok = false;
                break;
            }
        }
    }
    ok = __syncthreads_and(ok);
    if (!ok && threadIdx.x == 0)
        raise_flag(flags, TAV_FLAG_SYNC_TIMEOUT);
    return ok;
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

__global__ __launch_bounds__(kSvThreads) void spec_verify_kernel(SvArgs a)
{
    __shared__ ExpTable s_exp;
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_first[kMaxNodes];
    __shared__ int32_t s_next[kMaxNodes];
    __shared__ int32_t s_tok[kMaxNodes];
    __shared__ float s_tx[kMaxNodes];     // target logit of child c's token in its parent's row
    __shared__ float s_dx[kMaxNodes];     // draft logit of the same
    __shared__ double s_red[2 * kSvWaves];
    __shared__ double s_mass[kMaxWpg];    // mass of every member's chunk in the current distribution
    __shared__ double s_zhist[kMaxNodes]; // residual normalisers after each rejection at u
    __shared__ double s_slot[kSvEpt * kSvWaves];
    __shared__ double s_hit_off;
    __shared__ int s_bad;
    __shared__ int s_found;
    __shared__ int s_last_live;
    __shared__ int s_hit;
    __shared__ int s_is_last;

    const int g = blockIdx.x % a.ngroups;
    const int rank = blockIdx.x / a.ngroups;
    const int tid = threadIdx.x;
    const int N = a.N;
    const int wpg = a.wpg;
    const int64_t base = (int64_t)rank * a.chunk;
    const int64_t lim = std::min<int64_t>((int64_t)a.V, base + a.chunk);
    uint64_t *box = a.box + (size_t)g * 2 * wpg * kSlotWords;
    const double invT = 1.0 / a.T;
    uint32_t gen = 0;
    bool alive = true;
    exp_table_init(s_exp);

    for (int b = g; b < a.B && alive; b += a.ngroups) {
        const int64_t rowbase = (int64_t)b * N;
        // ---- tree structure in LDS, validated ------------------------------
        __syncthreads();
        if (tid == 0)
            s_bad = 0;
        if (tid < N) {
            s_par[tid] = a.parent[rowbase + tid];
            s_tok[tid] = a.token[rowbase + tid];
            s_first[tid] = N;
            s_next[tid] = -1;
        }
        __syncthreads();
        if (tid < N) {
            const int p = s_par[tid];
            if (tid == 0 ? p != -1 : (p < 0 || p >= tid))
                atomicOr(&s_bad, 1);
            if (tid > 0 && (s_tok[tid] < 0 || s_tok[tid] >= a.V))
                atomicOr(&s_bad, 2);
        }
        __syncthreads();
        if (s_bad == 0 && tid >= 1 && tid < N) {
            atomicMin(&s_first[s_par[tid]], tid);
            for (int c2 = tid + 1; c2 < N; ++c2)
                if (s_par[c2] == s_par[tid]) {
                    s_next[tid] = c2;
                    break;
                }
        }
        __syncthreads();
        if (tid < N && s_first[tid] == N)
            s_first[tid] = -1;
        __syncthreads();

        const bool lead = rank == 0 && tid == 0;
        int nacc = 0;
        bool failed = s_bad != 0;
        if (failed && lead)
            raise_flag(a.flags, (s_bad & 1 ? TAV_FLAG_BAD_PARENT : 0u) |
                                    (s_bad & 2 ? TAV_FLAG_BAD_TOKEN : 0u));

        // rows of the likeliest next node, fetched a level ahead
        int pf_node = -1;
        float pf_t[kSvEpt], pf_d[kSvEpt];
        float pf_tx = 0.f, pf_dx = 0.f;   // logits of child `tid` of pf_node, if any

        int u = 0;
        while (!failed) {
            const float *trow = a.tl + (rowbase + u) * a.V;
            const float *drow = a.dl + (rowbase + u) * a.V;
            const bool has_kids = s_first[u] >= 0;

            // ---- 1. local (max, sum exp) of target and draft rows ------------
            float tf[kSvEpt], df[kSvEpt];
            if (pf_node == u) {
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    tf[e] = pf_t[e];
                    df[e] = has_kids ? pf_d[e] : -INFINITY;
                }
                if (tid < N && s_par[tid] == u) {
                    s_tx[tid] = pf_tx;
                    s_dx[tid] = pf_dx;
                }
            } else {
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const int64_t idx = base + (int64_t)e * kSvThreads + tid;
                    tf[e] = -INFINITY;
                    df[e] = -INFINITY;
                    if (idx < lim) {
                        tf[e] = trow[idx];
                        if (has_kids)
                            df[e] = drow[idx];
                    }
                }
                if (tid < N && s_par[tid] == u) {
                    const int x = s_tok[tid];
                    s_tx[tid] = trow[x];
                    s_dx[tid] = drow[x];
                }
            }
            // maxima of the raw fp32 logits (exact); x -> x/T is monotone
            bool nan_seen = false;
            double mt_d = -INFINITY, mq_d = -INFINITY;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e) {
                nan_seen |= __builtin_isnan(tf[e]) || __builtin_isnan(df[e]);
                mt_d = fmax(mt_d, (double)tf[e]);
                mq_d = fmax(mq_d, (double)df[e]);
            }
            block_max2(mt_d, mq_d, s_red);
            const float mt_raw = (float)mt_d, mq_raw = (float)mq_d;
            const double mts = (double)mt_raw * invT, mqs = (double)mq_raw * invT;
            double pr[kSvEpt], qv[kSvEpt];
            double zt = 0.0, zq = 0.0;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e) {
                pr[e] = (mt_raw == -INFINITY) ? 0.0 : exp_f64((double)tf[e] * invT - mts, s_exp);
                qv[e] = (mq_raw == -INFINITY) ? 0.0 : exp_f64((double)df[e] * invT - mqs, s_exp);
                zt += pr[e];
                zq += qv[e];
            }
            block_sum2(zt, zq, s_red);
            if (__syncthreads_or(nan_seen))
                zt = NAN;

            // the first child's rows and its children's logits, for the next level
            if (has_kids) {
                const int c1 = s_first[u];
                pf_node = c1;
                const float *t1 = a.tl + (rowbase + c1) * a.V;
                const float *d1 = a.dl + (rowbase + c1) * a.V;
                const bool c1_kids = s_first[c1] >= 0;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const int64_t idx = base + (int64_t)e * kSvThreads + tid;
                    pf_t[e] = -INFINITY;
                    pf_d[e] = -INFINITY;
                    if (idx < lim) {
                        pf_t[e] = t1[idx];
                        if (c1_kids)
                            pf_d[e] = d1[idx];
                    }
                }
                if (tid < N && s_par[tid] == c1) {
                    const int x = s_tok[tid];
                    pf_tx = t1[x];
                    pf_dx = d1[x];
                }
            }

            double m_got = -INFINITY, z_got = 0.0, mq_got = -INFINITY, zq_got = 0.0;
            {
                const uint32_t mine[6] = {f32_bits(mt_raw), f64_hi(zt), f64_lo(zt),
                                          f32_bits(mq_raw), f64_hi(zq), f64_lo(zq)};
                uint32_t words[6];
                if (!group_sync<6>(box, wpg, rank, ++gen, mine, words, a.flags)) {
                    alive = false;
                    break;
                }
                if (tid < wpg) {
                    m_got = (double)bits_f32(words[0]) * invT;
                    z_got = bits_f64(words[1], words[2]);
                    mq_got = (double)bits_f32(words[3]) * invT;
                    zq_got = bits_f64(words[4], words[5]);
                }
            }
            // merge the members' (max, sum) pairs in a fixed order
            double Mp = m_got, Mq = mq_got;
            block_max2(Mp, Mq, s_red);
            double em = 0.0, Zp = 0.0, Zq = 0.0;
            if (tid < wpg) {
                em = (m_got == -INFINITY) ? 0.0 : exp_f64(m_got - Mp, s_exp);
                // a NaN sum travels through; an empty chunk adds nothing
                Zp = (m_got == -INFINITY) ? (z_got != z_got ? z_got : 0.0) : z_got * em;
                Zq = (mq_got == -INFINITY) ? 0.0 : zq_got * exp_f64(mq_got - Mq, s_exp);
            }
            block_sum2(Zp, Zq, s_red);
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
            // chunk masses of p, and p and q of this chunk in registers
            if (tid < wpg)
                s_mass[tid] = z_got * em / Zp;
            {
                const double sp = (mt_raw == -INFINITY) ? 0.0 : exp_f64(mts - Mp, s_exp) / Zp;
                const double sq = (mq_raw == -INFINITY) ? 0.0 : exp_f64(mqs - Mq, s_exp) / Zq;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    pr[e] *= sp;
                    qv[e] *= sq;
                }
            }
            __syncthreads();   // s_mass, s_tx, s_dx visible

            // ---- 2./3. children in ascending order against the running residual
            int k = 0;
            bool accepted = false;
            for (int c = s_first[u]; c >= 0; c = s_next[c]) {
                const int x = s_tok[c];
                const double px = exp_f64((double)s_tx[c] * invT - Mp, s_exp) / Zp;
                const double qx = exp_f64((double)s_dx[c] * invT - Mq, s_exp) / Zq;
                double prx = px;
                for (int j = 0; j < k; ++j) {
                    const double zj = s_zhist[j];
                    if (zj > 0.0) {
                        const double d = prx - qx;
                        prx = (d > 0.0 ? d : 0.0) / zj;
                    }
                }
                const NodeUniforms r = node_uniforms(a.seed, a.offset, b, c);
                if (r.acc * qx < prx) {
                    if (lead) {
                        a.out_tok[rowbase + nacc] = x;
                        a.path[rowbase + nacc + 1] = c;
                    }
                    ++nacc;
                    u = c;
                    accepted = true;
                    break;
                }
                // rejected: chunk sums of the residual, exchanged
                double s = 0.0, unused = 0.0;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const double d = pr[e] - qv[e];
                    s += d > 0.0 ? d : 0.0;
                }
                block_sum2(s, unused, s_red);
                double rs = 0.0;
                {
                    const uint32_t mine[2] = {f64_hi(s), f64_lo(s)};
                    uint32_t words[2];
                    if (!group_sync<2>(box, wpg, rank, ++gen, mine, words, a.flags)) {
                        alive = false;
                        break;
                    }
                    if (tid < wpg)
                        rs = bits_f64(words[0], words[1]);
                }
                double Z = rs, unused2 = 0.0;
                block_sum2(Z, unused2, s_red);
                if (Z > 0.0) {
                    if (tid < wpg)
                        s_mass[tid] = rs / Z;
                    const double inv = 1.0 / Z;
#pragma unroll
                    for (int e = 0; e < kSvEpt; ++e) {
                        const double d = pr[e] - qv[e];
                        pr[e] = (d > 0.0 ? d : 0.0) * inv;
                    }
                }
                if (tid == 0)
                    s_zhist[k] = Z;
                ++k;
                __syncthreads();   // s_zhist, s_mass visible
            }
            if (!alive)
                break;
            if (accepted)
                continue;

            // ---- 4. inverse-CDF draw from the final distribution at u ---------
            // Member w's interval is [before_w, before_w + mass_w) with the
            // masses summed in member order, identically in every workgroup.
            if (tid == 0) {
                double run = 0.0, before = 0.0;
                for (int w = 0; w < wpg; ++w) {
                    if (w == rank)
                        before = run;
                    run += s_mass[w];
                }
                s_red[0] = before;
                s_red[1] = run;
                s_found = -1;
                s_last_live = -1;
                s_hit = -1;
            }
            __syncthreads();
            const double before = s_red[0], total = s_red[1];
            const double mass = s_mass[rank];
            const double target = node_uniforms(a.seed, a.offset, b, u).res * total;
            __syncthreads();
            if (!(total > 0.0)) {
                if (lead)
                    raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
                failed = true;
                break;
            }
            if (mass > 0.0 && before <= target && target < before + mass) {
                // element e of thread t is token base + e*512 + t, so token
                // order is (e, wave, lane). Totals of every (e, wave) slot
                // first, in that order; then the one wave holding the target
                // scans its lanes.
                const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const double t = wave_sum_ordered(pr[e]);
                    if (lane == 0)
                        s_slot[e * kSvWaves + wave] = t;
                }
                __syncthreads();
                if (tid == 0) {
                    double run = before;
                    for (int k2 = 0; k2 < kSvEpt * kSvWaves; ++k2) {
                        const double nxt = run + s_slot[k2];
                        if (s_slot[k2] > 0.0 && run <= target && target < nxt) {
                            s_hit = k2;
                            s_hit_off = run;
                            break;
                        }
                        run = nxt;
                    }
                }
                __syncthreads();
                const int hit = s_hit;
                if (hit >= 0 && wave == hit % kSvWaves) {
                    const int e_hit = hit / kSvWaves;
                    double v = 0.0;
#pragma unroll
                    for (int e = 0; e < kSvEpt; ++e)
                        if (e == e_hit)
                            v = pr[e];
                    double incl = v;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const double y = __shfl_up(incl, o);
                        if (lane >= o)
                            incl += y;
                    }
                    double excl = __shfl_up(incl, 1);
                    if (lane == 0)
                        excl = 0.0;
                    const double lo = s_hit_off + excl, hi = s_hit_off + incl;
                    const int64_t idx = base + (int64_t)e_hit * kSvThreads + tid;
                    if (v > 0.0) {
                        atomicMax(&s_last_live, (int)idx);
                        if (lo <= target && target < hi)
                            s_found = (int)idx;   // at most one lane qualifies
                    }
                }
                // rounding left the target past the chunk's summed slots: the
                // chunk's last live token takes it
                if (hit < 0) {
#pragma unroll
                    for (int e = 0; e < kSvEpt; ++e)
                        if (pr[e] > 0.0)
                            atomicMax(&s_last_live, (int)(base + (int64_t)e * kSvThreads + tid));
                }
                __syncthreads();
                if (tid == 0)
                    a.out_tok[rowbase + nacc] = s_found >= 0 ? s_found : s_last_live;
            }
            break;
        }

        // ---- outputs owned by the group leader ------------------------------
        if (lead) {
            if (failed || !alive) {
                for (int i = 0; i < N; ++i) {
                    a.path[rowbase + i] = i == 0 ? 0 : -1;
                    a.out_tok[rowbase + i] = -1;
                }
                a.n_acc[b] = 0;
            } else {
                a.path[rowbase] = 0;
                for (int i = nacc + 1; i < N; ++i) {
                    a.path[rowbase + i] = -1;
                    a.out_tok[rowbase + i] = -1;
                }
                a.n_acc[b] = nacc;
            }
        }
    }

    // ---- exit: the last workgroup out clears every mailbox word -------------
    // Each workgroup counts itself out only after its last poll, so the last
    // one knows no slot is still being read.
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
    int wpg, ngroups, chunk;
    size_t box_bytes;
};

bool sv_plan(int32_t B, int32_t V, SvPlan &p)
{
    const int cus = device_cu_count();
    if (cus <= 0)
        return false;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, spec_verify_kernel, kSvThreads,
                                                     0) != hipSuccess ||
        per_cu <= 0)
        return false;
    const int64_t resident = (int64_t)per_cu * cus;
    p.wpg = (int)ceil_div(V, kSvChunk);
    if (p.wpg > resident || p.wpg > kMaxWpg)
        return false;
    p.chunk = (int)ceil_div(V, p.wpg);
    p.ngroups = (int)std::min<int64_t>(B, resident / p.wpg);
    p.box_bytes = (size_t)p.ngroups * 2 * p.wpg * kSlotWords * sizeof(uint64_t);
    return true;
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
    __shared__ ExpTable s_exp;
    __shared__ double red[2 * kSvWaves];
    exp_table_init(s_exp);
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
        z += exp_f64((double)row[x] * invT - ms, s_exp);
    block_sum2(z, unused2, red);
    if (__syncthreads_or(nan_seen) || m == -INFINITY || __builtin_isinf(m)) {
        if (threadIdx.x == 0)
            raise_flag(flags, TAV_FLAG_NONFINITE_LOGITS);
        return;
    }
    for (int x = threadIdx.x; x < V; x += kSvThreads)
        out[x] = exp_f64((double)row[x] * invT - ms, s_exp) / z;
}

} // namespace
} // namespace tav

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t N, int32_t V)
{
    using namespace tav;
    if (B < 1 || N < 1 || N > kMaxNodes || V < 1 || V > kMaxVocab)
        return 0;
    SvPlan p;
    if (!sv_plan(B, V, p))
        return 0;
    return kHeaderBytes + p.box_bytes;
}

extern "C" tav_status spec_verify_sample(const float *target_logits, const float *draft_logits,
                                         const int32_t *parent, const int32_t *token, int32_t B,
                                         int32_t N, int32_t V, double temperature, uint64_t seed,
                                         uint64_t offset, int32_t *path, int32_t *n_accepted,
                                         int32_t *out_tokens, void *workspace, size_t ws_bytes,
                                         uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!target_logits || !draft_logits || !parent || !token || !path || !n_accepted ||
        !out_tokens)
        return TAV_ERR_ARG;
    if (B < 1 || N < 1 || V < 1 || !(temperature > 0.0) || !(temperature < INFINITY))
        return TAV_ERR_ARG;
    if (N > kMaxNodes || V > kMaxVocab)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(target_logits, 4) || !aligned(draft_logits, 4))
        return TAV_ERR_ARG;
    SvPlan p;
    if (!sv_plan(B, V, p))
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
    hipLaunchKernelGGL(spec_verify_kernel, dim3(p.wpg * p.ngroups), dim3(kSvThreads), 0,
                       as_stream(stream), a);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
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
