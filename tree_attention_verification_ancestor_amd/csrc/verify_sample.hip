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
// [r*chunk, (r+1)*chunk) and keeps them in registers (16 per thread), so
// every pass over a row after the first is register-resident. The walk is
// serial: for each visited node u the group
//   1. loads its chunk of target row u (and draft row u if u has children),
//      reduces a local (max, sum exp), publishes it and meets at a barrier;
//      every workgroup merges the wpg pairs in the same order, so all hold
//      bit-identical (max, normaliser) pairs;
//   2. tests the children in order. The test values p(x), q(x) and the
//      residual at x are recomputed from the logits at x by every workgroup
//      with the same instructions, so every workgroup takes the same decision;
//   3. after each rejection reduces sum(max(0, p_res - q)) (one barrier) and
//      updates its register chunk;
//   4. at the stopping node reduces the chunk masses (one barrier); the one
//      workgroup whose prefix interval holds r * total scans its chunk.
// Barriers are group-local (an arrival counter plus a generation word in the
// workspace) and every wait is bounded: on expiry the kernel raises
// TAV_FLAG_SYNC_TIMEOUT and the workgroup stops, so every wave exits. The
// launch is cooperative, which guarantees all workgroups are resident.

#include <algorithm>

#include "common.h"
#include "philox.h"

namespace tav {
namespace {

constexpr int kSvThreads = 256;
constexpr int kSvWaves = kSvThreads / 64;
constexpr int kSvEpt = 16;                      // vocabulary entries per thread
constexpr int kSvChunk = kSvThreads * kSvEpt;   // per workgroup
constexpr uint32_t kSpinLimit = 1u << 21;       // polls before a wait gives up
constexpr int kSyncStride = 32;                 // uint32 words per group (128 B)

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
    double *xch;      // [ngroups][2][wpg][4]
    uint32_t *sync;   // [ngroups][kSyncStride]: [0] arrivals, [16] generation
    uint32_t *flags;
    int32_t wpg, ngroups, chunk;
};

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_max(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmax(v, __shfl_xor(v, o));
    return v;
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

// Workgroup-wide reductions; every thread gets the result. `red` holds
// kSvWaves doubles; waves combine in index order.
__device__ double block_sum(double v, double *red)
{
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kSvWaves; ++w)
        s += red[w];
    return s;
}

__device__ double block_max(double v, double *red)
{
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    double m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSvWaves; ++w)
        m = fmax(m, red[w]);
    return m;
}

// Group barrier (sense by generation). Returns false if the wait expired.
//
// Everything workgroups exchange (the partial sums in `xch`, the arrival
// count, the generation word) moves through agent-scope atomics, which the
// hardware keeps coherent across XCDs at the memory side without flushing or
// invalidating the L2. Ordering comes from completion waits instead of
// release/acquire fences: thread 0, which also wrote this workgroup's
// exchange slots, waits until those stores and its read of the generation
// have completed before it counts itself in; the last arrival resets the
// count and only then publishes the next generation. Waiters poll the
// generation; the exchange slots they read afterwards were complete before
// any arrival that let the generation move.
__device__ bool group_barrier(uint32_t *cnt, uint32_t *gen, uint32_t members, uint32_t *flags,
                              int *s_ok)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        const uint32_t g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        const uint32_t arrived =
            __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == members - 1) {
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);
            __hip_atomic_store(gen, g0 + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            uint32_t polls = 0;
            while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
                __builtin_amdgcn_s_sleep(1);
                if (++polls > kSpinLimit) {
                    ok = 0;
                    raise_flag(flags, TAV_FLAG_SYNC_TIMEOUT);
                    break;
                }
            }
        }
        *s_ok = ok;
    }
    __syncthreads();
    return *s_ok != 0;
}

__device__ __forceinline__ void xch_put(double *slot, double v)
{
    __hip_atomic_store(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ double xch_get(const double *slot)
{
    return __hip_atomic_load(const_cast<double *>(slot), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kSvThreads) void spec_verify_kernel(SvArgs a)
{
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_first[kMaxNodes];
    __shared__ int32_t s_next[kMaxNodes];
    __shared__ double s_red[kSvWaves];
    __shared__ double s_zhist[kMaxNodes];
    __shared__ double s_stats[4];
    __shared__ int s_ok;
    __shared__ int s_bad;
    __shared__ int s_found;
    __shared__ int s_last_live;
    __shared__ int s_hit;
    __shared__ double s_slot[kSvEpt * kSvWaves];

    const int g = blockIdx.x % a.ngroups;
    const int rank = blockIdx.x / a.ngroups;
    const int tid = threadIdx.x;
    const int N = a.N;
    const int64_t base = (int64_t)rank * a.chunk;
    const int64_t lim = std::min<int64_t>((int64_t)a.V, base + a.chunk);
    uint32_t *cnt = a.sync + (int64_t)g * kSyncStride;
    uint32_t *gen = cnt + 16;
    double *xch = a.xch + (int64_t)g * 2 * a.wpg * 4;
    const uint32_t members = (uint32_t)a.wpg;
    int parity = 0;
    bool alive = true;

    for (int b = g; b < a.B && alive; b += a.ngroups) {
        const int64_t rowbase = (int64_t)b * N;
        // ---- tree structure in LDS, validated ------------------------------
        __syncthreads();
        if (tid == 0)
            s_bad = 0;
        for (int i = tid; i < N; i += kSvThreads) {
            s_par[i] = a.parent[rowbase + i];
            s_first[i] = N;
            s_next[i] = -1;
        }
        __syncthreads();
        for (int i = tid; i < N; i += kSvThreads) {
            const int p = s_par[i];
            if (i == 0 ? p != -1 : (p < 0 || p >= i))
                atomicOr(&s_bad, 1);
            if (i > 0) {
                const int x = a.token[rowbase + i];
                if (x < 0 || x >= a.V)
                    atomicOr(&s_bad, 2);
            }
        }
        __syncthreads();
        if (s_bad == 0) {
            for (int c = 1 + tid; c < N; c += kSvThreads) {
                atomicMin(&s_first[s_par[c]], c);
                for (int c2 = c + 1; c2 < N; ++c2)
                    if (s_par[c2] == s_par[c]) {
                        s_next[c] = c2;
                        break;
                    }
            }
        }
        __syncthreads();
        for (int i = tid; i < N; i += kSvThreads)
            if (s_first[i] == N)
                s_first[i] = -1;
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
            double pr[kSvEpt], qv[kSvEpt];
            bool nan_seen = false;
            double mt = -INFINITY, mq = -INFINITY;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e) {
                const int64_t idx = base + (int64_t)e * kSvThreads + tid;
                pr[e] = -INFINITY;
                qv[e] = -INFINITY;
                if (idx < lim) {
                    pr[e] = (double)trow[idx] / a.T;
                    if (has_kids)
                        qv[e] = (double)drow[idx] / a.T;
                }
                nan_seen |= __builtin_isnan(pr[e]) || __builtin_isnan(qv[e]);
                mt = fmax(mt, pr[e]);
                mq = fmax(mq, qv[e]);
            }
            mt = block_max(mt, s_red);
            mq = block_max(mq, s_red);
            double zt = 0.0, zq = 0.0;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e) {
                pr[e] = (mt == -INFINITY) ? 0.0 : exp(pr[e] - mt);
                qv[e] = (mq == -INFINITY) ? 0.0 : exp(qv[e] - mq);
                zt += pr[e];
                zq += qv[e];
            }
            zt = block_sum(zt, s_red);
            zq = block_sum(zq, s_red);
            if (__syncthreads_or(nan_seen))
                zt = NAN;
            double *mine = xch + ((int64_t)parity * a.wpg + rank) * 4;
            if (tid == 0) {
                xch_put(mine + 0, mt);
                xch_put(mine + 1, zt);
                xch_put(mine + 2, mq);
                xch_put(mine + 3, zq);
            }
            if (!group_barrier(cnt, gen, members, a.flags, &s_ok)) {
                alive = false;
                break;
            }
            // every workgroup merges the wpg pairs in rank order
            if (tid == 0) {
                const double *all = xch + (int64_t)parity * a.wpg * 4;
                double Mp = -INFINITY, Mq = -INFINITY;
                for (int w = 0; w < a.wpg; ++w) {
                    Mp = fmax(Mp, xch_get(all + w * 4 + 0));
                    Mq = fmax(Mq, xch_get(all + w * 4 + 2));
                }
                double Zp = 0.0, Zq = 0.0;
                for (int w = 0; w < a.wpg; ++w) {
                    const double m1 = xch_get(all + w * 4 + 0), z1 = xch_get(all + w * 4 + 1);
                    const double m2 = xch_get(all + w * 4 + 2), z2 = xch_get(all + w * 4 + 3);
                    Zp += (m1 == -INFINITY) ? (z1 != z1 ? z1 : 0.0) : z1 * exp(m1 - Mp);
                    Zq += (m2 == -INFINITY) ? 0.0 : z2 * exp(m2 - Mq);
                }
                s_stats[0] = Mp;
                s_stats[1] = Zp;
                s_stats[2] = Mq;
                s_stats[3] = Zq;
            }
            parity ^= 1;
            __syncthreads();
            const double Mp = s_stats[0], Zp = s_stats[1], Mq = s_stats[2], Zq = s_stats[3];
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
            // registers now hold p and q of this chunk
            {
                const double sp = (mt == -INFINITY) ? 0.0 : exp(mt - Mp) / Zp;
                const double sq = (mq == -INFINITY) ? 0.0 : exp(mq - Mq) / Zq;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    pr[e] *= sp;
                    qv[e] *= sq;
                }
            }

            // ---- 2./3. children in ascending order against the running residual
            int k = 0;
            bool accepted = false;
            for (int c = s_first[u]; c >= 0; c = s_next[c]) {
                const int x = a.token[rowbase + c];
                const double px = exp((double)trow[x] / a.T - Mp) / Zp;
                const double qx = exp((double)drow[x] / a.T - Mq) / Zq;
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
                // rejected: residual normaliser over the whole vocabulary
                double s = 0.0;
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const double d = pr[e] - qv[e];
                    s += d > 0.0 ? d : 0.0;
                }
                s = block_sum(s, s_red);
                double *slot = xch + ((int64_t)parity * a.wpg + rank) * 4;
                if (tid == 0)
                    xch_put(slot, s);
                if (!group_barrier(cnt, gen, members, a.flags, &s_ok)) {
                    alive = false;
                    break;
                }
                if (tid == 0) {
                    const double *all = xch + (int64_t)parity * a.wpg * 4;
                    double Z = 0.0;
                    for (int w = 0; w < a.wpg; ++w)
                        Z += xch_get(all + w * 4);
                    s_zhist[k] = Z;
                }
                parity ^= 1;
                __syncthreads();
                const double Z = s_zhist[k];
                ++k;
                if (Z > 0.0) {
#pragma unroll
                    for (int e = 0; e < kSvEpt; ++e) {
                        const double d = pr[e] - qv[e];
                        pr[e] = (d > 0.0 ? d : 0.0) / Z;
                    }
                }
            }
            if (!alive)
                break;
            if (accepted)
                continue;

            // ---- 4. inverse-CDF draw from the final distribution at u ---------
            double mass = 0.0;
#pragma unroll
            for (int e = 0; e < kSvEpt; ++e)
                mass += pr[e];
            mass = block_sum(mass, s_red);
            double *slot = xch + ((int64_t)parity * a.wpg + rank) * 4;
            if (tid == 0)
                xch_put(slot, mass);
            if (!group_barrier(cnt, gen, members, a.flags, &s_ok)) {
                alive = false;
                break;
            }
            if (tid == 0) {
                const double *all = xch + (int64_t)parity * a.wpg * 4;
                double before = 0.0, run = 0.0;
                for (int w = 0; w < a.wpg; ++w) {
                    if (w == rank)
                        before = run;
                    run += xch_get(all + w * 4);
                }
                s_stats[0] = before;
                s_stats[1] = run;   // total mass
                s_found = -1;
                s_last_live = -1;
            }
            parity ^= 1;
            __syncthreads();
            const double before = s_stats[0], total = s_stats[1];
            const double target = node_uniforms(a.seed, a.offset, b, u).res * total;
            // this workgroup's interval is [before, before + mass) in the same
            // summation order the total used
            const double after = before + mass;
            if (!(total > 0.0)) {
                if (lead)
                    raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
                failed = true;
                break;
            }
            if (mass > 0.0 && before <= target && target < after) {
                // element e of thread t is token base + e*256 + t, so token order
                // is (e, wave, lane). Totals of every (e, wave) slot first, in
                // that order; then the one wave holding the target scans its lanes.
                const int lane = tid & 63, wave = tid >> 6;
                double *slot_tot = s_slot;     // [kSvEpt][kSvWaves]
#pragma unroll
                for (int e = 0; e < kSvEpt; ++e) {
                    const double t = wave_sum_ordered(pr[e]);
                    if (lane == 0)
                        slot_tot[e * kSvWaves + wave] = t;
                }
                __syncthreads();
                if (tid == 0) {
                    double run = before;
                    int hit = -1;
                    double hit_off = 0.0;
                    for (int k2 = 0; k2 < kSvEpt * kSvWaves; ++k2) {
                        const double nxt = run + slot_tot[k2];
                        if (slot_tot[k2] > 0.0 && run <= target && target < nxt) {
                            hit = k2;
                            hit_off = run;
                            break;
                        }
                        run = nxt;
                    }
                    s_hit = hit;
                    s_stats[2] = hit_off;
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
                    const double off = s_stats[2];
                    const double lo = off + excl, hi = off + incl;
                    const int64_t idx = base + (int64_t)e_hit * kSvThreads + tid;
                    if (v > 0.0) {
                        atomicMax(&s_last_live, (int)idx);
                        if (lo <= target && target < hi)
                            s_found = (int)idx;   // at most one lane qualifies
                    }
                }
                // rounding left the target past the last live token: take that token
                if (hit < 0) {
#pragma unroll
                    for (int e = 0; e < kSvEpt; ++e)
                        if (pr[e] > 0.0)
                            atomicMax(&s_last_live, (int)(base + (int64_t)e * kSvThreads + tid));
                }
                __syncthreads();
                // the lane intervals of the hit slot partition its total exactly
                // (same scan), so s_found is set unless rounding put the target
                // past the chunk's summed slots; then the last live token wins
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
}

__global__ void zero_words_kernel(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

struct SvPlan {
    int wpg, ngroups, chunk;
    size_t xch_bytes, sync_bytes;
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
    if (p.wpg > resident)
        return false;
    p.chunk = (int)ceil_div(V, p.wpg);
    p.ngroups = (int)std::min<int64_t>(B, resident / p.wpg);
    p.xch_bytes = (size_t)p.ngroups * 2 * p.wpg * 4 * sizeof(double);
    p.sync_bytes = (size_t)p.ngroups * kSyncStride * sizeof(uint32_t);
    return true;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

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

__global__ __launch_bounds__(kSvThreads) void target_probs_kernel(const float *logits,
                                                                  int32_t V, double T,
                                                                  double *p, uint32_t *flags)
{
    __shared__ double red[kSvWaves];
    const float *row = logits + (int64_t)blockIdx.x * V;
    double *out = p + (int64_t)blockIdx.x * V;
    double m = -INFINITY;
    bool nan_seen = false;
    for (int x = threadIdx.x; x < V; x += kSvThreads) {
        const double v = (double)row[x] / T;
        nan_seen |= __builtin_isnan(v);
        m = fmax(m, v);
    }
    m = block_max(m, red);
    double z = 0.0;
    for (int x = threadIdx.x; x < V; x += kSvThreads)
        z += exp((double)row[x] / T - m);
    z = block_sum(z, red);
    if (__syncthreads_or(nan_seen) || m == -INFINITY || __builtin_isinf(m)) {
        if (threadIdx.x == 0)
            raise_flag(flags, TAV_FLAG_NONFINITE_LOGITS);
        return;
    }
    for (int x = threadIdx.x; x < V; x += kSvThreads)
        out[x] = exp((double)row[x] / T - m) / z;
}

} // namespace
} // namespace tav

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t N, int32_t V)
{
    using namespace tav;
    if (B < 1 || N < 1 || N > kMaxNodes || V < 1 || V > (1 << 24))
        return 0;
    SvPlan p;
    if (!sv_plan(B, V, p))
        return 0;
    return round_up(p.xch_bytes, 256) + round_up(p.sync_bytes, 256);
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
    if (N > kMaxNodes || V > (1 << 24))
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(target_logits, 4) || !aligned(draft_logits, 4))
        return TAV_ERR_ARG;
    SvPlan p;
    if (!sv_plan(B, V, p))
        return TAV_ERR_LAUNCH;
    const size_t need = round_up(p.xch_bytes, 256) + round_up(p.sync_bytes, 256);
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
    a.xch = reinterpret_cast<double *>(ws);
    a.sync = reinterpret_cast<uint32_t *>(ws + round_up(p.xch_bytes, 256));
    a.flags = dev_flags;
    a.wpg = p.wpg;
    a.ngroups = p.ngroups;
    a.chunk = p.chunk;
    hipStream_t s = as_stream(stream);
    const int64_t words = (int64_t)p.ngroups * kSyncStride;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(words, 256), 64)),
                       dim3(256), 0, s, a.sync, words);
    if (hipGetLastError() != hipSuccess)
        return TAV_ERR_LAUNCH;
    void *args[] = {&a};
    const hipError_t err =
        hipLaunchCooperativeKernel(reinterpret_cast<const void *>(spec_verify_kernel),
                                   dim3(p.wpg * p.ngroups), dim3(kSvThreads), args, 0, s);
    return err == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
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
