// tree_expand_topk: for each draft row, the k most likely tokens with their
// log-probabilities and the distribution's entropy. Top-k branching expands a
// node by its draft's k most likely tokens, and entropy-based branching gives
// a node more branches the higher its draft entropy (jisaku.com glossary,
// tree-topology strategies); both read these per frontier node.
//
// With q = softmax(x / T), M the row maximum and y = (x - M) / T:
//   log q(x) = y_x - log S0,  H(q) = log S0 - S1 / S0,
//   S0 = sum e^y,  S1 = sum y e^y.
// Two kernels. The first splits each row into 2048-entry shares, one per
// wave (32 entries per lane, 16-byte loads): each wave takes its k best
// (value, token) keys in k rounds of a wave-wide 64-bit key maximum (the
// value's order-preserving bits above the complement of the token, so ties go
// to the lower token) and its (max, S0, S1) relative to its own maximum, with
// each term's exponential in fp32 and the sums in fp64, and writes them: no
// barrier. The second, one workgroup per row, rebases the partial sums to the
// row maximum (S1 -> e^d (S1 + d S0), S0 -> e^d S0 with d = (m - M) / T) and
// takes the k best keys among the waves' candidates; one wave per row does it. Within a lane, each run
// of four terms is summed in fp32 (same-sign terms: within three roundings)
// and the run totals in fp64.

#include <algorithm>

#include "common.h"
#include "philox.h"

namespace tav {
namespace {

constexpr int kExThreads = 512;
constexpr int kExWaves = kExThreads / 64;
constexpr int kExEpt = 32;                      // entries per thread
constexpr int kExChunk = kExThreads * kExEpt;   // entries per workgroup
constexpr int kExWaveChunk = 64 * kExEpt;       // entries per wave
constexpr int kExMaxK = 16;
constexpr int kExMaxWpr = 128;                  // workgroups per row (V <= 2^21)
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

struct ExPart {          // one wave's share of a row
    double s0, s1;
    float m;             // maximum of its entries (-inf if none)
    int32_t nan;
    uint64_t key[kExMaxK];
};

__device__ __forceinline__ uint32_t ordered_bits(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o)
{
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float v, int64_t t)
{
    return ((uint64_t)ordered_bits(v) << 32) | (0xFFFFFFFFu - (uint32_t)t);
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

__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    v = max_u64(v, dpp_u64<kQuadSwap1>(v));
    v = max_u64(v, dpp_u64<kQuadSwap2>(v));
    v = max_u64(v, dpp_u64<kRowHalfMirror>(v));
    v = max_u64(v, dpp_u64<kRowMirror>(v));
    return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)), max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

__device__ __forceinline__ double wave_sum(double v)
{
    auto dpp = [](double x, auto ctrl) __attribute__((always_inline)) {
        constexpr int C = decltype(ctrl)::value;
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, C, 0xF, 0xF, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), C, 0xF, 0xF, false);
        return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    v += dpp(v, std::integral_constant<int, kQuadSwap1>{});
    v += dpp(v, std::integral_constant<int, kQuadSwap2>{});
    v += dpp(v, std::integral_constant<int, kRowHalfMirror>{});
    v += dpp(v, std::integral_constant<int, kRowMirror>{});
    auto rl = [](double x, int l) __attribute__((always_inline)) {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
        return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}

struct ExArgs {
    const float *x;
    int64_t R;
    int32_t V, k, wpr, vec4;
    float invT32;
    double invT;
    ExPart *part;        // [R][wpr * kExWaves]
    int32_t *top_token;  // [R][k]
    double *top_logq;    // [R][k]
    double *entropy;     // [R]
    uint32_t *flags;
    int32_t sampled;     // rank by x/T + Gumbel noise instead of x
    uint64_t seed, offset;
};

// One wave's partial of a row from its entries v (lane order: tokens rise
// with e). kClean: every entry is in the row and none is NaN, so the
// per-entry tests drop out.
template <bool kClean, bool kSampled, typename Tok>
__device__ __forceinline__ void wave_partial(const ExArgs &a, const float (&v)[kExEpt],
                                             const float (&sk)[kExEpt], Tok tok, int lane,
                                             ExPart *out)
{
    // sk: the values the k best are chosen by (v itself, or the sampling
    // keys, which are NaN exactly where v is); v: the logits of the sums
    const int64_t lim = a.V;
    bool nan_seen = false;
#pragma unroll
    for (int e = 0; e < kExEpt; ++e)
        nan_seen |= (!kClean && __builtin_isnan(v[e])) && tok(e) < lim;
    // The wave's k best keys. Fast path: each lane's best entry (the first of
    // equal values, i.e. its lower token) as a key, and the k best of those
    // in k rounds of a wave-wide key maximum; tau, the k-th of them, bounds
    // every entry of the wave's top k from below (k lanes hold an entry of
    // at least tau). If no lane holds two entries >= tau, the wave's top k
    // are those lane keys. Otherwise every round rescans: each lane offers
    // its best entry not yet taken, and the winner's lane marks it taken.
    float lm = 0.f;
    int le = -1;
#pragma unroll
    for (int e = 0; e < kExEpt; ++e) {
        if (!(!kClean && __builtin_isnan(sk[e])) && (le < 0 || sk[e] > lm)) {
            lm = sk[e];
            le = e;
        }
    }
    const uint64_t lkey = le < 0 ? 0ull : make_key(lm, tok(le));
    uint64_t first = 0, last = 0;
    {
        uint64_t offer = lkey;
        for (int i = 0; i < a.k; ++i) {
            const uint64_t win = wave_max_key(offer);
            if (offer == win)
                offer = 0ull;
            if (i == 0)
                first = win;
            last = win;
            if (lane == 0)
                out->key[i] = win;
        }
    }
    const float tau = last == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(last >> 32));
    int above = 0;
#pragma unroll
    for (int e = 0; e < kExEpt; ++e)
        above += (!(!kClean && __builtin_isnan(sk[e])) && sk[e] >= tau) ? 1 : 0;
    if (last == 0ull || __any(above > 1)) {
        uint32_t taken = 0;
        for (int i = 0; i < a.k; ++i) {
            float bv = 0.f;
            int be = -1;
#pragma unroll
            for (int e = 0; e < kExEpt; ++e) {
                const bool ok = !((taken >> e) & 1u) && !(!kClean && __builtin_isnan(sk[e]));
                if (ok && (be < 0 || sk[e] > bv)) {
                    bv = sk[e];
                    be = e;
                }
            }
            const uint64_t mine = be < 0 ? 0ull : make_key(bv, tok(be));
            const uint64_t win = wave_max_key(mine);
            if (be >= 0 && mine == win)
                taken |= 1u << be;
            if (lane == 0)
                out->key[i] = win;
        }
    }
    // sums relative to the wave's maximum logit (-inf when it holds no
    // entry): the best key's value, unless the keys are sampling keys
    float m;
    if constexpr (kSampled) {
        float lx = -INFINITY;
        bool any = false;
#pragma unroll
        for (int e = 0; e < kExEpt; ++e) {
            if (!(!kClean && __builtin_isnan(v[e]))) {
                lx = any ? fmaxf(lx, v[e]) : v[e];
                any = true;
            }
        }
        const uint64_t mk = wave_max_key(any ? (uint64_t)ordered_bits(lx) << 32 : 0ull);
        m = mk == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(mk >> 32));
    } else {
        m = first == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(first >> 32));
    }
    const float ms = m * a.invT32;
    // Each run of four entries is summed in fp32 (same-sign terms, so within
    // three fp32 roundings of exact), the run totals in fp64.
    double s0 = 0.0, s1 = 0.0;
    if (m != -INFINITY) {
#pragma unroll
        for (int h = 0; h < kExEpt / 4; ++h) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = v[4 * h + j];
                const float y = fmaf(x, a.invT32, -ms);   // one rounding
                const float ev = __builtin_amdgcn_exp2f(y * 0x1.715476p+0f);
                if constexpr (kClean) {
                    // -inf gives ev = 0; y clamped so y * 0 stays 0
                    r0 += ev;
                    r1 = fmaf(fmaxf(y, -1.0e4f), ev, r1);
                } else {
                    const bool live = x != -INFINITY && !__builtin_isnan(x);
                    r0 += live ? ev : 0.f;
                    r1 = live ? fmaf(y, ev, r1) : r1;
                }
            }
            s0 += (double)r0;
            s1 += (double)r1;
        }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    const bool wnan = __any(nan_seen);
    if (lane == 0) {
        out->s0 = s0;
        out->s1 = s1;
        out->m = m;
        out->nan = wnan;
    }
}

template <bool kSampled>
__global__ __launch_bounds__(kExThreads) void expand_part_kernel(ExArgs a)
{
    // Each wave owns kExWaveChunk consecutive entries of one row: lane l holds
    // tokens wbase + 256 h + 4 l + j (h < 8, j < 4), read 16 bytes at a time,
    // so a lane's entries rise in token order. No barrier: every wave writes
    // its own partial.
    const int64_t r = blockIdx.x / a.wpr;
    const int w = (int)(blockIdx.x % a.wpr);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *row = a.x + r * a.V;
    const int64_t wbase = (int64_t)w * kExChunk + (int64_t)wave * kExWaveChunk;
    const int64_t lim = a.V;
    // A share wholly inside the row (every share but a row's last) is read
    // without per-entry range tests; if it also holds no NaN (one
    // NaN-propagating maximum tells), the passes below skip the per-entry
    // NaN tests too.
    const bool full = a.vec4 && wbase + kExWaveChunk <= lim;   // wave-uniform
    float v[kExEpt];
    if (full) {
#pragma unroll
        for (int h = 0; h < kExEpt / 4; ++h) {
            const f32x4 q = *reinterpret_cast<const f32x4 *>(row + wbase + (int64_t)h * 256 + 4 * lane);
            v[4 * h] = q.x;
            v[4 * h + 1] = q.y;
            v[4 * h + 2] = q.z;
            v[4 * h + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int h = 0; h < kExEpt / 4; ++h) {
            const int64_t i0 = wbase + (int64_t)h * 256 + 4 * lane;
            if (a.vec4 && i0 + 3 < lim) {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(row + i0);
                v[4 * h] = q.x;
                v[4 * h + 1] = q.y;
                v[4 * h + 2] = q.z;
                v[4 * h + 3] = q.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[4 * h + j] = i0 + j < lim ? row[i0 + j] : NAN;   // NaN: not an entry
            }
        }
    }
    bool clean = false;
    if (full) {
        float mx = v[0];
#pragma unroll
        for (int e = 1; e < kExEpt; ++e)
            mx = __builtin_elementwise_maximum(mx, v[e]);   // NaN-propagating
        clean = !__any(__builtin_isnan(mx));
    }
    auto tok = [&](int e) __attribute__((always_inline)) {
        return wbase + (int64_t)(e >> 2) * 256 + 4 * lane + (e & 3);
    };
    ExPart *out = a.part + (r * a.wpr + w) * kExWaves + wave;
    if constexpr (kSampled) {
        // sampling keys fl32(fl32(x * (1/T)) + fl32(G)), G = -log(-log u) in
        // fp64, u from word (token mod 4) of Philox at counter (offset, row,
        // token / 4, 1): each run of four tokens is one Philox block
        float sk[kExEpt];
#pragma unroll
        for (int h = 0; h < kExEpt / 4; ++h) {
            uint64_t wd[4];
            philox4x64_10(a.offset, (uint64_t)r, (uint64_t)(tok(4 * h) >> 2), 1, a.seed, 0, wd);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double u = ((double)(wd[j] >> 11) + 0.5) * 0x1p-53;
                const float g = (float)(-log(-log(u)));
                sk[4 * h + j] = __fadd_rn(__fmul_rn(v[4 * h + j], a.invT32), g);
            }
        }
        if (clean)
            wave_partial<true, true>(a, v, sk, tok, lane, out);
        else
            wave_partial<false, true>(a, v, sk, tok, lane, out);
    } else if (clean) {
        wave_partial<true, false>(a, v, v, tok, lane, out);
    } else {
        wave_partial<false, false>(a, v, v, tok, lane, out);
    }
}

// One wave per row: a row has wpr * 8 partials (64 for a 128256-entry row),
// so the merge needs no barrier.
constexpr int kMergeThreads = 64;

__global__ __launch_bounds__(kMergeThreads) void expand_merge_kernel(ExArgs a)
{
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    const int np = a.wpr * kExWaves;
    const ExPart *p = a.part + r * np;
    // the row maximum and any NaN
    uint64_t mk = 0;
    bool nan_seen = false;
    for (int w = lane; w < np; w += kMergeThreads) {
        // the largest key's value is the largest logit unless the keys are
        // sampling keys; then the partials' own maxima
        mk = max_u64(mk, a.sampled ? (p[w].m == -INFINITY ? 0ull
                                                          : (uint64_t)ordered_bits(p[w].m) << 32)
                                   : p[w].key[0]);
        nan_seen |= p[w].nan != 0;
    }
    const uint64_t top = wave_max_key(mk);
    const bool any_nan = __any(nan_seen);
    const float M = top == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(top >> 32));
    if (any_nan || !__builtin_isfinite(M)) {
        if (lane == 0)
            raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
        for (int i = lane; i < a.k; i += kMergeThreads) {
            a.top_token[r * a.k + i] = -1;
            a.top_logq[r * a.k + i] = NAN;
        }
        if (lane == 0)
            a.entropy[r] = NAN;
        return;
    }
    // partial sums rebased to the row maximum
    const double Ms = (double)(M * a.invT32);
    double s0 = 0.0, s1 = 0.0;
    for (int w = lane; w < np; w += kMergeThreads) {
        if (p[w].m == -INFINITY)
            continue;
        const double d = (double)(p[w].m * a.invT32) - Ms;   // <= 0
        const double e = exp(d);
        s0 += e * p[w].s0;
        s1 += e * (p[w].s1 + d * p[w].s0);
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    const double logS0 = log(s0);
    // the k best keys among every wave's k candidates: round i takes the
    // largest key below round i-1's (keys are unique: they carry the token)
    const int ncand = np * a.k;
    uint64_t prev = ~0ull;
    for (int i = 0; i < a.k; ++i) {
        uint64_t best = 0;
        for (int c = lane; c < ncand; c += kMergeThreads) {
            const uint64_t kk = p[c / a.k].key[c % a.k];
            if (kk < prev)
                best = max_u64(best, kk);
        }
        const uint64_t win = wave_max_key(best);
        prev = win;
        if (lane == 0) {
            const int32_t t = win == 0ull ? -1 : (int32_t)(0xFFFFFFFFu - (uint32_t)win);
            const float x = a.sampled ? (t < 0 ? -INFINITY : a.x[r * a.V + t])
                                      : from_ordered_bits((uint32_t)(win >> 32));
            a.top_token[r * a.k + i] = t;
            a.top_logq[r * a.k + i] =
                win == 0ull ? -INFINITY : (double)fmaf(x, a.invT32, -(float)Ms) - logS0;
        }
    }
    if (lane == 0)
        a.entropy[r] = logS0 - s1 / s0;
}

bool ex_plan(int32_t V, int32_t &wpr)
{
    wpr = (int32_t)ceil_div(V, kExChunk);
    return wpr <= kExMaxWpr;
}

} // namespace
} // namespace tav

extern "C" size_t tree_expand_workspace_bytes(int64_t R, int32_t V, int32_t k)
{
    using namespace tav;
    int32_t wpr = 0;
    if (R < 1 || V < 1 || k < 1 || k > kExMaxK || k > V || !ex_plan(V, wpr))
        return 0;
    return (size_t)R * wpr * kExWaves * sizeof(ExPart);
}

namespace {

tav_status ex_launch(const float *draft_logits, int64_t R, int32_t V, int32_t k,
                     double temperature, bool sampled, uint64_t seed, uint64_t offset,
                     int32_t *top_token, double *top_logq, double *entropy, void *workspace,
                     size_t ws_bytes, uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!draft_logits || !top_token || !top_logq || !entropy)
        return TAV_ERR_ARG;
    if (R < 1 || V < 1 || k < 1 || k > V || !(temperature > 0.0) || !(temperature < INFINITY))
        return TAV_ERR_ARG;
    int32_t wpr = 0;
    if (k > kExMaxK || !ex_plan(V, wpr) || R * wpr > (int64_t)INT32_MAX)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(draft_logits, 4) || !aligned(top_logq, 8) || !aligned(entropy, 8))
        return TAV_ERR_ARG;
    const size_t need = (size_t)R * wpr * kExWaves * sizeof(ExPart);
    if (!workspace || ws_bytes < need || !aligned(workspace, 16))
        return TAV_ERR_WORKSPACE;
    ExArgs a;
    a.x = draft_logits;
    a.R = R;
    a.V = V;
    a.k = k;
    a.wpr = wpr;
    a.vec4 = V % 4 == 0 && aligned(draft_logits, 16);
    a.invT = 1.0 / temperature;
    a.invT32 = (float)a.invT;
    a.part = static_cast<ExPart *>(workspace);
    a.top_token = top_token;
    a.top_logq = top_logq;
    a.entropy = entropy;
    a.flags = dev_flags;
    a.sampled = sampled ? 1 : 0;
    a.seed = seed;
    a.offset = offset;
    hipStream_t s = as_stream(stream);
    if (sampled)
        hipLaunchKernelGGL(expand_part_kernel<true>, dim3((unsigned)(R * wpr)), dim3(kExThreads), 0,
                           s, a);
    else
        hipLaunchKernelGGL(expand_part_kernel<false>, dim3((unsigned)(R * wpr)), dim3(kExThreads),
                           0, s, a);
    if (hipGetLastError() != hipSuccess)
        return TAV_ERR_LAUNCH;
    hipLaunchKernelGGL(expand_merge_kernel, dim3((unsigned)R), dim3(kMergeThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}

} // namespace

extern "C" tav_status tree_expand_topk(const float *draft_logits, int64_t R, int32_t V, int32_t k,
                                       double temperature, int32_t *top_token, double *top_logq,
                                       double *entropy, void *workspace, size_t ws_bytes,
                                       uint32_t *dev_flags, void *stream)
{
    return ex_launch(draft_logits, R, V, k, temperature, false, 0, 0, top_token, top_logq,
                     entropy, workspace, ws_bytes, dev_flags, stream);
}

extern "C" tav_status tree_expand_sample(const float *draft_logits, int64_t R, int32_t V,
                                         int32_t k, double temperature, uint64_t seed,
                                         uint64_t offset, int32_t *top_token, double *top_logq,
                                         double *entropy, void *workspace, size_t ws_bytes,
                                         uint32_t *dev_flags, void *stream)
{
    return ex_launch(draft_logits, R, V, k, temperature, true, seed, offset, top_token, top_logq,
                     entropy, workspace, ws_bytes, dev_flags, stream);
}
