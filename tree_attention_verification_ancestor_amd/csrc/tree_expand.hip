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

// No implicit contraction of a * b + c into one fused operation in this
// file: the exponents below rely on the product being rounded on its own
// (every fused multiply-add that is wanted is written as fmaf).
#pragma clang fp contract(off)

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

// x * y rounded to fp32 on its own
__device__ __forceinline__ float mul_rn(float x, float y) { return x * y; }

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

struct ExSPart;

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
    // sampled expansion
    uint64_t seed, offset;
    uint64_t K;          // SplitMix64 key of the call (word 0 of Philox at (offset, 0, 0, 3))
    double T;            // temperature, as given
    ExSPart *spart;      // [R][wpr * kExWaves]
};

// S0 = sum e^y and S1 = sum y e^y over a wave's entries v, y = (x - m)/T
// (m the wave's maximum logit, -inf when it holds none), y formed as
// fl(x fl(1/T)) - fl(m fl(1/T)): never above 0, exactly 0 at the maximum
// (a fused multiply-add would leave the product's rounding error there,
// which overflows e^y for huge logits). Each run of four
// entries is summed in fp32 (same-sign terms, so within three fp32 roundings
// of exact), the run totals in fp64.
template <bool kClean>
__device__ __forceinline__ void wave_sums(const ExArgs &a, const float (&v)[kExEpt], float m,
                                          double &s0, double &s1)
{
    const float ms = mul_rn(m, a.invT32);
    s0 = 0.0;
    s1 = 0.0;
    if (m != -INFINITY) {
#pragma unroll
        for (int h = 0; h < kExEpt / 4; ++h) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = v[4 * h + j];
                const float y = mul_rn(x, a.invT32) - ms;   // <= 0: fl(x/T) <= fl(m/T)
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
}

// One wave's partial of a row from its entries v (lane order: tokens rise
// with e). kClean: every entry is in the row and none is NaN, so the
// per-entry tests drop out.
template <bool kClean, typename Tok>
__device__ __forceinline__ void wave_partial(const ExArgs &a, const float (&v)[kExEpt], Tok tok,
                                             int lane, ExPart *out)
{
    const float (&sk)[kExEpt] = v;   // the values the k best are chosen by
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
    // entry), which is the best key's value
    const float m = first == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(first >> 32));
    double s0, s1;
    wave_sums<kClean>(a, v, m, s0, s1);
    const bool wnan = __any(nan_seen);
    if (lane == 0) {
        out->s0 = s0;
        out->s1 = s1;
        out->m = m;
        out->nan = wnan;
    }
}

// A wave's share of a row: lane l holds entries wbase + 64 RUN h + RUN l + j
// (h < kExEpt / RUN, j < RUN), read 16 bytes at a time, so a lane's entries
// rise in token order and each run of RUN tokens is consecutive. Entries past
// the row read as NaN (not an entry). `clean`: the share lies wholly inside
// the row and holds no NaN (one NaN-propagating maximum tells), so the
// passes over it may skip the per-entry range and NaN tests.
template <int RUN>
__device__ __forceinline__ void load_share(const ExArgs &a, const float *row, int64_t wbase,
                                           int lane, float (&v)[kExEpt], bool &clean)
{
    static_assert(RUN % 4 == 0 && kExEpt % RUN == 0, "runs of whole 16-byte loads");
    const int64_t lim = a.V;
    const bool full = a.vec4 && wbase + kExWaveChunk <= lim;   // wave-uniform
#pragma unroll
    for (int h = 0; h < kExEpt / RUN; ++h) {
#pragma unroll
        for (int q4 = 0; q4 < RUN / 4; ++q4) {
            const int64_t i0 = wbase + (int64_t)h * 64 * RUN + RUN * lane + 4 * q4;
            const int e0 = RUN * h + 4 * q4;
            if (full || (a.vec4 && i0 + 3 < lim)) {
                const f32x4 q = *reinterpret_cast<const f32x4 *>(row + i0);
                v[e0] = q.x;
                v[e0 + 1] = q.y;
                v[e0 + 2] = q.z;
                v[e0 + 3] = q.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[e0 + j] = i0 + j < lim ? row[i0 + j] : NAN;   // NaN: not an entry
            }
        }
    }
    clean = false;
    if (full) {
        float mx = v[0];
#pragma unroll
        for (int e = 1; e < kExEpt; ++e)
            mx = __builtin_elementwise_maximum(mx, v[e]);   // NaN-propagating
        clean = !__any(__builtin_isnan(mx));
    }
}

__global__ __launch_bounds__(kExThreads) void expand_part_kernel(ExArgs a)
{
    // Each wave owns kExWaveChunk consecutive entries of one row, in runs of
    // four tokens per lane. No barrier: every wave writes its own partial.
    const int64_t r = blockIdx.x / a.wpr;
    const int w = (int)(blockIdx.x % a.wpr);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *row = a.x + r * a.V;
    const int64_t wbase = (int64_t)w * kExChunk + (int64_t)wave * kExWaveChunk;
    float v[kExEpt];
    bool clean;
    load_share<4>(a, row, wbase, lane, v, clean);
    auto tok = [&](int e) __attribute__((always_inline)) {
        return wbase + (int64_t)(e >> 2) * 256 + 4 * lane + (e & 3);
    };
    ExPart *out = a.part + (r * a.wpr + w) * kExWaves + wave;
    if (clean)
        wave_partial<true>(a, v, tok, lane, out);
    else
        wave_partial<false>(a, v, tok, lane, out);
}

// One wave per row: a row has wpr * 8 partials (64 for a 128256-entry row),
// so the merge needs no barrier.
constexpr int kMergeThreads = 64;

// The row's maximum logit M (from the waves' maxima), any NaN, and log S0
// and S1 / S0 with the waves' sums rebased to M. false: the row has a NaN or
// no finite maximum (flag raised, outputs written as missing).
template <typename Part>
__device__ __forceinline__ bool row_stats(const ExArgs &a, const Part *p, int np, int64_t r,
                                          int lane, double &Ms, double &logS0, double &ratio)
{
    float M = -INFINITY;
    bool nan_seen = false;
    for (int w = lane; w < np; w += kMergeThreads) {
        M = fmaxf(M, p[w].m);
        nan_seen |= p[w].nan != 0;
    }
    const uint64_t top = wave_max_key(M == -INFINITY ? 0ull : (uint64_t)ordered_bits(M) << 32);
    M = top == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(top >> 32));
    if (__any(nan_seen) || !__builtin_isfinite(M)) {
        if (lane == 0)
            raise_flag(a.flags, TAV_FLAG_NONFINITE_LOGITS);
        for (int i = lane; i < a.k; i += kMergeThreads) {
            a.top_token[r * a.k + i] = -1;
            a.top_logq[r * a.k + i] = NAN;
        }
        if (lane == 0)
            a.entropy[r] = NAN;
        return false;
    }
    Ms = (double)mul_rn(M, a.invT32);
    double s0 = 0.0, s1 = 0.0;
    for (int w = lane; w < np; w += kMergeThreads) {
        if (p[w].m == -INFINITY)
            continue;
        const double d = (double)mul_rn(p[w].m, a.invT32) - Ms;   // <= 0
        const double e = exp(d);
        s0 += e * p[w].s0;
        s1 += e * (p[w].s1 + d * p[w].s0);
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    logS0 = log(s0);
    ratio = s1 / s0;
    return true;
}

__global__ __launch_bounds__(kMergeThreads) void expand_merge_kernel(ExArgs a)
{
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    const int np = a.wpr * kExWaves;
    const ExPart *p = a.part + r * np;
    double Ms, logS0, ratio;
    if (!row_stats(a, p, np, r, lane, Ms, logS0, ratio))
        return;
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
            const float x = from_ordered_bits((uint32_t)(win >> 32));
            a.top_token[r * a.k + i] = t;
            a.top_logq[r * a.k + i] =
                win == 0ull ? -INFINITY : ((double)mul_rn(x, a.invT32) - Ms) - logS0;
        }
    }
    if (lane == 0)
        a.entropy[r] = logS0 - ratio;
}

// ---------------------------------------------------------------------------
// Sampled expansion: the k largest keys x/T + G(u) of a row (Gumbel top-k),
// each key in fp64 exactly as defined, u = fl64(m + 1/2) 2^-53 with
// m = hi 2^21 + lo. hi, the 32 high bits, comes from SplitMix64 (Steele, Lea
// and Flood, OOPSLA 2014; two tokens per output); lo, the 21 low bits, from
// Philox4x64-10 (eight tokens per block). Almost every token is ruled out by
// its high word alone:
//   part kernel  each token's key lies in an fp32 interval [L, U] computed
//                from y = x fl(1/T) and hi; tau, the k-th largest of the
//                lanes' best L, is a lower bound on the wave's k-th key, so
//                only tokens with U >= tau can be among its k best. Those
//                contenders (typically k: the intervals are ~1e-4 wide) go to
//                the merge with their intervals. If more than kSpKC contend,
//                the wave resolves them itself with exact keys and sends its
//                exact k best.
//   merge        the row's contenders are cut the same way against the k-th
//                largest L of the row, the survivors get their low bits and
//                exact fp64 keys, and the k best are taken by key, the lower
//                token first among equal keys.
// Tokens with logit -inf have key -inf whatever u is; a wave with fewer than
// k finite tokens also sends its lowest -inf tokens, exact.

constexpr int kSpKC = 32;                     // contenders a wave sends
constexpr uint64_t kSmGamma = 0x9E3779B97F4A7C15ull;
constexpr float kLn2F = 0x1.62e430p-1f;

struct SpCand {
    int32_t tok;
    uint32_t hi;     // high word of the token's uniform
    float lo, up;    // interval holding its key (equal to it when `exact`)
    double key;      // the exact key, when `exact`
    int32_t exact;
    int32_t pad_;
};

struct ExSPart {     // one wave's share of a row
    double s0, s1;
    float m;
    int32_t nan;
    int32_t n;       // contenders in c[]
    int32_t pad_;
    SpCand c[kSpKC];
};

__device__ __forceinline__ uint64_t splitmix_out(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// An fp32 interval [lo, up] holding the key x/T + G(u) (fp64, exact as
// defined) of a token with y = x fl32(1/T) (finite) and high word hi, over
// every u its 21 unknown low bits allow: u lies in [hi, hi + 1] 2^-32.
// G = -log E, E = -log u, is evaluated in fp32 at the interval's midpoint:
// for u >= 1/2 from d = 1 - u (a series below 2^-9, else log2(1 - d)), for
// u < 1/2 from u itself, so E keeps ~2^-15 relative accuracy. Over the
// interval G moves by at most 2 / min(c - 1, hi) (c = 2^32 - hi): G'(d) <=
// 2/d for d <= 1/2 and <= 1.45/u for u < 1/2. Unbounded when hi is 0 or all
// ones (u can reach 0 or 1). `pad` covers the fp32 rounding of y, E, G and
// the sums with a wide margin (2^-12 plus 2^-19 of |y| + |G|).
__device__ __forceinline__ void key_bounds(float y, uint32_t hi, float &lo, float &up)
{
    const uint32_t cm1 = ~hi;   // c - 1
    float E;
    if (hi >= 0x80000000u) {
        const float d = ((float)cm1 + 0.5f) * 0x1p-32f;
        const float series = d * fmaf(d, fmaf(d, fmaf(d, 0.25f, 0x1.555556p-2f), 0.5f), 1.0f);
        const float viaLog = -__builtin_amdgcn_logf(1.0f - d) * kLn2F;
        E = d < 0x1p-9f ? series : viaLog;
    } else {
        const float um = ((float)hi + 0.5f) * 0x1p-32f;
        E = -__builtin_amdgcn_logf(um) * kLn2F;
    }
    const float G = -__builtin_amdgcn_logf(E) * kLn2F;
    const uint32_t mn = cm1 < hi ? cm1 : hi;
    const float wdt = mn == 0u ? INFINITY : 2.0f * __builtin_amdgcn_rcpf((float)mn);
    const float A = y + G;
    const float pad = 0x1p-12f + (fabsf(y) + fabsf(G)) * 0x1p-19f;
    lo = A - (wdt + pad);
    up = A + (wdt + pad);
}

// The exact key of token t of row r (logit x, high word hi): the low bits
// from Philox, then x/T + G(u) in fp64 as defined.
__device__ __forceinline__ double exact_key(const ExArgs &a, int64_t r, int64_t t, uint32_t hi,
                                            float x)
{
    if (x == -INFINITY)
        return -INFINITY;
    uint64_t w[4];
    philox4x64_10(a.offset, (uint64_t)r, (uint64_t)(t >> 3), 2, a.seed, 0, w);
    const int j = (int)(t & 7);
    const uint64_t word = w[j & 3];
    const uint32_t half = j < 4 ? (uint32_t)(word >> 32) : (uint32_t)word;
    const uint64_t m = ((uint64_t)hi << 21) | (half >> 11);
    const double u = ((double)m + 0.5) * 0x1p-53;
    const double g = -log(-log(u));
    return (double)x / a.T + g;
}

// Order-preserving image of a double that is not NaN (-0 as +0); never 0.
__device__ __forceinline__ uint64_t ordered64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v == 0.0 ? 0.0 : v);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double from_ordered64(uint64_t o)
{
    return __builtin_bit_cast(double, (o >> 63) ? (o & 0x7FFFFFFFFFFFFFFFull) : ~o);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    auto dpp = [](uint32_t x, auto ctrl) __attribute__((always_inline)) {
        constexpr int C = decltype(ctrl)::value;
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, C, 0xF, 0xF, false);
    };
    v = max(v, dpp(v, std::integral_constant<int, kQuadSwap1>{}));
    v = max(v, dpp(v, std::integral_constant<int, kQuadSwap2>{}));
    v = max(v, dpp(v, std::integral_constant<int, kRowHalfMirror>{}));
    v = max(v, dpp(v, std::integral_constant<int, kRowMirror>{}));
    auto rl = [](uint32_t x, int l) __attribute__((always_inline)) {
        return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
    };
    return max(max(rl(v, 0), rl(v, 16)), max(rl(v, 32), rl(v, 48)));
}

// The wave's best of the lanes' offers (ordered key, token; key 0 = none):
// the largest key, the lowest token among equal keys. Returns the key (0 if
// no lane offers) and sets tok; `mine`: this lane's offer won.
__device__ __forceinline__ uint64_t wave_best(uint64_t okey, int32_t otok, int32_t &tok, bool &mine)
{
    const uint64_t wk = wave_max_key(okey);
    const uint32_t nt = wave_max_u32(okey == wk && wk != 0ull ? ~(uint32_t)otok : 0u);
    tok = (int32_t)~nt;
    mine = wk != 0ull && okey == wk && otok == tok;
    return wk;
}

// Running k best (exact key, token) of a stream of batches, lane i < k
// holding the i-th: one batch entry per lane (valid or not) is merged in by
// k rounds of a wave-wide best.
struct TopRun {
    uint64_t key = 0;   // ordered key; 0: none
    int32_t tok = -1;
};

__device__ __forceinline__ void top_merge(int k, int lane, uint64_t bkey, int32_t btok, TopRun &run)
{
    bool run_taken = false, b_taken = false;
    TopRun next;
    for (int i = 0; i < k; ++i) {
        const bool hr = run.key != 0ull && !run_taken, hb = bkey != 0ull && !b_taken;
        const bool pick_r = hr && (!hb || run.key > bkey || (run.key == bkey && run.tok < btok));
        const uint64_t ok = pick_r ? run.key : (hb ? bkey : 0ull);
        const int32_t ot = pick_r ? run.tok : btok;
        int32_t wt;
        bool mine;
        const uint64_t wk = wave_best(ok, ot, wt, mine);
        if (wk == 0ull)
            break;
        if (mine) {
            if (pick_r)
                run_taken = true;
            else
                b_taken = true;
        }
        if (lane == i) {
            next.key = wk;
            next.tok = wt;
        }
    }
    run = next;
}

// LDS staging of one wave's batch of contenders (64 at a time).
struct SpBatch {
    int32_t tok[64];
    uint32_t hi[64];
    float x[64];
};

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum over the wave's lanes, and the total.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int &total)
{
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o)
            incl += y;
    }
    total = __shfl(incl, 63);
    return incl - v;
}

// One wave's share of a sampled expansion. Entries past the row were loaded
// as NaN, so "live" (a finite or +inf logit: not NaN, not -inf) needs no
// range test; only the NaN flag looks at the range.
// kClean: every entry of the wave is in the row and none is NaN (as
// load_share found), so the maxima need no range or NaN test.
template <bool kClean>
__device__ __forceinline__ void sample_wave(const ExArgs &a, const float (&v)[kExEpt], int64_t r,
                                            int32_t wbase, int lane, ExSPart *out, SpBatch *lds)
{
    // token of entry e: runs of eight per lane (tokens fit 32 bits: V <= 2^21)
    auto tok = [&](int e) __attribute__((always_inline)) {
        return wbase + (e >> 3) * 512 + 8 * lane + (e & 7);
    };
    const int32_t lim = a.V;
    // high word of token t: SplitMix64 output r 2^20 + t/2 + 1 of the call's
    // key, its high half for even t, its low half for odd t
    const uint64_t rbase = a.K + kSmGamma * (((uint64_t)r << 20) + 1ull);
    auto high_word = [&](int32_t t) __attribute__((always_inline)) {
        const uint64_t z = splitmix_out(rbase + kSmGamma * (uint64_t)(t >> 1));
        return (t & 1) ? (uint32_t)z : (uint32_t)(z >> 32);
    };
    bool nan_seen = false;
    float lmax = -INFINITY, amax = 0.0f;
#pragma unroll
    for (int e = 0; e < kExEpt; ++e) {
        if constexpr (kClean) {
            lmax = fmaxf(lmax, v[e]);
            amax = fmaxf(amax, v[e] != -INFINITY ? fabsf(v[e]) : 0.0f);
        } else {
            nan_seen |= tok(e) < lim && __builtin_isnan(v[e]);
            if (!__builtin_isnan(v[e])) {
                lmax = fmaxf(lmax, v[e]);
                if (v[e] != -INFINITY)
                    amax = fmaxf(amax, fabsf(v[e]));
            }
        }
    }
    const uint64_t mkey = wave_max_key(lmax == -INFINITY ? 0ull : (uint64_t)ordered_bits(lmax) << 32);
    // the largest |x / T| of a finite logit of the wave (for rounding margins)
    const float ymax = from_ordered_bits((uint32_t)(wave_max_key((uint64_t)ordered_bits(amax) << 32) >> 32)) *
                       a.invT32 * (1.0f + 0x1p-20f);
    const float m = mkey == 0ull ? -INFINITY : from_ordered_bits((uint32_t)(mkey >> 32));
    const bool wnan = __any(nan_seen);

    // Pass 1 over the registers: the sums (as wave_sums forms them: each run
    // of four entries in fp32, the run totals in fp64) and, per token, one
    // number for pass 2 (SplitMix64 gives two tokens' high words per output):
    //   sc = e^y / (c - 1)  for u >= 1/2 (hi >= 2^31; c = 2^32 - hi), +inf if
    //                       c = 1 (u may reach 1);
    //   sc = -1             for u < 1/2;
    //   sc = -1/2           for a token that is not live (past the row, NaN
    //                       or -inf logit).
    // e^y / (1 - u) is about e^(key - ms) for u near 1, so each lane's
    // largest sc also picks its likeliest token (a choice only: any token's
    // lower bound serves below). The pick is one integer maximum per token
    // over sc's bits as a signed integer (ordered like sc for sc >= 0, then
    // -1, then -1/2) with the low five bits replaced by 31 - e: the first
    // entry among (nearly) equal values.
    const float ms = mul_rn(m, a.invT32);
    double s0 = 0.0, s1 = 0.0;
    float sc[kExEpt];
    int32_t pick = INT32_MIN;
    int finite = 0;   // live tokens of the wave (wave-uniform)
#pragma unroll
    for (int h = 0; h < kExEpt / 8; ++h) {
        const uint64_t sbase = rbase + kSmGamma * (uint64_t)(tok(8 * h) >> 1);
        uint32_t hw[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint64_t z = splitmix_out(sbase + kSmGamma * (uint64_t)q);
            hw[2 * q] = (uint32_t)(z >> 32);
            hw[2 * q + 1] = (uint32_t)z;
        }
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 8 * h + 4 * q4 + j;
                const float x = v[e];
                const float y = mul_rn(x, a.invT32) - ms;
                const float ev = __builtin_amdgcn_exp2f(y * 0x1.715476p+0f);
                const bool live = x > -INFINITY;   // not NaN, not -inf
                r0 += live ? ev : 0.f;
                r1 = live ? fmaf(y, ev, r1) : r1;
                const uint32_t hi = hw[4 * q4 + j];
                const uint32_t cm1 = ~hi;
                const float ratio = cm1 == 0u ? INFINITY : ev * __builtin_amdgcn_rcpf((float)cm1);
                const float t = live ? (hi >= 0x80000000u ? ratio : -1.0f) : -0.5f;
                sc[e] = t;
                pick = max(pick, (int32_t)((__builtin_bit_cast(uint32_t, t) & ~31u) | (uint32_t)(31 - e)));
                finite += __builtin_popcountll(__ballot(live));
            }
            if (m != -INFINITY) {
                s0 += (double)r0;
                s1 += (double)r1;
            }
        }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    const float *row = a.x + r * a.V;
    auto entry_token = [&](int e) __attribute__((always_inline)) {
        return wbase + (e >> 3) * 512 + 8 * lane + (e & 7);
    };
    // the lane's chosen token's lower bound (none if all its tokens are dead)
    static_assert(kExEpt <= 32, "entry index in five bits");
    const int ebest =
        ((uint32_t)pick >> 5) == (__builtin_bit_cast(uint32_t, -0.5f) >> 5) ? -1 : 31 - (pick & 31);
    float lbest = -INFINITY;
    if (ebest >= 0) {
        const int32_t t = entry_token(ebest);
        float lo, u;
        key_bounds(row[t] * a.invT32, high_word(t), lo, u);
        lbest = lo;
    }
    const int nfin = finite;
    // tau: the k-th largest of the lanes' lower bounds (k rounds of a wave
    // maximum; one lane holding the maximum drops out each round), at most
    // the wave's k-th key
    float tau = -INFINITY;
    {
        uint32_t offer = lbest == -INFINITY ? 0u : ordered_bits(lbest);
        for (int i = 0; i < a.k; ++i) {
            const uint32_t win = wave_max_u32(offer);
            if (win == 0u) {
                tau = -INFINITY;
                break;
            }
            const uint64_t holders = __ballot(offer == win);
            if (lane == (int)__builtin_ctzll(holders))
                offer = 0u;
            tau = from_ordered_bits(win);
        }
    }
    // Pass 2: a necessary condition for key >= tau, one comparison per token.
    // u >= 1/2: G(u) <= -log(1 - u) <= 32 ln 2 - ln(c - 1), so key >= tau
    // needs e^(x/T - ms) / (c - 1) >= e^-(ms - tau + 32 ln 2): sc against
    // thr1, the exponent widened by 2^-8 plus 2^-18 of the magnitudes
    // involved for the fp32 roundings of y, e^y, 1/(c - 1) and thr1 itself.
    // Where e^y underflows (y < -87) sc is 0, which is safe while tau is
    // within 64 of ms (such a key is below ms - 65); otherwise every such
    // token passes (thr1 = 0). u < 1/2: G <= 0.3666, so key >= tau needs
    // fl(x/T) >= thr2.
    const bool far = !(tau >= ms - 64.0f);
    const float thr1 = far ? 0.0f
                           : __builtin_amdgcn_exp2f(-(ms - tau + 22.180710f + 0x1p-8f +
                                                      (ymax + fabsf(ms) + fabsf(tau)) * 0x1p-18f) *
                                                    0x1.715476p+0f);
    const float thr2 = tau - (0.36652f + 0x1p-8f + ymax * 0x1p-20f);
    uint32_t cand = 0;
#pragma unroll
    for (int e = 0; e < kExEpt; ++e) {
        const bool pass = sc[e] >= thr1 || (sc[e] == -1.0f && mul_rn(v[e], a.invT32) >= thr2);
        cand |= pass ? 1u << e : 0u;
    }
    // exact intervals of the survivors: keep those whose top reaches tau
    {
        uint32_t c = cand;
        while (c) {
            const int e = __builtin_ctz(c);
            c &= c - 1;
            const int32_t t = entry_token(e);
            float lo, u;
            key_bounds(row[t] * a.invT32, high_word(t), lo, u);
            if (!(u >= tau))
                cand &= ~(1u << e);
        }
    }
    int total;
    const int base = wave_excl_scan(__builtin_popcount(cand), lane, total);
    if (lane == 0) {
        out->s0 = s0;
        out->s1 = s1;
        out->m = m;
        out->nan = wnan;
    }
    int n_out = 0;
    if (total <= kSpKC) {
        // send the contenders with their intervals
        uint32_t c = cand;
        int slot = base;
        while (c) {
            const int e = __builtin_ctz(c);
            c &= c - 1;
            const int32_t t = entry_token(e);
            const uint32_t hw = high_word(t);
            float lo, u;
            key_bounds(row[t] * a.invT32, hw, lo, u);
            SpCand &o = out->c[slot++];
            o.tok = t;
            o.hi = hw;
            o.lo = lo;
            o.up = u;
            o.key = 0.0;
            o.exact = 0;
        }
        n_out = total;
    } else {
        // too many contenders: resolve them here, 64 at a time, with exact keys
        TopRun run;
        for (int b0 = 0; b0 < total; b0 += 64) {
            uint32_t c = cand;
            int idx = base;
            while (c) {
                const int e = __builtin_ctz(c);
                c &= c - 1;
                if (idx >= b0 && idx < b0 + 64) {
                    const int32_t t = entry_token(e);
                    lds->tok[idx - b0] = t;
                    lds->hi[idx - b0] = high_word(t);
                    lds->x[idx - b0] = row[t];
                }
                ++idx;
            }
            wave_lds_sync();
            uint64_t bk = 0ull;
            int32_t bt = -1;
            if (b0 + lane < total) {
                bt = lds->tok[lane];
                bk = ordered64(exact_key(a, r, bt, lds->hi[lane], lds->x[lane]));
            }
            wave_lds_sync();
            top_merge(a.k, lane, bk, bt, run);
        }
        n_out = min(a.k, total);
        if (lane < n_out) {
            const double key = from_ordered64(run.key);
            SpCand &o = out->c[lane];
            o.tok = run.tok;
            o.hi = 0u;
            o.key = key;
            o.exact = 1;
            // an fp32 interval holding the key (its nearest float is within
            // half an ulp), for the merge's cut
            const float kf = (float)key;
            const float slack = fabsf(kf) * 0x1p-22f + 0x1p-126f;
            o.lo = __builtin_isinf(kf) ? kf : kf - slack;
            o.up = __builtin_isinf(kf) ? kf : kf + slack;
        }
    }
    // fewer than k finite tokens: the wave's lowest -inf tokens, exact
    if (nfin < a.k) {
        const int need = a.k - nfin;
        uint32_t taken = 0;
        for (int i = 0; i < need; ++i) {
            int32_t best = 0x7FFFFFFF;
            int be = -1;
#pragma unroll
            for (int e = 0; e < kExEpt; ++e) {
                const bool ninf = tok(e) < lim && row[tok(e)] == -INFINITY && !((taken >> e) & 1u);
                if (ninf && tok(e) < best) {
                    best = tok(e);
                    be = e;
                }
            }
            const uint32_t win = wave_max_u32(be >= 0 ? ~(uint32_t)best : 0u);
            if (win == 0u)
                break;
            const int32_t wt = (int32_t)~win;
            if (be >= 0 && best == wt)
                taken |= 1u << be;
            if (lane == 0 && n_out < kSpKC) {
                SpCand &o = out->c[n_out];
                o.tok = wt;
                o.hi = 0u;
                o.key = -INFINITY;
                o.exact = 1;
                o.lo = -INFINITY;
                o.up = -INFINITY;
            }
            ++n_out;
        }
    }
    if (lane == 0)
        out->n = min(n_out, kSpKC);
}

__global__ __launch_bounds__(kExThreads) __attribute__((amdgpu_waves_per_eu(4))) void expand_sample_part_kernel(ExArgs a)
{
    __shared__ SpBatch s_batch[kExWaves];
    const int64_t r = blockIdx.x / a.wpr;
    const int w = (int)(blockIdx.x % a.wpr);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *row = a.x + r * a.V;
    const int32_t wbase = w * kExChunk + wave * kExWaveChunk;
    float v[kExEpt];
    bool clean;
    load_share<8>(a, row, wbase, lane, v, clean);
    ExSPart *out = a.spart + (r * a.wpr + w) * kExWaves + wave;
    if (clean)
        sample_wave<true>(a, v, r, wbase, lane, out, &s_batch[wave]);
    else
        sample_wave<false>(a, v, r, wbase, lane, out, &s_batch[wave]);
}

__global__ __launch_bounds__(kMergeThreads) void expand_sample_merge_kernel(ExArgs a)
{
    __shared__ SpBatch s_batch;
    __shared__ double s_key[64];
    __shared__ int32_t s_exact[64];
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    const int np = a.wpr * kExWaves;
    const ExSPart *p = a.spart + r * np;
    // The first kMergeRegs contenders of partial `lane` (token, interval) are
    // read once into registers; the selection rounds below scan them there.
    // Contenders past those, and partials lane + 64, ..., are read where
    // they are used.
    constexpr int kMergeRegs = 8;
    int32_t rtok[kMergeRegs];
    float rlo[kMergeRegs], rup[kMergeRegs];
    const int n0 = lane < np ? p[lane].n : 0;
#pragma unroll
    for (int i = 0; i < kMergeRegs; ++i) {
        rtok[i] = 0;
        rlo[i] = rup[i] = -INFINITY;
        if (i < n0) {
            const SpCand &c = p[lane].c[i];
            rtok[i] = c.tok;
            rlo[i] = c.lo;
            rup[i] = c.up;
        }
    }
    double Ms, logS0, ratio;
    if (!row_stats(a, p, np, r, lane, Ms, logS0, ratio))
        return;
    // fn(w, i, lo, up, tok) for every contender i of partials lane, lane + 64, ...
    auto for_each = [&](auto &&fn) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kMergeRegs; ++i)
            if (i < n0)
                fn(lane, i, rlo[i], rup[i], rtok[i]);
        for (int i = kMergeRegs; i < n0; ++i) {
            const SpCand &c = p[lane].c[i];
            fn(lane, i, c.lo, c.up, c.tok);
        }
        for (int w = lane + kMergeThreads; w < np; w += kMergeThreads) {
            const int n = p[w].n;
            for (int i = 0; i < n; ++i) {
                const SpCand &c = p[w].c[i];
                fn(w, i, c.lo, c.up, c.tok);
            }
        }
    };
    // the row's k-th largest lower bound: k rounds of "each lane offers its
    // best not yet taken"
    float tau = -INFINITY;
    {
        float prev_v = INFINITY;
        int32_t prev_t = -1;
        for (int i = 0; i < a.k; ++i) {
            // the best (lo, token) below the previous winner in that order
            float bv = -INFINITY;
            int32_t bt = 0x7FFFFFFF;
            bool any = false;
            for_each([&](int, int, float lo, float, int32_t tok) __attribute__((always_inline)) {
                const bool below = lo < prev_v || (lo == prev_v && tok > prev_t);
                if (below && (!any || lo > bv || (lo == bv && tok < bt))) {
                    bv = lo;
                    bt = tok;
                    any = true;
                }
            });
            int32_t wt;
            bool mine;
            const uint64_t wk = wave_best(any ? make_key(bv, 0) : 0ull, any ? bt : 0, wt, mine);
            if (wk == 0ull) {
                tau = -INFINITY;
                break;
            }
            prev_v = from_ordered_bits((uint32_t)(wk >> 32));
            prev_t = wt;
            tau = prev_v;
        }
    }
    // survivors: up >= tau; exact keys 64 at a time, k best kept
    int cnt = 0;
    for_each([&](int, int, float, float up, int32_t) __attribute__((always_inline)) {
        cnt += up >= tau ? 1 : 0;
    });
    int total;
    const int base = wave_excl_scan(cnt, lane, total);
    TopRun run;
    for (int b0 = 0; b0 < total; b0 += 64) {
        int idx = base;
        for_each([&](int w, int i, float, float up, int32_t tok) __attribute__((always_inline)) {
            if (up >= tau) {
                if (idx >= b0 && idx < b0 + 64) {
                    const SpCand &c = p[w].c[i];
                    s_batch.tok[idx - b0] = tok;
                    s_batch.hi[idx - b0] = c.hi;
                    s_key[idx - b0] = c.key;
                    s_exact[idx - b0] = c.exact;
                }
                ++idx;
            }
        });
        wave_lds_sync();
        uint64_t bk = 0ull;
        int32_t bt = -1;
        if (b0 + lane < total) {
            bt = s_batch.tok[lane];
            const double key = s_exact[lane] ? s_key[lane]
                                             : exact_key(a, r, bt, s_batch.hi[lane], a.x[r * a.V + bt]);
            bk = ordered64(key);
        }
        wave_lds_sync();
        top_merge(a.k, lane, bk, bt, run);
    }
    // outputs: lane i holds the i-th draw
    if (lane < a.k) {
        const int32_t t = run.key == 0ull ? -1 : run.tok;
        a.top_token[r * a.k + lane] = t;
        if (t < 0) {
            a.top_logq[r * a.k + lane] = -INFINITY;
        } else {
            const float x = a.x[r * a.V + t];
            a.top_logq[r * a.k + lane] =
                x == -INFINITY ? -INFINITY : ((double)mul_rn(x, a.invT32) - Ms) - logS0;
        }
    }
    if (lane == 0)
        a.entropy[r] = logS0 - ratio;
}

// word 0 of Philox4x64-10 on the host (the same published rounds as the
// device's), for the call's SplitMix64 key
uint64_t host_philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                           uint64_t k1)
{
    constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
    constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += kWeyl0;
            k1 += kWeyl1;
        }
        const unsigned __int128 p0 = (unsigned __int128)kMul0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)kMul1 * c2;
        const uint64_t n0 = (uint64_t)(p1 >> 64) ^ c1 ^ k0;
        const uint64_t n2 = (uint64_t)(p0 >> 64) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint64_t)p1;
        c2 = n2;
        c3 = (uint64_t)p0;
    }
    return c0;
}

bool ex_plan(int32_t V, int32_t &wpr)
{
    wpr = (int32_t)ceil_div(V, kExChunk);
    return wpr <= kExMaxWpr;
}

// one partial per wave of a row's shares; the sampled form is the larger
constexpr size_t kPartBytes = sizeof(ExPart) > sizeof(ExSPart) ? sizeof(ExPart) : sizeof(ExSPart);

} // namespace
} // namespace tav

extern "C" size_t tree_expand_workspace_bytes(int64_t R, int32_t V, int32_t k)
{
    using namespace tav;
    int32_t wpr = 0;
    if (R < 1 || V < 1 || k < 1 || k > kExMaxK || k > V || !ex_plan(V, wpr))
        return 0;
    return (size_t)R * wpr * kExWaves * kPartBytes;
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
    const size_t need = (size_t)R * wpr * kExWaves * kPartBytes;
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
    a.spart = static_cast<ExSPart *>(workspace);
    a.top_token = top_token;
    a.top_logq = top_logq;
    a.entropy = entropy;
    a.flags = dev_flags;
    a.seed = seed;
    a.offset = offset;
    a.T = temperature;
    a.K = sampled ? host_philox_word0(offset, 0, 0, 3, seed, 0) : 0;
    hipStream_t s = as_stream(stream);
    if (sampled)
        hipLaunchKernelGGL(expand_sample_part_kernel, dim3((unsigned)(R * wpr)), dim3(kExThreads),
                           0, s, a);
    else
        hipLaunchKernelGGL(expand_part_kernel, dim3((unsigned)(R * wpr)), dim3(kExThreads), 0, s,
                           a);
    if (hipGetLastError() != hipSuccess)
        return TAV_ERR_LAUNCH;
    if (sampled)
        hipLaunchKernelGGL(expand_sample_merge_kernel, dim3((unsigned)R), dim3(kMergeThreads), 0,
                           s, a);
    else
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
