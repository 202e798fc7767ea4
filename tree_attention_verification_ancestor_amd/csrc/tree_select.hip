// tree_select_topm: keep the M best nodes of a candidate tree, renumbered;
// tree_widths_by_entropy: branching widths from the frontier's entropy ranks.
//
// The budget rule of tree construction (jisaku.com glossary, tree-topology
// strategies, budget-constrained optimisation) caps the node count and
// allots branches to maximise the expected number of accepted tokens;
// EAGLE-2 grows its draft tree dynamically and keeps the most promising
// paths (LLM Primer ch. 9, section 9.2). With a node's acceptance estimated
// by the draft as the product of q along its path, the score of node i is
// score(parent) + log q(token i), score(root) = 0, and since no child scores
// above its parent the M best nodes by score (lower index first among
// equals, so an ancestor before its descendants) are the budget's optimum
// and already a subtree.
//
// One workgroup per tree, a thread per candidate node (up to 1024). Depths
// come from climbing parent pointers; scores are summed level by level from
// the root, one fp64 addition per node, so every score is the same sum in
// the same order as a sequential pass. A node's rank counts the nodes ahead
// of it (higher score, or equal score and lower index), counted by up to
// four threads per node over shares of the scores, read from LDS by all
// lanes at once; the kept nodes get new indices from a ballot prefix sum in
// ascending original index, which keeps the tree topological.

#include "common.h"

namespace tav {
namespace {

constexpr int kSelThreads = 1024;

// Nodes ahead of node n among the scores s[0, W) (padded past the real
// count with values that never count), over the share [j_begin, j_end) of
// them: descending order counts #{j < n: s_j >= s_n} + #{j > n: s_j > s_n},
// ascending the mirror image. Sixteen scores per step, as eight 16-byte LDS
// reads that every lane of the wave shares; a block wholly below or above
// the wave's 64 nodes needs one comparison per score.
template <bool kDescending>
__device__ __forceinline__ int count_ahead(const double *s, int n, double sn, int j_begin,
                                           int j_end)
{
    auto before = [&](double v) __attribute__((always_inline)) {   // j < n
        return kDescending ? v >= sn : v <= sn;
    };
    auto after = [&](double v) __attribute__((always_inline)) {    // j > n
        return kDescending ? v > sn : v < sn;
    };
    const int w0 = n & ~63;
    int r = 0;
    for (int j0 = j_begin; j0 < j_end; j0 += 16) {
        double2 v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            v[t] = *reinterpret_cast<const double2 *>(&s[j0 + 2 * t]);
        if (j0 + 16 <= w0) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                r += (int)before(v[t].x) + (int)before(v[t].y);
        } else if (j0 >= w0 + 64) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                r += (int)after(v[t].x) + (int)after(v[t].y);
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = j0 + 2 * t;
                r += (int)(j < n ? before(v[t].x) : after(v[t].x));
                r += (int)(j + 1 < n ? before(v[t].y) : after(v[t].y));
            }
        }
    }
    return r;
}

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ token,
    const double *__restrict__ logq, int32_t Nc, int32_t M, int32_t *__restrict__ out_parent,
    int32_t *__restrict__ out_token, int32_t *__restrict__ out_src, uint32_t *flags)
{
    __shared__ int32_t s_par[kSelThreads];
    __shared__ __align__(16) double s_score[kSelThreads];
    __shared__ int32_t s_new[kSelThreads];
    __shared__ int32_t s_rank[kSelThreads];
    __shared__ int32_t s_wcount[kSelThreads / 64];
    __shared__ int s_bad, s_maxd;

    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int lane = i & 63, wave = i >> 6;
    const int64_t row = (int64_t)b * Nc;
    const bool live = i < Nc;

    int p = -1;
    double l = 0.0;
    if (i == 0) {
        s_bad = 0;
        s_maxd = 0;
    }
    if (live) {
        p = parent[row + i];
        l = logq[row + i];
        s_par[i] = p;
    }
    __syncthreads();
    if (live) {
        if (i == 0 ? p != -1 : (p < 0 || p >= i))
            atomicOr(&s_bad, 1);
        if (i > 0 && __builtin_isnan(l))
            atomicOr(&s_bad, 2);
    }
    __syncthreads();
    const int bad = s_bad;
    if (bad) {
        if (i == 0)
            raise_flag(flags, (bad & 1 ? TAV_FLAG_BAD_PARENT : 0u) |
                                  (bad & 2 ? TAV_FLAG_NONFINITE_LOGITS : 0u));
        return;
    }

    // depth by climbing (parent[j] < j, so at most i steps)
    int d = 0;
    if (live) {
        for (int j = i; j != 0; j = s_par[j])
            ++d;
        atomicMax(&s_maxd, d);
    }
    // scores past Nc (up to the next multiple of 64) are -inf at a higher
    // index than any node, so they never count as ahead of one
    const int W = ((Nc + 63) >> 6) * 64;
    if (i == 0)
        s_score[0] = 0.0;
    else if (i >= Nc && i < W)
        s_score[i] = -INFINITY;
    if (i < W)
        s_rank[i] = 0;
    __syncthreads();
    // a log q above 0 can only be rounding; it counts as 0
    const double inc = l < 0.0 ? l : 0.0;
    const int maxd = s_maxd;
    for (int lev = 1; lev <= maxd; ++lev) {
        if (live && d == lev)
            s_score[i] = s_score[p] + inc;
        __syncthreads();
    }

    // rank of node n: the nodes ahead of it, counted by blockDim / W
    // threads per node over contiguous shares of the scores
    {
        const int n = i % W;
        const int part = i / W;
        const int share = W / (blockDim.x / W);
        atomicAdd(&s_rank[n],
                  count_ahead<true>(s_score, n, s_score[n], part * share, (part + 1) * share));
    }
    __syncthreads();
    const bool sel = live && s_rank[i] < M;
    const uint64_t bal = __ballot(sel);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0)
        s_wcount[wave] = __popcll(bal);
    __syncthreads();
    int newi = below;
    for (int w = 0; w < wave; ++w)
        newi += s_wcount[w];
    if (live)
        s_new[i] = sel ? newi : -1;
    __syncthreads();
    if (sel) {
        const int64_t o = (int64_t)b * M + newi;
        out_src[o] = i;
        out_token[o] = token[row + i];
        out_parent[o] = i == 0 ? -1 : s_new[p];
    }
}

// Entropy-ranked widths: one workgroup per frontier, the same rank counts
// in ascending order; width = w_min + span * rank / F.
__global__ __launch_bounds__(kSelThreads) void widths_kernel(const double *__restrict__ entropy,
                                                             int32_t F, int32_t w_min,
                                                             int32_t span,
                                                             int32_t *__restrict__ width,
                                                             uint32_t *flags)
{
    __shared__ __align__(16) double s_h[kSelThreads];
    __shared__ int32_t s_rank[kSelThreads];
    __shared__ int s_bad;
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int W = ((F + 63) >> 6) * 64;
    if (i == 0)
        s_bad = 0;
    if (i < W) {
        // past F: +inf at a higher index than any node, never ahead of one
        const double h = i < F ? entropy[(int64_t)b * F + i] : INFINITY;
        s_h[i] = h;
        s_rank[i] = 0;
    }
    __syncthreads();
    if (i < F && __builtin_isnan(s_h[i]))
        atomicOr(&s_bad, 1);
    __syncthreads();
    if (s_bad) {
        if (i == 0)
            raise_flag(flags, TAV_FLAG_NONFINITE_LOGITS);
        return;
    }
    {
        const int n = i % W;
        const int part = i / W;
        const int share = W / (blockDim.x / W);
        atomicAdd(&s_rank[n], count_ahead<false>(s_h, n, s_h[n], part * share, (part + 1) * share));
    }
    __syncthreads();
    if (i < F)
        width[(int64_t)b * F + i] = w_min + (int32_t)(((int64_t)span * s_rank[i]) / F);
}

int rank_threads(int32_t n)
{
    // a thread per node (whole waves), and up to four per node for the
    // rank counts while they fit in 1024
    const int W = (int)ceil_div(n, 64) * 64;
    return W * (W <= 256 ? 4 : W <= 512 ? 2 : 1);
}

} // namespace
} // namespace tav

extern "C" tav_status tree_select_topm(const int32_t *parent, const int32_t *token,
                                       const double *logq, int32_t B, int32_t Nc, int32_t M,
                                       int32_t *out_parent, int32_t *out_token, int32_t *out_src,
                                       uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!parent || !token || !logq || !out_parent || !out_token || !out_src)
        return TAV_ERR_ARG;
    if (B < 1 || Nc < 1 || M < 1 || M > Nc)
        return TAV_ERR_ARG;
    if (Nc > kSelThreads)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(parent, 4) || !aligned(token, 4) || !aligned(logq, 8) ||
        !aligned(out_parent, 4) || !aligned(out_token, 4) || !aligned(out_src, 4))
        return TAV_ERR_ARG;
    hipLaunchKernelGGL(tree_select_kernel, dim3(B), dim3(rank_threads(Nc)), 0, as_stream(stream),
                       parent, token, logq, Nc, M, out_parent, out_token, out_src, dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}

extern "C" tav_status tree_widths_by_entropy(const double *entropy, int32_t B, int32_t F,
                                             int32_t w_min, int32_t w_max, int32_t *width,
                                             uint32_t *dev_flags, void *stream)
{
    using namespace tav;
    if (!entropy || !width || B < 1 || F < 1 || w_min < 0 || w_max < w_min)
        return TAV_ERR_ARG;
    if (F > kSelThreads)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(entropy, 8) || !aligned(width, 4))
        return TAV_ERR_ARG;
    hipLaunchKernelGGL(widths_kernel, dim3(B), dim3(rank_threads(F)), 0, as_stream(stream),
                       entropy, F, w_min, w_max - w_min + 1, width, dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}
