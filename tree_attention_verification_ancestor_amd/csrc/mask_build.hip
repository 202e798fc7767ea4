// tree_mask_build: parent[] -> packed ancestor-or-self bitmasks.
//
// M[i][j] = 1 exactly when node j is node i or one of its ancestors
// (jisaku.com glossary, "tree-based speculative decoding", tree-attention
// section; the 5-node instance is the radar-34b blog's §3 matrix).
//
// One workgroup per tree: the parent row is staged in LDS, then every thread
// climbs from its node to the root setting one bit per node met. Nodes are
// numbered topologically (parent[i] < i), so each climb ends in at most
// depth+1 steps and no climb depends on another's result.

#include "common.h"

namespace tav {
namespace {

__global__ __launch_bounds__(256) void mask_build_kernel(const int32_t *__restrict__ parent,
                                                         int32_t N, int32_t W,
                                                         uint64_t *__restrict__ mask,
                                                         int32_t *__restrict__ depth,
                                                         uint32_t *flags)
{
    __shared__ int32_t par[kMaxNodes];
    const int b = blockIdx.x;
    const int32_t *row = parent + (int64_t)b * N;
    for (int i = threadIdx.x; i < N; i += blockDim.x)
        par[i] = row[i];
    __syncthreads();

    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        uint64_t words[4] = {0, 0, 0, 0};
        bool bad = (i == 0) ? (par[0] != -1) : (par[i] < 0 || par[i] >= i);
        int d = 0;
        int j = i;
        while (!bad) {
            words[j >> 6] |= 1ull << (j & 63);
            if (j == 0)
                break;
            const int pj = par[j];
            if (pj < 0 || pj >= j) {
                bad = true;
                break;
            }
            j = pj;
            ++d;
        }
        if (bad)
            raise_flag(flags, TAV_FLAG_BAD_PARENT);
        uint64_t *out = mask + ((int64_t)b * N + i) * W;
        for (int w = 0; w < W; ++w)
            out[w] = words[w];
        if (depth)
            depth[(int64_t)b * N + i] = d;
    }
}

} // namespace
} // namespace tav

extern "C" tav_status tree_mask_build(const int32_t *parent, int32_t B, int32_t N,
                                      uint64_t *mask, int32_t *depth, uint32_t *dev_flags,
                                      void *stream)
{
    using namespace tav;
    if (!parent || !mask || B < 1 || N < 1)
        return TAV_ERR_ARG;
    if (N > kMaxNodes)
        return TAV_ERR_UNSUPPORTED;
    if (!aligned(mask, 8) || !aligned(parent, 4) || (depth && !aligned(depth, 4)))
        return TAV_ERR_ARG;
    const int32_t W = (int32_t)ceil_div(N, 64);
    const int threads = N <= 64 ? 64 : (N <= 128 ? 128 : 256);
    hipLaunchKernelGGL(mask_build_kernel, dim3(B), dim3(threads), 0, as_stream(stream), parent,
                       N, W, mask, depth, dev_flags);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}
