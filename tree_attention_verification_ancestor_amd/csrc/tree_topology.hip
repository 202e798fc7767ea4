// tree_topology_dp: the budget-constrained tree topology by dynamic
// programming. The node count is capped and branches are allotted to
// maximise the expected number of accepted tokens, a problem solved by
// dynamic programming (jisaku.com glossary, tree-topology strategies); the
// Sequoia paragraph has the topology chosen for the hardware. The acceptance
// model is by sibling rank: the k-th child of a node, once reached, is
// accepted with probability p_k, at any depth, so a node contributes the
// product of the p of the ranks along its path.
//
// For a subtree of m nodes with r levels allowed below its root:
//   F(1, r) = 0, F(m, 0) = -inf (m > 1), F(m, r) = C(m - 1, r - 1, 1);
//   C(0, r, j) = 0, C(s, r, j) = -inf for j > K,
//   C(s, r, j) = max_{t = 1..s} p_j (1 + F(t, r)) + C(s - t, r, j + 1),
// the smallest t among equal maxima. One workgroup: level by level (r), rank
// by rank (j = K..1), every s in parallel (one thread per s), the t loop in
// each thread. The argmax of every (r, j, s) goes to the workspace, and one
// thread writes the tree out breadth-first from it: node 0 the root, each
// node's children appended in rank order as nodes are reached, so the
// output is topological and siblings are in the order the walk tries them.

#include <algorithm>

#include "common.h"

// Every value is formed exactly as written (a = 1 + F; b = p a; b + C), with
// no operation fused into another.
#pragma clang fp contract(off)

namespace tav {
namespace {

constexpr int kTopoMaxK = 16;
constexpr int kTopoMaxN = kMaxNodes;     // nodes in the tree
constexpr int kTopoMaxDepth = 64;
constexpr int kTopoThreads = 256;

struct TopoArgs {
    double p[kTopoMaxK];
    int32_t K, n, depth;
    int32_t *parent, *rank;
    double *value;
    int16_t *arg;        // [depth][K + 2][n]: argmax t of C(s, r, j)
};

__global__ __launch_bounds__(kTopoThreads) void tree_topology_kernel(TopoArgs a)
{
    __shared__ double s_fprev[kTopoMaxN + 1], s_fcur[kTopoMaxN + 1];
    __shared__ double s_c[2][kTopoMaxN];
    __shared__ int32_t s_queue_node[kTopoMaxN], s_queue_m[kTopoMaxN], s_queue_r[kTopoMaxN];
    const int tid = threadIdx.x;
    const int n = a.n, K = a.K;
    for (int m = tid; m <= n; m += kTopoThreads)
        s_fprev[m] = m == 1 ? 0.0 : -INFINITY;   // F(., 0)
    __syncthreads();
    for (int r = 1; r <= a.depth; ++r) {
        const int rr = r - 1;
        // C(., rr, K + 1): only s = 0
        int cur = 0;
        for (int s = tid; s < n; s += kTopoThreads)
            s_c[cur][s] = s == 0 ? 0.0 : -INFINITY;
        __syncthreads();
        for (int j = K; j >= 1; --j) {
            const double pj = a.p[j - 1];
            const double *cnext = s_c[cur];
            double *cnew = s_c[cur ^ 1];
            for (int s = tid; s < n; s += kTopoThreads) {
                double best = -INFINITY;
                int arg = 0;
                if (s == 0) {
                    best = 0.0;
                } else {
                    for (int t = 1; t <= s; ++t) {
                        const double f = s_fprev[t];
                        const double rest = cnext[s - t];
                        if (f == -INFINITY || rest == -INFINITY)
                            continue;
                        const double av = 1.0 + f;
                        const double bv = pj * av;
                        const double v = bv + rest;
                        if (v > best) {
                            best = v;
                            arg = t;
                        }
                    }
                }
                cnew[s] = best;
                a.arg[((int64_t)rr * (K + 2) + j) * n + s] = (int16_t)arg;
            }
            __syncthreads();
            cur ^= 1;
        }
        for (int m = tid; m <= n; m += kTopoThreads)
            s_fcur[m] = m == 0 ? -INFINITY : (m == 1 ? 0.0 : s_c[cur][m - 1]);
        __syncthreads();
        for (int m = tid; m <= n; m += kTopoThreads)
            s_fprev[m] = s_fcur[m];
        __syncthreads();
    }
    if (tid != 0)
        return;
    // breadth-first write-out: node, its subtree size and levels left
    a.value[0] = s_fprev[n];
    int count = 1, head = 0;
    a.parent[0] = -1;
    a.rank[0] = 0;
    s_queue_node[0] = 0;
    s_queue_m[0] = n;
    s_queue_r[0] = a.depth;
    while (head < count) {
        const int node = s_queue_node[head], m = s_queue_m[head], r = s_queue_r[head];
        ++head;
        int s = m - 1, j = 1;
        while (s > 0 && j <= K && count < n) {
            const int t = a.arg[((int64_t)(r - 1) * (K + 2) + j) * n + s];
            if (t <= 0)
                break;   // unreachable for a feasible n (checked on the host)
            a.parent[count] = node;
            a.rank[count] = j;
            s_queue_node[count] = count;
            s_queue_m[count] = t;
            s_queue_r[count] = r - 1;
            ++count;
            s -= t;
            ++j;
        }
    }
}

// Largest tree of depth <= depth with at most K children per node, capped.
int64_t topo_capacity(int K, int depth, int64_t cap)
{
    int64_t total = 1, level = 1;
    for (int d = 0; d < depth && total < cap; ++d) {
        level = std::min<int64_t>(level * K, cap);
        total = std::min<int64_t>(total + level, cap);
    }
    return total;
}

} // namespace
} // namespace tav

extern "C" size_t tree_topology_workspace_bytes(int32_t K, int32_t n, int32_t depth)
{
    using namespace tav;
    if (K < 1 || K > kTopoMaxK || n < 1 || n > kTopoMaxN || depth < 0 || depth > kTopoMaxDepth)
        return 0;
    return (size_t)std::max(depth, 1) * (K + 2) * n * sizeof(int16_t);
}

extern "C" tav_status tree_topology_dp(const double *p_rank, int32_t K, int32_t n, int32_t depth,
                                       int32_t *parent, int32_t *rank, double *value,
                                       void *workspace, size_t ws_bytes, void *stream)
{
    using namespace tav;
    if (!p_rank || !parent || !rank || !value || K < 1 || n < 1 || depth < 0)
        return TAV_ERR_ARG;
    if (K > kTopoMaxK || n > kTopoMaxN || depth > kTopoMaxDepth)
        return TAV_ERR_UNSUPPORTED;
    for (int k = 0; k < K; ++k)
        if (!(p_rank[k] >= 0.0 && p_rank[k] <= 1.0))
            return TAV_ERR_ARG;
    if (topo_capacity(K, depth, n) < n)
        return TAV_ERR_UNSUPPORTED;   // no n-node tree fits the depth and width
    if (!aligned(value, 8) || !aligned(parent, 4) || !aligned(rank, 4))
        return TAV_ERR_ARG;
    const size_t need = tree_topology_workspace_bytes(K, n, depth);
    if (!workspace || ws_bytes < need || !aligned(workspace, 8))
        return TAV_ERR_WORKSPACE;
    TopoArgs a;
    for (int k = 0; k < kTopoMaxK; ++k)
        a.p[k] = k < K ? p_rank[k] : 0.0;
    a.K = K;
    a.n = n;
    a.depth = depth;
    a.parent = parent;
    a.rank = rank;
    a.value = value;
    a.arg = static_cast<int16_t *>(workspace);
    hipLaunchKernelGGL(tree_topology_kernel, dim3(1), dim3(kTopoThreads), 0, as_stream(stream), a);
    return hipGetLastError() == hipSuccess ? TAV_OK : TAV_ERR_LAUNCH;
}
