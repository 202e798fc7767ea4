// Philox4x64-10 on the device, and the node-uniform convention of the sampler.
//
// J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
// numbers: as easy as 1, 2, 3" (SC'11): the 4x64 round multiplies words 0 and
// 2 by two fixed odd constants, swaps the halves across the lanes and mixes in
// the key, which is bumped by two Weyl constants between rounds.
//
// Node i of sequence b uses counter (offset, b, i, 0) and key (seed, 0).
// Word 0 is its acceptance uniform, word 1 the resampling uniform used if the
// walk stops at i; each keeps its top 24 bits: u = (w >> 40) * 2^-24, exact in
// fp32 and fp64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tav {

struct NodeUniforms {
    double acc;
    double res;
};

// Ten Philox4x64 rounds on counter (c0, c1, c2, c3) under key (k0, k1).
__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              uint64_t k0, uint64_t k1, uint64_t (&w)[4])
{
    constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
    constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += kWeyl0;
            k1 += kWeyl1;
        }
        const uint64_t hi0 = __umul64hi(kMul0, c0), lo0 = kMul0 * c0;
        const uint64_t hi1 = __umul64hi(kMul1, c2), lo1 = kMul1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0;
        const uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    w[0] = c0;
    w[1] = c1;
    w[2] = c2;
    w[3] = c3;
}

__device__ __forceinline__ NodeUniforms node_uniforms(uint64_t seed, uint64_t offset, int64_t b,
                                                      int64_t i)
{
    uint64_t w[4];
    philox4x64_10(offset, (uint64_t)b, (uint64_t)i, 0, seed, 0, w);
    NodeUniforms u;
    u.acc = (double)(w[0] >> 40) * 0x1p-24;
    u.res = (double)(w[1] >> 40) * 0x1p-24;
    return u;
}

} // namespace tav
