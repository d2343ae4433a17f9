// dA_cumsum.hip - stage 1: per-chunk prefix sums of dt * A.
//
// The decay between positions s < l of a chunk is the product of the
// per-step decays a_j = exp(dt_j A_h) for j = s+1..l (the matrix-mixer
// entries of the "Mamba-2" wiki note, section "Matrix Mixer View"; the
// discretisation Abar = exp(Delta A) of the mohakchugh blog, section "State
// Space Models: The Core Abstraction").  Its logarithm is a difference of
// in-chunk prefix sums of dt_j A_h, which this kernel writes once so the
// matrix-core stages form exp(cs[l] - cs[s]) on the fly and never store a
// chunk x chunk decay tile.  The sum restarts at every chunk, which keeps
// its magnitude (and the rounding of the difference) bounded by one chunk.
//
// One workgroup per (batch, chunk, 16 heads): the chunk's dt rows are read
// once (16 heads = 64 contiguous bytes per token), transposed through LDS,
// and each wavefront scans one head's chunk with 4 tokens per lane and a
// DPP wavefront prefix sum.  Outputs are (batch, head, chunk, position),
// contiguous per chunk, for coalesced reads by the later stages.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kHeadsPerBlock = 16;
constexpr int kMaxChunk = 256;

__global__ __launch_bounds__(256) void dA_cumsum_kernel(const float* __restrict__ dt,
                                                        const float* __restrict__ A,
                                                        float* __restrict__ dA_cs,
                                                        float* __restrict__ dt_chunked, int seqlen,
                                                        int nheads, int Q, int nc)
{
    __shared__ float tile[kHeadsPerBlock][kMaxChunk + 4];
    const int h0 = blockIdx.x * kHeadsPerBlock;
    const int c = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x;
    const int nh = min(kHeadsPerBlock, nheads - h0);
    const int64_t t0 = (int64_t)c * Q;

    for (int i = tid; i < Q * kHeadsPerBlock; i += blockDim.x) {
        const int l = i / kHeadsPerBlock, hh = i % kHeadsPerBlock;
        float v = 0.f;
        if (hh < nh && t0 + l < seqlen) v = dt[(b * seqlen + t0 + l) * nheads + h0 + hh];
        tile[hh][l] = v;
    }
    __syncthreads();

    const int wave = tid / kWave, lane = lane_id();
    for (int hh = wave; hh < nh; hh += blockDim.x / kWave) {
        const float a = A[h0 + hh];
        float v[4], s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int l = 4 * lane + j;
            v[j] = l < Q ? tile[hh][l] : 0.f;
        }
        s[0] = v[0] * a;
#pragma unroll
        for (int j = 1; j < 4; ++j) s[j] = s[j - 1] + v[j] * a;
        const float incl = wave_inclusive_sum(s[3]);
        const float excl = incl - s[3];
        const int64_t base = ((b * nheads + h0 + hh) * nc + c) * Q;
        if (4 * lane + 3 < Q) {
            store4(dA_cs + base + 4 * lane, s[0] + excl, s[1] + excl, s[2] + excl, s[3] + excl);
            store4(dt_chunked + base + 4 * lane, v[0], v[1], v[2], v[3]);
        }
    }
}

}  // namespace

hipError_t launch_dA_cumsum(const float* dt, const float* A, float* dA_cs, float* dt_chunked,
                            const Dims& d, hipStream_t stream)
{
    const int nc = (int)d.nchunks();
    if (d.batch == 0 || nc == 0) return hipSuccess;
    dim3 grid((unsigned)((d.nheads + kHeadsPerBlock - 1) / kHeadsPerBlock), (unsigned)nc,
              (unsigned)d.batch);
    hipLaunchKernelGGL(dA_cumsum_kernel, grid, dim3(256), 0, stream, dt, A, dA_cs, dt_chunked,
                       (int)d.seqlen, (int)d.nheads, (int)d.chunk, nc);
    return hipGetLastError();
}

}  // namespace ssd
