// varlen_meta.hip - sequence boundaries of a packed variable-length batch, per token and per chunk.
//
// Packed sequences share one token axis without padding (the variable-length batches of the ql.gl
// page, section "Mamba-2 Changes More Than the Algorithm"); sequence k is tokens cu[k] ..
// cu[k+1]-1 and its state starts from zero: the recurrence is reset at every sequence start, so
// the chunked form must not carry state or decay across a start.  The chunk grid stays the grid of
// the packed axis, so a chunk may hold the end of one sequence, whole short sequences and the
// start of another.  This kernel tabulates what the stage kernels need:
//   tstart[t]  first token of t's sequence (tokens s <= t of one chunk belong to t's sequence
//              exactly when s >= tstart[t])
//   cmeta[c]   {cont, whole, kend, pe}: cont = the chunk's first token continues a sequence begun
//              in an earlier chunk; whole = so does its last token (no sequence starts inside
//              the chunk); kend = that continued sequence when it ends inside the chunk (else
//              -1), pe = its last token's position in the chunk.
// cu is read with clamped indices, so any content keeps every access in bounds (results are
// then unspecified).
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

// index of the sequence holding token t: the largest k < nseq with cu[k] <= t
__device__ __forceinline__ int seq_of(const int* __restrict__ cu, int nseq, int t)
{
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void varlen_meta_kernel(const int* __restrict__ cu, int nseq, int total, int Q,
                                                          int nc, int* __restrict__ tstart, int4* __restrict__ cmeta)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < total) {
        const int k = seq_of(cu, nseq, i);
        tstart[i] = min(max(cu[k], 0), i);
    }
    if (i < nc) {
        const int first = i * Q;
        const int last = min(first + Q, total) - 1;
        const int k = seq_of(cu, nseq, first);
        const int kl = seq_of(cu, nseq, last);
        const int start = min(max(cu[k], 0), first);
        const int startl = min(max(cu[kl], 0), last);
        const int end = min(max(cu[k + 1], first + 1), total) - 1;       // last token of the first token's sequence
        const int cont = start < first;
        const int whole = startl < first;
        const int kend = (cont && end <= last) ? k : -1;
        cmeta[i] = make_int4(cont, whole, kend, end - first);
    }
}

}  // namespace

hipError_t launch_varlen_meta(const int* cu_seqlens, int64_t nseq, int64_t total, int64_t chunk, int* tstart,
                              int* cmeta, hipStream_t stream)
{
    const int64_t nc = (total + chunk - 1) / chunk;
    const int64_t n = total > nc ? total : nc;
    if (n == 0 || nseq == 0) return hipSuccess;
    hipLaunchKernelGGL(varlen_meta_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, cu_seqlens,
                       (int)nseq, (int)total, (int)chunk, (int)nc, tstart, reinterpret_cast<int4*>(cmeta));
    return hipGetLastError();
}

}  // namespace ssd
