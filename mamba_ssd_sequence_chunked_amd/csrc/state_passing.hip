// state_passing.hip - stage 3: the recurrence between chunks.
//
//   S = init (or 0);  for c = 0 .. nc-1:  entry[c] = S;  S = exp(cs_c[Q-1]) * S + S_c
//   final = S
//
// The chunk-level form of the same linear recurrence, with the whole chunk's
// decay as the transition (ql.gl, "The Core of SSD"; the state update of the
// mohakchugh blog's block-decomposition outline, which reads the state
// entering a chunk before updating it).  It is sequential over chunks and
// embarrassingly parallel over (batch, head, headdim, dstate), and it does
// almost no arithmetic: one read of every chunk state and one write of every
// entry state, so it is bound by HBM bandwidth.
//
// Each thread owns 4 consecutive state elements of one (batch, head) and
// walks the chunks with 16-byte loads and stores; the loads of the next
// chunks do not depend on the running state, so unrolling lets several be
// in flight.  A workgroup covers 1024 elements of a single (batch, head), so
// the chunk decay is one uniform value per chunk.  The running state stays
// in fp32; entry states are rounded to T once, as the next stage consumes
// them as matrix-core operands (or, for the backward's split products, given
// as bf16 hi and lo planes that carry the fp32 state to 2^-18).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kElemsPerBlock = 1024;

// Packed variable-length batches (batch 1; cmeta from varlen_meta.hip, per chunk {cont, whole,
// kend, pe}): the state entering chunk c is the running state only when the chunk's first token
// continues a sequence (else zero, a reset); the running state after the chunk is the chunk's
// own state (masked to its last sequence) plus the decayed entering state only when no sequence
// starts inside it; and the sequence that continues into the chunk and ends there at position pe
// gets exp(cs[pe]) times the entering state added to its final state, which stage 2 has set to
// the sequence's own part.  final_states is (nseq, H, P, N) and no initial state is taken.
template <typename T, bool kVarlen>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float* __restrict__ chunk_states, const float* __restrict__ dA_cs,
    const float* __restrict__ init, T* __restrict__ entry, float* __restrict__ final_states,
    const int4* __restrict__ cmeta, int64_t lo_off, int nheads, int PN, int Q, int nc)
{
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int e = blockIdx.x * kElemsPerBlock + 4 * threadIdx.x;
    if (e >= PN) return;
    const int64_t bh = b * nheads + h;

    float4 s = init ? *reinterpret_cast<const float4*>(init + bh * PN + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float* cs = dA_cs + bh * (int64_t)nc * Q + (Q - 1);
    const int64_t stride = (int64_t)nheads * PN;               // one chunk
    const float* src = chunk_states + (b * nc * nheads + h) * (int64_t)PN + e;
    T* dst = entry + (b * nc * nheads + h) * (int64_t)PN + e;

    if constexpr (kVarlen) {
        const float* csc = dA_cs + bh * (int64_t)nc * Q;
#pragma unroll 4
        for (int c = 0; c < nc; ++c) {
            const float4 sc = *reinterpret_cast<const float4*>(src + c * stride);
            const int4 m = cmeta[c];
            if (!m.x) s = make_float4(0.f, 0.f, 0.f, 0.f);            // a sequence starts at the chunk
            store4(dst + c * stride, s.x, s.y, s.z, s.w);
            if (m.z >= 0) {
                // the continued sequence ends in this chunk at position m.w
                float4* f = reinterpret_cast<float4*>(final_states + ((int64_t)m.z * nheads + h) * PN + e);
                const float de = __expf(csc[(int64_t)c * Q + min(max(m.w, 0), Q - 1)]);
                const float4 fv = *f;
                *f = make_float4(fmaf(de, s.x, fv.x), fmaf(de, s.y, fv.y), fmaf(de, s.z, fv.z), fmaf(de, s.w, fv.w));
            }
            const float dec = m.y ? __expf(cs[(int64_t)c * Q]) : 0.f;   // no start inside: carry on
            s.x = fmaf(dec, s.x, sc.x);
            s.y = fmaf(dec, s.y, sc.y);
            s.z = fmaf(dec, s.z, sc.z);
            s.w = fmaf(dec, s.w, sc.w);
        }
        return;
    }
#pragma unroll 4
    for (int c = 0; c < nc; ++c) {
        const float4 sc = *reinterpret_cast<const float4*>(src + c * stride);
        const float dec = __expf(cs[(int64_t)c * Q]);
        store4(dst + c * stride, s.x, s.y, s.z, s.w);
        if constexpr (std::is_same_v<T, bf16>) {
            if (lo_off) {                   // the rounding remainders as a second plane
                auto rem = [](float v) { return v - static_cast<float>(static_cast<bf16>(v)); };
                store4(dst + lo_off + c * stride, rem(s.x), rem(s.y), rem(s.z), rem(s.w));
            }
        }
        s.x = fmaf(dec, s.x, sc.x);
        s.y = fmaf(dec, s.y, sc.y);
        s.z = fmaf(dec, s.z, sc.z);
        s.w = fmaf(dec, s.w, sc.w);
    }
    *reinterpret_cast<float4*>(final_states + bh * PN + e) = s;
}

}  // namespace

template <typename T>
hipError_t launch_state_passing(const float* chunk_states, const float* dA_cs, const float* init,
                                T* entry_states, float* final_states, const Dims& d,
                                hipStream_t stream)
{
    if (d.batch == 0) return hipSuccess;
    const int PN = (int)(d.headdim * d.dstate);
    dim3 grid((unsigned)((PN + kElemsPerBlock - 1) / kElemsPerBlock), (unsigned)d.nheads,
              (unsigned)d.batch);
    hipLaunchKernelGGL((state_passing_kernel<T, false>), grid, dim3(256), 0, stream, chunk_states, dA_cs, init,
                       entry_states, final_states, nullptr, (int64_t)0, (int)d.nheads, PN, (int)d.chunk,
                       (int)d.nchunks());
    return hipGetLastError();
}

hipError_t launch_state_passing_split(const float* chunk_states, const float* dA_cs, const float* init,
                                      bf16* entry_hi, int64_t lo_off, float* final_states, const Dims& d,
                                      hipStream_t stream)
{
    if (d.batch == 0) return hipSuccess;
    const int PN = (int)(d.headdim * d.dstate);
    dim3 grid((unsigned)((PN + kElemsPerBlock - 1) / kElemsPerBlock), (unsigned)d.nheads,
              (unsigned)d.batch);
    hipLaunchKernelGGL((state_passing_kernel<bf16, false>), grid, dim3(256), 0, stream, chunk_states, dA_cs, init,
                       entry_hi, final_states, nullptr, lo_off, (int)d.nheads, PN, (int)d.chunk, (int)d.nchunks());
    return hipGetLastError();
}

template <typename T>
hipError_t launch_state_passing_varlen(const float* chunk_states, const float* dA_cs, const int* cmeta,
                                       T* entry_states, float* final_states, const Dims& d, hipStream_t stream)
{
    if (d.seqlen == 0) return hipSuccess;
    const int PN = (int)(d.headdim * d.dstate);
    dim3 grid((unsigned)((PN + kElemsPerBlock - 1) / kElemsPerBlock), (unsigned)d.nheads, 1u);
    hipLaunchKernelGGL((state_passing_kernel<T, true>), grid, dim3(256), 0, stream, chunk_states, dA_cs, nullptr,
                       entry_states, final_states, reinterpret_cast<const int4*>(cmeta), (int64_t)0, (int)d.nheads, PN,
                       (int)d.chunk, (int)d.nchunks());
    return hipGetLastError();
}

template hipError_t launch_state_passing<float>(const float*, const float*, const float*, float*,
                                                float*, const Dims&, hipStream_t);
template hipError_t launch_state_passing<bf16>(const float*, const float*, const float*, bf16*,
                                               float*, const Dims&, hipStream_t);
template hipError_t launch_state_passing_varlen<float>(const float*, const float*, const int*, float*, float*,
                                                       const Dims&, hipStream_t);
template hipError_t launch_state_passing_varlen<bf16>(const float*, const float*, const int*, bf16*, float*,
                                                      const Dims&, hipStream_t);

}  // namespace ssd
