// selective_scan.hip - the Mamba-1 selective scan, the layer the SSD form replaces.
//
//   a_t[d, n] = exp(delta_t[d] A[d, n])
//   h_t[d, n] = a_t[d, n] h_{t-1}[d, n] + (delta_t[d] x_t[d]) B_t[n]
//   y_t[d]    = sum_n C_t[n] h_t[d, n] + D[d] x_t[d]
//
// Every channel d has a diagonal transition of its own (one decay per state
// entry), B and C belong to the token and are shared by all channels
// (mohakchugh blog, section "Mamba-1: Selective State Spaces"; the diagonal
// transition of the "Transformers are SSMs" paper card, "How It Works").
// Because the decay differs per state entry there is no scalar decay to
// factor out of a block of tokens, so this recurrence has no dense
// matrix-product form (the point the pages make for the SSD restriction):
// it runs on the vector ALUs, one exponential and three multiply-adds per
// (token, channel, state entry), and is bound by the ALUs, not by HBM.
//
// Each channel's N state entries are spread over W adjacent lanes (S = N / W
// entries per lane, kept in registers for the whole sequence), so a 256-lane
// workgroup walks 256 / W channels of one batch row through all tokens.
// Tokens are processed in blocks of TB: the workgroup stages the block's x,
// delta, delta*x (channels x tokens) and B, C (tokens x states, converted to
// fp32) in LDS with coalesced 16-byte loads, the next block's loads being in
// flight while the current block is computed; every lane then steps its S
// entries through the block, the W partial readouts of a channel are summed
// with DPP lane moves, and the block's y (plus the skip term) leaves through
// coalesced 16-byte stores.  exp is evaluated as exp2 of delta * (A log2 e)
// with A log2 e formed once per lane.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                 // channels per staging load/store (16 bytes of bf16)

// sum over aligned groups of W lanes (W in {1, 2, 4, 8, 16}) with DPP lane moves; every lane of a
// group ends with the group's sum
template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
    if constexpr (W >= 2)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
    if constexpr (W >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, true));   // quad_perm 2,3,0,1
    if constexpr (W >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, true));  // row_half_mirror
    if constexpr (W >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, true));  // row_mirror
    return v;
}

template <typename T, int W, int S>
struct ScanShape {
    static constexpr int N = W * S;
    static constexpr int CPW = kThreads / W;            // channels per workgroup
    static constexpr int TB = 2048 / CPW;               // tokens per block
    static constexpr int XV = TB * CPW / kVec / kThreads;   // 8-channel vectors per thread per block
    static constexpr int BCE = TB * N;                  // B (or C) elements per block
    static constexpr int BCV = (BCE + 4 * kThreads - 1) / (4 * kThreads);   // 4-element loads per thread
    static_assert(XV >= 1 && TB * CPW == XV * kVec * kThreads, "staging layout");
};

template <typename T, int W, int S>
__global__ __launch_bounds__(kThreads) void selective_scan_kernel(
    const T* __restrict__ x, const float* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dv,
    const float* __restrict__ init, T* __restrict__ y, float* __restrict__ final_states, int seqlen,
    int dim, int ncblk)
{
    using SH = ScanShape<T, W, S>;
    constexpr int N = SH::N, CPW = SH::CPW, TB = SH::TB;
    __shared__ float xs[TB][CPW];
    __shared__ float dls[TB][CPW];
    __shared__ float us[TB][CPW];
    __shared__ float ys[TB][CPW];
    __shared__ __attribute__((aligned(16))) float bs[TB][N];
    __shared__ __attribute__((aligned(16))) float cs[TB][N];

    const int cb = blockIdx.x % ncblk;
    const int64_t b = blockIdx.x / ncblk;
    const int c0 = cb * CPW;
    const int tid = threadIdx.x;
    const int ch = tid / W, sub = tid % W;
    const int c = min(c0 + ch, dim - 1);                 // lanes past the last channel compute on a copy
    const bool live = c0 + ch < dim;

    float h[S], a2[S];
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = sub * S + s;
        a2[s] = A[(int64_t)c * N + n] * kLog2e;
        h[s] = init ? init[(b * dim + c) * N + n] : 0.f;
    }

    // staging registers: XV vectors of 8 channels of x and delta, BCV groups of 4 B and C entries
    Vec8<T> xr[SH::XV];
    float4 dr[SH::XV][2];
    float br[SH::BCV][4], cr[SH::BCV][4];
    const T* xb = x + b * seqlen * (int64_t)dim;
    const float* db = delta + b * seqlen * (int64_t)dim;
    const T* bb = Bm + b * seqlen * (int64_t)N;
    const T* cbp = Cm + b * seqlen * (int64_t)N;

    auto load_block = [&](int t0) {
#pragma unroll
        for (int v = 0; v < SH::XV; ++v) {
            const int e = (v * kThreads + tid) * kVec;
            const int t = min(t0 + e / CPW, seqlen - 1);
            const int cc = min(c0 + e % CPW, dim - kVec);
            load8(xr[v], xb + (int64_t)t * dim + cc);
            const float4* dp = reinterpret_cast<const float4*>(db + (int64_t)t * dim + cc);
            dr[v][0] = dp[0];
            dr[v][1] = dp[1];
        }
#pragma unroll
        for (int v = 0; v < SH::BCV; ++v) {
            const int e = min((v * kThreads + tid) * 4, SH::BCE - 4);
            const int t = min(t0 + e / N, seqlen - 1);
            const int64_t off = (int64_t)t * N + e % N;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                br[v][k] = to_f32(bb[off + k]);
                cr[v][k] = to_f32(cbp[off + k]);
            }
        }
    };
    // tokens past the sequence get delta = 0 and delta*x = 0: their step leaves h unchanged
    // (decay exp(0) = 1, no input), so every block runs TB steps
    auto store_block = [&](int t0) {
#pragma unroll
        for (int v = 0; v < SH::XV; ++v) {
            const int e = (v * kThreads + tid) * kVec;
            const int t = e / CPW, cc = e % CPW;
            const bool in_seq = t0 + t < seqlen;
            float xv[kVec];
#pragma unroll
            for (int k = 0; k < kVec; ++k) xv[k] = in_seq ? xr[v].get(k) : 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float4 d4 = in_seq ? dr[v][q] : make_float4(0.f, 0.f, 0.f, 0.f);
                const float* x4 = xv + 4 * q;
                *reinterpret_cast<float4*>(&xs[t][cc + 4 * q]) = make_float4(x4[0], x4[1], x4[2], x4[3]);
                *reinterpret_cast<float4*>(&dls[t][cc + 4 * q]) = d4;
                *reinterpret_cast<float4*>(&us[t][cc + 4 * q]) =
                    make_float4(d4.x * x4[0], d4.y * x4[1], d4.z * x4[2], d4.w * x4[3]);
            }
        }
#pragma unroll
        for (int v = 0; v < SH::BCV; ++v) {
            const int e = (v * kThreads + tid) * 4;
            if (e < SH::BCE) {
                const int t = e / N, n = e % N;
                *reinterpret_cast<float4*>(&bs[t][n]) = make_float4(br[v][0], br[v][1], br[v][2], br[v][3]);
                *reinterpret_cast<float4*>(&cs[t][n]) = make_float4(cr[v][0], cr[v][1], cr[v][2], cr[v][3]);
            }
        }
    };

    // skip weights of the channels this thread writes y for (fixed over the blocks)
    float dskip[SH::XV][kVec];
#pragma unroll
    for (int v = 0; v < SH::XV; ++v) {
        const int cc = ((v * kThreads + tid) * kVec) % CPW;
#pragma unroll
        for (int q = 0; q < kVec; ++q) dskip[v][q] = Dv[min(c0 + cc + q, dim - 1)];
    }

    const int nblk = (seqlen + TB - 1) / TB;
    if (nblk > 0) load_block(0);
    for (int k = 0; k < nblk; ++k) {
        const int t0 = k * TB;
        __syncthreads();                       // the previous block's LDS reads are done
        store_block(t0);
        __syncthreads();
        if (k + 1 < nblk) load_block(t0 + TB);
        const int nt = min(TB, seqlen - t0);
#pragma unroll 4
        for (int t = 0; t < TB; ++t) {
            const float dl = dls[t][ch];
            const float u = us[t][ch];
            float part = 0.f;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int n = sub * S + s;
                const float a = __builtin_amdgcn_exp2f(dl * a2[s]);
                h[s] = fmaf(a, h[s], u * bs[t][n]);
                part = fmaf(cs[t][n], h[s], part);
            }
            // all W lanes of the channel hold the sum and store it to the same word (no branch)
            ys[t][ch] = lane_group_sum<W>(part);
        }
        __syncthreads();
        // y of the block: readout plus the skip term, 8 channels per 16-byte store
#pragma unroll
        for (int v = 0; v < SH::XV; ++v) {
            const int e = (v * kThreads + tid) * kVec;
            const int t = e / CPW, cc = e % CPW;
            if (t < nt && c0 + cc < dim) {
                Vec8<T> o;
#pragma unroll
                for (int q = 0; q < kVec; ++q) o.set(q, fmaf(dskip[v][q], xs[t][cc + q], ys[t][cc + q]));
                store8(y + (b * seqlen + t0 + t) * (int64_t)dim + c0 + cc, o);
            }
        }
    }
    if (live) {
#pragma unroll
        for (int s = 0; s < S; ++s) final_states[(b * dim + c) * N + sub * S + s] = h[s];
    }
}

template <typename T, int W, int S>
hipError_t launch(const T* x, const float* delta, const float* A, const T* B, const T* C, const float* D,
                  const float* init, T* y, float* final_states, int64_t batch, int64_t seqlen, int64_t dim,
                  hipStream_t stream)
{
    constexpr int CPW = ScanShape<T, W, S>::CPW;
    const int ncblk = (int)((dim + CPW - 1) / CPW);
    const int64_t nblocks = batch * ncblk;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((selective_scan_kernel<T, W, S>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream, x,
                       delta, A, B, C, D, init, y, final_states, (int)seqlen, (int)dim, ncblk);
    return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_selective_scan(const T* x, const float* delta, const float* A, const T* B, const T* C,
                                 const float* D, const float* init, T* y, float* final_states, int64_t batch,
                                 int64_t seqlen, int64_t dim, int64_t dstate, hipStream_t stream)
{
    switch (dstate) {
    case 4: return launch<T, 4, 1>(x, delta, A, B, C, D, init, y, final_states, batch, seqlen, dim, stream);
    case 8: return launch<T, 8, 1>(x, delta, A, B, C, D, init, y, final_states, batch, seqlen, dim, stream);
    case 16: return launch<T, 8, 2>(x, delta, A, B, C, D, init, y, final_states, batch, seqlen, dim, stream);
    case 32: return launch<T, 8, 4>(x, delta, A, B, C, D, init, y, final_states, batch, seqlen, dim, stream);
    case 64: return launch<T, 8, 8>(x, delta, A, B, C, D, init, y, final_states, batch, seqlen, dim, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_selective_scan<float>(const float*, const float*, const float*, const float*,
                                                 const float*, const float*, const float*, float*, float*,
                                                 int64_t, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_selective_scan<bf16>(const bf16*, const float*, const float*, const bf16*,
                                                const bf16*, const float*, const float*, bf16*, float*,
                                                int64_t, int64_t, int64_t, int64_t, hipStream_t);

}  // namespace ssd
