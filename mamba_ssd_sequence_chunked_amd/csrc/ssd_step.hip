// ssd_step.hip - the recurrent mode: one token per call, state updated in place.
//
//   a = exp(dt A);   S[p, n] = a S[p, n] + (dt x[p]) B[n];   y[p] = sum_n C[n] S[p, n] + D x[p]
//
// The linear-time form of the same operator, the one used for generation
// (mohakchugh blog, section "Why This Matters for Hardware"): constant work
// and memory per token ("Transformers are SSMs" paper card, "Why It
// Matters").  The whole fp32 state is read and written once per token and
// there are 3 flops per state element, so the kernel is bound by HBM
// bandwidth; it does exactly one pass.
//
// Workgroup = one (batch, head): its P x N state block is contiguous.  A
// thread owns 4 consecutive state columns (one 16-byte vector) of every
// (256 / (N/4))-th row; all of its rows are loaded before any arithmetic so
// a thread keeps several 16-byte loads in flight.  B, C, x and the scalars
// are read once into registers; the readout over N is a reduction inside
// aligned groups of lanes (a power of two >= N/4; surplus lanes contribute 0).
// The state is streamed with non-temporal loads and stores: it is touched
// once per call and is larger than the last-level cache, so keeping it out
// of the caches leaves them to the small operands.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

template <typename T, int W, int P>      // W = lanes per state row (power of two, 4*W >= N)
__global__ __launch_bounds__(256) void ssd_step_kernel(
    float* __restrict__ state, const T* __restrict__ x, const float* __restrict__ dt,
    const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, T* __restrict__ y, int nheads, int N, int ngroups)
{
    constexpr int kRowsPerPass = 256 / W;
    constexpr int kPass = (P + kRowsPerPass - 1) / kRowsPerPass;
    const int bh = blockIdx.x;
    const int h = bh % nheads;
    const int b = bh / nheads;
    const int g = h / (nheads / ngroups);
    const int tid = threadIdx.x;
    const int col = 4 * (tid % W);
    const int rsub = tid / W;
    const bool colok = col < N;

    const float dtv = dt[bh];
    const float a = __expf(dtv * A[h]);
    const float dh = Dv[h];
    float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {0.f, 0.f, 0.f, 0.f};
    if (colok) {
        const T* bp = Bm + ((int64_t)b * ngroups + g) * N + col;
        const T* cp = Cm + ((int64_t)b * ngroups + g) * N + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) { bv[e] = to_f32(bp[e]); cv[e] = to_f32(cp[e]); }
    }
    float* S = state + (int64_t)bh * P * N;
    const T* xr = x + (int64_t)bh * P;
    T* yr = y + (int64_t)bh * P;
    float4 s[kPass];
    float xv[kPass];
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
        const int p = k * kRowsPerPass + rsub;
        const bool live = p < P;
        xv[k] = live ? to_f32(xr[p]) : 0.f;
        f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (live && colok) t4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (int64_t)p * N + col));
        s[k] = make_float4(t4[0], t4[1], t4[2], t4[3]);
    }
#pragma unroll
    for (int k = 0; k < kPass; ++k) {
        const int p = k * kRowsPerPass + rsub;
        const bool live = p < P;
        const float u = dtv * xv[k];
        float4 v = s[k];
        v.x = fmaf(a, v.x, u * bv[0]);
        v.y = fmaf(a, v.y, u * bv[1]);
        v.z = fmaf(a, v.z, u * bv[2]);
        v.w = fmaf(a, v.w, u * bv[3]);
        if (live && colok) __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(S + (int64_t)p * N + col));
        float part = (live && colok) ? cv[0] * v.x + cv[1] * v.y + cv[2] * v.z + cv[3] * v.w : 0.f;
        part = group_sum<W>(part);
        if ((tid % W) == 0 && live) yr[p] = from_f32<T>(part + dh * xv[k]);
    }
}

template <typename T, int W, int P>
hipError_t launch(float* state, const T* x, const float* dt, const float* A, const T* B, const T* C,
                  const float* D, T* y, const Dims& d, hipStream_t stream)
{
    const int64_t nblocks = d.batch * d.nheads;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((ssd_step_kernel<T, W, P>), dim3((unsigned)nblocks), dim3(256), 0, stream, state, x,
                       dt, A, B, C, D, y, (int)d.nheads, (int)d.dstate, (int)d.ngroups);
    return hipGetLastError();
}

template <typename T, int W>
hipError_t launch_w(float* state, const T* x, const float* dt, const float* A, const T* B, const T* C,
                    const float* D, T* y, const Dims& d, hipStream_t stream)
{
    switch (d.headdim) {
    case 16: return launch<T, W, 16>(state, x, dt, A, B, C, D, y, d, stream);
    case 32: return launch<T, W, 32>(state, x, dt, A, B, C, D, y, d, stream);
    case 64: return launch<T, W, 64>(state, x, dt, A, B, C, D, y, d, stream);
    case 128: return launch<T, W, 128>(state, x, dt, A, B, C, D, y, d, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

template <typename T>
hipError_t launch_ssd_step(float* state, const T* x, const float* dt, const float* A, const T* B,
                           const T* C, const float* D, T* y, const Dims& d, hipStream_t stream)
{
    const int64_t q = d.dstate / 4;
    if (q <= 4) return launch_w<T, 4>(state, x, dt, A, B, C, D, y, d, stream);
    if (q <= 8) return launch_w<T, 8>(state, x, dt, A, B, C, D, y, d, stream);
    if (q <= 16) return launch_w<T, 16>(state, x, dt, A, B, C, D, y, d, stream);
    if (q <= 32) return launch_w<T, 32>(state, x, dt, A, B, C, D, y, d, stream);
    return launch_w<T, 64>(state, x, dt, A, B, C, D, y, d, stream);
}

template hipError_t launch_ssd_step<float>(float*, const float*, const float*, const float*,
                                           const float*, const float*, const float*, float*,
                                           const Dims&, hipStream_t);
template hipError_t launch_ssd_step<bf16>(float*, const bf16*, const float*, const float*, const bf16*,
                                          const bf16*, const float*, bf16*, const Dims&, hipStream_t);

}  // namespace ssd
