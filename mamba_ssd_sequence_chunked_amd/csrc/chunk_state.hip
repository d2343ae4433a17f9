// chunk_state.hip - stage 2: the state every chunk reaches from a zero state.
//
//   S_c[p, n] = sum_l x[l, p] * w_l * B[l, n],   w_l = dt_l * exp(cs[Q-1] - cs[l])
//
// i.e. the rank-N factor of the off-diagonal blocks of the semiseparable
// mixing matrix ("Mamba-2" wiki note, section "Structured Semiseparable
// Matrices"), the quantity a chunk hands to the recurrence between chunks
// (ql.gl, "The Core of SSD").  Per (chunk, head) it is a (P x Q) @ (Q x N)
// contraction over the chunk's tokens, run on the matrix cores with fp32
// accumulation.
//
// Workgroup = (batch, chunk, head), all N state columns; 4 wavefronts, each
// owning every 4th 16-column tile of S_c x all P rows.  Tokens are the
// contraction axis of both operands but the slow axis in memory: x and B are
// staged through LDS in their natural (token, column) order, 64 tokens at a
// time, and both operands are read with the gfx950 LDS transpose read, which
// delivers 8 consecutive-token slots per lane.  w_l is computed once per
// chunk into LDS and applied to the B fragment in fp32 before it is rounded
// to the operand type.  The next 64 tokens are loaded into registers while
// the current ones are multiplied; those loads are unconditional (indices
// clamped) and masks are applied when writing LDS.
//
// Workgroups are numbered head-fastest within a chunk and renumbered so
// consecutive ones share an XCD: the heads of a group read the same B tile
// from that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kKB = 64;       // tokens per LDS stage
constexpr int kMaxQ = 256;

template <typename T, int P, int NT>     // NT = 16-column tiles per wavefront (4 * 16 * NT >= N)
struct StateSmem {
    static constexpr int NW = 64 * NT;                  // padded state width
    static constexpr int x_pitch = tr_pitch<T>(P);
    static constexpr int b_pitch = tr_pitch<T>(NW);
    static constexpr int x_n = kKB * P / 8;             // 8-element items per stage
    static constexpr int b_n = kKB * NW / 8;
    static constexpr int x_items = (x_n + 255) / 256;
    static constexpr int b_items = (b_n + 255) / 256;
};

template <typename T, int P, int NT>
__global__ __launch_bounds__(256, 2) void chunk_state_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ dt_chunked,
    const float* __restrict__ dA_cs, float* __restrict__ chunk_states, int seqlen, int nheads,
    int ngroups, int N, int Q, int nc, int nblocks)
{
    using S = StateSmem<T, P, NT>;
    __shared__ __attribute__((aligned(16))) T XS[kKB * S::x_pitch];
    __shared__ __attribute__((aligned(16))) T BS[kKB * S::b_pitch];
    __shared__ __attribute__((aligned(16))) float ws[kMaxQ + kKB];

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int h = id % nheads; id /= nheads;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int g = h / (nheads / ngroups);
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;

    const int64_t dbase = (((int64_t)b * nheads + h) * nc + c) * Q;
    const float cs_last = dA_cs[dbase + Q - 1];
    for (int l = tid; l < kMaxQ + kKB; l += 256) {
        const int lc = min(l, Q - 1);
        const float w = dt_chunked[dbase + lc] * __expf(cs_last - dA_cs[dbase + lc]);
        ws[l] = select(l < len, w, 0.f);
    }

    f32x4 acc[NT][P / 16];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[j][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    Vec8<T> px[S::x_items], pb[S::b_items];
    auto fetch = [&](int l0) {
#pragma unroll
        for (int k = 0; k < S::x_items; ++k) {
            const int i = min(tid + 256 * k, S::x_n - 1);
            const int r = i / (P / 8), o = i % (P / 8);
            const int l = min(l0 + r, len - 1);
            load8(px[k], x + ((b * seqlen + t0 + l) * nheads + h) * P + 8 * o);
        }
#pragma unroll
        for (int k = 0; k < S::b_items; ++k) {
            const int i = min(tid + 256 * k, S::b_n - 1);
            const int r = i / (S::NW / 8), o = i % (S::NW / 8);
            const int l = min(l0 + r, len - 1);
            load8(pb[k], Bm + ((b * seqlen + t0 + l) * ngroups + g) * N + min(8 * o, N - 8));
        }
    };

    fetch(0);
    for (int l0 = 0; l0 < len; l0 += kKB) {
        __syncthreads();
#pragma unroll
        for (int k = 0; k < S::x_items; ++k) {
            const int i = tid + 256 * k;
            const int r = i / (P / 8), o = i % (P / 8);
            if (i < S::x_n) store8(XS + r * S::x_pitch + 8 * o, masked(px[k], l0 + r < len));
        }
#pragma unroll
        for (int k = 0; k < S::b_items; ++k) {
            const int i = tid + 256 * k;
            const int r = i / (S::NW / 8), o = i % (S::NW / 8);
            if (i < S::b_n) store8(BS + r * S::b_pitch + 8 * o, masked(pb[k], l0 + r < len && 8 * o < N));
        }
        __syncthreads();
        if (l0 + kKB < len) fetch(l0 + kKB);
#pragma unroll
        for (int ks = 0; ks < kKB / 32; ++ks) {
            Vec8<T> af[P / 16];
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) load_row_slots(af[pt], XS, S::x_pitch, 32 * ks, 16 * pt);
            const float4 wa = *reinterpret_cast<const float4*>(ws + l0 + 32 * ks + 4 * grp);
            const float4 wb = *reinterpret_cast<const float4*>(ws + l0 + 32 * ks + 16 + 4 * grp);
            const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int nt = wave + 4 * j;
                if (16 * nt < N) {
                    Vec8<T> bf;
                    load_row_slots(bf, BS, S::b_pitch, 32 * ks, 16 * nt);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bf.set(e, bf.get(e) * wv[e]);
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) mma(acc[j][pt], af[pt], bf);
                }
            }
        }
    }

    float* out = chunk_states + ((((int64_t)b * nc + c) * nheads + h) * P) * N;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = 16 * (wave + 4 * j) + r16;
        if (n < N) {
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                for (int q = 0; q < 4; ++q) out[(int64_t)(16 * pt + 4 * grp + q) * N + n] = acc[j][pt][q];
        }
    }
}

template <typename T, int P, int NT>
hipError_t launch(const T* x, const T* B, const float* dtc, const float* cs, float* out, const Dims& d,
                  hipStream_t stream)
{
    const int nc = (int)d.nchunks();
    const int64_t nblocks = d.batch * nc * d.nheads;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_state_kernel<T, P, NT>), dim3((unsigned)nblocks), dim3(256), 0, stream, x, B,
                       dtc, cs, out, (int)d.seqlen, (int)d.nheads, (int)d.ngroups, (int)d.dstate,
                       (int)d.chunk, nc, (int)nblocks);
    return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_p(const T* x, const T* B, const float* dtc, const float* cs, float* out, const Dims& d,
                    hipStream_t stream)
{
    if (d.dstate <= 64) return launch<T, P, 1>(x, B, dtc, cs, out, d, stream);
    if (d.dstate <= 128) return launch<T, P, 2>(x, B, dtc, cs, out, d, stream);
    return launch<T, P, 4>(x, B, dtc, cs, out, d, stream);
}

}  // namespace

template <typename T>
hipError_t launch_chunk_state(const T* x, const T* B, const float* dt_chunked, const float* dA_cs,
                              float* chunk_states, const Dims& d, hipStream_t stream)
{
    switch (d.headdim) {
    case 16: return launch_p<T, 16>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 32: return launch_p<T, 32>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 64: return launch_p<T, 64>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 128: return launch_p<T, 128>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_chunk_state<float>(const float*, const float*, const float*, const float*,
                                              float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state<bf16>(const bf16*, const bf16*, const float*, const float*,
                                             float*, const Dims&, hipStream_t);

}  // namespace ssd
