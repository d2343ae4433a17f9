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
// Workgroup = (batch, chunk, head, 64 state columns); 4 wavefronts, each
// owning 16 state columns x all P rows.  Tokens are the contraction axis but
// the slow axis in memory, so each 64-token stage is staged through LDS
// transposed (token-contiguous rows): every thread loads a 4-token x
// 8-element block with 16-byte global loads, applies w_l to x in fp32,
// rounds once to T and writes 8 token-quads.  Operand fragments are then
// single 16-byte LDS reads.  Row pitch is padded by 8 elements so the 16
// rows read by one fragment load fall in distinct banks.
//
// Workgroups are numbered head-fastest within a chunk and renumbered so
// consecutive ones share an XCD: the heads of a group read the same B tile
// from that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kKB = 64;       // tokens per LDS stage
constexpr int kNT = 64;       // state columns per workgroup
constexpr int kPad = 8;       // row padding (elements)

template <typename T, int P>
__global__ __launch_bounds__(256) void chunk_state_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const float* __restrict__ dt_chunked,
    const float* __restrict__ dA_cs, float* __restrict__ chunk_states, int seqlen, int nheads,
    int ngroups, int N, int Q, int nc, int n_ntiles, int nblocks)
{
    __shared__ __attribute__((aligned(16))) T XT[P][kKB + kPad];
    __shared__ __attribute__((aligned(16))) T BT[kNT][kKB + kPad];

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int nt = id % n_ntiles; id /= n_ntiles;
    const int h = id % nheads; id /= nheads;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int g = h / (nheads / ngroups);
    const int n0 = nt * kNT;
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;

    const int64_t dbase = (((int64_t)b * nheads + h) * nc + c) * Q;
    const float cs_last = dA_cs[dbase + Q - 1];

    f32x4 acc[P / 16];
#pragma unroll
    for (int i = 0; i < P / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int nXb = (kKB / 4) * (P / 8);
    constexpr int nBb = (kKB / 4) * (kNT / 8);

    for (int l0 = 0; l0 < len; l0 += kKB) {
        for (int i = tid; i < nXb + nBb; i += 256) {
            if (i < nXb) {
                const int q = i / (P / 8), o = i % (P / 8);
                float v[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = l0 + 4 * q + r;
                    Vec8<T> row;
                    float w = 0.f;
                    if (l < len) {
                        load8(row, x + ((b * seqlen + t0 + l) * nheads + h) * P + 8 * o);
                        w = dt_chunked[dbase + l] * __expf(cs_last - dA_cs[dbase + l]);
                    } else {
                        row.zero();
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[r][e] = row.get(e) * w;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) store4(&XT[8 * o + e][4 * q], v[0][e], v[1][e], v[2][e], v[3][e]);
            } else {
                const int j = i - nXb;
                const int q = j / (kNT / 8), o = j % (kNT / 8);
                const int n = n0 + 8 * o;
                float v[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int l = l0 + 4 * q + r;
                    Vec8<T> row;
                    if (l < len && n < N)
                        load8(row, Bm + ((b * seqlen + t0 + l) * ngroups + g) * N + n);
                    else
                        row.zero();
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[r][e] = row.get(e);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) store4(&BT[8 * o + e][4 * q], v[0][e], v[1][e], v[2][e], v[3][e]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kKB / 32; ++ks) {
            Vec8<T> bf;
            load8(bf, &BT[16 * wave + r16][32 * ks + 8 * grp]);
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                Vec8<T> af;
                load8(af, &XT[16 * pt + r16][32 * ks + 8 * grp]);
                mma(acc[pt], af, bf);
            }
        }
        __syncthreads();
    }

    const int n = n0 + 16 * wave + r16;
    if (n < N) {
        float* out = chunk_states + ((((int64_t)b * nc + c) * nheads + h) * P) * N + n;
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int j = 0; j < 4; ++j) out[(int64_t)(16 * pt + 4 * grp + j) * N] = acc[pt][j];
    }
}

template <typename T, int P>
hipError_t launch(const T* x, const T* B, const float* dtc, const float* cs, float* out, const Dims& d,
                  hipStream_t stream)
{
    const int nc = (int)d.nchunks();
    const int ntiles = (int)((d.dstate + kNT - 1) / kNT);
    const int64_t nblocks = d.batch * nc * d.nheads * ntiles;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_state_kernel<T, P>), dim3((unsigned)nblocks), dim3(256), 0, stream, x, B,
                       dtc, cs, out, (int)d.seqlen, (int)d.nheads, (int)d.ngroups, (int)d.dstate,
                       (int)d.chunk, nc, ntiles, (int)nblocks);
    return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_chunk_state(const T* x, const T* B, const float* dt_chunked, const float* dA_cs,
                              float* chunk_states, const Dims& d, hipStream_t stream)
{
    switch (d.headdim) {
    case 16: return launch<T, 16>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 32: return launch<T, 32>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 64: return launch<T, 64>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    case 128: return launch<T, 128>(x, B, dt_chunked, dA_cs, chunk_states, d, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_chunk_state<float>(const float*, const float*, const float*, const float*,
                                              float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state<bf16>(const bf16*, const bf16*, const float*, const float*,
                                             float*, const Dims&, hipStream_t);

}  // namespace ssd
