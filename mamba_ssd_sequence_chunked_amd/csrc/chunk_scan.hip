// chunk_scan.hip - stage 4: the output of every chunk.
//
//   y[l, p] = sum_{s <= l} G[l, s] x[s, p]  +  exp(cs[l]) sum_n C[l, n] S_in[p, n]  +  D x[l, p]
//   G[l, s] = (C_l . B_s) * exp(cs[l] - cs[s]) * dt_s
//
// The first term is the quadratic, attention-like form of the SSM restricted
// to one chunk (the masked matrix of the mohakchugh blog, sections "The
// Duality" and "The Tensor Core Connection"); the second reads out the state
// entering the chunk, decayed to position l (that blog's block-decomposition
// outline adds it before the state moves on); the third is the skip term.
//
// Workgroup = (batch, chunk, head, 64-row tile of the chunk); 4 wavefronts,
// each owning 16 rows x all P columns of y.  Everything runs on the matrix
// cores with fp32 accumulation:
//   * C rows of a wavefront are read once from global memory straight into
//     operand fragments (the state axis is contiguous, which is the
//     contraction axis of both C.B^T and C.S^T) and kept in registers.
//   * inter term: S_in is staged through LDS 64 state columns at a time and
//     multiplied against those fragments; rows are scaled by exp(cs[l]).
//   * intra term, 32 source tokens at a time: G^T (tokens x rows) = B_s C^T
//     comes out of the matrix core with each lane holding 4 consecutive
//     source tokens of one row; two such tiles are exactly one A operand for
//     G @ X_s once the 32 contraction slots are assigned to tokens in the
//     same order on the X side, so G never leaves registers.  The decay and
//     causal mask are applied in fp32 between the two products (entries above
//     the diagonal are selected to zero, never multiplied), then rounded once
//     to T.
//   * y tiles are staged through LDS so every store, and the x read of the
//     skip term, is a 16-byte vector access along the head dimension.
// Workgroups are numbered row-tile fastest, then head, then chunk, and
// renumbered so that consecutive ones share an XCD and its L2 (the row
// tiles of a (chunk, head) re-read the same x, B and S_in; the heads of a
// group the same B and C).
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kRows = 64;     // rows of y per workgroup
constexpr int kSB = 32;       // source tokens per intra step
constexpr int kSlab = 64;     // state columns of S_in per LDS stage
constexpr int kMaxQ = 256;

template <typename T, int P, int NK>
struct ScanSmem {
    static constexpr int NP = 32 * NK;                           // padded state width
    static constexpr int bs_pitch = NP + 8;
    static constexpr int xt_pitch = kSB + 8;
    static constexpr int ss_pitch = kSlab + 8;
    static constexpr int out_pitch = P + 4;
    static constexpr size_t bs_bytes = sizeof(T) * kSB * bs_pitch;
    static constexpr size_t xt_bytes = sizeof(T) * P * xt_pitch;
    static constexpr size_t ss_bytes = sizeof(T) * P * ss_pitch;
    static constexpr size_t out_bytes = sizeof(float) * kRows * out_pitch;
    static constexpr size_t m1 = ss_bytes > bs_bytes + xt_bytes ? ss_bytes : bs_bytes + xt_bytes;
    static constexpr size_t region = m1 > out_bytes ? m1 : out_bytes;
    static constexpr size_t total = 2 * sizeof(float) * kMaxQ + region;
};

template <typename T, int P, int NK>
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ dt_chunked, const float* __restrict__ dA_cs,
    const T* __restrict__ entry, const float* __restrict__ Dv, T* __restrict__ y, int seqlen,
    int nheads, int ngroups, int N, int Q, int nc, int nlt, int nblocks)
{
    using S = ScanSmem<T, P, NK>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::total];
    float* cs_s = reinterpret_cast<float*>(smem);
    float* dt_s = cs_s + kMaxQ;
    unsigned char* region = smem + 2 * sizeof(float) * kMaxQ;
    T* SS = reinterpret_cast<T*>(region);                       // inter phase
    T* BS = reinterpret_cast<T*>(region);                       // intra phase
    T* XT = reinterpret_cast<T*>(region + S::bs_bytes);         // intra phase
    float* OUT = reinterpret_cast<float*>(region);              // epilogue

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int lt = id % nlt; id /= nlt;
    const int h = id % nheads; id /= nheads;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int g = h / (nheads / ngroups);
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);
    const int row0 = lt * kRows;

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;
    const int lw0 = row0 + 16 * wave;                 // first row of this wavefront
    const int lrow = lw0 + r16;                       // the row this lane feeds into the products

    const int64_t dbase = (((int64_t)b * nheads + h) * nc + c) * Q;
    for (int i = tid; i < kMaxQ; i += 256) {
        cs_s[i] = i < Q ? dA_cs[dbase + i] : 0.f;
        dt_s[i] = i < Q ? dt_chunked[dbase + i] : 0.f;
    }

    // C rows of this wavefront as operand fragments (state axis = contraction slots).
    Vec8<T> cf[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
        const int n = 32 * ks + 8 * grp;
        if (lrow < len && n < N)
            load8(cf[ks], Cm + ((b * seqlen + t0 + lrow) * ngroups + g) * N + n);
        else
            cf[ks].zero();
    }

    f32x4 acc[P / 16];
#pragma unroll
    for (int i = 0; i < P / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- inter-chunk term: exp(cs[l]) * C_l . S_in[p, :]
    {
        f32x4 ai[P / 16];
#pragma unroll
        for (int i = 0; i < P / 16; ++i) ai[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        const T* ent = entry + (((int64_t)b * nc + c) * nheads + h) * (int64_t)P * N;
        constexpr int nslab = (NK + 1) / 2;
#pragma unroll
        for (int sl = 0; sl < nslab; ++sl) {
            __syncthreads();
            for (int i = tid; i < P * (kSlab / 8); i += 256) {
                const int p = i / (kSlab / 8), o = i % (kSlab / 8);
                const int n = sl * kSlab + 8 * o;
                Vec8<T> v;
                if (n < N) load8(v, ent + (int64_t)p * N + n);
                else v.zero();
                store8(SS + p * S::ss_pitch + 8 * o, v);
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ks = 2 * sl + kk;
                if (ks < NK) {
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> bf;
                        load8(bf, SS + (16 * pt + r16) * S::ss_pitch + 32 * kk + 8 * grp);
                        mma(ai[pt], cf[ks], bf);
                    }
                }
            }
        }
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = __expf(cs_s[lw0 + 4 * grp + j]);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[pt][j] += sc[j] * ai[pt][j];
    }

    // ---- intra-chunk term: sum_{s <= l} G[l, s] x[s, :]
    const int s_end = min(len, row0 + kRows);
    const float cl = cs_s[lrow];
    for (int s0 = 0; s0 < s_end; s0 += kSB) {
        __syncthreads();
        constexpr int nXb = (kSB / 4) * (P / 8);
        const int nBb = kSB * ((N + 7) / 8);
        for (int i = tid; i < nXb + nBb; i += 256) {
            if (i < nXb) {
                const int q = i / (P / 8), o = i % (P / 8);
                float v[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = s0 + 4 * q + r;
                    Vec8<T> row;
                    if (s < len) load8(row, x + ((b * seqlen + t0 + s) * nheads + h) * P + 8 * o);
                    else row.zero();
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[r][e] = row.get(e);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    store4(XT + (8 * o + e) * S::xt_pitch + 4 * q, v[0][e], v[1][e], v[2][e], v[3][e]);
            } else {
                const int j = i - nXb;
                const int r = j / ((N + 7) / 8), o = j % ((N + 7) / 8);
                const int s = s0 + r;
                Vec8<T> v;
                if (s < len) load8(v, Bm + ((b * seqlen + t0 + s) * ngroups + g) * N + 8 * o);
                else v.zero();
                store8(BS + r * S::bs_pitch + 8 * o, v);
            }
        }
        // zero the padded state columns N .. 32*NK of the B tile
        if (32 * NK > N) {
            const int padw = 32 * NK - N;
            for (int i = tid; i < kSB * (padw / 8); i += 256) {
                const int r = i / (padw / 8), o = i % (padw / 8);
                Vec8<T> z;
                z.zero();
                store8(BS + r * S::bs_pitch + N + 8 * o, z);
            }
        }
        __syncthreads();
        if (s0 <= lw0 + 15 && lw0 < len) {
            f32x4 gt[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                gt[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NK; ++ks) {
                    Vec8<T> af;
                    load8(af, BS + (16 * st + r16) * S::bs_pitch + 32 * ks + 8 * grp);
                    mma(gt[st], af, cf[ks]);
                }
            }
            Vec8<T> gf;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = s0 + 16 * st + 4 * grp + j;
                    const float dec = __expf(cl - cs_s[s]) * dt_s[s];
                    gf.set(4 * st + j, (s <= lrow && s < len) ? gt[st][j] * dec : 0.f);
                }
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                Vec8<T> xf;
                load4(xf, 0, XT + (16 * pt + r16) * S::xt_pitch + 4 * grp);
                load4(xf, 1, XT + (16 * pt + r16) * S::xt_pitch + 16 + 4 * grp);
                mma(acc[pt], gf, xf);
            }
        }
    }

    // ---- epilogue: y = acc + D x, staged through LDS for 16-byte accesses
    __syncthreads();
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
        for (int j = 0; j < 4; ++j) OUT[(16 * wave + 4 * grp + j) * S::out_pitch + 16 * pt + r16] = acc[pt][j];
    __syncthreads();
    const float dh = Dv[h];
    for (int i = tid; i < kRows * (P / 8); i += 256) {
        const int r = i / (P / 8), o = i % (P / 8);
        const int l = row0 + r;
        if (l >= len) continue;
        const int64_t off = ((b * seqlen + t0 + l) * nheads + h) * P + 8 * o;
        Vec8<T> xv, yv;
        load8(xv, x + off);
        const float* src = OUT + r * S::out_pitch + 8 * o;
#pragma unroll
        for (int e = 0; e < 8; ++e) yv.set(e, src[e] + dh * xv.get(e));
        store8(y + off, yv);
    }
}

template <typename T, int P, int NK>
hipError_t launch(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                  const float* D, T* y, const Dims& d, hipStream_t stream)
{
    const int nc = (int)d.nchunks();
    const int nlt = (int)((d.chunk + kRows - 1) / kRows);
    const int64_t nblocks = d.batch * nc * d.nheads * nlt;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_scan_kernel<T, P, NK>), dim3((unsigned)nblocks), dim3(256), 0, stream, x, B,
                       C, dtc, cs, entry, D, y, (int)d.seqlen, (int)d.nheads, (int)d.ngroups,
                       (int)d.dstate, (int)d.chunk, nc, nlt, (int)nblocks);
    return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_p(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                    const float* D, T* y, const Dims& d, hipStream_t stream)
{
    const int64_t nk = (d.dstate + 31) / 32;
    if (nk <= 1) return launch<T, P, 1>(x, B, C, dtc, cs, entry, D, y, d, stream);
    if (nk <= 2) return launch<T, P, 2>(x, B, C, dtc, cs, entry, D, y, d, stream);
    if (nk <= 4) return launch<T, P, 4>(x, B, C, dtc, cs, entry, D, y, d, stream);
    return launch<T, P, 8>(x, B, C, dtc, cs, entry, D, y, d, stream);
}

}  // namespace

template <typename T>
hipError_t launch_chunk_scan(const T* x, const T* B, const T* C, const float* dt_chunked,
                             const float* dA_cs, const T* entry_states, const float* D, T* y,
                             const Dims& d, hipStream_t stream)
{
    switch (d.headdim) {
    case 16: return launch_p<T, 16>(x, B, C, dt_chunked, dA_cs, entry_states, D, y, d, stream);
    case 32: return launch_p<T, 32>(x, B, C, dt_chunked, dA_cs, entry_states, D, y, d, stream);
    case 64: return launch_p<T, 64>(x, B, C, dt_chunked, dA_cs, entry_states, D, y, d, stream);
    case 128: return launch_p<T, 128>(x, B, C, dt_chunked, dA_cs, entry_states, D, y, d, stream);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch_chunk_scan<float>(const float*, const float*, const float*, const float*,
                                             const float*, const float*, const float*, float*,
                                             const Dims&, hipStream_t);
template hipError_t launch_chunk_scan<bf16>(const bf16*, const bf16*, const bf16*, const float*,
                                            const float*, const bf16*, const float*, bf16*,
                                            const Dims&, hipStream_t);

}  // namespace ssd
