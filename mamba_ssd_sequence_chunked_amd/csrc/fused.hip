// fused.hip - the chunked forward as one pass over the sequence per (batch, head).
//
// The block-decomposition outline of the mohakchugh blog (section "Block Decomposition: The
// Hardware-Aware Algorithm")
// walks the chunks in order: each chunk's output is its quadratic, attention-like part plus the
// state that enters it read out through C, and the state then moves on to the next chunk
// (ql.gl, "The Core of SSD").  Here one workgroup per (batch, head, head-dimension slice) does
// exactly that, over blocks of 32 tokens, with the state kept on chip for the whole sequence -- no
// chunk states, entry states or cumulative sums go through memory and no workspace is needed:
//
//   cs[l]  = sum_{j <= l} dt_j A           (within the block)
//   y_l    = exp(cs[l]) S C_l  +  sum_{s <= l} (C_l . B_s) exp(cs[l] - cs[s]) dt_s x_s  +  D x_l
//   S     <- exp(cs[last]) S  +  sum_s x_s (dt_s exp(cs[last] - cs[s])) B_s^T
//
// The result is the chunked method's (the decomposition is exact; only the block size and the
// order of the sums differ), the same roundings included: products on the matrix cores with fp32
// sums, the decayed scores and the state rounded to the operand type where they enter a product,
// the running state itself in fp32.  All three products run on the matrix cores:
//   * G^T (tokens s x token l) = B C^T once per block, decayed and masked in fp32; in the
//     accumulator layout it is already the B operand of y^T = X^T G^T (the X fragments are read with
//     the same slot order: slots 0-3 hold tokens 4 grp + m, slots 4-7 tokens 16 + 4 grp + m)
//   * the state readout S C^T from a copy of the state rounded to the operand type in LDS
//   * the state update S^T += (w B)^T X straight into the accumulators that hold S^T
// A workgroup is 4 wavefronts: wavefront w computes y for the block's tokens 16 (w & 1) .. +15
// and the head-dimension tiles (w >> 1) + 2 i, and holds the state columns n in tiles w + 4 i.
// This trades the chunked kernels' parallelism over chunks for a sequential walk: batch x heads x
// slices workgroups, each stepping through seqlen / 32 blocks.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kTB = 32;          // tokens per block
constexpr int kMinSlice = 32;    // narrowest head-dimension slice per workgroup
constexpr int kThreads = 256;

template <typename T, int P, int NP>
__global__ __launch_bounds__(kThreads) void ssd_fused_kernel(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dv, const float* __restrict__ init, T* __restrict__ y,
    float* __restrict__ final_states, int seqlen, int nheads, int ngroups, int N, int hd)
{
    constexpr int XP = tr_pitch<T>(P), NPP = tr_pitch<T>(NP);   // padded LDS rows (elements)
    constexpr int PT = P / 16, NT = NP / 16, KN = NP / 32;
    constexpr int YT = (PT + 1) / 2;                 // head-dimension tiles of y per wavefront
    constexpr int NTW = (NT + 3) / 4;                // state column tiles per wavefront
    constexpr int EV = 16 / (int)sizeof(T);          // elements per 16-byte access
    __shared__ __attribute__((aligned(16))) T xs[kTB * XP];
    __shared__ __attribute__((aligned(16))) T bs[kTB * NPP];
    __shared__ __attribute__((aligned(16))) T cs_[kTB * NPP];
    __shared__ __attribute__((aligned(16))) T sp[P * NPP];           // the state rounded to T, rows p
    // per-block tables, two sets: wavefront 0 fills the next block's while the others use the current
    __shared__ float cum[2][kTB], ecs[2][kTB], wv[2][kTB], dtv[2][kTB];

    // P is the width of the head-dimension slice this workgroup owns (hd / P slices per head): y and
    // the state rows of one slice depend on that slice of x only, so slices are independent and
    // each recomputes the block's scores.  Consecutive slices and heads run on one XCD (shared L2).
    const int nsl = hd / P, lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int bh = lb / nsl, p0 = (lb % nsl) * P, h = bh % nheads;
    const int64_t b = bh / nheads;
    const int g = h / (nheads / ngroups);
    const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float a = A[h], dsk = Dv[h];

    // S^T accumulators: sacc[i][pt] holds, per lane, p = 16 pt + r16 and n = 16 (wu + 4 i) + 4 grp + q
    f32x4 sacc[NTW][PT];
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int nt = wu + 4 * i, n = 16 * nt + 4 * grp;
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
            if (init && nt < NT && n < N)
                v = *reinterpret_cast<const f32x4*>(init + ((int64_t)bh * hd + p0 + 16 * pt + r16) * N + n);
            sacc[i][pt] = v;
        }
    auto put_state = [&]() {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int nt = wu + 4 * i;
            if (nt < NT) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    T* d = sp + (16 * pt + r16) * NPP + 16 * nt + 4 * grp;
#pragma unroll
                    for (int q = 0; q < 4; ++q) d[q] = from_f32<T>(sacc[i][pt][q]);
                }
            }
        }
    };
    put_state();

    // The block's x, B, C rows and dt go through registers: the next block's are loaded while the
    // current one is multiplied.  Every access is one unconditional buffer instruction over a resource
    // that ends at the block's last token (rows past the sequence, state columns past N and idle lanes
    // read zeros), so the only wait before the rows are used is for these loads.
    constexpr int NXV = (kTB * P / EV + kThreads - 1) / kThreads;      // 16-byte pieces per thread
    constexpr int NBV = (kTB * NP / EV + kThreads - 1) / kThreads;
    constexpr int ES = (int)sizeof(T);
    uint4 rx[NXV], rb[NBV], rc[NBV];
    float rdt = 0.f;
    auto fetch = [&](int t0) {
        const int rows = min(kTB, seqlen - t0);
        const int64_t tok = b * seqlen + t0;
        const __amdgpu_buffer_rsrc_t rxs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(x + tok * nheads * hd), 0, rows * nheads * hd * ES, kBufferDword3);
        const __amdgpu_buffer_rsrc_t rbs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(Bm + tok * ngroups * N), 0, rows * ngroups * N * ES, kBufferDword3);
        const __amdgpu_buffer_rsrc_t rcs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(Cm + tok * ngroups * N), 0, rows * ngroups * N * ES, kBufferDword3);
        const __amdgpu_buffer_rsrc_t rds = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(dt + tok * nheads), 0, rows * nheads * 4, kBufferDword3);
#pragma unroll
        for (int k = 0; k < NXV; ++k) {
            const int i = tid + k * kThreads, r = i / (P / EV), c = (i % (P / EV)) * EV;
            const int vo = i < kTB * P / EV ? ((r * nheads + h) * hd + p0 + c) * ES : kDropped;
            rx[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rxs, vo, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < NBV; ++k) {
            const int i = tid + k * kThreads, r = i / (NP / EV), c = (i % (NP / EV)) * EV;
            const int vo = i < kTB * NP / EV && c < N ? ((r * ngroups + g) * N + c) * ES : kDropped;
            rb[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rbs, vo, 0, 0));
            rc[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rcs, vo, 0, 0));
        }
        rdt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rds, tid < kTB ? (tid * nheads + h) * 4 : kDropped, 0, 0));
    };
    auto stash = [&]() {
#pragma unroll
        for (int k = 0; k < NXV; ++k) {
            const int i = tid + k * kThreads, r = i / (P / EV), c = (i % (P / EV)) * EV;
            if (i < kTB * P / EV) *reinterpret_cast<uint4*>(xs + r * XP + c) = rx[k];
        }
#pragma unroll
        for (int k = 0; k < NBV; ++k) {
            const int i = tid + k * kThreads, r = i / (NP / EV), c = (i % (NP / EV)) * EV;
            if (i < kTB * NP / EV) {
                *reinterpret_cast<uint4*>(bs + r * NPP + c) = rb[k];
                *reinterpret_cast<uint4*>(cs_ + r * NPP + c) = rc[k];
            }
        }
    };
    // in-block prefix sums of dt A, the readout decays exp(cs) and the state weights of the block whose
    // dt wavefront 0 holds in registers (lane j: token j), into table set u
    auto tables = [&](int u) {
        if (wu == 0) {
            const float v = lane < kTB ? rdt * a : 0.f;
            const float c = wave_inclusive_sum(v);
            const float last = __shfl(c, kTB - 1, kWave);
            if (lane < kTB) {
                cum[u][lane] = c;
                ecs[u][lane] = __expf(c);
                wv[u][lane] = rdt * __expf(last - c);
                dtv[u][lane] = rdt;
            }
        }
    };
    if (seqlen > 0) {
        fetch(0);
        tables(0);
    }
    for (int t0 = 0, u = 0; t0 < seqlen; t0 += kTB, u ^= 1) {
        stash();
        if (t0 + kTB < seqlen) fetch(t0 + kTB);
        __syncthreads();                                 // this block's tiles, tables and state copy are in LDS
        const float* cum_ = cum[u];
        const float* ecs_ = ecs[u];
        const float* wv_ = wv[u];
        const float* dtv_ = dtv[u];
        const float elast = __expf(cum_[kTB - 1]);

        // ---- y of the wavefront's tokens l = 16 lt + r16 (the lane's column) and head-dimension tiles
        const int lt = wu & 1, l = 16 * lt + r16;
        Vec8<T> gf;                                      // G^T[s][l], slot order as in the header
        {
            f32x4 d0 = f32x4{0.f, 0.f, 0.f, 0.f}, d1 = d0;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
                Vec8<T> cf, b0, b1;
                load8(cf, cs_ + l * NPP + 32 * kk + 8 * grp);
                load8(b0, bs + r16 * NPP + 32 * kk + 8 * grp);
                load8(b1, bs + (16 + r16) * NPP + 32 * kk + 8 * grp);
                mma(d0, b0, cf);
                mma(d1, b1, cf);
            }
            const float cl = cum_[l];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int s0 = 4 * grp + q, s1 = 16 + s0;
                gf.set(q, select(s0 <= l, d0[q] * (__expf(fminf(cl - cum_[s0], 0.f)) * dtv_[s0]), 0.f));
                gf.set(4 + q, select(s1 <= l, d1[q] * (__expf(fminf(cl - cum_[s1], 0.f)) * dtv_[s1]), 0.f));
            }
        }
        const float el = ecs_[l];
        // y rows of this block; rows past the sequence fall outside the resource and are dropped
        const __amdgpu_buffer_rsrc_t rys = __builtin_amdgcn_make_buffer_rsrc(
            y + (b * seqlen + t0) * nheads * hd, 0, min(kTB, seqlen - t0) * nheads * hd * ES, kBufferDword3);
#pragma unroll
        for (int i = 0; i < YT; ++i) {
            const int pt = (wu >> 1) + 2 * i;
            if (pt < PT) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    Vec8<T> sf, cf;
                    load8(sf, sp + (16 * pt + r16) * NPP + 32 * kk + 8 * grp);
                    load8(cf, cs_ + l * NPP + 32 * kk + 8 * grp);
                    mma(acc, sf, cf);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] *= el;
                Vec8<T> xf;
                load_row_slots(xf, xs, XP, 0, 16 * pt);
                mma(acc, xf, gf);
                const int p = 16 * pt + 4 * grp;
                const T* xr = xs + l * XP + p;
                const f32x4 o = f32x4{acc[0] + dsk * to_f32(xr[0]), acc[1] + dsk * to_f32(xr[1]),
                                      acc[2] + dsk * to_f32(xr[2]), acc[3] + dsk * to_f32(xr[3])};
                buffer_store4(rys, ((l * nheads + h) * hd + p0 + p) * ES, 0, o, T());
            }
        }

        // ---- the state: S^T (n x p) <- exp(cs[last]) S^T + (w B)^T X over the block's tokens (slots as for
        // the X fragments above: tokens 4 grp + m and 16 + 4 grp + m)
        float wsl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wsl[e] = wv_[(e < 4 ? 0 : 16) + 4 * grp + (e & 3)];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            Vec8<T> xb;
            load_row_slots(xb, xs, XP, 0, 16 * pt);
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int nt = wu + 4 * i;
                if (nt < NT) {
                    Vec8<T> wb;
                    load_row_slots(wb, bs, NPP, 0, 16 * nt);
#pragma unroll
                    for (int e = 0; e < 8; ++e) wb.set(e, wb.get(e) * wsl[e]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) sacc[i][pt][q] *= elast;
                    mma(sacc[i][pt], wb, xb);
                }
            }
        }
        if (t0 + kTB < seqlen) tables(u ^ 1);           // the other set was last read before this block's barrier
        __syncthreads();                                 // every read of this block's tiles and state is done
        put_state();                                     // (read after the next block's barrier)
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int nt = wu + 4 * i, n = 16 * nt + 4 * grp;
        if (nt < NT && n < N) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *reinterpret_cast<f32x4*>(final_states + ((int64_t)bh * hd + p0 + 16 * pt + r16) * N + n) = sacc[i][pt];
        }
    }
}

template <typename T, int P, int NP>
hipError_t launch(const T* x, const float* dt, const float* A, const T* B, const T* C, const float* D,
                  const float* init, T* y, float* final_states, const Dims& d, hipStream_t s)
{
    const int64_t nblocks = d.batch * d.nheads * (d.headdim / P);
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((ssd_fused_kernel<T, P, NP>), dim3((unsigned)nblocks), dim3(kThreads), 0, s, x, dt, A, B, C,
                       D, init, y, final_states, (int)d.seqlen, (int)d.nheads, (int)d.ngroups, (int)d.dstate,
                       (int)d.headdim);
    return hipGetLastError();
}

}  // namespace

int fused_state_width(int64_t dstate) { return dstate <= 32 ? 32 : dstate <= 64 ? 64 : dstate <= 128 ? 128 : 256; }

bool fused_supported(const Dims& d) { return d.headdim * fused_state_width(d.dstate) <= 16384; }

// Head-dimension slice per workgroup: a workgroup per (batch, head) is too little parallelism on
// 256 CUs, so wide heads are split until there are enough workgroups (each slice recomputes the
// block's C.B^T, a small share of its work).
static int fused_slice_width(const Dims& d)
{
    int w = (int)d.headdim;
    while (w > kMinSlice && d.batch * d.nheads * (d.headdim / w) < 1024) w /= 2;
    return w;
}

template <typename T>
hipError_t launch_ssd_fused(const T* x, const float* dt, const float* A, const T* B, const T* C, const float* D,
                            const float* init, T* y, float* final_states, const Dims& d, hipStream_t s)
{
    const int np = fused_state_width(d.dstate), pw = fused_slice_width(d);
#define SSD_FUSED_CASE(PP, NN) \
    if (pw == PP && np == NN) return launch<T, PP, NN>(x, dt, A, B, C, D, init, y, final_states, d, s);
#define SSD_FUSED_P(PP) SSD_FUSED_CASE(PP, 32) SSD_FUSED_CASE(PP, 64) SSD_FUSED_CASE(PP, 128)
    SSD_FUSED_P(16) SSD_FUSED_P(32) SSD_FUSED_P(64) SSD_FUSED_P(128)
    SSD_FUSED_CASE(16, 256) SSD_FUSED_CASE(32, 256) SSD_FUSED_CASE(64, 256)
#undef SSD_FUSED_P
#undef SSD_FUSED_CASE
    return hipErrorInvalidValue;
}

template hipError_t launch_ssd_fused<float>(const float*, const float*, const float*, const float*, const float*,
                                            const float*, const float*, float*, float*, const Dims&, hipStream_t);
template hipError_t launch_ssd_fused<bf16>(const bf16*, const float*, const float*, const bf16*, const bf16*,
                                           const float*, const float*, bf16*, float*, const Dims&, hipStream_t);

}  // namespace ssd
