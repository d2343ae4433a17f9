// bwd_dbc.hip - dB and dC of the backward pass for bf16 inputs, with the sums over each group's
// heads taken inside the kernels.
//
// Within one chunk (tokens l, s; cs_h the head's in-chunk cumulative log-decay, dt_h its steps), let
//   M_h[l, s] = (dy_h,l . x_h,s) exp(cs_h[l] - cs_h[s]) dt_h[s]    for s <= l, else 0,
// the decayed, masked score of the quadratic form (the masked matrix of the mohakchugh blog, section
// "The Duality") with dy in the place of C.  Inside a chunk, y_h,l takes C_l and B_s (s <= l) through
// the products C_l . B_s of that form; C_l also reads out the state entering the chunk, and B_s also
// feeds the state the chunk hands on.  So for a group's B and C
//   dC[l] = sum_s M[l, s] B_s  +  sum_h exp(cs_h[l]) S_in,h^T dy_h,l
//   dB[s] = sum_l M[l, s] C_l  +  sum_h exp(cs_h[Q-1] - cs_h[s]) dt_h[s] Gout_h^T x_h,s
// with M = sum over the group's heads of M_h (one Q x Q matrix per batch, chunk and group),
// S_in,h the state entering the chunk and Gout_h the adjoint state that reaches the chunk's last
// token from later ones.  Three kernels:
//   bwd_score   M, per (batch, chunk, group, 128-row block, slice of the heads): per head, the
//               products dy x^T on the matrix cores (bf16, fp32 sums), then decay and mask in fp32
//               added into fp32 accumulators; the slices' partial sums go to workspace
//   bwd_inter   the two state terms, per (batch, chunk, group, 64-row block, half of the state
//               columns, slice of the heads; partial sums per slice): per head, the rows of dy (x)
//               scaled by their decay and rounded to bf16 as one operand, the S_in (Gout) tile
//               (bf16, the hi plane of the pair) read transposed from LDS as the other; the sum
//               over heads runs in the matrix-core accumulators
//   bwd_dbc     dC and dB of the group: M (the slices summed, split into bf16 hi + lo) times the
//               chunk's B and C tiles, plus the state terms (their slices summed), rounded to bf16
//               once
// Operands reach LDS by asynchronous global->LDS copies (XOR-swizzled tiles; the next head's
// tiles fly while the current head is multiplied) or registers by range-checked buffer loads (rows
// past the sequence read zero).  Requires headdim % 32 == 0 and chunk % 64 == 0.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kMaxQ = 256;
constexpr int kT = 256;                 // bwd_inter, bwd_dbc: 4 wavefronts (64 rows)
constexpr int kW8 = 8;                  // bwd_score: 8 wavefronts (128 rows)

// Copy rows [0, nrows) of a (rows x CH chunks) swizzled tile, row r from src(r) (a pointer to the
// row's first element; rows are clamped by the caller), over the workgroup's NW wavefronts.
template <int CH, int NW, class F>
__device__ __forceinline__ void rows_load_async(unsigned base, int nrows, int wu, int lane, F src) {
    using TL = SwzTile<CH>;
    const int ninst = nrows * CH / 64;
    for (int i = wu; i < ninst; i += NW) {
        const int pos = i * 64 + lane;
        const int r = pos / CH, slot = pos % CH;
        dma16(src(r) + 8 * (slot ^ (r & TL::kMask)), base + i * 1024u);
    }
}

// The chunk's cumulative log-decays and steps of one head, Q floats each, into LDS (one wavefront
// instruction per row; slots past Q repeat the last value and are not read).
__device__ __forceinline__ void tables_load_async(const float* cs_row, const float* dt_row, unsigned cs_lds,
                                                  unsigned dt_lds, int wu, int lane, int Q) {
    if (wu == 0) dma16(cs_row + min(4 * lane, Q - 4), cs_lds);
    if (wu == 1) dma16(dt_row + min(4 * lane, Q - 4), dt_lds);
}

// ---------------------------------------------------------------------------------------------
// M partial sums.  Wavefront w of row block rb owns rows l = 16 (8 rb + w) + r16 and the column
// tiles ct <= 8 rb + w (s < 16 (8 rb + w + 1)); the accumulator of tile ct holds, per lane, row l
// and columns s = 16 ct + 4 grp + q.  Products are formed as T[s][l] = x_s . dy_l (x rows from the
// LDS tile, dy rows in registers); for a tile wholly before the rows the decay is split at the
// tile's last token e: exp(cs[l] - cs[e]) per row times exp(cs[e] - cs[s]) dt[s] per token
// (tabulated per head), both exponents <= 0; the diagonal tile takes the full decay and the mask.
template <int P>
__global__ __launch_bounds__(64 * kW8, 1) void bwd_score_kernel(const bf16* __restrict__ x, const bf16* __restrict__ dy,
                                                          const float* __restrict__ dtc, const float* __restrict__ cs,
                                                          float* __restrict__ Mp, int batch, int64_t L, int H, int G,
                                                          int Q, int nc, int nrb, int nsl, int hps, int nblocks)
{
    constexpr int KS = P / 32, CH = P / 8;
    constexpr int kTiles = kMaxQ / 16;
    constexpr int xt_bytes = kMaxQ * P * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char xt[2][xt_bytes];
    __shared__ __attribute__((aligned(16))) float tab[2][2][kMaxQ];
    __shared__ __attribute__((aligned(16))) float vt[kMaxQ];

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int rb = id % nrb; id /= nrb;
    const int sl = id % nsl; id /= nsl;
    const int g = id % G; id /= G;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int hpg = H / G;
    const int j0 = sl * hps, j1 = min(hpg, j0 + hps);
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, L - t0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int rbl = kW8 * rb + wu;                       // this wavefront's 16-row block
    const int l = 16 * rbl + r16;
    const int nrows = min(16 * kW8 * (rb + 1), Q);        // x rows the workgroup reads

    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(dy + (b * L + t0) * H * P), 0, len * H * P * 2, kBufferDword3);
    auto load_dy = [&](int j, Vec8<bf16> (&f)[KS]) {
        const int h = g * hpg + j;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            buffer_load8(f[ks], rdy, l < len ? ((l * H + h) * P + 32 * ks + 8 * grp) * 2 : kDropped);
    };
    auto issue = [&](int j, int q) {
        const int h = g * hpg + j;
        const bf16* xs = x + ((b * L + t0) * H + h) * (int64_t)P;
        rows_load_async<CH, kW8>(lds_addr(xt[q]), nrows, wu, lane,
                                 [&](int r) { return xs + (int64_t)min(r, len - 1) * H * P; });
        const int64_t row = ((b * H + h) * nc + c) * (int64_t)Q;
        tables_load_async(cs + row, dtc + row, lds_addr(tab[q][0]), lds_addr(tab[q][1]), wu, lane, Q);
    };

    f32x4 m[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) m[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    Vec8<bf16> dyc[KS], dyn[KS];
    if (j0 < j1) {
        load_dy(j0, dyc);
        issue(j0, 0);
    }
    wait_vmem();
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
        const int q = (j - j0) & 1;
        if (j + 1 < j1) {
            load_dy(j + 1, dyn);
            issue(j + 1, q ^ 1);
        }
        const float* cst = tab[q][0];
        const float* dtt = tab[q][1];
        // per-token factor exp(cs[e] - cs[s]) dt[s], e = last token of s's 16-token tile
        for (int s = tid; s < Q; s += 64 * kW8) vt[s] = __expf(cst[(s | 15)] - cst[s]) * dtt[s];
        __syncthreads();
        const float csl = cst[min(l, Q - 1)];
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
            if (ct <= rbl) {   // (a guard, not a break: the loop unrolls and m stays in registers)
                f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Vec8<bf16> a;
                    swz_load8<CH>(a, xt[q], 16 * ct + r16, 32 * ks + 8 * grp);
                    mma(d, a, dyc[ks]);
                }
                const int s0 = 16 * ct + 4 * grp;
                if (ct < rbl) {
                    const float u = __expf(csl - cst[16 * ct + 15]);
                    const float4 v = *reinterpret_cast<const float4*>(vt + s0);
                    m[ct][0] += d[0] * (u * v.x);
                    m[ct][1] += d[1] * (u * v.y);
                    m[ct][2] += d[2] * (u * v.z);
                    m[ct][3] += d[3] * (u * v.w);
                } else {
                    const float4 c4 = *reinterpret_cast<const float4*>(cst + s0);
                    const float4 t4 = *reinterpret_cast<const float4*>(dtt + s0);
                    const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        m[ct][i] += select(s0 + i <= l, d[i] * (__expf(fminf(csl - cv[i], 0.f)) * tv[i]), 0.f);
                }
            }
        }
        wait_vmem();                 // the next head's rows and tiles
        __syncthreads();             // and every wavefront is done with this head's buffers
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dyc[ks] = dyn[ks];
    }

    // rows l < Q of the partial sum, all Q columns (zeros above the diagonal)
    if (l < Q) {
        float* mr = Mp + ((((int64_t)sl * batch + b) * nc + c) * G + g) * (int64_t)Q * Q + (int64_t)l * Q;
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
            if (16 * ct < Q) {
                const f32x4 v = ct <= rbl ? m[ct] : f32x4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4*>(mr + 16 * ct + 4 * grp) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// The state terms.  Wavefront w owns tokens l = 64 rb + 16 w + r16; products are formed
// transposed, D[n][l] = sum_p S^T[n][p] (e dy)[l][p], so a lane holds 4 consecutive state columns
// of its token.  S_in and Gout come as (batch, nc, H, P, N) bf16 (Gout in reversed chunk order); a
// head's (P x NH) tile is read transposed from LDS (contraction slots p = 32 ks + 4 grp + m and
// 32 ks + 16 + 4 grp + m), and the dy / x rows are loaded in the same slot order.
template <int P, int NT>
__global__ __launch_bounds__(kT, 2) void bwd_inter_kernel(const bf16* __restrict__ x, const bf16* __restrict__ dy,
                                                          const float* __restrict__ dtc, const float* __restrict__ cs,
                                                          const bf16* __restrict__ Sin, const bf16* __restrict__ Gout,
                                                          float* __restrict__ dCi, float* __restrict__ dBi, int batch,
                                                          int64_t L, int H, int G, int N, int Q, int nc, int nrb,
                                                          int nsplit, int nsl, int hps, int nblocks)
{
    constexpr int KS = P / 32, NH = 16 * NT, CHN = NH / 8;
    constexpr int tile_bytes = NH * P * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char tiles[2][2][tile_bytes];   // [buffer][S_in^T, Gout^T]
    __shared__ __attribute__((aligned(16))) float tab[2][2][kMaxQ];

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int k = id % nsplit; id /= nsplit;
    const int rb = id % nrb; id /= nrb;
    const int sl = id % nsl; id /= nsl;
    const int g = id % G; id /= G;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int hpg = H / G;
    const int j0 = sl * hps, j1 = min(hpg, j0 + hps);
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, L - t0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int l = 16 * (4 * rb + wave) + r16;
    const bool lok = l < len;

    const int64_t rbase = (b * L + t0) * H * P;
    const __amdgpu_buffer_rsrc_t rdy =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(dy + rbase), 0, len * H * P * 2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(x + rbase), 0, len * H * P * 2, kBufferDword3);
    auto load_rows = [&](int j, Vec8<bf16> (&fd)[KS], Vec8<bf16> (&fx)[KS]) {
        const int h = g * hpg + j;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int off = lok ? ((l * H + h) * P + 32 * ks + 16 * hf + 4 * grp) * 2 : kDropped;
                buffer_load4(fd[ks], hf, rdy, off);
                buffer_load4(fx[ks], hf, rx, off);
            }
    };
    auto issue = [&](int j, int q) {
        const int h = g * hpg + j;
        const bf16* sp = Sin + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N + k * NH;
        const bf16* gp = Gout + (((int64_t)b * nc + (nc - 1 - c)) * H + h) * (int64_t)P * N + k * NH;
        rows_load_async<CHN, 4>(lds_addr(tiles[q][0]), P, wu, lane, [&](int r) { return sp + (int64_t)r * N; });
        rows_load_async<CHN, 4>(lds_addr(tiles[q][1]), P, wu, lane, [&](int r) { return gp + (int64_t)r * N; });
        const int64_t row = ((b * H + h) * nc + c) * (int64_t)Q;
        tables_load_async(cs + row, dtc + row, lds_addr(tab[q][0]), lds_addr(tab[q][1]), wu, lane, Q);
    };

    f32x4 accC[NT], accB[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) accC[nt] = accB[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    Vec8<bf16> dyc[KS], xc[KS], dyn[KS], xn[KS];
    if (j0 < j1) {
        load_rows(j0, dyc, xc);
        issue(j0, 0);
    }
    wait_vmem();
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
        const int q = (j - j0) & 1;
        if (j + 1 < j1) {
            load_rows(j + 1, dyn, xn);
            issue(j + 1, q ^ 1);
        }
        const float* cst = tab[q][0];
        const float* dtt = tab[q][1];
        const int lc = min(l, Q - 1);
        const float eC = lok ? __expf(cst[lc]) : 0.f;
        const float eB = lok ? __expf(cst[Q - 1] - cst[lc]) * dtt[lc] : 0.f;
        Vec8<bf16> bC[KS], bB[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bC[ks].set(e, dyc[ks].get(e) * eC);
                bB[ks].set(e, xc[ks].get(e) * eB);
            }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Vec8<bf16> a;
                swz_row_slots<CHN>(a, tiles[q][0], 32 * ks, 16 * nt);
                mma(accC[nt], a, bC[ks]);
                swz_row_slots<CHN>(a, tiles[q][1], 32 * ks, 16 * nt);
                mma(accB[nt], a, bB[ks]);
            }
        wait_vmem();
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            dyc[ks] = dyn[ks];
            xc[ks] = xn[ks];
        }
    }
    if (lok) {
        const int64_t o = (int64_t)sl * batch * L * G * N + ((b * L + t0 + l) * G + g) * (int64_t)N + k * NH + 4 * grp;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            *reinterpret_cast<f32x4*>(dCi + o + 16 * nt) = accC[nt];
            *reinterpret_cast<f32x4*>(dBi + o + 16 * nt) = accB[nt];
        }
    }
}

// ---------------------------------------------------------------------------------------------
// dC and dB of the group.  Wavefront w owns tokens r = 64 rb + 16 w + r16 (a row of dC, a column
// of M for dB); D[n][r] = sum_s B^T[n][s] M[r][s] (dC) and sum_l C^T[n][l] M[l][r] (dB), the B and
// C tiles read transposed from LDS (8 contraction slots per lane: tokens k0 + 4 grp + m and
// k0 + 16 + 4 grp + m), M (the slices summed in fp32) split into bf16 hi + lo; the state terms'
// slices are added before the one rounding to bf16.
template <int NT>
__global__ __launch_bounds__(kT) void bwd_dbc_kernel(const bf16* __restrict__ Bm, const bf16* __restrict__ Cm,
                                                     const float* __restrict__ Mp, const float* __restrict__ dCi,
                                                     const float* __restrict__ dBi, bf16* __restrict__ dB,
                                                     bf16* __restrict__ dC, int batch, int64_t L, int G, int N, int Q,
                                                     int nc, int nrb, int nsplit, int nsl, int nblocks)
{
    constexpr int NH = 16 * NT, CHN = NH / 8;
    constexpr int tile_bytes = kMaxQ * NH * 2;
    __shared__ __attribute__((aligned(1024))) unsigned char bt[tile_bytes];
    __shared__ __attribute__((aligned(1024))) unsigned char ctl[tile_bytes];

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int k = id % nsplit; id /= nsplit;
    const int rb = id % nrb; id /= nrb;
    const int g = id % G; id /= G;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, L - t0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int rbl = 4 * rb + wu;
    const int r = 16 * rbl + r16;                        // this lane's token (row of dC, column of M for dB)

    // the chunk's B and C rows (state columns of this half), rows past the sequence clamped
    const bf16* bg = Bm + ((b * L + t0) * G + g) * (int64_t)N + k * NH;
    const bf16* cg = Cm + ((b * L + t0) * G + g) * (int64_t)N + k * NH;
    rows_load_async<CHN, 4>(lds_addr(bt), Q, wu, lane, [&](int rr) { return bg + (int64_t)min(rr, len - 1) * G * N; });
    rows_load_async<CHN, 4>(lds_addr(ctl), Q, wu, lane, [&](int rr) { return cg + (int64_t)min(rr, len - 1) * G * N; });
    wait_vmem();
    __syncthreads();

    const int64_t mstride = (int64_t)batch * nc * G * Q * Q;  // between slices
    const float* mb = Mp + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    f32x4 accC[NT], accB[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) accC[nt] = accB[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // dC: tokens s <= r, in blocks of 32 (s < 16 (rbl + 1))
    const int nks = (16 * rbl + 16 + 31) / 32;
    for (int kb = 0; kb < nks; ++kb) {
        const int k0 = 32 * kb;
        float mv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mv[i] = 0.f;
        for (int z = 0; z < nsl; ++z) {
            const float* row = mb + z * mstride + (int64_t)min(r, Q - 1) * Q;
            const float4 a = *reinterpret_cast<const float4*>(row + k0 + 4 * grp);
            const float4 a2 = *reinterpret_cast<const float4*>(row + min(k0 + 16 + 4 * grp, Q - 4));
            mv[0] += a.x; mv[1] += a.y; mv[2] += a.z; mv[3] += a.w;
            mv[4] += a2.x; mv[5] += a2.y; mv[6] += a2.z; mv[7] += a2.w;
        }
        Vec8<bf16> hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) split_set(hi, lo, i, k0 + 16 * (i >> 2) + 4 * grp + (i & 3) < Q ? mv[i] : 0.f);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            Vec8<bf16> a;
            swz_row_slots<CHN>(a, bt, k0, 16 * nt);
            mma(accC[nt], a, hi);
            mma(accC[nt], a, lo);
        }
    }
    // dB: tokens l >= r, in blocks of 32 from the block holding 16 rbl
    for (int kb = (16 * rbl) / 32; kb < (Q + 31) / 32; ++kb) {
        const int k0 = 32 * kb;
        float mv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mv[i] = 0.f;
        for (int z = 0; z < nsl; ++z) {
            const float* col = mb + z * mstride + min(r, Q - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int li = min(k0 + 16 * (i >> 2) + 4 * grp + (i & 3), Q - 1);
                mv[i] += col[(int64_t)li * Q];
            }
        }
        Vec8<bf16> hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) split_set(hi, lo, i, k0 + 16 * (i >> 2) + 4 * grp + (i & 3) < Q ? mv[i] : 0.f);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            Vec8<bf16> a;
            swz_row_slots<CHN>(a, ctl, k0, 16 * nt);
            mma(accB[nt], a, hi);
            mma(accB[nt], a, lo);
        }
    }
    if (r < len) {
        const int64_t o = ((b * L + t0 + r) * G + g) * (int64_t)N + k * NH + 4 * grp;
        const int64_t istride = (int64_t)batch * L * G * N;      // between the state terms' slices
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 c4 = accC[nt], b4 = accB[nt];
            for (int z = 0; z < nsl; ++z) {
                const float4 ic = *reinterpret_cast<const float4*>(dCi + z * istride + o + 16 * nt);
                const float4 ib = *reinterpret_cast<const float4*>(dBi + z * istride + o + 16 * nt);
                c4[0] += ic.x; c4[1] += ic.y; c4[2] += ic.z; c4[3] += ic.w;
                b4[0] += ib.x; b4[1] += ib.y; b4[2] += ib.z; b4[3] += ib.w;
            }
            store4(dC + o + 16 * nt, c4[0], c4[1], c4[2], c4[3]);
            store4(dB + o + 16 * nt, b4[0], b4[1], b4[2], b4[3]);
        }
    }
}

template <int P, int NT>
hipError_t launch_pn(const bf16* x, const bf16* dy, const bf16* B, const bf16* C, const float* dtc, const float* cs,
                     const bf16* Sin, const bf16* Gout_rev, float* Mp, float* dCi, float* dBi, bf16* dB, bf16* dC,
                     int nsl, const Dims& d, hipStream_t s)
{
    const int nc = (int)d.nchunks(), Q = (int)d.chunk, G = (int)d.ngroups, H = (int)d.nheads, N = (int)d.dstate;
    const int nrb = Q / 64, nrb8 = (Q + 16 * kW8 - 1) / (16 * kW8), nsplit = N / (16 * NT), hpg = H / G;
    const int hps = (hpg + nsl - 1) / nsl;
    const int64_t ngroups_all = d.batch * nc * G;
    const int nb_score = (int)(ngroups_all * nrb8 * nsl);
    const int nb_inter = (int)(ngroups_all * nrb * nsplit * nsl);
    const int nb_dbc = (int)(ngroups_all * nrb * nsplit);
    if (nb_score == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_score_kernel<P>), dim3(nb_score), dim3(64 * kW8), 0, s, x, dy, dtc, cs, Mp, (int)d.batch,
                       d.seqlen, H, G, Q, nc, nrb8, nsl, hps, nb_score);
    hipLaunchKernelGGL((bwd_inter_kernel<P, NT>), dim3(nb_inter), dim3(kT), 0, s, x, dy, dtc, cs, Sin, Gout_rev,
                       dCi, dBi, (int)d.batch, d.seqlen, H, G, N, Q, nc, nrb, nsplit, nsl, hps, nb_inter);
    hipLaunchKernelGGL((bwd_dbc_kernel<NT>), dim3(nb_dbc), dim3(kT), 0, s, B, C, Mp, dCi, dBi, dB, dC,
                       (int)d.batch, d.seqlen, G, N, Q, nc, nrb, nsplit, nsl, nb_dbc);
    return hipGetLastError();
}

}  // namespace

bool bwd_dbc_supported(const Dims& d) { return d.headdim % 32 == 0 && d.headdim <= 128 && d.chunk % 64 == 0; }

int bwd_dbc_slices(const Dims& d) { return (int)std::min<int64_t>(4, std::max<int64_t>(1, d.nheads / d.ngroups / 16)); }

hipError_t launch_bwd_dbc(const bf16* x, const bf16* dy, const bf16* B, const bf16* C, const float* dtc,
                          const float* cs, const bf16* Sin, const bf16* Gout_rev, float* Mp, float* dCi, float* dBi,
                          bf16* dB, bf16* dC, const Dims& d, hipStream_t s)
{
    const int nsl = bwd_dbc_slices(d);
    const int nh = (int)std::min<int64_t>(d.dstate, 128);
#define SSD_DBC_CASE(PP, TT) \
    if (d.headdim == PP && nh == 16 * TT) return launch_pn<PP, TT>(x, dy, B, C, dtc, cs, Sin, Gout_rev, Mp, dCi, dBi, dB, dC, nsl, d, s);
#define SSD_DBC_P(PP) SSD_DBC_CASE(PP, 1) SSD_DBC_CASE(PP, 2) SSD_DBC_CASE(PP, 4) SSD_DBC_CASE(PP, 8)
    SSD_DBC_P(32) SSD_DBC_P(64) SSD_DBC_P(128)
#undef SSD_DBC_P
#undef SSD_DBC_CASE
    return hipErrorInvalidValue;
}

}  // namespace ssd
