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
// Workgroup = (batch, chunk, group, 64-row tile of the chunk, up to 256/P
// heads of the group); 4 wavefronts, each owning 16 rows of y for every one
// of those heads.  Everything runs on the matrix cores with fp32
// accumulation, and the products are formed transposed (y^T = X^T G^T and
// S_in C^T), so each lane ends up holding 4 consecutive head-dimension values
// of one row:
//   * C rows of a wavefront are read once from global memory straight into
//     operand fragments (the state axis is contiguous, and it is the
//     contraction axis of both C.B^T and S_in.C^T) and kept in registers.
//   * inter term, head by head: S_in of the head is the A operand, read from
//     LDS; columns (rows of y) are scaled by exp(cs[l]).
//   * intra term, 32 source tokens per stage: G^T (tokens x rows) = B_s C^T
//     is computed ONCE for all the heads of the workgroup (B and C belong to
//     the group), then each head applies its own decay and dt in fp32, and
//     the result, still in the accumulator layout, is the B operand of
//     X_s^T G^T: no shuffle, no LDS round trip.  Entries above the diagonal
//     are selected to zero, never multiplied.
//   * every tile (S_in, x, B) reaches LDS through asynchronous global->LDS
//     loads into two alternating buffers: the next stage is in flight while
//     the current one is multiplied, and no register holds staged data.
//     Tiles are XOR-swizzled by 16-byte chunk, so the 16-byte operand reads
//     and the transpose reads (x is kept in natural token-major order and
//     read token-wise with ds_read_b64_tr_b16) are bank-conflict free.
//     Out-of-range rows are loaded from a clamped, valid address; their
//     products are removed by the causal mask or by zero C entries.
//   * the skip term D x reads x from the last two stages' tiles, which hold
//     exactly this workgroup's rows; y is then staged through LDS so it
//     leaves as full 16-byte row segments (8 lanes per 128-byte row).
// Workgroups are numbered row-tile fastest, then head block, group, chunk,
// and renumbered so that consecutive ones share an XCD and its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kRows = 64;     // rows of y per workgroup
constexpr int kSB = 32;       // source tokens per intra step
constexpr int kMaxQ = 256;

template <typename T, int P, int NK, int HB> struct ScanCfg;

// heads per workgroup: 256 / P (at most 8), so the y accumulators stay at
// 64 registers per lane whatever the head dimension, halved while the
// workgroup's LDS would not fit twice in a CU (bf16) or once (fp32).
template <typename T, int P, int NK, int HB = (256 / P > 8 ? 8 : 256 / P)>
constexpr int heads_per_block() {
    if constexpr (HB > 1 && ScanCfg<T, P, NK, HB>::total > (sizeof(T) == 2 ? 80 : 160) * 1024)
        return heads_per_block<T, P, NK, HB / 2>();
    else
        return HB;
}

template <typename T, int P, int NK, int HB>
struct ScanCfg {
    static constexpr int EPC = 16 / (int)sizeof(T);               // elements per 16-byte chunk
    static constexpr int NP = 32 * NK;                             // state width padded to the contraction block
    static constexpr int SW = (P * NP * (int)sizeof(T) <= 32 * 1024) ? NP
                            : (P * 128 * (int)sizeof(T) <= 32 * 1024 ? 128 : 64);
    static constexpr int S_CH = SW * (int)sizeof(T) / 16;          // chunks per S_in row
    static constexpr int X_CH = P * (int)sizeof(T) / 16;           // chunks per x row
    static constexpr int B_CH = NP * (int)sizeof(T) / 16;          // chunks per B row
    static constexpr int s_bytes = P * SW * (int)sizeof(T);        // one S_in stage
    static constexpr int xh_bytes = kSB * P * (int)sizeof(T);      // x of one head, one stage
    static constexpr int xb_bytes = HB * xh_bytes + kSB * NP * (int)sizeof(T);
    static constexpr int region = 2 * (s_bytes > xb_bytes ? s_bytes : xb_bytes);
    static constexpr int dec_bytes = 3 * (int)sizeof(float) * HB * kMaxQ;    // cs, dt, source factors
    static constexpr int total = dec_bytes + region;
};

template <typename T, int P, int NK, int HB>
__global__ __launch_bounds__(256, 2) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ dt_chunked, const float* __restrict__ dA_cs,
    const T* __restrict__ entry, const float* __restrict__ Dv, T* __restrict__ y, int seqlen,
    int nheads, int ngroups, int N, int Q, int nc, int nlt, int nhb, int hpw, int nblocks)
{
    using S = ScanCfg<T, P, NK, HB>;
    constexpr int EPC = S::EPC, SW = S::SW, NP = S::NP;
    __shared__ float csh[HB * kMaxQ];
    __shared__ float dth[HB * kMaxQ];
    // vsrc[hh][s] = exp(cs[row0] - cs[s]) dt[s] for s < row0: the source side of the decay of
    // every source block before this workgroup's first row (0 elsewhere)
    __shared__ float vsrc[HB * kMaxQ];
    __shared__ __attribute__((aligned(1024))) unsigned char region[S::region];   // two stage buffers

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int lt = id % nlt; id /= nlt;
    const int hb = id % nhb; id /= nhb;
    const int g = id % ngroups; id /= ngroups;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int hpg = nheads / ngroups;
    const int h0 = g * hpg + hb * hpw;
    const int nh = min(hpw, hpg - hb * hpw);                       // heads of this workgroup (<= HB)
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);
    const int row0 = lt * kRows;

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;
    const int lw0 = row0 + 16 * wave;
    const int lrow = lw0 + r16;                                     // the y row this lane owns

    for (int i = tid; i < HB * kMaxQ; i += 256) {
        const int hh = i / kMaxQ, l = i % kMaxQ;
        const int64_t o = (((int64_t)b * nheads + h0 + min(hh, nh - 1)) * nc + c) * Q + min(l, Q - 1);
        const float cv = dA_cs[o], dv = dt_chunked[o];
        const bool ok = hh < nh && l < Q;
        csh[i] = select(ok, cv, 0.f);
        dth[i] = select(ok, dv, 0.f);
    }

    __syncthreads();
    for (int i = tid; i < HB * kMaxQ; i += 256) {
        const int hh = i / kMaxQ, sidx = i % kMaxQ;
        const float v = __expf(csh[hh * kMaxQ + row0] - csh[i]) * dth[i];
        vsrc[i] = select(sidx < row0, v, 0.f);
    }

    // C rows of this wavefront as operand fragments (state axis = contraction slots)
    Vec8<T> cf[NK];
    {
        const T* crow = Cm + ((b * seqlen + t0 + min(lrow, len - 1)) * ngroups + g) * N;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) load8(cf[ks], crow + min(32 * ks + 8 * grp, N - 8));
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) cf[ks] = masked(cf[ks], lrow < len && 32 * ks + 8 * grp < N);
    }

    // y^T accumulators: lane (r16, grp) holds y[lrow][16 pt + 4 grp + j]
    f32x4 acc[HB][P / 16];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[hh][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---------------- inter-chunk term, head by head: exp(cs[l]) * S_in[p, :] . C_l
    {
        const T* ent = entry + (((int64_t)b * nc + c) * nheads + h0) * (int64_t)P * N;
        constexpr int nslab = NP / SW;
        auto issue = [&](int hh, int sl, int buf) {
            const T* src = ent + (int64_t)hh * P * N;
            tile_load_async<S::S_CH, P>(region + buf * S::s_bytes, [&](int r, int ch) -> const void* {
                return src + (int64_t)r * N + min(sl * SW + ch * EPC, N - EPC);
            });
        };
        issue(0, 0, 0);
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            if (hh >= nh) break;
            f32x4 ai[P / 16];
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) ai[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sl = 0; sl < nslab; ++sl) {
                const int j = hh * nslab + sl;
                wait_vmem();
                __syncthreads();
                if (sl + 1 < nslab) issue(hh, sl + 1, (j + 1) & 1);
                else if (hh + 1 < nh) issue(hh + 1, 0, (j + 1) & 1);
                const unsigned char* tile = region + (j & 1) * S::s_bytes;
#pragma unroll
                for (int kk = 0; kk < SW / 32; ++kk) {
                    const int ks = sl * (SW / 32) + kk;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> af;
                        swz_load8<S::S_CH>(af, tile, 16 * pt + r16, 32 * kk + 8 * grp);
                        mma(ai[pt], af, cf[ks]);
                    }
                }
            }
            // exp(cs[l]) = exp(cs[row0]) * exp(cs[l] - cs[row0]); the second factor is applied with
            // the source blocks before row0 (both exponents are <= 0)
            const float e = __expf(csh[hh * kMaxQ + row0]);
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[hh][pt][q] = e * ai[pt][q];
        }
    }

    // ---------------- intra-chunk term: y^T += X_s^T G^T, 32 source tokens per stage
    const int s_end = min(len, row0 + kRows);
    const int nsb = (s_end + kSB - 1) / kSB;
    auto xtile = [&](int buf, int hh) { return region + buf * S::xb_bytes + hh * S::xh_bytes; };
    auto issue_xb = [&](int s0, int buf) {
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            const T* xh = x + (int64_t)(h0 + min(hh, nh - 1)) * P;
            tile_load_async<S::X_CH, kSB>(xtile(buf, hh), [&](int r, int ch) -> const void* {
                return xh + (b * seqlen + t0 + min(s0 + r, len - 1)) * (int64_t)nheads * P + ch * EPC;
            });
        }
        const T* bg = Bm + (int64_t)g * N;
        tile_load_async<S::B_CH, kSB>(region + buf * S::xb_bytes + HB * S::xh_bytes,
                                      [&](int r, int ch) -> const void* {
            return bg + (b * seqlen + t0 + min(s0 + r, len - 1)) * (int64_t)ngroups * N + min(ch * EPC, N - EPC);
        });
    };
    __syncthreads();                                  // the inter phase's buffers are free
    if (nsb > 0) issue_xb(0, 0);
    for (int sb = 0; sb < nsb; ++sb) {
        const int s0 = sb * kSB;
        wait_vmem();
        __syncthreads();
        if (sb + 1 < nsb) issue_xb(s0 + kSB, (sb + 1) & 1);
        if (s0 <= lw0 + 15 && lw0 < len) {
            const unsigned char* bt = region + (sb & 1) * S::xb_bytes + HB * S::xh_bytes;
            f32x4 gt[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                gt[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NK; ++ks) {
                    Vec8<T> af;
                    swz_load8<S::B_CH>(af, bt, 16 * st + r16, 32 * ks + 8 * grp);
                    mma(gt[st], af, cf[ks]);
                }
            }
            if (s0 + kSB <= row0) {
                // a block strictly before this workgroup's rows: G = C.B * vsrc[s]
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    if (hh >= nh) break;
                    const float* vr = vsrc + hh * kMaxQ;
                    Vec8<T> gf;
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const float4 v4 = *reinterpret_cast<const float4*>(vr + s0 + 16 * st + 4 * grp);
                        gf.set(4 * st + 0, gt[st][0] * v4.x);
                        gf.set(4 * st + 1, gt[st][1] * v4.y);
                        gf.set(4 * st + 2, gt[st][2] * v4.z);
                        gf.set(4 * st + 3, gt[st][3] * v4.w);
                    }
                    const unsigned char* xt = xtile(sb & 1, hh);
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> xf;
                        swz_row_slots<S::X_CH>(xf, xt, 0, 16 * pt);
                        mma(acc[hh][pt], xf, gf);
                    }
                }
            } else {
                // a block inside this workgroup's 64 rows: on the first one, apply the row side
                // exp(cs[l] - cs[row0]) to everything accumulated so far; then add the block with the
                // full per-entry decay and the causal mask
                if (s0 == row0) {
#pragma unroll
                    for (int hh = 0; hh < HB; ++hh) {
                        if (hh >= nh) break;
                        const float u = __expf(csh[hh * kMaxQ + lrow] - csh[hh * kMaxQ + row0]);
#pragma unroll
                        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[hh][pt][q] *= u;
                    }
                }
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    if (hh >= nh) break;
                    const float* csr = csh + hh * kMaxQ;
                    const float* dtr = dth + hh * kMaxQ;
                    const float cl = csr[lrow];
                    Vec8<T> gf;                                   // G[lrow][s], s = s0 + 16 st + 4 grp + j
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const int sb4 = s0 + 16 * st + 4 * grp;
                        const float4 c4 = *reinterpret_cast<const float4*>(csr + sb4);
                        const float4 d4 = *reinterpret_cast<const float4*>(dtr + sb4);
                        const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float v = gt[st][j] * (__expf(cl - cv[j]) * dv[j]);
                            gf.set(4 * st + j, select(sb4 + j <= lrow, v, 0.f));
                        }
                    }
                    const unsigned char* xt = xtile(sb & 1, hh);
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> xf;
                        swz_row_slots<S::X_CH>(xf, xt, 0, 16 * pt);
                        mma(acc[hh][pt], xf, gf);
                    }
                }
            }
        }
    }

    // ---------------- epilogue: y = acc + D x (x from the tiles of the last two stages), then
    // through LDS so every global store is a full 16-byte segment of a y row
    float yv[HB][P / 16][4];
    {
        const int sbl = min(lrow, len - 1) / kSB;
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            const float dh = Dv[h0 + min(hh, nh - 1)];
            const T* xt = reinterpret_cast<const T*>(xtile(sbl & 1, hh));
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                const float4 xv = swz_load4f<S::X_CH>(xt, min(lrow, len - 1) % kSB, 16 * pt + 4 * grp);
                yv[hh][pt][0] = acc[hh][pt][0] + dh * xv.x;
                yv[hh][pt][1] = acc[hh][pt][1] + dh * xv.y;
                yv[hh][pt][2] = acc[hh][pt][2] + dh * xv.z;
                yv[hh][pt][3] = acc[hh][pt][3] + dh * xv.w;
            }
        }
    }
    __syncthreads();                                  // every wave is done with the x tiles
    constexpr int out_bytes = kRows * P * (int)sizeof(T);           // one head's y tile
    static_assert(HB * out_bytes <= S::region, "y staging fits the stage buffers");
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
        unsigned char* ot = region + hh * out_bytes;
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const int col = 16 * pt + 4 * grp;
            unsigned char* dst = ot + SwzTile<S::X_CH>::offset(16 * wave + r16, col / EPC) + (int)sizeof(T) * (col % EPC);
            store4(reinterpret_cast<T*>(dst), yv[hh][pt][0], yv[hh][pt][1], yv[hh][pt][2], yv[hh][pt][3]);
        }
    }
    __syncthreads();
    for (int i = tid; i < nh * kRows * S::X_CH; i += 256) {
        const int hh = i / (kRows * S::X_CH), r = (i / S::X_CH) % kRows, ch = i % S::X_CH;
        if (row0 + r >= len) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(region + hh * out_bytes + SwzTile<S::X_CH>::offset(r, ch));
        *reinterpret_cast<uint4*>(y + ((b * seqlen + t0 + row0 + r) * nheads + h0 + hh) * P + ch * EPC) = v;
    }
}

template <typename T, int P, int NK>
hipError_t launch(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                  const float* D, T* y, const Dims& d, hipStream_t stream)
{
    constexpr int HB = heads_per_block<T, P, NK>();
    static_assert(ScanCfg<T, P, NK, HB>::total <= 160 * 1024, "LDS budget");
    const int nc = (int)d.nchunks();
    const int nlt = (int)((d.chunk + kRows - 1) / kRows);
    const int hpg = (int)(d.nheads / d.ngroups);
    const int nhb = (hpg + HB - 1) / HB;                 // head blocks per group
    const int hpw = (hpg + nhb - 1) / nhb;               // heads per workgroup, balanced
    const int64_t nblocks = d.batch * nc * d.ngroups * nhb * nlt;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_scan_kernel<T, P, NK, HB>), dim3((unsigned)nblocks), dim3(256), 0, stream, x,
                       B, C, dtc, cs, entry, D, y, (int)d.seqlen, (int)d.nheads, (int)d.ngroups,
                       (int)d.dstate, (int)d.chunk, nc, nlt, nhb, hpw, (int)nblocks);
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
