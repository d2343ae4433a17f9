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
// Workgroup = (batch, chunk, group, 64-row tile of the chunk, up to HB heads
// of the group); 4 wavefronts, each owning 16 rows x all P columns of y for
// every one of those heads.  Everything runs on the matrix cores with fp32
// accumulation:
//   * C rows of a wavefront are read once from global memory straight into
//     operand fragments (the state axis is contiguous, and it is the
//     contraction axis of both C.B^T and C.S^T) and kept in registers.
//   * inter term, head by head: S_in of the head is staged through LDS and
//     multiplied against those fragments; rows are scaled by exp(cs[l]).
//   * intra term, 32 source tokens at a time: G^T (tokens x rows) = B_s C^T
//     is computed ONCE for all the heads of the workgroup (B and C belong to
//     the group), then each head applies its own decay and dt in fp32 and
//     multiplies by its x tile.  G^T comes out of the matrix core with each
//     lane holding 4 consecutive source tokens of one row; two such tiles
//     are exactly one A operand for G @ X_s once the 32 contraction slots
//     are assigned to tokens in the same order on the X side, so G never
//     leaves registers.  Entries above the diagonal are selected to zero,
//     never multiplied.
//   * the next 32 tokens' B and x (and the next head's S_in) are loaded into
//     registers while the current tile is being multiplied, so global
//     latency overlaps matrix-core work.  Those loads are unconditional
//     (indices clamped into the tensor) and the masks are applied when the
//     registers are written to LDS, so no branch ever waits on a load.
//   * x is kept in LDS in its natural (token, column) order; the G @ X
//     operand, whose contraction runs over tokens, is read with the gfx950
//     LDS transpose read, so no thread transposes data by hand.
//   * y tiles are staged through LDS so every store, and the x read of the
//     skip term, is a 16-byte vector access along the head dimension.
// Workgroups are numbered row-tile fastest, then head block, group, chunk,
// and renumbered so that consecutive ones share an XCD and its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kRows = 64;     // rows of y per workgroup
constexpr int kSB = 32;       // source tokens per intra step
constexpr int kMaxQ = 256;

// heads per workgroup: bounded by the accumulator registers (HB * P <= 512)
// and, for the widest state, by the fragment registers it keeps live.
constexpr int heads_per_block(int P, int NK) {
    return (NK >= 8 ? 5 : 8) < 512 / P ? (NK >= 8 ? 5 : 8) : 512 / P;
}

template <typename T, int P, int NK, int HB>
struct ScanSmem {
    static constexpr int NP = 32 * NK;                       // state width padded to the contraction block
    static constexpr bool kFullS = sizeof(T) * P * (NP + 8) <= 40 * 1024;
    static constexpr int SW = kFullS ? NP : 64;              // state columns of S_in per LDS stage
    static constexpr int ss_pitch = SW + 8;                  // rows read as 16-byte fragments
    static constexpr int bs_pitch = NP + 8;
    static constexpr int xs_pitch = tr_pitch<T>(P);          // x tile read down its rows
    static constexpr int out_pitch = P + 4;
    static constexpr size_t ss_bytes = sizeof(T) * P * ss_pitch;
    static constexpr size_t bs_bytes = sizeof(T) * kSB * bs_pitch;
    static constexpr size_t xs_bytes = sizeof(T) * HB * kSB * xs_pitch;
    static constexpr size_t out_bytes = sizeof(float) * kRows * out_pitch;
    static constexpr size_t m1 = ss_bytes > bs_bytes + xs_bytes ? ss_bytes : bs_bytes + xs_bytes;
    static constexpr size_t region = m1 > out_bytes ? m1 : out_bytes;
    static constexpr size_t dec_bytes = 2 * sizeof(float) * HB * kMaxQ;
    static constexpr size_t total = dec_bytes + region;
    // register-prefetch shares per thread (256 threads), 8 elements each
    static constexpr int s_n = P * SW / 8;
    static constexpr int x_n = HB * kSB * P / 8;
    static constexpr int b_n = kSB * NP / 8;
    static constexpr int s_items = (s_n + 255) / 256;
    static constexpr int x_items = (x_n + 255) / 256;
    static constexpr int b_items = (b_n + 255) / 256;
};

template <typename T, int P, int NK, int HB>
__global__ __launch_bounds__(256, 2) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ dt_chunked, const float* __restrict__ dA_cs,
    const T* __restrict__ entry, const float* __restrict__ Dv, T* __restrict__ y, int seqlen,
    int nheads, int ngroups, int N, int Q, int nc, int nlt, int nhb, int hpw, int nblocks)
{
    using S = ScanSmem<T, P, NK, HB>;
    constexpr int NP = S::NP, SW = S::SW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::total];
    float* csh = reinterpret_cast<float*>(smem);                    // [HB][kMaxQ]
    float* dth = csh + HB * kMaxQ;                                  // [HB][kMaxQ]
    unsigned char* region = smem + S::dec_bytes;
    T* SS = reinterpret_cast<T*>(region);                           // inter phase [P][ss_pitch]
    T* BS = reinterpret_cast<T*>(region);                           // intra phase [kSB][bs_pitch]
    T* XS = reinterpret_cast<T*>(region + S::bs_bytes);             // intra phase [HB][kSB][xs_pitch]
    float* OUT = reinterpret_cast<float*>(region);                  // epilogue [kRows][out_pitch]

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
    const int lrow = lw0 + r16;

    for (int i = tid; i < HB * kMaxQ; i += 256) {
        const int hh = i / kMaxQ, l = i % kMaxQ;
        const int64_t o = (((int64_t)b * nheads + h0 + min(hh, nh - 1)) * nc + c) * Q + min(l, Q - 1);
        const float cv = dA_cs[o], dv = dt_chunked[o];
        const bool ok = hh < nh && l < Q;
        csh[i] = select(ok, cv, 0.f);
        dth[i] = select(ok, dv, 0.f);
    }

    // C rows of this wavefront as operand fragments (state axis = contraction slots)
    Vec8<T> cf[NK];
    {
        const T* crow = Cm + ((b * seqlen + t0 + min(lrow, len - 1)) * ngroups + g) * N;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            const int n = 32 * ks + 8 * grp;
            load8(cf[ks], crow + min(n, N - 8));
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) cf[ks] = masked(cf[ks], lrow < len && 32 * ks + 8 * grp < N);
    }

    f32x4 acc[HB][P / 16];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh)
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[hh][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---------------- inter-chunk term, head by head: exp(cs[l]) * C_l . S_in[p, :]
    {
        const int64_t ent0 = (((int64_t)b * nc + c) * nheads + h0) * (int64_t)P * N;
        constexpr int nslab = NP / SW;
        Vec8<T> pf[S::s_items];
        auto fetch_s = [&](int hh, int sl) {
            const T* src = entry + ent0 + (int64_t)hh * P * N;
#pragma unroll
            for (int k = 0; k < S::s_items; ++k) {
                const int i = min(tid + 256 * k, S::s_n - 1);
                const int p = i / (SW / 8), o = i % (SW / 8);
                load8(pf[k], src + (int64_t)p * N + min(sl * SW + 8 * o, N - 8));
            }
        };
        fetch_s(0, 0);
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            if (hh >= nh) break;
            f32x4 ai[P / 16];
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) ai[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sl = 0; sl < nslab; ++sl) {
                __syncthreads();
#pragma unroll
                for (int k = 0; k < S::s_items; ++k) {
                    const int i = tid + 256 * k;
                    const int p = i / (SW / 8), o = i % (SW / 8);
                    if (i < S::s_n) store8(SS + p * S::ss_pitch + 8 * o, masked(pf[k], sl * SW + 8 * o < N));
                }
                __syncthreads();
                if (sl + 1 < nslab) fetch_s(hh, sl + 1);
                else if (hh + 1 < nh) fetch_s(hh + 1, 0);
#pragma unroll
                for (int kk = 0; kk < SW / 32; ++kk) {
                    const int ks = sl * (SW / 32) + kk;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> bf;
                        load8(bf, SS + (16 * pt + r16) * S::ss_pitch + 32 * kk + 8 * grp);
                        mma(ai[pt], cf[ks], bf);
                    }
                }
            }
            const float4 c4 = *reinterpret_cast<const float4*>(csh + hh * kMaxQ + lw0 + 4 * grp);
            const float sc[4] = {__expf(c4.x), __expf(c4.y), __expf(c4.z), __expf(c4.w)};
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[hh][pt][j] = sc[j] * ai[pt][j];
        }
    }

    // ---------------- intra-chunk term: sum_{s <= l} G[l, s] x[s, :]
    {
        const int s_end = min(len, row0 + kRows);
        const int nsb = (s_end + kSB - 1) / kSB;
        Vec8<T> px[S::x_items];
        Vec8<T> pb[S::b_items];
        // loads always hit valid addresses (indices clamped); masks are applied when storing to LDS
        auto fetch = [&](int s0) {
#pragma unroll
            for (int k = 0; k < S::x_items; ++k) {
                const int i = min(tid + 256 * k, S::x_n - 1);     // (head, token, 8-column group)
                const int hh = i / (kSB * P / 8), r = (i / (P / 8)) % kSB, o = i % (P / 8);
                const int s = min(s0 + r, len - 1);
                load8(px[k], x + ((b * seqlen + t0 + s) * nheads + h0 + min(hh, nh - 1)) * P + 8 * o);
            }
#pragma unroll
            for (int k = 0; k < S::b_items; ++k) {
                const int i = min(tid + 256 * k, S::b_n - 1);     // (token, 8-column group)
                const int r = i / (NP / 8), o = i % (NP / 8);
                const int s = min(s0 + r, len - 1);
                load8(pb[k], Bm + ((b * seqlen + t0 + s) * ngroups + g) * N + min(8 * o, N - 8));
            }
        };
        if (nsb > 0) fetch(0);
        for (int sb = 0; sb < nsb; ++sb) {
            const int s0 = sb * kSB;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < S::x_items; ++k) {
                const int i = tid + 256 * k;
                const int hh = i / (kSB * P / 8), r = (i / (P / 8)) % kSB, o = i % (P / 8);
                if (i < S::x_n)
                    store8(XS + (hh * kSB + r) * S::xs_pitch + 8 * o, masked(px[k], hh < nh && s0 + r < len));
            }
#pragma unroll
            for (int k = 0; k < S::b_items; ++k) {
                const int i = tid + 256 * k;
                const int r = i / (NP / 8), o = i % (NP / 8);
                if (i < S::b_n) store8(BS + r * S::bs_pitch + 8 * o, masked(pb[k], s0 + r < len && 8 * o < N));
            }
            __syncthreads();
            if (sb + 1 < nsb) fetch(s0 + kSB);
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
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    if (hh >= nh) break;
                    const float* csr = csh + hh * kMaxQ;
                    const float* dtr = dth + hh * kMaxQ;
                    const float cl = csr[lrow];
                    Vec8<T> gf;
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
                    const T* xh = XS + hh * kSB * S::xs_pitch;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> xf;
                        load_row_slots(xf, xh, S::xs_pitch, 0, 16 * pt);
                        mma(acc[hh][pt], gf, xf);
                    }
                }
            }
        }
    }

    // ---------------- epilogue, head by head: y = acc + D x through LDS for 16-byte accesses
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
        if (hh >= nh) break;
        __syncthreads();
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int j = 0; j < 4; ++j) OUT[(16 * wave + 4 * grp + j) * S::out_pitch + 16 * pt + r16] = acc[hh][pt][j];
        __syncthreads();
        const int h = h0 + hh;
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
}

template <typename T, int P, int NK>
hipError_t launch(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                  const float* D, T* y, const Dims& d, hipStream_t stream)
{
    constexpr int HB = heads_per_block(P, NK);
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
