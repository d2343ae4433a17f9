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
// Row blocks of 16 rows are paired (p, nrb-1-p), which gives every pair the
// same amount of causal work.  Workgroup = (batch, chunk, group, up to HB
// heads of the group, one half of the pairs): 4 wavefronts, one pair each;
// at 256-token chunks a chunk's 8 pairs make two workgroups, and the LDS use
// is held to 80 KB so that two workgroups share a CU and one's loads and
// stores overlap the other's products.  All products run on the matrix cores
// with fp32 accumulation and are formed transposed (y^T = X^T G^T and
// S_in C^T), so a lane holds 4 consecutive head-dimension values of one row:
//   * C rows of a wavefront are read once from global memory straight into
//     operand fragments (the state axis is contiguous, and it is the
//     contraction axis of both C.B^T and S_in.C^T) through range-checked
//     buffer loads (rows past the sequence read as zero) and kept in
//     registers.  They are issued first, and the per-head decay tables come
//     by asynchronous copies right after, so that the prologue is one round
//     trip to memory: no wait for a register load also waits for the copies.
//   * the heads' S_in tiles (in slabs of 32 state columns) and the source
//     tokens' x and B tiles reach LDS through asynchronous global->LDS
//     copies.  Slabs are double-buffered (odd slabs in the ring slot that the
//     source tokens use last), source tokens stream through a 2-deep ring of
//     32-token stages, the next stage in flight while the current one is
//     multiplied, and every byte of x, B and S_in is read once per workgroup.  Tiles are
//     XOR-swizzled by 16-byte chunk, so the 16-byte operand reads and the
//     transpose reads (x is kept token-major and read token-wise with
//     ds_read_b64_tr_b16) are bank-conflict free.  Rows past the sequence
//     are copied from a clamped, valid address; their products are removed
//     by the causal mask or by zero C entries.
//   * inter term first: every S_in fragment read from LDS feeds both row
//     blocks of the wavefront; the sum is then scaled by exp(cs[l]).
//   * intra term, per stage and row block: G^T (tokens x rows) = B_s C^T is
//     computed once for all the heads of the workgroup (B and C belong to the
//     group); each head applies its decay and dt in fp32 and the result, still
//     in the accumulator layout, is the B operand of X_s^T G^T.  For a stage
//     wholly before the row block the decay is split at the stage's last
//     token e: exp(cs[l] - cs[e]) per row times a per-token factor
//     exp(cs[e] - cs[s]) dt_s tabulated once per workgroup (both exponents
//     are <= 0); the stage holding the rows uses the full per-entry decay and
//     the causal mask (entries above the diagonal are selected to zero, never
//     multiplied).  The heads run as one straight-line sequence (heads past
//     the workgroup compute on clamped data and are never stored), so the
//     compiler can overlap one head's LDS reads with another's products.
//   * the skip term D x is added in the stage holding the rows, from the x
//     tile already in LDS, in fp32.
//   * y leaves through LDS when it is bf16 (the ring is free by then): one
//     row block at a time, each wavefront stages its 16 rows of all the
//     workgroup's heads and stores whole token rows -- a token's heads are
//     adjacent in y, so a row is HB * P * 2 contiguous bytes -- in 16-byte
//     pieces (fp32 y goes straight from the accumulators, 4 consecutive
//     values per lane); stores of rows past the sequence or of heads past the
//     workgroup fall outside the buffer's range and are dropped.
// Workgroups are numbered head block fastest and renumbered so that
// consecutive ones share an XCD (and the chunk's B and C in its L2).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kSB = 32;        // source tokens per stage
constexpr int kMaxQ = 256;
constexpr int kWaves = 4;                      // one row-block pair per wavefront
constexpr int kThreads = 64 * kWaves;

template <typename T, int P, int NK, int HB, int STG, int SW, bool V = false, int SP = 1>
struct ScanCfg {
    static constexpr int kHeads = HB;
    static constexpr bool kSplit = SP == 2;                       // S_in as bf16 hi and lo planes
    static constexpr int kStages = STG;                            // depth of the source-token ring
    static constexpr int EPC = 16 / (int)sizeof(T);               // elements per 16-byte chunk
    static constexpr int NP = 32 * NK;                             // state width padded to the contraction block
    static constexpr int SWD = SW;                                 // state columns of S_in per LDS slab
    static constexpr int NSL = NP / SW;                            // slabs
    static constexpr int X_CH = P * (int)sizeof(T) / 16;           // chunks per x row
    static constexpr int EPB = 16 / (int)sizeof(T);              // B / C elements per 16-byte chunk
    static constexpr int B_CH = NP * (int)sizeof(T) / 16;         // chunks per B row
    static constexpr int S_CH = SW * (int)sizeof(T) / 16;          // chunks per S_in slab row
    static constexpr int S_RS = swz_row_shift(S_CH);               // slab rows read 16 at a time
    static constexpr int xh_bytes = kSB * P * (int)sizeof(T);      // x of one head, one stage
    static constexpr int b_bytes = kSB * NP * (int)sizeof(T);
    static constexpr int stage_bytes = HB * xh_bytes + b_bytes;
    static constexpr int sh_bytes = P * SW * (int)sizeof(T);       // one S_in slab of one head (one plane)
    static constexpr int ring_bytes = STG * stage_bytes;
    static constexpr int s_inst = HB * SP * P * S_CH / 64;          // copy instructions of one slab (all heads)
    // odd slabs go to the ring slot that the source tokens use last when they fit there, else after
    // the even slabs' area
    static constexpr bool odd_in_ring = HB * SP * sh_bytes <= stage_bytes;
    static constexpr int main_bytes = ring_bytes + HB * SP * sh_bytes * (NSL > 1 && !odd_in_ring ? 2 : 1);
    static constexpr int odd_off = odd_in_ring ? (STG - 1) * stage_bytes : ring_bytes + HB * SP * sh_bytes;
    static constexpr int region = main_bytes;
    static constexpr int tab_bytes = 3 * 4 * HB * kMaxQ + (V ? 4 * kMaxQ : 0);   // cs, dt, per-token decay factor
                                                                                // (+ sequence starts)
    static constexpr int total = tab_bytes + region;
    static constexpr bool pair_fits = total <= 80 * 1024;           // two workgroups per CU
    static constexpr bool fits = total <= 160 * 1024;
    // asynchronous copy instructions per wavefront per stage (uniform when divisible)
    static constexpr int x_inst = HB * kSB * X_CH / 64;             // dealt over all waves as one sequence
    static constexpr int b_inst = kSB * B_CH / 64;
    static constexpr bool uniform = x_inst % kWaves == 0 && b_inst % kWaves == 0;
    static constexpr int per_wave = uniform ? (x_inst + b_inst) / kWaves : 0;
};

// Launch shape for (T, P, NK): heads per workgroup keep the y accumulators
// (2 row blocks x HB heads x P columns) at 128 registers per lane (64 with the
// widest state, whose C fragments take the room), with a 2-deep ring and S_in
// in 32-column slabs; the heads are halved until two workgroups fit in a CU's
// LDS (one workgroup's loads and stores then overlap the other's products),
// and a single head takes a CU alone when it must.
template <class C> struct TypeBox { using type = C; };

template <typename T, int P, int NK, int HB, bool V, int SP = 1>
constexpr auto pick_shape() {
    using C = ScanCfg<T, P, NK, HB, 2, 32, V, SP>;
    if constexpr (C::pair_fits || (HB == 1 && C::fits)) return TypeBox<C>{};
    else if constexpr (HB > 1) return pick_shape<T, P, NK, HB / 2, V, SP>();
    else return TypeBox<C>{};                 // does not fit: rejected by a static_assert at launch
}

template <typename T, int P, int NK, bool V = false, int SP = 1>
using ScanShape = typename decltype(pick_shape<T, P, NK,
    ((NK >= 8 ? 128 : 256) / P > 8 ? 8 : (NK >= 8 ? 128 : 256) / P), V, SP>())::type;

// kVarlen: a packed variable-length batch (batch 1; tstart from varlen_meta.hip).  A pair (l, s)
// of one chunk is kept only when s >= tstart[l] (same sequence); since sequences are contiguous,
// for a stage ending at token e wholly before row l this factors into [tstart[l] <= e] per row
// times [s >= tstart[e]] per token, which fold into the row decay and the token table; the state
// entering the chunk reaches only the rows of the sequence holding the chunk's first token.
// TY: the type y is stored in (T, or float when the caller needs the sum unrounded).
// S::kSplit (T = bf16, TY = float): the fp32 products of the backward's readout passes from bf16
// ones, with x, B, C holding bf16 values: S_in comes as two bf16 planes, hi at entry and lo at
// entry + lo_off (hi + lo = the fp32 state to 2^-18), G is split the same way in registers, and
// each product is taken twice on the bf16 matrix cores (hi, then lo) into the fp32 accumulators.
// EPI (split mode): 0 stores y; 1 and 2 reduce it per (token, head) as ScanEpi describes (kernels.hpp).
template <typename T, typename TY, int P, int NK, class S, bool kVarlen, int EPI = 0>
__global__ __launch_bounds__(kThreads, 2) void chunk_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ dt_chunked, const float* __restrict__ dA_cs,
    const T* __restrict__ entry, int64_t lo_off, const float* __restrict__ Dv, const int* __restrict__ tstart,
    TY* __restrict__ y, XLayout xl, int seqlen, int nheads, int ngroups, int N, int Q, int nc, int nhb, int hpw, int nhalf, int nblocks,
    ScanEpi epi)
{
    constexpr int EPC = S::EPC, HB = S::kHeads, kStages = S::kStages, SW = S::SWD;
    __shared__ __attribute__((aligned(16))) float cst[HB * kMaxQ];
    __shared__ __attribute__((aligned(16))) float dtt[HB * kMaxQ];
    __shared__ float vst[HB * kMaxQ];          // exp(cs[e(s)] - cs[s]) dt[s], e(s) = last token of s's stage
    __shared__ int lst[kVarlen ? kMaxQ : 1];   // first token of each token's sequence, chunk-relative
    __shared__ __attribute__((aligned(1024))) unsigned char region[S::region];
    unsigned char* const ring = region;
    unsigned char* const stile = region + S::ring_bytes;

    int id = xcd_logical_block(blockIdx.x, nblocks);
    const int half = id % nhalf; id /= nhalf;
    const int hb = id % nhb; id /= nhb;
    const int g = id % ngroups; id /= ngroups;
    const int c = id % nc;
    const int64_t b = id / nc;
    const int hpg = nheads / ngroups;
    const int h0 = g * hpg + hb * hpw;
    const int nh = min(hpw, hpg - hb * hpw);                       // heads of this workgroup (<= HB)
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);
    const int nrb = Q / 16;
    // the workgroup's row-block pairs (p, nrb-1-p) for p in [half kWaves, half kWaves + kWaves): its last
    // row lies in the first pair's second block, so it needs the stages up to that block's
    const int last_rb = nrb - 1 - half * kWaves;
    const int nsb = min((len + kSB - 1) / kSB, (16 * last_rb + 15) / kSB + 1);

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;
    // this wavefront's row blocks: the pair (p, nrb-1-p), each block once
    const int pair = half * kWaves + wave;
    const int rbk[2] = {pair, nrb - 1 - pair};
    const bool has[2] = {2 * pair < nrb, 2 * pair < nrb - 1};

    // ---- C rows of this wavefront's row blocks as operand fragments (state axis = contraction slots),
    // by range-checked buffer loads (rows past the chunk's tokens and missing blocks read as zero).
    // Issued first: no later wait for them then also waits for the asynchronous copies below.
    Vec8<T> cf[2][S::NP / 32];
    {
        const T* cb = Cm + ((b * seqlen + t0) * ngroups + g) * (int64_t)N;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(cb), 0, ((len - 1) * ngroups + 1) * N * (int)sizeof(T), kBufferDword3);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int l = 16 * rbk[j] + r16;
            const bool rok = has[j] && l < len;
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
                const int col = 32 * ks + 8 * grp;
                buffer_load8(cf[j][ks], crs, rok && col < N ? (l * ngroups * N + col) * (int)sizeof(T) : kDropped);
            }
        }
    }
    // ---- decay tables by asynchronous copies: per head, the chunk's Q cumulative log-decays and dt
    // values (contiguous), one wavefront instruction each.  Heads past the workgroup copy its last head
    // (computed on, never stored); slots past Q repeat the row's last values (never used unmasked).
    const int wu = __builtin_amdgcn_readfirstlane(wave);           // (wave-uniform, and known to be)
#pragma unroll
    for (int k = 0; k < (2 * HB + kWaves - 1) / kWaves; ++k) {
        const int q = wu + k * kWaves;
        if (q >= 2 * HB) break;
        const int hh = q >> 1;
        const float* row = ((q & 1) ? dt_chunked : dA_cs) + (((int64_t)b * nheads + h0 + min(hh, nh - 1)) * nc + c) * Q;
        dma16(row + min(4 * lane, Q - 4), ((q & 1) ? lds_addr(dtt) : lds_addr(cst)) + hh * (kMaxQ * 4));
    }

    // ---- then the heads' S_in tiles (first two slabs) and the first stages of the ring.  With bf16
    // operands and head dimensions up to 64 the copies' per-lane source offsets are worked out once and
    // each slab and stage only moves the base (the wider shapes have no registers to spare for them).
    constexpr bool kPlanned = std::is_same_v<T, bf16> && P <= 64;
    const T* ent = entry + (((int64_t)b * nc + c) * nheads + h0) * (int64_t)P * N;
    // slab buffers: when every slab of the heads' S_in fits the region (the ring is free until the stage
    // loop), all of them side by side from the region's start, loaded at once; else even slabs in the
    // slab area and odd slabs in the last ring slot or, when they do not fit there, after the even ones
    constexpr int kSlabSet = HB * (S::kSplit ? 2 : 1) * S::sh_bytes;     // one slab of every head (and plane)
    constexpr bool kAllSlabs = S::NSL > 1 && S::NSL * kSlabSet <= S::region;
    auto slab_off = [&](int sl) -> int {
        return kAllSlabs ? sl * kSlabSet : ((sl & 1) ? S::odd_off : S::ring_bytes);
    };
    auto sbuf = [&](int sl) -> unsigned char* { return region + slab_off(sl); };
    // slab tiles 0 .. HB-1 the heads' (hi) slabs, HB .. 2 HB-1 their lo slabs (split mode)
    using SCopies = TileCopies<S::S_CH, P, HB * (S::kSplit ? 2 : 1), kWaves, S::S_RS>;
    SCopies scp;
    if constexpr (kPlanned)
        scp.plan(wu, [&](int t, int r, int ch) -> unsigned {
            return (unsigned)(((min(t % HB, nh - 1) * P + r) * N + ch * EPC) * (int)sizeof(T));
        });
    auto issue_s = [&](int sl) {
        const unsigned dst = lds_addr(region) + slab_off(sl);
        if (kPlanned && sl * SW + SW <= N) {
            scp.issue(wu, [&](int t) -> const void* { return ent + (t >= HB ? lo_off : 0) + sl * SW; }, dst, S::sh_bytes);
        } else {
            // (and the last slab of a state width that is not a multiple of its width: columns clamped)
            tiles_load_async<S::S_CH, P, HB * (S::kSplit ? 2 : 1), kWaves, S::S_RS>(dst, S::sh_bytes,
                [&](int t, int r, int ch) -> const void* {
                    const int hh = t % HB;
                    return ent + (t >= HB ? lo_off : 0) + (int64_t)min(hh, nh - 1) * P * N + (int64_t)r * N +
                           min(sl * SW + ch * EPC, N - EPC);
                });
        }
    };
    if constexpr (kAllSlabs) {
#pragma unroll
        for (int sl = 0; sl < S::NSL; ++sl) issue_s(sl);
    } else {
        issue_s(0);
        if (S::NSL > 1) issue_s(1);
    }
    // stage tiles: x of the HB heads (tile = head), then the group's B
    using XCopies = TileCopies<S::X_CH, kSB, HB, kWaves>;
    using BCopies = TileCopies<S::B_CH, kSB, 1, kWaves>;
    XCopies xcp;
    BCopies bcp;
    const unsigned xrow_bytes = (unsigned)(xl.row * (int64_t)sizeof(T));
    const unsigned brow_bytes = (unsigned)(ngroups * N * (int)sizeof(T));
    if constexpr (kPlanned) {
        if constexpr (EPI != 2)
            xcp.plan(wu, [&](int hh, int r, int ch) -> unsigned {
                return r * xrow_bytes +
                       (unsigned)((((h0 + min(hh, nh - 1)) / xl.hdiv) * xl.hs + ch * EPC) * (int)sizeof(T));
            });
        bcp.plan(wu, [&](int, int r, int ch) -> unsigned {
            return r * brow_bytes + (unsigned)(min(ch * S::EPB, N - S::EPB) * (int)sizeof(T));
        });
    }
    auto issue_stage = [&](int sb) {
        const int s0 = sb * kSB;
        const unsigned stg = lds_addr(region) + (sb % kStages) * S::stage_bytes;
        const int rmax = len - 1 - s0;                    // rows past it (past the sequence) read its row
        if constexpr (EPI == 2 || !kPlanned) {
            tiles_load_async<S::X_CH, kSB, HB, kWaves>(stg, S::xh_bytes, [&](int hh, int r, int ch) -> const void* {
                const int64_t tau = t0 + min(s0 + r, len - 1);
                int64_t tok = b * seqlen + tau;
                // reversed x: row tau of the reversed sequence is the caller's token seqlen - 1 - tau
                if constexpr (EPI == 2) tok = b * xl.rev_L + min((int64_t)seqlen - 1 - tau, xl.rev_L - 1);
                return x + tok * xl.row + (int64_t)((h0 + min(hh, nh - 1)) / xl.hdiv) * xl.hs + ch * EPC;
            });
        } else {
            const T* xb = x + (b * seqlen + t0 + s0) * xl.row;
            xcp.issue(wu, [&](int) -> const void* { return xb; }, stg, S::xh_bytes, rmax, xrow_bytes);
        }
        if constexpr (kPlanned) {
            const T* bb = Bm + ((b * seqlen + t0 + s0) * ngroups + g) * (int64_t)N;
            bcp.issue(wu, [&](int) -> const void* { return bb; }, stg + HB * S::xh_bytes, 0, rmax, brow_bytes);
        } else {
            const T* bg = Bm + (int64_t)g * N;
            tile_load_async<S::B_CH, kSB, kWaves>(stg + HB * S::xh_bytes, [&](int r, int ch) -> const void* {
                return bg + (b * seqlen + t0 + min(s0 + r, len - 1)) * (int64_t)ngroups * N +
                       min(ch * S::EPB, N - S::EPB);
            });
        }
    };
    if constexpr (!kAllSlabs) {
#pragma unroll
        for (int sb = 0; sb < kStages - 1; ++sb)
            if (sb < nsb) issue_stage(sb);
    }

    float dsk[HB];                                                  // skip weights D of the heads
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) dsk[hh] = Dv[h0 + min(hh, nh - 1)];
    if constexpr (kVarlen) {
        for (int l = tid; l < kMaxQ; l += kThreads) lst[l] = tstart[t0 + min(l, len - 1)] - (int)t0;
    }
    // the tables have landed once only the copies issued after them may still fly
    constexpr int kAfter = kAllSlabs ? S::NSL * (S::s_inst / kWaves)
                                     : (1 + (S::NSL > 1)) * (S::s_inst / kWaves) + (kStages - 1) * S::per_wave;
    if constexpr (!kVarlen && S::uniform && S::s_inst % kWaves == 0 && kAfter < 64) {
        if (kAllSlabs || nsb >= kStages - 1) wait_vmem_below<kAfter>();
        else wait_vmem();
    } else {
        wait_vmem();
    }
    __syncthreads();
    for (int i = tid; i < HB * kMaxQ; i += kThreads) {
        const int hh = i / kMaxQ, sidx = i % kMaxQ;
        const int e = min(kSB * (sidx / kSB) + kSB - 1, kMaxQ - 1);
        const float v = __expf(cst[hh * kMaxQ + e] - cst[i]) * dtt[i];
        if constexpr (kVarlen) vst[i] = select(sidx >= lst[e], v, 0.f);
        else vst[i] = v;
    }
    wait_vmem();                   // S_in slabs and the first stages
    __syncthreads();

    // y^T accumulators: acc[j][hh][pt] lane (r16, grp) holds y[16 rb_j + r16][16 pt + 4 grp + q]
    f32x4 acc[2][HB][P / 16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh)
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) acc[j][hh][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- inter-chunk term: exp(cs[l]) * S_in[p, :] . C_l (slab by slab when S_in does not fit whole)
#pragma unroll
    for (int sl = 0; sl < S::NSL; ++sl) {
        if (!kAllSlabs && sl > 0) {
            __syncthreads();                       // slab sl-1 consumed: its buffer takes slab sl+1
            if (sl + 1 < S::NSL) {
                issue_s(sl + 1);
                wait_vmem_below<S::s_inst / kWaves>();
            } else {
                wait_vmem();
            }
            __syncthreads();
        }
        // every S_in fragment serves both row blocks (a missing row block has zero C fragments)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            const unsigned char* stl = sbuf(sl) + hh * S::sh_bytes;
#pragma unroll
            for (int kk = 0; kk < SW / 32; ++kk)
#pragma unroll
                for (int pt = 0; pt < P / 16; ++pt) {
                    Vec8<T> af;
                    swz_load8<S::S_CH, S::S_RS>(af, stl, 16 * pt + r16, 32 * kk + 8 * grp);
                    mma(acc[0][hh][pt], af, cf[0][sl * (SW / 32) + kk]);
                    mma(acc[1][hh][pt], af, cf[1][sl * (SW / 32) + kk]);
                    if constexpr (S::kSplit) {
                        swz_load8<S::S_CH, S::S_RS>(af, stl + HB * S::sh_bytes, 16 * pt + r16, 32 * kk + 8 * grp);
                        mma(acc[0][hh][pt], af, cf[0][sl * (SW / 32) + kk]);
                        mma(acc[1][hh][pt], af, cf[1][sl * (SW / 32) + kk]);
                    }
                }
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (!has[j]) continue;
        const int l = min(16 * rbk[j] + r16, kMaxQ - 1);
        // (packed batches: only rows whose sequence holds the chunk's first token see the entering state)
        const bool carried = !kVarlen || lst[l] <= 0;
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            const float e = select(carried, __expf(cst[hh * kMaxQ + l]), 0.f);
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[j][hh][pt][q] *= e;
        }
    }

    if (S::NSL > 1) __syncthreads();               // the ring held slabs
    // stages issued before the loop: with all slabs loaded at once the first kStages go now
    int issued = kAllSlabs ? 0 : min(nsb, kStages - 1);
    if constexpr (kAllSlabs) {
#pragma unroll
        for (int sb = 0; sb < kStages; ++sb)
            if (sb < nsb) issue_stage(sb);
        issued = min(nsb, kStages);
    }
    // ---- intra-chunk term, one 32-token stage at a time
    for (int sb = 0; sb < nsb; ++sb) {
        const int s0 = sb * kSB;
        if (kAllSlabs || sb > 0) {
            // stage sb landed; the stages issued after it (up to kStages - 1) may still fly
            const int after = min(issued, nsb) - 1 - sb;
            if (S::uniform && after == kStages - 1) wait_vmem_below<(kStages - 1) * S::per_wave>();
            else if (S::uniform && kStages > 2 && after == kStages - 2) wait_vmem_below<(kStages - 2) * S::per_wave>();
            else wait_vmem();
            __syncthreads();
        }
        if (sb + kStages - 1 < nsb && sb + kStages - 1 >= issued) {
            issue_stage(sb + kStages - 1);
            issued = sb + kStages;
        }
        const unsigned char* stg = ring + (sb % kStages) * S::stage_bytes;
        const unsigned char* bt = stg + HB * S::xh_bytes;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int lb = 16 * rbk[j];                           // first row of the block
            if (!has[j] || lb + 15 < s0 || lb >= len) continue;   // block not reached yet / empty
            const int lrow = lb + r16;
            f32x4 gt[2];
#pragma unroll
            for (int st2 = 0; st2 < 2; ++st2) {
                gt[st2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NK; ++ks) {
                    Vec8<T> af;
                    swz_load8<S::B_CH>(af, bt, 16 * st2 + r16, 32 * ks + 8 * grp);
                    mma(gt[st2], af, cf[j][ks]);
                }
            }
            if (s0 + kSB <= lb) {
                // the stage lies wholly before the block: G = C.B * exp(cs[l] - cs[e]) * vst[s]
                const bool rin = !kVarlen || lst[min(lrow, kMaxQ - 1)] <= s0 + kSB - 1;
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    const float u = select(rin, __expf(cst[hh * kMaxQ + lrow] - cst[hh * kMaxQ + s0 + kSB - 1]), 0.f);
                    const float* vr = vst + hh * kMaxQ + s0 + 4 * grp;
                    const float4 va = *reinterpret_cast<const float4*>(vr);
                    const float4 vb = *reinterpret_cast<const float4*>(vr + 16);
                    Vec8<T> gf, gl;                               // gl: the lo parts (split mode)
                    const float gv[8] = {gt[0][0] * (u * va.x), gt[0][1] * (u * va.y), gt[0][2] * (u * va.z),
                                         gt[0][3] * (u * va.w), gt[1][0] * (u * vb.x), gt[1][1] * (u * vb.y),
                                         gt[1][2] * (u * vb.z), gt[1][3] * (u * vb.w)};
                    if constexpr (S::kSplit) pack8_split(gf, gl, gv);
                    else pack8(gf, gv);
                    const unsigned char* xt = stg + hh * S::xh_bytes;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> xf;
                        swz_row_slots<S::X_CH>(xf, xt, 0, 16 * pt);
                        mma(acc[j][hh][pt], xf, gf);
                        if constexpr (S::kSplit) mma(acc[j][hh][pt], xf, gl);
                    }
                }
            } else {
                // the stage holding the block's rows: full per-entry decay and the causal mask
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    const float* csr = cst + hh * kMaxQ;
                    const float* dtr = dtt + hh * kMaxQ;
                        const float cl = csr[lrow];
                    const int rst = kVarlen ? lst[min(lrow, kMaxQ - 1)] : 0;   // first token of the row's sequence
                    Vec8<T> gf, gl;                               // G[lrow][s], s = s0 + 16 st2 + 4 grp + i
                    float gv[8];
#pragma unroll
                    for (int st2 = 0; st2 < 2; ++st2) {
                        if (st2 == 1 && lb == s0) {
                            // a block at the stage's start: the stage's second 16 tokens all follow its rows
#pragma unroll
                            for (int i = 0; i < 4; ++i) gv[4 + i] = 0.f;
                            continue;
                        }
                        const int sb4 = s0 + 16 * st2 + 4 * grp;
                        const float4 c4 = *reinterpret_cast<const float4*>(csr + sb4);
                        const float4 d4 = *reinterpret_cast<const float4*>(dtr + sb4);
                        const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = gt[st2][i] * (__expf(cl - cv[i]) * dv[i]);
                            gv[4 * st2 + i] = select(sb4 + i <= lrow && (!kVarlen || sb4 + i >= rst), v, 0.f);
                        }
                    }
                    if constexpr (S::kSplit) pack8_split(gf, gl, gv);
                    else pack8(gf, gv);
                    const unsigned char* xt = stg + hh * S::xh_bytes;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        Vec8<T> xf;
                        swz_row_slots<S::X_CH>(xf, xt, 0, 16 * pt);
                        mma(acc[j][hh][pt], xf, gf);
                        if constexpr (S::kSplit) mma(acc[j][hh][pt], xf, gl);
                    }
                }
                // skip term: x of the block's own rows is in this stage's tiles
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) {
                    const T* xt = reinterpret_cast<const T*>(stg + hh * S::xh_bytes);
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        const float4 xv = swz_load4f<S::X_CH>(xt, lrow - s0, 16 * pt + 4 * grp);
                        acc[j][hh][pt][0] += dsk[hh] * xv.x;
                        acc[j][hh][pt][1] += dsk[hh] * xv.y;
                        acc[j][hh][pt][2] += dsk[hh] * xv.z;
                        acc[j][hh][pt][3] += dsk[hh] * xv.w;
                    }
                }
            }
        }
    }

    if constexpr (EPI == 1) {
        // o1 = dy . y per (token, head), from the accumulator layout: 4 columns per lane and tile,
        // then the 4 lanes of a row
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 16 * rbk[j] + r16;
            const bool rok = has[j] && row < len;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
                const bool ok = rok && hh < nh;
                const int64_t r = (b * seqlen + t0 + min(row, len - 1)) * nheads + h0 + min(hh, nh - 1);
                float dot = 0.f;
                if (ok) {
                    const bf16* dr = epi.dy + r * P + 4 * grp;
#pragma unroll
                    for (int pt = 0; pt < P / 16; ++pt) {
                        const float4 d4 = load4f(dr + 16 * pt);
                        const f32x4 v = acc[j][hh][pt];
                        dot += v[0] * d4.x + v[1] * d4.y + v[2] * d4.z + v[3] * d4.w;
                    }
                }
                dot += __shfl_xor(dot, 16, kWave);
                dot += __shfl_xor(dot, 32, kWave);
                if (ok && grp == 0)
                    epi.o1[((int64_t)b * nheads + h0 + hh) * seqlen + t0 + row] = dot;   // (batch, head, token)
            }
        }
    } else if constexpr (EPI == 2) {
        // y = du on the reversed sequence (row t0 + row is the caller's token seqlen - 1 - (t0 + row)):
        // dx = dt du + D dy, o1 = x . du, o2 = x . dy per (token, head).  One row block at a time, each
        // wavefront stages its 16 rows of all the workgroup's heads in LDS (the ring is free now) and
        // reads them back row-major, 8 consecutive columns per lane -- a token's heads are adjacent in
        // x, dy and dx, so those move as 16-byte pieces of HB * P * 2 contiguous bytes -- and P / 8
        // lanes reduce each (token, head).  (The dot pass reduces straight from the accumulators: with
        // one array to read, the staging's barriers cost it more than they save.)
        constexpr int kPitch = HB * P + 4;                     // floats per staged row
        constexpr int LPR = HB * P / 8;                        // lanes per row
        constexpr int LPH = P / 8;                             // lanes per (row, head)
        constexpr int RPI = 64 / LPR;                          // rows per pass
        constexpr int kIter = (16 + RPI - 1) / RPI;
        static_assert(kWaves * 16 * kPitch * 4 <= S::region && LPR <= 64, "epilogue staging");
        float* const ep = reinterpret_cast<float*>(region) + wave * 16 * kPitch;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            __syncthreads();                                   // the ring, or the previous row block, is free
#pragma unroll
            for (int hh = 0; hh < HB; ++hh)
#pragma unroll
                for (int pt = 0; pt < P / 16; ++pt)
                    *reinterpret_cast<f32x4*>(ep + r16 * kPitch + hh * P + 16 * pt + 4 * grp) = acc[j][hh][pt];
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kIter; ++it) {
                const int rr = it * RPI + lane / LPR, c8 = 8 * (lane % LPR);
                const int hh = c8 / P, row = 16 * rbk[j] + rr;
                const int h = h0 + min(hh, nh - 1);
                float v[8];
                {
                    const float* e = ep + min(rr, 15) * kPitch + c8;
                    const float4 a = *reinterpret_cast<const float4*>(e);
                    const float4 b4 = *reinterpret_cast<const float4*>(e + 4);
                    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                    v[4] = b4.x; v[5] = b4.y; v[6] = b4.z; v[7] = b4.w;
                }
                float s1 = 0.f, s2 = 0.f;
                const int64_t t = (int64_t)seqlen - 1 - (t0 + row);
                const bool ok = has[j] && rr < 16 && row < len && t >= 0 && t < epi.L && hh < nh;
                const int64_t tc = min(max(t, (int64_t)0), epi.L - 1);
                const int64_t r = (b * epi.L + tc) * nheads + h;
                const int64_t rt = ((int64_t)b * nheads + h) * epi.L + tc;     // (batch, head, token)
                if (ok) {
                    const float dtv = epi.dt[r], dh = epi.D[h];
                    Vec8<bf16> x8, d8, o8;
                    load8(x8, epi.x + r * P + c8 % P);
                    load8(d8, epi.dy + r * P + c8 % P);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float xv = x8.get(e), dv = d8.get(e);
                        o8.set(e, fmaf(dtv, v[e], dh * dv));
                        s1 += xv * v[e];
                        s2 += xv * dv;
                    }
                    store8(epi.dx + r * P + c8 % P, o8);
                }
#pragma unroll
                for (int m = 1; m < LPH; m <<= 1) {
                    s1 += __shfl_xor(s1, m, kWave);
                    s2 += __shfl_xor(s2, m, kWave);
                }
                if (ok && c8 % P == 0) {
                    epi.o1[rt] = s1;
                    epi.o2[rt] = s2;
                }
            }
        }
    } else if constexpr (std::is_same_v<TY, bf16>) {
        // y through LDS (the ring is free now): one row block at a time, each wavefront stages its 16
        // rows of all the workgroup's heads as bf16, then stores whole token rows -- the heads of a
        // token are adjacent in y, so a row is HB * P * 2 contiguous bytes -- in 16-byte pieces
        // 4-byte words per staged row, padded to 4 mod 32 so that the rows of a 16-byte write start 4 banks
        // apart and a write of 8 lanes (8 rows) covers every bank once
        constexpr int kRowW = HB * P / 2 + 4;
        constexpr int CPR = HB * P * 2 / 16;                    // 16-byte pieces per row
        constexpr int kIter = (16 * CPR + 63) / 64;
        static_assert(kWaves * 16 * kRowW * 4 <= S::region, "y staging");
        unsigned* const ys = reinterpret_cast<unsigned*>(region) + wave * 16 * kRowW;
        TY* yb = y + ((b * seqlen + t0) * nheads + h0) * (int64_t)P;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(yb, 0, len * nheads * P * (int)sizeof(TY), kBufferDword3);
        __syncthreads();                                        // every wavefront is done with the ring
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
                if constexpr (P >= 32) {
                    // a lane holds 4 columns of each 16-column tile; swapping the upper 16-lane row of a pair
                    // with the lower row of the next tile's values leaves 8 adjacent columns per lane, so one
                    // 16-byte write replaces two 8-byte ones: lanes of the even rows (grp 0, 2) then hold
                    // columns 32 pp + 8 (grp / 2) .. + 7, lanes of the odd rows the same 16 columns further
#pragma unroll
                    for (int pp = 0; pp < P / 32; ++pp) {
                        const uint2 a = pack4_bf16(acc[j][hh][2 * pp]), c = pack4_bf16(acc[j][hh][2 * pp + 1]);
                        const auto sx = __builtin_amdgcn_permlane16_swap(a.x, c.x, false, false);
                        const auto sy = __builtin_amdgcn_permlane16_swap(a.y, c.y, false, false);
                        const int col = 32 * pp + 16 * (grp & 1) + 8 * (grp >> 1);
                        *reinterpret_cast<uint4*>(ys + r16 * kRowW + hh * (P / 2) + col / 2) =
                            make_uint4(sx[0], sy[0], sx[1], sy[1]);
                    }
                } else {
                    *reinterpret_cast<uint2*>(ys + r16 * kRowW + hh * (P / 2) + 2 * grp) = pack4_bf16(acc[j][hh][0]);
                }
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kIter; ++it) {
                const int idx = it * 64 + lane, rr = min(idx / CPR, 15), cc = idx % CPR;
                const int row = 16 * rbk[j] + rr, hh = cc * 8 / P;
                const uint4 v = *reinterpret_cast<const uint4*>(ys + rr * kRowW + 4 * cc);
                const bool ok = idx < 16 * CPR && has[j] && row < len && hh < nh;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                                       ok ? (row * nheads * P + cc * 8) * 2 : kDropped, 0, 0);
            }
            __syncthreads();                                    // the staging area is rewritten next
        }
    } else {
        TY* yb = y + ((b * seqlen + t0) * nheads + h0) * (int64_t)P;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(yb, 0, len * nheads * P * (int)sizeof(TY), kBufferDword3);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 16 * rbk[j] + r16;
            const bool rok = has[j] && row < len;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
                const bool ok = rok && hh < nh;
#pragma unroll
                for (int pt = 0; pt < P / 16; ++pt) {
                    const int off = ok ? ((row * nheads + hh) * P + 16 * pt + 4 * grp) * (int)sizeof(TY) : kDropped;
                    buffer_store4(rs, off, 0, acc[j][hh][pt], TY{});
                }
            }
        }
    }
}

template <typename T, typename TY, int P, int NK, bool V, class S, int EPI>
hipError_t launch_shape(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                        int64_t lo_off, const float* D, const int* tstart, TY* y, const XLayout& xl, const Dims& d,
                        hipStream_t stream, const ScanEpi& epi)
{
    static_assert(S::fits, "LDS budget");
    static_assert(!S::kSplit || (std::is_same_v<T, bf16> && std::is_same_v<TY, float>),
                  "split products: bf16 operands, fp32 output");
    constexpr int HB = S::kHeads;
    const int nc = (int)d.nchunks();
    const int hpg = (int)(d.nheads / d.ngroups);
    const int nhb = (hpg + HB - 1) / HB;                 // head blocks per group
    const int hpw = (hpg + nhb - 1) / nhb;               // heads per workgroup, balanced
    const int npairs = (int)(d.chunk / 16 + 1) / 2;
    const int nhalf = (npairs + kWaves - 1) / kWaves;    // workgroups per (chunk, head block)
    const int64_t nblocks = d.batch * nc * d.ngroups * nhb * nhalf;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_scan_kernel<T, TY, P, NK, S, V, EPI>), dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                       x, B, C, dtc, cs, entry, lo_off, D, tstart, y, xl, (int)d.seqlen, (int)d.nheads, (int)d.ngroups,
                       (int)d.dstate, (int)d.chunk, nc, nhb, hpw, nhalf, (int)nblocks, epi);
    return hipGetLastError();
}

// groups of a single head (the backward's per-head passes) take the one-head shape: a wider one
// would compute a clamped copy of the head in its other slots
template <typename T, typename TY, int P, int NK, bool V, int SP, int EPI>
hipError_t launch(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                  int64_t lo_off, const float* D, const int* tstart, TY* y, const XLayout& xl, const Dims& d,
                  hipStream_t stream, const ScanEpi& epi)
{
    using S = ScanShape<T, P, NK, V, SP>;
    if constexpr (S::kHeads > 1) {
        if (d.nheads == d.ngroups) {
            using S1 = typename decltype(pick_shape<T, P, NK, 1, V, SP>())::type;
            return launch_shape<T, TY, P, NK, V, S1, EPI>(x, B, C, dtc, cs, entry, lo_off, D, tstart, y, xl, d,
                                                              stream, epi);
        }
    }
    return launch_shape<T, TY, P, NK, V, S, EPI>(x, B, C, dtc, cs, entry, lo_off, D, tstart, y, xl, d, stream,
                                                     epi);
}

template <typename T, typename TY, bool V, int SP = 1, int EPI = 0>
hipError_t launch_any(const T* x, const T* B, const T* C, const float* dtc, const float* cs, const T* entry,
                      const float* D, const int* tstart, TY* y, const Dims& d, hipStream_t stream,
                      XLayout xl = XLayout{0, 0, 0}, int64_t lo_off = 0, const ScanEpi& epi = ScanEpi{})
{
    const int64_t nk = (d.dstate + 31) / 32;
    const int nki = nk <= 1 ? 1 : nk <= 2 ? 2 : nk <= 4 ? 4 : 8;
    if (xl.hdiv == 0) {                                   // x in (B, L, H, P)
        xl.row = d.nheads * d.headdim;
        xl.hdiv = 1;
        xl.hs = (int)d.headdim;
    }
#define SSD_SCAN_CASE(PP, KK) \
    if (d.headdim == PP && nki == KK) \
        return launch<T, TY, PP, KK, V, SP, EPI>(x, B, C, dtc, cs, entry, lo_off, D, tstart, y, xl, d, stream, epi);
#define SSD_SCAN_P(PP) SSD_SCAN_CASE(PP, 1) SSD_SCAN_CASE(PP, 2) SSD_SCAN_CASE(PP, 4) SSD_SCAN_CASE(PP, 8)
    SSD_SCAN_P(16) SSD_SCAN_P(32) SSD_SCAN_P(64) SSD_SCAN_P(128)
#undef SSD_SCAN_P
#undef SSD_SCAN_CASE
    return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t launch_chunk_scan(const T* x, const T* B, const T* C, const float* dt_chunked,
                             const float* dA_cs, const T* entry_states, const float* D, T* y,
                             const Dims& d, hipStream_t stream)
{
    return launch_any<T, T, false>(x, B, C, dt_chunked, dA_cs, entry_states, D, nullptr, y, d, stream);
}

template <typename T>
hipError_t launch_chunk_scan_f32out(const T* x, const T* B, const T* C, const float* dt_chunked,
                                    const float* dA_cs, const T* entry_states, const float* D, float* y,
                                    const Dims& d, hipStream_t stream)
{
    return launch_any<T, float, false>(x, B, C, dt_chunked, dA_cs, entry_states, D, nullptr, y, d, stream);
}

template <typename T>
hipError_t launch_chunk_scan_f32out_xl(const T* x, const XLayout& xl, const T* B, const T* C, const float* dt_chunked,
                                       const float* dA_cs, const T* entry_states, const float* D, float* y,
                                       const Dims& d, hipStream_t stream)
{
    return launch_any<T, float, false>(x, B, C, dt_chunked, dA_cs, entry_states, D, nullptr, y, d, stream, xl);
}

hipError_t launch_chunk_scan_split_dot(const bf16* x, const bf16* B, const bf16* C, const float* dt_chunked,
                                       const float* dA_cs, const bf16* entry_hi, int64_t lo_off, const float* D,
                                       const ScanEpi& epi, const Dims& d, hipStream_t stream)
{
    return launch_any<bf16, float, false, 2, 1>(x, B, C, dt_chunked, dA_cs, entry_hi, D, nullptr, nullptr, d,
                                                      stream, XLayout{0, 0, 0}, lo_off, epi);
}

hipError_t launch_chunk_scan_split_grad(const bf16* x, const bf16* B, const bf16* C, const float* dt_chunked,
                                        const float* dA_cs, const bf16* entry_hi, int64_t lo_off, const float* D,
                                        const ScanEpi& epi, const Dims& d, hipStream_t stream)
{
    return launch_any<bf16, float, false, 2, 2>(x, B, C, dt_chunked, dA_cs, entry_hi, D, nullptr, nullptr, d,
                                                      stream, XLayout{0, 0, 0, epi.L}, lo_off, epi);
}

template <typename T>
hipError_t launch_chunk_scan_varlen(const T* x, const T* B, const T* C, const float* dt_chunked,
                                    const float* dA_cs, const T* entry_states, const float* D, const int* tstart,
                                    T* y, const Dims& d, hipStream_t stream)
{
    return launch_any<T, T, true>(x, B, C, dt_chunked, dA_cs, entry_states, D, tstart, y, d, stream);
}

template hipError_t launch_chunk_scan<float>(const float*, const float*, const float*, const float*,
                                             const float*, const float*, const float*, float*,
                                             const Dims&, hipStream_t);
template hipError_t launch_chunk_scan<bf16>(const bf16*, const bf16*, const bf16*, const float*,
                                            const float*, const bf16*, const float*, bf16*,
                                            const Dims&, hipStream_t);
template hipError_t launch_chunk_scan_f32out<float>(const float*, const float*, const float*, const float*,
                                                    const float*, const float*, const float*, float*,
                                                    const Dims&, hipStream_t);
template hipError_t launch_chunk_scan_f32out_xl<float>(const float*, const XLayout&, const float*, const float*,
                                                       const float*, const float*, const float*, const float*,
                                                       float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_scan_f32out_xl<bf16>(const bf16*, const XLayout&, const bf16*, const bf16*,
                                                      const float*, const float*, const bf16*, const float*, float*,
                                                      const Dims&, hipStream_t);
template hipError_t launch_chunk_scan_varlen<float>(const float*, const float*, const float*, const float*,
                                                    const float*, const float*, const float*, const int*, float*,
                                                    const Dims&, hipStream_t);
template hipError_t launch_chunk_scan_varlen<bf16>(const bf16*, const bf16*, const bf16*, const float*,
                                                   const float*, const bf16*, const float*, const int*, bf16*,
                                                   const Dims&, hipStream_t);

}  // namespace ssd
