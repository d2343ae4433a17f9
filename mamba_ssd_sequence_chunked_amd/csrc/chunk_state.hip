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
// Workgroup = (batch, chunk, up to HB heads of one group), 8 wavefronts;
// wavefront w owns head w / NSPLIT of the tile and one NSPLIT-th of the state
// columns, all P rows.  The product is formed transposed, S^T = (w B)^T x, so
// a lane holds 4 consecutive state columns of one row and stores them as one
// 16-byte segment.  Tokens are the contraction axis of both operands but the
// slow axis in memory: the heads' x tiles and the group's B tile stream
// through a 3-deep ring of 32-token stages filled by asynchronous
// global->LDS copies (XOR-swizzled by 16-byte chunk), every byte read once
// per workgroup -- so B is read once for all the heads that share it -- and
// both operands are read with the gfx950 LDS transpose read, which delivers
// 8 token slots per lane.  w is tabulated per head once per workgroup and
// applied to the B fragment in fp32 before it is rounded to the operand type;
// tokens past the sequence have w = 0 (their copies come from a clamped,
// valid row).  Workgroups are numbered head block fastest and renumbered so
// that consecutive ones share an XCD (and the chunk's B in its L2).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kSB = 32;        // tokens per stage
constexpr int kStages = 3;
constexpr int kMaxQ = 256;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <typename T, int P, int NK, int HB>
struct StateCfg {
    static constexpr int kHeads = HB;
    static constexpr int NSPLIT = kWaves / HB;                     // wavefronts per head
    static constexpr int NP = 32 * NK;                             // state width padded to 32
    // a head's (NP / 16) x (P / 16) output tiles split over its wavefronts: NSN along the state
    // columns, NSP along the rows; each wavefront takes NT x PT tiles
    static constexpr int NSN = NSPLIT < NP / 16 ? NSPLIT : NP / 16;
    static constexpr int NSP = NSPLIT / NSN;
    static constexpr int NT = NP / 16 / NSN;
    static constexpr int PT = P / 16 / NSP > 0 ? P / 16 / NSP : 1;
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int X_CH = P * (int)sizeof(T) / 16;
    static constexpr int B_CH = NP * (int)sizeof(T) / 16;
    // B rows of 256 bytes read with the transpose read take the doubled swizzle key (common.hpp)
    static constexpr int B_KM = (sizeof(T) == 2 && B_CH == 16) ? 2 : 1;
    static constexpr int xh_bytes = kSB * P * (int)sizeof(T);
    static constexpr int stage_bytes = HB * xh_bytes + kSB * NP * (int)sizeof(T);
    static constexpr int lds = kStages * stage_bytes + 4 * HB * kMaxQ;
    static constexpr int acc_regs = NT * PT * 4;
    // asynchronous copy instructions per stage, dealt over the wavefronts (uniform when divisible)
    static constexpr int x_inst = HB * kSB * X_CH / 64;
    static constexpr int b_inst = kSB * B_CH / 64;
    static constexpr bool uniform = x_inst % kWaves == 0 && b_inst % kWaves == 0;
    static constexpr int per_wave = uniform ? (x_inst + b_inst) / kWaves : 0;
    static constexpr bool fits = lds <= 160 * 1024 && NT >= 1;
    // two workgroups per CU need 4 wavefronts per SIMD, so at most 128 VGPRs: asked of the compiler
    // for the shapes whose LDS allows two workgroups and whose accumulators and fragments fit that
    // budget without spilling (bf16 or fp32 with head dimension up to 64 and state width up to 128,
    // single products); the others take what they need
    static constexpr int kMinWaves = lds <= 80 * 1024 && P <= 64 && NK <= 4 ? 4 : 2;
};

// Heads per workgroup: as many as keep a wavefront's accumulators within 64
// registers and two workgroups' LDS within a CU, so that one workgroup's
// loads and stores overlap the other's products.
template <typename T, int P, int NK, int HB>
constexpr int pick_heads() {
    using C = StateCfg<T, P, NK, HB>;
    if constexpr (HB == 1 || (C::lds <= 80 * 1024 && C::acc_regs <= 64)) return HB;
    else return pick_heads<T, P, NK, HB / 2>();
}

// kOwnCumsum: the workgroup also does stage 1 for its heads and chunk -- it reads dt (B, L, H)
// and A, forms the in-chunk prefix sums of dt A with the same arithmetic as dA_cumsum.hip (4
// tokens per lane summed in order, then a DPP wavefront prefix sum) and writes dA_cs and
// dt_chunked for the later stages -- so the chunked forward needs no separate stage-1 launch.
// kVarlen (requires kOwnCumsum): a packed variable-length batch (batch 1, sequences given by cu,
// tstart from varlen_meta.hip).  The first nblocks workgroups are the chunks': their state counts
// only the tokens of the sequence holding the chunk's last token (w = 0 before its start).  The
// nseq * ngroups * nhb workgroups after them compute, per sequence, its own part of its final
// state: the same contraction over its tokens in the chunk where it ends, decayed to its last
// token (pe) instead of the chunk's, written to final_states (nseq, H, P, N); stage 3 then adds
// the decayed entering state when the sequence began in an earlier chunk.  An empty sequence
// gets zeros.
struct VarlenArgs {
    const int* cu;               // (nseq + 1) sequence boundaries
    const int* tstart;           // (T) first token of each token's sequence
    float* final_states;         // (nseq, H, P, N)
    int nseq;
};

// kSplit (T = bf16, x and B holding bf16 values; the backward's fp32 states): the fp32 product w B is
// split into bf16 hi + lo (hi = bf16(v), lo = bf16(v - hi), together v to 2^-18) and each product is
// taken twice on the bf16 matrix cores into the fp32 accumulators.
template <typename T, int P, int NK, int HB, bool kOwnCumsum, bool kVarlen, bool kSplit = false>
__global__ __launch_bounds__(kThreads, (kSplit ? 2 : StateCfg<T, P, NK, HB>::kMinWaves)) void chunk_state_kernel(
    const T* __restrict__ x, const T* __restrict__ Bm, float* __restrict__ dt_chunked,
    float* __restrict__ dA_cs, const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ chunk_states, VarlenArgs va, int seqlen, int nheads, int ngroups, int N, int Q,
    int nc, int nhb, int hpw, int nblocks)
{
    static_assert(!kVarlen || kOwnCumsum, "the sequence workgroups form their own prefix sums");
    static_assert(!kSplit || std::is_same_v<T, bf16>, "split products take bf16 operands");
    using S = StateCfg<T, P, NK, HB>;
    constexpr int EPC = S::EPC, NT = S::NT, PT = S::PT;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * S::stage_bytes];
    __shared__ __attribute__((aligned(16))) float wt[HB * kMaxQ];

    const bool seqwg = kVarlen && (int)blockIdx.x >= nblocks;      // a sequence's final-state workgroup
    int id = seqwg ? (int)blockIdx.x - nblocks : xcd_logical_block(blockIdx.x, nblocks);
    const int hb = id % nhb; id /= nhb;
    const int g = id % ngroups; id /= ngroups;
    int c;
    int64_t b;
    int lo = 0, pe = 0, kseq = 0;                                   // token range [lo, pe] of the chunk that counts
    if (seqwg) {
        kseq = id;
        b = 0;
        const int s0 = min(max(va.cu[kseq], 0), seqlen);
        const int s1 = min(max(va.cu[kseq + 1], s0), seqlen);
        if (s1 == s0) {
            // an empty sequence: zero final state for this workgroup's heads
            const int hpg0 = nheads / ngroups;
            const int h00 = g * hpg0 + hb * hpw;
            const int nh0 = min(hpw, hpg0 - hb * hpw);
            float* f = va.final_states + ((int64_t)kseq * nheads + h00) * P * N;
            for (int i = threadIdx.x; i < nh0 * P * N; i += kThreads) f[i] = 0.f;
            return;
        }
        c = (s1 - 1) / Q;
        pe = s1 - 1 - c * Q;
        lo = max(s0 - c * Q, 0);
    } else {
        c = id % nc;
        b = id / nc;
    }
    const int hpg = nheads / ngroups;
    const int h0 = g * hpg + hb * hpw;
    const int nh = min(hpw, hpg - hb * hpw);                       // heads of this workgroup (<= HB)
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, (int64_t)seqlen - t0);
    if (!seqwg) {
        pe = len - 1;
        if constexpr (kVarlen) lo = max(va.tstart[t0 + len - 1] - (int)t0, 0);
    }
    const int nsb = (pe + kSB) / kSB;                               // stages up to token pe

    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const int r16 = lane & 15, grp = lane >> 4;
    const int hh = wave / S::NSPLIT;                               // this wavefront's head in the tile,
    const int n0 = (wave % S::NSPLIT % S::NSN) * NT * 16;          // its first state column
    const int p0 = (wave % S::NSPLIT / S::NSN) * PT * 16;          // and its first row (>= P: no rows)

    // stage copies (rows past the sequence read its last token).  Outside the pair-product mode, whose
    // registers are all taken, the per-lane source offsets are worked out once and each stage only
    // moves the base.
    constexpr bool kPlanned = !kSplit;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    TileCopies<S::X_CH, kSB, HB, kWaves> xcp;
    TileCopies<S::B_CH, kSB, 1, kWaves, 0, S::B_KM> bcp;
    const unsigned xrow_bytes = (unsigned)(nheads * P * (int)sizeof(T));
    const unsigned brow_bytes = (unsigned)(ngroups * N * (int)sizeof(T));
    if constexpr (kPlanned) {
        xcp.plan(wu, [&](int ht, int r, int ch) -> unsigned {
            return r * xrow_bytes + (unsigned)((min(ht, nh - 1) * P + ch * EPC) * (int)sizeof(T));
        });
        bcp.plan(wu, [&](int, int r, int ch) -> unsigned {
            return r * brow_bytes + (unsigned)(min(ch * EPC, N - EPC) * (int)sizeof(T));
        });
    }
    auto issue_stage = [&](int sb) {
        const int s0 = sb * kSB;
        const unsigned stg = lds_addr(ring) + (sb % kStages) * S::stage_bytes;
        if constexpr (kPlanned) {
            const int rmax = len - 1 - s0;
            const T* xs = x + ((b * seqlen + t0 + s0) * nheads + h0) * (int64_t)P;
            xcp.issue(wu, [&](int) -> const void* { return xs; }, stg, S::xh_bytes, rmax, xrow_bytes);
            const T* bs = Bm + ((b * seqlen + t0 + s0) * ngroups + g) * (int64_t)N;
            bcp.issue(wu, [&](int) -> const void* { return bs; }, stg + HB * S::xh_bytes, 0, rmax, brow_bytes);
        } else {
            const T* xs = x + (b * seqlen + t0) * (int64_t)nheads * P + (int64_t)h0 * P;
            tiles_load_async<S::X_CH, kSB, HB, kWaves>(stg, S::xh_bytes, [&](int ht, int r, int ch) -> const void* {
                return xs + (int64_t)min(s0 + r, len - 1) * nheads * P + (int64_t)min(ht, nh - 1) * P + ch * EPC;
            });
            const T* bg = Bm + (int64_t)g * N;
            tile_load_async<S::B_CH, kSB, kWaves, 0, S::B_KM>(stg + HB * S::xh_bytes, [&](int r, int ch) -> const void* {
                return bg + (b * seqlen + t0 + min(s0 + r, len - 1)) * (int64_t)ngroups * N + min(ch * EPC, N - EPC);
            });
        }
    };
#pragma unroll
    for (int sb = 0; sb < kStages - 1; ++sb)
        if (sb < nsb) issue_stage(sb);

    // w_l = dt_l exp(cs[Q-1] - cs[l]) per head, 0 past the sequence and for heads past the workgroup
    if constexpr (!kOwnCumsum) {
        for (int i = tid; i < HB * kMaxQ; i += kThreads) {
            const int ht = i / kMaxQ, l = i % kMaxQ;
            const int64_t base = (((int64_t)b * nheads + h0 + min(ht, nh - 1)) * nc + c) * Q;
            const float w = dt_chunked[base + min(l, Q - 1)] * __expf(dA_cs[base + Q - 1] - dA_cs[base + min(l, Q - 1)]);
            wt[i] = select(l < len && ht < nh, w, 0.f);
        }
    } else if (wave < HB) {
        // wavefront hh = wave scans its head: lane owns tokens 4 lane .. 4 lane + 3
        const int hs = h0 + min(wave, nh - 1);
        const float a = A[hs];
        float v[4], cs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int l = 4 * lane + j;
            v[j] = l < len ? dt[(b * seqlen + t0 + l) * nheads + hs] : 0.f;
        }
        cs[0] = v[0] * a;
#pragma unroll
        for (int j = 1; j < 4; ++j) cs[j] = cs[j - 1] + v[j] * a;
        const float incl = wave_inclusive_sum(cs[3]);
        const float excl = incl - cs[3];
#pragma unroll
        for (int j = 0; j < 4; ++j) cs[j] += excl;
        // cs[pe]: the decay reference (pe = Q - 1 for a whole chunk; cs is flat past the sequence)
        const int pq = kVarlen ? pe : Q - 1;
        const float cq = (pq & 3) == 0 ? cs[0] : (pq & 3) == 1 ? cs[1] : (pq & 3) == 2 ? cs[2] : cs[3];
        const float last = __shfl(cq, pq / 4, kWave);
        if (!seqwg && wave < nh && 4 * lane + 3 < Q) {
            const int64_t base = (((int64_t)b * nheads + hs) * nc + c) * Q + 4 * lane;
            store4(dA_cs + base, cs[0], cs[1], cs[2], cs[3]);
            store4(dt_chunked + base, v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int l = 4 * lane + j;
            wt[wave * kMaxQ + l] = select(l >= lo && l <= pe && wave < nh, v[j] * __expf(last - cs[j]), 0.f);
        }
    }
    wait_vmem();                       // the first stages and the tables' loads
    __syncthreads();

    // S^T accumulators: acc[nt][pt] lane (r16, grp) holds S[p0 + 16 pt + r16][n0 + 16 nt + 4 grp + q]
    f32x4 acc[NT][PT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[nt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int pr = min(p0, P - 16 * PT);                            // rows read (a wavefront past P reads valid rows)

    for (int sb = 0; sb < nsb; ++sb) {
        if (sb > 0) {
            // stage sb landed; the kStages - 2 stages issued after it may still fly
            if (S::uniform && kStages > 2 && sb + kStages - 2 < nsb) wait_vmem_below<(kStages - 2) * S::per_wave>();
            else wait_vmem();
            __syncthreads();
        }
        if (sb + kStages - 1 < nsb) issue_stage(sb + kStages - 1);
        const unsigned char* stg = ring + (sb % kStages) * S::stage_bytes;
        const unsigned char* xt = stg + hh * S::xh_bytes;
        const unsigned char* bt = stg + HB * S::xh_bytes;
        // w of this lane's 8 token slots (tokens 4 grp + m and 16 + 4 grp + m of the stage)
        const float* wr = wt + hh * kMaxQ + sb * kSB + 4 * grp;
        const float4 wa = *reinterpret_cast<const float4*>(wr);
        const float4 wb = *reinterpret_cast<const float4*>(wr + 16);
        const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        Vec8<T> xf[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) swz_row_slots<S::X_CH>(xf[pt], xt, 0, pr + 16 * pt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            Vec8<T> bf, bl;                                   // bl: the lo parts (split mode)
            swz_row_slots<S::B_CH, S::B_KM>(bf, bt, 0, n0 + 16 * nt);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = bf.get(e) * wv[e];
                if constexpr (kSplit) split_set(bf, bl, e, v);
                else bf.set(e, v);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                mma(acc[nt][pt], bf, xf[pt]);
                if constexpr (kSplit) mma(acc[nt][pt], bl, xf[pt]);
            }
        }
    }

    // The states leave through LDS (the ring is free now), RB row blocks at a time: each wavefront
    // stages its rows and stores them back as contiguous row pieces of NT * 16 floats, 16 bytes per
    // lane, instead of 64-byte pieces of 16 rows (when a ring is too small for one row block of
    // every wavefront, and in the pair-product mode, where the staging measured slower, the
    // accumulators are stored directly).
    constexpr int kPitch = NT * 16 + 4;                          // floats per staged row
    constexpr int kRing = kStages * S::stage_bytes;
    constexpr int kBlock = kWaves * 16 * kPitch * 4;             // one row block of every wavefront
    constexpr int RB = kBlock * PT <= kRing ? PT : (PT % 2 == 0 && kBlock * (PT / 2) <= kRing) ? PT / 2 : 1;
    constexpr int kPieces = NT * 4;                               // 16-byte pieces per staged row
    const bool live = hh < nh && p0 < P;
    float* out = seqwg ? va.final_states + (((int64_t)kseq * nheads + h0 + min(hh, nh - 1)) * P) * N
                       : chunk_states + ((((int64_t)b * nc + c) * nheads + h0 + min(hh, nh - 1)) * P) * N;
    if constexpr (kBlock <= kRing && !kSplit) {
        float* const st = reinterpret_cast<float*>(ring) + wave * RB * 16 * kPitch;
#pragma unroll
        for (int r0 = 0; r0 < PT; r0 += RB) {
            __syncthreads();                   // the ring (first round) or the previous round is free
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int q = 0; q < RB; ++q)
                    *reinterpret_cast<f32x4*>(st + (16 * q + r16) * kPitch + 16 * nt + 4 * grp) = acc[nt][r0 + q];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < RB * 16 * kPieces / 64; ++i) {
                const int idx = i * 64 + lane, row = idx / kPieces, pc = idx % kPieces;
                const int n = n0 + 4 * pc;
                const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * kPitch + 4 * pc);
                if (live && n < N) *reinterpret_cast<f32x4*>(out + (int64_t)(p0 + 16 * r0 + row) * N + n) = v;
            }
        }
    } else if (live) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = n0 + 16 * nt + 4 * grp;
            if (n < N) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    *reinterpret_cast<f32x4*>(out + (int64_t)(p0 + 16 * pt + r16) * N + n) = acc[nt][pt];
            }
        }
    }
}

template <typename T, int P, int NK, bool OWN, bool VARLEN, bool SPLIT>
hipError_t launch(const T* x, const T* B, float* dtc, float* cs, const float* dt, const float* A, float* out,
                  const VarlenArgs& va, const Dims& d, hipStream_t stream)
{
    constexpr int HB = pick_heads<T, P, NK, 8>();
    static_assert(StateCfg<T, P, NK, HB>::fits, "LDS budget");
    const int nc = (int)d.nchunks();
    const int hpg = (int)(d.nheads / d.ngroups);
    const int nhb = (hpg + HB - 1) / HB;
    const int hpw = (hpg + nhb - 1) / nhb;
    const int64_t nblocks = d.batch * nc * d.ngroups * nhb;
    const int64_t nseqwg = VARLEN ? (int64_t)va.nseq * d.ngroups * nhb : 0;
    if (nblocks + nseqwg == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_state_kernel<T, P, NK, HB, OWN, VARLEN, SPLIT>), dim3((unsigned)(nblocks + nseqwg)),
                       dim3(kThreads), 0, stream, x, B, dtc, cs, dt, A, out, va, (int)d.seqlen, (int)d.nheads,
                       (int)d.ngroups, (int)d.dstate, (int)d.chunk, nc, nhb, hpw, (int)nblocks);
    return hipGetLastError();
}

template <typename T, bool OWN, bool VARLEN, bool SPLIT = false>
hipError_t launch_any(const T* x, const T* B, float* dtc, float* cs, const float* dt, const float* A, float* out,
                      const VarlenArgs& va, const Dims& d, hipStream_t stream)
{
    const int64_t nk = (d.dstate + 31) / 32;
    const int nki = nk <= 1 ? 1 : nk <= 2 ? 2 : nk <= 4 ? 4 : 8;
#define SSD_CS_CASE(PP, KK) \
    if (d.headdim == PP && nki == KK) return launch<T, PP, KK, OWN, VARLEN, SPLIT>(x, B, dtc, cs, dt, A, out, va, d, stream);
#define SSD_CS_P(PP) SSD_CS_CASE(PP, 1) SSD_CS_CASE(PP, 2) SSD_CS_CASE(PP, 4) SSD_CS_CASE(PP, 8)
    SSD_CS_P(16) SSD_CS_P(32) SSD_CS_P(64) SSD_CS_P(128)
#undef SSD_CS_P
#undef SSD_CS_CASE
    return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t launch_chunk_state(const T* x, const T* B, const float* dt_chunked, const float* dA_cs,
                              float* chunk_states, const Dims& d, hipStream_t stream)
{
    // stage 2 alone: the prefix sums come from stage 1 and are only read
    return launch_any<T, false, false>(x, B, const_cast<float*>(dt_chunked), const_cast<float*>(dA_cs), nullptr,
                                       nullptr, chunk_states, VarlenArgs{}, d, stream);
}

template <typename T>
hipError_t launch_chunk_state_cumsum(const T* x, const T* B, const float* dt, const float* A, float* dt_chunked,
                                     float* dA_cs, float* chunk_states, const Dims& d, hipStream_t stream)
{
    return launch_any<T, true, false>(x, B, dt_chunked, dA_cs, dt, A, chunk_states, VarlenArgs{}, d, stream);
}

hipError_t launch_chunk_state_split(const bf16* x, const bf16* B, const float* dt_chunked, const float* dA_cs,
                                    float* chunk_states, const Dims& d, hipStream_t stream)
{
    return launch_any<bf16, false, false, true>(x, B, const_cast<float*>(dt_chunked), const_cast<float*>(dA_cs),
                                                nullptr, nullptr, chunk_states, VarlenArgs{}, d, stream);
}

hipError_t launch_chunk_state_cumsum_split(const bf16* x, const bf16* B, const float* dt, const float* A,
                                           float* dt_chunked, float* dA_cs, float* chunk_states, const Dims& d,
                                           hipStream_t stream)
{
    return launch_any<bf16, true, false, true>(x, B, dt_chunked, dA_cs, dt, A, chunk_states, VarlenArgs{}, d, stream);
}

template <typename T>
hipError_t launch_chunk_state_varlen(const T* x, const T* B, const float* dt, const float* A, const int* cu,
                                     int64_t nseq, const int* tstart, float* dt_chunked, float* dA_cs,
                                     float* chunk_states, float* final_states, const Dims& d, hipStream_t stream)
{
    const VarlenArgs va{cu, tstart, final_states, (int)nseq};
    return launch_any<T, true, true>(x, B, dt_chunked, dA_cs, dt, A, chunk_states, va, d, stream);
}

template hipError_t launch_chunk_state<float>(const float*, const float*, const float*, const float*,
                                              float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state<bf16>(const bf16*, const bf16*, const float*, const float*,
                                             float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state_cumsum<float>(const float*, const float*, const float*, const float*,
                                                     float*, float*, float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state_cumsum<bf16>(const bf16*, const bf16*, const float*, const float*,
                                                    float*, float*, float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state_varlen<float>(const float*, const float*, const float*, const float*,
                                                    const int*, int64_t, const int*, float*, float*, float*,
                                                    float*, const Dims&, hipStream_t);
template hipError_t launch_chunk_state_varlen<bf16>(const bf16*, const bf16*, const float*, const float*,
                                                   const int*, int64_t, const int*, float*, float*, float*,
                                                   float*, const Dims&, hipStream_t);

}  // namespace ssd
