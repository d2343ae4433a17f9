// bwd.hip - gradients of the chunked forward (the training pass).
//
// For a loss L with dL/dy = dy and dL/d(final state) = dfinal, the adjoint state
// g_t = dL/dh_t obeys g_{t-1} = a_t g_t + dy_{t-1} C_{t-1}^T: the same kind of linear
// recurrence as the forward, run backwards in time with dy as its input and C in the role of B.
// The pass therefore reuses the forward's stage kernels, each fed the arrays that put the wanted
// quantity in the place of y:
//
//   forward recompute    chunk states, entry states S_in, the final state, and yhat = y - D x
//                        (chunk_scan with D = 0; bf16 inputs: reduced to dy . yhat per token as it
//                        leaves the accumulators)
//   adjoint chunk states Ghat_c = sum_{s in c} exp(cs[s]) dy_s C_s^T   (chunk_state with w = exp(cs))
//   adjoint passing      Gout[c] (adjoint at chunk c's last token from later tokens), backwards
//                        over chunks from dfinal; what is left at the front is dinit = a_0 g_0
//   du = g B             chunk_scan on the time-reversed sequence: x <- dy, B <- C, C <- B,
//                        entry <- Gout, no dt scaling, decays cs'[l'] = cs[last] - cs[l] (bf16
//                        inputs: dy read in reversed order, and du reduced as it leaves the
//                        accumulators to dx = dt du + D dy, x . du and x . dy per token)
//   dB, dC               bf16 inputs (headdim % 32 == 0, chunk % 64 == 0): summed over each group's
//                        heads inside the kernels of bwd_dbc.hip; otherwise per head -- dB by a
//                        time-reversed chunk_scan with x <- C, B <- dy, C <- u = dt x, entry <-
//                        Gout^T, dC by a chunk_scan with x <- B, B <- x (dt scaled), C <- dy, entry
//                        <- S_in^T (the head dimension as the contraction; B and C read from the
//                        group's arrays) -- and summed over the heads of each group afterwards
//   per token            with q_t = dy_t . yhat_t - u_t . du_t the gradient of the log-decay dt_t A
//                        is the suffix sum of q from t plus <dfinal, h_final> (the telescoping of
//                        <g_t, h_t> over t); it is taken within t's chunk only: the gradient at the
//                        token after the chunk (and, for bf16 inputs, also at its first token, the
//                        mean of the two exact forms) is an inner product of adjoint and forward
//                        states at the boundary, formed by the adjoint passing; then
//                        ddt = A dl + x . du, dA = sum dt dl, dD = sum x . dy
//
// The reversal pads the sequence in front to whole chunks (zero tokens, unit decay), so the
// reversed chunks line up with the forward's.
//
// The gradient of the log-decays is a suffix sum of differences of two nearly equal products per
// token, and dA sums it over all tokens: rounding the matrix-core operands to bf16 (as the forward
// does) leaves dA with errors up to several times its size (up to ~4e-5 of the size of its terms),
// against ~1e-8 with fp32 operands.  The recompute, the adjoint chunk states and the two readouts
// therefore take fp32 operands: on the fp32 matrix cores for fp32 inputs; for bf16 inputs (x, B, C,
// dy hold bf16 values) each fp32 operand -- the weighted B or C, the decay-weighted C.B^T, the
// entry and adjoint states -- is split into bf16 hi + lo (the value to 2^-18) and each product is
// taken twice on the bf16 matrix cores into fp32 sums (dA then within ~1e-7 of its terms' size).
// dB and dC take plain operands of the inputs' type; dx, dB and dC are rounded to the inputs'
// type once at the end.
#include <algorithm>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssd {

namespace {

constexpr int kT = 256;

__device__ __forceinline__ int64_t grid_stride() { return (int64_t)gridDim.x * kT; }
__device__ __forceinline__ int64_t gtid() { return (int64_t)blockIdx.x * kT + threadIdx.x; }

// original token of reversed position tau (padded length nc Q), or -1 for a padding position
__device__ __forceinline__ int64_t unrev(int64_t tau, int Q, int nc, int64_t L)
{
    const int64_t cr = tau / Q, lr = tau % Q;
    const int64_t t = (nc - 1 - cr) * (int64_t)Q + (Q - 1 - lr);
    return t < L ? t : -1;
}

// weight and decay tables of the adjoint chunk states and of the reversed passes
__global__ __launch_bounds__(kT) void bwd_tables_kernel(const float* __restrict__ cs, float* __restrict__ W,
                                                        float* __restrict__ Z, float* __restrict__ dtp,
                                                        float* __restrict__ csp, int64_t nrows, int L, int Q, int nc)
{
    for (int64_t i = gtid(); i < nrows * Q; i += grid_stride()) {
        const int64_t row = i / Q;                  // (b, h, c)
        const int l = (int)(i % Q);
        const int c = (int)(row % nc);
        const int len = min(Q, L - c * Q);
        W[i] = l < len ? __expf(cs[i]) : 0.f;
        Z[i] = 0.f;
        // reversed chunk c' = nc - 1 - c of the same (b, h), position l' = Q - 1 - l
        const int64_t rrow = row - c + (nc - 1 - c);
        const int lr = Q - 1 - l;
        const bool ok = l < len;
        dtp[rrow * Q + lr] = ok ? 1.f : 0.f;
        csp[rrow * Q + lr] = ok ? cs[row * Q + len - 1] - cs[i] : 0.f;
    }
}

// reversed (front-padded) copies, inputs in TD: dy (B, Lp, H, P) in fp32 for the fp32 adjoint readout
// (if dy_rev is given); B, C (B, Lp, G, N) in TD (the readout's B and C, and the dB pass's C, read
// per group); in TD (the operand type of the later passes) dy and u = dt x (B, Lp, H, P); eight
// elements per thread
template <typename TD>
__global__ __launch_bounds__(kT) void bwd_prep_kernel(const TD* __restrict__ x, const float* __restrict__ dt,
                                                      const TD* __restrict__ Bm, const TD* __restrict__ Cm,
                                                      const TD* __restrict__ dy, float* __restrict__ dy_rev,
                                                      TD* __restrict__ B_rev, TD* __restrict__ C_rev,
                                                      TD* __restrict__ dy_revD, TD* __restrict__ u_revD, int batch,
                                                      int64_t L, int nc, int Q, int H, int P, int N, int G)
{
    const int64_t Lp = (int64_t)nc * Q;
    // 1. per (b, tau, h): dy_rev (fp32 and TD) and u = dt x reversed (TD), P / 8 vectors each
    const int64_t n1 = dy_rev || dy_revD ? (int64_t)batch * Lp * H * (P / 8) : 0;
    for (int64_t i = gtid(); i < n1; i += grid_stride()) {
        const int v = (int)(i % (P / 8));
        const int64_t r = i / (P / 8);             // (b, tau, h)
        const int h = (int)(r % H);
        const int64_t bt = r / H;
        const int64_t b = bt / Lp, tau = bt % Lp;
        const int64_t t = unrev(tau, Q, nc, L);
        Vec8<float> a;
        Vec8<TD> ad, ud;
        if (t >= 0) {
            const int64_t o = ((b * L + t) * H + h) * P + 8 * v;
            load8(ad, dy + o);
#pragma unroll
            for (int k = 0; k < 8; ++k) a.set(k, ad.get(k));
            if (u_revD) {
                Vec8<TD> xv;
                load8(xv, x + o);
                const float d = dt[(b * L + t) * H + h];
#pragma unroll
                for (int k = 0; k < 8; ++k) ud.set(k, d * xv.get(k));
            }
        } else {
            a.zero();
            ad.zero();
            ud.zero();
        }
        if (dy_rev) store8(dy_rev + r * P + 8 * v, a);
        if (dy_revD) store8(dy_revD + r * P + 8 * v, ad);
        if (u_revD) store8(u_revD + r * P + 8 * v, ud);
    }
    // 2. per (b, tau, g): B_rev, C_rev (TD: exact, B and C hold values of the inputs' type)
    const int64_t n2 = (int64_t)batch * Lp * G * (N / 8);
    for (int64_t i = gtid(); i < n2; i += grid_stride()) {
        const int v = (int)(i % (N / 8));
        const int64_t r = i / (N / 8);             // (b, tau, g)
        const int g = (int)(r % G);
        const int64_t bt = r / G;
        const int64_t b = bt / Lp, tau = bt % Lp;
        const int64_t t = unrev(tau, Q, nc, L);
        Vec8<TD> ob, oc;
        if (t >= 0) {
            const int64_t o = ((b * L + t) * G + g) * N + 8 * v;
            load8(ob, Bm + o);
            load8(oc, Cm + o);
        } else {
            ob.zero();
            oc.zero();
        }
        store8(B_rev + r * N + 8 * v, ob);
        store8(C_rev + r * N + 8 * v, oc);
    }
}

// A state per (b, c, h) block, (P x N) row-major, transposed and split into column halves:
// dst[((k nblk + blk) Nh + j) P + p] = src[(blk P + p) N + k Nh + j], Nh = N / nsplit.  Workgroup =
// (block, half, 64-row slice): the slice goes through an LDS tile (4-byte words, rows padded by one
// word, so both phases are free of bank conflicts) with 16-byte global reads and writes.
template <typename E>
__global__ __launch_bounds__(kT) void bwd_transpose_kernel(const E* __restrict__ src, E* __restrict__ dst,
                                                           int64_t nblk, int P, int N, int nsplit)
{
    constexpr int kR = 64;                               // rows per slice
    constexpr int V = 16 / (int)sizeof(E);               // elements per 16-byte access
    constexpr int kW = 4 / (int)sizeof(E);               // elements per LDS word
    __shared__ uint32_t tile[kR * (128 / kW + 1)];
    const int Nh = N / nsplit, WS = Nh / kW + 1;
    const int npc = (P + kR - 1) / kR;
    int64_t id = blockIdx.x;
    const int pc = (int)(id % npc);
    id /= npc;
    const int k = (int)(id % nsplit);
    const int64_t blk = id / nsplit;
    const int p0 = pc * kR, rows = min(kR, P - p0);
    const E* sp = src + (blk * P + p0) * (int64_t)N + k * Nh;
    for (int i = threadIdx.x; i < rows * (Nh / V); i += kT) {
        const int r = i / (Nh / V), c = (i % (Nh / V)) * V;
        const uint4 v = *reinterpret_cast<const uint4*>(sp + (int64_t)r * N + c);
        uint32_t* t = tile + r * WS + c / kW;
        t[0] = v.x; t[1] = v.y; t[2] = v.z; t[3] = v.w;
    }
    __syncthreads();
    E* dp = dst + (((int64_t)k * nblk + blk) * Nh) * P + p0;
    if constexpr (kW == 2) {
        // a thread takes a column pair (the two halves of a word) and 8 rows: two 16-byte stores
        for (int i = threadIdx.x; i < (Nh / 2) * (rows / 8); i += kT) {
            const int pr = (i % (rows / 8)) * 8, n2 = i / (rows / 8);
            uint32_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = tile[(pr + e) * WS + n2];
            uint4 lo, hi;
            lo.x = (w[0] & 0xffffu) | (w[1] << 16); hi.x = (w[0] >> 16) | (w[1] & 0xffff0000u);
            lo.y = (w[2] & 0xffffu) | (w[3] << 16); hi.y = (w[2] >> 16) | (w[3] & 0xffff0000u);
            lo.z = (w[4] & 0xffffu) | (w[5] << 16); hi.z = (w[4] >> 16) | (w[5] & 0xffff0000u);
            lo.w = (w[6] & 0xffffu) | (w[7] << 16); hi.w = (w[6] >> 16) | (w[7] & 0xffff0000u);
            *reinterpret_cast<uint4*>(dp + (int64_t)(2 * n2) * P + pr) = lo;
            *reinterpret_cast<uint4*>(dp + (int64_t)(2 * n2 + 1) * P + pr) = hi;
        }
    } else {
        for (int i = threadIdx.x; i < Nh * (rows / 4); i += kT) {
            const int pr = (i % (rows / 4)) * 4, n = i / (rows / 4);
            uint4 o;
            o.x = tile[pr * WS + n]; o.y = tile[(pr + 1) * WS + n];
            o.z = tile[(pr + 2) * WS + n]; o.w = tile[(pr + 3) * WS + n];
            *reinterpret_cast<uint4*>(dp + (int64_t)n * P + pr) = o;
        }
    }
}

// Sum over the 64 lanes of a wavefront, in fp64; every lane gets the sum.
__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// backwards over chunks: Gout[c] = state entering from later tokens, written in reversed chunk
// order (P x N: fp32, or for TD = bf16 as bf16 hi / lo planes, the lo plane lo_off elements after
// the hi one); dinit at the end.  With them, the log-decay gradient at the first token of chunks
// 1 .. nc-1, <Gout[c-1], entry state of chunk c> (same planes as Gout), and at token 0,
// <dinit, init> (0 without an initial state), as fp64 partial sums, one per wavefront:
// Bp[((b H + h) (nc + 1) + c) nparts + part], nparts = 4 gridDim.x (slot nc is not written)
template <typename TD>
__global__ __launch_bounds__(kT) void bwd_passing_kernel(const float* __restrict__ Ghat, const float* __restrict__ cs,
                                                         const float* __restrict__ dfinal, const TD* __restrict__ entry,
                                                         const float* __restrict__ init,
                                                         void* __restrict__ Gout_rev, float* __restrict__ dinit,
                                                         double* __restrict__ Bp, int64_t lo_off, int H, int P, int N,
                                                         int Q, int nc)
{
    const int PN = P * N;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int e = blockIdx.x * (4 * kT) + 4 * threadIdx.x;
    const bool on = e < PN;                         // whole wavefronts are on or off (PN % 256 == 0)
    const int64_t bh = b * H + h;
    const int nparts = (int)gridDim.x * (kT / 64);
    const int part = (int)blockIdx.x * (kT / 64) + (int)threadIdx.x / 64;
    float4 s = on && dfinal ? *reinterpret_cast<const float4*>(dfinal + bh * PN + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = nc - 1; c >= 0; --c) {
        const int cr = nc - 1 - c;
        const int64_t go = ((b * nc + cr) * H + h) * (int64_t)PN + e;
        if (c < nc - 1) {
            double r = 0.0;
            if (on) {
                const int64_t eo = ((b * nc + c + 1) * H + h) * (int64_t)PN + e;
                float4 hv = load4f(entry + eo);
                if constexpr (std::is_same_v<TD, bf16>) {
                    const float4 lo = load4f(entry + lo_off + eo);
                    hv.x += lo.x; hv.y += lo.y; hv.z += lo.z; hv.w += lo.w;
                }
                r = (double)s.x * hv.x + (double)s.y * hv.y + (double)s.z * hv.z + (double)s.w * hv.w;
            }
            r = wave_sum_f64(r);
            if ((threadIdx.x & 63) == 0) Bp[(bh * (nc + 1) + c + 1) * nparts + part] = r;
        }
        if (!on) continue;
        if constexpr (std::is_same_v<TD, bf16>) {
            auto rem = [](float v) { return v - static_cast<float>(static_cast<bf16>(v)); };
            bf16* gh = static_cast<bf16*>(Gout_rev) + go;
            store4(gh, s.x, s.y, s.z, s.w);
            store4(gh + lo_off, rem(s.x), rem(s.y), rem(s.z), rem(s.w));
        } else {
            store4(static_cast<float*>(Gout_rev) + go, s.x, s.y, s.z, s.w);
        }
        const float4 gh = *reinterpret_cast<const float4*>(Ghat + ((b * nc + c) * H + h) * (int64_t)PN + e);
        const float dec = __expf(cs[(bh * nc + c) * Q + Q - 1]);
        s.x = fmaf(dec, s.x, gh.x);
        s.y = fmaf(dec, s.y, gh.y);
        s.z = fmaf(dec, s.z, gh.z);
        s.w = fmaf(dec, s.w, gh.w);
    }
    double r0 = 0.0;
    if (on) {
        *reinterpret_cast<float4*>(dinit + bh * PN + e) = s;
        if (init) {
            const float4 iv = *reinterpret_cast<const float4*>(init + bh * PN + e);
            r0 = (double)s.x * iv.x + (double)s.y * iv.y + (double)s.z * iv.z + (double)s.w * iv.w;
        }
    }
    r0 = wave_sum_f64(r0);
    if ((threadIdx.x & 63) == 0) Bp[bh * (nc + 1) * nparts + part] = r0;
}

// per (b, t, h) row, all rows in parallel: dx = dt du + D dy, and the scalars the decay
// gradients need: dy . yhat, x . du and x . dy (stored (batch, head, token)).
// 16 lanes share a row (P / 16 values each), so a wavefront reads four whole rows per load.
template <typename TD>
__global__ __launch_bounds__(kT) void bwd_rows_kernel(const TD* __restrict__ x, const float* __restrict__ dt,
                                                      const float* __restrict__ Dv, const TD* __restrict__ dy,
                                                      const float* __restrict__ yhat, const float* __restrict__ du_rev,
                                                      TD* __restrict__ dx, float* __restrict__ yd_out,
                                                      float* __restrict__ xdu_out, float* __restrict__ xdy_out, int64_t L,
                                                      int H, int P, int Q, int nc)
{
    const int64_t Lp = (int64_t)nc * Q;
    const int64_t b = blockIdx.y;                                // one grid row per batch row
    const int sub = threadIdx.x & 15;
    const int64_t step = (int64_t)gridDim.x * (kT / 16);
    for (int64_t row = (int64_t)blockIdx.x * (kT / 16) + threadIdx.x / 16; row < L * H; row += step) {
        const int h = (int)(row % H);
        const int64_t t = row / H;
        const int64_t r = (b * L + t) * H + h;
        const int64_t tau = (int64_t)(nc - 1 - t / Q) * Q + (Q - 1 - t % Q);
        const int64_t rr = (b * Lp + tau) * H + h;
        const float dtv = dt[r], dh = Dv[h];
        float dyy = 0.f, xdu = 0.f, xdy = 0.f;
        for (int p = 4 * sub; p < P; p += 64) {
            const float4 xv = load4f(x + r * P + p);
            const float4 dv = load4f(dy + r * P + p);
            const float4 yv = *reinterpret_cast<const float4*>(yhat + r * P + p);
            const float4 uv = *reinterpret_cast<const float4*>(du_rev + rr * P + p);
            dyy += dv.x * yv.x + dv.y * yv.y + dv.z * yv.z + dv.w * yv.w;
            xdu += xv.x * uv.x + xv.y * uv.y + xv.z * uv.z + xv.w * uv.w;
            xdy += xv.x * dv.x + xv.y * dv.y + xv.z * dv.z + xv.w * dv.w;
            store4(dx + r * P + p, fmaf(dtv, uv.x, dh * dv.x), fmaf(dtv, uv.y, dh * dv.y), fmaf(dtv, uv.z, dh * dv.z),
                   fmaf(dtv, uv.w, dh * dv.w));
        }
        dyy = group_sum<16>(dyy);
        xdu = group_sum<16>(xdu);
        xdy = group_sum<16>(xdy);
        if (sub == 0) {
            const int64_t rt = (b * H + h) * L + t;              // (batch, head, token)
            yd_out[rt] = dyy;
            xdu_out[rt] = xdu;
            xdy_out[rt] = xdy;
        }
    }
}

// per (b, h): with q_t = dy_t . yhat_t - dt_t x_t . du_t (the three scalars stored (batch, head, token),
// dt read from the chunked copy (batch, head, padded token)), the log-decay gradient dl of a token t in
// chunk k, from either end of its chunk:
//   dl_t = Bnd[k + 1] + sum_{t <= t' < (k + 1) Q} q_t'     (Bnd[nc] = <dfinal, h_final>)
//   dl_t = Bnd[k]     - sum_{k Q <= t' < t} q_t'
// Bnd[j] the gradient at token j Q, from the states (Bp).  Both forms are exact; each q carries the
// rounding of the products it is formed from (a suffix sum over the whole sequence gathered every
// later chunk's errors into each token; these stay within the chunk).  two_ended (bf16 inputs, whose
// pair products leave q the larger error) takes the mean of the two forms, which halves the largest
// weight with which one q's error enters dA; otherwise (fp32 inputs, where the boundary values' own
// rounding dominates and Bnd[k + 1] agrees best with the chunk's q) the first form alone.  Measured
// on the backward's test shapes: worst dA error 1.5e-5 (fp32) and 1.6e-3 (bf16), against 6.7e-5 with
// the mean for fp32 and 1.1e-2 with the first form for bf16.  Then ddt = A dl + x.du, and the per-(b, h) parts of
// dA = sum dt dl and dD = sum x.dy.  The sums run in fp64: thread i takes the 16 tokens ending at
// hi - 16 i, a pass covers whole chunks (hi and hi - span are chunk boundaries, so each thread's tokens
// lie in one chunk), and the suffix sum S over the whole sequence is a prefix sum over threads, from
// which the two forms are dl_t = S_t + (Bnd[k + 1] - S_{(k+1) Q}) = S_t + (Bnd[k] - S_{k Q}).
__global__ __launch_bounds__(kT) void bwd_scan_kernel(const float* __restrict__ dtc, const float* __restrict__ A,
                                                      const float* __restrict__ yd, const float* __restrict__ xdu,
                                                      const float* __restrict__ xdy,
                                                      const float* __restrict__ dfinal,
                                                      const float* __restrict__ hfinal, const double* __restrict__ Bp,
                                                      int nparts, float* __restrict__ ddt, double* __restrict__ dAp,
                                                      double* __restrict__ dDp, int64_t L, int64_t Lp, int H, int P,
                                                      int N, int Q, int nc, int two_ended)
{
    constexpr int kPer = 16;
    __shared__ double sc[kT];
    __shared__ double ex[kT];           // S + <dfinal, h_final> after each thread's tokens
    __shared__ double in[kT];           // the same from each thread's first token on
    __shared__ double corr[kT];         // per chunk of the pass: the offset of the form(s) used
    const int h = blockIdx.x % H;
    const int64_t b = blockIdx.x / H;
    const int64_t bh = b * H + h;
    const int tid = threadIdx.x;
    // inclusive prefix sum over the block's threads, in fp64 (Hillis-Steele in LDS)
    auto block_scan = [&](double v) {
        __syncthreads();
        sc[tid] = v;
        __syncthreads();
        for (int off = 1; off < kT; off <<= 1) {
            const double o = tid >= off ? sc[tid - off] : 0.0;
            __syncthreads();
            sc[tid] += o;
            __syncthreads();
        }
        return sc[tid];
    };
    auto block_sum = [&](double v) {
        block_scan(v);
        return sc[kT - 1];
    };
    auto bnd = [&](int64_t j) {                          // Bnd[j], j < nc
        const double* bp = Bp + (bh * (nc + 1) + j) * nparts;
        double r = 0.0;
        for (int i = 0; i < nparts; ++i) r += bp[i];
        return r;
    };
    double fh = 0.0;
    if (dfinal) {
        const int64_t PN = (int64_t)P * N;
        for (int64_t i = tid; i < PN; i += kT) fh += (double)dfinal[bh * PN + i] * hfinal[bh * PN + i];
    }
    fh = block_sum(fh);
    double carry = fh;
    const double a = A[h];
    double dA_acc = 0.0, dD_acc = 0.0;
    const int64_t span = (int64_t)(kT * kPer / Q) * Q;   // whole chunks per pass (Q <= 256)
    const int nact = (int)(span / kPer);                  // threads with tokens
    for (int64_t hi = (int64_t)nc * Q; hi > 0; hi -= span) {
        // this thread's tokens: [hi - kPer (tid + 1), hi - kPer tid), latest first
        const int64_t t1 = hi - (int64_t)kPer * tid;
        float qs[kPer], xs[kPer];
        double own = 0.0;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t t = t1 - 1 - k;
            float q = 0.f, xu = 0.f;
            if (tid < nact && t >= 0 && t < L) {
                const int64_t rt = bh * L + t;
                xu = xdu[rt];
                q = yd[rt] - dtc[bh * Lp + t] * xu;
                dD_acc += xdy[rt];
            }
            qs[k] = q;
            xs[k] = xu;
            own += q;
        }
        const double incl = block_scan(own);
        const double total = sc[kT - 1];
        ex[tid] = carry + incl - own;
        in[tid] = carry + incl;
        __syncthreads();
        const int64_t lo = hi - span > 0 ? hi - span : 0;
        const int64_t k0 = lo / Q, k1 = hi / Q - 1;       // the pass's chunks (at most kT of them)
        for (int64_t k = k0 + tid; k <= k1; k += kT) {
            const double right = (k + 1 < nc ? bnd(k + 1) : fh) - ex[(hi - (k + 1) * Q) / kPer];
            corr[k - k0] = two_ended ? 0.5 * (right + bnd(k) - in[(hi - k * Q) / kPer - 1]) : right;
        }
        __syncthreads();
        double run = ex[tid];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t t = t1 - 1 - k;
            run += qs[k];
            if (tid < nact && t >= 0 && t < L) {
                const double dl = run + corr[t / Q - k0];
                ddt[(b * L + t) * H + h] = (float)(a * dl + xs[k]);
                dA_acc += (double)dtc[bh * Lp + t] * dl;
            }
        }
        carry += total;
    }
    const double sa = block_sum(dA_acc);
    const double sd = block_sum(dD_acc);
    if (tid == 0) {
        dAp[bh] = sa;
        dDp[bh] = sd;
    }
}

// dB and dC: the per-head parts summed over each group's heads (dB's parts are in reversed time)
template <typename T>
__global__ __launch_bounds__(kT) void bwd_group_sum_kernel(const float* __restrict__ dBh_rev,
                                                           const float* __restrict__ dCh, T* __restrict__ dB,
                                                           T* __restrict__ dC, int batch, int64_t L, int H, int N,
                                                           int G, int Q, int nc, int nsplit)
{
    const int hpg = H / G, Nh = N / nsplit;
    const int64_t Lp = (int64_t)nc * Q;
    const int64_t n = (int64_t)batch * L * G * (N / 4);
    for (int64_t i = gtid(); i < n; i += grid_stride()) {
        const int n0 = (int)(i % (N / 4)) * 4;
        int64_t r = i / (N / 4);
        const int g = (int)(r % G);
        const int64_t bt = r / G;
        const int64_t b = bt / L, t = bt % L;
        const int64_t tau = (int64_t)(nc - 1 - t / Q) * Q + (Q - 1 - t % Q);
        const int k = n0 / Nh, j = n0 % Nh;
        float4 sb = make_float4(0.f, 0.f, 0.f, 0.f), sc = sb;
        for (int hh = 0; hh < hpg; ++hh) {
            const int h = g * hpg + hh;
            const float4 vb = *reinterpret_cast<const float4*>(dBh_rev + ((((int64_t)k * batch + b) * Lp + tau) * H + h) * Nh + j);
            const float4 vc = *reinterpret_cast<const float4*>(dCh + ((((int64_t)k * batch + b) * L + t) * H + h) * Nh + j);
            sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
            sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
        }
        const int64_t o = ((b * L + t) * G + g) * N + n0;
        store4(dB + o, sb.x, sb.y, sb.z, sb.w);
        store4(dC + o, sc.x, sc.y, sc.z, sc.w);
    }
}

__global__ __launch_bounds__(kT) void bwd_heads_kernel(const double* __restrict__ dAp, const double* __restrict__ dDp,
                                                       float* __restrict__ dA, float* __restrict__ dD, int batch, int H)
{
    for (int h = blockIdx.x * kT + threadIdx.x; h < H; h += gridDim.x * kT) {
        double sa = 0.0, sd = 0.0;
        for (int b = 0; b < batch; ++b) {
            sa += dAp[(int64_t)b * H + h];
            sd += dDp[(int64_t)b * H + h];
        }
        dA[h] = (float)sa;
        dD[h] = (float)sd;
    }
}

__global__ __launch_bounds__(kT) void fill_zero_kernel(float* __restrict__ p, int64_t n)
{
    for (int64_t i = gtid(); i < n; i += grid_stride()) p[i] = 0.f;
}

unsigned grid_for(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + kT - 1) / kT, 8192)); }

}  // namespace

BwdLayout bwd_layout(const Dims& d, int elemD)
{
    BwdLayout w;
    const int64_t nc = d.nchunks(), Lp = nc * d.chunk;
    const int64_t B = d.batch, H = d.nheads, P = d.headdim, N = d.dstate, G = d.ngroups;
    const int64_t tab = B * H * nc * d.chunk * 4;
    const int64_t st = B * nc * H * P * N;
    size_t o = 0;
    auto take = [&](int64_t bytes) { const size_t at = o; o += (size_t)((bytes + 255) / 256 * 256); return at; };
    w.cs = take(tab);
    w.dtc = take(tab);
    w.W = take(tab);
    w.Z = take(tab);
    w.dtp = take(tab);
    w.csp = take(tab);
    w.states = take(st * 4);
    w.entry = take(st * 4);
    const bool dbc0 = elemD == 2 && bwd_dbc_supported(d);
    w.SinT = take(dbc0 ? 0 : st * elemD);
    w.Gout_rev = take(st * 4);
    w.GoutT_rev = take(dbc0 ? 0 : st * elemD);
    w.hfinal = take(B * H * P * N * 4);
    w.yhat = take(elemD == 4 ? B * d.seqlen * H * P * 4 : 0);          // fp32 pass only (the bf16 one
                                                                       // reduces yhat and du in place)
    w.dy_rev = take(elemD == 4 ? B * Lp * H * P * 4 : 0);        // the fp32 readout's operand only
    w.B_rev = take(B * Lp * G * N * elemD);
    w.C_rev = take(B * Lp * G * N * elemD);
    w.dy_revD = take(elemD == 2 && bwd_dbc_supported(d) ? 0 : B * Lp * H * P * elemD);
    w.u_revD = take(elemD == 2 && bwd_dbc_supported(d) ? 0 : B * Lp * H * P * elemD);
    w.du_rev = take(elemD == 4 ? B * Lp * H * P * 4 : 0);
    // dB, dC: per-head parts summed afterwards, or (bf16 inputs) the group sums formed in the kernels
    const bool dbc = elemD == 2 && bwd_dbc_supported(d);
    w.dBh_rev = take(dbc ? 0 : B * Lp * H * N * 4);
    w.dCh = take(dbc ? 0 : B * d.seqlen * H * N * 4);
    w.Mp = take(dbc ? (int64_t)bwd_dbc_slices(d) * B * nc * G * d.chunk * d.chunk * 4 : 0);
    w.dCi = take(dbc ? (int64_t)bwd_dbc_slices(d) * B * d.seqlen * G * N * 4 : 0);   // per slice of the heads
    w.dBi = take(dbc ? (int64_t)bwd_dbc_slices(d) * B * d.seqlen * G * N * 4 : 0);
    w.zeros = take(std::max<int64_t>(H, 1) * 4);
    w.yd = take(B * d.seqlen * H * 4);
    w.xdu = take(B * d.seqlen * H * 4);
    w.xdy = take(B * d.seqlen * H * 4);
    w.dAp = take(B * H * 8);
    w.dDp = take(B * H * 8);
    w.Rp = take(B * H * (nc + 1) * ((P * N + 1023) / 1024 * 4) * 8);   // per (b, h, chunk boundary): one fp64
                                                                        // sum per wavefront
    w.total = std::max<size_t>(o, 256);
    return w;
}

namespace {

// The pass on the caller's arrays in TD (x, B, C, dy and the outputs dx, dB, dC).  fp32 inputs take
// the fp32 matrix-core path for the recompute, the adjoint states and the readouts; bf16 inputs take
// split bf16 products there (see the header), and bf16 operands for the per-head dB / dC passes.
template <typename TD>
hipError_t run_backward(const TD* x, const float* dt, const float* A, const TD* Bm, const TD* Cm, const float* D,
                        const float* init, const TD* dy, const float* dfinal, TD* dx, float* ddt, float* dA, TD* dB,
                        TD* dC, float* dD, float* dinit, const Dims& d, void* workspace, hipStream_t s)
{
    constexpr bool kBf16 = std::is_same_v<TD, bf16>;
    const BwdLayout w = bwd_layout(d, (int)sizeof(TD));
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    auto TT = [&](size_t off) { return reinterpret_cast<TD*>(ws + off); };
    const int nc = (int)d.nchunks(), Q = (int)d.chunk;
    const int B = (int)d.batch, H = (int)d.nheads, P = (int)d.headdim, N = (int)d.dstate, G = (int)d.ngroups;
    const int nsplit = N > 128 ? 2 : 1;
    const int Nh = N / nsplit;
    const int64_t L = d.seqlen, Lp = (int64_t)nc * Q;
    hipError_t e;
#define SSD_TRY(expr) do { e = (expr); if (e != hipSuccess) return e; } while (0)
    float* zeros = F(w.zeros);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(kT), 0, s, zeros, (int64_t)H);
    SSD_TRY(hipGetLastError());
    // forward recompute in fp32: chunk states, entry states, the final state, yhat = y - D x
    // (bf16 inputs: the fp32 states leave as bf16 hi / lo planes, st elements apart, and the readout
    // passes take split bf16 products)
    const int64_t st = (int64_t)B * nc * H * P * N;
    if constexpr (kBf16) {
        SSD_TRY(launch_chunk_state_cumsum_split(x, Bm, dt, A, F(w.dtc), F(w.cs), F(w.states), d, s));
        SSD_TRY(launch_state_passing_split(F(w.states), F(w.cs), init, TT(w.entry), st, F(w.hfinal), d, s));
        // yhat is reduced to dy . yhat per (token, head) as it leaves the accumulators
        const ScanEpi ey{dy, x, dt, D, nullptr, F(w.yd), nullptr, L};
        SSD_TRY(launch_chunk_scan_split_dot(x, Bm, Cm, F(w.dtc), F(w.cs), TT(w.entry), st, zeros, ey, d, s));
    } else {
        SSD_TRY(launch_chunk_state_cumsum<float>(x, Bm, dt, A, F(w.dtc), F(w.cs), F(w.states), d, s));
        SSD_TRY(launch_state_passing<float>(F(w.states), F(w.cs), init, F(w.entry), F(w.hfinal), d, s));
        SSD_TRY(launch_chunk_scan_f32out<float>(x, Bm, Cm, F(w.dtc), F(w.cs), F(w.entry), zeros, F(w.yhat), d, s));
    }
    // tables, adjoint chunk states (into the chunk-state buffer, free again), adjoint passing
    const int64_t nrows = (int64_t)B * H * nc;
    hipLaunchKernelGGL(bwd_tables_kernel, dim3(grid_for(nrows * Q)), dim3(kT), 0, s, F(w.cs), F(w.W), F(w.Z), F(w.dtp),
                       F(w.csp), nrows, (int)L, Q, nc);
    SSD_TRY(hipGetLastError());
    if constexpr (kBf16) SSD_TRY(launch_chunk_state_split(dy, Cm, F(w.W), F(w.Z), F(w.states), d, s));
    else SSD_TRY(launch_chunk_state<float>(dy, Cm, F(w.W), F(w.Z), F(w.states), d, s));
    const unsigned npass = (unsigned)((P * N + 4 * kT - 1) / (4 * kT));
    const int nparts = (int)npass * (kT / 64);
    hipLaunchKernelGGL((bwd_passing_kernel<TD>), dim3(npass, (unsigned)H, (unsigned)B), dim3(kT), 0, s, F(w.states),
                       F(w.cs), dfinal, TT(w.entry), init, (void*)(ws + w.Gout_rev), dinit,
                       reinterpret_cast<double*>(ws + w.Rp), st, H, P, N, Q, nc);
    SSD_TRY(hipGetLastError());
    // reversed and per-head copies, S_in^T
    // (bf16 inputs: the du pass reads dy itself in reversed order; the reversed dy and u copies serve the
    // per-head dB pass only)
    float* const dy_rev32 = kBf16 ? nullptr : F(w.dy_rev);
    const bool dbc = kBf16 && bwd_dbc_supported(d);          // dB, dC summed over heads in the kernels
    const int64_t nprep = std::max<int64_t>(dbc ? 0 : (int64_t)B * Lp * H * (P / 8), (int64_t)B * Lp * G * (N / 8));
    hipLaunchKernelGGL((bwd_prep_kernel<TD>), dim3(grid_for(nprep)), dim3(kT), 0, s, x, dt, Bm, Cm, dy, dy_rev32,
                       TT(w.B_rev), TT(w.C_rev), dbc ? nullptr : TT(w.dy_revD), dbc ? nullptr : TT(w.u_revD), B, L, nc,
                       Q, H, P, N, G);
    SSD_TRY(hipGetLastError());
    // S_in^T and Gout^T for the per-head dC and dB passes (bf16 inputs: of their hi planes)
    const unsigned ntr = dbc ? 0u : (unsigned)(nrows * nsplit * ((P + 63) / 64));
    if (ntr > 0) {
        hipLaunchKernelGGL((bwd_transpose_kernel<TD>), dim3(ntr), dim3(kT), 0, s, TT(w.entry), TT(w.SinT), nrows, P,
                           N, nsplit);
        hipLaunchKernelGGL((bwd_transpose_kernel<TD>), dim3(ntr), dim3(kT), 0, s, TT(w.Gout_rev), TT(w.GoutT_rev),
                           nrows, P, N, nsplit);
    }
    SSD_TRY(hipGetLastError());
    // du: the adjoint readout, on the reversed sequence, in fp32
    const Dims dr{d.batch, Lp, d.nheads, d.headdim, d.dstate, d.ngroups, d.chunk};
    if constexpr (kBf16) {
        // du leaves the accumulators as dx = dt du + D dy, x . du and x . dy
        const ScanEpi eu{dy, x, dt, D, dx, F(w.xdu), F(w.xdy), L};
        SSD_TRY(launch_chunk_scan_split_grad(dy, TT(w.C_rev), TT(w.B_rev), F(w.dtp), F(w.csp), TT(w.Gout_rev), st,
                                             zeros, eu, dr, s));
    } else
        SSD_TRY(launch_chunk_scan_f32out<float>(F(w.dy_rev), F(w.C_rev), F(w.B_rev), F(w.dtp), F(w.csp),
                                                F(w.Gout_rev), zeros, F(w.du_rev), dr, s));
    // dB and dC: the group sums formed in the kernels (bwd_dbc.hip), or per-head dB (reversed) and dC,
    // contraction over the head dimension, one call per column half, summed over heads afterwards
    // (the x role, C reversed or B, read from the group's array by every head of the group)
    if constexpr (kBf16) {
        if (dbc)
            SSD_TRY(launch_bwd_dbc(x, dy, Bm, Cm, F(w.dtc), F(w.cs), TT(w.entry), TT(w.Gout_rev), F(w.Mp), F(w.dCi),
                                   F(w.dBi), dB, dC, d, s));
    }
    const Dims dbd{d.batch, Lp, d.nheads, Nh, d.headdim, d.nheads, d.chunk};
    const Dims dcd{d.batch, L, d.nheads, Nh, d.headdim, d.nheads, d.chunk};
    const XLayout xg{(int64_t)G * N, H / G, N};
    for (int k = 0; k < (dbc ? 0 : nsplit); ++k) {
        SSD_TRY(launch_chunk_scan_f32out_xl<TD>(TT(w.C_rev) + (int64_t)k * Nh, xg, TT(w.dy_revD), TT(w.u_revD),
                                                F(w.dtp), F(w.csp), TT(w.GoutT_rev) + (int64_t)k * B * nc * H * Nh * P,
                                                zeros, F(w.dBh_rev) + (int64_t)k * B * Lp * H * Nh, dbd, s));
        SSD_TRY(launch_chunk_scan_f32out_xl<TD>(Bm + (int64_t)k * Nh, xg, x, dy, F(w.dtc), F(w.cs),
                                                TT(w.SinT) + (int64_t)k * B * nc * H * Nh * P, zeros,
                                                F(w.dCh) + (int64_t)k * B * L * H * Nh, dcd, s));
    }
    // per token (all rows in parallel), then the suffix sums per (b, h), then the group and batch sums
    {
        if (!kBf16) {
            hipLaunchKernelGGL((bwd_rows_kernel<TD>), dim3(grid_for(L * H * 16), (unsigned)B), dim3(kT), 0, s, x, dt, D,
                               dy, F(w.yhat), F(w.du_rev), dx, F(w.yd), F(w.xdu), F(w.xdy), L, H, P, Q, nc);
            SSD_TRY(hipGetLastError());
        }
        hipLaunchKernelGGL(bwd_scan_kernel, dim3((unsigned)(B * H)), dim3(kT), 0, s, F(w.dtc), A, F(w.yd), F(w.xdu),
                           F(w.xdy), dfinal, F(w.hfinal), reinterpret_cast<const double*>(ws + w.Rp), nparts, ddt,
                           reinterpret_cast<double*>(ws + w.dAp), reinterpret_cast<double*>(ws + w.dDp), L, Lp, H, P,
                           N, Q, nc, kBf16 ? 1 : 0);
        SSD_TRY(hipGetLastError());
    }
    if (!dbc) {
        hipLaunchKernelGGL((bwd_group_sum_kernel<TD>), dim3(grid_for((int64_t)B * L * G * (N / 4))), dim3(kT), 0, s,
                           F(w.dBh_rev), F(w.dCh), dB, dC, B, L, H, N, G, Q, nc, nsplit);
        SSD_TRY(hipGetLastError());
    }
    hipLaunchKernelGGL(bwd_heads_kernel, dim3(1), dim3(kT), 0, s, reinterpret_cast<double*>(ws + w.dAp),
                       reinterpret_cast<double*>(ws + w.dDp), dA, dD, B, H);
    SSD_TRY(hipGetLastError());
#undef SSD_TRY
    return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(const Dims& d, bool bf16_inputs)
{
    return bwd_layout(d, bf16_inputs ? 2 : 4).total;
}

hipError_t launch_backward_f32(const float* x, const float* dt, const float* A, const float* Bm, const float* Cm,
                               const float* D, const float* init, const float* dy, const float* dfinal, float* dx,
                               float* ddt, float* dA, float* dB, float* dC, float* dD, float* dinit, const Dims& d,
                               void* workspace, hipStream_t s)
{
    return run_backward<float>(x, dt, A, Bm, Cm, D, init, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit, d, workspace, s);
}

hipError_t launch_backward_bf16(const bf16* x, const float* dt, const float* A, const bf16* Bm, const bf16* Cm,
                                const float* D, const float* init, const bf16* dy, const float* dfinal, bf16* dx,
                                float* ddt, float* dA, bf16* dB, bf16* dC, float* dD, float* dinit, const Dims& d,
                                void* workspace, hipStream_t s)
{
    return run_backward<bf16>(x, dt, A, Bm, Cm, D, init, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit, d, workspace, s);
}

}  // namespace ssd
