// kernels.hpp - host-side launchers of the SSD kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Dims {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int64_t nchunks() const { return (seqlen + chunk - 1) / chunk; }
};

// Where stage 4 finds the x row of token t, head h: x + t * row + (h / hdiv) * hs (elements); the
// caller's (B, L, H, P) array is {H * P, 1, P}.  The backward's per-head passes read an array shared
// by the heads of a group ({G * N, H / G, N}).
struct XLayout {
    int64_t row;
    int hdiv, hs;
    // the caller's sequence length when x is read in reversed token order (the du pass): row tau of the
    // padded (seqlen) sequence is the caller's token seqlen - 1 - tau, clamped to rev_L - 1 for the
    // front padding (whose weights are zero)
    int64_t rev_L;
};

hipError_t launch_dA_cumsum(const float* dt, const float* A, float* dA_cs, float* dt_chunked,
                            const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_chunk_state(const T* x, const T* B, const float* dt_chunked, const float* dA_cs,
                              float* chunk_states, const Dims& d, hipStream_t stream);

// stage 2 with stage 1 folded in: also writes dA_cs and dt_chunked from dt and A
template <typename T>
hipError_t launch_chunk_state_cumsum(const T* x, const T* B, const float* dt, const float* A, float* dt_chunked,
                                     float* dA_cs, float* chunk_states, const Dims& d, hipStream_t stream);

// stage 2 (alone / with stage 1) in fp32 from bf16 products: x and B given in bf16 (arrays that hold bf16
// values), the weighted B split into bf16 hi + lo (each product to within 2^-18)
hipError_t launch_chunk_state_split(const bf16* x, const bf16* B, const float* dt_chunked, const float* dA_cs,
                                    float* chunk_states, const Dims& d, hipStream_t stream);
hipError_t launch_chunk_state_cumsum_split(const bf16* x, const bf16* B, const float* dt, const float* A,
                                           float* dt_chunked, float* dA_cs, float* chunk_states, const Dims& d,
                                           hipStream_t stream);

// packed variable-length batches (d.batch == 1, d.seqlen = total tokens)
hipError_t launch_varlen_meta(const int* cu_seqlens, int64_t nseq, int64_t total, int64_t chunk, int* tstart,
                              int* cmeta, hipStream_t stream);

template <typename T>
hipError_t launch_chunk_state_varlen(const T* x, const T* B, const float* dt, const float* A, const int* cu,
                                     int64_t nseq, const int* tstart, float* dt_chunked, float* dA_cs,
                                     float* chunk_states, float* final_states, const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_state_passing_varlen(const float* chunk_states, const float* dA_cs, const int* cmeta,
                                       T* entry_states, float* final_states, const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_chunk_scan_varlen(const T* x, const T* B, const T* C, const float* dt_chunked,
                                    const float* dA_cs, const T* entry_states, const float* D, const int* tstart,
                                    T* y, const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_state_passing(const float* chunk_states, const float* dA_cs, const float* init,
                                T* entry_states, float* final_states, const Dims& d,
                                hipStream_t stream);
// the entry states as bf16 hi / lo planes (hi = bf16(S), lo = bf16(S - hi); lo plane at entry_hi + lo_off)
hipError_t launch_state_passing_split(const float* chunk_states, const float* dA_cs, const float* init,
                                      bf16* entry_hi, int64_t lo_off, float* final_states, const Dims& d,
                                      hipStream_t stream);

template <typename T>
hipError_t launch_chunk_scan(const T* x, const T* B, const T* C, const float* dt_chunked,
                             const float* dA_cs, const T* entry_states, const float* D, T* y,
                             const Dims& d, hipStream_t stream);

// stage 4 with y stored in fp32 (no rounding to T)
template <typename T>
hipError_t launch_chunk_scan_f32out(const T* x, const T* B, const T* C, const float* dt_chunked,
                                    const float* dA_cs, const T* entry_states, const float* D, float* y,
                                    const Dims& d, hipStream_t stream);

// stage 4 with y in fp32 and x read through an XLayout
template <typename T>
hipError_t launch_chunk_scan_f32out_xl(const T* x, const XLayout& xl, const T* B, const T* C, const float* dt_chunked,
                                       const float* dA_cs, const T* entry_states, const float* D, float* y,
                                       const Dims& d, hipStream_t stream);

// the backward's readouts for bf16 inputs: fp32 results to within 2^-18 of each product from bf16
// products -- x, B, C given in bf16 (arrays that hold bf16 values), the entry states as two bf16
// planes (hi at entry_hi, lo at entry_hi + lo_off), the fp32 decayed scores split likewise in
// registers.
// The backward's readout passes with the per-token work folded into the output stage (y not stored):
// (o1, o2 indexed (batch, head, token))
//   ..._dot:  o1[b, h, t] = sum_p dy[b, t, h, p] y[b, t, h, p]
//   ..._grad: y = du on the time-reversed, front-padded sequence (token t = Lp - 1 - row, pads
//             skipped): dx = dt du + D dy (bf16), o1 = x . du, o2 = x . dy per (b, h, t); its x
//             operand is the caller's dy (B, L, H, P), read in reversed token order
struct ScanEpi {
    const bf16* dy;
    const bf16* x;
    const float* dt;      // (B, L, H)
    const float* D;       // (H)
    bf16* dx;
    float* o1;
    float* o2;
    int64_t L;            // the caller's sequence length
};
hipError_t launch_chunk_scan_split_dot(const bf16* x, const bf16* B, const bf16* C, const float* dt_chunked,
                                       const float* dA_cs, const bf16* entry_hi, int64_t lo_off, const float* D,
                                       const ScanEpi& epi, const Dims& d, hipStream_t stream);
hipError_t launch_chunk_scan_split_grad(const bf16* x, const bf16* B, const bf16* C, const float* dt_chunked,
                                        const float* dA_cs, const bf16* entry_hi, int64_t lo_off, const float* D,
                                        const ScanEpi& epi, const Dims& d, hipStream_t stream);

// the forward as one pass over the sequence per (batch, head), the state on chip (fused.hip):
// headdim * (dstate rounded up to 32, 64, 128 or 256) <= 16384
bool fused_supported(const Dims& d);
template <typename T>
hipError_t launch_ssd_fused(const T* x, const float* dt, const float* A, const T* B, const T* C, const float* D,
                            const float* init, T* y, float* final_states, const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_ssd_step(float* state, const T* x, const float* dt, const float* A, const T* B,
                           const T* C, const float* D, T* y, const Dims& d, hipStream_t stream);

template <typename T>
hipError_t launch_selective_scan(const T* x, const float* delta, const float* A, const T* B, const T* C,
                                 const float* D, const float* init, T* y, float* final_states, int64_t batch,
                                 int64_t seqlen, int64_t dim, int64_t dstate, hipStream_t stream);

// the backward pass (bwd.hip): workspace parts (byte offsets) and the launcher
struct BwdLayout {
    size_t cs, dtc, W, Z, dtp, csp, states, entry, SinT, Gout_rev, GoutT_rev, hfinal, yhat, dy_rev, B_rev,
        C_rev, dy_revD, u_revD, du_rev, dBh_rev, dCh, Mp, dCi, dBi, zeros, yd, xdu, xdy, dAp, dDp, Rp, total;
};
// dB and dC summed over the heads inside the kernels (bwd_dbc.hip): bf16 inputs, headdim % 32 == 0,
// chunk % 64 == 0; Mp holds bwd_dbc_slices() partial sums of the (B, nc, G, Q, Q) score matrices,
// dCi / dBi as many partial sums of the (B, L, G, N) state terms (the heads split into slices)
bool bwd_dbc_supported(const Dims& d);
int bwd_dbc_slices(const Dims& d);
// (Sin: the entry states' hi plane (B, nc, H, P, N); Gout_rev: the adjoint states' hi plane, reversed
// chunk order)
hipError_t launch_bwd_dbc(const bf16* x, const bf16* dy, const bf16* B, const bf16* C, const float* dtc,
                          const float* cs, const bf16* Sin, const bf16* Gout_rev, float* Mp, float* dCi, float* dBi,
                          bf16* dB, bf16* dC, const Dims& d, hipStream_t stream);
BwdLayout bwd_layout(const Dims& d, int elem_bytes);
size_t bwd_workspace_bytes(const Dims& d, bool bf16_inputs);

// bf16 inputs: the precision-critical products as split bf16 pairs (fp32 to 2^-18), the dB / dC
// passes on the bf16 operands, dx / dB / dC rounded to bf16 once (see bwd.hip)
hipError_t launch_backward_bf16(const bf16* x, const float* dt, const float* A, const bf16* B, const bf16* C,
                                const float* D, const float* init, const bf16* dy, const float* dfinal, bf16* dx,
                                float* ddt, float* dA, bf16* dB, bf16* dC, float* dD, float* dinit, const Dims& d,
                                void* workspace, hipStream_t stream);

hipError_t launch_backward_f32(const float* x, const float* dt, const float* A, const float* B, const float* C,
                               const float* D, const float* init, const float* dy, const float* dfinal, float* dx,
                               float* ddt, float* dA, float* dB, float* dC, float* dD, float* dinit, const Dims& d,
                               void* workspace, hipStream_t stream);

}  // namespace ssd
