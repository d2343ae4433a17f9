// ssd_api.hip - the C ABI: argument validation, workspace layout and the
// launch sequence of the chunked mode.  Declarations and the contract of
// every entry point are in include/ssd.h.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "ssd.h"
#include "common.hpp"
#include "kernels.hpp"

using ssd::bf16;
using ssd::Dims;

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kMaxChunks = 65535;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int dtype) { return dtype == SSD_BF16 ? 2 : 4; }

bool valid_dtype(int dtype) { return dtype == SSD_F32 || dtype == SSD_BF16; }

int check_common(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups)
{
    if (batch < 0 || batch > 65535) return SSD_ERR_SHAPE;
    if (nheads < 1 || nheads > 65535) return SSD_ERR_SHAPE;
    if (headdim != 16 && headdim != 32 && headdim != 64 && headdim != 128) return SSD_ERR_SHAPE;
    if (dstate < 16 || dstate > 256 || dstate % 16 != 0) return SSD_ERR_SHAPE;
    if (ngroups < 1 || nheads % ngroups != 0) return SSD_ERR_SHAPE;
    if (nheads * headdim > (int64_t(1) << 20)) return SSD_ERR_SHAPE;   // one chunk's rows of y stay <= 2^30 bytes
    if (ngroups * dstate > (int64_t(1) << 20)) return SSD_ERR_SHAPE;   // and its rows of B and C too
    return SSD_OK;
}

int check_seq(const Dims& d)
{
    int rc = check_common(d.batch, d.nheads, d.headdim, d.dstate, d.ngroups);
    if (rc != SSD_OK) return rc;
    if (d.seqlen < 0 || d.chunk < 16 || d.chunk > 256 || d.chunk % 16 != 0) return SSD_ERR_SHAPE;
    if (d.nchunks() > kMaxChunks) return SSD_ERR_SHAPE;
    // every element index of the largest tensor must fit in 32 bits per batch row set
    const int64_t big = d.batch * d.seqlen * d.nheads * (d.headdim > d.dstate ? d.headdim : d.dstate);
    const int64_t st = d.batch * d.nchunks() * d.nheads * d.headdim * d.dstate;
    if (big > (int64_t(1) << 40) || st > (int64_t(1) << 40)) return SSD_ERR_SHAPE;
    if (d.batch * d.nchunks() * d.nheads * 4 > INT32_MAX) return SSD_ERR_SHAPE;
    return SSD_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlaps(Span a, Span b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool any_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins)
{
    for (const Span& o : outs) {
        for (const Span& i : ins)
            if (overlaps(o, i)) return true;
    }
    // outputs must not overlap each other either
    for (auto it = outs.begin(); it != outs.end(); ++it)
        for (auto jt = it + 1; jt != outs.end(); ++jt)
            if (overlaps(*it, *jt)) return true;
    return false;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

struct Workspace {
    size_t cs, dtc, states, entry, total;
};

Workspace layout(const Dims& d, int dtype)
{
    Workspace w;
    const int64_t nc = d.nchunks();
    const int64_t ncs = d.batch * d.nheads * nc * d.chunk * 4;
    const int64_t nst = d.batch * nc * d.nheads * d.headdim * d.dstate;
    w.cs = 0;
    w.dtc = align_up(ncs);
    w.states = w.dtc + align_up(ncs);
    w.entry = w.states + align_up(nst * 4);
    w.total = w.entry + align_up(nst * (int64_t)elem_size(dtype));
    if (w.total < (size_t)kAlign) w.total = kAlign;     // never 0 for valid sizes
    return w;
}

// ssd_forward's body (argument checks and the launch sequence on a caller workspace).
int forward_impl(const void* x, const float* dt, const float* A, const void* B, const void* C,
                 const float* D, const float* init_states, void* y, float* final_states,
                 int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

constexpr size_t kScratchBytes = size_t(64) << 20;

}  // namespace

// The static scratch of ssd_forward_noalloc: device memory of the code object, one copy per GPU the
// library is loaded on, held until the process ends.  In host code its name is a host-side stand-in,
// not a device address: the address on a device comes from hipGetSymbolAddress with that device
// current, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

struct VarlenWorkspace {
    size_t cs, dtc, states, entry, tstart, cmeta, total;
};

VarlenWorkspace layout_varlen(const Dims& d, int dtype)
{
    VarlenWorkspace w;
    const int64_t nc = d.nchunks();
    const int64_t ncs = d.nheads * nc * d.chunk * 4;
    const int64_t nst = nc * d.nheads * d.headdim * d.dstate;
    w.cs = 0;
    w.dtc = align_up(ncs);
    w.states = w.dtc + align_up(ncs);
    w.entry = w.states + align_up(nst * 4);
    w.tstart = w.entry + align_up(nst * (int64_t)elem_size(dtype));
    w.cmeta = w.tstart + align_up(d.seqlen * 4);
    w.total = w.cmeta + align_up(nc * 16);
    if (w.total < (size_t)kAlign) w.total = kAlign;
    return w;
}

}  // namespace

extern "C" {

const char* ssd_status_string(int status)
{
    switch (status) {
    case SSD_OK: return "SSD_OK: enqueued";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE:
        return "SSD_ERR_SHAPE: sizes out of range (headdim in {16,32,64,128}; dstate a multiple of 16 "
               "in [16,256]; ngroups divides nheads; chunk_size a multiple of 16 in [16,256]; "
               "0 <= batch <= 65535; seqlen >= 0; tensors 16-byte aligned)";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: dtype must be SSD_F32 (0) or SSD_BF16 (1)";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace smaller than ssd_forward_workspace_bytes()";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: the HIP runtime reported an error at launch";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output buffer overlaps an input or another output";
    case SSD_ERR_SCRATCH:
        return "SSD_ERR_SCRATCH: one batch row's forward workspace exceeds the library's static scratch "
               "(ssd_forward_noalloc_scratch_bytes(); use ssd_forward with a caller workspace)";
    default: return "unknown ssd status";
    }
}

int ssd_abi_version(void) { return 104; }

int64_t ssd_num_chunks(int64_t seqlen, int64_t chunk_size)
{
    if (seqlen < 0 || chunk_size <= 0) return -1;
    return (seqlen + chunk_size - 1) / chunk_size;
}

size_t ssd_forward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                   int64_t dstate, int64_t chunk_size, int dtype)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, 1, chunk_size};
    if (!valid_dtype(dtype) || check_seq(d) != SSD_OK) return 0;
    return layout(d, dtype).total;
}

int ssd_dA_cumsum(const float* dt, const float* A, float* dA_cs, float* dt_chunked, int64_t batch,
                  int64_t seqlen, int64_t nheads, int64_t chunk_size, void* stream)
{
    Dims d{batch, seqlen, nheads, 16, 16, 1, chunk_size};
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0 || seqlen == 0) return SSD_OK;
    if (!dt || !A || !dA_cs || !dt_chunked) return SSD_ERR_NULL;
    if (!aligned16(dA_cs) || !aligned16(dt_chunked)) return SSD_ERR_SHAPE;
    const size_t nin = (size_t)(batch * seqlen * nheads) * 4, nout = (size_t)(batch * nheads * d.nchunks() * chunk_size) * 4;
    if (any_overlap({{dA_cs, nout}, {dt_chunked, nout}}, {{dt, nin}, {A, (size_t)nheads * 4}}))
        return SSD_ERR_ALIAS;
    return hip_status(ssd::launch_dA_cumsum(dt, A, dA_cs, dt_chunked, d, (hipStream_t)stream));
}

int ssd_chunk_state(const void* x, const void* B, const float* dt_chunked, const float* dA_cs,
                    float* chunk_states, int64_t batch, int64_t seqlen, int64_t nheads,
                    int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype,
                    void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0 || seqlen == 0) return SSD_OK;
    if (!x || !B || !dt_chunked || !dA_cs || !chunk_states) return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(chunk_states)) return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nout = (size_t)(batch * d.nchunks() * nheads * headdim * dstate) * 4;
    const size_t ncs = (size_t)(batch * nheads * d.nchunks() * chunk_size) * 4;
    if (any_overlap({{chunk_states, nout}},
                    {{x, (size_t)(batch * seqlen * nheads * headdim) * es},
                     {B, (size_t)(batch * seqlen * ngroups * dstate) * es}, {dt_chunked, ncs}, {dA_cs, ncs}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_chunk_state<bf16>((const bf16*)x, (const bf16*)B, dt_chunked, dA_cs,
                                                        chunk_states, d, s));
    return hip_status(ssd::launch_chunk_state<float>((const float*)x, (const float*)B, dt_chunked, dA_cs,
                                                     chunk_states, d, s));
}

int ssd_state_passing(const float* chunk_states, const float* dA_cs, const float* init_states,
                      void* entry_states, float* final_states, int64_t batch, int64_t seqlen,
                      int64_t nheads, int64_t headdim, int64_t dstate, int64_t chunk_size, int dtype,
                      void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, 1, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0) return SSD_OK;
    const int64_t nc = d.nchunks();
    if (!final_states || (nc > 0 && (!chunk_states || !dA_cs || !entry_states))) return SSD_ERR_NULL;
    if (!aligned16(final_states) || !aligned16(init_states) || !aligned16(chunk_states) || !aligned16(entry_states))
        return SSD_ERR_SHAPE;
    const size_t nst = (size_t)(batch * nc * nheads * headdim * dstate);
    const size_t nfin = (size_t)(batch * nheads * headdim * dstate) * 4;
    const size_t ncs = (size_t)(batch * nheads * nc * chunk_size) * 4;
    if (any_overlap({{entry_states, nst * elem_size(dtype)}, {final_states, nfin}},
                    {{chunk_states, nst * 4}, {dA_cs, ncs}, {init_states, nfin}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_state_passing<bf16>(chunk_states, dA_cs, init_states, (bf16*)entry_states,
                                                          final_states, d, s));
    return hip_status(ssd::launch_state_passing<float>(chunk_states, dA_cs, init_states, (float*)entry_states,
                                                       final_states, d, s));
}

int ssd_chunk_scan(const void* x, const void* B, const void* C, const float* dt_chunked,
                   const float* dA_cs, const void* entry_states, const float* D, void* y,
                   int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, int64_t chunk_size, int dtype, void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0 || seqlen == 0) return SSD_OK;
    if (!x || !B || !C || !dt_chunked || !dA_cs || !entry_states || !D || !y) return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(entry_states) || !aligned16(y))
        return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(batch * seqlen * nheads * headdim) * es;
    const size_t nb = (size_t)(batch * seqlen * ngroups * dstate) * es;
    const size_t ncs = (size_t)(batch * nheads * d.nchunks() * chunk_size) * 4;
    const size_t nst = (size_t)(batch * d.nchunks() * nheads * headdim * dstate) * es;
    if (any_overlap({{y, nx}}, {{x, nx}, {B, nb}, {C, nb}, {dt_chunked, ncs}, {dA_cs, ncs},
                                {entry_states, nst}, {D, (size_t)nheads * 4}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_chunk_scan<bf16>((const bf16*)x, (const bf16*)B, (const bf16*)C, dt_chunked,
                                                       dA_cs, (const bf16*)entry_states, D, (bf16*)y, d, s));
    return hip_status(ssd::launch_chunk_scan<float>((const float*)x, (const float*)B, (const float*)C, dt_chunked,
                                                    dA_cs, (const float*)entry_states, D, (float*)y, d, s));
}

int ssd_forward(const void* x, const float* dt, const float* A, const void* B, const void* C,
                const float* D, const float* init_states, void* y, float* final_states,
                int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                size_t workspace_bytes, void* stream)
{
    return forward_impl(x, dt, A, B, C, D, init_states, y, final_states, batch, seqlen, nheads, headdim, dstate,
                        ngroups, chunk_size, dtype, workspace, workspace_bytes, stream);
}

size_t ssd_forward_noalloc_scratch_bytes(void) { return kScratchBytes; }

int ssd_forward_noalloc(const void* x, const float* dt, const float* A, const void* B, const void* C,
                        const float* D, const float* init_states, void* y, float* final_states, int64_t batch,
                        int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                        int64_t chunk_size, int dtype, void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0) return SSD_OK;
    // batch rows are independent: run the forward on slices of rows whose workspace fits the scratch
    Dims one = d;
    one.batch = 1;
    const size_t per_row = layout(one, dtype).total;
    if (per_row > kScratchBytes) return SSD_ERR_SCRATCH;
    int64_t nb = std::min<int64_t>(batch, (int64_t)(kScratchBytes / per_row));
    for (;;) {
        Dims sl = d;
        sl.batch = nb;
        if (layout(sl, dtype).total <= kScratchBytes || nb == 1) break;
        --nb;
    }
    void* ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc != SSD_OK) return rc;
    const size_t es = elem_size(dtype);
    const int64_t row_x = seqlen * nheads * headdim, row_dt = seqlen * nheads, row_b = seqlen * ngroups * dstate;
    const int64_t row_s = nheads * headdim * dstate;
    for (int64_t b0 = 0; b0 < batch; b0 += nb) {
        const int64_t n = std::min(nb, batch - b0);
        auto off = [&](const void* p, int64_t elems) -> const void* {
            return p ? static_cast<const unsigned char*>(p) + b0 * elems : nullptr;
        };
        rc = forward_impl(off(x, row_x * es), (const float*)off(dt, row_dt * 4), A, off(B, row_b * es),
                          off(C, row_b * es), D, (const float*)off(init_states, row_s * 4),
                          const_cast<void*>(off(y, row_x * es)), (float*)off(final_states, row_s * 4), n, seqlen,
                          nheads, headdim, dstate, ngroups, chunk_size, dtype, ws, kScratchBytes, stream);
        if (rc != SSD_OK) return rc;
    }
    return SSD_OK;
}
}  // extern "C"

namespace {

int forward_impl(const void* x, const float* dt, const float* A, const void* B, const void* C,
                 const float* D, const float* init_states, void* y, float* final_states,
                 int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (batch == 0) return SSD_OK;
    if (!final_states) return SSD_ERR_NULL;
    if (seqlen > 0 && (!x || !dt || !A || !B || !C || !D || !y)) return SSD_ERR_NULL;
    const Workspace w = layout(d, dtype);
    if (workspace_bytes < w.total) return SSD_ERR_WORKSPACE;
    if (seqlen > 0 && !workspace) return SSD_ERR_NULL;
    if (!aligned16(workspace) || !aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
        !aligned16(init_states) || !aligned16(final_states))
        return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(batch * seqlen * nheads * headdim) * es;
    const size_t nb = (size_t)(batch * seqlen * ngroups * dstate) * es;
    const size_t nfin = (size_t)(batch * nheads * headdim * dstate) * 4;
    const size_t ndt = (size_t)(batch * seqlen * nheads) * 4;
    if (any_overlap({{y, nx}, {final_states, nfin}, {workspace, w.total}},
                    {{x, nx}, {dt, ndt}, {A, (size_t)nheads * 4}, {B, nb}, {C, nb}, {D, (size_t)nheads * 4},
                     {init_states, nfin}}))
        return SSD_ERR_ALIAS;

    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* cs = reinterpret_cast<float*>(ws + w.cs);
    float* dtc = reinterpret_cast<float*>(ws + w.dtc);
    float* states = reinterpret_cast<float*>(ws + w.states);
    void* entry = ws + w.entry;
    if (seqlen == 0) {
        // no tokens: the final state is the initial state (or zeros)
        if (dtype == SSD_BF16)
            return hip_status(ssd::launch_state_passing<bf16>(nullptr, nullptr, init_states, nullptr, final_states, d, s));
        return hip_status(ssd::launch_state_passing<float>(nullptr, nullptr, init_states, nullptr, final_states, d, s));
    }
    // stage 1 runs inside the stage-2 kernel (each workgroup scans dt A for its heads and chunk)
    hipError_t e;
    if (dtype == SSD_BF16) {
        e = ssd::launch_chunk_state_cumsum<bf16>((const bf16*)x, (const bf16*)B, dt, A, dtc, cs, states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_state_passing<bf16>(states, cs, init_states, (bf16*)entry, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_chunk_scan<bf16>((const bf16*)x, (const bf16*)B, (const bf16*)C, dtc, cs,
                                             (const bf16*)entry, D, (bf16*)y, d, s);
    } else {
        e = ssd::launch_chunk_state_cumsum<float>((const float*)x, (const float*)B, dt, A, dtc, cs, states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_state_passing<float>(states, cs, init_states, (float*)entry, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_chunk_scan<float>((const float*)x, (const float*)B, (const float*)C, dtc, cs,
                                              (const float*)entry, D, (float*)y, d, s);
    }
    return hip_status(e);
}

}  // namespace

extern "C" {

int ssd_forward_fused(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                      const float* init_states, void* y, float* final_states, int64_t batch, int64_t seqlen,
                      int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int dtype, void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, 256};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (!ssd::fused_supported(d)) return SSD_ERR_SHAPE;
    if (batch == 0) return SSD_OK;
    if (!final_states) return SSD_ERR_NULL;
    if (seqlen > 0 && (!x || !dt || !A || !B || !C || !D || !y)) return SSD_ERR_NULL;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) || !aligned16(init_states) ||
        !aligned16(final_states))
        return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(batch * seqlen * nheads * headdim) * es;
    const size_t nb = (size_t)(batch * seqlen * ngroups * dstate) * es;
    const size_t nfin = (size_t)(batch * nheads * headdim * dstate) * 4;
    const size_t ndt = (size_t)(batch * seqlen * nheads) * 4;
    if (any_overlap({{y, nx}, {final_states, nfin}},
                    {{x, nx}, {dt, ndt}, {A, (size_t)nheads * 4}, {B, nb}, {C, nb}, {D, (size_t)nheads * 4},
                     {init_states, nfin}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_ssd_fused<bf16>((const bf16*)x, dt, A, (const bf16*)B, (const bf16*)C, D,
                                                      init_states, (bf16*)y, final_states, d, s));
    return hip_status(ssd::launch_ssd_fused<float>((const float*)x, dt, A, (const float*)B, (const float*)C, D,
                                                   init_states, (float*)y, final_states, d, s));
}

size_t ssd_forward_varlen_workspace_bytes(int64_t total_tokens, int64_t nheads, int64_t headdim, int64_t dstate,
                                          int64_t chunk_size, int dtype)
{
    if (!valid_dtype(dtype)) return 0;
    Dims d{1, total_tokens, nheads, headdim, dstate, 1, chunk_size};
    if (check_seq(d) != SSD_OK) return 0;
    return layout_varlen(d, dtype).total;
}

int ssd_forward_varlen(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                       const int32_t* cu_seqlens, int64_t nseq, void* y, float* final_states, int64_t total_tokens,
                       int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    Dims d{1, total_tokens, nheads, headdim, dstate, ngroups, chunk_size};
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    if (nseq < 0 || nseq > (int64_t(1) << 24) || (nseq == 0 && total_tokens > 0)) return SSD_ERR_SHAPE;
    if (nseq == 0) return SSD_OK;
    if (!cu_seqlens || !A || !final_states) return SSD_ERR_NULL;
    if (total_tokens > 0 && (!x || !dt || !B || !C || !D || !y)) return SSD_ERR_NULL;
    const VarlenWorkspace w = layout_varlen(d, dtype);
    if (workspace_bytes < w.total) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL;
    if (!aligned16(workspace) || !aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) ||
        !aligned16(final_states))
        return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(total_tokens * nheads * headdim) * es;
    const size_t nb = (size_t)(total_tokens * ngroups * dstate) * es;
    const size_t nfin = (size_t)(nseq * nheads * headdim * dstate) * 4;
    const size_t ndt = (size_t)(total_tokens * nheads) * 4;
    if (any_overlap({{y, nx}, {final_states, nfin}, {workspace, w.total}},
                    {{x, nx}, {dt, ndt}, {A, (size_t)nheads * 4}, {B, nb}, {C, nb}, {D, (size_t)nheads * 4},
                     {cu_seqlens, (size_t)(nseq + 1) * 4}}))
        return SSD_ERR_ALIAS;

    hipStream_t s = (hipStream_t)stream;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* cs = reinterpret_cast<float*>(ws + w.cs);
    float* dtc = reinterpret_cast<float*>(ws + w.dtc);
    float* states = reinterpret_cast<float*>(ws + w.states);
    void* entry = ws + w.entry;
    int* tstart = reinterpret_cast<int*>(ws + w.tstart);
    int* cmeta = reinterpret_cast<int*>(ws + w.cmeta);
    hipError_t e = ssd::launch_varlen_meta(cu_seqlens, nseq, total_tokens, chunk_size, tstart, cmeta, s);
    if (dtype == SSD_BF16) {
        if (e == hipSuccess)
            e = ssd::launch_chunk_state_varlen<bf16>((const bf16*)x, (const bf16*)B, dt, A, cu_seqlens, nseq, tstart,
                                                     dtc, cs, states, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_state_passing_varlen<bf16>(states, cs, cmeta, (bf16*)entry, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_chunk_scan_varlen<bf16>((const bf16*)x, (const bf16*)B, (const bf16*)C, dtc, cs,
                                                    (const bf16*)entry, D, tstart, (bf16*)y, d, s);
    } else {
        if (e == hipSuccess)
            e = ssd::launch_chunk_state_varlen<float>((const float*)x, (const float*)B, dt, A, cu_seqlens, nseq,
                                                      tstart, dtc, cs, states, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_state_passing_varlen<float>(states, cs, cmeta, (float*)entry, final_states, d, s);
        if (e == hipSuccess)
            e = ssd::launch_chunk_scan_varlen<float>((const float*)x, (const float*)B, (const float*)C, dtc, cs,
                                                     (const float*)entry, D, tstart, (float*)y, d, s);
    }
    return hip_status(e);
}

namespace {
int check_backward(const Dims& d, int dtype)
{
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_seq(d);
    if (rc != SSD_OK) return rc;
    // the per-head dB / dC passes put dstate in the head dimension's place
    if (d.dstate != 16 && d.dstate != 32 && d.dstate != 64 && d.dstate != 128 && d.dstate != 256) return SSD_ERR_SHAPE;
    if (d.nheads * d.dstate > (int64_t(1) << 20)) return SSD_ERR_SHAPE;
    return SSD_OK;
}
}  // namespace

size_t ssd_backward_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                                    int64_t ngroups, int64_t chunk_size, int dtype)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    if (check_backward(d, dtype) != SSD_OK) return 0;
    return ssd::bwd_workspace_bytes(d, dtype == SSD_BF16);
}

int ssd_backward(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                 const float* init_states, const void* dy, const float* dfinal, void* dx, float* ddt, float* dA,
                 void* dB, void* dC, float* dD, float* dinit, int64_t batch, int64_t seqlen, int64_t nheads,
                 int64_t headdim, int64_t dstate, int64_t ngroups, int64_t chunk_size, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream)
{
    Dims d{batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size};
    int rc = check_backward(d, dtype);
    if (rc != SSD_OK) return rc;
    if (!A || !D || !dA || !dD || !dinit) return SSD_ERR_NULL;
    if (batch == 0) return SSD_OK;
    if (seqlen > 0 && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return SSD_ERR_NULL;
    const size_t need = ssd::bwd_workspace_bytes(d, dtype == SSD_BF16);
    if (workspace_bytes < need) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL;
    if (!aligned16(workspace) || !aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(dy) ||
        !aligned16(dx) || !aligned16(dB) || !aligned16(dC) || !aligned16(init_states) || !aligned16(dfinal) ||
        !aligned16(dinit))
        return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(batch * seqlen * nheads * headdim) * es;
    const size_t nb = (size_t)(batch * seqlen * ngroups * dstate) * es;
    const size_t nst = (size_t)(batch * nheads * headdim * dstate) * 4;
    const size_t ndt = (size_t)(batch * seqlen * nheads) * 4;
    const size_t nh = (size_t)nheads * 4;
    if (any_overlap({{dx, nx}, {ddt, ndt}, {dA, nh}, {dB, nb}, {dC, nb}, {dD, nh}, {dinit, nst}, {workspace, need}},
                    {{x, nx}, {dt, ndt}, {A, nh}, {B, nb}, {C, nb}, {D, nh}, {init_states, init_states ? nst : 0},
                     {dy, nx}, {dfinal, dfinal ? nst : 0}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_backward_bf16((const bf16*)x, dt, A, (const bf16*)B, (const bf16*)C, D,
                                                    init_states, (const bf16*)dy, dfinal, (bf16*)dx, ddt, dA,
                                                    (bf16*)dB, (bf16*)dC, dD, dinit, d, workspace, s));
    return hip_status(ssd::launch_backward_f32((const float*)x, dt, A, (const float*)B, (const float*)C, D,
                                               init_states, (const float*)dy, dfinal, (float*)dx, ddt, dA,
                                               (float*)dB, (float*)dC, dD, dinit, d, workspace, s));
}

int ssd_step(float* state, const void* x, const float* dt, const float* A, const void* B,
             const void* C, const float* D, void* y, int64_t batch, int64_t nheads,
             int64_t headdim, int64_t dstate, int64_t ngroups, int dtype, void* stream)
{
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    int rc = check_common(batch, nheads, headdim, dstate, ngroups);
    if (rc != SSD_OK) return rc;
    if (batch * nheads > INT32_MAX) return SSD_ERR_SHAPE;
    if (batch == 0) return SSD_OK;
    if (!state || !x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_NULL;
    if (!aligned16(state)) return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nst = (size_t)(batch * nheads * headdim * dstate) * 4;
    const size_t nx = (size_t)(batch * nheads * headdim) * es;
    const size_t nb = (size_t)(batch * ngroups * dstate) * es;
    if (any_overlap({{y, nx}, {state, nst}},
                    {{x, nx}, {dt, (size_t)(batch * nheads) * 4}, {A, (size_t)nheads * 4}, {B, nb}, {C, nb},
                     {D, (size_t)nheads * 4}}))
        return SSD_ERR_ALIAS;
    Dims d{batch, 1, nheads, headdim, dstate, ngroups, 16};
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_ssd_step<bf16>(state, (const bf16*)x, dt, A, (const bf16*)B, (const bf16*)C,
                                                     D, (bf16*)y, d, s));
    return hip_status(ssd::launch_ssd_step<float>(state, (const float*)x, dt, A, (const float*)B, (const float*)C,
                                                  D, (float*)y, d, s));
}

int ssd_selective_scan(const void* x, const float* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* init_states, void* y, float* final_states, int64_t batch,
                       int64_t seqlen, int64_t dim, int64_t dstate, int dtype, void* stream)
{
    if (!valid_dtype(dtype)) return SSD_ERR_DTYPE;
    if (batch < 0 || batch > 65535 || seqlen < 0 || seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    if (dim < 8 || dim % 8 != 0 || dim > (int64_t(1) << 20)) return SSD_ERR_SHAPE;
    if (dstate != 4 && dstate != 8 && dstate != 16 && dstate != 32 && dstate != 64) return SSD_ERR_SHAPE;
    if (batch * ((dim + 31) / 32) > INT32_MAX) return SSD_ERR_SHAPE;
    if (batch == 0) return SSD_OK;
    if (!A || !D || !final_states) return SSD_ERR_NULL;
    if (seqlen > 0 && (!x || !delta || !B || !C || !y)) return SSD_ERR_NULL;   // empty tensors may be NULL
    if (!aligned16(x) || !aligned16(delta) || !aligned16(y)) return SSD_ERR_SHAPE;
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)(batch * seqlen * dim) * es;
    const size_t nd = (size_t)(batch * seqlen * dim) * 4;
    const size_t nb = (size_t)(batch * seqlen * dstate) * es;
    const size_t nst = (size_t)(batch * dim * dstate) * 4;
    if (any_overlap({{y, nx}, {final_states, nst}},
                    {{x, nx}, {delta, nd}, {A, (size_t)(dim * dstate) * 4}, {B, nb}, {C, nb},
                     {D, (size_t)dim * 4}, {init_states, init_states ? nst : 0}}))
        return SSD_ERR_ALIAS;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == SSD_BF16)
        return hip_status(ssd::launch_selective_scan<bf16>((const bf16*)x, delta, A, (const bf16*)B, (const bf16*)C,
                                                           D, init_states, (bf16*)y, final_states, batch, seqlen,
                                                           dim, dstate, s));
    return hip_status(ssd::launch_selective_scan<float>((const float*)x, delta, A, (const float*)B, (const float*)C,
                                                        D, init_states, (float*)y, final_states, batch, seqlen, dim,
                                                        dstate, s));
}

}  // extern "C"
