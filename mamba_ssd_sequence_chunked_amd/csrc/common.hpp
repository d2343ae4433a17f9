// common.hpp - device helpers shared by the SSD kernels (gfx950 / CDNA4).
//
// * element types: T is float or __bf16; bf16 <-> fp32 conversion uses the
//   hardware round-to-nearest-even convert (v_cvt_pk_bf16_f32) and a shift.
// * matrix-core fragments: every product runs on 16x16 output tiles with a
//   contraction block of 32.  A lane holds 8 contraction slots of its row
//   (A operand) or column (B operand):  lane = 16 * g + r, slots (g, 0..7).
//   For bf16 this is one v_mfma_f32_16x16x32_bf16; for fp32 it is eight
//   v_mfma_f32_16x16x4_f32, the i-th taking slot (g, i) of every lane.  Both
//   contract the same 32 (g, i) slots, so which index a slot stands for is
//   the caller's choice as long as A and B agree.  The accumulator layout
//   (both types) is: lane 16 * g + c holds rows 4g .. 4g+3 of column c.
// * contraction slots along the rows of a row-major LDS tile: for bf16 two
//   gfx950 transpose reads (ds_read_b64_tr_b16) deliver them directly in
//   operand order; for fp32, eight scalar LDS reads.
// * a wavefront inclusive prefix sum built from DPP row shifts and row
//   broadcasts (64 lanes, no LDS).
// * an XCD-aware block index: the dispatcher hands consecutive workgroups
//   to the 8 XCDs in turn, so related tiles are renumbered to share an XCD
//   (and its L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// 8 consecutive elements of T, as one operand fragment.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ float get(int i) const { return static_cast<float>(v[i]); }
    __device__ __forceinline__ void set(int i, float f) { v[i] = static_cast<bf16>(f); }
    __device__ __forceinline__ void zero() {
        *reinterpret_cast<uint4*>(&v) = make_uint4(0u, 0u, 0u, 0u);
    }
};
template <> struct Vec8<float> {
    float v[8];
    __device__ __forceinline__ float get(int i) const { return v[i]; }
    __device__ __forceinline__ void set(int i, float f) { v[i] = f; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
};

// Load / store 8 consecutive elements (16 B for bf16, 32 B for fp32); the
// address must be aligned to the vector size.
__device__ __forceinline__ void load8(Vec8<bf16>& d, const bf16* p) {
    d.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load8(Vec8<float>& d, const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    d.v[0] = a.x; d.v[1] = a.y; d.v[2] = a.z; d.v[3] = a.w;
    d.v[4] = b.x; d.v[5] = b.y; d.v[6] = b.z; d.v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const Vec8<bf16>& d) {
    *reinterpret_cast<bf16x8*>(p) = d.v;
}
__device__ __forceinline__ void store8(float* p, const Vec8<float>& d) {
    reinterpret_cast<float4*>(p)[0] = make_float4(d.v[0], d.v[1], d.v[2], d.v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(d.v[4], d.v[5], d.v[6], d.v[7]);
}

// 4 consecutive elements (8 B bf16 / 16 B fp32), used for half fragments.
__device__ __forceinline__ void load4(Vec8<bf16>& d, int half, const bf16* p) {
    const bf16x4 q = *reinterpret_cast<const bf16x4*>(p);
    d.v[4 * half + 0] = q[0]; d.v[4 * half + 1] = q[1];
    d.v[4 * half + 2] = q[2]; d.v[4 * half + 3] = q[3];
}
__device__ __forceinline__ void load4(Vec8<float>& d, int half, const float* p) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    d.v[4 * half + 0] = q.x; d.v[4 * half + 1] = q.y;
    d.v[4 * half + 2] = q.z; d.v[4 * half + 3] = q.w;
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    bf16x4 q;
    q[0] = static_cast<bf16>(a); q[1] = static_cast<bf16>(b);
    q[2] = static_cast<bf16>(c); q[3] = static_cast<bf16>(d);
    *reinterpret_cast<bf16x4*>(p) = q;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
// 4 consecutive elements as fp32 (8 B bf16 / 16 B fp32, aligned to that size)
__device__ __forceinline__ float4 load4f(const bf16* p) {
    const bf16x4 q = *reinterpret_cast<const bf16x4*>(p);
    return make_float4(static_cast<float>(q[0]), static_cast<float>(q[1]), static_cast<float>(q[2]),
                       static_cast<float>(q[3]));
}
__device__ __forceinline__ float4 load4f(const float* p) { return *reinterpret_cast<const float4*>(p); }

// acc (16x16 fp32 tile) += A (16 x 32) * B (32 x 16).
__device__ __forceinline__ void mma(f32x4& acc, const Vec8<bf16>& a, const Vec8<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Vec8<float>& a, const Vec8<float>& b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// An fp32 value as a pair of bf16 values: hi = bf16(v), lo = bf16(v - hi) (v - hi is exact in fp32),
// so |v - hi - lo| <= 2^-9 |v - hi| <= 2^-18 |v| (normal range).  A product with a bf16-valued
// operand then takes two bf16 matrix-core products, hi and lo, instead of the fp32 ones.
__device__ __forceinline__ void split_set(Vec8<bf16>& hi, Vec8<bf16>& lo, int i, float v) {
    const bf16 h = static_cast<bf16>(v);
    hi.v[i] = h;
    lo.v[i] = static_cast<bf16>(v - static_cast<float>(h));
}

// 8 fp32 values as one operand fragment; bf16 converts them in pairs (v_cvt_pk_bf16_f32, round to
// nearest even), so selects made on the fp32 values stay in front of the conversion.
__device__ __forceinline__ void pack8(Vec8<bf16>& f, const float (&v)[8]) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
    const bf16x2 b = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
    const bf16x2 c = __builtin_convertvector((f32x2{v[4], v[5]}), bf16x2);
    const bf16x2 d = __builtin_convertvector((f32x2{v[6], v[7]}), bf16x2);
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    f.v = __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}
// A 16x16 accumulator fragment's 4 values as bf16 (round to nearest even), in two 4-byte words.
__device__ __forceinline__ uint2 pack4_bf16(const f32x4& v) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
    const bf16x2 b = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
    return make_uint2(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b));
}
__device__ __forceinline__ void pack8(Vec8<float>& f, const float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = v[i];
}
// The pair form of split_set for 8 values: hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void pack8_split(Vec8<bf16>& hi, Vec8<bf16>& lo, const float (&v)[8]) {
    pack8(hi, v);
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = v[i] - static_cast<float>(hi.v[i]);
    pack8(lo, r);
}

// LDS pointer for a generic pointer known to point into LDS: the low 32 bits
// of such a flat address are the LDS address (taken as an integer, so no
// null-pointer check of a generic -> local cast is generated).
template <typename V>
__device__ __forceinline__ __attribute__((address_space(3))) V* as_lds(const void* p) {
    return (__attribute__((address_space(3))) V*)(uintptr_t)(unsigned)(uintptr_t)p;
}

// Operand fragment whose 8 contraction slots run down the ROWS of a row-major
// LDS tile: lane 16 * g + r receives column c0 + r of rows k0 + 4g + m (slots
// 0..3) and k0 + 16 + 4g + m (slots 4..7), m = 0..3.  The bf16 form uses the
// gfx950 transpose read: in every 16-lane group, lane i receives element i % 4
// of the 8-byte chunks read by lanes i / 4 + 4 m, so lane j of the group reads
// row k0 + 4g + j / 4 at columns c0 + 4 (j % 4) .. + 3.  Rows k0 .. k0 + 31 and
// columns c0 .. c0 + 15 must lie inside the tile; the row pitch must keep
// 8-byte alignment.
__device__ __forceinline__ void load_row_slots(Vec8<bf16>& f, const bf16* tile, int pitch, int k0, int c0) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const bf16* p0 = tile + (k0 + 4 * g + (r >> 2)) * pitch + c0 + 4 * (r & 3);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<v4i16>(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<v4i16>(p0 + 16 * pitch));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    f.v = __builtin_bit_cast(bf16x8, ab);
}
__device__ __forceinline__ void load_row_slots(Vec8<float>& f, const float* tile, int pitch, int k0, int c0) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const float* p0 = tile + (k0 + 4 * g) * pitch + c0 + r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f.v[m] = p0[m * pitch];
        f.v[4 + m] = p0[(16 + m) * pitch];
    }
}

// Row pitch (elements) for a tile read with load_row_slots: the 16-byte row
// segments of 8 consecutive rows then fall in distinct LDS banks.
template <typename T>
constexpr int tr_pitch(int width) {
    return sizeof(T) == 2 ? ((width / 16) % 2 == 0 ? width + 16 : width) : width + 4;
}

// Select without a branch (the masked value is computed but discarded).
__device__ __forceinline__ float select(bool c, float a, float b) { return c ? a : b; }

// v if ok, else zeros, without a branch (so a load into v never has to be
// waited for on a path that overwrites the same registers).
__device__ __forceinline__ Vec8<bf16> masked(const Vec8<bf16>& v, bool ok) {
    Vec8<bf16> r;
    const uint4 u = __builtin_bit_cast(uint4, v.v);
    const uint4 z = make_uint4(ok ? u.x : 0u, ok ? u.y : 0u, ok ? u.z : 0u, ok ? u.w : 0u);
    r.v = __builtin_bit_cast(bf16x8, z);
    return r;
}
__device__ __forceinline__ Vec8<float> masked(const Vec8<float>& v, bool ok) {
    Vec8<float> r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = ok ? v.v[i] : 0.f;
    return r;
}

// ---------------------------------------------------------------------------------------------
// Swizzled LDS tiles filled by asynchronous global->LDS loads.
//
// A tile is R rows of CH 16-byte chunks (CH a power of two).  Logical chunk c
// of row r lives at slot c ^ (r & M), M = min(CH, 16) - 1, so 16 rows read at
// one column, or 8 rows read 8 bytes apiece through the transpose read, fall
// in distinct banks.  The tile is filled with gfx950 global_load_lds_dwordx4:
// one wavefront instruction writes 64 consecutive chunks (lane i -> chunk
// slot i of that 1 KB), so each lane loads the global chunk that belongs in
// its slot.  R * CH must be a multiple of 64.
//
// RS > 0 takes the XOR key from row / 2^RS instead: for tiles read as 16 rows x one 16-byte chunk
// per 16-lane group whose rows are shorter than the 256 bytes of one pass over the banks
// (CH = 16 / 2^RS), so that the rows sharing a pass get different slots.  KM = 2 doubles the key:
// for 256-byte rows read with the transpose read (8 rows x two adjacent chunks per pass), so that
// rows r and r ^ 1 do not land on the same pair of slots.
template <int CH, int RS = 0, int KM = 1>
struct SwzTile {
    static constexpr int kMask = (CH < 16 ? CH : 16) - 1;
    static constexpr int kRowBytes = CH * 16;
    __device__ __forceinline__ static int key(int r) { return ((r >> RS) * KM) & kMask; }
    __device__ __forceinline__ static int offset(int r, int c) { return r * kRowBytes + ((c ^ key(r)) << 4); }
};

// Row shift of SwzTile for CH-chunk rows read 16 rows at a time (see above).
constexpr int swz_row_shift(int ch) { return ch >= 16 ? 0 : ch == 8 ? 1 : ch == 4 ? 2 : ch == 2 ? 3 : 4; }

// LDS address (an integer) of a __shared__ object, taken from its local
// address-space form so that no generic pointer is materialised.
#define lds_addr(obj) ((unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)(obj))

// One 16-byte global->LDS load per lane: lane i's data goes to LDS address
// lds_base + 16 i (lds_base wave-uniform; see lds_addr).  Issued through inline asm so that the
// compiler's wait-count bookkeeping does not treat every later LDS read as
// possibly aliasing the in-flight copy (it cannot tell the two stage buffers
// apart and would wait for the prefetch before any LDS read); the kernels
// order these copies explicitly with wait_vmem() and a barrier.  M0 carries
// the LDS address and is restored right after the issue.
__device__ __forceinline__ void dma16(const void* gsrc, unsigned lds_base) {
    const unsigned a = __builtin_amdgcn_readfirstlane(lds_base);
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(gsrc), "s"(a)
                 : "memory");
}

// Issue the loads of one tile: src(r, c) returns the global address of logical
// chunk c of row r (it must always be a valid address).  Returns nothing; the
// data is in LDS once this wave's vmcnt reaches zero and a barrier has passed.
template <int CH, int R, int NW = 4, int RS = 0, int KM = 1, class F>
__device__ __forceinline__ void tile_load_async(unsigned tile, F src) {
    using TL = SwzTile<CH, RS, KM>;
    constexpr int kInst = R * CH / 64;                 // wavefront instructions for the tile
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int q = wave; q < kInst; q += NW) {
        const int pos = q * 64 + lane;
        const int r = pos / CH, slot = pos % CH;
        const int c = slot ^ TL::key(r);
        dma16(src(r, c), tile + q * 1024u);
    }
}

// The same for NT tiles of one shape laid out every `stride` bytes: their
// copies are dealt round-robin over the NW wavefronts as one sequence, so
// every wavefront issues (NT * R * CH / 64) / NW of them when that divides.
// src(t, r, c) returns the global address of logical chunk c of row r of tile t.
template <int CH, int R, int NT, int NW, int RS = 0, int KM = 1, class F>
__device__ __forceinline__ void tiles_load_async(unsigned base, int stride, F src) {
    using TL = SwzTile<CH, RS, KM>;
    constexpr int kPer = R * CH / 64;                  // wavefront instructions per tile
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int q = wave; q < NT * kPer; q += NW) {
        const int t = q / kPer, qq = q % kPer;
        const int pos = qq * 64 + lane;
        const int r = pos / CH, slot = pos % CH;
        const int c = slot ^ TL::key(r);
        dma16(src(t, r, c), base + t * stride + qq * 1024u);
    }
}

// The same 16-byte global->LDS load with a wave-uniform base address and a per-lane 32-bit byte
// offset (the instruction's scalar-base form): lane i's data, at sbase + voff, goes to LDS address
// lds_base + 16 i.
__device__ __forceinline__ void dma16_off(const void* sbase, unsigned voff, unsigned lds_base) {
    const unsigned a = __builtin_amdgcn_readfirstlane(lds_base);
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(sbase), "s"(a)
                 : "memory");
}

// One wavefront's share of the copies of NT swizzled tiles of R rows x CH chunks (the copies of
// all tiles dealt round robin over NW wavefronts as one sequence, as tiles_load_async deals them),
// with the per-lane source offsets worked out once: plan() stores them, issue() sends the copies
// from a base that may change between calls (the next block of rows) at the cost of a scalar add.
// Copy k of the wavefront is q = wave + NW k: tile q / kPer, 1 KB piece q % kPer of the tile.
template <int CH, int R, int NT, int NW, int RS = 0, int KM = 1>
struct TileCopies {
    using TL = SwzTile<CH, RS, KM>;
    static constexpr int kPer = R * CH / 64;          // wavefront instructions per tile
    static constexpr int kTotal = NT * kPer;
    static constexpr int kK = (kTotal + NW - 1) / NW; // copies per wavefront (at most)
    unsigned off[kK];

    // off_of(t, r, c): byte offset, from the base of tile t, of logical chunk c of row r
    template <class F>
    __device__ __forceinline__ void plan(int wave, F off_of) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < kK; ++k) {
            const int q = wave + NW * k;
            const int t = min(q, kTotal - 1) / kPer, qq = q % kPer;
            const int pos = qq * 64 + lane;
            const int r = pos / CH, c = (pos % CH) ^ TL::key(r);
            off[k] = off_of(t, r, c);
        }
    }
    // base_of(t): base address of tile t; lds: LDS address of tile 0, the tiles stride bytes apart.
    // When rows are row_bytes apart in the source and offsets below row_bytes pick the column, rows
    // past rmax (0 <= rmax < R - 1) read row rmax instead.  (The row is recovered from the offset by a
    // division, on that path only, so no register holds it through the caller's loop.)
    template <class F>
    __device__ __forceinline__ void issue(int wave, F base_of, unsigned lds, int stride, int rmax = R,
                                          unsigned row_bytes = 0) const {
#pragma unroll
        for (int k = 0; k < kK; ++k) {
            const int q = wave + NW * k;
            if (kTotal % NW != 0 && q >= kTotal) break;
            const int t = q / kPer, qq = q % kPer;
            unsigned o = off[k];
            if (rmax < R - 1) {
                const unsigned r = o / row_bytes;
                if (r > (unsigned)rmax) o -= (r - (unsigned)rmax) * row_bytes;
            }
            dma16_off(base_of(t), o, lds + t * stride + qq * 1024u);
        }
    }
};

// Wait for all of this wavefront's outstanding vector-memory operations.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wavefront's vector-memory operations are outstanding
// (they complete in issue order for this counter), N < 64.
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Fragment of 8 consecutive elements along a row of a swizzled tile (columns
// c0 .. c0+7, c0 a multiple of 8 for bf16 / 4 for fp32).
template <int CH, int RS = 0>
__device__ __forceinline__ void swz_load8(Vec8<bf16>& f, const unsigned char* tile, int r, int c0) {
    f.v = *reinterpret_cast<const bf16x8*>(tile + SwzTile<CH, RS>::offset(r, c0 >> 3));
}
template <int CH, int RS = 0>
__device__ __forceinline__ void swz_load8(Vec8<float>& f, const unsigned char* tile, int r, int c0) {
    const float4 a = *reinterpret_cast<const float4*>(tile + SwzTile<CH, RS>::offset(r, c0 >> 2));
    const float4 b = *reinterpret_cast<const float4*>(tile + SwzTile<CH, RS>::offset(r, (c0 >> 2) + 1));
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// 4 consecutive elements along a row (c0 a multiple of 4), as floats.
template <int CH>
__device__ __forceinline__ float4 swz_load4f(const bf16* tile_, int r, int c0) {
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(tile_);
    const bf16x4 q = *reinterpret_cast<const bf16x4*>(tile + SwzTile<CH>::offset(r, c0 >> 3) + 2 * (c0 & 7));
    return make_float4((float)q[0], (float)q[1], (float)q[2], (float)q[3]);
}
template <int CH>
__device__ __forceinline__ float4 swz_load4f(const float* tile_, int r, int c0) {
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(tile_);
    return *reinterpret_cast<const float4*>(tile + SwzTile<CH>::offset(r, c0 >> 2));
}

// Fragment whose 8 contraction slots run down the rows of a swizzled tile
// (the slot layout of load_row_slots): lane 16 g + r gets column c0 + r of
// rows k0 + 4g + m and k0 + 16 + 4g + m, m = 0..3.
template <int CH, int KM = 1>
__device__ __forceinline__ void swz_row_slots(Vec8<bf16>& f, const unsigned char* tile, int k0, int c0) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int row = k0 + 4 * g + (r >> 2);
    const int col = c0 + 4 * (r & 3);                          // 4 elements = 8 bytes, inside one chunk
    const unsigned char* p0 = tile + SwzTile<CH, 0, KM>::offset(row, col >> 3) + 2 * (col & 7);
    const unsigned char* p1 = tile + SwzTile<CH, 0, KM>::offset(row + 16, col >> 3) + 2 * (col & 7);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<v4i16>(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(as_lds<v4i16>(p1));
    const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    f.v = __builtin_bit_cast(bf16x8, ab);
}
template <int CH, int KM = 1>
__device__ __forceinline__ void swz_row_slots(Vec8<float>& f, const unsigned char* tile, int k0, int c0) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int col = c0 + r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r0 = k0 + 4 * g + m, r1 = r0 + 16;
        f.v[m] = *reinterpret_cast<const float*>(tile + SwzTile<CH, 0, KM>::offset(r0, col >> 2) + 4 * (col & 3));
        f.v[4 + m] = *reinterpret_cast<const float*>(tile + SwzTile<CH, 0, KM>::offset(r1, col >> 2) + 4 * (col & 3));
    }
}

// Buffer-resource accesses: one instruction whatever the offset; a store
// whose offset (voff + soff) reaches the resource's size is dropped by the
// hardware and such a load reads zeros, which masks rows (voff) and heads
// (soff) without branching.  kDropped marks a dropped access: resources here
// stay below 2^30 bytes, and two kDropped offsets still sum below 2^32.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;     // raw buffer, 32-bit data format, range-checked
constexpr int kDropped = 0x40000000;

// Load 8 consecutive elements (the fp32 form reads two 16-byte halves, at voff and voff + 16).
__device__ __forceinline__ void buffer_load8(Vec8<bf16>& f, __amdgpu_buffer_rsrc_t r, int voff) {
    f.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// Load 4 consecutive bf16 elements into half h (elements 4 h .. 4 h + 3) of a fragment.
__device__ __forceinline__ void buffer_load4(Vec8<bf16>& f, int h, __amdgpu_buffer_rsrc_t r, int voff) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    const bf16x4_t q = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
    f.v[4 * h + 0] = q[0]; f.v[4 * h + 1] = q[1]; f.v[4 * h + 2] = q[2]; f.v[4 * h + 3] = q[3];
}
__device__ __forceinline__ void buffer_load8(Vec8<float>& f, __amdgpu_buffer_rsrc_t r, int voff) {
    const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
    const float4 b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0));
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Store 4 consecutive elements.
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int voff, int soff, const f32x4& v, bf16) {
    bf16x4 q;
    q[0] = static_cast<bf16>(v[0]); q[1] = static_cast<bf16>(v[1]);
    q[2] = static_cast<bf16>(v[2]); q[3] = static_cast<bf16>(v[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, q), r, voff, soff, 0);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int voff, int soff, const f32x4& v, float) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 0);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (lane order).
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    // rows of 16: shift right by 1, 2, 4, 8 (lanes shifted in from outside the row read 0)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    // lane 15 of rows 0 and 2 into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of a group gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Renumber a linear workgroup index so that consecutive logical indices run on the same XCD.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    const int q = nblocks / kNumXcd, r = nblocks % kNumXcd;
    const int xcd = bid % kNumXcd, local = bid / kNumXcd;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + local;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace ssd
