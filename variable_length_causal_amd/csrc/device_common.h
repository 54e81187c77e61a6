// Device-side building blocks shared by the gtms kernels (gfx950 / CDNA4, wave64).
//
//  - element IO through buffer instructions: every row gets its own buffer resource whose
//    size is the number of bytes the kernel may touch, so the hardware range check turns
//    loads past the kept prefix into zeros that fetch nothing, and drops stores past the
//    row end; 16-byte vectors (dwordx4) on aligned rows, single elements otherwise;
//  - fp32 <-> binary16 / bfloat16 conversions, round-to-nearest-even;
//  - wavefront reductions over 64 lanes: DPP butterflies inside each 16-lane row, then the
//    four row results combined in scalar registers; every lane ends with the same bits;
//  - XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gtms {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, blocks dealt round-robin

// Cache-policy bits of a buffer access on gfx950: SC0 = 1, NT = 2 (non-temporal), SC1 = 16.
constexpr int kPolicyDefault = 0;
// Output stores (written once, never read back by the kernel): non-temporal at device scope.
// Measured against NT alone on MI355X: forward +0.4% to +5%, backward +1% to +3%.
constexpr int kPolicyStream = 2 | 16;
// Loads of data used once (the backward's y and dy): non-temporal. Backward +2.5% to +5.7%;
// in the forward they gained nothing.
constexpr int kPolicyReadOnce = 2;
// Non-temporal only, for stores that fill a line in several pieces (the attention output's
// 8-byte stores): the device-scope bit measured 3% to 18% slower there.
constexpr int kPolicyNt = 2;

// Raw buffer resource over [base, base + bytes): stride 0, 32-bit data format word.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// ------------------------------------------------------------------------- element IO
// Io<DT, WIDE>: WIDE moves 16 bytes per lane per access (VEC elements); otherwise one
// element per access. raw_t is the in-memory unit; unpack/pack convert VEC elements.
template <int DT, bool WIDE> struct Io;

struct Wide16 {
    using raw_t = u32x4;
    static constexpr int BYTES = 16;
    __device__ __forceinline__ static raw_t zero() { return raw_t{0u, 0u, 0u, 0u}; }
    template <int POL> __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
    }
    template <int POL> __device__ __forceinline__ static void store(rsrc_t r, int off, raw_t v) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POL);
    }
};

template <> struct Io<DT_F32, true> : Wide16 {
    static constexpr int VEC = 4;
    __device__ __forceinline__ static void unpack(raw_t r, float (&f)[VEC]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the lane out first: clang's __builtin_bit_cast of a vector element
            // expression reads element 0 whatever the index
            const uint32_t w = r[i];
            f[i] = __builtin_bit_cast(float, w);
        }
    }
    __device__ __forceinline__ static raw_t pack(const float (&f)[VEC]) {
        raw_t r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, f[i]);
        return r;
    }
};

template <> struct Io<DT_F32, false> {
    static constexpr int VEC = 1;
    static constexpr int BYTES = 4;
    using raw_t = uint32_t;
    __device__ __forceinline__ static raw_t zero() { return 0u; }
    template <int POL> __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL);
    }
    template <int POL> __device__ __forceinline__ static void store(rsrc_t r, int off, raw_t v) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, POL);
    }
    __device__ __forceinline__ static void unpack(raw_t r, float (&f)[VEC]) {
        f[0] = __builtin_bit_cast(float, r);
    }
    __device__ __forceinline__ static raw_t pack(const float (&f)[VEC]) {
        return __builtin_bit_cast(uint32_t, f[0]);
    }
};

// binary16: hardware conversions; bfloat16: widening is a 16-bit shift, narrowing uses the
// gfx950 round-to-nearest-even conversion.
template <int DT> struct Cvt16 {
    __device__ __forceinline__ static f32x2 widen(uint32_t w) {
        if constexpr (DT == DT_F16) {
            return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        } else {
            return f32x2{__builtin_bit_cast(float, w << 16),
                         __builtin_bit_cast(float, w & 0xffff0000u)};
        }
    }
    __device__ __forceinline__ static uint32_t narrow(float a, float b) {
        if constexpr (DT == DT_F16) {
            return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
        } else {
            return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
        }
    }
};

template <int DT> struct Io16Wide : Wide16 {
    static constexpr int VEC = 8;
    __device__ __forceinline__ static void unpack(raw_t r, float (&f)[VEC]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2 p = Cvt16<DT>::widen(r[i]);
            f[2 * i] = p[0];
            f[2 * i + 1] = p[1];
        }
    }
    __device__ __forceinline__ static raw_t pack(const float (&f)[VEC]) {
        raw_t r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = Cvt16<DT>::narrow(f[2 * i], f[2 * i + 1]);
        return r;
    }
};

template <int DT> struct Io16Narrow {
    static constexpr int VEC = 1;
    static constexpr int BYTES = 2;
    using raw_t = uint32_t;  // the element in the low 16 bits
    __device__ __forceinline__ static raw_t zero() { return 0u; }
    template <int POL> __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POL);
    }
    template <int POL> __device__ __forceinline__ static void store(rsrc_t r, int off, raw_t v) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, POL);
    }
    __device__ __forceinline__ static void unpack(raw_t r, float (&f)[VEC]) {
        f[0] = Cvt16<DT>::widen(r)[0];
    }
    __device__ __forceinline__ static raw_t pack(const float (&f)[VEC]) {
        return Cvt16<DT>::narrow(f[0], 0.0f) & 0xffffu;
    }
};

template <> struct Io<DT_F16, true> : Io16Wide<DT_F16> {};
template <> struct Io<DT_BF16, true> : Io16Wide<DT_BF16> {};
template <> struct Io<DT_F16, false> : Io16Narrow<DT_F16> {};
template <> struct Io<DT_BF16, false> : Io16Narrow<DT_BF16> {};

// ------------------------------------------------------------------ explicit mask bytes
// The kept flags of one vector of VEC elements from a byte mask (non-zero = kept), loaded
// as one VEC-byte access at a byte offset that is a multiple of VEC.
template <int VEC> struct MaskIo;
template <> struct MaskIo<1> {
    using raw_t = uint32_t;
    __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kPolicyDefault);
    }
    __device__ __forceinline__ static bool kept(raw_t m, int) { return m != 0; }
};
template <> struct MaskIo<4> {
    using raw_t = uint32_t;
    __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kPolicyDefault);
    }
    __device__ __forceinline__ static bool kept(raw_t m, int q) { return (m >> (8 * q)) & 0xFFu; }
};
template <> struct MaskIo<8> {
    struct raw_t { uint32_t lo, hi; };
    __device__ __forceinline__ static raw_t load(rsrc_t r, int off) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicyDefault);
        const uint32_t lo = v[0], hi = v[1];
        return {lo, hi};
    }
    __device__ __forceinline__ static bool kept(raw_t m, int q) {
        return ((q < 4 ? m.lo : m.hi) >> (8 * (q & 3))) & 0xFFu;
    }
};

// ------------------------------------------------------------------ wave64 reductions
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    // every lane named by the butterfly patterns below exists, so bound_ctrl is irrelevant
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, v), __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

struct OpMax { __device__ __forceinline__ static float f(float a, float b) { return fmaxf(a, b); } };
struct OpSum { __device__ __forceinline__ static float f(float a, float b) { return a + b; } };

// Reduce over the 64 lanes of the calling wavefront (all lanes active). DPP butterflies
// leave every lane of a 16-lane row holding the row's result; the four row results are
// then read into scalar registers and combined, so the value returned is wave-uniform and
// bit-identical for every lane.
template <class Op> __device__ __forceinline__ float wave_reduce(float v) {
    v = Op::f(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: neighbours
    v = Op::f(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: pairs within a quad
    v = Op::f(v, dpp<0x141>(v));  // row_half_mirror: quads within 8 lanes
    v = Op::f(v, dpp<0x140>(v));  // row_mirror: halves within a 16-lane row
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return Op::f(Op::f(r0, r1), Op::f(r2, r3));
}

// ------------------------------------------------------------------ block ordering
// Blocks are dealt to the XCDs round-robin (block i runs on XCD i % 8), and each XCD then
// advances through its share at its own pace. Renumber them so that each XCD works through
// chunks of 2^shift consecutive logical blocks (XCD x takes chunks x, x + 8, x + 16, ...):
// the blocks one XCD has in flight then cover one contiguous stretch of memory however far
// the XCDs drift apart. Blocks past the last whole round of 8 chunks keep their number.
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t bid, uint32_t nblk, uint32_t shift) {
    const uint32_t full = (nblk >> (shift + 3)) << (shift + 3);
    if (bid >= full) return bid;
    const uint32_t x = bid % kXcds, i = bid / kXcds;
    return ((((i >> shift) * kXcds) + x) << shift) + (i & ((1u << shift) - 1u));
}

// The same renumbering with chunks of any size ch: XCD x takes chunks x, x + 8, ...
__device__ __forceinline__ uint32_t xcd_grouped(uint32_t bid, uint32_t nblk, uint32_t ch) {
    const uint32_t span = kXcds * ch;
    const uint32_t full = nblk / span * span;
    if (bid >= full) return bid;
    const uint32_t x = bid % kXcds, i = bid / kXcds;
    return ((i / ch) * kXcds + x) * ch + i % ch;
}

__device__ __forceinline__ int clamp_len(int32_t raw, int S) {
    return raw < 0 ? 0 : (raw > S ? S : raw);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Hides a register value from the optimiser (an empty asm that claims to rewrite it), so that
// values derived from it before this point are recomputed rather than kept live after it. The
// row kernels use it so that neither the unpacked fp32 copy of a packed 16-bit row (twice its
// registers) nor the per-element keep conditions (one 64-bit lane mask in scalar registers
// each) live across a loop or a reduction: recomputing either costs one instruction.
template <class T> __device__ __forceinline__ void opaque(T& v) { asm volatile("" : "+v"(v)); }
template <bool ON, class T> __device__ __forceinline__ T fresh_if(T v) {
    if constexpr (ON) opaque(v);
    return v;
}

}  // namespace gtms
