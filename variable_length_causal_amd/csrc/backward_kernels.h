// Backward kernels of the grouped tril mask softmax (gfx950).
//
// For a row r of plane p with forward output y and upstream gradient g, the softmax
// derivative dy_i/dz_j = y_i (delta_ij - y_j) (page "ops(8) self-attention CUDA (下)",
// section 2.1) and z = scale * x give
//   dx_c = scale * y_c * (g_c - D),   D = sum over kept k of g_k * y_k,
// for kept c; every other element of dx is +0 (masked elements and padded rows do not
// reach the output). The kept set follows the mask kind MK of the forward kernels.
// Arithmetic is fp32; results are rounded to nearest-even into the element type.
//
// Memory: reads the kept intervals of y and g (for the tril mask, two triangles), with
// non-temporal loads where the read is the last; writes every row of dx in full. The layout,
// buffer-resource range checks, non-temporal stores, live-slot specialisation and line
// ownership are those of the forward kernels; the reduction is a plain sum (wave DPP +
// readlane, then LDS across the waves of a workgroup).
//
// Four kernels:
//   bwd_wave   one wavefront per row, y and g held in registers;
//   bwd_block  one workgroup of W wavefronts per row, up to 8 vectors of each per lane;
//   bwd_stash  16 wavefronts per row, 8 vectors per lane in registers and the rest of the
//              row (up to kStashVecs pairs) in LDS, for the computed masks on 16-byte rows;
//   bwd_stream one workgroup per row, two passes over both intervals, any length.
#pragma once

#include "forward_kernels.h"

namespace gtms {

// LEAN (kernels with NV * VEC >= kLeanElems) as for the forward row parts; here it also makes
// the output pass unpack y and g again instead of keeping the fp32 copies that dot() made.
template <class IO, int NA, int STRIDE, int MK, bool LEAN>
struct GradPart {
    using MIO = MaskIo<IO::VEC>;
    typename IO::raw_t ry[NA], rg[NA];
    typename MIO::raw_t mk[MK == MK_MASK ? NA : 1];
    float d;  // this thread's part of D

    __device__ __forceinline__ static int kept_count(int t, int j, int hv, const Cols& k) {
        const int v = t + j * STRIDE - hv;
        return v < 0 ? 0 : k.c1 + 1 - v * IO::VEC;
    }
    __device__ __forceinline__ static int kept_from(int t, int j, int hv, const Cols& k) {
        return MK == MK_TRIL ? 0 : k.c0 - (t + j * STRIDE - hv) * IO::VEC;
    }
    // The mask bytes of slot j (a placeholder for the other mask kinds).
    __device__ __forceinline__ typename MIO::raw_t mask_of(int j) const {
        if constexpr (MK == MK_MASK) return mk[j];
        else return typename MIO::raw_t{};
    }
    __device__ __forceinline__ static bool kept(const typename MIO::raw_t& mb, int q, int ka,
                                                int kc) {
        bool r = q < kc && (MK == MK_TRIL || q >= ka);
        if constexpr (MK == MK_MASK) r = r && MIO::kept(mb, q);
        return r;
    }

    __device__ __forceinline__ void load(rsrc_t iny, rsrc_t ing, rsrc_t min, int t, int hv,
                                         const Cols& k) {
        const int v0 = MK == MK_TRIL ? 0 : k.c0 / IO::VEC;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int v = t + j * STRIDE - hv;
            const int off = v < v0 ? kOutOfRange : v * IO::BYTES;
            ry[j] = IO::template load<kPolicyReadOnce>(iny, off);
            rg[j] = IO::template load<kPolicyReadOnce>(ing, off);
            if constexpr (MK == MK_MASK) mk[j] = MIO::load(min, v < v0 ? kOutOfRange : v * IO::VEC);
        }
    }

    __device__ __forceinline__ void dot(int t, int hv, const Cols& k) {
        constexpr int VEC = IO::VEC;
        d = 0.0f;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int kc = kept_count(t, j, hv, k), ka = kept_from(t, j, hv, k);
            const auto mb = mask_of(j);
            float fy[VEC], fg[VEC];
            IO::unpack(ry[j], fy);
            IO::unpack(rg[j], fg);
#pragma unroll
            for (int q = 0; q < VEC; ++q) d += kept(mb, q, ka, kc) ? fy[q] * fg[q] : 0.0f;
        }
    }

    template <int SP>
    __device__ __forceinline__ void write(rsrc_t out, int t, int hv, const Cols& k, float scale,
                                          float D) const {
        constexpr int VEC = IO::VEC;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int kc = fresh_if<LEAN>(kept_count(t, j, hv, k)),
                      ka = fresh_if<LEAN>(kept_from(t, j, hv, k));
            const auto mb = mask_of(j);
            const typename IO::raw_t y = fresh_if<LEAN>(ry[j]), g = fresh_if<LEAN>(rg[j]);
            float fy[VEC], fg[VEC], o[VEC];
            IO::unpack(y, fy);
            IO::unpack(g, fg);
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                o[q] = kept(mb, q, ka, kc) ? scale * fy[q] * (fg[q] - D) : 0.0f;
            IO::template store<SP>(out, (t + j * STRIDE) * IO::BYTES, IO::pack(o));
        }
    }
};

// Buffer resources over the row's interval [0, c1] of y, g and (explicit mask) the mask.
struct GradRows {
    rsrc_t y, g, m;
};

template <class IO, int MK>
__device__ __forceinline__ GradRows grad_rows(const FwdArgs& a, uint32_t plane, int r, int nin) {
    GradRows q;
    q.y = make_rsrc(row_ptr(a.x, plane, r, a), (uint32_t)(nin * IO::BYTES));
    q.g = make_rsrc(row_ptr(a.g, plane, r, a), (uint32_t)(nin * IO::BYTES));
    q.m = MK == MK_MASK ? make_rsrc(mask_row(a, plane, r), (uint32_t)(nin * IO::VEC)) : q.y;
    return q;
}

// ---------------------------------------------------------------------------- bwd_wave
template <int DT, bool WIDE, int NV, int SP, int MK>
__device__ __forceinline__ void bwd_wave_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                             int lane) {
    using IO = Io<DT, WIDE>;
    const Span sp = row_span<MK, IO::BYTES / IO::VEC>(a, plane, r, L);
    const rsrc_t out = make_rsrc(sp.out, sp.out_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_span<IO, SP>(sp, out, lane, kWave);
        else write_zero_slots<IO, 0, NV, kWave, SP>(out, lane);
        return;
    }
    const int nin = k.c1 / IO::VEC + 1;
    const GradRows in = grad_rows<IO, MK>(a, plane, r, nin);
    const IvRel iv = iv_layout<IO, MK>(a, sp, k, nin, out);
    const int hv = iv.shift;
    with_live_slots<NV>((iv.live + kWave - 1) / kWave, [&]<int NA>() {
        GradPart<IO, NA, kWave, MK, NV * IO::VEC >= kLeanElems> p;
        p.load(in.y, in.g, in.m, lane, hv, k);
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_outside<IO, SP>(sp, out, iv, lane, kWave);
        else write_zero_slots<IO, NA, NV, kWave, SP>(out, lane);
        p.dot(lane, hv, k);
        p.template write<SP>(iv.out, lane, hv, k, a.k, wave_reduce<OpSum>(p.d));
    });
}

template <int DT, bool WIDE, int NV, int WPB, int SP, int MK>
__global__ __launch_bounds__(WPB * kWave) void bwd_wave(FwdArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = WPB == 1 ? 0u : (uint32_t)uniform(threadIdx.x / kWave);
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = (uint64_t)blk * WPB + wave; unit < a.n_units;
         unit += (uint64_t)nblk * WPB) {
        const Unit u = decode_unit<MK, false>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        bwd_wave_row<DT, WIDE, NV, SP, MK>(a, u.plane, u.r0, L, lane);
        if (u.r1 >= 0) bwd_wave_row<DT, WIDE, NV, SP, MK>(a, u.plane, u.r1, L, lane);
    }
}

// --------------------------------------------------------------------------- bwd_block
template <int DT, bool WIDE, int NV, int W, int SP, int MK>
__device__ __forceinline__ void bwd_block_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                              float* pd) {
    using IO = Io<DT, WIDE>;
    constexpr int T = W * kWave;
    const int t = threadIdx.x;
    const Span sp = row_span<MK, IO::BYTES / IO::VEC>(a, plane, r, L);
    const rsrc_t out = make_rsrc(sp.out, sp.out_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_span<IO, SP>(sp, out, t, T);
        else write_zero_slots<IO, 0, NV, T, SP>(out, t);
        return;
    }
    const int wave = uniform(t / kWave);
    const int nin = k.c1 / IO::VEC + 1;
    const GradRows in = grad_rows<IO, MK>(a, plane, r, nin);
    const IvRel iv = iv_layout<IO, MK>(a, sp, k, nin, out);
    const int hv = iv.shift;
    with_live_slots<NV>((iv.live + T - 1) / T, [&]<int NA>() {
        GradPart<IO, NA, T, MK, NV * IO::VEC >= kLeanElems> p;
        p.load(in.y, in.g, in.m, t, hv, k);
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_outside<IO, SP>(sp, out, iv, t, T);
        else write_zero_slots<IO, NA, NV, T, SP>(out, t);
        p.dot(t, hv, k);
        const float dw = wave_reduce<OpSum>(p.d);
        if ((t & (kWave - 1)) == 0) pd[wave] = dw;
        __syncthreads();
        float D = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) D += pd[w];
        p.template write<SP>(iv.out, t, hv, k, a.k, D);
    });
}

template <int DT, bool WIDE, int NV, int W, int SP, int MK>
__global__ __launch_bounds__(W * kWave) void bwd_block(FwdArgs a) {
    __shared__ float part[2][W];  // [row of the unit][wave]
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = blk; unit < a.n_units; unit += nblk) {
        const Unit u = decode_unit<MK, (W >= 8)>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        bwd_block_row<DT, WIDE, NV, W, SP, MK>(a, u.plane, u.r0, L, part[0]);
        if (u.r1 >= 0) bwd_block_row<DT, WIDE, NV, W, SP, MK>(a, u.plane, u.r1, L, part[1]);
        __syncthreads();  // the next unit rewrites the partials
    }
}

// --------------------------------------------------------------------------- bwd_stash
// Rows past 8 vectors per lane of a 16-wavefront workgroup (16-bit rows of more than 65536
// elements, binary32 rows of more than 32768), for the computed masks on rows of 16-byte
// vectors. Both passes need y and g, 32 bytes per vector position, and a lane of such a
// workgroup has 128 registers: at 16 vectors per lane bwd_block's row part spills. So each
// lane keeps 8 slots in registers (bwd_block's GradPart) and the row's further vectors, up to
// kStashVecs of each of y and g, go to LDS. The buffer unit writes them there itself (loads
// with the LDS flag: lane l's 16 bytes land at the wavefront's base + 16 l, a lane whose
// offset fails the range check writes zeros), so they take no registers. Stash entry
// i = n * T + t (slot NV + n of thread t) is filled by thread t's own load and read only by
// thread t, so a wait for the thread's own loads orders them, and the next row's loads
// follow this row's reads in program order. Every element of y and g crosses HBM once, as
// on the block path; the stream path reads both twice.
constexpr int kStashVecs = 5056;  // 2 x 5056 x 16 = 161792 bytes of the 160 KiB of LDS
static_assert(kStashVecs % kWave == 0, "each wavefront fills whole 1 KiB blocks");

// Zeros into the span's slots [from, end of span), thread t of T taking every T-th slot.
template <class IO, int SP>
__device__ __forceinline__ void write_zeros_from(const Span& sp, rsrc_t out, int from, int t,
                                                 int T) {
    const int nspan = (int)(sp.out_bytes / IO::BYTES);
    for (int s = from + t; s < nspan; s += T) IO::template store<SP>(out, s * IO::BYTES, IO::zero());
}

template <int DT, int NV, int W, int SP, int MK>
__device__ __forceinline__ void bwd_stash_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                              float* pd, u32x4* ys, u32x4* gs) {
    using IO = Io<DT, true>;
    constexpr int T = W * kWave;
    constexpr int VEC = IO::VEC;
    constexpr bool LEAN = NV * VEC >= kLeanElems;
    constexpr int NSL = (kStashVecs + T - 1) / T;  // stash slots per thread, at most
    static_assert(MK != MK_MASK, "the explicit mask's bytes have no stash");
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const Span sp = row_span<MK, IO::BYTES / VEC>(a, plane, r, L);
    const rsrc_t out = make_rsrc(sp.out, sp.out_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {
        write_zeros_span<IO, SP>(sp, out, t, T);
        return;
    }
    const int wave = uniform(t / kWave);
    const int nin = k.c1 / VEC + 1;
    const GradRows in = grad_rows<IO, MK>(a, plane, r, nin);
    const IvRel iv = iv_layout<IO, MK>(a, sp, k, nin, out);
    const bool ivrel = MK == MK_BAND && (a.flags & F_IVREL);
    const int hv = iv.shift;
    auto merge = [&](float d) {
        const float dw = wave_reduce<OpSum>(d);
        if (lane == 0) pd[wave] = dw;
        __syncthreads();
        float D = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) D += pd[w];
        return D;
    };
    if (iv.live <= NV * T) {  // uniform: the row fits the registers (bwd_block's row)
        with_live_slots<NV>((iv.live + T - 1) / T, [&]<int NA>() {
            GradPart<IO, NA, T, MK, LEAN> p;
            p.load(in.y, in.g, in.m, t, hv, k);
            if (ivrel) write_zeros_outside<IO, SP>(sp, out, iv, t, T);
            else write_zeros_from<IO, SP>(sp, out, NA * T, t, T);
            p.dot(t, hv, k);
            p.template write<SP>(iv.out, t, hv, k, a.k, merge(p.d));
        });
        return;
    }
    // Slots NV and up live in LDS: the held positions [NV*T, live) of the row part, at most
    // kStashVecs of them (the host's choice of this kernel guarantees it).
    using GP = GradPart<IO, NV, T, MK, LEAN>;
    const int nst = iv.live - NV * T;
    const int v0 = MK == MK_TRIL ? 0 : k.c0 / VEC;
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
        const int base = n * T + wave * kWave;  // the wavefront's first entry of this slot
        if (base < nst) {                       // uniform; base + 64 <= nst rounded up <= kStashVecs
            const int i = base + lane, v = NV * T + i - hv;
            const int off = i >= nst || v < v0 ? kOutOfRange : v * IO::BYTES;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                in.y, (__attribute__((address_space(3))) void*)(ys + base), 16, off, 0, 0,
                kPolicyReadOnce);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                in.g, (__attribute__((address_space(3))) void*)(gs + base), 16, off, 0, 0,
                kPolicyReadOnce);
        }
    }
    GP p;
    p.load(in.y, in.g, in.m, t, hv, k);
    if (ivrel) write_zeros_outside<IO, SP>(sp, out, iv, t, T);
    else write_zeros_from<IO, SP>(sp, out, iv.live, t, T);
    p.dot(t, hv, k);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stash entries have landed
    float d = p.d;
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
        const int i = n * T + t;
        if (i < nst) {
            const int j = NV + n;
            const int kc = GP::kept_count(t, j, hv, k), ka = GP::kept_from(t, j, hv, k);
            float fy[VEC], fg[VEC];
            IO::unpack(ys[i], fy);
            IO::unpack(gs[i], fg);
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                d += GP::kept(typename GP::MIO::raw_t{}, q, ka, kc) ? fy[q] * fg[q] : 0.0f;
        }
    }
    const float D = merge(d);
    p.template write<SP>(iv.out, t, hv, k, a.k, D);
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
        const int i = n * T + t;
        if (i < nst) {
            const int j = NV + n;
            const int kc = GP::kept_count(t, j, hv, k), ka = GP::kept_from(t, j, hv, k);
            float fy[VEC], fg[VEC], o[VEC];
            IO::unpack(ys[i], fy);
            IO::unpack(gs[i], fg);
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                o[q] = GP::kept(typename GP::MIO::raw_t{}, q, ka, kc) ? a.k * fy[q] * (fg[q] - D)
                                                                       : 0.0f;
            IO::template store<SP>(iv.out, (t + j * T) * IO::BYTES, IO::pack(o));
        }
    }
}

template <int DT, int NV, int W, int SP, int MK>
__global__ __launch_bounds__(W * kWave) void bwd_stash(FwdArgs a) {
    __shared__ __attribute__((aligned(16))) u32x4 ys[kStashVecs], gs[kStashVecs];
    __shared__ float part[2][W];
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = blk; unit < a.n_units; unit += nblk) {
        const Unit u = decode_unit<MK, false>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        bwd_stash_row<DT, NV, W, SP, MK>(a, u.plane, u.r0, L, part[0], ys, gs);
        if (u.r1 >= 0) bwd_stash_row<DT, NV, W, SP, MK>(a, u.plane, u.r1, L, part[1], ys, gs);
        __syncthreads();
    }
}

// -------------------------------------------------------------------------- bwd_stream
// Rows of any length: pass 1 accumulates D, pass 2 re-reads both intervals and writes.
template <int DT, bool WIDE, int W, int SP, int MK>
__device__ __forceinline__ void bwd_stream_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                               float* pd) {
    using IO = Io<DT, WIDE>;
    using MIO = MaskIo<IO::VEC>;
    constexpr int VEC = IO::VEC;
    constexpr int T = W * kWave;
    const int t = threadIdx.x;
    const int nraw = a.row_bytes / IO::BYTES;
    const rsrc_t out = make_rsrc(row_ptr(a.y, plane, r, a), (uint32_t)a.row_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {
        for (int v = t; v < nraw; v += T) IO::template store<SP>(out, v * IO::BYTES, IO::zero());
        return;
    }
    const int wave = uniform(t / kWave);
    const int v0 = k.c0 / VEC, nin = k.c1 / VEC + 1;
    const GradRows in = grad_rows<IO, MK>(a, plane, r, nin);
    for (int v = t; v < v0; v += T) IO::template store<SP>(out, v * IO::BYTES, IO::zero());
    for (int v = nin + t; v < nraw; v += T) IO::template store<SP>(out, v * IO::BYTES, IO::zero());
    auto kept = [&](int v, int e, const typename MIO::raw_t& mb) {
        const int c = v * VEC + e;
        bool r = c >= k.c0 && c <= k.c1;
        if constexpr (MK == MK_MASK) r = r && MIO::kept(mb, e);
        return r;
    };
    float d = 0.0f;
    for (int v = v0 + t; v < nin; v += T) {
        float fy[VEC], fg[VEC];
        IO::unpack(IO::template load<kPolicyDefault>(in.y, v * IO::BYTES), fy);
        IO::unpack(IO::template load<kPolicyDefault>(in.g, v * IO::BYTES), fg);
        typename MIO::raw_t mb{};
        if constexpr (MK == MK_MASK) mb = MIO::load(in.m, v * VEC);
#pragma unroll
        for (int q = 0; q < VEC; ++q) d += kept(v, q, mb) ? fy[q] * fg[q] : 0.0f;
    }
    const float dw = wave_reduce<OpSum>(d);
    if ((t & (kWave - 1)) == 0) pd[wave] = dw;
    __syncthreads();
    float D = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) D += pd[w];
    for (int v = v0 + t; v < nin; v += T) {
        float fy[VEC], fg[VEC], o[VEC];
        IO::unpack(IO::template load<kPolicyReadOnce>(in.y, v * IO::BYTES), fy);
        IO::unpack(IO::template load<kPolicyReadOnce>(in.g, v * IO::BYTES), fg);
        typename MIO::raw_t mb{};
        if constexpr (MK == MK_MASK) mb = MIO::load(in.m, v * VEC);
#pragma unroll
        for (int q = 0; q < VEC; ++q) o[q] = kept(v, q, mb) ? a.k * fy[q] * (fg[q] - D) : 0.0f;
        IO::template store<SP>(out, v * IO::BYTES, IO::pack(o));
    }
}

template <int DT, bool WIDE, int W, int SP, int MK>
__global__ __launch_bounds__(W * kWave) void bwd_stream(FwdArgs a) {
    __shared__ float part[2][W];
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = blk; unit < a.n_units; unit += nblk) {
        const Unit u = decode_unit<MK, true>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        bwd_stream_row<DT, WIDE, W, SP, MK>(a, u.plane, u.r0, L, part[0]);
        if (u.r1 >= 0) bwd_stream_row<DT, WIDE, W, SP, MK>(a, u.plane, u.r1, L, part[1]);
        __syncthreads();
    }
}

}  // namespace gtms
