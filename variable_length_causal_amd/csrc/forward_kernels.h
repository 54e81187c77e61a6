// Forward kernels of the grouped tril mask softmax (gfx950).
//
// Operation (page "Fused grouped tril mask softmax", github aoxy/Attention-Mask-Optimization
// README, operator-behaviour section): for plane p = b*M + m of X[B, M, S, S] and row r,
// with L = clamp(seq_lens[b], 0, S):
//   r <  L : y[c] = exp(s*x[c] - max) / sum_{k<=r} exp(s*x[k] - max) for c <= r, else +0
//   r >= L : y[c] = +0 for every c
// The mask is the predicate (c <= r < L), evaluated in registers. The README's
// implementation notes split the work the same way: a load side that supplies the masked
// value without reading memory and a store side that writes the zeros.
//
// Arithmetic: z = x * k with k = scale * log2(e), so exp is the hardware v_exp_f32 (2^z)
// and the max subtraction happens in the log2 domain. Accumulation is fp32.
//
// Memory: only the kept prefix of a row is read. Its buffer resource ends at the 16-byte
// vector that holds column r, so lanes past it get zeros from the range check without a
// fetch, and the elements of that last vector past column r are discarded by the
// predicate. Every row is written in full with non-temporal dwordx4 stores; padded rows
// are stores only. Writes are about 85-90% of the bytes. Stores of vectors that lie wholly
// past the prefix need no data, so they are issued right after the prefix loads and drain
// while those loads are in flight.
//
// Three kernels:
//   fwd_wave   one wavefront per row, kept prefix held in registers (NV vectors per lane);
//   fwd_block  one workgroup of W wavefronts per row, per-wave (max, sum) partials merged
//              through LDS with the log-sum-exp rule of the split-KV reduction in
//              ColossalAI's flash_decoding.py (_flash_decoding_fwd_reduce_kernel); at 16
//              vectors per lane a lane keeps raw vectors only (RowPart's RAW mode), so that
//              a workgroup of 16 wavefronts holds 256 KB of a row;
//   fwd_stream one workgroup per row, two passes (online max/sum, then normalise) for rows
//              too long for registers.
// A work unit is one row, or optionally the pair (r, S-1-r), whose kept prefixes add up to
// S+1 columns whatever r is. Units are taken in row order, each XCD working through chunks
// of consecutive workgroups (xcd_chunked): the rows written at any moment then sit close
// together in memory, which HBM rewards (measured on MI355X: pairing rows cost 5-10%).
// With an explicit mask whose rows several planes share (F_ACROSS), units run in blocks of
// rows taken plane after plane, so that the planes' uses of one mask row fall together in
// time while the rows written still form runs of whole blocks.
//
// Mask variants (page "优化ScaledMaskSoftmax算子", the ScaledMaskSoftmax article): masked
// scores count as minus infinity (section 2.1), a row with no kept element is zeros
// (section 4.1), and section 6 builds window masks with tril, per-task masks broadcast over
// the batch and per-sample length masks. The template parameter MK selects the kept set of
// row r (valid length L; nothing is kept when r >= L):
//   MK_TRIL  c <= r                                   (the grouped tril mask)
//   MK_BAND  lo <= c - r <= hi, c < L                 (computed, never loaded)
//   MK_MASK  mask[b, m, r, c] != 0, c < L             (one byte per element, loaded with
//                                                      the scores; broadcast by strides)
// In every case the kept columns lie in one interval [c0, c1] (Cols); only the vectors of
// that interval are read, and everything outside it is written as zeros.
#pragma once

#include "device_common.h"

namespace gtms {

enum : unsigned { F_PAIR = 1u, F_XCD = 2u, F_LINES = 4u, F_IVREL = 8u, F_ACROSS = 16u };
enum : int { MK_TRIL = 0, MK_BAND = 1, MK_MASK = 2 };


// Arguments of the forward (x -> y) and backward (y = x, upstream gradient g -> dx = y)
// kernels.
struct FwdArgs {
    const void* x;
    void* y;
    const void* g;             // backward only: the upstream gradient
    const int32_t* seq_lens;
    uint32_t n_units;          // work units in the launch (< 2^32, checked on the host)
    uint32_t units_per_plane;  // S, or ceil(S/2) when rows are paired
    uint32_t n_planes;         // B * M
    uint32_t M;
    int S;
    int row_bytes;             // S * element size
    float k;                   // forward: scale * log2(e); backward: scale
    unsigned flags;
    uint32_t xcd_shift;        // F_XCD: log2 of the blocks in one XCD chunk
    uint32_t across_shift;     // F_ACROSS: log2 of the rows per block of the unit order
    int lo, hi;                // MK_BAND: kept when lo <= c - r <= hi (clamped to [-S, S])
    const uint8_t* mask;       // MK_MASK: element (b, m, r, c) at mask[b*sb + m*sm + r*sr + c]
    int64_t mask_sb, mask_sm, mask_sr;
};

struct Unit {
    uint32_t plane;
    int r0, r1;  // rows of the unit; r1 < 0 when the unit is one row
};

// ACROSS: the kernel honours F_ACROSS (compiled into the kernels of long rows only: the block
// path at 8 or more wavefronts per row and the stream path); the others ignore the flag,
// which changes the order of the units and nothing else.
template <int MK, bool ACROSS>
__device__ __forceinline__ Unit decode_unit(uint32_t unit, const FwdArgs& a) {
    Unit u;
    if (MK == MK_MASK && ACROSS && (a.flags & F_ACROSS)) {
        // blocks of R = 2^across_shift rows, each taken plane after plane:
        // unit = (rb * n_planes + plane) * R + (r0 - rb * R); the last, shorter block of
        // T < R rows follows as unit = full_units + plane * T + (r0 - full * R)
        const uint32_t sh = a.across_shift;
        const uint32_t full = a.units_per_plane >> sh;  // whole blocks per plane
        const uint32_t full_units = (full * a.n_planes) << sh;
        if (unit < full_units) {
            const uint32_t per = a.n_planes << sh;  // at most n_units, as full >= 1
            const uint32_t rb = unit / per, rem = unit - rb * per;
            u.plane = rem >> sh;
            u.r0 = (int)((rb << sh) + (rem & ((1u << sh) - 1)));
        } else {
            const uint32_t t = unit - full_units, T = a.units_per_plane - (full << sh);
            u.plane = t / T;
            u.r0 = (int)((full << sh) + (t - u.plane * T));
        }
    } else {  // unit = plane * units_per_plane + r0
        u.plane = unit / a.units_per_plane;
        u.r0 = (int)(unit - u.plane * a.units_per_plane);
    }
    const int partner = a.S - 1 - u.r0;
    u.r1 = !(a.flags & F_PAIR) || partner == u.r0 ? -1 : partner;
    return u;
}

__device__ __forceinline__ const char* row_ptr(const void* base, uint32_t plane, int r,
                                               const FwdArgs& a) {
    return (const char*)base +
           ((uint64_t)plane * (uint64_t)a.S + (uint64_t)r) * (uint64_t)a.row_bytes;
}

// Valid length of the plane's batch: seq_lens[b] clamped to [0, S], or S without lengths
// (the mask variants accept none).
template <int MK>
__device__ __forceinline__ int valid_len(const FwdArgs& a, uint32_t plane) {
    if (MK != MK_TRIL && !a.seq_lens) return a.S;
    return clamp_len(a.seq_lens[plane / a.M], a.S);
}

// The interval [c0, c1] of columns that may be kept in row r; empty when c1 < c0.
struct Cols {
    int c0, c1;
    __device__ __forceinline__ bool empty() const { return c1 < c0; }
};

template <int MK>
__device__ __forceinline__ Cols kept_cols(const FwdArgs& a, int r, int L) {
    if (r >= L) return {0, -1};
    if constexpr (MK == MK_TRIL) return {0, r};
    else if constexpr (MK == MK_BAND) return {max(0, r + a.lo), min(L - 1, r + a.hi)};
    else return {0, L - 1};
}

__device__ __forceinline__ const uint8_t* mask_row(const FwdArgs& a, uint32_t plane, int r) {
    const uint32_t b = plane / a.M, m = plane - b * a.M;
    return a.mask + (int64_t)b * a.mask_sb + (int64_t)m * a.mask_sm + (int64_t)r * a.mask_sr;
}

// Zeros into slots [FROM, TO) of a row held with stride STRIDE (slots past the row end are
// dropped by the range check of `out`).
template <class IO, int FROM, int TO, int STRIDE, int SP>
__device__ __forceinline__ void write_zero_slots(rsrc_t out, int t) {
#pragma unroll
    for (int j = FROM; j < TO; ++j)
        IO::template store<SP>(out, (t + j * STRIDE) * IO::BYTES, IO::zero());
}

// ------------------------------------------------------------------ line ownership
// Rows of binary32 X[., ., 1000, 1000] are 4000 bytes long, so most rows start and end in
// the middle of a 128-byte line. Two wavefronts writing the two halves of one line at
// different times cost HBM a partial-line write each (measured on MI355X: pure stores of
// 4000-byte rows reach 4.6 TB/s this way, 5.6 TB/s when every wavefront writes whole
// lines). So on rows of 128 bytes or more, each boundary line is written by ONE row:
//   - a row's tail zone (the part of its last line that lies in the row) is handed to the
//     next row when it holds only zeros, i.e. when the row is padded or its kept prefix
//     ends before the zone; the next row then writes the zone's zeros in front of its own
//     data, and the whole line goes out in one store;
//   - otherwise the row keeps its tail zone and the line is written in two parts.
// The first row of the tensor never extends before the tensor, nor the last one after it.
// A row that takes the zone shifts its vectors by hv = zone bytes / 16 slots, so lane t
// slot j holds the row's natural vector t + j*STRIDE - hv (negative: the zone's zeros).
struct Span {
    const char* out;     // first byte this row writes
    uint32_t out_bytes;  // bytes it writes
    int hv;              // leading slots that belong to the previous row's tail zone
};

// Whether the last `zone` bytes of row r (valid length L) may hold kept elements (for an
// explicit mask: whether they lie in the row's interval, whatever the mask bytes say).
template <int MK>
__device__ __forceinline__ bool tail_zone_has_data(const FwdArgs& a, int r, int L, int zone,
                                                   int esize) {
    if (zone == 0) return false;
    const Cols k = kept_cols<MK>(a, r, L);
    return !k.empty() && k.c1 >= a.S - zone / esize;
}

template <int MK, int ESIZE>
__device__ __forceinline__ Span row_span(const FwdArgs& a, uint32_t plane, int r, int L) {
    Span sp;
    const char* row = row_ptr(a.y, plane, r, a);
    sp.out = row;
    sp.out_bytes = (uint32_t)a.row_bytes;
    sp.hv = 0;
    if (!(a.flags & F_LINES)) return sp;
    const int head = (int)((uintptr_t)row & 127);                  // previous row's tail zone
    const int tail = (int)((uintptr_t)(row + a.row_bytes) & 127);  // this row's tail zone
    const bool first = plane == 0 && r == 0;
    const bool last = plane + 1 == a.n_planes && r + 1 == a.S;
    if (head && !first) {
        bool prev_data;
        if (r > 0) {
            prev_data = tail_zone_has_data<MK>(a, r - 1, L, head, ESIZE);
        } else {
            const int Lp = valid_len<MK>(a, plane - 1);
            prev_data = tail_zone_has_data<MK>(a, a.S - 1, Lp, head, ESIZE);
        }
        if (!prev_data) {
            sp.out -= head;
            sp.out_bytes += head;
            sp.hv = head / 16;
        }
    }
    if (tail && !last && !tail_zone_has_data<MK>(a, r, L, tail, ESIZE)) sp.out_bytes -= tail;
    return sp;
}

// ------------------------------------------------------------- narrow bands (F_IVREL)
// A band narrower than the row keeps only its interval's vectors in registers: slot j of
// thread t holds the natural vector v0 + t + j*STRIDE, v0 the first vector of the interval's
// first 128-byte line, so that the row parts run with the shift -v0, and everything outside
// those lines is plain zero stores. The host picks the kernel from the interval's width instead of S: a
// 512-column causal window on rows of 4096 takes one wavefront per row, without the
// workgroup's barrier. Full-width bands keep the row-relative slots, and so the tril mask's
// bits.
struct IvRel {
    int shift;   // the row parts' slot shift: -v0 (interval-relative) or the span's hv
    int live;    // vectors the row parts hold
    rsrc_t out;  // where the row parts write: the interval's vectors, or the whole span
};

template <class IO, int MK>
__device__ __forceinline__ IvRel iv_layout(const FwdArgs& a, const Span& sp, const Cols& k,
                                           int nin, rsrc_t span_out) {
    if (MK == MK_BAND && (a.flags & F_IVREL)) {
        // The held region is the interval widened to whole 128-byte lines inside the span, so
        // that no line is written in two parts at two times (the zero stores early, the data
        // late); its vectors before c0 and after c1 are written as zeros with the data.
        const int nspan = (int)(sp.out_bytes / IO::BYTES);
        const uintptr_t base = (uintptr_t)sp.out;
        const uintptr_t first = (base + (uintptr_t)(k.c0 / IO::VEC + sp.hv) * IO::BYTES) & ~uintptr_t(127);
        const uintptr_t last = (base + (uintptr_t)(nin + sp.hv) * IO::BYTES + 127) & ~uintptr_t(127);
        const int s0 = first <= base ? 0 : (int)((first - base) / IO::BYTES);
        const int s1 = min(nspan, (int)((last - base) / IO::BYTES));
        return {sp.hv - s0, s1 - s0,
                make_rsrc(sp.out + s0 * IO::BYTES, (uint32_t)((s1 - s0) * IO::BYTES))};
    }
    return {sp.hv, nin + sp.hv, span_out};
}

// Interval-relative rows: zeros into the whole span (a row with nothing kept: the kernel's
// slots are sized for the interval, not the row), thread t of T taking every T-th slot.
template <class IO, int SP>
__device__ __forceinline__ void write_zeros_span(const Span& sp, rsrc_t out, int t, int T) {
    const int nspan = (int)(sp.out_bytes / IO::BYTES);
    for (int s = t; s < nspan; s += T) IO::template store<SP>(out, s * IO::BYTES, IO::zero());
}

// Interval-relative rows: zeros into the span's slots before and after the held region (slots
// [sp.hv - shift, sp.hv - shift + live)), thread t of T taking every T-th slot.
template <class IO, int SP>
__device__ __forceinline__ void write_zeros_outside(const Span& sp, rsrc_t out, const IvRel& iv,
                                                    int t, int T) {
    const int nspan = (int)(sp.out_bytes / IO::BYTES);
    const int a = sp.hv - iv.shift, b = a + iv.live;
    for (int s = t; s < a; s += T) IO::template store<SP>(out, s * IO::BYTES, IO::zero());
    for (int s = b + t; s < nspan; s += T) IO::template store<SP>(out, s * IO::BYTES, IO::zero());
}

// ------------------------------------------------------------ one row, NA live slots
// A row is held by a group of threads: thread `t` owns slots t + j*STRIDE, slot i holding
// the row's natural vector i - hv. Only the first NA slots can hold kept columns (the
// caller picks NA from the prefix length, so the code for each NA is straight-line); the
// caller writes the other slots as zeros.
//
// Each thread first reduces its own elements: m_t = max z, e = 2^(z - m_t), s_t = sum e,
// keeping e in registers. The group then merges the partials as the split-KV reduction of
// ColossalAI's flash_decoding.py does (_flash_decoding_fwd_reduce_kernel):
//   M = max_t m_t,  S = sum_t s_t * 2^(m_t - M),  y = e * 2^(m_t - M) / S,
// so each element costs one exp. A thread without kept columns has m_t = -inf, s_t = 0.
//
// LEAN is set by kernels whose lanes hold 64 or more elements (NV * VEC >= 64). The keep
// conditions of the output pass are then rebuilt from opaque copies of their inputs (see
// opaque()) instead of being kept live across the reduction: at that size they no longer fit
// in scalar registers and spill. Smaller kernels run faster without it.
constexpr int kOutOfRange = (int)0x80000000u;  // an offset every buffer range check rejects

// Lanes holding this many elements or more run the LEAN variants of the row parts.
constexpr int kLeanElems = 64;
// Rows that need this many vectors per lane run the RAW variants: a lane keeps only its raw
// 16-byte vectors (64 registers at 16 vectors), and the max, sum and write passes each unpack
// them again; the write pass recomputes 2^(z - m) instead of keeping it. The fp32 values of 16
// vectors (128 registers for 16-bit types) would not fit beside them: with RAW a workgroup of
// 16 wavefronts holds 256 KB of a row (16-bit rows of 131072 elements, binary32 of 65536).
constexpr int kRawNV = 16;

template <class IO, int NA, int STRIDE, int MK, bool LEAN, bool RAW = false>
struct RowPart {
    using MIO = MaskIo<IO::VEC>;
    typename IO::raw_t raw[NA];
    typename MIO::raw_t mk[MK == MK_MASK ? NA : 1];
    float e[RAW ? 1 : NA][IO::VEC];
    float m, s;
    float kk;  // RAW: the scale, kept for the write pass

    // Element q of the vector in slot j is kept when its column c = v*VEC + q lies in
    // [c0, c1] (and, for an explicit mask, its mask byte is non-zero): q >= ka and q < kc.
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

    // Vectors before the interval (and the previous row's zone, v < 0) are not fetched.
    __device__ __forceinline__ void load(rsrc_t in, rsrc_t min, int t, int hv, const Cols& k) {
        const int v0 = MK == MK_TRIL ? 0 : k.c0 / IO::VEC;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int v = t + j * STRIDE - hv;
            const bool skip = v < v0;
            // an explicit mask's scores stream past (non-temporal), so that the mask rows the
            // planes share stay in L2
            raw[j] = IO::template load<MK == MK_MASK ? kPolicyReadOnce : kPolicyDefault>(
                in, skip ? kOutOfRange : v * IO::BYTES);
            if constexpr (MK == MK_MASK)
                mk[j] = MIO::load(min, skip ? kOutOfRange : v * IO::VEC);
        }
    }

    // RAW: every pass starts from opaque copies of the thread's position and the interval
    // (fresh_pass), and each slot's raw vector (and mask bytes) passes through an opaque copy
    // (raw_slot), so that no pass reuses another pass's unpacked values or keep bounds.
    struct Fresh {
        int t, hv;
        Cols k;
    };
    __device__ __forceinline__ static Fresh fresh_pass(int t, int hv, const Cols& k) {
        Fresh f{t, hv, k};
        opaque(f.t);
        opaque(f.hv);
        opaque(f.k.c0);
        opaque(f.k.c1);
        return f;
    }
    // `after`: the previous slot's result; the copy takes it as an input, so that the slots
    // are worked through one after another (otherwise every slot's values are computed
    // first, and all of them are live at once).
    __device__ __forceinline__ void raw_slot(const Fresh& fr, int j, float after, float (&f)[IO::VEC],
                                             typename MIO::raw_t& mb, int& kc, int& ka) const {
        typename IO::raw_t r = raw[j];
        asm volatile("" : "+v"(r) : "v"(after));
        IO::unpack(r, f);
        mb = mask_of(j);
        if constexpr (MK == MK_MASK) opaque(mb);
        kc = kept_count(fr.t, j, fr.hv, fr.k);
        ka = kept_from(fr.t, j, fr.hv, fr.k);
    }
    // RAW: what slot j holds for the whole wavefront (uniform): no kept element, only kept
    // elements (never for an explicit mask, whose bytes decide), or a mix. Slots of a long
    // row's thread often lie wholly before or past its interval, or wholly inside it.
    enum : int { kSlotEmpty = 0, kSlotFull = 1, kSlotMixed = 2 };
    __device__ __forceinline__ static int slot_class(int t, int j, int hv, const Cols& k) {
        constexpr int VEC = IO::VEC;
        const int lo = uniform(t & ~(kWave - 1)) + j * STRIDE - hv;  // the wave's first vector
        const int hi = lo + kWave - 1;
        if (hi < 0 || lo * VEC > k.c1 || hi * VEC + VEC - 1 < k.c0) return kSlotEmpty;
        if (MK != MK_MASK && lo >= 0 && lo * VEC >= k.c0 && hi * VEC + VEC - 1 <= k.c1)
            return kSlotFull;
        return kSlotMixed;
    }
    __device__ __forceinline__ static float tree_sum(const float (&x)[IO::VEC]) {
        if constexpr (IO::VEC == 1) {
            return x[0];
        } else {
            float y[IO::VEC / 2];
#pragma unroll
            for (int i = 0; i < IO::VEC / 2; ++i) y[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
            for (int w = IO::VEC / 4; w >= 1; w /= 2)
#pragma unroll
                for (int i = 0; i < w; ++i) y[i] = y[2 * i] + y[2 * i + 1];
            return y[0];
        }
    }

    __device__ __forceinline__ void compute(int t, int hv, const Cols& k, float kscale) {
        constexpr int VEC = IO::VEC;
        if constexpr (RAW) {
            kk = kscale;
            m = -INFINITY;
            const Fresh f1 = fresh_pass(t, hv, k);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int sc = slot_class(t, j, hv, k);
                if (sc == kSlotEmpty) continue;
                float f[VEC];
                typename MIO::raw_t mb;
                int kc, ka;
                raw_slot(f1, j, m, f, mb, kc, ka);
                float lm = -INFINITY;
                if (sc == kSlotFull) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q) lm = fmaxf(lm, f[q] * kscale);
                } else {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        lm = fmaxf(lm, kept(mb, q, ka, kc) ? f[q] * kscale : -INFINITY);
                }
                m = fmaxf(m, lm);
            }
            const float mm = m == -INFINITY ? 0.0f : m;
            s = 0.0f;
            const Fresh f2 = fresh_pass(t, hv, k);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int sc = slot_class(t, j, hv, k);
                if (sc == kSlotEmpty) continue;
                float f[VEC];
                typename MIO::raw_t mb;
                int kc, ka;
                raw_slot(f2, j, s, f, mb, kc, ka);
                if (sc == kSlotFull) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q) f[q] = __builtin_amdgcn_exp2f(f[q] * kscale - mm);
                } else {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        f[q] = kept(mb, q, ka, kc) ? __builtin_amdgcn_exp2f(f[q] * kscale - mm) : 0.0f;
                }
                s += tree_sum(f);
            }
            return;
        }
        m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int kc = kept_count(t, j, hv, k), ka = kept_from(t, j, hv, k);
            const auto mb = mask_of(j);
            float f[VEC];
            IO::unpack(raw[j], f);
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                e[j][q] = kept(mb, q, ka, kc) ? f[q] * kscale : -INFINITY;
                m = fmaxf(m, e[j][q]);
            }
        }
        s = 0.0f;
        const float mm = m == -INFINITY ? 0.0f : m;  // keeps 2^(-inf - mm) = 0 well defined
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int kc = kept_count(t, j, hv, k), ka = kept_from(t, j, hv, k);
            const auto mb = mask_of(j);
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                const float x = __builtin_amdgcn_exp2f(e[j][q] - mm);
                s += x;
                // LEAN explicit mask: a dropped element is marked by a negative e (no kept e
                // is negative, a NaN compares false), so the mask bytes need not stay live.
                if constexpr (MK == MK_MASK && LEAN) e[j][q] = kept(mb, q, ka, kc) ? x : -1.0f;
                else e[j][q] = x;
            }
        }
    }

    // This thread's partial sum rescaled to the group max M.
    __device__ __forceinline__ float sum_at(float M) const {
        return m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f(m - M);
    }

    // Scale of this thread's e once the group max M and sum S are known. A row whose kept
    // set turns out empty (an explicit mask row of zeros) has S = 0 and every m = -inf:
    // the gain is 0 and the row is written as zeros.
    __device__ __forceinline__ float gain(float M, float S) const {
        return m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M) / S;
    }

    // Writes slots 0..NA-1. The select keeps masked columns at +0 even when g is NaN (a
    // NaN among the kept scores).
    template <int SP>
    __device__ __forceinline__ void write(rsrc_t out, int t, int hv, const Cols& k,
                                          float g) const {
        constexpr int VEC = IO::VEC;
        if constexpr (RAW) {  // y = 2^(z - m) * g: the element's exponential again
            const Fresh f3 = fresh_pass(t, hv, k);
            float last = g;
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int sc = slot_class(t, j, hv, k);
                if (sc == kSlotEmpty) {
                    IO::template store<SP>(out, (t + j * STRIDE) * IO::BYTES, IO::zero());
                    continue;
                }
                float f[VEC];
                typename MIO::raw_t mb;
                int kc, ka;
                raw_slot(f3, j, last, f, mb, kc, ka);
                if (sc == kSlotFull) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q) f[q] = __builtin_amdgcn_exp2f(f[q] * kk - m) * g;
                } else {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        f[q] = kept(mb, q, ka, kc) ? __builtin_amdgcn_exp2f(f[q] * kk - m) * g : 0.0f;
                }
                last = f[VEC - 1];
                IO::template store<SP>(out, (t + j * STRIDE) * IO::BYTES, IO::pack(f));
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int kc = fresh_if<LEAN>(kept_count(t, j, hv, k)),
                      ka = fresh_if<LEAN>(kept_from(t, j, hv, k));
            const auto mb = mask_of(j);
            float f[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                if constexpr (MK == MK_MASK && LEAN) f[q] = e[j][q] < 0.0f ? 0.0f : e[j][q] * g;
                else f[q] = kept(mb, q, ka, kc) ? e[j][q] * g : 0.0f;
            }
            IO::template store<SP>(out, (t + j * STRIDE) * IO::BYTES, IO::pack(f));
        }
    }
};

// Calls f.operator()<NA>() with NA the smallest power of two (at most NV) that covers `na`
// live slots.
template <int NV, class F>
__device__ __forceinline__ void with_live_slots(int na, F&& f) {
    if (na <= 1) f.template operator()<1>();
    else if (NV >= 2 && na <= 2) f.template operator()<(NV >= 2 ? 2 : 1)>();
    else if (NV >= 4 && na <= 4) f.template operator()<(NV >= 4 ? 4 : 1)>();
    else if (NV >= 8 && na <= 8) f.template operator()<(NV >= 8 ? 8 : 1)>();
    else f.template operator()<NV>();
}

// --------------------------------------------------------------------------- fwd_wave
template <int DT, bool WIDE, int NV, int SP, int MK>
__device__ __forceinline__ void wave_row(const FwdArgs& a, uint32_t plane, int r, int L,
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
    const int nin = k.c1 / IO::VEC + 1;  // natural vectors holding columns 0..c1
    const rsrc_t in = make_rsrc(row_ptr(a.x, plane, r, a), (uint32_t)(nin * IO::BYTES));
    const rsrc_t min = MK == MK_MASK ? make_rsrc(mask_row(a, plane, r), (uint32_t)(nin * IO::VEC))
                                     : in;
    const IvRel iv = iv_layout<IO, MK>(a, sp, k, nin, out);
    const int hv = iv.shift;
    with_live_slots<NV>((iv.live + kWave - 1) / kWave, [&]<int NA>() {
        RowPart<IO, NA, kWave, MK, NV * IO::VEC >= kLeanElems, NA >= kRawNV> p;
        p.load(in, min, lane, hv, k);
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_outside<IO, SP>(sp, out, iv, lane, kWave);
        else write_zero_slots<IO, NA, NV, kWave, SP>(out, lane);
        p.compute(lane, hv, k, a.k);
        const float M = wave_reduce<OpMax>(p.m);
        const float S = wave_reduce<OpSum>(p.sum_at(M));
        p.template write<SP>(iv.out, lane, hv, k, p.gain(M, S));
    });
}

// WPB wavefronts per workgroup, each on its own unit (a row, or a row pair).
template <int DT, bool WIDE, int NV, int WPB, int SP, int MK>
__global__ __launch_bounds__(WPB * kWave) void fwd_wave(FwdArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = WPB == 1 ? 0u : (uint32_t)uniform(threadIdx.x / kWave);
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = (uint64_t)blk * WPB + wave; unit < a.n_units;
         unit += (uint64_t)nblk * WPB) {
        const Unit u = decode_unit<MK, false>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        wave_row<DT, WIDE, NV, SP, MK>(a, u.plane, u.r0, L, lane);
        if (u.r1 >= 0) wave_row<DT, WIDE, NV, SP, MK>(a, u.plane, u.r1, L, lane);
    }
}

// -------------------------------------------------------------------------- fwd_block
// Merge of per-wave partials (m_w, s_w), s_w = sum over the wave's kept elements of
// 2^(z - m_w): m = max_w m_w, s = sum_w s_w * 2^(m_w - m). A wave without kept elements has
// m_w = -inf and s_w = 0 and contributes nothing.
template <int W>
__device__ __forceinline__ void merge_partials(const float* pm, const float* ps, float& m,
                                               float& s) {
    if constexpr (W >= 8) {
        // lane w takes wave w's partial, and the merge is two wave reductions: two registers
        // instead of 2 * W (a lane of a 16-wavefront workgroup has 128 in all)
        const int lane = threadIdx.x & (kWave - 1);
        const float pw = lane < W ? pm[lane] : -INFINITY;
        const float sw = lane < W ? ps[lane] : 0.0f;
        m = wave_reduce<OpMax>(pw);
        s = wave_reduce<OpSum>(pw == -INFINITY ? 0.0f : sw * __builtin_amdgcn_exp2f(pw - m));
        return;
    }
    m = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) m = fmaxf(m, pm[w]);
    s = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
        s += pm[w] == -INFINITY ? 0.0f : ps[w] * __builtin_amdgcn_exp2f(pm[w] - m);
}

template <int DT, bool WIDE, int NV, int W, int SP, int MK>
__device__ __forceinline__ void block_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                          float* pm, float* ps) {
    using IO = Io<DT, WIDE>;
    constexpr int T = W * kWave;
    const int t = threadIdx.x;
    const Span sp = row_span<MK, IO::BYTES / IO::VEC>(a, plane, r, L);
    const rsrc_t out = make_rsrc(sp.out, sp.out_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {  // uniform over the workgroup
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_span<IO, SP>(sp, out, t, T);
        else write_zero_slots<IO, 0, NV, T, SP>(out, t);
        return;
    }
    const int wave = uniform(t / kWave);
    const int nin = k.c1 / IO::VEC + 1;
    const rsrc_t in = make_rsrc(row_ptr(a.x, plane, r, a), (uint32_t)(nin * IO::BYTES));
    const rsrc_t min = MK == MK_MASK ? make_rsrc(mask_row(a, plane, r), (uint32_t)(nin * IO::VEC))
                                     : in;
    const IvRel iv = iv_layout<IO, MK>(a, sp, k, nin, out);
    const int hv = iv.shift;
    with_live_slots<NV>((iv.live + T - 1) / T, [&]<int NA>() {
        RowPart<IO, NA, T, MK, NV * IO::VEC >= kLeanElems, NA >= kRawNV> p;
        p.load(in, min, t, hv, k);
        if (MK == MK_BAND && (a.flags & F_IVREL)) write_zeros_outside<IO, SP>(sp, out, iv, t, T);
        else write_zero_slots<IO, NA, NV, T, SP>(out, t);
        p.compute(t, hv, k, a.k);
        // wave partials, then the workgroup merge through LDS
        const float mw = wave_reduce<OpMax>(p.m);
        const float sw = mw == -INFINITY ? 0.0f : wave_reduce<OpSum>(p.sum_at(mw));
        if ((t & (kWave - 1)) == 0) {
            pm[wave] = mw;
            ps[wave] = sw;
        }
        __syncthreads();
        float M, S;
        merge_partials<W>(pm, ps, M, S);
        p.template write<SP>(iv.out, t, hv, k, p.gain(M, S));
    });
}

template <int DT, bool WIDE, int NV, int W, int SP, int MK>
__global__ __launch_bounds__(W * kWave) void fwd_block(FwdArgs a) {
    __shared__ float part[2][2][W];  // [row of the unit][max, sum][wave]
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = blk; unit < a.n_units; unit += nblk) {
        const Unit u = decode_unit<MK, (W >= 8)>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        block_row<DT, WIDE, NV, W, SP, MK>(a, u.plane, u.r0, L, part[0][0], part[0][1]);
        if (u.r1 >= 0)
            block_row<DT, WIDE, NV, W, SP, MK>(a, u.plane, u.r1, L, part[1][0], part[1][1]);
        __syncthreads();  // the next unit rewrites the partials
    }
}

// ------------------------------------------------------------------------- fwd_stream
// Two passes over a row of any length. Pass 1 keeps a running (m, s) per thread, updated
// per vector: m' = max(m, max of the vector), s' = s * 2^(m - m') + sum 2^(z - m'); the
// wave and workgroup merges follow the same rule. Pass 2 re-reads the interval and writes
// 2^(z - m) / s. The zeros outside the interval are written first: they need no data.
template <int DT, bool WIDE, int W, int SP, int MK>
__device__ __forceinline__ void stream_row(const FwdArgs& a, uint32_t plane, int r, int L,
                                           float* pm, float* ps) {
    using IO = Io<DT, WIDE>;
    using MIO = MaskIo<IO::VEC>;
    constexpr int VEC = IO::VEC;
    constexpr int T = W * kWave;
    const int t = threadIdx.x;
    const int nraw = a.row_bytes / IO::BYTES;
    const rsrc_t out = make_rsrc(row_ptr(a.y, plane, r, a), (uint32_t)a.row_bytes);
    const Cols k = kept_cols<MK>(a, r, L);
    if (k.empty()) {
        for (int v = t; v < nraw; v += T)
            IO::template store<SP>(out, v * IO::BYTES, IO::zero());
        return;
    }
    const int wave = uniform(t / kWave);
    const int v0 = k.c0 / VEC, nin = k.c1 / VEC + 1;
    const rsrc_t in = make_rsrc(row_ptr(a.x, plane, r, a), (uint32_t)(nin * IO::BYTES));
    const rsrc_t min = MK == MK_MASK ? make_rsrc(mask_row(a, plane, r), (uint32_t)(nin * VEC))
                                     : in;
    for (int v = t; v < v0; v += T) IO::template store<SP>(out, v * IO::BYTES, IO::zero());
    for (int v = nin + t; v < nraw; v += T)
        IO::template store<SP>(out, v * IO::BYTES, IO::zero());
    auto kept = [&](int v, int e, const typename MIO::raw_t& mb) {
        const int c = v * VEC + e;
        bool r = c >= k.c0 && c <= k.c1;
        if constexpr (MK == MK_MASK) r = r && MIO::kept(mb, e);
        return r;
    };
    float m = -INFINITY, s = 0.0f;
    for (int v = v0 + t; v < nin; v += T) {
        float f[VEC];
        IO::unpack(IO::template load<kPolicyDefault>(in, v * IO::BYTES), f);
        typename MIO::raw_t mb{};
        if constexpr (MK == MK_MASK) mb = MIO::load(min, v * VEC);
        float vm = -INFINITY;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (kept(v, e, mb)) vm = fmaxf(vm, f[e] * a.k);
        const float mn = fmaxf(m, vm);
        float add = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            add += kept(v, e, mb) ? __builtin_amdgcn_exp2f(f[e] * a.k - mn) : 0.0f;
        s = (mn == -INFINITY ? 0.0f : (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f(m - mn)) + add);
        m = mn;
    }
    const float mw = wave_reduce<OpMax>(m);
    const float sw =
        wave_reduce<OpSum>(m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f(m - mw));
    if ((t & (kWave - 1)) == 0) {
        pm[wave] = mw;
        ps[wave] = sw;
    }
    __syncthreads();
    float mt, st;
    merge_partials<W>(pm, ps, mt, st);
    const float inv = mt == -INFINITY ? 0.0f : 1.0f / st;  // an explicit mask row of zeros
    for (int v = v0 + t; v < nin; v += T) {
        float f[VEC];
        IO::unpack(IO::template load<kPolicyDefault>(in, v * IO::BYTES), f);
        typename MIO::raw_t mb{};
        if constexpr (MK == MK_MASK) mb = MIO::load(min, v * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            f[e] = kept(v, e, mb) ? __builtin_amdgcn_exp2f(f[e] * a.k - mt) * inv : 0.0f;
        IO::template store<SP>(out, v * IO::BYTES, IO::pack(f));
    }
}

template <int DT, bool WIDE, int W, int SP, int MK>
__global__ __launch_bounds__(W * kWave) void fwd_stream(FwdArgs a) {
    __shared__ float part[2][2][W];
    const uint32_t nblk = gridDim.x;
    const uint32_t blk = (a.flags & F_XCD) ? xcd_chunked(blockIdx.x, nblk, a.xcd_shift) : blockIdx.x;
    for (uint64_t unit = blk; unit < a.n_units; unit += nblk) {
        const Unit u = decode_unit<MK, true>((uint32_t)unit, a);
        const int L = valid_len<MK>(a, u.plane);
        stream_row<DT, WIDE, W, SP, MK>(a, u.plane, u.r0, L, part[0][0], part[0][1]);
        if (u.r1 >= 0) stream_row<DT, WIDE, W, SP, MK>(a, u.plane, u.r1, L, part[1][0], part[1][1]);
        __syncthreads();
    }
}

}  // namespace gtms
