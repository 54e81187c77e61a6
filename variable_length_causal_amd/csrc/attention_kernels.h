// Attention with the grouped tril mask, fused (gfx950): O = softmax_mask(scale * Q K^T) V.
//
// The self-attention article ("ops(8) self-attention CUDA") computes attention in three
// steps: scores, a softmax of each score row, and the weighted sum of values. Here the
// softmax is the grouped tril mask softmax: for plane p = b*M + m of Q, K, V, O [B, M, S, D]
// (16-bit elements, row-major) with valid length L = clamp(seq_lens[b], 0, S), query row
// r < L attends to the keys c <= r, and a row r >= L is all zeros. Nothing of the S x S
// score matrix reaches memory: the steps run tile by tile with an online (max, sum), the
// split merge of ColossalAI's flash_decoding.py (_flash_decoding_fwd_reduce_kernel) applied
// to consecutive key blocks.
//
// Work: one workgroup of 4 wavefronts per (plane, tile of 128 query rows); wavefront w owns
// rows q0 + 32w .. q0 + 32w + 31, one row per lane pair (lanes l and l + 32 hold row l % 32).
// Key blocks of 64 are staged in LDS (K row-major, V transposed) by the whole workgroup; the
// next block's K and V are loaded into registers while the current one computes. Per
// 32-key tile each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (D/16
// instructions; Q stays in registers as the B operand), so a lane holds 16 scores of ITS OWN
// row: the row max and the rescaling are lane-local plus one exchange with lane l ^ 32.
// Blocks wholly below the wavefront's diagonal and the length skip the mask. The
// probabilities P are rounded to the element type and used, in the registers they were
// computed in, as the B operand of O^T += V^T P^T (2 * D/32 instructions); the A operand
// V^T is read from LDS in the key order the score layout implies (keys are a contraction
// index, so any order shared by both operands gives the same sum).
//
// MFMA lane layout of the 32x32x16 16-bit instructions (checked on MI355X): A lane l holds
// A[l % 32][8*(l/32) + j], B lane l holds B[8*(l/32) + j][l % 32], j = 0..7, and the
// accumulator register e of lane l holds C[8*(e/4) + 4*(l/32) + e%4][l % 32].
#pragma once

#include "device_common.h"

namespace gtms {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const int32_t* seq_lens;
    uint32_t n_planes;  // B * M
    uint32_t M;
    int S;
    int n_tiles;        // ceil(S / kAttnRows)
    float k2;           // scale * log2(e)
    int tile_major;     // block order (see attn_fwd)
};

constexpr int kAttnRows = 128;  // query rows per workgroup (4 wavefronts x 32)
// The accumulators stay scaled to a row's reference max m until a block's max exceeds m by
// more than this (log2 domain) on a block that takes the exact path: the rescale then runs only
// on the few blocks that raise some row's max that far.
constexpr float kAttnSlack = 8.0f;
// Blocks after a group's first skip the max: their probabilities, formed against the current
// reference, are kept when each lane's sum of them is at most this, so every probability is
// at most 2^15, inside binary16's range (65504). Larger sums take the exact path. After an
// exact block the reference trails the max by at most kAttnSlack, so a lane's 32 probabilities
// sum to at most 2^13 and rising maxima keep the fast path for several blocks.
constexpr float kAttnSumMax = 32768.0f;
// keys per block: 64 for head size 64, 32 for 128 (keeps two workgroups' registers per SIMD)
template <int D> constexpr int kAttnKeys = D <= 64 ? 64 : 32;

template <int DT> struct Mfma16;
template <> struct Mfma16<DT_BF16> {
    using elem_t = __bf16;
    typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma16<DT_F16> {
    using elem_t = _Float16;
    typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Exchange with lane l ^ 32 (the other half of the wavefront holds the same rows).
__device__ __forceinline__ float swap_halves(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
        (int)((threadIdx.x ^ 32) & 63) * 4, __builtin_bit_cast(int, v)));
}

// SPLIT = 2 (head size 64): the workgroup has two groups of 4 wavefronts on the same 128 query
// rows; group 0 takes the tile's first floor(n/2) key blocks, group 1 the rest (the diagonal
// blocks included). Each group keeps its own online (max, sum) and accumulators over its keys,
// and group 0 merges group 1's partials through LDS at the end by the split-KV reduction of
// flash_decoding.py (_flash_decoding_fwd_reduce_kernel): m = max(m0, m1), l = sum_i l_i 2^(m_i - m),
// O = sum_i O_i 2^(m_i - m). A tile's chain of key blocks, which sets the launch's length when
// there are few tiles per CU, is then half as long.
template <int DT, int D, int SPLIT>
__global__ __launch_bounds__(256 * SPLIT) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : 2))) void attn_fwd(AttnArgs a) {
    using MF = Mfma16<DT>;
    using vec8 = typename MF::vec8;
    using elem_t = typename MF::elem_t;
    typedef elem_t vec4 __attribute__((ext_vector_type(4)));
    typedef elem_t vec2 __attribute__((ext_vector_type(2)));
    constexpr int BN = kAttnKeys<D>;       // keys per block
    constexpr int KP = D + 8;              // K row pitch in LDS (elements)
    constexpr int VP = BN + 8;             // V^T row pitch in LDS (elements, 16-byte rows)
    constexpr int NT = D / 32;             // 32-wide output tiles per row
    constexpr int CPR = D / 8;             // 16-byte chunks per K or V row
    constexpr int KCH = BN * CPR / 256;    // K chunks per thread per block
    constexpr int VCH = BN / 2 * CPR / 256;  // V key pairs (two chunks) per thread per block
    static_assert(KCH >= 1 && VCH >= 1 && BN % 32 == 0, "block shape");
    static_assert(SPLIT == 1 || (SPLIT == 2 && D == 64), "key split at head size 64 only");
    // two buffers: block i computes from buffer i % 2 while block i + 1 is written into the
    // other one
    __shared__ __attribute__((aligned(16))) elem_t k_lds_all[SPLIT][2][BN * KP];
    __shared__ __attribute__((aligned(16))) elem_t vt_lds_all[SPLIT][2][D * VP];

    // Block order, chosen by the host:
    //  - tile-major: the last tile of every plane first, then the one before, and so on, so
    //    the longest tiles start first and none waits behind whole planes. With a multiple of
    //    8 planes, block i runs on XCD i % 8 and each plane stays on one XCD;
    //  - plane-major: all the tiles of one plane run on one XCD, one after the other, longest
    //    first; its L2 then holds the plane's K and V once for all of them.
    // Tile-major re-reads a plane's K and V after a sweep over all planes, which costs HBM
    // bandwidth once they no longer fit in the memory-side cache and the tiles run fast.
    const uint32_t nt = (uint32_t)a.n_tiles;
    uint32_t plane;
    int qt;
    if (a.tile_major) {
        const uint32_t rank = blockIdx.x / a.n_planes;
        plane = blockIdx.x - rank * a.n_planes;
        qt = (int)(nt - 1 - rank);
    } else {
        const uint32_t lb = xcd_grouped(blockIdx.x, gridDim.x, nt);
        plane = lb / nt;
        qt = (int)(nt - 1 - lb % nt);
    }
    const int q0 = qt * kAttnRows;
    const int L = clamp_len(a.seq_lens[plane / a.M], a.S);
    // grp: the key group (0 unless SPLIT = 2); tid: the thread within its group
    const int grp = SPLIT == 1 ? 0 : uniform((int)threadIdx.x >> 8);
    const int tid = threadIdx.x & 255, lane = tid & 63, wave = uniform(tid >> 6), g = lane >> 5;
    auto& k_lds = k_lds_all[grp];
    auto& vt_lds = vt_lds_all[grp];
    const uint64_t head = (uint64_t)plane * (uint64_t)a.S * D;  // first element of the head
    const uint32_t head_bytes = (uint32_t)((uint64_t)a.S * D * 2);
    const rsrc_t out = make_rsrc((const char*)a.o + head * 2, head_bytes);

    // rows q0 .. q0+127 that lie at or past L are zeros (all of them when q0 >= L)
    {
        const int z0 = max(q0, L), z1 = min(q0 + kAttnRows, a.S);
        for (int i = (int)threadIdx.x; i < (z1 - z0) * CPR; i += 256 * SPLIT) {
            const int r = z0 + i / CPR, c = (i % CPR) * 8;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, out, (r * D + c) * 2, 0,
                                                   kPolicyNt);
        }
    }
    if (q0 >= L) return;

    const int row = q0 + wave * 32 + (lane & 31);      // this lane's query row
    const int row_lo = q0 + wave * 32;                 // the wavefront's first row
    const int kv_end = min(q0 + kAttnRows, L);         // keys the workgroup needs

    // Q^T as the B operand: lane l holds Q[row][16*kk + 8*g + j]
    const rsrc_t qin = make_rsrc((const char*)a.q + head * 2, head_bytes);
    // A negative scale is applied as |scale| to -Q (a sign-bit flip, exact), so that the
    // row max is always the max of the raw scores. A scale of +-0 (or one whose k2 is below
    // the smallest normal float) makes every kept score 0, so that softmax is uniform over
    // the kept keys: Q is zeroed and k2 set to 1. Masked keys (score -inf) then still meet
    // a positive factor, where -inf * 0 would give NaN.
    const bool zero_scale = fabsf(a.k2) < __FLT_MIN__;
    const uint32_t qsign = a.k2 < 0.0f ? 0x80008000u : 0u;
    const uint32_t qkeep = zero_scale ? 0u : 0xffffffffu;
    const float k2 = zero_scale ? 1.0f : fabsf(a.k2);
    vec8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(
            vec8, (__builtin_amdgcn_raw_buffer_load_b128(qin, (row * D + 16 * kk + 8 * g) * 2, 0, 0) ^
                   qsign) & qkeep);
    // K and V of this head, keys < L only (the range check zero-fills keys past L, so the
    // masked probabilities meet finite values)
    const uint32_t kv_bytes = (uint32_t)((uint64_t)L * D * 2);
    const rsrc_t kin = make_rsrc((const char*)a.k + head * 2, kv_bytes);
    const rsrc_t vin = make_rsrc((const char*)a.v + head * 2, kv_bytes);

    // the next block's K chunks and V key pairs, held in registers while a block computes
    u32x4 kr[KCH], vr[VCH][2];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int n = 0; n < KCH; ++n) {
            const int i = tid + 256 * n, key = i / CPR, c = (i % CPR) * 8;
            kr[n] = __builtin_amdgcn_raw_buffer_load_b128(kin, ((kb + key) * D + c) * 2, 0, 0);
        }
#pragma unroll
        for (int n = 0; n < VCH; ++n) {
            const int i = tid + 256 * n, key = 2 * (i % (BN / 2)), c = (i / (BN / 2)) * 8;
            vr[n][0] = __builtin_amdgcn_raw_buffer_load_b128(vin, ((kb + key) * D + c) * 2, 0, 0);
            vr[n][1] = __builtin_amdgcn_raw_buffer_load_b128(vin, ((kb + key + 1) * D + c) * 2, 0, 0);
        }
    };
    // K row-major; V transposed, two keys per 4-byte write: consecutive lanes take
    // consecutive key pairs of one 8-column chunk, so that a write instruction covers whole
    // LDS rows (no bank conflicts). Within each group of 16 keys the
    // key 16h + 8a + 4b + i sits at column 16h + 8b + 4a + i, so that the 8 keys one lane
    // needs for a product (b = its half of the wavefront, a = 0, 1) are one 16-byte read.
    auto vcol = [](int key) { return (key & ~12) | ((key & 8) >> 1) | ((key & 4) << 1); };
    auto stage = [&](int buf) {
#pragma unroll
        for (int n = 0; n < KCH; ++n) {
            const int i = tid + 256 * n, key = i / CPR, c = (i % CPR) * 8;
            *(u32x4*)&k_lds[buf][key * KP + c] = kr[n];
        }
#pragma unroll
        for (int n = 0; n < VCH; ++n) {
            const int i = tid + 256 * n, key = 2 * (i % (BN / 2)), c = (i / (BN / 2)) * 8;
            const vec8 v0 = __builtin_bit_cast(vec8, vr[n][0]);
            const vec8 v1 = __builtin_bit_cast(vec8, vr[n][1]);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *(vec2*)&vt_lds[buf][(c + j) * VP + vcol(key)] = vec2{v0[j], v1[j]};
        }
    };

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float m_run = -INFINITY, l_part = 0.0f;

    // The group's key blocks [k_begin, k_end): all of [0, kv_end) unless SPLIT = 2, where
    // group 0 takes the first nb0 = floor(nb / 2) blocks and group 1 the others.
    const int nb = (kv_end + BN - 1) / BN, nb0 = SPLIT == 1 ? 0 : nb / 2;
    const int k_begin = grp == 0 ? 0 : nb0 * BN;
    const int k_end = SPLIT == 2 && grp == 0 ? nb0 * BN : kv_end;

    // Pipeline: global loads run two blocks ahead of the computation, LDS writes one block
    // ahead; one barrier per block separates the writes of a buffer from its readers.
    if (k_begin < k_end) {
        fetch(k_begin);
        stage(0);
        if (k_begin + BN < k_end) fetch(k_begin + BN);
    }
    __syncthreads();
    for (int kb = k_begin, buf = 0; kb < k_end; kb += BN, buf ^= 1) {
        {  // a wavefront whose rows need no key of the block computes it masked

        // S^T[key][row] for the 32-key tiles of the block that this wavefront needs
        constexpr int NS = BN / 32;
        f32x16 s[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            s[st] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const vec8 kf =
                    *(const vec8*)&k_lds[buf][(32 * st + (lane & 31)) * KP + 16 * kk + 8 * g];
                s[st] = MF::mfma(kf, qf[kk], s[st]);
            }
        }
        // z = s * k2 (k2 = |scale| * log2 e >= 0). The row max is taken on the raw scores,
        // so that each probability costs one fma and one exp: p = 2^(s*k2 - m). Masked keys
        // (only in blocks that reach the wavefront's diagonal or the length) get s = -inf.
        if (!(kb + BN - 1 <= row_lo && kb + BN <= L)) {  // uniform over the wavefront
            // key = kb + 4g + (32st + 8(e/4) + e%4) is kept when key <= min(row, L - 1)
            const int lim = min(row, L - 1) - kb - 4 * g;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s[st][e] = 32 * st + 8 * (e / 4) + (e & 3) <= lim ? s[st][e] : -INFINITY;
            }
        }
        // Probabilities p = 2^(s*k2 - m) against the row's reference m (log2 domain), rounded
        // to the element type for the second product. Softmax does not depend on the
        // reference, so it changes rounding only.
        vec8 p[2 * NS];
        float ps = 0.0f;
        auto probs = [&]() {
            const float m_use = m_run == -INFINITY ? 0.0f : m_run;
            ps = 0.0f;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], k2, -m_use));
                    ps += pe;
                    p[2 * st + e / 8][e % 8] = (elem_t)pe;
                }
            }
        };
        // Fast path, every block after the group's first: no max. The probabilities are
        // formed against the current reference and kept when every lane's sum, which bounds
        // its probabilities, is at most kAttnSumMax (a NaN or infinite sum fails the test).
        // Otherwise, and on the group's first block, where the rows have no reference yet,
        // the exact path: the block's max moves the reference when some row gains more than
        // kAttnSlack, and the probabilities are formed again.
        bool exact = kb == k_begin;
        if (!exact) {
            probs();
            exact = __builtin_amdgcn_ballot_w64(!(ps <= kAttnSumMax)) != 0;
        }
        if (exact) {
            // this lane's half of the row: max over its 8 keys per 32-key tile
            float mh = -INFINITY;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
#pragma unroll
                for (int e = 0; e < 16; ++e) mh = fmaxf(mh, s[st][e]);
            }
            // The reference moves to the running max m' = max over kept keys of s * k2 only
            // when some row of the wavefront gains more than kAttnSlack (a wave-uniform
            // branch); the sums are then rescaled by 2^(m - m'), and every probability stays
            // below 2^kAttnSlack. A row's max exceeds the bound exactly when one of its two
            // halves does (m_run is the same on both lanes of a row, and k2 >= 0), so the
            // wave-wide test runs on the halves and the exchange with lane l ^ 32 that gives
            // the row max happens only inside the branch.
            const float mkh = mh == -INFINITY ? -INFINITY : mh * k2;
            if (__builtin_amdgcn_ballot_w64(mkh > m_run + kAttnSlack) != 0) {
                const float mb = fmaxf(mh, swap_halves(mh));
                const float mk = mb == -INFINITY ? -INFINITY : mb * k2;
                const float m_new = fmaxf(m_run, mk);
                const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_part *= alpha;
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] *= alpha;
            }
            probs();
        }
        l_part += ps;
        // O^T[d][row] += V^T[d][keys] P^T[keys][row]; vector 2*st + h covers the lane's keys
        // kb + 32*st + 16h + 8*(j/4) + 4*g + j%4, j = 0..7
#pragma unroll
        for (int st = 0; st < NS; ++st) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    // keys 32st + 16h + 8*(j/4) + 4g + j%4 sit at columns 32st + 16h + 8g + j
                    const vec8 vf = *(const vec8*)&vt_lds[buf][(32 * t + (lane & 31)) * VP +
                                                               32 * st + 16 * h + 8 * g];
                    acc[t] = MF::mfma(vf, p[2 * st + h], acc[t]);
                }
            }
        }
        }
        // the next block into the other buffer (its readers finished before the last
        // barrier), then the loads of the block after it
        if (kb + BN < k_end) {
            stage(buf ^ 1);
            if (kb + 2 * BN < k_end) fetch(kb + 2 * BN);
        }
        __syncthreads();
    }
    if constexpr (SPLIT == 2) {
        // Group 0 has nb0 blocks, group 1 nb - nb0 (at most one more): the barrier count of
        // group 0 is made up here (a barrier waits for every wavefront's arrival, wherever
        // in the code it is).
        if (grp == 0 && nb - nb0 > nb0) __syncthreads();
        // Group 1's partials go through the K buffers (free since the last barrier: their
        // last reads came before it), 34 floats per lane laid out [wave][value][lane].
        float* part = reinterpret_cast<float*>(&k_lds_all[0][0][0]) + wave * 34 * 64 + lane;
        static_assert(4 * 34 * 64 * 4 <= sizeof(k_lds_all), "merge area");
        if (grp == 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
#pragma unroll
                for (int e = 0; e < 16; ++e) part[(16 * t + e) * 64] = acc[t][e];
            }
            part[32 * 64] = m_run;
            part[33 * 64] = l_part;
        }
        __syncthreads();
        if (grp == 1) return;
        // m_run is a row's reference in the log2 domain (equal on both lanes of the row, in
        // each group); the partials are sums relative to 2^m_run
        const float m1 = part[32 * 64], l1 = part[33 * 64];
        const float m = fmaxf(m_run, m1);
        const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
        const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
        l_part = l_part * a0 + l1 * a1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = acc[t][e] * a0 + part[(16 * t + e) * 64] * a1;
        }
    }

    // Normalise and store the rows below L (acc[t] register e: d = 32t + 8*(e/4) + 4g + e%4).
    // A lane holds 4-element pieces of its row, so stores straight from the accumulators
    // would fill each 128-byte line in eight partial writes. Each wavefront therefore stages
    // its 32 rows, 64 columns at a time, in the V^T buffer (free since the loop's last
    // barrier) and reads them back as 16-byte row chunks: every store instruction then
    // writes 8 whole rows of 64 columns. Only this wavefront touches its staging rows, so a
    // fence (no barrier) orders its LDS writes before its reads and its reads before the next
    // pass's writes.
    constexpr int OP = 64 + 8;  // staging row pitch (elements)
    static_assert(4 * 32 * OP <= 2 * D * VP, "staging area");
    const float l_row = l_part + swap_halves(l_part);
    const float inv = row < L ? 1.0f / l_row : 0.0f;
    elem_t* obuf = reinterpret_cast<elem_t*>(vt_lds) + wave * 32 * OP;
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += 2) {
#pragma unroll
        for (int t = t0; t < t0 + 2; ++t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                vec4 o4;
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = (elem_t)(acc[t][4 * q + i] * inv);
                *(vec4*)&obuf[(lane & 31) * OP + 32 * (t - t0) + 8 * q + 4 * g] = o4;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        u32x4 val[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            val[i] = *(const u32x4*)&obuf[(8 * i + (lane >> 3)) * OP + 8 * (lane & 7)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // rows at or past L keep the zeros written above: their stores get an offset that
            // the buffer range check drops
            const int grow = row_lo + 8 * i + (lane >> 3);
            __builtin_amdgcn_raw_buffer_store_b128(
                val[i], out, grow < L ? (grow * D + 32 * t0 + 8 * (lane & 7)) * 2 : (int)0x80000000,
                0, kPolicyNt);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    }
}

}  // namespace gtms
