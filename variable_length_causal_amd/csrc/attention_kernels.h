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
// Key blocks of 32 are staged in LDS (K row-major, V transposed) by the whole workgroup.
// Per block each wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (D/16
// instructions; Q stays in registers as the B operand), so a lane holds 16 scores of ITS OWN
// row: the row max and the rescaling are lane-local plus one exchange with lane l ^ 32. The
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
};

constexpr int kAttnRows = 128;  // query rows per workgroup (4 wavefronts x 32)
constexpr int kAttnKeys = 32;   // keys per block

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

template <int DT, int D>
__global__ __launch_bounds__(256) void attn_fwd(AttnArgs a) {
    using MF = Mfma16<DT>;
    using vec8 = typename MF::vec8;
    using elem_t = typename MF::elem_t;
    typedef elem_t vec4 __attribute__((ext_vector_type(4)));
    constexpr int KP = D + 8;              // K row pitch in LDS (elements)
    constexpr int VP = kAttnKeys + 4;      // V^T row pitch in LDS (elements)
    constexpr int NT = D / 32;             // 32-wide output tiles per row
    __shared__ __attribute__((aligned(16))) elem_t k_lds[kAttnKeys * KP];
    __shared__ __attribute__((aligned(16))) elem_t vt_lds[D * VP];

    // tiles with the most key blocks first: tile index descends with blockIdx
    const uint32_t plane = blockIdx.x % a.n_planes;
    const int qt = a.n_tiles - 1 - (int)(blockIdx.x / a.n_planes);
    const int q0 = qt * kAttnRows;
    const int L = clamp_len(a.seq_lens[plane / a.M], a.S);
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6), g = lane >> 5;
    const uint64_t head = (uint64_t)plane * (uint64_t)a.S * D;  // first element of the head
    const uint32_t head_bytes = (uint32_t)((uint64_t)a.S * D * 2);
    const rsrc_t out = make_rsrc((const char*)a.o + head * 2, head_bytes);

    // rows q0 .. q0+127 that lie at or past L are zeros (all of them when q0 >= L)
    {
        const int z0 = max(q0, L), z1 = min(q0 + kAttnRows, a.S);
        for (int i = tid; i < (z1 - z0) * (D / 8); i += 256) {
            const int r = z0 + i / (D / 8), c = (i % (D / 8)) * 8;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, out, (r * D + c) * 2, 0,
                                                   kPolicyStream);
        }
    }
    if (q0 >= L) return;

    const int row = q0 + wave * 32 + (lane & 31);   // this lane's query row
    const int kv_end = min(q0 + kAttnRows, L);       // keys the workgroup needs
    const int wave_end = min(q0 + wave * 32 + 32, L);  // keys this wavefront needs

    // Q^T as the B operand: lane l holds Q[row][16*kk + 8*g + j]
    const rsrc_t qin = make_rsrc((const char*)a.q + head * 2, head_bytes);
    vec8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(vec8, __builtin_amdgcn_raw_buffer_load_b128(
                                              qin, (row * D + 16 * kk + 8 * g) * 2, 0, 0));
    // K and V of this head, keys < L only (the range check zero-fills keys past L, so the
    // masked probabilities meet finite values)
    const uint32_t kv_bytes = (uint32_t)((uint64_t)L * D * 2);
    const rsrc_t kin = make_rsrc((const char*)a.k + head * 2, kv_bytes);
    const rsrc_t vin = make_rsrc((const char*)a.v + head * 2, kv_bytes);

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float m_run = -INFINITY, l_part = 0.0f;

    for (int kb = 0; kb < kv_end; kb += kAttnKeys) {
        // stage the block: K row-major, V transposed (vt[d][key])
        __syncthreads();  // the previous block's readers are done
#pragma unroll
        for (int i = tid; i < kAttnKeys * (D / 8); i += 256) {
            const int key = i / (D / 8), c = (i % (D / 8)) * 8;
            const int off = ((kb + key) * D + c) * 2;
            const u32x4 kw = __builtin_amdgcn_raw_buffer_load_b128(kin, off, 0, 0);
            const u32x4 vw = __builtin_amdgcn_raw_buffer_load_b128(vin, off, 0, 0);
            *(u32x4*)&k_lds[key * KP + c] = kw;
            const vec8 vv = __builtin_bit_cast(vec8, vw);
#pragma unroll
            for (int j = 0; j < 8; ++j) vt_lds[(c + j) * VP + key] = vv[j];
        }
        __syncthreads();
        if (kb >= wave_end) continue;  // this wavefront's rows need no key of the block

        // S^T[key][row] for the 32 keys of the block
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const vec8 kf = *(const vec8*)&k_lds[(lane & 31) * KP + 16 * kk + 8 * g];
            s = MF::mfma(kf, qf[kk], s);
        }
        // mask, scale, block max of the row
        float z[16];
        float mb = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kb + 8 * (e / 4) + 4 * g + (e & 3);
            z[e] = (key <= row && key < L) ? s[e] * a.k2 : -INFINITY;
            mb = fmaxf(mb, z[e]);
        }
        mb = fmaxf(mb, swap_halves(mb));
        const float m_new = fmaxf(m_run, mb);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        // probabilities, rounded to the element type for the second product
        vec8 p[2];
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float pe = __builtin_amdgcn_exp2f(z[e] - m_use);
            ps += pe;
            p[e / 8][e % 8] = (elem_t)pe;
        }
        l_part = l_part * alpha + ps;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
        // O^T[d][row] += V^T[d][keys] P^T[keys][row]; half h covers the lane's e = 8h..8h+7,
        // that is keys 16h + 8*(j/4) + 4*g + j%4 for j = 0..7
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const elem_t* vr = &vt_lds[(32 * t + (lane & 31)) * VP + 16 * h + 4 * g];
                const vec4 v0 = *(const vec4*)vr, v1 = *(const vec4*)(vr + 8);
                const vec8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[t] = MF::mfma(vf, p[h], acc[t]);
            }
        }
    }

    // normalise and store the rows below L (acc[t] register e: d = 32t + 8*(e/4) + 4g + e%4)
    const float l_row = l_part + swap_halves(l_part);
    if (row < L) {
        const float inv = 1.0f / l_row;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                vec4 o4;
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = (elem_t)(acc[t][4 * q + i] * inv);
                const int d = 32 * t + 8 * q + 4 * g;
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), out,
                                                      (row * D + d) * 2, 0, kPolicyStream);
            }
        }
    }
}

}  // namespace gtms
