// Flash attention forward on bf16 MFMA (gfx950) with 3D RoPE fused into the Q and K loads.
//
// What it computes: for every query row n of a sequence, out[n] = sum_j softmax_j(q~_n . k~_j /
// sqrt(128)) v_j over the sequence's key rows j, where q~ and k~ are q and k turned by the 3D
// rotation of their own (t, h, w) ("A video model's architecture: spatiotemporal attention and
// the 3D VAE", self-test answers 2 and 4; "CogVideoX Architecture: ...", section "3. 3D Rotary
// Position Embeddings (3D RoPE)").  A sequence is all N rows (full 3D attention) or the H*W rows
// of one frame (the spatial stage of factorised attention, "How attention sees time").
//
// Design (one workgroup = 8 waves = 256 query rows of one head and one sequence):
//  * Scores are formed transposed, S^T = K~ Q~^T, with v_mfma_f32_32x32x16_bf16: a lane then owns
//    one query column and 16 keys per 32x32 block, so the softmax row max and row sum are
//    in-lane except for one exchange between the two 32-lane halves.
//  * Q~ stays in registers as the B operand (rotated once at load).  K~ tiles of 64 keys are
//    rotated while being copied global -> registers -> LDS; V tiles are transposed on the same
//    copy, so both MFMA A operands are single 16-byte LDS reads.
//  * P^T leaves the score accumulator already in the B-operand layout of the PV product; the V^T
//    tile in LDS stores keys in the matching order (within each 16 keys: 0-3, 8-11, 4-7, 12-15).
//  * Double-buffered LDS: the global loads of tile j+1 are issued before tile j's MFMAs and
//    written to the other buffer after them; one barrier per tile.
//  * Online softmax in fp32 with exp2 and the log2(e)/sqrt(d) factor folded into one FMA.
#include "st_internal.h"

namespace st {
namespace {

constexpr int D = 128;          // head dimension (bf16 path)
constexpr int BM = 256;         // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 512;   // 8 waves
constexpr int KS = 136;         // K tile row stride in LDS (bf16): 272 B, rows start 4 banks apart
constexpr int VS = 72;          // V^T tile row stride in LDS (bf16): 144 B

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    const float2* table;
    RopeGeom g;
    int heads;
    int seg_len;
    int n_segs;
    int q_tiles;
    int total_wg;
    float scale_log2;  // log2(e) / sqrt(D)
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Rotate 8 channels (a 16-byte chunk starting at pair 4*c) of a row at (t, h, w).
__device__ __forceinline__ uint4 rope_chunk(uint4 raw, int c, int t, int h, int w, bool text,
                                            const RopeGeom& g, const float2* __restrict__ table) {
    uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float2 cs = table[pair_entry(4 * c + i, t, h, w, text, g)];
        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
        rotate_pair(x0, x1, cs);
        wd[i] = pack_bf16x2(x0, x1);
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

__device__ __forceinline__ uint32_t half16(uint2 v, int e) {
    uint32_t w = (e < 2) ? v.x : v.y;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__global__ void __launch_bounds__(NTHREADS, 1) attn_fwd_bf16_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][D * VS];

    const int logical = xcd_remap(blockIdx.x, p.total_wg);
    const int qt = logical % p.q_tiles;
    const int rest = logical / p.q_tiles;
    const int seg = rest % p.n_segs;
    const int head = rest / p.n_segs;
    const int seg_base = seg * p.seg_len;
    const int seg_len = p.seg_len;
    const long long row_stride = (long long)p.heads * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const uint16_t* __restrict__ kbase = p.k + (long long)head * D;
    const uint16_t* __restrict__ vbase = p.v + (long long)head * D;
    const RopeGeom& g = p.g;

    // ---- loader geometry -------------------------------------------------------------------
    // K: thread owns 16-byte chunk kc (channels 8kc..8kc+7) of tile rows kr0 and kr0 + 32.
    const int kc = tid & 15;
    const int kr0 = tid >> 4;
    // V: thread owns channels 4vd..4vd+3 of keys 4vg..4vg+3, written transposed.
    const int vd = tid & 31;
    const int vg = tid >> 5;
    const int vsb = vg & 3;
    const int vpos = 16 * (vg >> 2) + ((vsb & 1) << 3) + ((vsb >> 1) << 2);

    const int ntiles = (seg_len + BN - 1) / BN;

    uint4 kraw[2];
    uint2 vraw[4];

    auto load_tile = [&](int j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int kl = j * BN + kr0 + 32 * i;
            kraw[i] = kl < seg_len ? ld16(kbase + (seg_base + kl) * row_stride + 8 * kc)
                                   : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int kl = j * BN + 4 * vg + r;
            vraw[r] = kl < seg_len ? ld8(vbase + (seg_base + kl) * row_stride + 4 * vd)
                                   : make_uint2(0, 0);
        }
    };
    auto store_tile = [&](int j, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int r = kr0 + 32 * i;
            int n = seg_base + j * BN + r;
            int t = 0, h = 0, w = 0;
            bool text = n >= g.Nv;
            if (!text) decode_pos(n, g, t, h, w);
            uint4 rot = rope_chunk(kraw[i], kc, t, h, w, text, g, p.table);
            *reinterpret_cast<uint4*>(&lds_k[buf][r * KS + 8 * kc]) = rot;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t w0 = half16(vraw[0], e) | (half16(vraw[1], e) << 16);
            uint32_t w1 = half16(vraw[2], e) | (half16(vraw[3], e) << 16);
            *reinterpret_cast<uint2*>(&lds_v[buf][(4 * vd + e) * VS + vpos]) = make_uint2(w0, w1);
        }
    };

    // ---- prologue: first K/V tile, then Q (rotated, kept in registers) ------------------------
    load_tile(0);

    const int q_local = qt * BM + wave * 32 + l32;
    const bool q_valid = q_local < seg_len;
    const int q_row = seg_base + (q_valid ? q_local : 0);
    bf16x8_t qreg[8];
    {
        int t = 0, h = 0, w = 0;
        bool text = q_row >= g.Nv;
        if (!text) decode_pos(q_row, g, t, h, w);
        const uint16_t* qp = p.q + q_row * row_stride + (long long)head * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            int c = 2 * ks + hh;
            uint4 raw = q_valid ? ld16(qp + 8 * c) : make_uint4(0, 0, 0, 0);
            qreg[ks] = __builtin_bit_cast(bf16x8_t, rope_chunk(raw, c, t, h, w, text, g, p.table));
        }
    }

    store_tile(0, 0);
    __syncthreads();

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;
    const float sl2 = p.scale_log2;

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool has_next = j + 1 < ntiles;
        if (has_next) load_tile(j + 1);

        // S^T = K~ Q~^T for two 32-key blocks.
        f32x16_t sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[mb][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                    &lds_k[buf][(32 * mb + l32) * KS + 16 * ks + 8 * hh]);
                sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[mb], 0, 0, 0);
            }
        }

        // Keys past the end of the sequence (last tile only) get -inf.
        if (j == ntiles - 1 && (seg_len % BN) != 0) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    int key = j * BN + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key >= seg_len) sacc[mb][i] = -INFINITY;
                }
        }

        // Online softmax (lane = one query, 32 of the tile's keys; partner lane l^32 the rest).
        float mx = sacc[0][0];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
        const float mneg = -m_new * sl2;
        m_run = m_new;
        float lsum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = __builtin_amdgcn_exp2f(fmaf(sacc[mb][i], sl2, mneg));
                sacc[mb][i] = e;
                lsum += e;
            }
        l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

        // P^T as the B operand: chunk c (16 keys) = block c/2, accumulator entries 8(c%2)..+7.
        bf16x8_t pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int mb = c >> 1, o = 8 * (c & 1);
            uint4 u;
            u.x = pack_bf16x2(sacc[mb][o + 0], sacc[mb][o + 1]);
            u.y = pack_bf16x2(sacc[mb][o + 2], sacc[mb][o + 3]);
            u.z = pack_bf16x2(sacc[mb][o + 4], sacc[mb][o + 5]);
            u.w = pack_bf16x2(sacc[mb][o + 6], sacc[mb][o + 7]);
            pb[c] = __builtin_bit_cast(bf16x8_t, u);
        }

        // O^T += V~^T P^T: four 32-row blocks of d, four 16-key chunks.
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                    &lds_v[buf][(32 * db + l32) * VS + 16 * c + 8 * hh]);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
            }

        if (has_next) store_tile(j + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O / l -> bf16 ---------------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (q_valid) {
        uint16_t* op = p.out + q_row * row_stride + (long long)head * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d0 = 32 * db + 8 * grp + 4 * hh;
                uint2 u;
                u.x = pack_bf16x2(oacc[db][4 * grp + 0] * inv, oacc[db][4 * grp + 1] * inv);
                u.y = pack_bf16x2(oacc[db][4 * grp + 2] * inv, oacc[db][4 * grp + 3] * inv);
                *reinterpret_cast<uint2*>(op + d0) = u;
            }
    }
}

}  // namespace

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* out, const float2* table, const RopeGeom& g, int N,
                            int heads, int seg_len, int n_segs, hipStream_t stream) {
    (void)N;
    AttnParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.seg_len = seg_len;
    p.n_segs = n_segs;
    p.q_tiles = (seg_len + BM - 1) / BM;
    p.total_wg = p.q_tiles * n_segs * heads;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(p.total_wg), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace st
