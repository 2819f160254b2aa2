// Flash attention forward on MFMA (gfx950) for the bf16 storage path, with 3D RoPE.
//
// What it computes: for every query row n of a sequence, out[n] = sum_j softmax_j(q~_n . k~_j /
// sqrt(128)) v_j over the sequence's key rows j, where q~ and k~ are q and k turned by the 3D
// rotation of their own (t, h, w) ("A video model's architecture: spatiotemporal attention and
// the 3D VAE", self-test answers 2 and 4; "CogVideoX Architecture: ...", section "3. 3D Rotary
// Position Embeddings (3D RoPE)").  A sequence is all N rows (full 3D attention) or the H*W rows
// of one frame (the spatial stage of factorised attention, "How attention sees time").
//
// Numerics: rotated q and k are rounded once to fp16 (11 significant bits) for the score product
// (v_mfma_f32_32x32x16_f16, same rate as bf16); softmax weights are rounded to bf16 and multiply
// the exact bf16 values (v_mfma_f32_32x32x16_bf16); accumulation, the running max and the row
// sums are fp32, and the row sum adds exactly the rounded weights the product used.
//
// Two ways to feed K and V (template flag FUSED):
//  * FUSED: K and V tiles are read from the caller's [N][heads][128] tensors; every K tile is
//    rotated (position decoded from the flat row index) while it is copied into LDS, and every V
//    tile is transposed on the same copy.  Nothing else runs before the kernel.
//  * staged (default): a preparation kernel first rotates K into fp16 tiles and transposes V into
//    the V^T tile order, once per key; the attention kernel then copies tiles without arithmetic.
//    Q is rotated inside the attention kernel in both modes (once per workgroup).
//
// Design (one workgroup = 8 waves = 256 query rows of one head and one sequence):
//  * Scores are formed transposed, S^T = K~ Q~^T: a lane owns one query column and 16 keys per
//    32x32 block, so the softmax row max and row sum are in-lane plus one exchange between the
//    two 32-lane halves (v_permlane32_swap).
//  * P^T leaves the score accumulator already in the B-operand layout of the PV product; the V^T
//    tile in LDS stores keys in the matching order (within each 16 keys: 0-3, 8-11, 4-7, 12-15).
//  * Three LDS tile buffers: tile j+2 is written while tiles j (PV) and j+1 (scores) are read,
//    so one barrier per tile suffices; tile j+3 is fetched into registers meanwhile.
//  * The score product of tile j+1 is issued before the softmax of tile j, so the MFMA pipe works
//    while the VALU computes exponentials.
//  * Online softmax with a lazily updated running max: the accumulator is rescaled only when a
//    row max exceeds the stored one by more than 2^8 (exact in any case; the stored max is only
//    an offset for the exponentials).
#include "st_internal.h"

namespace st {
namespace {

constexpr int D = 128;          // head dimension
constexpr int BM = 256;         // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 512;   // 8 waves
constexpr int KS = 136;         // K tile row stride in LDS (fp16): 272 B, rows start 4 banks apart
constexpr int VS = 72;          // V^T tile row stride in LDS (bf16): 144 B
constexpr int KTILE = BN * KS;
constexpr int VTILE = D * VS;
constexpr int NBUF = 3;
constexpr float LAZY_LOG2 = 8.0f;  // rescale when the max grows by more than this (log2 units)

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;     // FUSED: K [N][heads][D] bf16; staged: K~ tiles, fp16
    const uint16_t* v;     // FUSED: V [N][heads][D] bf16; staged: V^T tiles, bf16
    uint16_t* out;
    const float2* table;
    RopeGeom g;
    int heads;
    int seg_len;
    int n_segs;
    int q_tiles;
    int k_tiles;
    int total_wg;
    float scale_log2;      // log2(e) / sqrt(D)
};

struct PrepParams {
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* kt;          // [heads][n_segs][k_tiles][BN][D] fp16
    uint16_t* vt;          // [heads][n_segs][k_tiles][D][BN] bf16, keys permuted within 16
    const float2* table;
    RopeGeom g;
    int heads;
    int seg_len;
    int n_segs;
    int k_tiles;
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Rotate 8 bf16 channels (pairs 4c .. 4c+3) of a row at (t, h, w) and return them as fp16.
__device__ __forceinline__ uint4 rope_chunk_f16(uint4 raw, int c, int t, int h, int w, bool text,
                                                const RopeGeom& g, const float2* __restrict__ table) {
    uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float2 cs = table[pair_entry(4 * c + i, t, h, w, text, g)];
        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
        rotate_pair(x0, x1, cs);
        wd[i] = pack_f16x2(x0, x1);
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

__device__ __forceinline__ uint32_t half16(uint2 v, int e) {
    uint32_t w = (e < 2) ? v.x : v.y;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Position of key 4*grp (a group of 4 consecutive keys) inside a V^T row of 64 keys.
__device__ __forceinline__ int vt_pos(int grp) {
    const int sb = grp & 3;
    return 16 * (grp >> 2) + ((sb & 1) << 3) + ((sb >> 1) << 2);
}

// Sum over the two 32-lane halves (lane i and i ^ 32) of a wave.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool FUSED>
__global__ void __launch_bounds__(NTHREADS, 1) attn_fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[NBUF][KTILE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[NBUF][VTILE];

    const int logical = xcd_remap(blockIdx.x, p.total_wg);
    const int qt = logical % p.q_tiles;
    const int rest = logical / p.q_tiles;
    const int seg = rest % p.n_segs;
    const int head = rest / p.n_segs;
    const int seg_base = seg * p.seg_len;
    const int seg_len = p.seg_len;
    const long long row_stride = (long long)p.heads * D;
    const int ntiles = p.k_tiles;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const RopeGeom& g = p.g;

    // ---- tile copy: global -> registers (load_tile) -> LDS (store_tile) -------------------------
    uint4 st0, st1, st2, st3;      // staged tile data (meaning depends on the mode)
    // FUSED geometry: K chunk kc of rows kr0, kr0+32; V channels 4vd.. of keys 4vg..
    const int kc = tid & 15;
    const int kr0 = tid >> 4;
    const int vd = tid & 31;
    const int vg = tid >> 5;
    const uint16_t* __restrict__ kbase = p.k + (FUSED ? (long long)head * D : 0);
    const uint16_t* __restrict__ vbase = p.v + (FUSED ? (long long)head * D : 0);
    const long long tile0 = ((long long)head * p.n_segs + seg) * ntiles;

    auto load_tile = [&](int j) {
        if constexpr (FUSED) {
            int kl0 = j * BN + kr0, kl1 = kl0 + 32;
            st0 = kl0 < seg_len ? ld16(kbase + (seg_base + kl0) * row_stride + 8 * kc) : make_uint4(0, 0, 0, 0);
            st1 = kl1 < seg_len ? ld16(kbase + (seg_base + kl1) * row_stride + 8 * kc) : make_uint4(0, 0, 0, 0);
            uint2 vr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int kl = j * BN + 4 * vg + r;
                vr[r] = kl < seg_len ? ld8(vbase + (seg_base + kl) * row_stride + 4 * vd) : make_uint2(0, 0);
            }
            st2 = make_uint4(vr[0].x, vr[0].y, vr[1].x, vr[1].y);
            st3 = make_uint4(vr[2].x, vr[2].y, vr[3].x, vr[3].y);
        } else {
            const uint16_t* kt = kbase + (tile0 + j) * (BN * D);
            const uint16_t* vt = vbase + (tile0 + j) * (BN * D);
            st0 = ld16(kt + 8 * tid);
            st1 = ld16(kt + 8 * (tid + NTHREADS));
            st2 = ld16(vt + 8 * tid);
            st3 = ld16(vt + 8 * (tid + NTHREADS));
        }
    };
    auto store_tile = [&](int j, int buf) {
        uint16_t* lk = lds_k[buf];
        uint16_t* lv = lds_v[buf];
        if constexpr (FUSED) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = kr0 + 32 * i;
                const int n = seg_base + j * BN + r;
                int t = 0, h = 0, w = 0;
                const bool text = n >= g.Nv;
                if (!text) decode_pos(n, g, t, h, w);
                uint4 rot = rope_chunk_f16(i == 0 ? st0 : st1, kc, t, h, w, text, g, p.table);
                *reinterpret_cast<uint4*>(&lk[r * KS + 8 * kc]) = rot;
            }
            uint2 vr[4] = {make_uint2(st2.x, st2.y), make_uint2(st2.z, st2.w),
                           make_uint2(st3.x, st3.y), make_uint2(st3.z, st3.w)};
            const int pos = vt_pos(vg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w0 = half16(vr[0], e) | (half16(vr[1], e) << 16);
                uint32_t w1 = half16(vr[2], e) | (half16(vr[3], e) << 16);
                *reinterpret_cast<uint2*>(&lv[(4 * vd + e) * VS + pos]) = make_uint2(w0, w1);
            }
        } else {
            (void)j;
            const int c0 = tid, c1 = tid + NTHREADS;
            *reinterpret_cast<uint4*>(&lk[(c0 >> 4) * KS + 8 * (c0 & 15)]) = st0;
            *reinterpret_cast<uint4*>(&lk[(c1 >> 4) * KS + 8 * (c1 & 15)]) = st1;
            *reinterpret_cast<uint4*>(&lv[(c0 >> 3) * VS + 8 * (c0 & 7)]) = st2;
            *reinterpret_cast<uint4*>(&lv[(c1 >> 3) * VS + 8 * (c1 & 7)]) = st3;
        }
    };

    // ---- prologue ---------------------------------------------------------------------------------
    load_tile(0);
    store_tile(0, 0);
    if (ntiles > 1) {
        load_tile(1);
        store_tile(1, 1);
    }
    if (ntiles > 2) load_tile(2);

    const int q_local = qt * BM + wave * 32 + l32;
    const bool q_valid = q_local < seg_len;
    const int q_row = seg_base + (q_valid ? q_local : 0);
    f16x8_t qreg[8];
    {
        int t = 0, h = 0, w = 0;
        const bool text = q_row >= g.Nv;
        if (!text) decode_pos(q_row, g, t, h, w);
        const uint16_t* qp = p.q + q_row * row_stride + (long long)head * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int c = 2 * ks + hh;
            uint4 raw = q_valid ? ld16(qp + 8 * c) : make_uint4(0, 0, 0, 0);
            qreg[ks] = __builtin_bit_cast(f16x8_t, rope_chunk_f16(raw, c, t, h, w, text, g, p.table));
        }
    }
    __syncthreads();

    auto qk = [&](int buf, f32x16_t (&s)[2]) {
        const uint16_t* lk = lds_k[buf];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mb][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                f16x8_t a = *reinterpret_cast<const f16x8_t*>(&lk[(32 * mb + l32) * KS + 16 * ks + 8 * hh]);
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], s[mb], 0, 0, 0);
            }
        }
    };

    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;
    const float sl2 = p.scale_log2;
    const float lazy_raw = LAZY_LOG2 / sl2;
    const bool ragged = (seg_len % BN) != 0;
    const uint32_t one2 = 0x3f803f80u;  // bf16 pair (1, 1)

    // One tile step: softmax and PV of tile j (scores in sc) while the scores of tile j+1 are
    // formed into sn.
    auto step = [&](int j, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
        const int b = j % NBUF;
        if (j + 1 < ntiles) qk((j + 1) % NBUF, sn);

        if (ragged && j == ntiles - 1) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * BN + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key >= seg_len) sc[mb][i] = -INFINITY;
                }
        }
        float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[0][i], sc[0][i + 1]));
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[1][i], sc[1][i + 1]));
        mx = xhalf_max(mx);
        const bool grow = mx > m_run + lazy_raw;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float mneg = -m_run * sl2;
        bf16x8_t pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int mb = c >> 1, o = 8 * (c & 1);
            uint32_t u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[mb][o + 2 * e], sl2, mneg));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[mb][o + 2 * e + 1], sl2, mneg));
                u[e] = pack_bf16x2(p0, p1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e]),
                                                        __builtin_bit_cast(bf16x2_t, one2), l_run, false);
            }
            pb[c] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
        }
        const uint16_t* lv = lds_v[b];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&lv[(32 * db + l32) * VS + 16 * c + 8 * hh]);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
            }
        if (j + 2 < ntiles) store_tile(j + 2, (j + 2) % NBUF);
        if (j + 3 < ntiles) load_tile(j + 3);
        __syncthreads();
    };

    f32x16_t sa[2], sb[2];
    qk(0, sa);
    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
        step(j, sa, sb);
        step(j + 1, sb, sa);
    }
    if (j < ntiles) step(j, sa, sb);

    // ---- epilogue: O / l -> bf16 ---------------------------------------------------------------
    const float inv = 1.0f / xhalf_sum(l_run);
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

// Preparation for the staged mode: one workgroup per (head, segment, key tile) rotates the tile's
// 64 K rows into fp16 and writes the V tile transposed (keys permuted within each 16 as the PV
// operand expects).  Rows past the segment are written as zeros.
__global__ void __launch_bounds__(256) kv_prep_kernel(PrepParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lv[BN * KS];
    const int tile = blockIdx.x;
    const int kt = tile % p.k_tiles;
    const int rest = tile / p.k_tiles;
    const int seg = rest % p.n_segs;
    const int head = rest / p.n_segs;
    const long long row_stride = (long long)p.heads * D;
    const int tid = threadIdx.x;
    const RopeGeom& g = p.g;
    uint16_t* kt_out = p.kt + (long long)tile * (BN * D);
    uint16_t* vt_out = p.vt + (long long)tile * (BN * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int r = id >> 4, c = id & 15;
        const int kl = kt * BN + r;
        const bool valid = kl < p.seg_len;
        const int n = seg * p.seg_len + (valid ? kl : 0);
        const long long off = n * row_stride + (long long)head * D + 8 * c;
        uint4 kraw = valid ? ld16(p.k + off) : make_uint4(0, 0, 0, 0);
        uint4 vraw = valid ? ld16(p.v + off) : make_uint4(0, 0, 0, 0);
        int t = 0, h = 0, w = 0;
        const bool text = n >= g.Nv;
        if (!text) decode_pos(n, g, t, h, w);
        *reinterpret_cast<uint4*>(kt_out + r * D + 8 * c) = rope_chunk_f16(kraw, c, t, h, w, text, g, p.table);
        *reinterpret_cast<uint4*>(&lv[r * KS + 8 * c]) = vraw;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = tid + 256 * i;
        const int d = id >> 3, c8 = id & 7;
        const int k0 = 16 * (c8 >> 1) + 4 * (c8 & 1);
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ka = k0 + (e < 2 ? 2 * e : 8 + 2 * (e - 2));
            wd[e] = (uint32_t)lv[ka * KS + d] | ((uint32_t)lv[(ka + 1) * KS + d] << 16);
        }
        *reinterpret_cast<uint4*>(vt_out + d * BN + 8 * c8) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
}

AttnParams make_params(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                       const float2* table, const RopeGeom& g, int heads, int seg_len, int n_segs) {
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
    p.k_tiles = (seg_len + BN - 1) / BN;
    p.total_wg = p.q_tiles * n_segs * heads;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    return p;
}

}  // namespace

size_t attn_stage_elems(int heads, int seg_len, int n_segs) {
    const size_t k_tiles = (size_t)(seg_len + BN - 1) / BN;
    return (size_t)heads * n_segs * k_tiles * BN * D;
}

hipError_t launch_kv_prep(const uint16_t* k, const uint16_t* v, uint16_t* kt, uint16_t* vt,
                          const float2* table, const RopeGeom& g, int heads, int seg_len,
                          int n_segs, hipStream_t stream) {
    PrepParams p;
    p.k = k;
    p.v = v;
    p.kt = kt;
    p.vt = vt;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.seg_len = seg_len;
    p.n_segs = n_segs;
    p.k_tiles = (seg_len + BN - 1) / BN;
    const int blocks = heads * n_segs * p.k_tiles;
    hipLaunchKernelGGL(kv_prep_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_staged(const uint16_t* q, const uint16_t* kt, const uint16_t* vt,
                                   uint16_t* out, const float2* table, const RopeGeom& g,
                                   int heads, int seg_len, int n_segs, hipStream_t stream) {
    AttnParams p = make_params(q, kt, vt, out, table, g, heads, seg_len, n_segs);
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(p.total_wg), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* out, const float2* table, const RopeGeom& g,
                                  int heads, int seg_len, int n_segs, hipStream_t stream) {
    AttnParams p = make_params(q, k, v, out, table, g, heads, seg_len, n_segs);
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(p.total_wg), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace st
