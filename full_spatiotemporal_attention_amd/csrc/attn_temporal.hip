// Temporal stage of factorised attention on MFMA (gfx950), bf16 storage.
//
// After spatial attention inside each frame, every spatial position s attends along time: the T
// rows t * S + s, t < T, form one short sequence ("A video model's architecture: spatiotemporal
// attention and the 3D VAE", self-test answer 2: H'W' sequences of length T').  The same rotated
// q and k are used; the values are the spatial stage's output.  These sequences are short (T is
// 5 to 33 for the pages' grids) and many (H'W' x heads), so the kernel is bound by HBM traffic:
// each wave owns one (s, head) sequence, keeps its Q~ and K~ blocks in registers and stages only
// the transposed values through LDS.  Four waves of a workgroup take four consecutive heads of
// the same position, whose rows are adjacent in memory.  Numerics as in the full-attention
// kernel: rotated q and k in fp16 for the score product, weights in bf16 against the bf16
// values, fp32 accumulation.
#include "st_internal.h"

namespace st {
namespace {

constexpr int D = 128;
constexpr int TB = 32;      // rows per block (queries and keys)
constexpr int WAVES = 4;
constexpr int VTS = 40;     // V^T row stride (bf16) in LDS: 32 keys + 8 padding

struct TemporalParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* vs;
    uint16_t* out;
    const float2* table;
    RopeGeom g;
    int heads;
    int n_seq;        // S * heads
    float scale_log2;
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Rotate 8 bf16 channels (pairs 4c .. 4c+3) and return them as fp16 (the score-product type).
__device__ __forceinline__ uint4 rope_chunk(uint4 raw, int c, int t, int h, int w,
                                            const RopeGeom& g, const float2* __restrict__ table) {
    uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float2 cs = table[pair_entry(4 * c + i, t, h, w, false, g)];
        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
        rotate_pair(x0, x1, cs);
        f16x2_t hv = {(_Float16)x0, (_Float16)x1};
        wd[i] = __builtin_bit_cast(uint32_t, hv);
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

__device__ __forceinline__ uint32_t half16(uint2 v, int e) {
    uint32_t w = (e < 2) ? v.x : v.y;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__global__ void __launch_bounds__(WAVES * 64) attn_temporal_bf16_kernel(TemporalParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[WAVES][D * VTS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int id = blockIdx.x * WAVES + wave;
    const bool seq_valid = id < p.n_seq;
    const int idc = seq_valid ? id : 0;
    const int s = idc / p.heads;
    const int head = idc - s * p.heads;
    const RopeGeom& g = p.g;
    const int T = g.T;
    const int S = g.S;
    const long long row_stride = (long long)p.heads * D;
    const int sh = s / g.W;
    const int sw = s - sh * g.W;
    const int nblk = (T + TB - 1) / TB;
    const float sl2 = p.scale_log2;
    uint16_t* vt = lds_v[wave];

    const int vd = lane & 31;
    const int vg0 = lane >> 5;

    for (int qb = 0; qb < nblk; ++qb) {
        const int tq = qb * TB + l32;
        const bool qv = tq < T;
        f16x8_t qreg[8];
        {
            const uint16_t* qp = p.q + (long long)(tq * S + s) * row_stride + (long long)head * D;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                int c = 2 * ks + hh;
                uint4 raw = qv ? ld16(qp + 8 * c) : make_uint4(0, 0, 0, 0);
                qreg[ks] = __builtin_bit_cast(f16x8_t, rope_chunk(raw, c, qv ? tq : 0, sh, sw, g, p.table));
            }
        }
        f32x16_t oacc[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
        float m_run = -INFINITY, l_run = 0.0f;

        for (int kb = 0; kb < nblk; ++kb) {
            const int tk = kb * TB + l32;
            const bool kv = tk < T;
            f32x16_t sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
            {
                const uint16_t* kp = p.k + (long long)(tk * S + s) * row_stride + (long long)head * D;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    int c = 2 * ks + hh;
                    uint4 raw = kv ? ld16(kp + 8 * c) : make_uint4(0, 0, 0, 0);
                    f16x8_t a = __builtin_bit_cast(f16x8_t, rope_chunk(raw, c, kv ? tk : 0, sh, sw, g, p.table));
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], sacc, 0, 0, 0);
                }
            }
            // values of this key block -> LDS, transposed (keys within 16: 0-3, 8-11, 4-7, 12-15)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int grp = vg0 + 2 * gi;
                uint2 vr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int t = kb * TB + 4 * grp + r;
                    vr[r] = t < T ? ld8(p.vs + (long long)(t * S + s) * row_stride + (long long)head * D + 4 * vd)
                                  : make_uint2(0, 0);
                }
                const int sb = grp & 3;
                const int pos = 16 * (grp >> 2) + ((sb & 1) << 3) + ((sb >> 1) << 2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w0 = half16(vr[0], e) | (half16(vr[1], e) << 16);
                    uint32_t w1 = half16(vr[2], e) | (half16(vr[3], e) << 16);
                    *reinterpret_cast<uint2*>(&vt[(4 * vd + e) * VTS + pos]) = make_uint2(w0, w1);
                }
            }
            // mask keys past T
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int key = kb * TB + 8 * (i >> 2) + 4 * hh + (i & 3);
                if (key >= T) sacc[i] = -INFINITY;
            }
            float mx = sacc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
            const float mneg = -m_new * sl2;
            m_run = m_new;
            float lsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = __builtin_amdgcn_exp2f(fmaf(sacc[i], sl2, mneg));
                sacc[i] = e;
                lsum += e;
            }
            l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            bf16x8_t pb[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int o = 8 * c;
                uint4 u;
                u.x = pack_bf16x2(sacc[o + 0], sacc[o + 1]);
                u.y = pack_bf16x2(sacc[o + 2], sacc[o + 3]);
                u.z = pack_bf16x2(sacc[o + 4], sacc[o + 5]);
                u.w = pack_bf16x2(sacc[o + 6], sacc[o + 7]);
                pb[c] = __builtin_bit_cast(bf16x8_t, u);
            }
            __syncthreads();
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&vt[(32 * db + l32) * VTS + 16 * c + 8 * hh]);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
                }
            __syncthreads();
        }

        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const float inv = 1.0f / l_tot;
        if (seq_valid && qv) {
            uint16_t* op = p.out + (long long)(tq * S + s) * row_stride + (long long)head * D;
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
}

}  // namespace

hipError_t launch_attn_temporal_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* vs,
                                     uint16_t* out, const float2* table, const RopeGeom& g,
                                     int heads, hipStream_t stream) {
    TemporalParams p;
    p.q = q;
    p.k = k;
    p.vs = vs;
    p.out = out;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.n_seq = g.S * heads;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    int blocks = (p.n_seq + WAVES - 1) / WAVES;
    hipLaunchKernelGGL(attn_temporal_bf16_kernel, dim3(blocks), dim3(WAVES * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace st
