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
        float2 cs = table[pair_entry(4 * c + i, t, h, w, g)];
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

// ---- short sequences (T <= 32): one 32x32 block, everything loaded up front -----------------
//
// One wave per (position, head) sequence, four waves per workgroup (four consecutive heads of a
// position, adjacent in memory).  A wave issues all of its HBM reads before any arithmetic: the
// T value rows by LDS DMA into a private 8 KB LDS block, the T rotated fp16 K~ rows from the
// spatial stage's staging buffer (the same rotation, already applied), and the T raw q rows.
// Only then does it rotate q, form the 32x32 score block on MFMA, take the softmax in-lane and
// multiply by V^T read transposed from LDS.  Rows past T repeat row T-1 (their keys are
// masked, their query rows are not written), so no lane reads outside the tensors.
constexpr int SHORT_WAVES = 4;
constexpr int SHORT_T = 32;

struct ShortParams {
    const uint16_t* q;
    const uint16_t* kt;     // staged K~ [heads][T][k_tiles][64][D] fp16
    const uint16_t* vs;
    uint16_t* out;
    const float2* table;
    RopeGeom g;
    int heads;
    int n_seq;
    int k_tiles;
    float scale_log2;
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// LDS swizzle of 16-byte chunks for the transposed V reads (4 rows x 4 chunks per 32 lanes hit
// 16 distinct chunks of the 64 banks).
__device__ __forceinline__ int vs_swz(int r) { return (r & 3) << 2; }

__global__ void __launch_bounds__(SHORT_WAVES * 64) attn_temporal_short_kernel(ShortParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[SHORT_WAVES * SHORT_T * 256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int id = blockIdx.x * SHORT_WAVES + wave;
    if (id >= p.n_seq) return;   // whole waves only; the kernel has no barrier
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    // Wave-uniform (scalar) sequence coordinates: the DMA base address must sit in SGPRs.
    const int s = __builtin_amdgcn_readfirstlane(id / p.heads);
    const int head = __builtin_amdgcn_readfirstlane(id - s * p.heads);
    const RopeGeom& g = p.g;
    const int T = g.T;
    const int S = g.S;
    const long long row_stride = (long long)p.heads * D;
    const int sh = s / g.W;
    const int sw = s - sh * g.W;
    const uint32_t lds_w = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_raw
                           + wave * (SHORT_T * 256);

    // V rows -> LDS.  Copy i: rows 4i + lane/16, lane's physical chunk lane%16 holds logical
    // chunk (lane%16) ^ swz(row).  Offsets are 32-bit: the host checks the tensor size.
    {
        const uint16_t* vbase = p.vs + (long long)s * row_stride + (long long)head * D;
        const int pc = lane & 15;
#pragma unroll
        for (int i = 0; i < SHORT_T / 4; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int rc = r < T ? r : T - 1;
            const uint32_t off = 2u * (uint32_t)(rc * S * (int)row_stride + 8 * (pc ^ vs_swz(r)));
            dma16(vbase, off, lds_w + i * 1024);
        }
    }
    const int tr = l32 < T ? l32 : T - 1;
    // K~ operand rows (key tr) and raw q rows (query tr), chunks 2ks + hh.
    f16x8_t ka[8];
    {
        const uint16_t* kp = p.kt + (((long long)(head * T + tr) * p.k_tiles + (s >> 6)) * 64 + (s & 63)) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) ka[ks] = __builtin_bit_cast(f16x8_t, ld16(kp + 8 * (2 * ks + hh)));
    }
    uint4 qraw[8];
    {
        const uint16_t* qp = p.q + (long long)(tr * S + s) * row_stride + (long long)head * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qraw[ks] = ld16(qp + 8 * (2 * ks + hh));
    }
    f16x8_t qreg[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qreg[ks] = __builtin_bit_cast(f16x8_t, rope_chunk(qraw[ks], 2 * ks + hh, tr, sh, sw, g, p.table));

    // S^T = K~ Q~^T: lane holds query l32 and keys 8(i/4) + 4hh + i%4.
    f32x16_t sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], qreg[ks], sacc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= T) sacc[i] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float sl2 = p.scale_log2;
    const float mneg = -mx * sl2;
    const uint32_t one2 = 0x3f803f80u;
    bf16x8_t pb[2];
    float lsum = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * c + 2 * e], sl2, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[8 * c + 2 * e + 1], sl2, mneg));
            u[e] = pack_bf16x2(p0, p1);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e]),
                                                   __builtin_bit_cast(bf16x2_t, one2), lsum, false);
        }
        pb[c] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
    }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lsum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }

    // The value rows have landed in this wave's LDS block once its copies have completed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // O^T += V^T P^T: V^T read transposed.  Lane (i = lane%16, gq = lane/16) reads row
    // 4(gq/2) + i/4 (+8 for the upper half, +16 per key chunk) at logical chunk 4db + u.
    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
    {
        const int i = lane & 15, gq = lane >> 4;
        const int row = 4 * (gq >> 1) + (i >> 2);
        const int u = 2 * (gq & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint32_t a = lds_w + (row + 16 * c) * 256 + 16 * ((4 * db + u) ^ vs_swz(row)) + 8 * (i & 1);
                i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a);
                i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)(a + 8 * 256));
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], oacc[db], 0, 0, 0);
            }
    }

    // Output rows through this wave's LDS block (its V rows are consumed): bf16 row-major with
    // 16-byte chunk c of row r at physical chunk c ^ (r & 15), then written back as whole rows,
    // 16 bytes per lane, four rows per store.
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const u32x2_t w = {pack_bf16x2(oacc[db][4 * grp + 0] * inv, oacc[db][4 * grp + 1] * inv),
                               pack_bf16x2(oacc[db][4 * grp + 2] * inv, oacc[db][4 * grp + 3] * inv)};
            const uint32_t a = lds_w + l32 * 256 + 16 * ((4 * db + grp) ^ (l32 & 15)) + 8 * hh;
            *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)a = w;
        }
    {
        const int pc = lane & 15;
#pragma unroll
        for (int i = 0; i < SHORT_T / 4; ++i) {
            const int r = 4 * i + (lane >> 4);
            const uint32_t a = lds_w + r * 256 + 16 * pc;
            const u32x4_t v = *(__attribute__((address_space(3))) const u32x4_t*)(uintptr_t)a;
            if (r < T) {
                uint16_t* op = p.out + (long long)(r * S + s) * row_stride + (long long)head * D +
                               8 * (pc ^ (r & 15));
                *reinterpret_cast<uint4*>(op) = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// ---- medium sequences (32 < T <= 64): two 32-row blocks, everything loaded up front ----------
//
// The short kernel's design over two blocks of 32 rows (HunyuanVideo's 33 latent frames need it).
// Two waves per (position, head) sequence, one per 32-row query block, and two sequences (two
// consecutive heads of a position) per workgroup.  A wave issues all of its HBM reads before any
// arithmetic: half of the sequence's 64 value rows by LDS DMA into the sequence's 16 KB LDS block
// (the other wave of the pair copies the other half), all 64 rotated fp16 K~ rows of the sequence
// from the staging buffer (the pair reads them twice; the second read hits in cache) and the raw q
// rows of its own query block.  It then rotates q, forms the two 32x32 score blocks on MFMA, takes
// the softmax over both in-lane and, after a barrier that makes the pair's value rows visible,
// multiplies by V^T read transposed from LDS.  Rows past T repeat row T-1 (their keys are masked,
// their query rows are not written), so no lane reads outside the tensors.  A workgroup whose
// second sequence lies past the last one computes a copy of the last and writes nothing for it.
constexpr int MID_T = 64;
constexpr int MID_SEQS = 2;   // sequences per workgroup (two waves each)

// At most 128 VGPRs, so that four waves share a SIMD (118 without spills; left free the compiler
// takes 204, two waves per SIMD).  The compiler then issues fewer of a wave's loads ahead of its
// first products, but the extra waves keep more of them in flight.
__global__ void __launch_bounds__(MID_SEQS * 2 * 64, 4) attn_temporal_mid_kernel(ShortParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[MID_SEQS * MID_T * 256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sq = wave >> 1;    // sequence of this workgroup
    const int qb = wave & 1;     // query block of this wave
    const int id = blockIdx.x * MID_SEQS + sq;
    const bool seq_valid = id < p.n_seq;
    const int idc = seq_valid ? id : p.n_seq - 1;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    // Wave-uniform (scalar) sequence coordinates: the DMA base address must sit in SGPRs.
    const int s = __builtin_amdgcn_readfirstlane(idc / p.heads);
    const int head = __builtin_amdgcn_readfirstlane(idc - s * p.heads);
    const RopeGeom& g = p.g;
    const int T = g.T;
    const int S = g.S;
    const long long row_stride = (long long)p.heads * D;
    const int sh = s / g.W;
    const int sw = s - sh * g.W;
    const uint32_t lds_s = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_raw
                           + sq * (MID_T * 256);

    // V rows 32 qb .. 32 qb + 31 -> LDS.  Copy i: rows 32 qb + 4i + lane/16, lane's physical
    // chunk lane%16 holds logical chunk (lane%16) ^ swz(row).  Offsets are 32-bit: the host checks
    // the tensor size.
    {
        const uint16_t* vbase = p.vs + (long long)s * row_stride + (long long)head * D;
        const int pc = lane & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 32 * qb + 4 * i + (lane >> 4);
            const int rc = r < T ? r : T - 1;
            const uint32_t off = 2u * (uint32_t)(rc * S * (int)row_stride + 8 * (pc ^ vs_swz(r)));
            dma16(vbase, off, lds_s + (32 * qb + 4 * i) * 256);
        }
    }
    // K~ operand rows (keys 32 kb + l32) and raw q rows (query 32 qb + l32), chunks 2ks + hh.
    f16x8_t ka[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int tk = 32 * kb + l32 < T ? 32 * kb + l32 : T - 1;
        const uint16_t* kp = p.kt + (((long long)(head * T + tk) * p.k_tiles + (s >> 6)) * 64 + (s & 63)) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) ka[kb][ks] = __builtin_bit_cast(f16x8_t, ld16(kp + 8 * (2 * ks + hh)));
    }
    const int tq_raw = 32 * qb + l32;
    const int tq = tq_raw < T ? tq_raw : T - 1;
    uint4 qraw[8];
    {
        const uint16_t* qp = p.q + (long long)(tq * S + s) * row_stride + (long long)head * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qraw[ks] = ld16(qp + 8 * (2 * ks + hh));
    }
    f16x8_t qreg[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qreg[ks] = __builtin_bit_cast(f16x8_t, rope_chunk(qraw[ks], 2 * ks + hh, tq, sh, sw, g, p.table));

    // S^T = K~ Q~^T per key block: lane holds query 32 qb + l32 and keys 32 kb + 8(i/4) + 4hh + i%4.
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[kb][ks], qreg[ks], sacc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (key >= T) sacc[kb][i] = -INFINITY;
        }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float sl2 = p.scale_log2;
    const float mneg = -mx * sl2;
    const uint32_t one2 = 0x3f803f80u;
    bf16x8_t pb[2][2];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * c + 2 * e], sl2, mneg));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * c + 2 * e + 1], sl2, mneg));
                u[e] = pack_bf16x2(p0, p1);
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e]),
                                                       __builtin_bit_cast(bf16x2_t, one2), lsum, false);
            }
            pb[kb][c] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
        }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lsum = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }

    // This wave's value rows have landed once its copies completed; the barrier makes the other
    // wave's half of the sequence visible too.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // O^T += V^T P^T over both key blocks: V^T read transposed.  Lane (i = lane%16, gq = lane/16)
    // reads row 32 kb + 4(gq/2) + i/4 (+8 for the upper half, +16 per key chunk) at logical chunk
    // 4db + u.
    f32x16_t oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
    {
        const int i = lane & 15, gq = lane >> 4;
        const int row = 4 * (gq >> 1) + (i >> 2);
        const int u = 2 * (gq & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const uint32_t a = lds_s + (32 * kb + row + 16 * c) * 256 + 16 * ((4 * db + u) ^ vs_swz(row)) +
                                       8 * (i & 1);
                    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a);
                    i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)(a + 8 * 256));
                    const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][c], oacc[db], 0, 0, 0);
                }
    }

    // Output rows through the wave's half of the LDS block, once both waves of the pair have read
    // all value rows: bf16 row-major with 16-byte chunk c of row r at physical chunk c ^ (r & 15),
    // then written back as whole rows, 16 bytes per lane, four rows per store.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t lds_w = lds_s + (32 * qb) * 256;
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const u32x2_t w = {pack_bf16x2(oacc[db][4 * grp + 0] * inv, oacc[db][4 * grp + 1] * inv),
                               pack_bf16x2(oacc[db][4 * grp + 2] * inv, oacc[db][4 * grp + 3] * inv)};
            const uint32_t a = lds_w + l32 * 256 + 16 * ((4 * db + grp) ^ (l32 & 15)) + 8 * hh;
            *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)a = w;
        }
    {
        const int pc = lane & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            const uint32_t a = lds_w + r * 256 + 16 * pc;
            const u32x4_t v = *(__attribute__((address_space(3))) const u32x4_t*)(uintptr_t)a;
            const int t = 32 * qb + r;
            if (seq_valid && t < T) {
                uint16_t* op = p.out + (long long)(t * S + s) * row_stride + (long long)head * D +
                               8 * (pc ^ (r & 15));
                *reinterpret_cast<uint4*>(op) = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_temporal_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* kt,
                                     const uint16_t* vs, uint16_t* out, const float2* table,
                                     const RopeGeom& g, int heads, hipStream_t stream) {
    const long long tensor_bytes = (long long)g.Nv * heads * D * 2;
    if (g.T <= SHORT_T && tensor_bytes < (1ll << 31)) {
        ShortParams sp;
        sp.q = q;
        sp.kt = kt;
        sp.vs = vs;
        sp.out = out;
        sp.table = table;
        sp.g = g;
        sp.heads = heads;
        sp.n_seq = g.S * heads;
        sp.k_tiles = (g.S + 63) / 64;
        sp.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
        const int blocks = (sp.n_seq + SHORT_WAVES - 1) / SHORT_WAVES;
        hipLaunchKernelGGL(attn_temporal_short_kernel, dim3(blocks), dim3(SHORT_WAVES * 64), 0, stream, sp);
        return hipGetLastError();
    }
    if (g.T <= MID_T && tensor_bytes < (1ll << 31)) {
        ShortParams sp;
        sp.q = q;
        sp.kt = kt;
        sp.vs = vs;
        sp.out = out;
        sp.table = table;
        sp.g = g;
        sp.heads = heads;
        sp.n_seq = g.S * heads;
        sp.k_tiles = (g.S + 63) / 64;
        sp.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
        const int blocks = (sp.n_seq + MID_SEQS - 1) / MID_SEQS;
        hipLaunchKernelGGL(attn_temporal_mid_kernel, dim3(blocks), dim3(MID_SEQS * 2 * 64), 0, stream, sp);
        return hipGetLastError();
    }
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
