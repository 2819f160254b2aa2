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
// How K reaches the kernel (template flag FUSED):
//  * staged (default): a preparation kernel rotates K once per key into fp16 tiles
//    [head][segment][tile][64][128]; the attention kernel copies them into LDS untouched.
//  * FUSED: K tiles are read from the caller's [N][heads][128] tensor and rotated (position
//    decoded from the flat row index) on every tile load, through registers.
// Q is rotated inside the attention kernel in both modes (once per workgroup); V is never
// rotated and is read straight from the caller's tensor.
//
// Design (one workgroup = 8 waves = 256 query rows of one head and one sequence):
//  * Scores are formed transposed, S^T = K~ Q~^T: a lane owns one query column and 16 keys per
//    32x32 block, so the softmax row max and row sum are in-lane plus one exchange between the
//    two 32-lane halves (v_permlane32_swap).
//  * Tiles of 64 keys move HBM -> LDS with global_load_lds_dwordx4 (no registers, no VALU) into
//    four LDS buffers; the copy of tile j+3 is in flight while tile j is consumed, one barrier per
//    tile.  16-byte chunks are XOR-swizzled by row so that every LDS read below is free of bank
//    conflicts without padding (the DMA writes each 1 KB block linearly).
//  * The PV product needs V with keys along each lane's operand; ds_read_b64_tr_b16 reads the
//    row-major V tile transposed, so V needs no staging pass and no VALU transpose.  The key
//    order inside each 16 keys matches the order in which the score accumulator hands P^T over
//    as the B operand (keys 4h..4h+3 then 8+4h..8+4h+3 for lane half h).
//  * The score product of tile j+1 is issued before the softmax of tile j, so the MFMA pipe has
//    work while the VALU computes exponentials.  The loop is unrolled by the buffer count so all
//    LDS addresses are a per-lane base plus an immediate.
//  * Online softmax with a lazily updated running max: the accumulator is rescaled only when a
//    row max exceeds the stored one by more than 2^8 (exact in any case; the stored max is only
//    an offset for the exponentials).
#include <type_traits>

#include "st_internal.h"

namespace st {
namespace {

constexpr int D = 128;          // head dimension
constexpr int BM = 256;         // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 512;   // 8 waves
constexpr int NBUF = 4;
constexpr int TILE_BYTES = BN * D * 2;           // 16 KB, one K~ or V tile
constexpr int V_LDS_BASE = NBUF * TILE_BYTES;    // K tiles first, then V tiles
constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES; // 128 KB
constexpr float LAZY_LOG2 = 8.0f;  // rescale when the max grows by more than this (log2 units)

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const void gptr_t;

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;     // staged: K~ tiles (fp16); FUSED: K [N][heads][D] bf16
    const uint16_t* v;     // V [N][heads][D] bf16
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
    uint16_t* kt;          // [heads][n_segs][k_tiles][BN][D] fp16
    const float2* table;
    RopeGeom g;
    int heads;
    int seg_len;
    int n_segs;
    int k_tiles;
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

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

// Swizzles: physical 16-byte chunk of logical chunk c in row r of a 256-byte tile row.
__device__ __forceinline__ int k_swz(int r) { return r & 7; }
__device__ __forceinline__ int v_swz(int r) { return (r & 3) << 1; }

__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_byte) {
    __builtin_amdgcn_global_load_lds((gptr_t*)src, (lds_u8*)(uintptr_t)lds_byte, 16, 0, 0);
}

template <int B> using Buf = std::integral_constant<int, B>;

template <bool FUSED>
__global__ void __launch_bounds__(NTHREADS, 1) attn_fwd_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const RopeGeom& g = p.g;

    // ---- tile copies ------------------------------------------------------------------------
    // Wave w, copy i in {0,1}: rows r = 8w + 4i + lane/16, physical chunk lane%16 of that row.
    const int dr0 = 8 * wave + (lane >> 4);
    const int pc = lane & 15;
    const uint16_t* vhead = p.v + (long long)head * D;
    const long long ktile0 = ((long long)head * p.n_segs + seg) * ntiles;
    int k_src_off[2];   // staged: element offset inside a K~ tile
    int v_chunk[2];     // element offset of the lane's logical chunk inside a V row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = dr0 + 4 * i;
        k_src_off[i] = r * D + 8 * (pc ^ k_swz(r));
        v_chunk[i] = 8 * (pc ^ v_swz(r));
    }
    // FUSED K copy through registers: thread owns chunks c = tid & 15 of rows tid>>4 and +32.
    const int fkc = tid & 15;
    const int fkr = tid >> 4;
    uint4 fk0 = make_uint4(0, 0, 0, 0), fk1 = make_uint4(0, 0, 0, 0);

    auto issue_tile = [&](int j, int buf) {
        const uint32_t kl = lds0 + buf * TILE_BYTES + (8 * wave) * 256;
        const uint32_t vl = lds0 + V_LDS_BASE + buf * TILE_BYTES + (8 * wave) * 256;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int key = j * BN + dr0 + 4 * i;
            key = key < seg_len ? key : seg_len - 1;   // rows past the end repeat the last row
            dma16(vhead + (seg_base + key) * row_stride + v_chunk[i], vl + i * 1024);
        }
        if constexpr (!FUSED) {
            const uint16_t* kt = p.k + (ktile0 + j) * (BN * D);
#pragma unroll
            for (int i = 0; i < 2; ++i) dma16(kt + k_src_off[i], kl + i * 1024);
        } else {
            const uint16_t* kh = p.k + (long long)head * D;
            const int k0 = j * BN + fkr, k1 = k0 + 32;
            fk0 = k0 < seg_len ? ld16(kh + (seg_base + k0) * row_stride + 8 * fkc) : make_uint4(0, 0, 0, 0);
            fk1 = k1 < seg_len ? ld16(kh + (seg_base + k1) * row_stride + 8 * fkc) : make_uint4(0, 0, 0, 0);
        }
    };
    // FUSED only: rotate the registers fetched by issue_tile(j, buf) and write them to LDS.
    auto finish_tile = [&](int j, int buf) {
        if constexpr (FUSED) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = fkr + 32 * i;
                const int n = seg_base + j * BN + r;
                int t = 0, h = 0, w = 0;
                const bool text = n >= g.Nv;
                if (!text) decode_pos(n, g, t, h, w);
                uint4 rot = rope_chunk_f16(i == 0 ? fk0 : fk1, fkc, t, h, w, text, g, p.table);
                const uint32_t a = lds0 + buf * TILE_BYTES + r * 256 + 16 * (fkc ^ k_swz(r));
                const u32x4_t rv = {rot.x, rot.y, rot.z, rot.w};
                *(__attribute__((address_space(3))) u32x4_t*)(uintptr_t)a = rv;
            }
        } else {
            (void)j;
            (void)buf;
        }
    };

    // ---- prologue -----------------------------------------------------------------------------
    issue_tile(0, 0);
    finish_tile(0, 0);
    if (ntiles > 1) { issue_tile(1, 1); finish_tile(1, 1); }
    if (ntiles > 2) { issue_tile(2, 2); finish_tile(2, 2); }

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
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // ---- per-lane LDS read addresses -------------------------------------------------------------
    // K operand of the score product: row l32 (+32 for the second block), logical chunk 2ks + hh.
    uint32_t k_rd[4];
    {
        const int x = l32 & 7;
#pragma unroll
        for (int t = 0; t < 4; ++t)
            k_rd[t] = lds0 + l32 * 256 + 16 * (((2 * t) ^ (x & 6)) + ((hh ^ x) & 1));
    }
    // V operand of the PV product, read transposed: lane (i = lane%16, g = lane/16) points at row
    // 4*(g/2) + i/4 (+ 16 per key chunk, + 8 for the upper half), channels 16*(g%2) + 4*(i%4).
    uint32_t v_rd[2];
    {
        const int i = lane & 15, gq = lane >> 4;
        const int row = 4 * (gq >> 1) + (i >> 2);
        const int u = 2 * (gq & 1) + ((i & 3) >> 1);
        const int ph = u ^ v_swz(row);
        v_rd[0] = lds0 + V_LDS_BASE + row * 256 + 16 * ph + 8 * (i & 1);
        v_rd[1] = lds0 + V_LDS_BASE + row * 256 + 16 * (ph ^ 4) + 8 * (i & 1);
    }

    auto qk = [&](auto bufc, f32x16_t (&s)[2]) {
        constexpr int b = decltype(bufc)::value;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const uint32_t a = k_rd[ks & 3] + b * TILE_BYTES + (ks >> 2) * 128 + mb * 32 * 256;
                f16x8_t op = *(__attribute__((address_space(3))) const f16x8_t*)(uintptr_t)a;
                s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op, qreg[ks], s[mb], 0, 0, 0);
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
    // formed into sn and tile j+3 is copied into LDS.
    auto step = [&](auto bufc, int j, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
        constexpr int b = decltype(bufc)::value;
        constexpr int b1 = (b + 1) % NBUF;
        constexpr int b3 = (b + 3) % NBUF;
        const bool issue = j + 3 < ntiles;
        if (issue) issue_tile(j + 3, b3);
        if (j + 1 < ntiles) qk(Buf<b1>{}, sn);

        if (ragged && j == ntiles - 1) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = j * BN + 32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key >= seg_len) sc[mb][i] = -INFINITY;
                }
        }
        float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[0][i]), sc[0][i + 1]);
        mx = fmaxf(mx, sc[0][15]);
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[1][i]), sc[1][i + 1]);
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
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint32_t a = v_rd[db & 1] + b * TILE_BYTES + (db >> 1) * 128 + c * 16 * 256;
                i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a);
                i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)(a + 8 * 256));
                const bf16x8_t op = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb[c], oacc[db], 0, 0, 0);
            }
        if constexpr (FUSED) {
            if (issue) finish_tile(j + 3, b3);
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        } else {
            // Tile j+2 (issued one step earlier) must have landed; tile j+3 may stay in flight.
            if (issue) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    f32x16_t sa[2], sb[2];
    qk(Buf<0>{}, sa);
    for (int j = 0; j < ntiles; j += 4) {
        step(Buf<0>{}, j, sa, sb);
        if (j + 1 >= ntiles) break;
        step(Buf<1>{}, j + 1, sb, sa);
        if (j + 2 >= ntiles) break;
        step(Buf<2>{}, j + 2, sa, sb);
        if (j + 3 >= ntiles) break;
        step(Buf<3>{}, j + 3, sb, sa);
    }

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

// Staging for the default mode: one workgroup per (head, segment, key tile) rotates the tile's
// 64 K rows into fp16.  Rows past the segment are written as zeros.
__global__ void __launch_bounds__(256) k_prep_kernel(PrepParams p) {
    const int tile = blockIdx.x;
    const int kt = tile % p.k_tiles;
    const int rest = tile / p.k_tiles;
    const int seg = rest % p.n_segs;
    const int head = rest / p.n_segs;
    const long long row_stride = (long long)p.heads * D;
    const RopeGeom& g = p.g;
    uint16_t* out = p.kt + (long long)tile * (BN * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = threadIdx.x + 256 * i;
        const int r = id >> 4, c = id & 15;
        const int kl = kt * BN + r;
        const bool valid = kl < p.seg_len;
        const int n = seg * p.seg_len + (valid ? kl : 0);
        uint4 raw = valid ? ld16(p.k + n * row_stride + (long long)head * D + 8 * c) : make_uint4(0, 0, 0, 0);
        int t = 0, h = 0, w = 0;
        const bool text = n >= g.Nv;
        if (!text) decode_pos(n, g, t, h, w);
        *reinterpret_cast<uint4*>(out + r * D + 8 * c) = rope_chunk_f16(raw, c, t, h, w, text, g, p.table);
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

template <bool FUSED>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(attn_fwd_kernel<FUSED>, dim3(p.total_wg), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t attn_stage_elems(int heads, int seg_len, int n_segs) {
    const size_t k_tiles = (size_t)(seg_len + BN - 1) / BN;
    return (size_t)heads * n_segs * k_tiles * BN * D;
}

hipError_t launch_k_prep(const uint16_t* k, uint16_t* kt, const float2* table, const RopeGeom& g,
                         int heads, int seg_len, int n_segs, hipStream_t stream) {
    PrepParams p;
    p.k = k;
    p.kt = kt;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.seg_len = seg_len;
    p.n_segs = n_segs;
    p.k_tiles = (seg_len + BN - 1) / BN;
    const int blocks = heads * n_segs * p.k_tiles;
    hipLaunchKernelGGL(k_prep_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_staged(const uint16_t* q, const uint16_t* kt, const uint16_t* v,
                                   uint16_t* out, const float2* table, const RopeGeom& g,
                                   int heads, int seg_len, int n_segs, hipStream_t stream) {
    return launch<false>(make_params(q, kt, v, out, table, g, heads, seg_len, n_segs), stream);
}

hipError_t launch_attn_bf16_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* out, const float2* table, const RopeGeom& g,
                                  int heads, int seg_len, int n_segs, hipStream_t stream) {
    return launch<true>(make_params(q, k, v, out, table, g, heads, seg_len, n_segs), stream);
}

}  // namespace st
