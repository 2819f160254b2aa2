// QKV projection with the 3D rotation fused into its epilogue.
//
// The step before the attention in a video DiT block ("04 · HunyuanVideo 与 Wan", section 3.1:
// Q = X W_Q, K = X W_K, V = X W_V; the first page's cost model counts it in the linear layers):
// y = x W^T + bias for x [N][C] and W [3C][C] (output features by input features, the usual
// layout of a linear layer's weight), then q and k are turned by each row's 3D RoPE ("A video
// model's architecture", "Position: RoPE in three dimensions") before they are stored.  Writing
// rotated q and k once here leaves the attention nothing to rotate.
//
// bf16 kernel (MFMA): one workgroup of 8 waves computes a 256-token x 256-feature tile of y^T
// (features as rows, so that each lane holds 4 consecutive features of one token: a RoPE pair is
// in-lane).  Wave w takes features 64 (w % 4) .. +63 and tokens 128 (w / 4) .. +127: 2 x 4 blocks
// of 32 x 32.  K advances 64 at a time through two LDS stages (x tile and W tile, 32 KB each),
// copied by LDS DMA one stage ahead of the MFMAs.  The output tile goes through LDS so that rows
// are written whole.
#include <type_traits>

#include "st_internal.h"

namespace st {
namespace {

constexpr int GM = 256;                     // tokens per tile
constexpr int GN = 256;                     // output features per tile
constexpr int GK = 64;                      // input features per stage
constexpr int G_TILE = GM * GK * 2;         // 32 KB: one x or W tile of a stage
constexpr int G_STAGE = 2 * G_TILE;         // x tile, then W tile
constexpr int G_LDS = 2 * G_STAGE;          // two stages; the output tile reuses all of it
constexpr int G_TABLE = 4096;               // rotation table entries kept in LDS (32 KB) when they fit
constexpr int GTHREADS = 512;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

struct QkvParams {
    const uint16_t* x;
    const uint16_t* w;
    const uint16_t* bias;   // [3C] or null
    uint16_t* q;
    uint16_t* k;
    uint16_t* v;
    const float2* table;
    RopeGeom g;
    int n_rows;
    int C;
    int m_tiles;
    int n_tiles;
    int total_wg;
};

// 16-byte chunk c of a 128-byte tile row r sits at physical chunk c ^ ((r >> 1) & 7): the 16
// lanes of a 16-byte read (16 consecutive rows, one chunk) then cover all 64 banks.
__device__ __forceinline__ int g_swz(int r) { return (r >> 1) & 7; }

__global__ void __launch_bounds__(GTHREADS, 1) qkv_rope_bf16_kernel(QkvParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[G_LDS];
    __shared__ __attribute__((aligned(16))) float2 lds_table[G_TABLE];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;

    // Tile order: each XCD takes a contiguous run of logical ids (xcd_remap), and consecutive ids
    // walk GROUP token tiles for one feature tile before the next feature tile, so the 32 tiles
    // an XCD runs at once share 8 x panels and 4 W panels through its L2.
    const int logical = xcd_remap(blockIdx.x, p.total_wg);
    constexpr int GROUP = 8;
    const int per_group = GROUP * p.n_tiles;
    const int grp = logical / per_group;
    const int first_m = grp * GROUP;
    const int gsize = min(p.m_tiles - first_m, GROUP);
    const int in_grp = logical - grp * per_group;
    const int mt = first_m + in_grp % gsize;
    const int nt = in_grp / gsize;
    const int m0 = mt * GM;                  // first token
    const int f0 = nt * GN;                  // first output feature
    const int C = p.C;
    const int F = 3 * C;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int fg = wave & 3;
    const int tg = wave >> 2;

    // ---- stage copies: wave w copies rows 32 w .. +31 of the x tile and of the W tile --------
    uint32_t x_off[4], w_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 32 * wave + 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ g_swz(r);
        const int tr = min(m0 + r, p.n_rows - 1);      // rows past the end repeat the last row
        const int fr = min(f0 + r, F - 1);
        x_off[i] = 2u * (uint32_t)(tr * C + 8 * c);
        w_off[i] = 2u * (uint32_t)(fr * C + 8 * c);
    }
    auto issue_stage = [&](int ks, int stage) {
        const uint16_t* xb = p.x + ks * GK;
        const uint16_t* wb = p.w + ks * GK;
        const uint32_t sb = lds0 + stage * G_STAGE + (32 * wave) * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(xb, x_off[i], sb + i * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(wb, w_off[i], sb + G_TILE + i * 1024);
    };

    // ---- operand reads -------------------------------------------------------------------------
    // A (W rows = features) for feature block fb, B (x rows = tokens) for token block tb, k16
    // step kk: row l32 of the block, logical chunk 2 kk + hh.
    uint32_t a_rd[2], b_rd[4];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) a_rd[fb] = lds0 + G_TILE + (64 * fg + 32 * fb + l32) * 128;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) b_rd[tb] = lds0 + (128 * tg + 32 * tb + l32) * 128;
    const int rsw = g_swz(l32);   // rows of a block start at multiples of 32: same swizzle
    auto rd = [&](uint32_t base, int stage, int kk) -> bf16x8_t {
        const uint32_t a = base + stage * G_STAGE + 16 * ((2 * kk + hh) ^ rsw);
        return *(__attribute__((address_space(3))) const bf16x8_t*)(uintptr_t)a;
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[fb][tb][i] = 0.0f;

    const int ksteps = C / GK;   // C is a multiple of 128: ksteps is even and at least 2
    // The rotation table goes into LDS by DMA before the first stages (so the wait for stage 0
    // covers it too): the epilogue then reads its 64 entries per lane from LDS instead of
    // gathering them from memory behind a wait per batch (8.5 us of a 54 us tile before).  The
    // table's allocation is 256-byte aligned, so whole 16-byte chunks stay inside it.
    const bool table_in_lds = p.g.identity < G_TABLE;
    if (table_in_lds) {
        const int chunks = (p.g.identity + 2) / 2;   // 16-byte chunks of identity + 1 entries
        const uint32_t tl = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float2*)lds_table;
        for (int r = 0; r * GTHREADS < chunks; ++r) {
            const int c = r * GTHREADS + tid;
            if (c < chunks) dma16(p.table, 16u * (uint32_t)c, tl + 16u * (uint32_t)(r * GTHREADS + 64 * wave));
        }
    }
    // Stages 0 and 1 in flight; stage 0 must land before the first reads.
    issue_stage(0, 0);
    issue_stage(1, 1);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // Operand double buffer; k16 step kk of a stage uses buffer kk & 1.
    bf16x8_t a[2][2], b[2][4];
    auto read_ops = [&](int buf, int stage, int kk) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) a[buf][fb] = rd(a_rd[fb], stage, kk);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) b[buf][tb] = rd(b_rd[tb], stage, kk);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][fb], b[buf][tb], acc[fb][tb], 0, 0, 0);
    };
    auto interleave = [&]() {   // 8 MFMAs with the 6 reads issued beside them
#pragma unroll
        for (int t = 0; t < 6; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    read_ops(0, 0, 0);

    // Step ks (stage st): k16 steps 0-2 with the next one's operands read beside them; then the
    // stage's reads and the next stage's copies are complete, the barrier releases the slot, the
    // copies of stage ks+2 go into it, and k16 step 3 runs beside the reads of stage ks+1's first
    // operands.  The barrier is crossed with 8 MFMAs in flight, and no step starts by waiting on
    // LDS.  After the last step those reads fetch a stale slot (in bounds, never used): a branch
    // around them would keep two operand sets live across it and spill.
    auto step = [&](auto stc, int ks) {
        constexpr int st = decltype(stc)::value;
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
            read_ops((kk + 1) & 1, st, kk + 1);
            mfmas(kk & 1);
            interleave();
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ks + 2 < ksteps) issue_stage(ks + 2, st);
        read_ops(0, st ^ 1, 0);
        mfmas(1);
        interleave();
    };
    for (int ks = 0; ks < ksteps; ks += 2) {
        step(std::integral_constant<int, 0>{}, ks);
        step(std::integral_constant<int, 1>{}, ks + 1);
    }

    // ---- epilogue: bias, rotation of q and k, bf16, through LDS to whole rows ------------------
    // Lane (l32, hh) holds, for block (fb, tb), token 128 tg + 32 tb + l32 and features
    // 64 fg + 32 fb + 8 (i / 4) + 4 hh + i % 4 of the tile.
    const RopeGeom& g = p.g;
    // The lane's 32 features are the same for all four token blocks: their bias is loaded once.
    // Tiles that end inside the last output feature (heads odd) test each load.
    uint2 bw[2][4];
    const bool bias_full = p.bias != nullptr && f0 + GN <= F;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int f = f0 + 64 * fg + 32 * fb + 8 * gi + 4 * hh;
            bw[fb][gi] = make_uint2(0u, 0u);
            if (bias_full)
                bw[fb][gi] = *reinterpret_cast<const uint2*>(p.bias + f);
            else if (p.bias != nullptr && f < F)
                bw[fb][gi] = *reinterpret_cast<const uint2*>(p.bias + f);
        }
    // A tile's 256 features are all q and k features (rotated) or all v features: 2C = heads x 256
    // is a multiple of the tile width, so the choice is one branch per workgroup.
    const int f1 = __builtin_amdgcn_readfirstlane(g.first[1]);
    const int f2 = __builtin_amdgcn_readfirstlane(g.first[2]);
    const int o0 = __builtin_amdgcn_readfirstlane(g.off[0]);
    const int o1 = __builtin_amdgcn_readfirstlane(g.off[1]);
    const int o2 = __builtin_amdgcn_readfirstlane(g.off[2]);
    const int s0 = __builtin_amdgcn_readfirstlane(g.pairs[0]);
    const int s1 = __builtin_amdgcn_readfirstlane(g.pairs[1]);
    const int s2 = __builtin_amdgcn_readfirstlane(g.pairs[2]);
    const int lane_p = 32 * (fg & 1) + 2 * hh;
    const int g1 = f1 - lane_p, g2 = f2 - lane_p;
    auto finish = [&](auto rotc) {
        constexpr bool ROT = decltype(rotc)::value;
        // Pair entries of token block tb for this lane's features.  The lane's pairs are
        // lane_p + 16 fb + 4 gi + e of the head (lane_p = 32 (fg % 2) + 2 hh), the same for every
        // token: per token the three axis bases are formed once, and each pair costs two compares,
        // two selects and an add.  Text rows take position (0, 0, 0), where every angle is 0.
        auto load_cs = [&](int tb, float2 (&cs)[2][4][2]) {
            if constexpr (ROT) {
                const int row = 128 * tg + 32 * tb + l32;
                const int n = min(m0 + row, p.n_rows - 1);
                const bool text = n >= g.Nv;
                int t, h, w;
                decode_pos(text ? 0 : n, g, t, h, w);
                const int bt = o0 + (int)__umul24((unsigned)t, (unsigned)s0) + lane_p;
                const int bh = o1 - f1 + (int)__umul24((unsigned)h, (unsigned)s1) + lane_p;
                const int bw = o2 - f2 + (int)__umul24((unsigned)w, (unsigned)s2) + lane_p;
                if (table_in_lds) {
#pragma unroll
                    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const int k = 16 * fb + 4 * gi + e;
                                const int base = k >= g2 ? bw : (k >= g1 ? bh : bt);
                                cs[fb][gi][e] = lds_table[base + k];
                            }
                } else {
#pragma unroll
                    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const int k = 16 * fb + 4 * gi + e;
                                const int base = k >= g2 ? bw : (k >= g1 ? bh : bt);
                                cs[fb][gi][e] = p.table[base + k];
                            }
                }
            } else {
                (void)tb;
                (void)cs;
            }
        };
        auto block = [&](int tb, const float2 (&cs)[2][4][2]) {
            const int row = 128 * tg + 32 * tb + l32;     // token row inside the tile
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int fl = 64 * fg + 32 * fb + 8 * gi + 4 * hh;   // first of 4 features, in tile
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[fb][tb][4 * gi + e];
                    y[0] += bf16_lo(bw[fb][gi].x);
                    y[1] += bf16_hi(bw[fb][gi].x);
                    y[2] += bf16_lo(bw[fb][gi].y);
                    y[3] += bf16_hi(bw[fb][gi].y);
                    if constexpr (ROT) {   // q or k: rotate pairs (f, f+1), (f+2, f+3)
#pragma unroll
                        for (int e = 0; e < 2; ++e) rotate_pair(y[2 * e], y[2 * e + 1], cs[fb][gi][e]);
                    }
                    const u32x2_t pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
                    const uint32_t a = lds0 + row * 512 + 16 * ((fl >> 3) ^ (row & 31)) + 8 * hh;
                    *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)a = pk;
                }
        };
        // Table entries of token block tb + 1 are loaded while block tb is rotated and stored.
        float2 csa[2][4][2], csb[2][4][2];
        load_cs(0, csa);
        load_cs(1, csb);
        block(0, csa);
        load_cs(2, csa);
        block(1, csb);
        load_cs(3, csb);
        block(2, csa);
        block(3, csb);
    };
    if (f0 < 2 * C)
        finish(std::true_type{});
    else
        finish(std::false_type{});
    __syncthreads();
    // Wave w writes tile rows 32 w .. +31, two rows (2 x 512 bytes) per store.
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int row = 32 * wave + 2 * i + (lane >> 5);
        const int c = lane & 31;                       // logical 16-byte chunk: features 8c .. 8c+7
        const u32x4_t val = *(__attribute__((address_space(3))) const u32x4_t*)(uintptr_t)(
            lds0 + row * 512 + 16 * (c ^ (row & 31)));
        const int n = m0 + row;
        const int f = f0 + 8 * c;
        if (n < p.n_rows && f < F) {
            const int sec = f / C;
            uint16_t* dst = (sec == 0 ? p.q : (sec == 1 ? p.k : p.v)) + (long long)n * C + (f - sec * C);
            *reinterpret_cast<uint4*>(dst) = make_uint4(val[0], val[1], val[2], val[3]);
        }
    }
}

// ---- float32 checking kernel: 64 x 64 output tiles, 4 x 4 per thread ---------------------------
struct QkvF32Params {
    const float* x;
    const float* w;
    const float* bias;
    float* q;
    float* k;
    float* v;
    const float2* table;
    RopeGeom g;
    int n_rows;
    int C;
    int d;
};

__global__ void __launch_bounds__(256) qkv_rope_f32_kernel(QkvF32Params p) {
    __shared__ float xs[16][64 + 1];
    __shared__ float ws[16][64 + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m0 = blockIdx.y * 64, f0 = blockIdx.x * 64;
    const int C = p.C, F = 3 * C;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
    for (int k0 = 0; k0 < C; k0 += 16) {
        for (int idx = threadIdx.x; idx < 16 * 64; idx += 256) {
            const int r = idx >> 4, kk = idx & 15;
            const int n = m0 + r, f = f0 + r, kc = k0 + kk;
            xs[kk][r] = (n < p.n_rows && kc < C) ? p.x[(long long)n * C + kc] : 0.0f;
            ws[kk][r] = (f < F && kc < C) ? p.w[(long long)f * C + kc] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(xs[kk][4 * ty + a], ws[kk][4 * tx + b], acc[a][b]);
        __syncthreads();
    }
    const RopeGeom& g = p.g;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int n = m0 + 4 * ty + a;
        if (n >= p.n_rows) continue;
        int t = 0, h = 0, w = 0;
        const bool text = n >= g.Nv;
        if (!text) decode_pos(n, g, t, h, w);
        float y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int f = f0 + 4 * tx + b;
            y[b] = acc[a][b] + ((p.bias && f < F) ? p.bias[f] : 0.0f);
        }
        const int fb = f0 + 4 * tx;               // 4 features, fb even: pairs (fb, fb+1), (fb+2, fb+3)
        if (fb < 2 * C) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int f = fb + 2 * e;
                const int pair = (f % p.d) >> 1;
                rotate_pair(y[2 * e], y[2 * e + 1], p.table[pair_entry(pair, t, h, w, g)]);
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int f = fb + b;
            if (f >= F) continue;
            const int sec = f / C;
            float* dst = sec == 0 ? p.q : (sec == 1 ? p.k : p.v);
            dst[(long long)n * C + (f - sec * C)] = y[b];
        }
    }
}

}  // namespace

hipError_t launch_qkv_rope_bf16(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                                uint16_t* q, uint16_t* k, uint16_t* v, const float2* table,
                                const RopeGeom& g, int n_rows, int C, hipStream_t stream) {
    QkvParams p;
    p.x = x;
    p.w = w;
    p.bias = bias;
    p.q = q;
    p.k = k;
    p.v = v;
    p.table = table;
    p.g = g;
    p.n_rows = n_rows;
    p.C = C;
    p.m_tiles = (n_rows + GM - 1) / GM;
    p.n_tiles = (3 * C + GN - 1) / GN;
    p.total_wg = p.m_tiles * p.n_tiles;
    hipLaunchKernelGGL(qkv_rope_bf16_kernel, dim3(p.total_wg), dim3(GTHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_qkv_rope_f32(const float* x, const float* w, const float* bias, float* q, float* k,
                               float* v, const float2* table, const RopeGeom& g, int n_rows, int C,
                               int d, hipStream_t stream) {
    QkvF32Params p;
    p.x = x;
    p.w = w;
    p.bias = bias;
    p.q = q;
    p.k = k;
    p.v = v;
    p.table = table;
    p.g = g;
    p.n_rows = n_rows;
    p.C = C;
    p.d = d;
    dim3 grid((3 * C + 63) / 64, (n_rows + 63) / 64);
    hipLaunchKernelGGL(qkv_rope_f32_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace st
