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
// (f16 MFMAs, same rate as bf16); q is multiplied by log2(e)/sqrt(128) before that rounding, so
// scores come out in log2 units.  Softmax weights are rounded to bf16 and multiply the exact bf16
// values (bf16 MFMAs); accumulation, the running max and the row sums are fp32, and the row sum
// adds exactly the rounded weights the product used.  (bf16 q and k would make the score product
// cheaper, but their rounding alone takes the Wan-14B-shaped 720p inputs, whose rows are scaled
// by U(0.5, 2), past a relative L2 error of 5e-3.)
//
// How K reaches the kernel (template flag FUSED):
//  * staged (default): a preparation kernel rotates K once per key into fp16 tiles
//    [head][segment][tile][64][128]; the attention kernel copies them into LDS untouched.
//  * FUSED: K tiles are read from the caller's [N][heads][128] tensor and rotated (position
//    decoded from the flat row index) on every tile load, through registers.
// Q is rotated inside the attention kernel in both modes (once per workgroup); V is never
// rotated and is read straight from the caller's tensor.
//
// Window mode (template flag WIN, staged K): the sequences are the local 3D windows of the grid
// (the CogVideoX record page, "Conditions", local 3D-window blocks); each lane maps its window-
// local row to a grid row for the Q load, the V tile copy and the output store, and the staging
// kernel does the same for K.
//
// Design (one item = 256 query rows of one head and one sequence, taken by a workgroup of 8 waves;
// the launch is persistent: one workgroup per CU loops over items).  Two kernels share it: the
// fast launch (attn_fast_kernel, 16x16x32 blocks, fixed score offset) and the running-max kernel
// (attn_fwd_kernel, 32x32x16 blocks), which is the guard of the fast launch and serves every
// other path.
//  * Scores are formed transposed, S^T = K~ Q~^T: a lane owns query columns and a few keys of
//    each block, so the softmax row max and row sum are in-lane plus exchanges between lane
//    groups (v_permlane32_swap, and v_permlane16_swap for the 16-lane groups of 16x16 blocks).
//  * Tiles of 64 keys move HBM -> LDS with global_load_lds_dwordx4 (no registers, no VALU) into
//    four LDS buffers; the copy of tile j+3 is in flight while tile j is consumed, one barrier per
//    tile.  16-byte chunks are XOR-swizzled by row so that every LDS read below is free of bank
//    conflicts without padding (the DMA writes each 1 KB block linearly).
//  * The PV product needs V with keys along each lane's operand; ds_read_b64_tr_b16 reads the
//    row-major V tile transposed, so V needs no staging pass and no VALU transpose.  The key
//    order inside the operand matches the order in which the score accumulator hands P^T over as
//    the B operand.
//  * The score product of tile j+1 is issued before the softmax of tile j, so the MFMA pipe has
//    work while the VALU computes exponentials.  The loop is unrolled by the buffer count so all
//    LDS addresses are a per-lane base plus an immediate.
//  * Online softmax with a lazily updated running max m: the accumulator is rescaled only when a
//    row max exceeds m by more than 8 (log2 units; exact in any case, m is only an offset for the
//    exponentials).  The score MFMAs start from -m instead of zero, so they return s - m and the
//    exponentials need no subtraction.
#include <type_traits>

#include "st_internal.h"

namespace st {
namespace {

constexpr int D = 128;          // head dimension
constexpr int BM = 256;         // query rows per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 512;   // 8 waves
constexpr int TILE_BYTES = BN * D * 2;           // 16 KB, one K~ or V tile
constexpr int NBUF = 4;                          // tile j lives in K and V slot j % NBUF
constexpr int PREF = 3;                          // step j fetches tile j + PREF
constexpr int KAHEAD = 6;                        // fast kernel: K~ operands read ahead of their MFMAs
constexpr int VAHEAD = 4;                        // fast kernel: V operands read ahead
constexpr int V_LDS_BASE = NBUF * TILE_BYTES;    // K slots first, then V slots
constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES; // 128 KB
constexpr int WIN_TABLE = 8192;                  // window mode: V row offsets kept in LDS (32 KB)
constexpr int LDS_TABLE = WIN_TABLE / 2;          // fast launch: rotation table entries kept in LDS
constexpr float OVF_SUM = 0x1p64f;   // fast launch: a row sum this large (or not finite) flags the item
constexpr float LAZY_LOG2 = 8.0f;  // move the offset when a row max exceeds it by more than this

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
    float* lse;            // optional [q rows][heads] log-sum-exp of the scaled scores
    int seg_len;           // key (and value) rows per sequence
    int q_len;             // query rows per sequence
    int n_segs;
    int q_pos_base;        // global row (for positions) of query buffer row 0
    int kv_pos_base;       // global row of key buffer row 0
    int q_tiles;
    int k_tiles;
    int total_wg;
    float scale_log2;      // log2(e) / sqrt(D)
    WinMap win;            // window mode only: segment s is window s, rows via win_origin/offset
    uint8_t* item_flags;   // 8 bytes per item: written by the fast launch, read by the guard launch
    // Key split (fast launch of staged self-attention only): with k_split = 2 every query tile
    // is two items, keys [0, split_tiles) and [split_tiles, k_tiles) of its sequence; the first
    // writes part_a and lse, the second part_b and lse_b (fp32, so that the result is rounded to
    // bf16 once, in the merge launch that combines them).  The guard launch (which never splits)
    // reads both items' flags.
    int k_split;
    int split_tiles;
    float* part_a;         // key split: each half's normalised output in fp32, [q rows][heads][D]
    float* part_b;
    float* lse_b;
};

struct PrepParams {
    const uint16_t* k;
    uint16_t* kt;          // [heads][n_segs][k_tiles][BN][D] fp16
    const float2* table;
    RopeGeom g;
    int heads;
    int seg_len;
    int n_segs;
    int kv_pos_base;
    int k_tiles;
    WinMap win;            // window mode only
    float2* table_fill;    // no video rows (g.Nv == 0): the table is written here, not read
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Rotate 8 bf16 channels (pairs 4c .. 4c+3) of a row at (t, h, w) and return them as fp16.
__device__ __forceinline__ uint4 rope_chunk_f16(uint4 raw, int c, int t, int h, int w,
                                                const RopeGeom& g, const float2* __restrict__ table,
                                                float scale = 1.0f) {
    uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float2 cs = table[pair_entry(4 * c + i, t, h, w, g)];
        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
        rotate_pair(x0, x1, cs);
        wd[i] = pack_f16x2(x0 * scale, x1 * scale);
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// Swizzles: logical 16-byte chunk c of tile row r (256 bytes) sits at physical chunk c ^ swz(r).
// gfx950 LDS serves 256 bytes per clock from 64 banks: 16 lanes of a 16-byte read or 32 lanes
// of an 8-byte read at a time.  The K operand read has 16 lanes on 16 consecutive rows at one
// logical chunk (both kernels).  The transposed V read of the running-max kernel has 32 lanes on
// 4 consecutive rows x 4 logical chunks (4db .. 4db+3); that of the fast kernel has 32 lanes on
// 8 consecutive rows (from a multiple of 8) x 2 logical chunks (2db, 2db+1), so its swizzle maps
// the 8 rows to 8 different chunk pairs.  With these swizzles each such group touches 16
// different physical chunks.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return (r & 3) << 2; }
__device__ __forceinline__ int v_swz16(int r) { return ((r & 3) << 2) | ((r >> 1) & 2); }

__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups).
__device__ __forceinline__ float xquad_max(float x) {
    x = xhalf_max(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xquad_sum(float x) {
    x = xhalf_sum(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int B> using Buf = std::integral_constant<int, B>;

// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002;
constexpr int SG_MFMA = 0x008;
constexpr int SG_DS_READ = 0x100;

// The running-max kernel: 32x32x16 score and PV blocks, the score offset following the lazy
// running max of every tile.  It serves cross-attention, partial attention, windows, the fused
// variant and short launches, and as the guard launch it redoes the items the fast launch flagged
// (p.item_flags non-null: only items whose 8 flag bytes are not all zero).
// WIN (staged K only): segment s is local window s of p.win, and query, value and output rows are
// the window's grid rows (win_origin + win_offset) instead of a contiguous run of buffer rows.
template <bool FUSED, bool WIN>
__global__ void __launch_bounds__(NTHREADS, 1) attn_fwd_kernel(AttnParams p) {
    static_assert(!(FUSED && WIN), "window mode reads staged K");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];
    __shared__ uint32_t win_vrow[WIN ? WIN_TABLE : 1];   // window mode: byte offset of each V row
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;

    // Guard launch: only the items the fast launch flagged.  Its flags are by item number, or,
    // after a key split (two items per query tile), by logical item: both halves are checked.
    auto flagged = [&](int item) {
        const unsigned long long* fl = reinterpret_cast<const unsigned long long*>(p.item_flags);
        if (p.k_split > 1) {
            const int logical = xcd_remap(item, p.total_wg);
            const int l0 = 2 * (logical - logical % p.q_tiles) + logical % p.q_tiles;
            return (fl[l0] | fl[l0 + p.q_tiles]) != 0;
        }
        return fl[item] != 0;
    };
    if (p.item_flags) {
        // The threads read the flags of all of the workgroup's items at once (one load latency
        // instead of one per item); a workgroup with nothing to redo ends here.
        int any = 0;
        for (int item = blockIdx.x + (int)threadIdx.x * (int)gridDim.x; item < p.total_wg;
             item += NTHREADS * (int)gridDim.x)
            any |= flagged(item) ? 1 : 0;
        // One vote per wave in the tile buffer (not yet in use; the LDS is otherwise full).
        uint32_t* const votes = reinterpret_cast<uint32_t*>(lds_raw);
        const bool wave_any = __ballot(any) != 0;
        if ((threadIdx.x & 63) == 0) votes[threadIdx.x >> 6] = wave_any ? 1u : 0u;
        __syncthreads();
        uint32_t all = 0;
#pragma unroll
        for (int w = 0; w < NTHREADS / 64; ++w) all |= votes[w];
        __syncthreads();   // every wave has read the votes before tile copies overwrite them
        if (!all) return;
    }

    // Persistent: workgroup b takes items b, b + G, b + 2G, ... (G = gridDim.x, a multiple of 8),
    // each through the XCD remap, so the items an XCD runs at one time are neighbouring tiles.
    for (int item = blockIdx.x; item < p.total_wg; item += gridDim.x) {
        const int logical = xcd_remap(item, p.total_wg);
        if (p.item_flags && !flagged(item)) continue;
        const int qt = logical % p.q_tiles;
        const int rest = logical / p.q_tiles;
        const int seg = rest % p.n_segs;
        const int head = rest / p.n_segs;
        const int seg_base = seg * p.seg_len;   // first key buffer row of the sequence
        const int win0 = WIN ? win_origin(seg, p.win) : 0;   // window mode: grid row of local row 0
        const int seg_len = p.seg_len;
        const int q_len = p.q_len;
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
        uint32_t k_src_off[2];   // staged: byte offset of the lane's chunk inside a K~ tile
        int v_chunk[2];          // element offset of the lane's logical chunk inside a V row
        uint32_t vch2[2];        // the same in bytes
        const uint32_t rs2 = 2u * (uint32_t)row_stride;   // bytes per V row (< 2^24)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = dr0 + 4 * i;
            k_src_off[i] = 2u * (uint32_t)(r * D + 8 * (pc ^ k_swz(r)));
            v_chunk[i] = 8 * (pc ^ v_swz(r));
            vch2[i] = 2u * (uint32_t)v_chunk[i];
        }
        // FUSED K copy through registers: thread owns chunks c = tid & 15 of rows tid>>4 and +32.
        const int fkc = tid & 15;
        const int fkr = tid >> 4;
        uint4 fk0 = make_uint4(0, 0, 0, 0), fk1 = make_uint4(0, 0, 0, 0);

        // issue_tile(j, slot): fetch tile j into K and V slot `slot`.
        auto issue_tile = [&](int j, int slot) {
            // The wave's LDS base passes through an empty asm so that the copies' LDS addresses are
            // formed here by scalar adds; hoisted out of the loop, their 16 values were spilled and
            // reloaded with VALU lane reads on every tile.
            uint32_t wl = lds0 + (8 * wave) * 256;
            asm volatile("" : "+s"(wl));
            const uint32_t kl = wl + slot * TILE_BYTES;
            const uint32_t vl = wl + V_LDS_BASE + slot * TILE_BYTES;
            const int last = seg_len - 1 - j * BN;   // rows past the end repeat the last row
            if constexpr (WIN) {
                // Each lane addresses its own grid row from the head's base (total bytes < 2^32):
                // from the item's table of row offsets, or by the window arithmetic past it.
                const bool from_table = j * BN + BN <= WIN_TABLE;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = dr0 + 4 * i;
                    const int re = r < last ? r : last;
                    const uint32_t rb = from_table ? win_vrow[j * BN + re]
                                                   : 2u * (uint32_t)(win0 + win_offset(j * BN + re, p.win)) * (uint32_t)row_stride;
                    dma16(vhead, rb + vch2[i], vl + i * 1024);
                }
            } else {
                const uint16_t* vt = vhead + (long long)(seg_base + j * BN) * row_stride;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = dr0 + 4 * i;
                    const int re = r < last ? r : last;
                    dma16(vt, __umul24((uint32_t)re, rs2) + vch2[i], vl + i * 1024);
                }
            }
            if constexpr (!FUSED) {
                const uint16_t* kt = p.k + (ktile0 + j) * (BN * D);
#pragma unroll
                for (int i = 0; i < 2; ++i) dma16(kt, k_src_off[i], kl + i * 1024);
            } else {
                const uint16_t* kh = p.k + (long long)head * D;
                const int k0 = j * BN + fkr, k1 = k0 + 32;
                fk0 = k0 < seg_len ? ld16(kh + (seg_base + k0) * row_stride + 8 * fkc) : make_uint4(0, 0, 0, 0);
                fk1 = k1 < seg_len ? ld16(kh + (seg_base + k1) * row_stride + 8 * fkc) : make_uint4(0, 0, 0, 0);
            }
        };
        // FUSED only: rotate the K registers fetched by issue_tile(j, slot) and write them to LDS.
        auto finish_tile = [&](int j, int slot) {
            if constexpr (FUSED) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = fkr + 32 * i;
                    const int n = p.kv_pos_base + seg_base + j * BN + r;
                    int t = 0, h = 0, w = 0;
                    const bool text = n >= g.Nv;
                    if (!text) decode_pos(n, g, t, h, w);
                    uint4 rot = rope_chunk_f16(i == 0 ? fk0 : fk1, fkc, t, h, w, g, p.table);
                    const uint32_t a = lds0 + slot * TILE_BYTES + r * 256 + 16 * (fkc ^ k_swz(r));
                    const u32x4_t rv = {rot.x, rot.y, rot.z, rot.w};
                    *(__attribute__((address_space(3))) u32x4_t*)(uintptr_t)a = rv;
                }
            } else {
                (void)j;
                (void)slot;
            }
        };

        // ---- prologue -----------------------------------------------------------------------------
        if constexpr (WIN) {
            // The window's V row offsets, once per item: the tile copies then read them instead of
            // doing two divisions per row and tile.  The previous item's copies were all issued
            // before its last barrier, so the table is free to overwrite.
            for (int li = tid; li < min(seg_len, WIN_TABLE); li += NTHREADS)
                win_vrow[li] = 2u * (uint32_t)(win0 + win_offset(li, p.win)) * (uint32_t)row_stride;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < PREF; ++j) {
            issue_tile(min(j, ntiles - 1), j);
            finish_tile(min(j, ntiles - 1), j);
        }

        const int q_local = qt * BM + wave * 32 + l32;
        const bool q_valid = q_local < q_len;
        const int q_row = WIN ? win0 + win_offset(q_valid ? q_local : 0, p.win)
                              : seg * q_len + (q_valid ? q_local : 0);   // query buffer row
        const int q_pos = p.q_pos_base + q_row;                    // its global row
        f16x8_t qreg[8];
        {
            // Lanes past the sequence read its first row (in bounds) and are never stored.  Pair p of
            // the row reads table entry base_a + p, a the axis p falls in: the three bases are formed
            // once per row, and each pair costs two compares and two selects.  Text rows take
            // position (0, 0, 0), where every angle is 0 (cos 1, sin 0 exactly): no rotation.
            const bool text = q_pos >= g.Nv;
            int t, h, w;
            decode_pos(text ? 0 : q_pos, g, t, h, w);
            const int f1 = __builtin_amdgcn_readfirstlane(g.first[1]);
            const int f2 = __builtin_amdgcn_readfirstlane(g.first[2]);
            const int lane_p = 4 * hh;   // this lane half's pairs are 8 ks + 4 hh + i
            const int bt = (int)__umul24((unsigned)t, (unsigned)g.pairs[0]) + lane_p;
            const int bh = g.off[1] - f1 + (int)__umul24((unsigned)h, (unsigned)g.pairs[1]) + lane_p;
            const int bw = g.off[2] - f2 + (int)__umul24((unsigned)w, (unsigned)g.pairs[2]) + lane_p;
            const int g1 = f1 - lane_p, g2 = f2 - lane_p;
            const float sc = p.scale_log2;
            const uint16_t* qp = p.q + q_row * row_stride + (long long)head * D + 8 * hh;
            uint4 raw[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) raw[ks] = ld16(qp + 16 * ks);
            if (g.Nv > 0) {
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const uint32_t wd[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
                    uint32_t o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int p0 = 8 * ks + i;
                        const int base = p0 >= g2 ? bw : (p0 >= g1 ? bh : bt);
                        const float2 cs = p.table[base + p0];
                        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
                        rotate_pair(x0, x1, cs);
                        o[i] = pack_f16x2(x0 * sc, x1 * sc);
                    }
                    qreg[ks] = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
                }
            } else {
                // No video rows (cross-attention): every angle is 0, so the rotation is the identity
                // and no table entry is read.
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const uint32_t wd[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
                    uint32_t o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = pack_f16x2(bf16_lo(wd[i]) * sc, bf16_hi(wd[i]) * sc);
                    qreg[ks] = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        // ---- per-lane LDS read addresses (slot 0; other slots add a multiple of TILE_BYTES) --------
        // K operand of the score product: row l32 (+32 for the second block), logical chunk 2ks + hh.
        uint32_t k_rd[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) k_rd[ks] = lds0 + l32 * 256 + 16 * ((2 * ks + hh) ^ k_swz(l32));
        // V operand of the PV product, read transposed: lane (i = lane%16, g = lane/16) points at row
        // 4*(g/2) + i/4 (+ 16 per key chunk, + 8 for the upper half) and channels 32 db + 16*(g%2) +
        // 4*(i%4), i.e. logical chunk 4 db + 2*(g%2) + (i%4)/2, byte 8*(i%2) inside it.
        uint32_t v_rd[4];
        {
            const int i = lane & 15, gq = lane >> 4;
            const int row = 4 * (gq >> 1) + (i >> 2);
            const int u = 2 * (gq & 1) + ((i & 3) >> 1);
#pragma unroll
            for (int db = 0; db < 4; ++db)
                v_rd[db] = lds0 + V_LDS_BASE + row * 256 + 16 * ((4 * db + u) ^ v_swz(row)) + 8 * (i & 1);
        }
        // K operand t (0..15) of the score product from K slot base kb (bytes): ks = t/2, block t%2.
        auto k_operand = [&](uint32_t kb, int t) -> f16x8_t {
            const int ks = t >> 1, mb = t & 1;
            const uint32_t a = k_rd[ks] + kb + mb * 32 * 256;
            return *(__attribute__((address_space(3))) const f16x8_t*)(uintptr_t)a;
        };
        // V operand of PV MFMA t (0..15) from V slot base vb: key chunk c = t/4, d block db = t%4.
        auto v_operand = [&](uint32_t vb, int t) -> bf16x8_t {
            const int c = t >> 2, db = t & 3;
            const uint32_t a = v_rd[db] + vb + c * 16 * 256;
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a);
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)(a + 8 * 256));
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // Keys of tile j past the end of the sequence get -inf (only the last tile can have any).
        // The limit passes through an empty asm so that its 32 compares stay in this rarely taken
        // branch: hoisted out of the loop they held 64 SGPRs and pushed other values into spills.
        auto mask_tail = [&](int j, f32x16_t (&s)[2]) {
            int lim = seg_len - j * BN - 4 * hh;   // first key offset in the tile past the end
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * mb + 8 * (i >> 2) + (i & 3) >= lim) s[mb][i] = -INFINITY;
        };
        // Row max of a 64-key score tile (both lane halves).
        auto row_max = [&](const f32x16_t (&s)[2]) -> float {
            float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
            for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[0][i]), s[0][i + 1]);
            mx = fmaxf(mx, s[0][15]);
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[1][i]), s[1][i + 1]);
            return xhalf_max(mx);
        };

        f32x16_t oacc[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
        // Scores are in log2 units (q carries log2(e)/sqrt(D)).  m_run is the offset already taken
        // off every score: the score MFMAs start from negm = -m_run instead of zero.
        float m_run = 0.0f;
        float l_run = 0.0f;
        f32x16_t negm;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = 0.0f;
        const bool ragged = (seg_len % BN) != 0;
        const uint32_t one2 = 0x3f803f80u;  // bf16 pair (1, 1)

        // Scores of tile 0.
        f32x16_t sa[2], sb[2];
        {
            f16x8_t ka[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) ka[t] = k_operand(0, t);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sa[mb][i] = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t)
                sa[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[t], qreg[t >> 1], sa[t & 1], 0, 0, 0);
        }

        // One tile step j (tile j in slot b): softmax weights and PV of tile j (scores sc) while the
        // scores of tile j+1 (sn) are formed and tile j+PREF is fetched into slot (b+PREF) % NBUF.
        auto step = [&](auto bufc, int j, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
            constexpr int b = decltype(bufc)::value;
            constexpr int b1 = (b + 1) % NBUF;
            constexpr int bp = (b + PREF) % NBUF;
            if (ragged && j == ntiles - 1) mask_tail(j, sc);
            {
                const float mx = row_max(sc);   // relative to m_run
                // Lazy running max: move the offset only when this tile's max is well above it (and on
                // the first tile, whose scores carry no offset yet).
                const bool grow = (j == 0) | (mx > LAZY_LOG2);
                if (__any(grow)) {
                    const float dm = grow ? mx : 0.0f;
                    const float alpha = j == 0 ? 1.0f : __builtin_amdgcn_exp2f(-dm);
                    m_run += dm;
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < 4; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) sc[mb][i] -= dm;
#pragma unroll
                    for (int i = 0; i < 16; ++i) negm[i] = -m_run;
                }
            }

            // Scores of tile j+1 (MFMA) while the weights of tile j are formed (VALU).  After the
            // last tile the K slot holds stale data and these scores are discarded.
            f16x8_t ka[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) ka[t] = k_operand(b1 * TILE_BYTES, t);
            // The rounded weights are summed in two chains, one of them the running row sum.
            bf16x8_t pb[4];
            float l2 = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int mb = c >> 1, o = 8 * (c & 1);
                uint32_t u[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(sc[mb][o + 2 * e]);
                    const float p1 = __builtin_amdgcn_exp2f(sc[mb][o + 2 * e + 1]);
                    u[e] = pack_bf16x2(p0, p1);
                    if (c & 1)
                        l2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e]),
                                                             __builtin_bit_cast(bf16x2_t, one2), l2, false);
                    else
                        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u[e]),
                                                                __builtin_bit_cast(bf16x2_t, one2), l_run, false);
                }
                pb[c] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0], u[1], u[2], u[3]));
            }
            l_run += l2;
            sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[0], qreg[0], negm, 0, 0, 0);
            sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[1], qreg[0], negm, 0, 0, 0);
#pragma unroll
            for (int t = 2; t < 16; ++t)
                sn[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[t], qreg[t >> 1], sn[t & 1], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 0);
#pragma unroll
            for (int t = 0; t < 12; ++t) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 5, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 5, 0);
            }

            // Fetch tile j+PREF into the slot read last before the previous barrier.  Past the last
            // tile the fetch repeats the last tile into that free slot (nothing reads it again);
            // issuing unconditionally keeps the count of copies in flight fixed.
            issue_tile(min(j + PREF, ntiles - 1), bp);

            // PV of tile j.
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const bf16x8_t va = v_operand(b * TILE_BYTES, t);
                oacc[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t >> 2], oacc[t & 3], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 6, 0);
#pragma unroll
            for (int t = 0; t < 13; ++t) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 3, 0);

            if constexpr (FUSED) {
                finish_tile(min(j + PREF, ntiles - 1), bp);
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            } else {
                // Tile j+2 must have landed before the barrier; tile j+3 (fetched above) may not.
                asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };

        if (qt * BM + wave * 32 < q_len) {
            for (int j = 0; j < ntiles; j += 4) {
                step(Buf<0>{}, j, sa, sb);
                if (j + 1 >= ntiles) break;
                step(Buf<1>{}, j + 1, sb, sa);
                if (j + 2 >= ntiles) break;
                step(Buf<2>{}, j + 2, sa, sb);
                if (j + 3 >= ntiles) break;
                step(Buf<3>{}, j + 3, sb, sa);
            }
        } else {
            // All 32 query rows of this wave lie past the sequence (the last query tile of a short
            // sequence): no products, only this wave's share of the tile copies and the barriers.
            for (int j = 0; j < ntiles; ++j) {
                issue_tile(min(j + PREF, ntiles - 1), (j + PREF) % NBUF);
                if constexpr (FUSED) {
                    finish_tile(min(j + PREF, ntiles - 1), (j + PREF) % NBUF);
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                }
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
        }
        // Copies issued by the last steps (repeats of the last tile) must land before the
        // workgroup's LDS is reused: every wave waits for its own, and the barrier for the others'.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        // ---- epilogue: O / l -> bf16, through LDS to whole rows -------------------------------------
        const float l_tot = xhalf_sum(l_run);
        const float inv = 1.0f / l_tot;
        if (p.lse && q_valid && hh == 0)
            p.lse[(long long)q_row * p.heads + head] = m_run * 0.6931471805599453f + __logf(l_tot);
        {
            // Wave w stages its 32 rows in LDS bytes 8 KB w ..: lane (l32, hh) holds channels
            // 32 db + 8 grp + 4 hh .. +3 of row l32, i.e. half hh of 16-byte chunk 4 db + grp,
            // stored at chunk (4 db + grp) ^ (l32 % 16) of the row.
            const uint32_t sb = lds0 + wave * 8192;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    typedef uint32_t st_u32x2_t __attribute__((ext_vector_type(2)));
                    st_u32x2_t u;
                    u[0] = pack_bf16x2(oacc[db][4 * grp + 0] * inv, oacc[db][4 * grp + 1] * inv);
                    u[1] = pack_bf16x2(oacc[db][4 * grp + 2] * inv, oacc[db][4 * grp + 3] * inv);
                    const uint32_t a = sb + l32 * 256 + 16 * ((4 * db + grp) ^ (l32 & 15)) + 8 * hh;
                    *(__attribute__((address_space(3))) st_u32x2_t*)(uintptr_t)a = u;
                }
            // Lane L then writes 16-byte chunk L % 16 of rows 4 it + L / 16: 16 lanes per row.
            const int qb0 = qt * BM + wave * 32;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int r = 4 * it + (lane >> 4);
                const int ql = qb0 + r;
                const u32x4_t val = *(__attribute__((address_space(3))) const u32x4_t*)(uintptr_t)(
                    sb + r * 256 + 16 * (pc ^ (r & 15)));
                if (ql < q_len) {
                    // Window mode: q, v and out share the row layout, so the item's table of V row
                    // byte offsets gives the output row too.
                    uint16_t* op;
                    if constexpr (WIN) {
                        const uint32_t rb = ql < WIN_TABLE ? win_vrow[ql]
                                                           : 2u * (uint32_t)(win0 + win_offset(ql, p.win)) * (uint32_t)row_stride;
                        op = p.out + (long long)head * D + 8 * pc + (rb >> 1);
                    } else {
                        op = p.out + (seg * q_len + ql) * row_stride + (long long)head * D + 8 * pc;
                    }
                    *reinterpret_cast<uint4*>(op) = make_uint4(val[0], val[1], val[2], val[3]);
                }
            }
        }
        // The next item's copies overwrite the staging area.
        __builtin_amdgcn_s_barrier();
    }  // item
}

// The fast launch (staged K): 16x16x32 score and PV blocks, and a score offset that is the first
// tile's row max and never moves.  A row's sum then only grows and bounds every weight it has
// used; an item whose row sum reaches OVF_SUM = 2^64 (or is not finite) is flagged in
// p.item_flags, and the guard launch of the running-max kernel on the same stream redoes exactly
// the flagged items.  Unflagged, the accumulator stays below 2^64 |v|.
//
// Against the 32x32x16 blocks of the running-max kernel, the 16x16x32 shape does the same work
// for about 13 % less energy per product on random operands, and the kernel runs power-limited.
// Its read addresses take more registers (8 V and 4 K bases), which the running-max kernel's
// rescaling code has no room for.
template <bool WIN, bool SPLIT>
__global__ void __launch_bounds__(NTHREADS, 1) attn_fast_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];
    // 32 KB beside the tiles: in window mode the byte offset of each V row of the window; otherwise
    // the rotation table, copied once per workgroup when it has at most LDS_TABLE entries.
    __shared__ __attribute__((aligned(16))) uint32_t lds_aux[WIN_TABLE];
    uint32_t* const win_vrow = lds_aux;
    const float2* const tab_lds = reinterpret_cast<const float2*>(lds_aux);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;

    // The Q rotation of every item gathers 32 table entries per lane.  From global memory these
    // gathers are most of the prologue's vector-memory instructions, which all CUs issue at the
    // same time; from LDS they cost a few cycles each.
    const bool table_in_lds = !WIN && p.g.identity < LDS_TABLE;
    if (table_in_lds) {
        float2* const t = reinterpret_cast<float2*>(lds_aux);
        for (int i = threadIdx.x; i <= p.g.identity; i += NTHREADS) t[i] = p.table[i];
        __syncthreads();
    }

    // Persistent: workgroup b takes items b, b + G, b + 2G, ... (G = gridDim.x, a multiple of 8),
    // each through the XCD remap, so the items an XCD runs at one time are neighbouring tiles.
    for (int item = blockIdx.x; item < p.total_wg; item += gridDim.x) {
        const int logical = xcd_remap(item, p.total_wg);
        const int qt = logical % p.q_tiles;
        int rest = logical / p.q_tiles;
        int half = 0;   // key split: which run of the sequence's key tiles this item takes
        if constexpr (SPLIT) {
            half = rest & 1;
            rest >>= 1;
        }
        const int seg = rest % p.n_segs;
        const int head = rest / p.n_segs;
        const int t0 = half * p.split_tiles;   // first key tile of the item
        // From here on "the sequence" is the item's run of keys: from key row t0 * BN to the end.
        const int seg_base = seg * p.seg_len + t0 * BN;   // first key buffer row of the run
        const int win0 = WIN ? win_origin(seg, p.win) : 0;   // window mode: grid row of local row 0
        const int seg_len = p.seg_len - t0 * BN;
        const int q_len = p.q_len;
        const long long row_stride = (long long)p.heads * D;
        const int ntiles = SPLIT ? (half ? p.k_tiles - p.split_tiles : p.split_tiles) : p.k_tiles;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l16 = lane & 15;
        const int lg = lane >> 4;
        const RopeGeom& g = p.g;

        // ---- tile copies ------------------------------------------------------------------------
        // Wave w, copy i in {0,1}: rows r = 8w + 4i + lane/16, physical chunk lane%16 of that row.
        const int dr0 = 8 * wave + (lane >> 4);
        const int pc = lane & 15;
        const uint16_t* vhead = p.v + (long long)head * D;
        const long long ktile0 = ((long long)head * p.n_segs + seg) * p.k_tiles + t0;
        uint32_t k_src_off[2];   // staged: byte offset of the lane's chunk inside a K~ tile
        int v_chunk[2];          // element offset of the lane's logical chunk inside a V row
        uint32_t vch2[2];        // the same in bytes
        const uint32_t rs2 = 2u * (uint32_t)row_stride;   // bytes per V row (< 2^24)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = dr0 + 4 * i;
            k_src_off[i] = 2u * (uint32_t)(r * D + 8 * (pc ^ k_swz(r)));
            v_chunk[i] = 8 * (pc ^ v_swz16(r));
            vch2[i] = 2u * (uint32_t)v_chunk[i];
        }

        // issue_tile(j, slot): fetch tile j into K and V slot `slot`.
        auto issue_tile = [&](int j, int slot) {
            // The wave's LDS base passes through an empty asm so that the copies' LDS addresses are
            // formed here by scalar adds; hoisted out of the loop, their 16 values were spilled and
            // reloaded with VALU lane reads on every tile.
            uint32_t wl = lds0 + (8 * wave) * 256;
            asm volatile("" : "+s"(wl));
            const uint32_t kl = wl + slot * TILE_BYTES;
            const uint32_t vl = wl + V_LDS_BASE + slot * TILE_BYTES;
            const int last = seg_len - 1 - j * BN;   // rows past the end repeat the last row
            if constexpr (WIN) {
                // Each lane addresses its own grid row from the head's base (total bytes < 2^32):
                // from the item's table of row offsets, or by the window arithmetic past it.
                const bool from_table = j * BN + BN <= WIN_TABLE;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = dr0 + 4 * i;
                    const int re = r < last ? r : last;
                    const uint32_t rb = from_table ? win_vrow[j * BN + re]
                                                   : 2u * (uint32_t)(win0 + win_offset(j * BN + re, p.win)) * (uint32_t)row_stride;
                    dma16(vhead, rb + vch2[i], vl + i * 1024);
                }
            } else {
                const uint16_t* vt = vhead + (long long)(seg_base + j * BN) * row_stride;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = dr0 + 4 * i;
                    const int re = r < last ? r : last;
                    dma16(vt, __umul24((uint32_t)re, rs2) + vch2[i], vl + i * 1024);
                }
            }
            const uint16_t* kt = p.k + (ktile0 + j) * (BN * D);
#pragma unroll
            for (int i = 0; i < 2; ++i) dma16(kt, k_src_off[i], kl + i * 1024);
        };
        // ---- prologue -----------------------------------------------------------------------------
        if constexpr (WIN) {
            // The window's V row offsets, once per item: the tile copies then read them instead of
            // doing two divisions per row and tile.  The previous item's copies were all issued
            // before its last barrier, so the table is free to overwrite.
            for (int li = tid; li < min(seg_len, WIN_TABLE); li += NTHREADS)
                win_vrow[li] = 2u * (uint32_t)(win0 + win_offset(li, p.win)) * (uint32_t)row_stride;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < PREF; ++j) issue_tile(min(j, ntiles - 1), j);

        // ---- queries ------------------------------------------------------------------------------
        // Lane (l16, lg) owns query columns l16 and 16 + l16 of the wave's 32 rows (qb = 0, 1) and,
        // as the B operand of the 16x16x32 score product, channels 32 ks + 8 lg .. +7 of each.
        int q_row[2];
        bool q_valid[2];
        f16x8_t qreg[2][4];
        {
            // Lanes past the sequence read its first row (in bounds) and are never stored.  Pair p of
            // a row reads table entry base_a + p, a the axis p falls in: the three bases are formed
            // once per row, and each pair costs two compares and two selects.  Text rows take
            // position (0, 0, 0), where every angle is 0 (cos 1, sin 0 exactly): no rotation.
            const int f1 = __builtin_amdgcn_readfirstlane(g.first[1]);
            const int f2 = __builtin_amdgcn_readfirstlane(g.first[2]);
            const int lane_p = 4 * lg;   // the pairs of chunk 4 ks + lg are 16 ks + 4 lg + i
            const int g1 = f1 - lane_p, g2 = f2 - lane_p;
            const float sc = p.scale_log2;
            uint4 raw[2][4];
            int bt[2], bh[2], bw[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int q_local = qt * BM + wave * 32 + 16 * qb + l16;
                q_valid[qb] = q_local < q_len;
                q_row[qb] = WIN ? win0 + win_offset(q_valid[qb] ? q_local : 0, p.win)
                                : seg * q_len + (q_valid[qb] ? q_local : 0);   // query buffer row
                const int q_pos = p.q_pos_base + q_row[qb];                   // its global row
                const bool text = q_pos >= g.Nv;
                int t, h, w;
                decode_pos(text ? 0 : q_pos, g, t, h, w);
                bt[qb] = (int)__umul24((unsigned)t, (unsigned)g.pairs[0]) + lane_p;
                bh[qb] = g.off[1] - f1 + (int)__umul24((unsigned)h, (unsigned)g.pairs[1]) + lane_p;
                bw[qb] = g.off[2] - f2 + (int)__umul24((unsigned)w, (unsigned)g.pairs[2]) + lane_p;
                const uint16_t* qp = p.q + q_row[qb] * row_stride + (long long)head * D + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) raw[qb][ks] = ld16(qp + 32 * ks);
            }
            // All 32 table entries are loaded before any is used: the empty asm (a memory clobber)
            // keeps the loads above it, so they are in flight together.  Left to itself the
            // compiler placed each load just before its use, behind a wait for everything issued
            // before it: 32 round trips per item.
            float2 cs[2][4][4];
            if (table_in_lds) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int p0 = 16 * ks + i;
                            const int base = p0 >= g2 ? bw[qb] : (p0 >= g1 ? bh[qb] : bt[qb]);
                            cs[qb][ks][i] = tab_lds[base + p0];
                        }
            } else {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int p0 = 16 * ks + i;
                            const int base = p0 >= g2 ? bw[qb] : (p0 >= g1 ? bh[qb] : bt[qb]);
                            cs[qb][ks][i] = p.table[base + p0];
                        }
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const uint32_t wd[4] = {raw[qb][ks].x, raw[qb][ks].y, raw[qb][ks].z, raw[qb][ks].w};
                    uint32_t o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
                        rotate_pair(x0, x1, cs[qb][ks][i]);
                        o[i] = pack_f16x2(x0 * sc, x1 * sc);
                    }
                    qreg[qb][ks] = __builtin_bit_cast(f16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
                }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        // ---- per-lane LDS read addresses (slot 0; other slots add a multiple of TILE_BYTES) --------
        // K operand of the score product, key block kb (keys 16 kb + l16), step ks: logical chunk
        // 4 ks + lg of row 16 kb + l16 (the swizzle depends on l16 only).
        uint32_t k_rd[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) k_rd[ks] = lds0 + l16 * 256 + 16 * ((4 * ks + lg) ^ k_swz(l16));
        // V operand of the PV product for channel block db, read transposed: the 16 lanes of group
        // lg read rows 4 lg .. 4 lg + 3 (+ 16 for the upper half, + 32 for the second key chunk) by
        // channels 16 db .. 16 db + 15.  Lane l16 addresses row 4 lg + l16 / 4 and channels
        // 16 db + 4 (l16 % 4) .. +3, i.e. logical chunk 2 db + (l16 % 4) / 2, byte 8 (l16 % 2); it
        // receives channel 16 db + l16 of the four rows.
        uint32_t v_rd[8];
        {
            const int row = 4 * lg + (l16 >> 2);
#pragma unroll
            for (int db = 0; db < 8; ++db)
                v_rd[db] = lds0 + V_LDS_BASE + row * 256 + 16 * ((2 * db + ((l16 & 3) >> 1)) ^ v_swz16(row)) +
                           8 * (l16 & 1);
        }
        auto k_operand = [&](uint32_t kb_slot, int kb, int ks) -> f16x8_t {
            const uint32_t a = k_rd[ks] + kb_slot + kb * 16 * 256;
            return *(__attribute__((address_space(3))) const f16x8_t*)(uintptr_t)a;
        };
        // Keys of V operand (db, kk): 32 kk + 4 lg + (0..3), then 32 kk + 16 + 4 lg + (0..3).
        auto v_operand = [&](uint32_t vb, int db, int kk) -> bf16x8_t {
            const uint32_t a = v_rd[db] + vb + kk * 32 * 256;
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)a);
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(uintptr_t)(a + 16 * 256));
            return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // Score block (kb, qb) holds, in lane (l16, lg), keys 16 kb + 4 lg + i (i = 0..3) of query
        // 16 qb + l16.  Keys of tile j past the end of the sequence get -inf (only the last tile can
        // have any).  The limit passes through an empty asm so that its compares stay in this
        // rarely taken branch: hoisted out of the loop they would hold SGPRs for the whole loop.
        auto mask_tail = [&](int j, f32x4_t (&s)[4][2]) {
            int lim = seg_len - j * BN - 4 * lg;   // first key offset in the tile past the end
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * kb + i >= lim) s[kb][qb][i] = -INFINITY;
        };
        // Row max of query block qb over a 64-key score tile (all four lane groups).
        auto row_max = [&](const f32x4_t (&s)[4][2], int qb) -> float {
            float mx = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), s[0][qb][2]);
            mx = fmaxf(fmaxf(mx, s[0][qb][3]), s[1][qb][0]);
            mx = fmaxf(fmaxf(mx, s[1][qb][1]), s[1][qb][2]);
            mx = fmaxf(fmaxf(mx, s[1][qb][3]), s[2][qb][0]);
            mx = fmaxf(fmaxf(mx, s[2][qb][1]), s[2][qb][2]);
            mx = fmaxf(fmaxf(mx, s[2][qb][3]), s[3][qb][0]);
            mx = fmaxf(fmaxf(mx, s[3][qb][1]), s[3][qb][2]);
            mx = fmaxf(mx, s[3][qb][3]);
            return xquad_max(mx);
        };


        // Output O^T block (db, qb): lane (l16, lg) holds channels 16 db + 4 lg + i of query
        // 16 qb + l16.
        f32x4_t oacc[8][2];
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[db][qb][i] = 0.0f;
        // Scores are in log2 units (q carries log2(e)/sqrt(D)).  m_run is the offset already taken
        // off every score: the score MFMAs start from negm = -m_run instead of zero.
        float m_run[2] = {0.0f, 0.0f};
        float l_run[2] = {0.0f, 0.0f};
        f32x4_t negm[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) negm[qb][i] = 0.0f;
        const bool ragged = (seg_len % BN) != 0;
        const uint32_t one2 = 0x3f803f80u;  // bf16 pair (1, 1)

        // Scores of tile 0.
        f32x4_t sa[4][2], sb[4][2];
        {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[kb][qb][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const f16x8_t ka = k_operand(0, kb, ks);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        sa[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[qb][ks], sa[kb][qb], 0, 0, 0);
                }
        }

        // One tile step j (tile j in slot b): softmax weights and PV of tile j (scores sc) while the
        // scores of tile j+1 (sn) are formed and tile j+PREF is fetched into slot (b+PREF) % NBUF.
        auto step = [&](auto bufc, int j, f32x4_t (&sc)[4][2], f32x4_t (&sn)[4][2]) {
            constexpr int b = decltype(bufc)::value;
            constexpr int b1 = (b + 1) % NBUF;
            constexpr int bp = (b + PREF) % NBUF;
            if (ragged && j == ntiles - 1) mask_tail(j, sc);
            if (j == 0) {
                // The offset: the first tile's row max, taken off its scores and, through negm, off
                // every later score.
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const float mx = row_max(sc, qb);
                    m_run[qb] = mx;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sc[kb][qb][i] -= mx;
#pragma unroll
                    for (int i = 0; i < 4; ++i) negm[qb][i] = -mx;
                }
            }

            // The step in a fixed order, fenced (sched_barrier) in groups of two MFMAs: one K~ or V
            // operand for both query blocks.  The fences keep the schedule of this loop from
            // depending on code elsewhere in the kernel (left to the scheduler, the K~ reads moved
            // next to their MFMAs whenever other code changed the register estimate), and cost
            // nothing against the scheduler's best order.
            // Scores of tile j+1 first: operand t = (ks, kb) = (t / 4, t % 4), K~ read KAHEAD
            // operands ahead.  After the last tile the K slot holds stale data and these scores
            // are discarded.  Into those 16 groups and the first 8 PV groups (chunk 0, which does
            // not need chunk 1's weights) go the 16 softmax pairs of tile j, pair i (chunk
            // kk = i / 8, query block (i / 4) % 2, element pair i % 4) in group 3 i / 2: two
            // exponentials and one bf16 pack each.  The 16 row-sum dot products take the last 8
            // groups; the weights are summed in two chains, one of them the running row sum.
            uint32_t pu[2][2][4];
            auto do_pair = [&](int i) {
                const int kk = i >> 3, qb = (i >> 2) & 1, e = i & 3;
                const int kb = 2 * kk + (e >> 1), i0 = 2 * (e & 1);
                const float p0 = __builtin_amdgcn_exp2f(sc[kb][qb][i0]);
                const float p1 = __builtin_amdgcn_exp2f(sc[kb][qb][i0 + 1]);
                pu[kk][qb][e] = pack_bf16x2(p0, p1);
            };
            auto pairs_in = [&](int grp) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((3 * i) / 2 == grp) do_pair(i);
            };
            float l2[2] = {0.0f, 0.0f};
            auto dots_in = [&](int grp) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (24 + (i >> 1) == grp) {
                        const int kk = i >> 3, qb = (i >> 2) & 1, e = i & 3;
                        if (kk)
                            l2[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu[kk][qb][e]),
                                                                     __builtin_bit_cast(bf16x2_t, one2), l2[qb], false);
                        else
                            l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu[kk][qb][e]),
                                                                        __builtin_bit_cast(bf16x2_t, one2), l_run[qb], false);
                    }
            };
            f16x8_t ka[16];
#pragma unroll
            for (int t = 0; t < KAHEAD; ++t) ka[t] = k_operand(b1 * TILE_BYTES, t & 3, t >> 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t + KAHEAD < 16) ka[t + KAHEAD] = k_operand(b1 * TILE_BYTES, (t + KAHEAD) & 3, (t + KAHEAD) >> 2);
                const int ks = t >> 2, kb = t & 3;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    sn[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t], qreg[qb][ks],
                                                                        ks == 0 ? negm[qb] : sn[kb][qb], 0, 0, 0);
                pairs_in(t);
                __builtin_amdgcn_sched_barrier(0);
            }

            // Fetch tile j+PREF into the slot read last before the previous barrier.  Past the last
            // tile the fetch repeats the last tile into that free slot (nothing reads it again);
            // issuing unconditionally keeps the count of copies in flight fixed.
            issue_tile(min(j + PREF, ntiles - 1), bp);
            __builtin_amdgcn_sched_barrier(0);

            // PV of tile j: operand t = (kk, db) = (t / 8, t % 8), V read VAHEAD operands ahead.
            bf16x8_t va[16];
            bf16x8_t pb[2][2];
#pragma unroll
            for (int t = 0; t < VAHEAD; ++t) va[t] = v_operand(b * TILE_BYTES, t & 7, t >> 3);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t + VAHEAD < 16) va[t + VAHEAD] = v_operand(b * TILE_BYTES, (t + VAHEAD) & 7, (t + VAHEAD) >> 3);
                const int kk = t >> 3, db = t & 7;
                if (t == 0 || t == 8) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
                        pb[kk][qb] = __builtin_bit_cast(bf16x8_t, make_uint4(pu[kk][qb][0], pu[kk][qb][1],
                                                                             pu[kk][qb][2], pu[kk][qb][3]));
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[t], pb[kk][qb], oacc[db][qb], 0, 0, 0);
                pairs_in(16 + t);
                dots_in(16 + t);
                __builtin_amdgcn_sched_barrier(0);
            }
            l_run[0] += l2[0];
            l_run[1] += l2[1];

            // Tile j+2 must have landed before the barrier; tile j+3 (fetched above) may not.
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };

        if (qt * BM + wave * 32 < q_len) {
            for (int j = 0; j < ntiles; j += 4) {
                step(Buf<0>{}, j, sa, sb);
                if (j + 1 >= ntiles) break;
                step(Buf<1>{}, j + 1, sb, sa);
                if (j + 2 >= ntiles) break;
                step(Buf<2>{}, j + 2, sa, sb);
                if (j + 3 >= ntiles) break;
                step(Buf<3>{}, j + 3, sb, sa);
            }
        } else {
            // All 32 query rows of this wave lie past the sequence (the last query tile of a short
            // sequence): no products, only this wave's share of the tile copies and the barriers.
            for (int j = 0; j < ntiles; ++j) {
                issue_tile(min(j + PREF, ntiles - 1), (j + PREF) % NBUF);
                asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
        }
        // Copies issued by the last steps (repeats of the last tile) must land before the
        // workgroup's LDS is released.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        if constexpr (SPLIT) {
            // A half of a key split.  Its coordinates again, from an opaque copy of the item number
            // (kept from before the loop they would hold registers through it): flags are indexed
            // by logical item (the guard reads both halves of a query tile), and the output is the
            // half's normalised rows in fp32, 16 bytes per lane and block, with its log-sum-exp.
            int item_e = item;
            asm volatile("" : "+s"(item_e));
            const int logical_e = xcd_remap(item_e, p.total_wg);
            const bool second = ((logical_e / p.q_tiles) & 1) != 0;
            float* const lsep = second ? p.lse_b : p.lse;
            float* const part = second ? p.part_b : p.part_a;
            {
                const bool flagged = __any(!(l_run[0] < OVF_SUM) || !(l_run[1] < OVF_SUM));
                if (lane == 0) p.item_flags[8ll * logical_e + wave] = flagged ? 1 : 0;
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float l_tot = xquad_sum(l_run[qb]);
                const float inv = 1.0f / l_tot;
                if (q_valid[qb] && lg == 0)
                    lsep[(long long)q_row[qb] * p.heads + head] = m_run[qb] * 0.6931471805599453f + __logf(l_tot);
                if (q_valid[qb]) {
                    float* const op = part + q_row[qb] * row_stride + (long long)head * D + 4 * lg;
#pragma unroll
                    for (int db = 0; db < 8; ++db)
                        *reinterpret_cast<float4*>(op + 16 * db) =
                            make_float4(oacc[db][qb][0] * inv, oacc[db][qb][1] * inv, oacc[db][qb][2] * inv,
                                        oacc[db][qb][3] * inv);
                }
            }
            continue;
        }
        {
            // Never rescaled, a lane's partial row sums bound every weight it has used.
            const bool flagged = __any(!(l_run[0] < OVF_SUM) || !(l_run[1] < OVF_SUM));
            if (lane == 0) p.item_flags[8ll * item + wave] = flagged ? 1 : 0;
        }

        // ---- epilogue: O / l -> bf16 ---------------------------------------------------------------
        // Lane (l16, lg) holds 4 channels of its row per channel block db.  Two lane swaps per pair
        // of blocks (2 d, 2 d + 1) give it 8 consecutive channels, 32 d + 8 lg .. +7.  Neighbouring
        // lanes l16 = 2 m, 2 m + 1 then trade one such piece, so that a store covers whole
        // 128-byte lines: 8 rows x 128 bytes per store, where storing the blocks as they are writes
        // 32 bytes into each of 16 rows (about half of the time between two items went there).
        // The lane's parity is formed here from the lane count (mbcnt), not kept from before the
        // loop: one more value live through the tile loop leaves its schedule too few registers
        // to read the K operands ahead.
        const bool odd = (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 1u) != 0;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float l_tot = xquad_sum(l_run[qb]);
            const float inv = 1.0f / l_tot;
            if (p.lse && q_valid[qb] && lg == 0)
                p.lse[(long long)q_row[qb] * p.heads + head] = m_run[qb] * 0.6931471805599453f + __logf(l_tot);
            uint32_t w[4][4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // A: block 2 d (channels 32 d + 4 lg ..), B: block 2 d + 1 (32 d + 16 + 4 lg ..).
                const uint32_t a0 = pack_bf16x2(oacc[2 * d][qb][0] * inv, oacc[2 * d][qb][1] * inv);
                const uint32_t a1 = pack_bf16x2(oacc[2 * d][qb][2] * inv, oacc[2 * d][qb][3] * inv);
                const uint32_t b0 = pack_bf16x2(oacc[2 * d + 1][qb][0] * inv, oacc[2 * d + 1][qb][1] * inv);
                const uint32_t b1 = pack_bf16x2(oacc[2 * d + 1][qb][2] * inv, oacc[2 * d + 1][qb][3] * inv);
                // Upper half (lg 2, 3) of A <-> lower half (lg 0, 1) of B: lanes lg 0, 1 then hold
                // A of lg and of lg + 2, lanes lg 2, 3 hold B of lg - 2 and of lg.
                const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                // Odd 16-lane groups of the first <-> even groups of the second: lane lg then holds
                // channels 32 d + 8 lg .. +7.
                const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
                const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
                w[d][0] = t0[0];
                w[d][1] = t1[0];
                w[d][2] = t0[1];
                w[d][3] = t1[1];
            }
            // The neighbour's row and whether it lies in the sequence (DPP quad_perm [1, 0, 3, 2]).
            const int nb_row = __builtin_amdgcn_update_dpp(0, q_row[qb], 0xB1, 0xF, 0xF, false);
            const int nb_valid = __builtin_amdgcn_update_dpp(0, q_valid[qb] ? 1 : 0, 0xB1, 0xF, 0xF, false);
            // Store A writes row 2 m, store B row 2 m + 1; the even lane of a pair writes bytes
            // 128 c + 16 lg .., the odd lane 128 c + 64 + 16 lg .. of that row.
            const int row_a = odd ? nb_row : q_row[qb];
            const int row_b = odd ? q_row[qb] : nb_row;
            const bool ok_a = odd ? nb_valid != 0 : q_valid[qb];
            const bool ok_b = odd ? q_valid[qb] : nb_valid != 0;
            const uint16_t* const hb = p.out + (long long)head * D + 8 * lg + (odd ? 32 : 0);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                uint32_t sent[4], got[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sent[k] = odd ? w[2 * c][k] : w[2 * c + 1][k];
                    got[k] = __builtin_amdgcn_update_dpp(0u, sent[k], 0xB1, 0xF, 0xF, false);
                }
                if (ok_a) {
                    const uint32_t* v = odd ? got : w[2 * c];
                    *reinterpret_cast<uint4*>(const_cast<uint16_t*>(hb) + row_a * row_stride + 64 * c) =
                        make_uint4(v[0], v[1], v[2], v[3]);
                }
                if (ok_b) {
                    const uint32_t* v = odd ? w[2 * c + 1] : got;
                    *reinterpret_cast<uint4*>(const_cast<uint16_t*>(hb) + row_b * row_stride + 64 * c) =
                        make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    }  // item
}

// Staging for the default mode: the K rows of every (segment, key tile) rotated into fp16 tiles,
// [head][segment][tile][64][D].  One wave per tile row: lane l takes the 16-byte chunk l % 16 of
// heads l / 16, l / 16 + 4, ..., so the row's position is decoded once per wave and the lane's
// four table entries serve all of its heads; a pass issues the loads of up to 16 heads before its
// stores.  Rows past the segment are written as zeros.  WIN: segment s is window s.
template <bool WIN>
__global__ void __launch_bounds__(256) k_prep_kernel(PrepParams p) {
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int h0 = lane >> 4;
    const int rt = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (int)(threadIdx.x >> 6));   // tile row
    const int r = rt & (BN - 1);
    const int tile = rt / BN;                  // segment * k_tiles + key tile
    const int kt = tile % p.k_tiles;
    const int seg = tile / p.k_tiles;
    const long long row_stride = (long long)p.heads * D;
    const RopeGeom& g = p.g;
    const int kl = kt * BN + r;
    const bool valid = kl < p.seg_len;
    const int nb = WIN ? win_origin(seg, p.win) + win_offset(valid ? kl : 0, p.win)
                       : seg * p.seg_len + (valid ? kl : 0);   // key buffer row
    const int n = p.kv_pos_base + nb;                        // its global row
    int t = 0, h = 0, w = 0;
    if (n < g.Nv) decode_pos(n, g, t, h, w);   // text rows: position (0, 0, 0), angles 0
    float2 cs[4];
    if (g.Nv == 0 && p.table_fill) {
        // No video rows (cross-attention): every angle is 0, so every entry is (1, 0).  The
        // table is written here for the attention launch that follows instead of being read,
        // which spares a launch of the table kernel.
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = make_float2(1.0f, 0.0f);
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e <= g.identity; e += blockDim.x) p.table_fill[e] = make_float2(1.0f, 0.0f);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = p.table[pair_entry(4 * c + i, t, h, w, g)];
    }
    const uint16_t* src = p.k + nb * row_stride + 8 * c;
    // Output row r of tile (head, seg, kt): ((head * n_segs + seg) * k_tiles + kt) * BN + r.
    const long long head_stride = (long long)p.n_segs * p.k_tiles * BN * D;
    uint16_t* dst = p.kt + ((long long)seg * p.k_tiles + kt) * (BN * D) + r * D + 8 * c;
    for (int hb = 0; hb < p.heads; hb += 16) {
        uint4 raw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int hd = hb + h0 + 4 * k;
            raw[k] = (valid && hd < p.heads) ? ld16(src + (long long)hd * D) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int hd = hb + h0 + 4 * k;
            if (hd < p.heads) {
                uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
                bool ovf = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x0 = bf16_lo(wd[i]), x1 = bf16_hi(wd[i]);
                    rotate_pair(x0, x1, cs[i]);
                    wd[i] = pack_f16x2(x0, x1);
                    ovf |= (wd[i] & 0x7fffu) == 0x7c00u || (wd[i] & 0x7fff0000u) == 0x7c000000u;
                }
                // A rotated key past fp16's range (the callers' precondition) would give some of
                // its scores infinite terms whose signs the true products need not share, and the
                // key could drop out unseen.  The whole row is made NaN instead, so every output
                // row of the head shows it.  A row is the 16 lanes of this lane's group.
                if ((__ballot(ovf) >> (lane & 48)) & 0xffffull) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) wd[i] = 0x7e007e00u;
                }
                *reinterpret_cast<uint4*>(dst + hd * head_stride) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
        }
    }
}

AttnParams make_params(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                       float* lse, const float2* table, const RopeGeom& g, int heads,
                       const SeqLayout& L) {
    AttnParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.seg_len = L.kv_len;
    p.q_len = L.q_len;
    p.n_segs = L.n_segs;
    p.q_pos_base = L.q_pos_base;
    p.kv_pos_base = L.kv_pos_base;
    p.q_tiles = (L.q_len + BM - 1) / BM;
    p.k_tiles = (L.kv_len + BN - 1) / BN;
    p.total_wg = p.q_tiles * L.n_segs * heads;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    p.win = WinMap{};
    p.item_flags = nullptr;
    p.k_split = 1;
    p.split_tiles = p.k_tiles;
    p.part_a = nullptr;
    p.part_b = nullptr;
    p.lse_b = nullptr;
    return p;
}

// The Q rotation reads table entry base_axis + pair for every pair of the head: the split must
// cover all D/2 pairs (text rows read the position-0 entries).
bool geom_covers_head(const RopeGeom& g) { return g.pairs[0] + g.pairs[1] + g.pairs[2] == D / 2; }

// Compute units of the current device, rounded down to a multiple of the 8 XCDs.
int cu_count() {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8)
        ncu = 256;
    return ncu - ncu % 8;
}

// Workgroups of a persistent launch: one per CU (each holds 128 KB of LDS), no more than there are
// items.
int persistent_grid(int total) {
    const int ncu = cu_count();
    return total < ncu ? total : ncu;
}

// The fast launch pays a second (guard) launch; below this many (item, key tile) pairs the safe
// kernel alone is as quick.  Above it the fast kernel wins also on short items: 7x10x13 windows
// of the 21x30x52 grid (25,920 pairs) 312 -> 280 us, cross-attention of 32,760 queries against
// 512 text keys (12,288 pairs) 130 -> 126 us, in A/Bs on one box.
constexpr long long kFastMinTiles = 4096;

// Key split of the fast launch: two items per query tile, each over one half of the key tiles,
// when the last round of the persistent grid would leave most CUs idle.  At 5x30x52 x 12 heads
// the 372 items fill 1.45 rounds of 256 CUs; 744 half-items fill 2.9.  The halves are merged by
// their log-sum-exp (one HBM pass over the output).  Self-attention over staged keys only.
int key_split(long long items, int k_tiles) {
    if (items * k_tiles < kFastMinTiles || k_tiles < 32) return 1;
    const long long ncu = cu_count();
    const double eff1 = (double)items / (double)(ncu * ((items + ncu - 1) / ncu));
    const double eff2 = (double)(2 * items) / (double)(ncu * ((2 * items + ncu - 1) / ncu));
    return eff2 >= eff1 + 0.15 ? 2 : 1;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Staged (FUSED = false) launches: with `flags` (attn_flag_bytes: 8 bytes per item, and the buffers
// of a key split), the fast
// kernel followed by the guard launch of the safe kernel; otherwise the safe kernel alone.
template <bool FUSED, bool WIN>
hipError_t launch(AttnParams p, uint8_t* flags, hipStream_t stream, bool allow_split = true) {
    if (!geom_covers_head(p.g)) return hipErrorInvalidValue;
    const dim3 grid(persistent_grid(p.total_wg));
    if constexpr (!FUSED) {
        if (flags && (long long)p.total_wg * p.k_tiles >= kFastMinTiles) {
            p.item_flags = flags;
            const int ks = (WIN || !allow_split) ? 1 : key_split(p.total_wg, p.k_tiles);
            AttnParams pf = p;
            const long long rows_heads = (long long)p.n_segs * p.q_len * p.heads;
            if (ks > 1) {
                // Scratch after the flags (attn_flag_bytes): the second half's output and the
                // log-sum-exp of both halves.
                uint8_t* cur = flags + align256((size_t)p.total_wg * 2 * 8);
                pf.part_a = reinterpret_cast<float*>(cur);
                cur += align256((size_t)rows_heads * D * 4);
                pf.part_b = reinterpret_cast<float*>(cur);
                cur += align256((size_t)rows_heads * D * 4);
                pf.lse = reinterpret_cast<float*>(cur);
                cur += align256((size_t)rows_heads * 4);
                pf.lse_b = reinterpret_cast<float*>(cur);
                pf.k_split = 2;
                pf.split_tiles = (p.k_tiles + 1) / 2;
                pf.total_wg = 2 * p.total_wg;
            }
            if (ks > 1)
                hipLaunchKernelGGL((attn_fast_kernel<false, true>), dim3(persistent_grid(pf.total_wg)), dim3(NTHREADS), 0,
                                   stream, pf);
            else
                hipLaunchKernelGGL((attn_fast_kernel<WIN, false>), grid, dim3(NTHREADS), 0, stream, pf);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (ks > 1) {
                e = launch_merge2_f32_bf16(pf.part_a, pf.part_b, pf.lse, pf.lse_b, rows_heads, D, p.out, p.lse,
                                           stream);
                if (e != hipSuccess) return e;
            }
            // The guard redoes, over all keys and into out (after the merge), every query tile
            // that one of its items flagged.
            AttnParams pg = p;
            pg.k_split = ks;
            hipLaunchKernelGGL((attn_fwd_kernel<false, WIN>), grid, dim3(NTHREADS), 0, stream, pg);
            return hipGetLastError();
        }
    }
    p.item_flags = nullptr;
    hipLaunchKernelGGL((attn_fwd_kernel<FUSED, WIN>), grid, dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t attn_stage_elems(int heads, int kv_len, int n_segs) {
    const size_t k_tiles = (size_t)(kv_len + BN - 1) / BN;
    return (size_t)heads * n_segs * k_tiles * BN * D;
}

size_t attn_flag_bytes_unsplit(int heads, int q_len, int n_segs) {
    return (size_t)((q_len + BM - 1) / BM) * n_segs * heads * 8;
}

size_t attn_flag_bytes(int heads, int q_len, int kv_len, int n_segs) {
    const long long items = (long long)((q_len + BM - 1) / BM) * n_segs * heads;
    const int ks = key_split(items, (kv_len + BN - 1) / BN);
    if (ks == 1) return (size_t)items * 8;
    const size_t rows_heads = (size_t)n_segs * q_len * heads;
    return align256((size_t)items * 2 * 8) + 2 * align256(rows_heads * D * 4) + 2 * align256(rows_heads * 4);
}

hipError_t launch_k_prep(const uint16_t* k, uint16_t* kt, const float2* table, const RopeGeom& g,
                         int heads, const SeqLayout& L, hipStream_t stream, float2* table_fill) {
    PrepParams p;
    p.k = k;
    p.kt = kt;
    p.table = table;
    p.table_fill = table_fill;
    p.g = g;
    p.heads = heads;
    p.seg_len = L.kv_len;
    p.n_segs = L.n_segs;
    p.kv_pos_base = L.kv_pos_base;
    p.k_tiles = (L.kv_len + BN - 1) / BN;
    p.win = WinMap{};
    const int blocks = L.n_segs * p.k_tiles * (BN / 4);   // one wave per tile row
    hipLaunchKernelGGL(k_prep_kernel<false>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_k_prep_win(const uint16_t* k, uint16_t* kt, const float2* table, const RopeGeom& g,
                             int heads, const WinMap& m, int n_windows, int L, hipStream_t stream) {
    PrepParams p;
    p.k = k;
    p.kt = kt;
    p.table = table;
    p.table_fill = nullptr;
    p.g = g;
    p.heads = heads;
    p.seg_len = L;
    p.n_segs = n_windows;
    p.kv_pos_base = 0;
    p.k_tiles = (L + BN - 1) / BN;
    p.win = m;
    const int blocks = n_windows * p.k_tiles * (BN / 4);   // one wave per tile row
    hipLaunchKernelGGL(k_prep_kernel<true>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_win(const uint16_t* q, const uint16_t* kt, const uint16_t* v,
                                uint16_t* out, const float2* table, const RopeGeom& g, int heads,
                                const WinMap& m, int n_windows, int L, uint8_t* flags,
                                hipStream_t stream) {
    SeqLayout sl;
    sl.n_segs = n_windows;
    sl.q_len = L;
    sl.kv_len = L;
    sl.q_pos_base = 0;
    sl.kv_pos_base = 0;
    AttnParams p = make_params(q, kt, v, out, nullptr, table, g, heads, sl);
    p.win = m;
    return launch<false, true>(p, flags, stream);
}

hipError_t launch_attn_bf16_staged(const uint16_t* q, const uint16_t* kt, const uint16_t* v,
                                   uint16_t* out, float* lse, const float2* table,
                                   const RopeGeom& g, int heads, const SeqLayout& L, uint8_t* flags,
                                   hipStream_t stream, bool allow_split) {
    return launch<false, false>(make_params(q, kt, v, out, lse, table, g, heads, L), flags, stream,
                                allow_split);
}

hipError_t launch_attn_bf16_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* out, float* lse, const float2* table,
                                  const RopeGeom& g, int heads, const SeqLayout& L,
                                  hipStream_t stream) {
    return launch<true, false>(make_params(q, k, v, out, lse, table, g, heads, L), nullptr, stream);
}

}  // namespace st
