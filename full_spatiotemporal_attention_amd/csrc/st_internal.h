// Internal declarations shared by the HIP sources of libstattn (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace st {

// ------------------------------------------------------------------------------------------
// Geometry of the token grid and of the RoPE angle table.
//
// Flat token order: n = (t * H + h) * W + w for n < Nv = T*H*W; rows n >= Nv are text rows.
// Angle table (float2 = cos, sin), built in fp64 and stored as fp32:
//   [T][pairs[0]] at off[0] = 0, [H][pairs[1]] at off[1], [W][pairs[2]] at off[2], then the
//   identity entry (1, 0) at `identity`.  Entry for axis a, position p, pair j:
//   off[a] + p * pairs[a] + j, angle p * theta^(-2j / (2 * pairs[a])).
// ------------------------------------------------------------------------------------------
struct RopeGeom {
    int T, H, W;
    int S;            // H * W, tokens per frame
    int Nv;           // T * H * W, video rows
    float inv_S;      // fp32 reciprocals used by the exact position decode below
    float inv_W;
    int pairs[3];     // rotation pairs per axis (t, h, w)
    int first[3];     // first pair index of each axis inside the head: 0, P_t, P_t + P_h
    int off[3];       // table offset (entries) of each axis block
    int identity;     // index of the (1, 0) entry; table size is identity + 1
};

// Host-side construction (defined in st_api.hip).
RopeGeom make_geom(int T, int H, int W, const int split[3]);

// Exact (t, h, w) of a video row.  n < 2^24 keeps float(n) exact; fl(n * fl(1/S)) is then off
// from n / S by less than one, so one correction step gives the exact quotient.
__device__ __forceinline__ void decode_pos(int n, const RopeGeom& g, int& t, int& h, int& w) {
    int q = (int)((float)n * g.inv_S);
    int r = n - q * g.S;
    if (r < 0) { q -= 1; r += g.S; } else if (r >= g.S) { q += 1; r -= g.S; }
    int qh = (int)((float)r * g.inv_W);
    int rw = r - qh * g.W;
    if (rw < 0) { qh -= 1; rw += g.W; } else if (rw >= g.W) { qh += 1; rw -= g.W; }
    t = q; h = qh; w = rw;
}

// Quotient and remainder of 0 <= n < 2^24 by d >= 1 through the fp32 reciprocal inv = fl(1/d)
// and one correction step (the same argument as decode_pos).
__device__ __forceinline__ int div_small(int n, int d, float inv, int& r) {
    int q = (int)((float)n * inv);
    r = n - q * d;
    if (r < 0) { q -= 1; r += d; } else if (r >= d) { q += 1; r -= d; }
    return q;
}

// Local 3D windows: the T x H x W grid cut into non-overlapping wt x wh x ww boxes, numbered
// window-major (t-box, then h-box, then w-box); inside a window, tokens are numbered t-major
// like the grid.  Token li of window s is the flat grid row origin(s) + offset(li).
struct WinMap {
    int nW, nHW;        // windows along w; windows per slab of wt frames
    float inv_nW, inv_nHW;
    int wS, ww;         // tokens per window frame (wh * ww); window width
    float inv_wS, inv_ww;
    int A, B;           // H*W - wh*ww and W - ww
    int oa, ob, oc;     // origin steps per window index along t, h, w: wt*H*W, wh*W, ww
};

// Host-side construction (defined in st_api.hip).
WinMap make_winmap(int T, int H, int W, int wt, int wh, int ww);

__device__ __forceinline__ int win_origin(int s, const WinMap& m) {
    int rem, c;
    const int a = div_small(s, m.nHW, m.inv_nHW, rem);
    const int b = div_small(rem, m.nW, m.inv_nW, c);
    return a * m.oa + b * m.ob + c * m.oc;
}

// offset(li) = lt*H*W + lh*W + lw for li = (lt*wh + lh)*ww + lw, written as li + lt*A + lh*B.
__device__ __forceinline__ int win_offset(int li, const WinMap& m) {
    int rem, lw;
    const int lt = div_small(li, m.wS, m.inv_wS, rem);
    const int lh = div_small(rem, m.ww, m.inv_ww, lw);
    (void)lw;
    return li + lt * m.A + lh * m.B;
}

// Table entry of head pair `p` (0 .. d/2-1) for a row at (t, h, w).  Text rows pass position
// (0, 0, 0), whose entries hold angle 0, i.e. (1, 0) exactly: no rotation, and no branch on the
// row kind (a select on it became a divergent branch around every table load).
// The geometry fields are uniform: they are taken into scalar registers once and the axis is
// chosen between values (a choice between array elements would become a per-lane memory load).
// pos * stride < 2^24, so the product is a 24-bit multiply.
__device__ __forceinline__ int pair_entry(int p, int t, int h, int w, const RopeGeom& g) {
    const int f1 = __builtin_amdgcn_readfirstlane(g.first[1]);
    const int f2 = __builtin_amdgcn_readfirstlane(g.first[2]);
    const int o0 = __builtin_amdgcn_readfirstlane(g.off[0]);
    const int o1 = __builtin_amdgcn_readfirstlane(g.off[1]);
    const int o2 = __builtin_amdgcn_readfirstlane(g.off[2]);
    const int s0 = __builtin_amdgcn_readfirstlane(g.pairs[0]);
    const int s1 = __builtin_amdgcn_readfirstlane(g.pairs[1]);
    const int s2 = __builtin_amdgcn_readfirstlane(g.pairs[2]);
    const bool a1 = p >= f1, a2 = p >= f2;
    const int first = a2 ? f2 : (a1 ? f1 : 0);
    const int base = a2 ? o2 : (a1 ? o1 : o0);
    const int stride = a2 ? s2 : (a1 ? s1 : s0);
    const int pos = a2 ? w : (a1 ? h : t);
    return base + (int)__umul24((unsigned)pos, (unsigned)stride) + (p - first);
}

// bfloat16 helpers (storage is uint16_t; conversions are exact widening and RNE narrowing).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Rotate one pair (x0, x1) by the table entry cs = (cos, sin).
__device__ __forceinline__ void rotate_pair(float& x0, float& x1, float2 cs) {
    float y0 = fmaf(x0, cs.x, -x1 * cs.y);
    float y1 = fmaf(x0, cs.y, x1 * cs.x);
    x0 = y0; x1 = y1;
}

// Workgroup remap for 8 XCDs.  Consecutive workgroup ids are dispatched round-robin over the
// XCDs; this gives each XCD a contiguous range of logical tiles, so tiles that share K/V (same
// head and segment) run on the same XCD and hit in its L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int b, int total) {
    const int nx = 8;
    int x = b % nx, slot = b / nx;
    int base = total / nx, rem = total % nx;
    return (x < rem) ? x * (base + 1) + slot : rem * (base + 1) + (x - rem) * base + slot;
}

// HBM -> LDS copy of 16 bytes per lane: lane L's bytes from base + voff land at LDS byte address
// lds + 16 L (global_load_lds_dwordx4, M0 = lds).  Written as inline asm so that the compiler does
// not treat later LDS reads as waiting on it; callers wait for these copies explicitly with
// s_waitcnt vmcnt before reading the data.
//
// LDS-poison debug build (ST_LDS_POISON defined): each lane first stores all-ones bits (NaN as
// fp16, bf16 and fp32) to the 16 bytes its copy will write and waits for that store, so the copy
// lands on poison.  A read of the tile that is not ordered after the copy (a missing vmcnt wait or
// barrier) then returns NaN, which reaches the output, rather than the plausible values of the
// tile the buffer held before.  Only the lanes that issue the copy store, exactly where it writes.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
#ifdef ST_LDS_POISON
    {
        const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        typedef uint32_t ones_t __attribute__((ext_vector_type(4)));
        __attribute__((address_space(3))) ones_t* dst =
            (__attribute__((address_space(3))) ones_t*)(uintptr_t)(lds + 16u * lane);
        *dst = ones_t{~0u, ~0u, ~0u, ~0u};
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
#endif
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// ------------------------------------------------------------------------------------------
// Launchers (one per kernel family).  Each returns hipSuccess or the launch error.
// ------------------------------------------------------------------------------------------

// Angle table: `table` receives g.identity + 1 float2 entries.
hipError_t launch_rope_table(const RopeGeom& g, double theta, float2* table, hipStream_t stream);

// Stand-alone rotation, [N][heads][d] bf16 (d % 8 == 0) or fp32 (d even).
hipError_t launch_rope_apply_bf16(const uint16_t* x, uint16_t* y, const RopeGeom& g, int N,
                                  int heads, int d, const float2* table, hipStream_t stream);
hipError_t launch_rope_apply_f32(const float* x, float* y, const RopeGeom& g, int N, int heads,
                                 int d, const float2* table, hipStream_t stream);

// Row layout of a batch of independent attention problems (per head).  Problem s reads query
// buffer rows s * q_len .. and key/value buffer rows s * kv_len ..; RoPE positions are the buffer
// row plus q_pos_base (queries) or kv_pos_base (keys), so a caller holding a run of a longer
// sequence passes that run's first global row.  Full attention: one problem of N rows.
// Factorised spatial stage: T problems of H*W rows.  Text cross-attention: one problem of
// q_len video rows against kv_len text rows, with a geometry that rotates nothing.
struct SeqLayout {
    int n_segs;
    int q_len;
    int kv_len;
    int q_pos_base;
    int kv_pos_base;
};

// Local window attention over the video rows of a T x H x W grid, bf16, d = 128: one problem per
// window of L = wt*wh*ww tokens (windows as in WinMap).  `kt` holds attn_stage_elems(heads, L,
// n_windows) elements.
hipError_t launch_k_prep_win(const uint16_t* k, uint16_t* kt, const float2* table, const RopeGeom& g,
                             int heads, const WinMap& m, int n_windows, int L, hipStream_t stream);
hipError_t launch_attn_bf16_win(const uint16_t* q, const uint16_t* kt, const uint16_t* v,
                                uint16_t* out, const float2* table, const RopeGeom& g, int heads,
                                const WinMap& m, int n_windows, int L, uint8_t* flags,
                                hipStream_t stream);

// Flash attention for bf16 storage, d = 128.
// Staged mode: launch_k_prep rotates K into fp16 tiles `kt` (attn_stage_elems(...) uint16
// elements), then launch_attn_bf16_staged reads them together with V.
// Fused mode: launch_attn_bf16_fused reads K directly and rotates it on every tile load.
// `lse`, when not null, receives [q rows][heads] log-sum-exp of the scaled scores.
// `flags` (attn_flag_bytes(heads, q_len, kv_len, n_segs) bytes of device memory, or null): scratch
// of the fast launch and its guard launch (flags, and for a key split the second half's output and
// both halves' log-sum-exp); with null only the kernel that tracks the running max runs.
size_t attn_stage_elems(int heads, int kv_len, int n_segs);
size_t attn_flag_bytes(int heads, int q_len, int kv_len, int n_segs);
// The flags alone (8 bytes per 256-row query block and head), for a launch that never splits.
size_t attn_flag_bytes_unsplit(int heads, int q_len, int n_segs);
// With no video rows (g.Nv == 0) and `table_fill` set, launch_k_prep reads no table: it writes
// the table (every entry (1, 0)) into table_fill for the launches after it.
hipError_t launch_k_prep(const uint16_t* k, uint16_t* kt, const float2* table, const RopeGeom& g,
                         int heads, const SeqLayout& L, hipStream_t stream, float2* table_fill = nullptr);
hipError_t launch_attn_bf16_staged(const uint16_t* q, const uint16_t* kt, const uint16_t* v,
                                   uint16_t* out, float* lse, const float2* table,
                                   const RopeGeom& g, int heads, const SeqLayout& L, uint8_t* flags,
                                   hipStream_t stream,
                                   bool allow_split = true);
hipError_t launch_attn_bf16_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* out, float* lse, const float2* table,
                                  const RopeGeom& g, int heads, const SeqLayout& L,
                                  hipStream_t stream);

// Factorised temporal stage, bf16, d = 128: for each spatial position s and head, the T rows
// t * S + s attend to each other; values come from `vs` (the spatial stage's output).
hipError_t launch_attn_temporal_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* kt,
                                     const uint16_t* vs, uint16_t* out, const float2* table,
                                     const RopeGeom& g, int heads, hipStream_t stream);

// fp32 checking kernel over row sets: problem s holds query buffer rows s * q_mul + i * q_stride
// (i < q_len) and key/value buffer rows s * kv_mul + j * kv_stride (j < kv_len), for s < n_seqs;
// positions are buffer rows plus the two position bases.  Output (and lse) rows are the query
// buffer rows.
// With `win` set, problem s is window s of `wm` instead: query and key/value rows are both
// win_origin(s) + win_offset(i) for i < q_len (= kv_len); the mul/stride fields are unused.
struct F32Layout {
    int n_seqs;
    int q_len, q_mul, q_stride, q_pos_base;
    int kv_len, kv_mul, kv_stride, kv_pos_base;
    int win;
    WinMap wm;
};
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                           const float2* table, const RopeGeom& g, int heads, int d,
                           const F32Layout& L, hipStream_t stream);

// QKV projection x [n_rows][C] times w^T (w [3C][C]) plus bias, q and k rotated, written to
// q, k, v [n_rows][C].  bf16 needs C % 64 == 0 and d == 128; the f32 kernel takes any even d.
hipError_t launch_qkv_rope_bf16(const uint16_t* x, const uint16_t* w, const uint16_t* bias,
                                uint16_t* q, uint16_t* k, uint16_t* v, const float2* table,
                                const RopeGeom& g, int n_rows, int C, hipStream_t stream);
hipError_t launch_qkv_rope_f32(const float* x, const float* w, const float* bias, float* q, float* k,
                               float* v, const float2* table, const RopeGeom& g, int n_rows, int C,
                               int d, hipStream_t stream);

// Merge of partial results: out = sum_i exp(lse_i - lse) o_i, lse = log sum_i exp(lse_i), per
// (row, head).  Up to kMaxMergeParts parts; out and lse_out may alias any part.
constexpr int kMaxMergeParts = 16;
hipError_t launch_merge_bf16(int n_parts, const uint16_t* const* o, const float* const* lse,
                             long long rows_heads, int d, uint16_t* out, float* lse_out,
                             hipStream_t stream);
// Two fp32 parts into bf16 output, d = 128 (the key split of the fast attention launch).
hipError_t launch_merge2_f32_bf16(const float* o0, const float* o1, const float* lse0, const float* lse1,
                                  long long rows_heads, int d, uint16_t* out, float* lse_out,
                                  hipStream_t stream);
hipError_t launch_merge_f32(int n_parts, const float* const* o, const float* const* lse,
                            long long rows_heads, int d, float* out, float* lse_out,
                            hipStream_t stream);

}  // namespace st
