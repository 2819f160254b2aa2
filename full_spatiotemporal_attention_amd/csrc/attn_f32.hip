// fp32 checking kernel: 3D RoPE plus softmax attention over sets of rows, all in float32.
//
// Serves the ST_F32 mode of every entry point: full attention (one set of all N rows), the
// factorised spatial stage (T sets of the H*W rows of a frame), the temporal stage (H*W sets
// of the T rows at one position, "A video model's architecture: spatiotemporal attention and the
// 3D VAE", self-test answer 2), text cross-attention, runs of rows for partial results, and local
// 3D windows (one set per window).  It is a correctness mode, not a fast path: one thread per query
// row, rotated Q in LDS, K and V tiles in LDS, fp32 FMA dot products, expf.
#include "st_internal.h"

namespace st {
namespace {

constexpr int DMAX = 128;
constexpr int QB = 64;    // queries per workgroup (one per thread)
constexpr int KB = 64;    // keys per LDS tile
constexpr int SUB = 16;   // keys per softmax update

struct F32Params {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    float* lse;
    const float2* table;
    RopeGeom g;
    int heads;
    int d;
    F32Layout L;
    float scale;
};

__device__ __forceinline__ void row_pos(int n, const RopeGeom& g, int& t, int& h, int& w, bool& text) {
    text = n >= g.Nv;
    t = h = w = 0;
    if (!text) decode_pos(n, g, t, h, w);
}

__global__ void __launch_bounds__(QB) attn_f32_kernel(F32Params p) {
    __shared__ float lds_q[DMAX * QB];   // [channel][query]
    __shared__ float lds_k[KB * DMAX];   // [key][channel]
    __shared__ float lds_v[KB * DMAX];

    const int tid = threadIdx.x;
    const int seq = blockIdx.y;
    const int head = blockIdx.z;
    const int d = p.d;
    const int half = d >> 1;
    const long long rs = (long long)p.heads * d;
    const RopeGeom& g = p.g;
    const F32Layout& L = p.L;
    const int q0 = L.win ? win_origin(seq, L.wm) : seq * L.q_mul;
    const int kv0 = L.win ? q0 : seq * L.kv_mul;
    // buffer row of the i-th query (key) of this set
    auto q_row_of = [&](int i) { return L.win ? q0 + win_offset(i, L.wm) : q0 + i * L.q_stride; };
    auto kv_row_of = [&](int i) { return L.win ? kv0 + win_offset(i, L.wm) : kv0 + i * L.kv_stride; };

    const int qi = blockIdx.x * QB + tid;
    const bool qv = qi < L.q_len;
    const int qrow = q_row_of(qv ? qi : 0);   // query buffer row
    {
        int t, h, w;
        bool text;
        row_pos(L.q_pos_base + qrow, g, t, h, w, text);
        const float* qp = p.q + qrow * rs + (long long)head * d;
        for (int pp = 0; pp < half; ++pp) {
            float2 x = qv ? *reinterpret_cast<const float2*>(qp + 2 * pp) : make_float2(0.f, 0.f);
            rotate_pair(x.x, x.y, p.table[pair_entry(pp, t, h, w, g)]);
            lds_q[(2 * pp) * QB + tid] = x.x;
            lds_q[(2 * pp + 1) * QB + tid] = x.y;
        }
    }

    float o[DMAX];
#pragma unroll
    for (int c = 0; c < DMAX; ++c) o[c] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    for (int k0 = 0; k0 < L.kv_len; k0 += KB) {
        const int nk = min(KB, L.kv_len - k0);
        __syncthreads();
        for (int idx = tid; idx < nk * half; idx += QB) {
            const int r = idx / half;
            const int pp = idx - r * half;
            const int krow = kv_row_of(k0 + r);   // key buffer row
            int t, h, w;
            bool text;
            row_pos(L.kv_pos_base + krow, g, t, h, w, text);
            const long long base = krow * rs + (long long)head * d + 2 * pp;
            float2 x = *reinterpret_cast<const float2*>(p.k + base);
            rotate_pair(x.x, x.y, p.table[pair_entry(pp, t, h, w, g)]);
            lds_k[r * DMAX + 2 * pp] = x.x;
            lds_k[r * DMAX + 2 * pp + 1] = x.y;
            float2 vv = *reinterpret_cast<const float2*>(p.v + base);
            lds_v[r * DMAX + 2 * pp] = vv.x;
            lds_v[r * DMAX + 2 * pp + 1] = vv.y;
        }
        __syncthreads();
        for (int j0 = 0; j0 < nk; j0 += SUB) {
            float sc[SUB];
            float mx = -INFINITY;
#pragma unroll
            for (int jj = 0; jj < SUB; ++jj) {
                const int j = j0 + jj;
                float s = -INFINITY;
                if (j < nk) {
                    float acc = 0.0f;
                    for (int c = 0; c < d; ++c) acc = fmaf(lds_q[c * QB + tid], lds_k[j * DMAX + c], acc);
                    s = acc * p.scale;
                }
                sc[jj] = s;
                mx = fmaxf(mx, s);
            }
            const float m_new = fmaxf(m_run, mx);
            const float alpha = expf(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) o[c] *= alpha;
#pragma unroll
            for (int jj = 0; jj < SUB; ++jj) {
                const int j = j0 + jj;
                if (j < nk) {
                    const float pj = expf(sc[jj] - m_new);
                    l_run += pj;
#pragma unroll
                    for (int c = 0; c < DMAX; ++c)
                        if (c < d) o[c] = fmaf(pj, lds_v[j * DMAX + c], o[c]);
                }
            }
            m_run = m_new;
        }
    }

    if (qv && p.lse) p.lse[(long long)qrow * p.heads + head] = m_run + logf(l_run);
    if (qv) {
        const float inv = 1.0f / l_run;
        float* op = p.out + qrow * rs + (long long)head * d;
#pragma unroll
        for (int c = 0; c < DMAX; ++c)
            if (c < d) op[c] = o[c] * inv;
    }
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                           const float2* table, const RopeGeom& g, int heads, int d,
                           const F32Layout& L, hipStream_t stream) {
    F32Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.table = table;
    p.g = g;
    p.heads = heads;
    p.d = d;
    p.L = L;
    p.scale = 1.0f / sqrtf((float)d);
    dim3 grid((L.q_len + QB - 1) / QB, L.n_seqs, heads);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(QB), 0, stream, p);
    return hipGetLastError();
}

}  // namespace st
