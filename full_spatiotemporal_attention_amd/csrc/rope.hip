// 3D RoPE: the angle table and the stand-alone rotation kernels.
//
// The rotation follows "A video model's architecture: spatiotemporal attention and the 3D VAE"
// (self-test answer 4, "Position: RoPE in three dimensions": the head dimension is cut into a t,
// an h and a w range, each rotated by its coordinate) and "CogVideoX Architecture: ...", section
// "3. 3D Rotary Position Embeddings (3D RoPE)" (block-diagonal R_3D = diag(R_t, R_y, R_x)).
// Pair j of a range of d_a channels turns by pos * theta^(-2j / d_a); the pages do not fix this
// schedule, it is the per-axis form of ordinary 1D RoPE.
#include "st_internal.h"

namespace st {

// One thread per table entry.  Angles are formed and evaluated in fp64 and rounded once to
// fp32, so the table error is half an fp32 ulp whatever the position.
__global__ void rope_table_kernel(RopeGeom g, double theta, float2* __restrict__ table) {
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e > g.identity) return;
    if (e == g.identity) {
        table[e] = make_float2(1.0f, 0.0f);
        return;
    }
    int a = (e >= g.off[1]) + (e >= g.off[2]);
    int P = g.pairs[a];
    int rem = e - g.off[a];
    int pos = rem / P;
    int j = rem - pos * P;
    double omega = pow(theta, -2.0 * (double)j / (double)(2 * P));
    double phi = (double)pos * omega;
    table[e] = make_float2((float)cos(phi), (float)sin(phi));
}

hipError_t launch_rope_table(const RopeGeom& g, double theta, float2* table, hipStream_t stream) {
    int total = g.identity + 1;
    int threads = 256;
    int blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(threads), 0, stream, g, theta, table);
    return hipGetLastError();
}

// bf16 (d = 128): one wave per row.  Lane l takes the 16-byte chunk c = l % 16 (channels 8c ..
// 8c+7, pairs 4c .. 4c+3) of heads l / 16, l / 16 + 4, ...: the row's position is decoded once
// per wave, and the lane's four table entries serve every head of the row.  HBM bound: every
// input byte is read once and every output byte written once.  x and y may be the same buffer:
// each lane reads its 16 bytes before writing them back.  Text rows take position (0, 0, 0),
// whose angles are 0: they are copied unchanged.
__global__ void __launch_bounds__(256) rope_apply_bf16_kernel(const uint16_t* x,
                                                              uint16_t* y, RopeGeom g,
                                                              int N, int heads,
                                                              const float2* __restrict__ table) {
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int h0 = lane >> 4;
    const int waves = gridDim.x * 4;
    for (int n = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (int)(threadIdx.x >> 6)); n < N; n += waves) {
        int t = 0, h = 0, w = 0;
        if (n < g.Nv) decode_pos(n, g, t, h, w);
        float2 cs[4];
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) cs[pi] = table[pair_entry(4 * c + pi, t, h, w, g)];
        const long long rb = (long long)n * heads * 128 + 8 * c;   // (row n, head 0, chunk c)
        // Up to 16 heads per pass; all of a pass's loads are issued before its first store (x and
        // y may alias, so the compiler would not move a load above an earlier store).
        for (int hb = 0; hb < heads; hb += 16) {
            uint4 raw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int hd = hb + h0 + 4 * k;
                if (hd < heads) raw[k] = *reinterpret_cast<const uint4*>(x + rb + (long long)hd * 128);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int hd = hb + h0 + 4 * k;
                if (hd < heads) {
                    uint32_t wds[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
                    for (int pi = 0; pi < 4; ++pi) {
                        float x0 = bf16_lo(wds[pi]), x1 = bf16_hi(wds[pi]);
                        rotate_pair(x0, x1, cs[pi]);
                        wds[pi] = pack_bf16x2(x0, x1);
                    }
                    *reinterpret_cast<uint4*>(y + rb + (long long)hd * 128) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
                }
            }
        }
    }
}

// bf16, any d % 8 == 0 other than 128: one wave per row, lane l takes the row's 16-byte chunks
// l, l + 64, ... (chunk ci is chunk ci % (d/8) of head ci / (d/8)); each chunk looks up its own
// four table entries.  All of a pass's loads are issued before its stores, as above.
__global__ void __launch_bounds__(256) rope_apply_bf16_any_kernel(const uint16_t* x, uint16_t* y,
                                                                  RopeGeom g, int N, int heads,
                                                                  int d,
                                                                  const float2* __restrict__ table) {
    const int lane = threadIdx.x & 63;
    const int cpr = d >> 3;                 // chunks per head
    const int chunks = heads * cpr;         // chunks per row
    const int waves = gridDim.x * 4;
    for (int n = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (int)(threadIdx.x >> 6)); n < N; n += waves) {
        int t = 0, h = 0, w = 0;
        if (n < g.Nv) decode_pos(n, g, t, h, w);
        const long long rb = (long long)n * chunks * 8;
        for (int cb = 0; cb < chunks; cb += 256) {
            uint4 raw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int ci = cb + lane + 64 * k;
                if (ci < chunks) raw[k] = *reinterpret_cast<const uint4*>(x + rb + 8ll * ci);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int ci = cb + lane + 64 * k;
                if (ci < chunks) {
                    const int c = ci % cpr;
                    uint32_t wds[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
                    for (int pi = 0; pi < 4; ++pi) {
                        float x0 = bf16_lo(wds[pi]), x1 = bf16_hi(wds[pi]);
                        rotate_pair(x0, x1, table[pair_entry(4 * c + pi, t, h, w, g)]);
                        wds[pi] = pack_bf16x2(x0, x1);
                    }
                    *reinterpret_cast<uint4*>(y + rb + 8ll * ci) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
                }
            }
        }
    }
}

// fp32: one thread handles one pair (8 bytes).
__global__ void __launch_bounds__(256) rope_apply_f32_kernel(const float* x,
                                                             float* y, RopeGeom g,
                                                             int N, int heads, int d,
                                                             const float2* __restrict__ table) {
    const int pairs_per_row = d >> 1;
    const long long total = (long long)N * heads * pairs_per_row;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        long long rh = i / pairs_per_row;
        int p = (int)(i - rh * pairs_per_row);
        int n = (int)(rh / heads);
        int t = 0, h = 0, w = 0;
        bool text = n >= g.Nv;
        if (!text) decode_pos(n, g, t, h, w);
        float2 v = *reinterpret_cast<const float2*>(x + i * 2);
        rotate_pair(v.x, v.y, table[pair_entry(p, t, h, w, g)]);
        *reinterpret_cast<float2*>(y + i * 2) = v;
    }
}

static int stream_grid(long long work, int threads) {
    long long blocks = (work + threads - 1) / threads;
    const long long cap = 256LL * 16;  // 16 workgroups per CU is plenty to saturate HBM
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

hipError_t launch_rope_apply_bf16(const uint16_t* x, uint16_t* y, const RopeGeom& g, int N,
                                  int heads, int d, const float2* table, hipStream_t stream) {
    // One wave per row, four rows per workgroup, up to 64 rows per wave.
    long long blocks = ((long long)N + 3) / 4;
    const long long cap = 256LL * 128;
    if (blocks > cap) blocks = cap;
    if (d == 128)
        hipLaunchKernelGGL(rope_apply_bf16_kernel, dim3((int)blocks), dim3(256), 0, stream,
                           x, y, g, N, heads, table);
    else
        hipLaunchKernelGGL(rope_apply_bf16_any_kernel, dim3((int)blocks), dim3(256), 0, stream,
                           x, y, g, N, heads, d, table);
    return hipGetLastError();
}

hipError_t launch_rope_apply_f32(const float* x, float* y, const RopeGeom& g, int N, int heads,
                                 int d, const float2* table, hipStream_t stream) {
    long long work = (long long)N * heads * (d / 2);
    hipLaunchKernelGGL(rope_apply_f32_kernel, dim3(stream_grid(work, 256)), dim3(256), 0, stream,
                       x, y, g, N, heads, d, table);
    return hipGetLastError();
}

}  // namespace st
