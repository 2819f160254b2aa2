// Merge of partial attention results over disjoint runs of keys.
//
// Context parallelism splits the keys of one long sequence across devices (the CogVideoX record
// page, "Budget for that cost, because it grows": 2D ring and Ulysses); a device that saw one run
// of keys holds o_i = softmax over that run times v and lse_i = log sum over the run of
// exp(s / sqrt(d)).  The result over all keys is lse = log sum_i exp(lse_i) and
// o = sum_i exp(lse_i - lse) o_i, per (row, head).  HBM-bound: each part is read once, the
// output written once.
//
// Thread layout: the channels of one (row, head) are spread over a power-of-two group of lanes
// (16 bytes per lane) inside one wavefront, so every lane of the group has read the lse values
// before any lane writes: out and lse_out may alias any part (an in-place running merge).
#include "st_internal.h"

namespace st {
namespace {

template <typename T>
struct MergeParams {
    const T* o[kMaxMergeParts];
    const float* lse[kMaxMergeParts];
    int n_parts;
    long long rows_heads;
    int d;
    int chunks;        // 16-byte chunks per (row, head)
    int group_log2;    // lanes per (row, head) = 1 << group_log2 >= chunks
    T* out;
    float* lse_out;
};

__device__ __forceinline__ void load_chunk(const uint16_t* p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}
__device__ __forceinline__ void store_chunk(uint16_t* p, const float (&x)[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                             pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ void load_chunk(const float* p, float (&x)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
}
__device__ __forceinline__ void store_chunk(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void unpack_chunk(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}
__device__ __forceinline__ void unpack_chunk(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
}

// NP > 0: exactly NP parts.  Every part's chunk is requested before the log-sum-exps, so a thread
// waits for one memory round trip, not two; the chunk registers are sized for NP.  NP = 0: any
// p.n_parts up to kMaxMergeParts, chunks loaded after the weights (registers for 16 chunks would
// halve the occupancy; with 8 parts the bf16 kernel would already drop to 5 waves per SIMD).
template <typename T, int E, int NP>
__global__ void __launch_bounds__(256) merge_kernel(MergeParams<T> p) {
    constexpr int MP = NP > 0 ? NP : kMaxMergeParts;
    const int n_parts = NP > 0 ? NP : p.n_parts;
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rh = tid >> p.group_log2;
    const int c = (int)(tid & ((1 << p.group_log2) - 1));
    if (rh >= p.rows_heads) return;
    const bool active = c < p.chunks;
    const long long off = rh * p.d + (long long)c * E;
    uint4 raw[NP > 0 ? NP : 1];
    if constexpr (NP > 0) {
#pragma unroll
        for (int i = 0; i < NP; ++i)
            if (active) raw[i] = *reinterpret_cast<const uint4*>(p.o[i] + off);
    }
    float m = -INFINITY;
    float l[MP];
#pragma unroll
    for (int i = 0; i < MP; ++i) {
        l[i] = i < n_parts ? p.lse[i][rh] : -INFINITY;
        m = fmaxf(m, l[i]);
    }
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < MP; ++i) {
        l[i] = (i < n_parts && m > -INFINITY) ? expf(l[i] - m) : 0.0f;
        tot += l[i];
    }
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    if (active) {
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < MP; ++i) {
            if (i < n_parts) {
                float x[E];
                if constexpr (NP > 0)
                    unpack_chunk(raw[i], x);
                else
                    load_chunk(p.o[i] + off, x);
                const float w = l[i] * inv;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] = fmaf(w, x[e], acc[e]);
            }
        }
        store_chunk(p.out + off, acc);
    }
    if (c == 0 && p.lse_out) p.lse_out[rh] = tot > 0.0f ? m + logf(tot) : -INFINITY;
}

template <typename T, int E>
hipError_t launch_merge(int n_parts, const T* const* o, const float* const* lse, long long rows_heads,
                        int d, T* out, float* lse_out, hipStream_t stream) {
    MergeParams<T> p;
    for (int i = 0; i < kMaxMergeParts; ++i) {
        p.o[i] = i < n_parts ? o[i] : nullptr;
        p.lse[i] = i < n_parts ? lse[i] : nullptr;
    }
    p.n_parts = n_parts;
    p.rows_heads = rows_heads;
    p.d = d;
    p.chunks = d / E;
    p.group_log2 = 0;
    while ((1 << p.group_log2) < p.chunks) ++p.group_log2;
    p.out = out;
    p.lse_out = lse_out;
    const long long threads = rows_heads << p.group_log2;
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (n_parts) {
        case 2: hipLaunchKernelGGL((merge_kernel<T, E, 2>), grid, dim3(256), 0, stream, p); break;
        case 3: hipLaunchKernelGGL((merge_kernel<T, E, 3>), grid, dim3(256), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((merge_kernel<T, E, 4>), grid, dim3(256), 0, stream, p); break;
        default: hipLaunchKernelGGL((merge_kernel<T, E, 0>), grid, dim3(256), 0, stream, p); break;
    }
    return hipGetLastError();
}

// Two fp32 parts into bf16 (the key split of the fast attention launch, d = 128): 16 threads per
// (row, head), 8 channels each.
__global__ void __launch_bounds__(256) merge2_f32_bf16_kernel(const float* o0, const float* o1,
                                                              const float* lse0, const float* lse1,
                                                              long long rows_heads, uint16_t* out,
                                                              float* lse_out) {
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rh = tid >> 4;
    if (rh >= rows_heads) return;
    const long long off = rh * 128 + (tid & 15) * 8;
    const float4 a0 = *reinterpret_cast<const float4*>(o0 + off);
    const float4 a1 = *reinterpret_cast<const float4*>(o0 + off + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(o1 + off);
    const float4 b1 = *reinterpret_cast<const float4*>(o1 + off + 4);
    const float l0 = lse0[rh], l1 = lse1[rh];
    const float m = fmaxf(l0, l1);
    const float e0 = expf(l0 - m), e1 = expf(l1 - m);
    const float tot = e0 + e1;
    const float w0 = e0 / tot, w1 = e1 / tot;
    *reinterpret_cast<uint4*>(out + off) =
        make_uint4(pack_bf16x2(fmaf(w0, a0.x, w1 * b0.x), fmaf(w0, a0.y, w1 * b0.y)),
                   pack_bf16x2(fmaf(w0, a0.z, w1 * b0.z), fmaf(w0, a0.w, w1 * b0.w)),
                   pack_bf16x2(fmaf(w0, a1.x, w1 * b1.x), fmaf(w0, a1.y, w1 * b1.y)),
                   pack_bf16x2(fmaf(w0, a1.z, w1 * b1.z), fmaf(w0, a1.w, w1 * b1.w)));
    if ((tid & 15) == 0 && lse_out) lse_out[rh] = m + logf(tot);
}

}  // namespace

hipError_t launch_merge2_f32_bf16(const float* o0, const float* o1, const float* lse0, const float* lse1,
                                  long long rows_heads, int d, uint16_t* out, float* lse_out,
                                  hipStream_t stream) {
    if (d != 128) return hipErrorInvalidValue;
    const long long threads = rows_heads * 16;
    hipLaunchKernelGGL(merge2_f32_bf16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       o0, o1, lse0, lse1, rows_heads, out, lse_out);
    return hipGetLastError();
}

hipError_t launch_merge_bf16(int n_parts, const uint16_t* const* o, const float* const* lse,
                             long long rows_heads, int d, uint16_t* out, float* lse_out,
                             hipStream_t stream) {
    return launch_merge<uint16_t, 8>(n_parts, o, lse, rows_heads, d, out, lse_out, stream);
}

hipError_t launch_merge_f32(int n_parts, const float* const* o, const float* const* lse,
                            long long rows_heads, int d, float* out, float* lse_out,
                            hipStream_t stream) {
    return launch_merge<float, 4>(n_parts, o, lse, rows_heads, d, out, lse_out, stream);
}

}  // namespace st
