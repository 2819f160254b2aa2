// C ABI of libstattn: argument checks, workspace layout and launch sequencing.
// The operations are described in include/st_attn.h.
#include "st_attn.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "st_internal.h"

namespace st {

RopeGeom make_geom(int T, int H, int W, const int split[3]) {
    RopeGeom g;
    g.T = T;
    g.H = H;
    g.W = W;
    g.S = H * W;
    g.Nv = T * H * W;
    g.inv_S = 1.0f / (float)g.S;
    g.inv_W = 1.0f / (float)W;
    for (int a = 0; a < 3; ++a) g.pairs[a] = split[a] / 2;
    g.first[0] = 0;
    g.first[1] = g.pairs[0];
    g.first[2] = g.pairs[0] + g.pairs[1];
    g.off[0] = 0;
    g.off[1] = T * g.pairs[0];
    g.off[2] = g.off[1] + H * g.pairs[1];
    g.identity = g.off[2] + W * g.pairs[2];
    return g;
}

WinMap make_winmap(int T, int H, int W, int wt, int wh, int ww) {
    (void)T;
    WinMap m;
    m.nW = W / ww;
    m.nHW = (H / wh) * m.nW;
    m.inv_nW = 1.0f / (float)m.nW;
    m.inv_nHW = 1.0f / (float)m.nHW;
    m.wS = wh * ww;
    m.ww = ww;
    m.inv_wS = 1.0f / (float)m.wS;
    m.inv_ww = 1.0f / (float)ww;
    m.A = H * W - wh * ww;
    m.B = W - ww;
    m.oa = wt * H * W;
    m.ob = wh * W;
    m.oc = ww;
    return m;
}

}  // namespace st

namespace {

thread_local int g_last_hip_error = 0;

constexpr long long kMaxRows = 1LL << 24;
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool grid_ok(int T, int H, int W, int n_text, long long* n_out) {
    if (T < 1 || H < 1 || W < 1 || n_text < 0) return false;
    long long nv = (long long)T * H * W;
    long long n = nv + n_text;
    if (n >= kMaxRows) return false;
    if (n_out) *n_out = n;
    return true;
}

st_status check_split(const int* split, int d) {
    if (!split) return ST_ERR_NULL;
    long long sum = 0;
    for (int a = 0; a < 3; ++a) {
        if (split[a] < 0 || (split[a] & 1)) return ST_ERR_SPLIT;
        sum += split[a];
    }
    if (sum != d) return ST_ERR_SPLIT;
    return ST_OK;
}

size_t table_bytes_for(int T, int H, int W, const int* split) {
    long long entries = (long long)T * (split[0] / 2) + (long long)H * (split[1] / 2) +
                        (long long)W * (split[2] / 2) + 1;
    return align_up((size_t)entries * sizeof(float2), kWsAlign);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

size_t elem_size(st_dtype dt) { return dt == ST_BF16 ? 2 : 4; }

bool theta_ok(float theta) { return isfinite(theta) && theta > 0.0f; }

// A C caller may pass any int as st_dtype; in C++ loading an enum value outside its enumerators'
// range is undefined, so the entry points check the code through its bytes before using it.
bool dtype_known(const st_dtype& dt) {
    int code;
    memcpy(&code, &dt, sizeof code);
    return code == ST_BF16 || code == ST_F32;
}

// Checks shared by the attention entry points (tensor pointers, shapes, dtype, split, aliasing).
st_status check_attn(const void* q, const void* k, const void* v, const void* out, int T, int H,
                     int W, int n_text, int heads, int d, const int* split, st_dtype dtype,
                     long long* n_out) {
    if (!q || !k || !v || !out) return ST_ERR_NULL;
    if (!split) return ST_ERR_NULL;
    long long n = 0;
    if (!grid_ok(T, H, W, n_text, &n)) return ST_ERR_SHAPE;
    *n_out = n;
    if (heads < 1 || d < 2 || (d & 1)) return ST_ERR_SHAPE;
    if ((long long)n * heads * d >= (1LL << 40)) return ST_ERR_SHAPE;
    st_status s = check_split(split, d);
    if (s != ST_OK) return s;
    if (dtype == ST_BF16) {
        if (d != 128) return ST_ERR_UNSUPPORTED;
    } else if (dtype == ST_F32) {
        if (d > 128) return ST_ERR_UNSUPPORTED;
    } else {
        return ST_ERR_UNSUPPORTED;
    }
    if (heads > 65535) return ST_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return ST_ERR_ALIGN;
    size_t bytes = (size_t)n * heads * d * elem_size(dtype);
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
        overlaps(out, bytes, v, bytes))
        return ST_ERR_ALIAS;
    return ST_OK;
}

// One problem of n query rows against the same n key rows (full attention).
st::SeqLayout self_layout(int n) {
    st::SeqLayout L;
    L.n_segs = 1;
    L.q_len = n;
    L.kv_len = n;
    L.q_pos_base = 0;
    L.kv_pos_base = 0;
    return L;
}

st::F32Layout f32_layout(int n_seqs, int q_len, int q_mul, int q_stride, int kv_len, int kv_mul,
                         int kv_stride, int q_pos_base = 0, int kv_pos_base = 0) {
    st::F32Layout L;
    L.n_seqs = n_seqs;
    L.q_len = q_len;
    L.q_mul = q_mul;
    L.q_stride = q_stride;
    L.q_pos_base = q_pos_base;
    L.kv_len = kv_len;
    L.kv_mul = kv_mul;
    L.kv_stride = kv_stride;
    L.kv_pos_base = kv_pos_base;
    L.win = 0;
    L.wm = st::WinMap{};
    return L;
}

// Table of the cross-attention geometry (1x1x1 grid, every pair on the t axis): d/2 zero angles
// and the identity entry.
size_t cross_table_bytes(int d) {
    const int t_only[3] = {d, 0, 0};
    return table_bytes_for(1, 1, 1, t_only);
}

// bf16 cross-attention workspace after the table: the fp16 key tiles, then the fast launch's
// flags (8 bytes per 256-row query block and head).
size_t cross_tiles_bytes(int n_kv, int heads) {
    return align_up(st::attn_stage_elems(heads, n_kv, 1) * 2, kWsAlign);
}

st_status hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return ST_ERR_HIP;
}

// Byte layout of the bf16 staged workspace: [table][K~ tiles][item flags], each 256-aligned.  The
// flags (8 bytes per 256-row query block of each sequence and head, and the buffers of a key split
// when the attention launch splits) are scratch of the attention launches; sequences are
// self-attention ones (query rows = key rows = seg_len).
struct StageLayout {
    size_t table_bytes;
    size_t tiles_bytes;
    size_t flags_bytes;
    size_t total;
    size_t flags_offset() const { return table_bytes + tiles_bytes; }
};

StageLayout stage_layout(int T, int H, int W, int heads, int seg_len, int n_segs, const int* split,
                         bool with_flags = true) {
    StageLayout L;
    L.table_bytes = table_bytes_for(T, H, W, split);
    L.tiles_bytes = align_up(st::attn_stage_elems(heads, seg_len, n_segs) * 2, kWsAlign);
    L.flags_bytes = with_flags ? align_up(st::attn_flag_bytes(heads, seg_len, seg_len, n_segs), kWsAlign) : 0;
    L.total = L.table_bytes + L.tiles_bytes + L.flags_bytes;
    return L;
}

bool ws_overlaps_tensors(const void* ws, size_t ws_bytes, size_t tensor_bytes, const void* a,
                         const void* b, const void* c, const void* d) {
    const void* ts[4] = {a, b, c, d};
    for (const void* t : ts)
        if (t && overlaps(ws, ws_bytes, t, tensor_bytes)) return true;
    return false;
}

// ---- scratch of the allocation-free entry point ------------------------------------------------
// Every GPU the library runs on holds one copy of `scratch` (ST_NOALLOC_SCRATCH_BYTES, from module
// load until the process ends).  In host code the array's name is only a stand-in: its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[ST_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (null and the HIP error on failure).
void* scratch_on_current_device(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { *err = e; return nullptr; }
    if (dev < 0 || dev >= kMaxDevices) { *err = hipErrorInvalidDevice; return nullptr; }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) { *err = e != hipSuccess ? e : hipErrorInvalidSymbol; return nullptr; }
        g_scratch_ptr[dev] = ptr;
    }
    *err = hipSuccess;
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t st_rope3d_table_bytes(int T, int H, int W, const int rope_split[3]) {
    if (!rope_split || !grid_ok(T, H, W, 0, nullptr)) return 0;
    for (int a = 0; a < 3; ++a)
        if (rope_split[a] < 0 || (rope_split[a] & 1)) return 0;
    return table_bytes_for(T, H, W, rope_split);
}

st_status st_rope3d_table_build(int T, int H, int W, const int rope_split[3], float theta,
                                void* table, size_t table_bytes, hipStream_t stream) {
    if (!rope_split || !table) return ST_ERR_NULL;
    if (!grid_ok(T, H, W, 0, nullptr)) return ST_ERR_SHAPE;
    for (int a = 0; a < 3; ++a)
        if (rope_split[a] < 0 || (rope_split[a] & 1)) return ST_ERR_SPLIT;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!aligned(table, kWsAlign)) return ST_ERR_ALIGN;
    if (table_bytes < table_bytes_for(T, H, W, rope_split)) return ST_ERR_WORKSPACE;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    hipError_t e = st::launch_rope_table(g, (double)theta, (float2*)table, stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

size_t st_attn3d_workspace_bytes(int T, int H, int W, int n_text, int heads, int d,
                                 const int rope_split[3], st_dtype dtype) {
    if (!dtype_known(dtype)) return 0;
    long long n = 0;
    if (!rope_split || !grid_ok(T, H, W, n_text, &n) || heads < 1) return 0;
    if (check_split(rope_split, d) != ST_OK) return 0;
    if (dtype == ST_F32) return d <= 128 ? table_bytes_for(T, H, W, rope_split) : 0;
    if (dtype != ST_BF16 || d != 128) return 0;
    return stage_layout(T, H, W, heads, (int)n, 1, rope_split).total;
}

size_t st_attn3d_fused_workspace_bytes(int T, int H, int W, const int rope_split[3]) {
    return st_rope3d_table_bytes(T, H, W, rope_split);
}

st_status st_attn3d_stage(const void* k, int T, int H, int W, int n_text, int heads, int d,
                          const int rope_split[3], float theta, st_dtype dtype, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    // Only k is read by this step; it stands in for q and v in the shared checks.
    st_status s = check_attn(k, k, k, workspace, T, H, W, n_text, heads, d, rope_split, dtype, &n);
    if (s == ST_ERR_ALIAS) s = ST_OK;  // workspace aliasing is checked below with its true size
    if (s != ST_OK) return s;
    if (dtype != ST_BF16) return ST_ERR_UNSUPPORTED;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    StageLayout L = stage_layout(T, H, W, heads, (int)n, 1, rope_split);
    if (ws_bytes < L.total) return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * 2, k, nullptr, nullptr, nullptr))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    char* ws = (char*)workspace;
    float2* table = (float2*)ws;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    e = st::launch_k_prep((const uint16_t*)k, (uint16_t*)(ws + L.table_bytes), table, g, heads,
                          self_layout((int)n), stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

st_status st_attn3d_attend(const void* q, const void* v, int T, int H, int W, int n_text, int heads,
                           int d, const int rope_split[3], st_dtype dtype, void* workspace,
                           size_t ws_bytes, void* out, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    if (!workspace) return ST_ERR_NULL;
    st_status s = check_attn(q, q, v, out, T, H, W, n_text, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (dtype != ST_BF16) return ST_ERR_UNSUPPORTED;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    StageLayout L = stage_layout(T, H, W, heads, (int)n, 1, rope_split);
    if (ws_bytes < L.total) return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * 2, q, v, out, nullptr))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    char* ws = (char*)workspace;
    hipError_t e = st::launch_attn_bf16_staged((const uint16_t*)q, (const uint16_t*)(ws + L.table_bytes),
                                               (const uint16_t*)v, (uint16_t*)out, nullptr,
                                               (const float2*)ws, g, heads, self_layout((int)n),
                                               (uint8_t*)(ws + L.flags_offset()), stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

st_status st_attn3d_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                        int n_text, int heads, int d, const int rope_split[3], float theta,
                        st_dtype dtype, void* workspace, size_t ws_bytes, void* out,
                        hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    st_status s = check_attn(q, k, v, out, T, H, W, n_text, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!workspace) return ST_ERR_NULL;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    if (ws_bytes < st_attn3d_workspace_bytes(T, H, W, n_text, heads, d, rope_split, dtype))
        return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * elem_size(dtype), q, k, v, out))
        return ST_ERR_ALIAS;
    if (dtype == ST_BF16) {
        s = st_attn3d_stage(k, T, H, W, n_text, heads, d, rope_split, theta, dtype, workspace,
                            ws_bytes, stream);
        if (s != ST_OK) return s;
        return st_attn3d_attend(q, v, T, H, W, n_text, heads, d, rope_split, dtype, workspace,
                                ws_bytes, out, stream);
    }
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    float2* table = (float2*)workspace;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, nullptr,
                            table, g, heads, d, f32_layout(1, (int)n, 0, 1, (int)n, 0, 1), stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

size_t st_attn3d_noalloc_scratch_bytes(void) { return ST_NOALLOC_SCRATCH_BYTES; }

st_status st_attn3d_fwd_noalloc(const void* q, const void* k, const void* v, int T, int H, int W,
                                int n_text, int heads, int d, const int rope_split[3], float theta,
                                st_dtype dtype, void* out, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    st_status s = check_attn(q, k, v, out, T, H, W, n_text, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    const size_t need = st_attn3d_workspace_bytes(T, H, W, n_text, heads, d, rope_split, dtype);
    if (need == 0) return ST_ERR_SHAPE;
    if (need > ST_NOALLOC_SCRATCH_BYTES) return ST_ERR_WORKSPACE;
    // The scratch is per device: the stream's device (the current one for the null stream) is
    // made current for the address lookup and the launches, and the caller's device restored.
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return hip_fail(e);
        dev = (int)sd;
    }
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
    void* ws = scratch_on_current_device(&e);
    // The same launches as st_attn3d_fwd with the scratch as its workspace (no byte of it needs to
    // start at zero: the table and the staged tiles are written whole, every block flag is
    // rewritten by the attention launch that reads it).
    const st_status r = ws ? st_attn3d_fwd(q, k, v, T, H, W, n_text, heads, d, rope_split, theta, dtype,
                                           ws, need, out, stream)
                           : hip_fail(e);
    if (dev != cur) hipSetDevice(cur);
    return r;
}

st_status st_attn3d_fwd_fused(const void* q, const void* k, const void* v, int T, int H, int W,
                              int n_text, int heads, int d, const int rope_split[3], float theta,
                              st_dtype dtype, void* workspace, size_t ws_bytes, void* out,
                              hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    st_status s = check_attn(q, k, v, out, T, H, W, n_text, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!workspace) return ST_ERR_NULL;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    if (ws_bytes < table_bytes_for(T, H, W, rope_split)) return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * elem_size(dtype), q, k, v, out))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    float2* table = (float2*)workspace;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16)
        e = st::launch_attn_bf16_fused((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                       (uint16_t*)out, nullptr, table, g, heads, self_layout((int)n),
                                       stream);
    else
        e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, nullptr,
                                table, g, heads, d, f32_layout(1, (int)n, 0, 1, (int)n, 0, 1), stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

size_t st_attn_factorized_workspace_bytes(int T, int H, int W, int heads, int d,
                                          const int rope_split[3], st_dtype dtype) {
    if (!dtype_known(dtype)) return 0;
    if (!rope_split || heads < 1 || d < 2 || (d & 1)) return 0;
    long long n = 0;
    if (!grid_ok(T, H, W, 0, &n)) return 0;
    if (check_split(rope_split, d) != ST_OK) return 0;
    size_t os = align_up((size_t)n * heads * d * elem_size(dtype), kWsAlign);
    if (dtype == ST_F32) return d <= 128 ? table_bytes_for(T, H, W, rope_split) + os : 0;
    if (dtype != ST_BF16 || d != 128) return 0;
    return stage_layout(T, H, W, heads, H * W, T, rope_split).total + os;
}

st_status st_attn_factorized_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                                 int heads, int d, const int rope_split[3], float theta,
                                 st_dtype dtype, void* workspace, size_t ws_bytes, void* out,
                                 hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    st_status s = check_attn(q, k, v, out, T, H, W, 0, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!workspace) return ST_ERR_NULL;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    if (dtype == ST_F32 && ((long long)H * W > 65535 || T > 65535)) return ST_ERR_SHAPE;
    size_t need = st_attn_factorized_workspace_bytes(T, H, W, heads, d, rope_split, dtype);
    if (need == 0) return ST_ERR_SHAPE;
    if (ws_bytes < need) return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * elem_size(dtype), q, k, v, out))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    char* ws = (char*)workspace;
    float2* table = (float2*)ws;
    const int S = H * W;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16) {
        StageLayout L = stage_layout(T, H, W, heads, S, T, rope_split);
        uint16_t* kt = (uint16_t*)(ws + L.table_bytes);
        uint16_t* o_s = (uint16_t*)(ws + L.total);
        st::SeqLayout SL;
        SL.n_segs = T;
        SL.q_len = S;
        SL.kv_len = S;
        SL.q_pos_base = 0;
        SL.kv_pos_base = 0;
        e = st::launch_k_prep((const uint16_t*)k, kt, table, g, heads, SL, stream);
        if (e != hipSuccess) return hip_fail(e);
        e = st::launch_attn_bf16_staged((const uint16_t*)q, kt, (const uint16_t*)v, o_s, nullptr, table,
                                        g, heads, SL, (uint8_t*)(ws + L.flags_offset()), stream);
        if (e != hipSuccess) return hip_fail(e);
        e = st::launch_attn_temporal_bf16((const uint16_t*)q, (const uint16_t*)k, kt, o_s,
                                          (uint16_t*)out, table, g, heads, stream);
    } else {
        float* o_s = (float*)(ws + table_bytes_for(T, H, W, rope_split));
        e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, o_s, nullptr, table,
                                g, heads, d, f32_layout(T, S, S, 1, S, S, 1), stream);
        if (e != hipSuccess) return hip_fail(e);
        e = st::launch_attn_f32((const float*)q, (const float*)k, o_s, (float*)out, nullptr, table, g,
                                heads, d, f32_layout(S, T, 1, S, T, 1, S), stream);
    }
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

size_t st_attn3d_window_workspace_bytes(int T, int H, int W, int heads, int d,
                                        const int rope_split[3], const int window[3],
                                        st_dtype dtype) {
    if (!dtype_known(dtype)) return 0;
    long long n = 0;
    if (!rope_split || !window || heads < 1 || !grid_ok(T, H, W, 0, &n)) return 0;
    if (check_split(rope_split, d) != ST_OK) return 0;
    const int dims[3] = {T, H, W};
    for (int a = 0; a < 3; ++a)
        if (window[a] < 1 || dims[a] % window[a]) return 0;
    if (dtype == ST_F32) return d <= 128 ? table_bytes_for(T, H, W, rope_split) : 0;
    if (dtype != ST_BF16 || d != 128) return 0;
    const int L = window[0] * window[1] * window[2];
    return stage_layout(T, H, W, heads, L, (int)(n / L), rope_split).total;
}

st_status st_attn3d_window_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                               int heads, int d, const int rope_split[3], float theta,
                               const int window[3], st_dtype dtype, void* workspace,
                               size_t ws_bytes, void* out, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    long long n = 0;
    st_status s = check_attn(q, k, v, out, T, H, W, 0, heads, d, rope_split, dtype, &n);
    if (s != ST_OK) return s;
    if (!window) return ST_ERR_NULL;
    const int dims[3] = {T, H, W};
    for (int a = 0; a < 3; ++a)
        if (window[a] < 1 || dims[a] % window[a]) return ST_ERR_SHAPE;
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!workspace) return ST_ERR_NULL;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    const int L = window[0] * window[1] * window[2];
    const int n_win = (int)(n / L);
    // bf16: value rows are addressed with 32-bit byte offsets from the tensor base.
    if (dtype == ST_BF16 && (unsigned long long)n * heads * d * 2 >= (1ULL << 32)) return ST_ERR_UNSUPPORTED;
    if (dtype == ST_F32 && n_win > 65535) return ST_ERR_SHAPE;
    size_t need = st_attn3d_window_workspace_bytes(T, H, W, heads, d, rope_split, window, dtype);
    if (need == 0) return ST_ERR_SHAPE;
    if (ws_bytes < need) return ST_ERR_WORKSPACE;
    if (ws_overlaps_tensors(workspace, ws_bytes, (size_t)n * heads * d * elem_size(dtype), q, k, v, out))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    st::WinMap m = st::make_winmap(T, H, W, window[0], window[1], window[2]);
    char* ws = (char*)workspace;
    float2* table = (float2*)ws;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16) {
        StageLayout SL = stage_layout(T, H, W, heads, L, n_win, rope_split);
        uint16_t* kt = (uint16_t*)(ws + SL.table_bytes);
        e = st::launch_k_prep_win((const uint16_t*)k, kt, table, g, heads, m, n_win, L, stream);
        if (e != hipSuccess) return hip_fail(e);
        e = st::launch_attn_bf16_win((const uint16_t*)q, kt, (const uint16_t*)v, (uint16_t*)out, table, g,
                                     heads, m, n_win, L, (uint8_t*)(ws + SL.flags_offset()), stream);
    } else {
        st::F32Layout FL = f32_layout(n_win, L, 0, 1, L, 0, 1);
        FL.win = 1;
        FL.wm = m;
        e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, nullptr,
                                table, g, heads, d, FL, stream);
    }
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

st_status st_rope3d_apply(const void* x, void* y, int T, int H, int W, int n_text, int heads,
                          int d, const int rope_split[3], float theta, st_dtype dtype,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    if (!x || !y || !rope_split || !workspace) return ST_ERR_NULL;
    long long n = 0;
    if (!grid_ok(T, H, W, n_text, &n)) return ST_ERR_SHAPE;
    if (heads < 1 || d < 2 || (d & 1)) return ST_ERR_SHAPE;
    st_status s = check_split(rope_split, d);
    if (s != ST_OK) return s;
    if (dtype == ST_BF16) {
        if (d % 8) return ST_ERR_UNSUPPORTED;
    } else if (dtype != ST_F32) {
        return ST_ERR_UNSUPPORTED;
    }
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(y, 16)) return ST_ERR_ALIGN;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    if (ws_bytes < table_bytes_for(T, H, W, rope_split)) return ST_ERR_WORKSPACE;
    size_t bytes = (size_t)n * heads * d * elem_size(dtype);
    if (x != y && overlaps(x, bytes, y, bytes)) return ST_ERR_ALIAS;
    if (overlaps(workspace, ws_bytes, x, bytes) || overlaps(workspace, ws_bytes, y, bytes))
        return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    float2* table = (float2*)workspace;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16)
        e = st::launch_rope_apply_bf16((const uint16_t*)x, (uint16_t*)y, g, (int)n, heads, d,
                                       table, stream);
    else
        e = st::launch_rope_apply_f32((const float*)x, (float*)y, g, (int)n, heads, d, table,
                                      stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

// ---- text cross-attention --------------------------------------------------------------------

size_t st_attn_cross_workspace_bytes(int n_q, int n_kv, int heads, int d, st_dtype dtype) {
    if (!dtype_known(dtype)) return 0;
    if (n_q < 1 || n_kv < 1 || n_q >= kMaxRows || n_kv >= kMaxRows || heads < 1 || heads > 65535)
        return 0;
    if (d < 2 || (d & 1)) return 0;
    const size_t table = cross_table_bytes(d);
    if (dtype == ST_F32) return (d >= 2 && !(d & 1) && d <= 128) ? table : 0;
    if (dtype != ST_BF16 || d != 128) return 0;
    return table + cross_tiles_bytes(n_kv, heads) + align_up(st::attn_flag_bytes(heads, n_q, n_kv, 1), kWsAlign);
}

st_status st_attn_cross_fwd(const void* q, const void* k, const void* v, int n_q, int n_kv,
                            int heads, int d, st_dtype dtype, void* workspace, size_t ws_bytes,
                            void* out, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    if (!q || !k || !v || !out || !workspace) return ST_ERR_NULL;
    if (n_q < 1 || n_kv < 1 || n_q >= kMaxRows || n_kv >= kMaxRows) return ST_ERR_SHAPE;
    if (heads < 1 || heads > 65535 || d < 2 || (d & 1)) return ST_ERR_SHAPE;
    if (dtype == ST_BF16) {
        if (d != 128) return ST_ERR_UNSUPPORTED;
    } else if (dtype == ST_F32) {
        if (d > 128) return ST_ERR_UNSUPPORTED;
    } else {
        return ST_ERR_UNSUPPORTED;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return ST_ERR_ALIGN;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    const size_t qb = (size_t)n_q * heads * d * elem_size(dtype);
    const size_t kb = (size_t)n_kv * heads * d * elem_size(dtype);
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kb) || overlaps(out, qb, v, kb))
        return ST_ERR_ALIAS;
    if (ws_bytes < st_attn_cross_workspace_bytes(n_q, n_kv, heads, d, dtype)) return ST_ERR_WORKSPACE;
    if (overlaps(workspace, ws_bytes, q, qb) || overlaps(workspace, ws_bytes, out, qb) ||
        overlaps(workspace, ws_bytes, k, kb) || overlaps(workspace, ws_bytes, v, kb))
        return ST_ERR_ALIAS;
    // A geometry with no video rows: every row is a text row, which the kernels treat as
    // position (0, 0, 0) or the identity entry; the table of a 1x1x1 grid with all pairs on the
    // t axis holds only zero angles.
    const int t_only[3] = {d, 0, 0};
    st::RopeGeom g = st::make_geom(1, 1, 1, t_only);
    g.Nv = 0;
    char* ws = (char*)workspace;
    float2* table = (float2*)ws;
    hipError_t e;
    if (dtype == ST_BF16) {
        st::SeqLayout L;
        L.n_segs = 1;
        L.q_len = n_q;
        L.kv_len = n_kv;
        L.q_pos_base = 0;
        L.kv_pos_base = 0;
        uint16_t* kt = (uint16_t*)(ws + cross_table_bytes(d));
        // The key staging launch writes the table of zero angles itself (no table launch).
        e = st::launch_k_prep((const uint16_t*)k, kt, table, g, heads, L, stream, table);
        if (e != hipSuccess) return hip_fail(e);
        uint8_t* flags = (uint8_t*)(ws + cross_table_bytes(d) + cross_tiles_bytes(n_kv, heads));
        e = st::launch_attn_bf16_staged((const uint16_t*)q, kt, (const uint16_t*)v, (uint16_t*)out,
                                        nullptr, table, g, heads, L, flags, stream);
    } else {
        e = st::launch_rope_table(g, 10000.0, table, stream);
        if (e != hipSuccess) return hip_fail(e);
        e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, nullptr,
                                table, g, heads, d, f32_layout(1, n_q, 0, 1, n_kv, 0, 1), stream);
    }
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

// ---- QKV projection with the rotation of q and k ------------------------------------------------

size_t st_qkv_rope_workspace_bytes(int T, int H, int W, const int rope_split[3]) {
    return st_rope3d_table_bytes(T, H, W, rope_split);
}

st_status st_qkv_rope_fwd(const void* x, const void* w, const void* bias, int T, int H, int W,
                          int n_text, int heads, int d, const int rope_split[3], float theta,
                          st_dtype dtype, void* workspace, size_t ws_bytes, void* q, void* k,
                          void* v, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    if (!x || !w || !q || !k || !v || !workspace || !rope_split) return ST_ERR_NULL;
    long long n = 0;
    if (!grid_ok(T, H, W, n_text, &n)) return ST_ERR_SHAPE;
    if (heads < 1 || heads > 65535 || d < 2 || (d & 1)) return ST_ERR_SHAPE;
    st_status s = check_split(rope_split, d);
    if (s != ST_OK) return s;
    const long long C = (long long)heads * d;
    if (dtype == ST_BF16) {
        if (d != 128) return ST_ERR_UNSUPPORTED;
        // 32-bit byte offsets inside the kernel
        if (n * C * 2 >= (1LL << 31) || 3 * C * C * 2 >= (1LL << 31)) return ST_ERR_SHAPE;
    } else if (dtype == ST_F32) {
        if (d > 128) return ST_ERR_UNSUPPORTED;
        if (n * C >= (1LL << 40)) return ST_ERR_SHAPE;
    } else {
        return ST_ERR_UNSUPPORTED;
    }
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        (bias && !aligned(bias, 8)))
        return ST_ERR_ALIGN;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    if (ws_bytes < st_qkv_rope_workspace_bytes(T, H, W, rope_split)) return ST_ERR_WORKSPACE;
    const size_t es = elem_size(dtype);
    const size_t xb = (size_t)(n * C) * es, wb = (size_t)(3 * C * C) * es, bb = (size_t)(3 * C) * es;
    const void* ins[3] = {x, w, bias};
    const size_t insz[3] = {xb, wb, bb};
    void* outs[3] = {q, k, v};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 3; ++i)
            if (ins[i] && overlaps(outs[o], xb, ins[i], insz[i])) return ST_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (overlaps(outs[o], xb, outs[o2], xb)) return ST_ERR_ALIAS;
        if (overlaps(workspace, ws_bytes, outs[o], xb)) return ST_ERR_ALIAS;
    }
    for (int i = 0; i < 3; ++i)
        if (ins[i] && overlaps(workspace, ws_bytes, ins[i], insz[i])) return ST_ERR_ALIAS;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    float2* table = (float2*)workspace;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16)
        e = st::launch_qkv_rope_bf16((const uint16_t*)x, (const uint16_t*)w, (const uint16_t*)bias,
                                     (uint16_t*)q, (uint16_t*)k, (uint16_t*)v, table, g, (int)n,
                                     (int)C, stream);
    else
        e = st::launch_qkv_rope_f32((const float*)x, (const float*)w, (const float*)bias, (float*)q,
                                    (float*)k, (float*)v, table, g, (int)n, (int)C, d, stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

// ---- partial attention over a run of keys, and the merge -----------------------------------------

size_t st_attn3d_partial_workspace_bytes(int T, int H, int W, int n_text, int heads, int d,
                                         const int rope_split[3], st_dtype dtype, int kv_count) {
    if (!dtype_known(dtype)) return 0;
    long long n = 0;
    if (!rope_split || !grid_ok(T, H, W, n_text, &n) || heads < 1 || heads > 65535) return 0;
    if (check_split(rope_split, d) != ST_OK) return 0;
    if (kv_count < 1 || kv_count > n) return 0;
    if (dtype == ST_F32) return d <= 128 ? table_bytes_for(T, H, W, rope_split) : 0;
    if (dtype != ST_BF16 || d != 128) return 0;
    // Table and key tiles, then the block flags of the fast launch for any query run (at most all
    // n rows; the launch never splits its keys, whose buffers would grow with the query run).
    return stage_layout(T, H, W, heads, kv_count, 1, rope_split, false).total +
           align_up(st::attn_flag_bytes_unsplit(heads, (int)n, 1), kWsAlign);
}

st_status st_attn3d_partial_fwd(const void* q, const void* k, const void* v, int T, int H, int W,
                                int n_text, int heads, int d, const int rope_split[3], float theta,
                                st_dtype dtype, int q_begin, int q_count, int kv_begin,
                                int kv_count, void* workspace, size_t ws_bytes, void* out,
                                float* lse, hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    if (!q || !k || !v || !out || !lse || !workspace || !rope_split) return ST_ERR_NULL;
    long long n = 0;
    if (!grid_ok(T, H, W, n_text, &n)) return ST_ERR_SHAPE;
    if (heads < 1 || heads > 65535 || d < 2 || (d & 1)) return ST_ERR_SHAPE;
    if (q_begin < 0 || q_count < 1 || (long long)q_begin + q_count > n) return ST_ERR_SHAPE;
    if (kv_begin < 0 || kv_count < 1 || (long long)kv_begin + kv_count > n) return ST_ERR_SHAPE;
    st_status s = check_split(rope_split, d);
    if (s != ST_OK) return s;
    if (dtype == ST_BF16) {
        if (d != 128) return ST_ERR_UNSUPPORTED;
    } else if (dtype == ST_F32) {
        if (d > 128) return ST_ERR_UNSUPPORTED;
    } else {
        return ST_ERR_UNSUPPORTED;
    }
    if (!theta_ok(theta)) return ST_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
        return ST_ERR_ALIGN;
    if (!aligned(workspace, kWsAlign)) return ST_ERR_ALIGN;
    const size_t qb = (size_t)q_count * heads * d * elem_size(dtype);
    const size_t kb = (size_t)kv_count * heads * d * elem_size(dtype);
    const size_t lb = (size_t)q_count * heads * sizeof(float);
    const void* ins[3] = {q, k, v};
    const size_t insz[3] = {qb, kb, kb};
    for (int i = 0; i < 3; ++i)
        if (overlaps(out, qb, ins[i], insz[i]) || overlaps(lse, lb, ins[i], insz[i]) ||
            overlaps(workspace, ws_bytes, ins[i], insz[i]))
            return ST_ERR_ALIAS;
    if (overlaps(out, qb, lse, lb) || overlaps(workspace, ws_bytes, out, qb) ||
        overlaps(workspace, ws_bytes, lse, lb))
        return ST_ERR_ALIAS;
    if (ws_bytes < st_attn3d_partial_workspace_bytes(T, H, W, n_text, heads, d, rope_split, dtype,
                                                     kv_count))
        return ST_ERR_WORKSPACE;
    st::RopeGeom g = st::make_geom(T, H, W, rope_split);
    char* ws = (char*)workspace;
    float2* table = (float2*)ws;
    hipError_t e = st::launch_rope_table(g, (double)theta, table, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (dtype == ST_BF16) {
        st::SeqLayout L;
        L.n_segs = 1;
        L.q_len = q_count;
        L.kv_len = kv_count;
        L.q_pos_base = q_begin;
        L.kv_pos_base = kv_begin;
        uint16_t* kt = (uint16_t*)(ws + table_bytes_for(T, H, W, rope_split));
        e = st::launch_k_prep((const uint16_t*)k, kt, table, g, heads, L, stream);
        if (e != hipSuccess) return hip_fail(e);
        uint8_t* flags = (uint8_t*)(ws + stage_layout(T, H, W, heads, kv_count, 1, rope_split, false).total);
        e = st::launch_attn_bf16_staged((const uint16_t*)q, kt, (const uint16_t*)v, (uint16_t*)out, lse,
                                        table, g, heads, L, flags, stream, /*allow_split=*/false);
    } else {
        e = st::launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, lse,
                                table, g, heads, d,
                                f32_layout(1, q_count, 0, 1, kv_count, 0, 1, q_begin, kv_begin), stream);
    }
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

st_status st_attn_merge(int n_parts, const void* const* o_parts, const float* const* lse_parts,
                        int n_rows, int heads, int d, st_dtype dtype, void* out, float* lse_out,
                        hipStream_t stream) {
    if (!dtype_known(dtype)) return ST_ERR_UNSUPPORTED;
    if (!o_parts || !lse_parts || !out) return ST_ERR_NULL;
    if (n_parts < 1 || n_parts > st::kMaxMergeParts) return ST_ERR_SHAPE;
    if (n_rows < 1 || n_rows >= kMaxRows || heads < 1 || heads > 65535) return ST_ERR_SHAPE;
    if ((long long)n_rows * heads >= (1LL << 31)) return ST_ERR_SHAPE;   // launch grid limit
    if (dtype == ST_BF16) {
        if (d < 8 || d % 8 || d > 512) return ST_ERR_UNSUPPORTED;
    } else if (dtype == ST_F32) {
        if (d < 4 || d % 4 || d > 256) return ST_ERR_UNSUPPORTED;
    } else {
        return ST_ERR_UNSUPPORTED;
    }
    if (!aligned(out, 16) || (lse_out && !aligned(lse_out, 4))) return ST_ERR_ALIGN;
    const size_t ob = (size_t)n_rows * heads * d * elem_size(dtype);
    const size_t lb = (size_t)n_rows * heads * sizeof(float);
    for (int i = 0; i < n_parts; ++i) {
        if (!o_parts[i] || !lse_parts[i]) return ST_ERR_NULL;
        if (!aligned(o_parts[i], 16) || !aligned(lse_parts[i], 4)) return ST_ERR_ALIGN;
        // Exact aliasing (in-place merge) is allowed; partial overlap is not.
        if (out != o_parts[i] && overlaps(out, ob, o_parts[i], ob)) return ST_ERR_ALIAS;
        if (lse_out && lse_out != lse_parts[i] && overlaps(lse_out, lb, lse_parts[i], lb))
            return ST_ERR_ALIAS;
        if (overlaps(out, ob, lse_parts[i], lb)) return ST_ERR_ALIAS;
        if (lse_out && overlaps(lse_out, lb, o_parts[i], ob)) return ST_ERR_ALIAS;
    }
    if (lse_out && overlaps(out, ob, lse_out, lb)) return ST_ERR_ALIAS;
    hipError_t e;
    if (dtype == ST_BF16)
        e = st::launch_merge_bf16(n_parts, (const uint16_t* const*)o_parts, lse_parts,
                                  (long long)n_rows * heads, d, (uint16_t*)out, lse_out, stream);
    else
        e = st::launch_merge_f32(n_parts, (const float* const*)o_parts, lse_parts,
                                 (long long)n_rows * heads, d, (float*)out, lse_out, stream);
    return e == hipSuccess ? ST_OK : hip_fail(e);
}

const char* st_status_str(st_status s) {
    // A C caller may pass any int; in C++ loading an st_status outside the enumerators' range is
    // undefined, so the code is read through its bytes.
    int code;
    memcpy(&code, &s, sizeof code);
    switch (code) {
        case ST_OK: return "ok";
        case ST_ERR_NULL: return "null pointer";
        case ST_ERR_SHAPE: return "shape out of range";
        case ST_ERR_SPLIT: return "invalid rope_split";
        case ST_ERR_UNSUPPORTED: return "unsupported argument combination";
        case ST_ERR_WORKSPACE: return "workspace too small";
        case ST_ERR_HIP: return "HIP launch failed";
        case ST_ERR_ALIAS: return "output overlaps an input";
        case ST_ERR_ALIGN: return "pointer misaligned";
    }
    return "unknown status";
}

int st_last_hip_error(void) { return g_last_hip_error; }

// The version names the sources the library was built from (a hash the build passes in) and
// whether it is the LDS-poison debug build, so that two builds can be matched.
#ifndef ST_SOURCE_HASH
#define ST_SOURCE_HASH "unknown"
#endif
#ifdef ST_LDS_POISON
#define ST_BUILD_TAG "+ldspoison"
#else
#define ST_BUILD_TAG ""
#endif
const char* st_version(void) { return "0.1.0+" ST_SOURCE_HASH ST_BUILD_TAG; }

}  // extern "C"
