// C-ABI entry points of libfa.so: argument checks on the host (before any
// HIP call), workspace sizing and dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

// Backward scratch of fa_bwd_noalloc: one array per GPU, set up by the HIP
// runtime when the library's code object is loaded on that GPU and held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not the device array: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[FA_BWD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The attention kernels move every tensor in 16-byte pieces (direct
// global -> LDS copies, vector loads and stores).
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool dim_ok(int d, int dtype) {
    if (dtype == FA_BF16) return d == 32 || d == 64 || d == 96 || d == 128 || d == 256;
    if (dtype == FA_F32) return d == 16 || d == 32 || d == 64 || d == 96 || d == 128;
    return false;
}

// Shared checks of the forward and backward calls. Sets *empty when there
// is nothing to compute for the query side (batch, heads or n_q is zero).
int check_common(int batch, int heads, int n_q, int n_k, int d, int dtype, int o_dtype,
                 int causal, float scale, bool* empty) {
    if (causal != FA_NO_MASK && causal != FA_CAUSAL_TOP_LEFT && causal != FA_CAUSAL_BOTTOM_RIGHT)
        return FA_E_CAUSAL;
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_E_DTYPE;
    if (o_dtype != FA_BF16 && o_dtype != FA_F32) return FA_E_DTYPE;
    if (dtype == FA_F32 && o_dtype != FA_F32) return FA_E_DTYPE;
    if (batch < 0 || heads < 0 || n_q < 0 || n_k < 0) return FA_E_SHAPE;
    if (!dim_ok(d, dtype)) return FA_E_HEADDIM;
    if (!(isfinite(scale) && scale > 0.0f)) return FA_E_SCALE;
    const long long bh = (long long)batch * heads;
    if (bh > 0x7fffffffLL) return FA_E_SHAPE;
    // Every element offset must fit in 63 bits and the per-row grids in 31.
    const long long n_max = n_q > n_k ? n_q : n_k;
    const long long rows = bh * n_max;
    if (rows > (1LL << 40)) return FA_E_SHAPE;
    // One head's Q, K or V is addressed with 32-bit byte offsets.
    if (n_max * d * (dtype == FA_BF16 ? 2 : 4) > 0x7fffffffLL) return FA_E_SHAPE;
    *empty = bh == 0 || n_q == 0;
    if (!(*empty) && n_k == 0) return FA_E_SHAPE;
    return FA_OK;
}

size_t workspace_bytes(long long bh, int n_q, int d, int dtype) {
    (void)d;
    if (dtype == FA_F32) return align_up((size_t)bh * (size_t)n_q * sizeof(float));  // D
    // bf16: D and L * log2(e), rows padded per head to a multiple of 32
    return 2 * align_up((size_t)bh * (size_t)fa::dq_rows_padded(n_q) * sizeof(float));
}

// Splits of the bf16 backward for these sizes (none for float32): keys of
// the dQ kernel, queries of the dK/dV kernel.
struct BwdPlan {
    fa::Split dq, kv;
};
BwdPlan bwd_plan(long long bh, int n_q, int n_k, int d, int dtype) {
    if (dtype != FA_BF16) return {{1, n_k}, {1, n_q}};
    return {fa::dq_split_plan(bh, n_q, n_k, d), fa::kv_split_plan(bh, n_q, n_k, d)};
}

// The backward's workspace: the row arrays, then the dQ partials, then the
// dK and dV partials (each 256-byte aligned).
size_t dq_part_offset(long long bh, int n_q, int d, int dtype) { return workspace_bytes(bh, n_q, d, dtype); }
size_t kv_part_offset(long long bh, int n_q, int d, int dtype, const BwdPlan& p) {
    return dq_part_offset(bh, n_q, d, dtype) + align_up(fa::dq_part_bytes(p.dq, bh, n_q, d));
}
size_t workspace_bytes_split(long long bh, int n_q, int n_k, int d, int dtype, const BwdPlan& p) {
    return kv_part_offset(bh, n_q, d, dtype, p) + align_up(fa::kv_part_bytes(p.kv, bh, n_k, d));
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_E_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL if the lookup fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Diagonal of the causal mask: key j is visible to query i iff j <= i + offset.
int causal_offset(int causal, int n_q, int n_k) {
    return causal == FA_CAUSAL_BOTTOM_RIGHT ? n_k - n_q : 0;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 5; }

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_E_NULLPTR: return "null pointer argument";
        case FA_E_SHAPE: return "invalid shape";
        case FA_E_DTYPE: return "unsupported dtype";
        case FA_E_HEADDIM: return "unsupported head dimension";
        case FA_E_SCALE: return "scale must be finite and > 0";
        case FA_E_WORKSPACE: return "workspace missing or too small";
        case FA_E_HIP: return "HIP runtime error";
        case FA_E_CAUSAL: return "causal must be 0, 1 or 2";
        case FA_E_SCRATCH: return "problem needs more than the library's static backward scratch";
        case FA_E_ALIGN: return "tensor pointer not 16-byte aligned";
        default: return "unknown status";
    }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
           int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
           void* stream) {
    bool empty = false;
    int st = check_common(batch, heads, n_q, n_k, d, dtype, o_dtype, causal, scale, &empty);
    if (st != FA_OK) return st;
    if (empty) return FA_OK;
    if (!q || !k || !v || !o || !lse) return FA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_E_ALIGN;
    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.bh = batch * heads; a.n_q = n_q; a.n_k = n_k; a.d = d;
    a.causal = causal != FA_NO_MASK; a.coff = causal_offset(causal, n_q, n_k);
    a.o_f32 = o_dtype == FA_F32; a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    return hip_status(dtype == FA_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s));
}

size_t fa_fwd_workspace_bytes(int batch, int heads, int n_q, int n_k, int d, int dtype, int causal) {
    bool empty = false;
    const int o_dtype = dtype == FA_F32 ? FA_F32 : FA_BF16;
    if (check_common(batch, heads, n_q, n_k, d, dtype, o_dtype, causal, 1.0f, &empty) != FA_OK)
        return SIZE_MAX;
    if (empty || dtype != FA_BF16) return 0;
    fa::FwdArgs a{};
    a.bh = batch * heads; a.n_q = n_q; a.n_k = n_k; a.d = d;
    return align_up(fa::fwd_split_workspace_bytes(a, fa::fwd_split_plan(a)));
}

int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
              int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
              void* workspace, size_t workspace_bytes, void* stream) {
    bool empty = false;
    int st = check_common(batch, heads, n_q, n_k, d, dtype, o_dtype, causal, scale, &empty);
    if (st != FA_OK) return st;
    if (empty) return FA_OK;
    if (!q || !k || !v || !o || !lse) return FA_E_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_E_ALIGN;
    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.bh = batch * heads; a.n_q = n_q; a.n_k = n_k; a.d = d;
    a.causal = causal != FA_NO_MASK; a.coff = causal_offset(causal, n_q, n_k);
    a.o_f32 = o_dtype == FA_F32; a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    if (dtype != FA_BF16) return hip_status(fa::launch_fwd_f32(a, s));
    const fa::Split sp = fa::fwd_split_plan(a);
    const size_t need = fa::fwd_split_workspace_bytes(a, sp);
    if (need == 0) return hip_status(fa::launch_fwd_bf16(a, s));
    if (!workspace || workspace_bytes < need) return FA_E_WORKSPACE;
    return hip_status(fa::launch_fwd_split(a, sp, (float*)workspace, s));
}

size_t fa_bwd_workspace_bytes(int batch, int heads, int n_q, int n_k, int d, int dtype, int causal) {
    bool empty = false;
    const int o_dtype = dtype == FA_F32 ? FA_F32 : FA_BF16;
    if (check_common(batch, heads, n_q, n_k, d, dtype, o_dtype, causal, 1.0f, &empty) != FA_OK)
        return SIZE_MAX;
    if (empty) return 0;
    const long long bh = (long long)batch * heads;
    return workspace_bytes_split(bh, n_q, n_k, d, dtype, bwd_plan(bh, n_q, n_k, d, dtype));
}

}  // extern "C"

namespace {

// The backward's host checks and launch, shared by fa_bwd_timed and
// fa_bwd_noalloc. get_ws(need, &ws) supplies the workspace once every
// argument has been checked (returns a status); it is not called for an
// empty call. fits(bytes) says whether a workspace of that size (with the
// dQ split's partials) is available; if not, dQ runs without the split.
template <typename GetWs, typename Fits>
int bwd_checked(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
                void* stream, void* const* events, GetWs&& get_ws, Fits&& fits) {
    bool empty = false;
    int st = check_common(batch, heads, n_q, n_k, d, dtype, o_dtype, causal, scale, &empty);
    if (st != FA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const long long bh = (long long)batch * heads;
    if (empty) {
        // No query rows: the gradient of K and V is zero.
        if (bh == 0 || n_k == 0) return FA_OK;
        if (!dk || !dv) return FA_E_NULLPTR;
        if (!aligned16(dk) || !aligned16(dv)) return FA_E_ALIGN;
        const size_t bytes = (size_t)bh * n_k * d * (dtype == FA_BF16 ? 2 : 4);
        hipError_t e = fa::launch_zero(dk, bytes, s);
        if (e == hipSuccess) e = fa::launch_zero(dv, bytes, s);
        return hip_status(e);
    }
    if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv) return FA_E_NULLPTR;
    for (const void* p : {q, k, v, o, d_o, (const void*)dq, (const void*)dk, (const void*)dv})
        if (!aligned16(p)) return FA_E_ALIGN;
    BwdPlan plan = bwd_plan(bh, n_q, n_k, d, dtype);
    if (!fits(workspace_bytes_split(bh, n_q, n_k, d, dtype, plan))) plan.kv = fa::Split{1, n_q};
    if (!fits(workspace_bytes_split(bh, n_q, n_k, d, dtype, plan))) plan.dq = fa::Split{1, n_k};
    void* workspace = nullptr;
    st = get_ws(workspace_bytes_split(bh, n_q, n_k, d, dtype, plan), &workspace);
    if (st != FA_OK) return st;
    fa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.d_o = d_o;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.bh = (int)bh; a.n_q = n_q; a.n_k = n_k; a.d = d;
    a.causal = causal != FA_NO_MASK; a.coff = causal_offset(causal, n_q, n_k);
    a.o_f32 = o_dtype == FA_F32; a.scale = scale;
    a.events = (hipEvent_t const*)events;
    char* w = (char*)workspace;
    a.drow = (float*)w;
    a.l2pad = dtype == FA_BF16
                  ? (float*)(w + align_up((size_t)bh * (size_t)fa::dq_rows_padded(n_q) * sizeof(float)))
                  : nullptr;
    a.dq_nsplit = plan.dq.nsplit;
    a.dq_chunk = plan.dq.chunk;
    a.dq_part = plan.dq.nsplit > 1 ? (float*)(w + dq_part_offset(bh, n_q, d, dtype)) : nullptr;
    a.kv_nsplit = plan.kv.nsplit;
    a.kv_chunk = plan.kv.chunk;
    a.kv_part = plan.kv.nsplit > 1 ? (float*)(w + kv_part_offset(bh, n_q, d, dtype, plan)) : nullptr;
    return hip_status(dtype == FA_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f32(a, s));
}

}  // namespace

extern "C" {

int fa_bwd_timed(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                 const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                 int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
                 void* workspace, size_t workspace_bytes_given, void* stream,
                 void* const* events) {
    return bwd_checked(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d, dtype,
                       causal, scale, stream, events, [&](size_t need, void** ws) {
        if (!workspace || workspace_bytes_given < need) return (int)FA_E_WORKSPACE;
        if (((uintptr_t)workspace) % kAlign != 0) return (int)FA_E_WORKSPACE;
        *ws = workspace;
        return (int)FA_OK;
    }, [](size_t) { return true; });
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype,
           const float* lse, const void* d_o, void* dq, void* dk, void* dv,
           int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
           void* workspace, size_t workspace_bytes_given, void* stream) {
    return fa_bwd_timed(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d,
                        dtype, causal, scale, workspace, workspace_bytes_given, stream, nullptr);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                   const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                   int batch, int heads, int n_q, int n_k, int d, int dtype, int causal, float scale,
                   void* stream) {
    // The row-term kernel overwrites every word of the scratch that the dK/dV
    // and dQ kernels read (padding rows included), so nothing is cleared
    // between calls.
    return bwd_checked(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d, dtype,
                       causal, scale, stream, nullptr, [](size_t need, void** ws) {
        if (need > FA_BWD_NOALLOC_SCRATCH_BYTES) return (int)FA_E_SCRATCH;
        *ws = scratch_on_current_device();
        return *ws ? (int)FA_OK : (int)FA_E_HIP;
    }, [](size_t need) { return need <= FA_BWD_NOALLOC_SCRATCH_BYTES; });
}

int fa_row_softmax(const void* x, int dtype, long long rows, int cols, float scale, float* lse,
                   void* y, int y_dtype, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_E_DTYPE;
    if (y_dtype != FA_BF16 && y_dtype != FA_F32) return FA_E_DTYPE;
    if (rows < 0 || cols < 0) return FA_E_SHAPE;
    if (!(isfinite(scale) && scale > 0.0f)) return FA_E_SCALE;
    if (rows == 0) return FA_OK;
    if (cols == 0 || rows > (1LL << 40) / cols) return FA_E_SHAPE;
    if (!x || !lse) return FA_E_NULLPTR;
    fa::RowArgs a;
    a.x = x; a.rows = rows; a.cols = cols; a.x_f32 = dtype == FA_F32; a.scale = scale;
    a.lse = lse; a.y = y; a.y_f32 = y_dtype == FA_F32;
    return hip_status(fa::launch_row_softmax(a, (hipStream_t)stream));
}

}  // extern "C"

