// Host-side launchers of the attention kernels (internal to libfa.so).
// Arguments are validated by the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int bh;  // batch * heads
    int n_q, n_k, d;
    bool causal;
    int coff;    // causal diagonal: key j visible to query i iff j <= i + coff
    bool o_f32;  // O stored as float32 (else bf16)
    float scale;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* d_o;
    void* dq;
    void* dk;
    void* dv;
    int bh;
    int n_q, n_k, d;
    bool causal;
    int coff;    // as in FwdArgs
    bool o_f32;
    float scale;
    float* drow;    // fp32 D = rowsum(dO * O): [bh, n_q] (fp32 path), or -D [bh, n_q_pad] (bf16)
    float* l2pad;   // fp32 [bh, n_q_pad] L * log2(e), +inf on padding rows (bf16 path)
    hipEvent_t const* events;  // NULL or 4 events: before D, before dK/dV, after dK/dV, end
    float* dq_part;  // NULL, or fp32 [bh * dq_nsplit, n_q, d]: key-split partials of dQ (bf16 path)
    int dq_nsplit;   // key chunks of the dQ kernel when dq_part is set
    int dq_chunk;    // keys per chunk, a multiple of 64
    float* kv_part;  // NULL, or fp32 partials of dK then dV, each [bh * kv_nsplit, n_k, d] (bf16 path)
    int kv_nsplit;   // query chunks of the dK/dV kernel when kv_part is set
    int kv_chunk;    // queries per chunk, a multiple of 256
};

// A split of one dimension (keys or queries) of a kernel's work into nsplit
// chunks of `chunk` rows each (the last one shorter); nsplit = 1: none.
struct Split {
    int nsplit;
    int chunk;
};

// The split rule shared by the forward, dQ and dK/dV kernels. A grid of nwg
// workgroups over `slots` resident workgroup slots is split only when it
// would fill at most half of them and the split dimension has n >= 2048
// rows; then into the fewest chunks (multiples of `unit` rows, at least
// 256) whose nwg * nsplit workgroups fill the slots in whole rounds or in
// four or more rounds; failing that, into as many as fill one round.
inline Split plan_split(long long nwg, long long slots, int n, int unit) {
    Split none{1, n};
    if (n < 2048 || slots <= 0 || 2 * nwg > slots) return none;
    const int s_max = n / 256;
    auto plan = [&](int s) {
        const int chunk = ((n + s - 1) / s + unit - 1) / unit * unit;
        return Split{(n + chunk - 1) / chunk, chunk};
    };
    for (int s = 2; s <= s_max && nwg * s <= 8 * slots; ++s) {
        const Split p = plan(s);
        const long long w = nwg * p.nsplit;
        if (w % slots == 0 || w >= 4 * slots) return p;
    }
    const long long s_round = (slots + nwg - 1) / nwg;
    const int s = (int)(s_round < s_max ? s_round : s_max);
    return s >= 2 ? plan(s) : none;
}

// Key split of the bf16 dQ kernel for grids with few query tiles and query
// split of the bf16 dK/dV kernel for grids with few key blocks (fa_bwd.hip),
// with the bytes of their fp32 partials.
Split dq_split_plan(long long bh, int n_q, int n_k, int d);
size_t dq_part_bytes(const Split& sp, long long bh, int n_q, int d);
Split kv_split_plan(long long bh, int n_q, int n_k, int d);
size_t kv_part_bytes(const Split& sp, long long bh, int n_k, int d);

// Record stage event i of a backward call (no-op without events).
inline hipError_t record_stage(const BwdArgs& a, int i, hipStream_t st) {
    return a.events ? hipEventRecord(a.events[i], st) : hipSuccess;
}

// Rows per head of the bf16 backward's L2 and D arrays: n_q rounded up to the
// 32-row query tile of the dK/dV kernel, so whole tiles can be copied.
inline int dq_rows_padded(int n_q) { return (n_q + 31) / 32 * 32; }

// bf16 path (MFMA).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st);
int fwd_bf16_rows_per_wg(const FwdArgs& a);
// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();
// Whether nwg workgroups of one per CU fill the CUs in whole rounds or in
// enough rounds that the last one matters little.
inline bool fills_cus(long long nwg) {
    const int cus = device_cu_count();
    return cus > 0 && (nwg % cus == 0 || nwg >= 4LL * cus);
}

// Phase-locked two-group forward (fa_fwd_pp.hip) for the head dims it serves.
bool fwd_pp_supports(const FwdArgs& a);
hipError_t launch_fwd_pp(const FwdArgs& a, hipStream_t st);

// Key-split forward (fa_fwd_pp.hip): nsplit workgroups per query tile, each
// over `chunk` keys (a multiple of 64), then a merge of their partials.
Split fwd_split_plan(const FwdArgs& a);
size_t fwd_split_workspace_bytes(const FwdArgs& a, const Split& sp);
hipError_t launch_fwd_split(const FwdArgs& a, const Split& sp, float* ws, hipStream_t st);

// float32 path (fp32 FMA).
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st);

// Row softmax / logsumexp of a [rows, cols] matrix (see fa_rows.hip).
struct RowArgs {
    const void* x;
    long long rows;
    int cols;
    bool x_f32;   // x float32 (else bf16)
    float scale;
    float* lse;   // [rows] fp32
    void* y;      // NULL or [rows, cols]
    bool y_f32;   // y float32 (else bf16)
};
hipError_t launch_row_softmax(const RowArgs& a, hipStream_t st);

// Zero `bytes` bytes (a multiple of 4) with a fill kernel; no memset node,
// so the call is safe under stream capture.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);


}  // namespace fa
