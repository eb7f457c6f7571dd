// float32 attention kernels (fp32 storage and arithmetic, VALU FMA).
//
// Same algorithm as the bf16 path: the tiled online-softmax forward of page 1
// ("05_flash_attention.py", section 2) and its recomputation backward
// (section 3), with the derivative rules of page 3 ("Flash Attention"),
// section 1.5. A group of G adjacent lanes owns one query row (forward, dQ)
// or one key row (dK, dV), each lane holding C = D / G of its columns in
// registers (at most 32: d = 128 is four lanes of 32), and the row's dot
// products are summed over the group with quad permutes; key/query tiles of
// 32 rows are copied global -> LDS without registers into two buffers (the
// next tile lands while the current one is used) and read as broadcasts.
// The backward's dQ comes from its own pass
// over the key tiles, so no atomics are needed and results are deterministic.
// The causal diagonal is a runtime offset coff (key j visible to query i iff
// j <= i + coff); a row that sees no key gets O = 0, L = -inf and zero dQ,
// and adds nothing to dK, dV.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kRows = 64;   // rows per workgroup
constexpr int kTile = 32;   // rows per staged tile

// A row's d values are spread over G adjacent lanes of C columns each
// (lanes 4i .. 4i + 3 hold one, two or four whole rows, so the quad permutes
// below stay inside a row): d = 16 one lane; 32 two lanes of 16; 64, 96,
// 128 four lanes of 16, 24, 32. A thread keeps at most 32 columns of each
// of its row vectors in registers, and a 64-row workgroup has 2-4 waves.
template <int D>
struct Split {
    static constexpr int G = D <= 16 ? 1 : (D == 32 ? 2 : 4);
    static constexpr int C = D / G;
    static constexpr int kThreads = kRows * G;
};

// Sum over the G lanes of a row (DPP quad permutes: lane ^ 1, lane ^ 2).
template <int G>
__device__ __forceinline__ float row_sum(float x) {
    if (G >= 2)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    if (G >= 4)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

// Tile of kTile rows from row r0 of a row-major [n, D] fp32 head (one
// contiguous block) straight into LDS at dst, without registers: the
// workgroup's waves issue its 1 KB pieces, `wave` taking every NW-th. Rows
// past n read as zeros through the buffer resource's bound. Byte offsets
// are unsigned: (n rounded up to the tile) * D * 4 < 2^32.
template <int D>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t rs, float* dst, int r0, int wave, int lane) {
    constexpr int NW = Split<D>::kThreads / 64;   // waves
    constexpr int NCH = kTile * D * 4 / 1024;      // 1 KB pieces per tile
    static_assert(NCH % NW == 0, "whole pieces per wave");
#pragma unroll
    for (int i = 0; i < NCH / NW; ++i) {
        const int b = NW * i + wave;
        load_lds16(rs, ((unsigned)r0 * D + 256u * (unsigned)b + 4u * (unsigned)lane) * 4u, dst + 256 * b);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(Split<D>::kThreads) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ Lse, int n_q, int n_k, int coff, int n_qtiles,
    float scale2) {
    constexpr int G = Split<D>::G, C = Split<D>::C;
    // Two buffers per tensor, one LDS object each: tile t + 1 is copied
    // while tile t is used.
    __shared__ __attribute__((aligned(16))) float Ks0[kTile * D];
    __shared__ __attribute__((aligned(16))) float Ks1[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs0[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs1[kTile * D];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col0 = (tid % G) * C;     // this lane's columns
    const int bh = blockIdx.x / n_qtiles;
    const int q0 = (blockIdx.x % n_qtiles) * kRows;
    const int row = q0 + tid / G;
    const float* Kh = K + (size_t)bh * n_k * D;
    const float* Vh = V + (size_t)bh * n_k * D;

    float q[C], o[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        q[c] = row < n_q ? Q[((size_t)bh * n_q + row) * D + col0 + c] * scale2 : 0.0f;
        o[c] = 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + kRows, n_q) + coff));
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh, n_k * D * 4);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vh, n_k * D * 4);
    auto issue = [&](float* Kd, float* Vd, int ks) __attribute__((always_inline)) {
        copy_tile<D>(krs, Kd, ks, wave, lane);
        copy_tile<D>(vrs, Vd, ks, wave, lane);
    };
    auto tile = [&](const float* Ks, const float* Vs, int ks) __attribute__((always_inline)) {
        float s[kTile];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) acc = fmaf(q[c], Ks[j * D + col0 + c], acc);
            acc = row_sum<G>(acc);
            const int key = ks + j;
            if (key >= n_k || (CAUSAL && key > row + coff)) acc = kNegInf;
            s[j] = acc;
            mx = fmaxf(mx, acc);
        }
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float corr = fast_exp2(m - m_use);
        l *= corr;
#pragma unroll
        for (int c = 0; c < C; ++c) o[c] *= corr;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float p = fast_exp2(s[j] - m_use);
            l += p;
#pragma unroll
            for (int c = 0; c < C; ++c) o[c] = fmaf(p, Vs[j * D + col0 + c], o[c]);
        }
        m = m_new;
    };
    // Tile t is in buffer t % 2; the barrier after a tile makes the next
    // one's copies visible and frees the buffer the following copy reuses.
    const int ntiles = (kend + kTile - 1) / kTile;
    if (ntiles > 0) {
        issue(Ks0, Vs0, 0);
        copies_barrier();
    }
    for (int t = 0; t < ntiles; ++t) {
        // one loop body with the buffers picked at run time: these kernels
        // wait for all copies at every barrier, so the compiler need not tell
        // the buffers apart, and a second copy of the body would only hold
        // more registers
        const bool odd = t & 1;
        if (t + 1 < ntiles) issue(odd ? Ks0 : Ks1, odd ? Vs0 : Vs1, (t + 1) * kTile);
        tile(odd ? Ks1 : Ks0, odd ? Vs1 : Vs0, t * kTile);
        copies_barrier();
    }
    if (row < n_q) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;   // no visible key: O = 0, L = -inf
#pragma unroll
        for (int c = 0; c < C; ++c) O[((size_t)bh * n_q + row) * D + col0 + c] = o[c] * inv;
        if (col0 == 0) Lse[(size_t)bh * n_q + row] = kLn2 * (m + fast_log2(l));
    }
}

// D = rowsum(dO * O), one row per thread.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(
    const float* __restrict__ O, const float* __restrict__ dO, float* __restrict__ drow, long long rows) {
    const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
        const float4 a = *(const float4*)(O + (size_t)row * D + d);
        const float4 b = *(const float4*)(dO + (size_t)row * D + d);
        acc = fmaf(a.x, b.x, acc); acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc); acc = fmaf(a.w, b.w, acc);
    }
    drow[row] = acc;
}

// dK, dV: one key row per G lanes, query tiles staged in LDS. Lanes of a
// key past n_k compute with zero K, V rows and store nothing (no branch
// around the row sums).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(Split<D>::kThreads) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    float* __restrict__ dK, float* __restrict__ dV, int n_q, int n_k, int coff, int n_ktiles,
    float scale, float scale2) {
    constexpr int G = Split<D>::G, C = Split<D>::C;
    // Two buffers per tensor (one LDS object each): query tile t + 1 is
    // copied while tile t is used, with its L2 and D values.
    __shared__ __attribute__((aligned(16))) float Qs0[kTile * D];
    __shared__ __attribute__((aligned(16))) float Qs1[kTile * D];
    __shared__ __attribute__((aligned(16))) float dOs0[kTile * D];
    __shared__ __attribute__((aligned(16))) float dOs1[kTile * D];
    __shared__ float Ls0[kTile], Ds0[kTile], Ls1[kTile], Ds1[kTile];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col0 = (tid % G) * C;
    const int bh = blockIdx.x / n_ktiles;
    const int k0 = (blockIdx.x % n_ktiles) * kRows;
    const int key = k0 + tid / G;
    const float* Qh = Q + (size_t)bh * n_q * D;
    const float* dOh = dO + (size_t)bh * n_q * D;

    float kr[C], vr[C], dk[C], dv[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        kr[c] = key < n_k ? K[((size_t)bh * n_k + key) * D + col0 + c] * scale2 : 0.0f;
        vr[c] = key < n_k ? V[((size_t)bh * n_k + key) * D + col0 + c] : 0.0f;
        dk[c] = dv[c] = 0.0f;
    }
    const int qbeg = CAUSAL ? (max(0, k0 - coff) / kTile) * kTile : 0;  // rows >= k0 - coff
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, n_q * D * 4);
    const __amdgpu_buffer_rsrc_t dors = make_rsrc(dOh, n_q * D * 4);
    auto issue = [&](float* Qd, float* dOd, int qs) __attribute__((always_inline)) {
        copy_tile<D>(qrs, Qd, qs, wave, lane);
        copy_tile<D>(dors, dOd, qs, wave, lane);
    };
    // L2 (L * log2 e; +inf for a row with no key, so its P is 0) and D of
    // query tile qs.., one per thread of the first kTile: loaded into
    // registers when the tile's copy is issued and written to LDS after the
    // current tile's work, so the loads' latency hides behind it.
    float l2_next = 0.0f, d_next = 0.0f;
    auto load_rows = [&](int qs) __attribute__((always_inline)) {
        if (tid < kTile) {
            const int q = qs + tid;
            const float lse = q < n_q ? Lse[(size_t)bh * n_q + q] : kNegInf;
            l2_next = lse > kNegInf ? lse * kLog2e : __builtin_huge_valf();
            d_next = q < n_q ? drow[(size_t)bh * n_q + q] : 0.0f;
        }
    };
    auto store_rows = [&](float* Ld, float* Dd) __attribute__((always_inline)) {
        if (tid < kTile) {
            Ld[tid] = l2_next;
            Dd[tid] = d_next;
        }
    };
    // Tile t (rows qbeg + t * kTile ..) is in buffer t % 2; the barrier after
    // a tile makes the next one visible and frees the buffer the following
    // copy reuses.
    const int ntiles = qbeg < n_q ? (n_q - qbeg + kTile - 1) / kTile : 0;
    if (ntiles > 0) {
        issue(Qs0, dOs0, qbeg);
        load_rows(qbeg);
        store_rows(Ls0, Ds0);
        copies_barrier();
    }
    for (int t = 0; t < ntiles; ++t) {
        // buffers picked at run time, as in the forward
        const bool odd = t & 1;
        const int qs = qbeg + t * kTile;
        if (t + 1 < ntiles) {
            issue(odd ? Qs0 : Qs1, odd ? dOs0 : dOs1, qs + kTile);
            load_rows(qs + kTile);
        }
        const float* Qs = odd ? Qs1 : Qs0;
        const float* dOs = odd ? dOs1 : dOs0;
        const float* Ls = odd ? Ls1 : Ls0;
        const float* Ds = odd ? Ds1 : Ds0;
#pragma unroll 4
        for (int i = 0; i < kTile; ++i) {
            const int q = qs + i;
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                s = fmaf(Qs[i * D + col0 + c], kr[c], s);
                dp = fmaf(dOs[i * D + col0 + c], vr[c], dp);
            }
            s = row_sum<G>(s);
            dp = row_sum<G>(dp);
            float p = fast_exp2(s - Ls[i]);
            if (key >= n_k || q >= n_q || (CAUSAL && key > q + coff)) p = 0.0f;
            const float ds = p * (dp - Ds[i]);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                dv[c] = fmaf(p, dOs[i * D + col0 + c], dv[c]);
                dk[c] = fmaf(ds, Qs[i * D + col0 + c], dk[c]);
            }
        }
        if (t + 1 < ntiles) store_rows(odd ? Ls0 : Ls1, odd ? Ds0 : Ds1);
        copies_barrier();
    }
    if (key < n_k) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            dK[((size_t)bh * n_k + key) * D + col0 + c] = dk[c] * scale;
            dV[((size_t)bh * n_k + key) * D + col0 + c] = dv[c];
        }
    }
}

// dQ: one query row per G lanes, key tiles staged in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(Split<D>::kThreads) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    float* __restrict__ dQ, int n_q, int n_k, int coff, int n_qtiles, float scale, float scale2) {
    constexpr int G = Split<D>::G, C = Split<D>::C;
    // Two buffers per tensor (one LDS object each): tile t + 1 is copied
    // while tile t is used.
    __shared__ __attribute__((aligned(16))) float Ks0[kTile * D];
    __shared__ __attribute__((aligned(16))) float Ks1[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs0[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs1[kTile * D];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col0 = (tid % G) * C;
    const int bh = blockIdx.x / n_qtiles;
    const int q0 = (blockIdx.x % n_qtiles) * kRows;
    const int row = q0 + tid / G;
    const float* Kh = K + (size_t)bh * n_k * D;
    const float* Vh = V + (size_t)bh * n_k * D;

    float q[C], dor[C], dq[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        q[c] = row < n_q ? Q[((size_t)bh * n_q + row) * D + col0 + c] * scale2 : 0.0f;
        dor[c] = row < n_q ? dO[((size_t)bh * n_q + row) * D + col0 + c] : 0.0f;
        dq[c] = 0.0f;
    }
    const float lse = row < n_q ? Lse[(size_t)bh * n_q + row] : kNegInf;
    const float l2 = lse > kNegInf ? lse * kLog2e : __builtin_huge_valf();   // P = 0 if no key
    const float Dr = row < n_q ? drow[(size_t)bh * n_q + row] : 0.0f;
    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + kRows, n_q) + coff));
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh, n_k * D * 4);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vh, n_k * D * 4);
    auto issue = [&](float* Kd, float* Vd, int ks) __attribute__((always_inline)) {
        copy_tile<D>(krs, Kd, ks, wave, lane);
        copy_tile<D>(vrs, Vd, ks, wave, lane);
    };
    // Tile t is in buffer t % 2, as in the forward.
    const int ntiles = (kend + kTile - 1) / kTile;
    if (ntiles > 0) {
        issue(Ks0, Vs0, 0);
        copies_barrier();
    }
    for (int t = 0; t < ntiles; ++t) {
        // one loop body with the buffers picked at run time: these kernels
        // wait for all copies at every barrier, so the compiler need not tell
        // the buffers apart, and a second copy of the body would only hold
        // more registers
        const bool odd = t & 1;
        if (t + 1 < ntiles) issue(odd ? Ks0 : Ks1, odd ? Vs0 : Vs1, (t + 1) * kTile);
        const float* Ks = odd ? Ks1 : Ks0;
        const float* Vs = odd ? Vs1 : Vs0;
        const int ks = t * kTile;
#pragma unroll 4
        for (int j = 0; j < kTile; ++j) {
            const int key = ks + j;
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                s = fmaf(q[c], Ks[j * D + col0 + c], s);
                dp = fmaf(dor[c], Vs[j * D + col0 + c], dp);
            }
            s = row_sum<G>(s);
            dp = row_sum<G>(dp);
            float p = fast_exp2(s - l2);
            if (key >= n_k || (CAUSAL && key > row + coff)) p = 0.0f;
            const float ds = p * (dp - Dr);
#pragma unroll
            for (int c = 0; c < C; ++c) dq[c] = fmaf(ds, Ks[j * D + col0 + c], dq[c]);
        }
        copies_barrier();
    }
    if (row < n_q) {
        // Ks holds K * 1 (unscaled); q was pre-scaled, so dq needs the scale.
#pragma unroll
        for (int c = 0; c < C; ++c) dQ[((size_t)bh * n_q + row) * D + col0 + c] = dq[c] * scale;
    }
}

template <int D, bool CAUSAL>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t st) {
    const int nt = (a.n_q + kRows - 1) / kRows;
    const long long nwg = (long long)a.bh * nt;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(Split<D>::kThreads), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.n_q, a.n_k, a.coff, nt, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_launch(const BwdArgs& a, hipStream_t st) {
    const long long rows = (long long)a.bh * a.n_q;
    const long long nb = (rows + 255) / 256;
    const int nqt = (a.n_q + kRows - 1) / kRows;
    const int nkt = (a.n_k + kRows - 1) / kRows;
    if (nb > 0x7fffffffLL || (long long)a.bh * nqt > 0x7fffffffLL || (long long)a.bh * nkt > 0x7fffffffLL)
        return hipErrorInvalidValue;
    hipError_t e = record_stage(a, 0, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)nb), dim3(256), 0, st,
                       (const float*)a.o, (const float*)a.d_o, a.drow, rows);
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 1, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nkt)), dim3(Split<D>::kThreads), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.d_o,
                       a.lse, a.drow, (float*)a.dk, (float*)a.dv, a.n_q, a.n_k, a.coff, nkt, a.scale,
                       a.scale * kLog2e);
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nqt)), dim3(Split<D>::kThreads), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.d_o,
                       a.lse, a.drow, (float*)a.dq, a.n_q, a.n_k, a.coff, nqt, a.scale, a.scale * kLog2e);
    e = hipGetLastError();
    return e == hipSuccess ? record_stage(a, 3, st) : e;
}

template <int D>
hipError_t fwd_d(const FwdArgs& a, hipStream_t st) {
    return a.causal ? fwd_launch<D, true>(a, st) : fwd_launch<D, false>(a, st);
}
template <int D>
hipError_t bwd_d(const BwdArgs& a, hipStream_t st) {
    return a.causal ? bwd_launch<D, true>(a, st) : bwd_launch<D, false>(a, st);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 16: return fwd_d<16>(a, st);
        case 32: return fwd_d<32>(a, st);
        case 64: return fwd_d<64>(a, st);
        case 96: return fwd_d<96>(a, st);
        case 128: return fwd_d<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 16: return bwd_d<16>(a, st);
        case 32: return bwd_d<32>(a, st);
        case 64: return bwd_d<64>(a, st);
        case 96: return bwd_d<96>(a, st);
        case 128: return bwd_d<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
