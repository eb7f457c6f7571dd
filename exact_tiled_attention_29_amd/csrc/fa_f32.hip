// float32 attention kernels (fp32 storage and arithmetic, VALU FMA).
//
// Same algorithm as the bf16 path: the tiled online-softmax forward of page 1
// ("05_flash_attention.py", section 2) and its recomputation backward
// (section 3), with the derivative rules of page 3 ("Flash Attention"),
// section 1.5. Each thread owns one query row (forward, dQ) or one key row
// (dK, dV) and keeps it in registers; key/query tiles of 32 rows are staged
// in LDS and read as broadcasts. The backward's dQ comes from its own pass
// over the key tiles, so no atomics are needed and results are deterministic.
// The causal diagonal is a runtime offset coff (key j visible to query i iff
// j <= i + coff); a row that sees no key gets O = 0, L = -inf and zero dQ,
// and adds nothing to dK, dV.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kRows = 64;   // rows (threads) per workgroup
constexpr int kTile = 32;   // rows per staged tile

template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int row0, int n, int tid) {
    // kTile x D floats, rows past n are zero.
    for (int i = tid; i < kTile * D / 4; i += kRows) {
        const int row = i / (D / 4), c = i % (D / 4);
        const int gr = row0 + row;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr < n) x = *(const float4*)(src + (size_t)gr * D + 4 * c);
        *(float4*)(dst + row * D + 4 * c) = x;
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ Lse, int n_q, int n_k, int coff, int n_qtiles,
    float scale2) {
    __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs[kTile * D];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / n_qtiles;
    const int q0 = (blockIdx.x % n_qtiles) * kRows;
    const int row = q0 + tid;
    const float* Kh = K + (size_t)bh * n_k * D;
    const float* Vh = V + (size_t)bh * n_k * D;

    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = row < n_q ? Q[((size_t)bh * n_q + row) * D + d] * scale2 : 0.0f;
        o[d] = 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + kRows, n_q) + coff));
    for (int ks = 0; ks < kend; ks += kTile) {
        __syncthreads();
        stage_rows<D>(Ks, Kh, ks, n_k, tid);
        stage_rows<D>(Vs, Vh, ks, n_k, tid);
        __syncthreads();
        float s[kTile];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j * D + d], acc);
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
        for (int d = 0; d < D; ++d) o[d] *= corr;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float p = fast_exp2(s[j] - m_use);
            l += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j * D + d], o[d]);
        }
        m = m_new;
    }
    if (row < n_q) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;   // no visible key: O = 0, L = -inf
#pragma unroll
        for (int d = 0; d < D; ++d) O[((size_t)bh * n_q + row) * D + d] = o[d] * inv;
        Lse[(size_t)bh * n_q + row] = kLn2 * (m + fast_log2(l));
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

// dK, dV: one key row per thread, query tiles staged in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    float* __restrict__ dK, float* __restrict__ dV, int n_q, int n_k, int coff, int n_ktiles,
    float scale, float scale2) {
    __shared__ __attribute__((aligned(16))) float Qs[kTile * D];
    __shared__ __attribute__((aligned(16))) float dOs[kTile * D];
    __shared__ float Ls[kTile], Ds[kTile];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / n_ktiles;
    const int k0 = (blockIdx.x % n_ktiles) * kRows;
    const int key = k0 + tid;
    const float* Qh = Q + (size_t)bh * n_q * D;
    const float* dOh = dO + (size_t)bh * n_q * D;

    float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        kr[d] = key < n_k ? K[((size_t)bh * n_k + key) * D + d] * scale2 : 0.0f;
        vr[d] = key < n_k ? V[((size_t)bh * n_k + key) * D + d] : 0.0f;
        dk[d] = dv[d] = 0.0f;
    }
    const int qbeg = CAUSAL ? (max(0, k0 - coff) / kTile) * kTile : 0;  // rows >= k0 - coff
    for (int qs = qbeg; qs < n_q; qs += kTile) {
        __syncthreads();
        stage_rows<D>(Qs, Qh, qs, n_q, tid);
        stage_rows<D>(dOs, dOh, qs, n_q, tid);
        if (tid < kTile) {
            const int q = qs + tid;
            const float lse = q < n_q ? Lse[(size_t)bh * n_q + q] : kNegInf;
            Ls[tid] = lse > kNegInf ? lse * kLog2e : __builtin_huge_valf();   // P = 0 if no key
            Ds[tid] = q < n_q ? drow[(size_t)bh * n_q + q] : 0.0f;
        }
        __syncthreads();
        if (key >= n_k) continue;
#pragma unroll 4
        for (int i = 0; i < kTile; ++i) {
            const int q = qs + i;
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                s = fmaf(Qs[i * D + d], kr[d], s);
                dp = fmaf(dOs[i * D + d], vr[d], dp);
            }
            float p = fast_exp2(s - Ls[i]);
            if (q >= n_q || (CAUSAL && key > q + coff)) p = 0.0f;
            const float ds = p * (dp - Ds[i]);
#pragma unroll
            for (int d = 0; d < D; ++d) {
                dv[d] = fmaf(p, dOs[i * D + d], dv[d]);
                dk[d] = fmaf(ds, Qs[i * D + d], dk[d]);
            }
        }
    }
    if (key < n_k) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            dK[((size_t)bh * n_k + key) * D + d] = dk[d] * scale;
            dV[((size_t)bh * n_k + key) * D + d] = dv[d];
        }
    }
}

// dQ: one query row per thread, key tiles staged in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    float* __restrict__ dQ, int n_q, int n_k, int coff, int n_qtiles, float scale, float scale2) {
    __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
    __shared__ __attribute__((aligned(16))) float Vs[kTile * D];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / n_qtiles;
    const int q0 = (blockIdx.x % n_qtiles) * kRows;
    const int row = q0 + tid;
    const float* Kh = K + (size_t)bh * n_k * D;
    const float* Vh = V + (size_t)bh * n_k * D;

    float q[D], dor[D], dq[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = row < n_q ? Q[((size_t)bh * n_q + row) * D + d] * scale2 : 0.0f;
        dor[d] = row < n_q ? dO[((size_t)bh * n_q + row) * D + d] : 0.0f;
        dq[d] = 0.0f;
    }
    const float lse = row < n_q ? Lse[(size_t)bh * n_q + row] : kNegInf;
    const float l2 = lse > kNegInf ? lse * kLog2e : __builtin_huge_valf();   // P = 0 if no key
    const float Dr = row < n_q ? drow[(size_t)bh * n_q + row] : 0.0f;
    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + kRows, n_q) + coff));
    for (int ks = 0; ks < kend; ks += kTile) {
        __syncthreads();
        stage_rows<D>(Ks, Kh, ks, n_k, tid);
        stage_rows<D>(Vs, Vh, ks, n_k, tid);
        __syncthreads();
        if (row >= n_q) continue;
#pragma unroll 4
        for (int j = 0; j < kTile; ++j) {
            const int key = ks + j;
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                s = fmaf(q[d], Ks[j * D + d], s);
                dp = fmaf(dor[d], Vs[j * D + d], dp);
            }
            float p = fast_exp2(s - l2);
            if (key >= n_k || (CAUSAL && key > row + coff)) p = 0.0f;
            const float ds = p * (dp - Dr);
#pragma unroll
            for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, Ks[j * D + d], dq[d]);
        }
    }
    if (row < n_q) {
        // Ks holds K * 1 (unscaled); q was pre-scaled, so dq needs the scale.
#pragma unroll
        for (int d = 0; d < D; ++d) dQ[((size_t)bh * n_q + row) * D + d] = dq[d] * scale;
    }
}

template <int D, bool CAUSAL>
hipError_t fwd_launch(const FwdArgs& a, hipStream_t st) {
    const int nt = (a.n_q + kRows - 1) / kRows;
    const long long nwg = (long long)a.bh * nt;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kRows), 0, st,
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
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nkt)), dim3(kRows), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.d_o,
                       a.lse, a.drow, (float*)a.dk, (float*)a.dv, a.n_q, a.n_k, a.coff, nkt, a.scale,
                       a.scale * kLog2e);
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nqt)), dim3(kRows), 0, st,
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
