// Backward attention kernels for bf16 inputs on gfx950.
//
// Algorithm: the recomputation backward of page 1 ("05_flash_attention.py",
// section 3, flash_attention_backward): outer loop over key tiles, inner
// loop over query tiles; P is rebuilt from the saved logsumexp as
// exp(S - L); dV += P^T dO; dP = dO V^T; dS = P * (dP - D) with
// D = rowsum(dO * O); dQ += scale * dS K; dK += scale * dS^T Q. Query tiles
// wholly before the key tile are skipped under the causal mask. The
// derivative rules are those of page 3 ("Flash Attention"), section 1.5.
//
// Three kernels on one stream:
//  1. bwd_pre:  D = rowsum(dO * O) in fp32, and zero the fp32 dQ accumulator;
//  2. bwd_dkdv: one workgroup per 128 keys of one (batch, head); each of its
//     4 waves keeps 32 keys' K and V rows in registers and their dK, dV in
//     fp32 accumulators, and walks the query tiles (32 rows each) staged in
//     LDS in both row-major and transposed (query-contiguous) form. dS goes
//     through LDS once to feed the dQ product, whose fp32 partial sums are
//     added to the accumulator with hardware float atomics;
//  3. bwd_dq_convert: dQ = scale * accumulator, rounded to bf16 (RNE).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// --------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero the dQ accumulator.
// --------------------------------------------------------------------------
template <int D, typename OT>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const OT* __restrict__ O, const bf16* __restrict__ dO, float* __restrict__ drow,
    float* __restrict__ dq_acc, long long rows) {
    constexpr int LPR = D / 8;               // lanes per row, 8 elements each
    constexpr int RPB = kThreads / LPR;      // rows per block
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * RPB + tid / LPR;
    const int sub = tid % LPR;
    float acc = 0.0f;
    if (row < rows) {
        const size_t base = (size_t)row * D + 8 * sub;
        const bf16x8 dov = *(const bf16x8*)(dO + base);
        float ov[8];
        if constexpr (sizeof(OT) == 4) {
            const float4 a = *(const float4*)(O + base), b = *(const float4*)(O + base + 4);
            ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
            ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
        } else {
            const bf16x8 x = *(const bf16x8*)(O + base);
#pragma unroll
            for (int i = 0; i < 8; ++i) ov[i] = bf2f(x[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(bf2f(dov[i]), ov[i], acc);
        *(float4*)(dq_acc + base) = make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(dq_acc + base + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && sub == 0) drow[row] = acc;
}

// --------------------------------------------------------------------------
// 2. dK, dV (and dQ partial sums) per key tile.
// --------------------------------------------------------------------------
// Query-contiguous tiles store each 16-query chunk permuted: position
// 8*h + 4*i + j holds query 8*i + 4*h + j, so that lane-half g of an MFMA
// whose other operand comes from an accumulator (rows 8i + 4g + j) reads its
// 8 queries with one 16-byte LDS read at position 8g.
__device__ __forceinline__ int tpos(int w) {
    return 16 * (w >> 4) + 8 * ((w >> 2) & 1) + 4 * ((w >> 3) & 1) + (w & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dq_acc,
    int n_q, int n_k, int n_ktiles, float scale, float scale2) {
    constexpr int BKV = 128;           // keys per workgroup (32 per wave)
    constexpr int BQ = 32;             // query rows per step
    constexpr int KK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int QSTR = D + 8;        // row-major Q / dO tile stride
    constexpr int TSTR = BQ + 8;       // transposed tile stride
    constexpr int SSTR = BKV + 8;      // dS tile stride
    constexpr int KSPLIT = 4 / NDB;    // waves sharing one d block of dQ
    constexpr int CPW = (BKV / 16) / KSPLIT;  // 16-key chunks of dQ per wave
    constexpr int CQ = BQ * D / 8 / kThreads; // 16-byte chunks per thread per tile
    static_assert(CQ >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) bf16 Qs[BQ * QSTR];
    __shared__ __attribute__((aligned(16))) bf16 dOs[BQ * QSTR];
    __shared__ __attribute__((aligned(16))) bf16 Qt[D * TSTR];
    __shared__ __attribute__((aligned(16))) bf16 dOt[D * TSTR];
    __shared__ __attribute__((aligned(16))) bf16 dSs[BQ * SSTR];
    __shared__ __attribute__((aligned(16))) float Ls[BQ];
    __shared__ __attribute__((aligned(16))) float Ds[BQ];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;

    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    const int bh = logical / n_ktiles;
    const int kt = logical % n_ktiles;   // ascending: longest causal work first
    const int k0 = kt * BKV;
    const int kw0 = k0 + 32 * wave;      // this wave's first key

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* dOh = dO + (size_t)bh * n_q * D;
    const bf16* Kh = K + (size_t)bh * n_k * D;
    const bf16* Vh = V + (size_t)bh * n_k * D;
    const float* Lh = Lse + (size_t)bh * n_q;
    const float* Dh = drow + (size_t)bh * n_q;
    float* dQh = dq_acc + (size_t)bh * n_q * D;

    // K, V rows of this wave's keys as B operands (column = key, k = d).
    bf16x8 kreg[KK], vreg[KK];
    {
        const int key = kw0 + r;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            kreg[kk] = key < n_k ? *(const bf16x8*)(Kh + (size_t)key * D + 16 * kk + 8 * g) : zero_bf16x8();
            vreg[kk] = key < n_k ? *(const bf16x8*)(Vh + (size_t)key * D + 16 * kk + 8 * g) : zero_bf16x8();
        }
    }
    // K as the B operand of dQ = dS K (column = d, k = key), for d block
    // dq_db and the wave's share of the workgroup's 16-key chunks.
    const int dq_db = wave % NDB;
    const int cbase = (wave / NDB) * CPW;
    bf16x8 kdt[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = k0 + 16 * (cbase + c) + 8 * g + e;
            kdt[c][e] = key < n_k ? Kh[(size_t)key * D + 32 * dq_db + r] : (bf16)0.0f;
        }

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero_f32x16();

    const int nqt = (n_q + BQ - 1) / BQ;
    const int t_begin = CAUSAL ? k0 / BQ : 0;

    for (int t = t_begin; t < nqt; ++t) {
        const int q0 = t * BQ;
        // ---- stage Q, dO (row-major and transposed), L (log2 domain), D ----
#pragma unroll
        for (int i = 0; i < CQ; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), cc = c % (D / 8);
            const int q = q0 + row;
            bf16x8 qv = zero_bf16x8(), dv8 = zero_bf16x8();
            if (q < n_q) {
                qv = *(const bf16x8*)(Qh + (size_t)q * D + 8 * cc);
                dv8 = *(const bf16x8*)(dOh + (size_t)q * D + 8 * cc);
            }
            *(bf16x8*)(&Qs[row * QSTR + 8 * cc]) = qv;
            *(bf16x8*)(&dOs[row * QSTR + 8 * cc]) = dv8;
            const int p = tpos(row);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Qt[(8 * cc + e) * TSTR + p] = qv[e];
                dOt[(8 * cc + e) * TSTR + p] = dv8[e];
            }
        }
        if (tid < BQ) {
            const int q = q0 + tid;
            // Rows past n_q get L = +inf so their P is exactly 0.
            Ls[tid] = q < n_q ? Lh[q] * kLog2e : __builtin_huge_valf();
            Ds[tid] = q < n_q ? Dh[q] : 0.0f;
        }
        __syncthreads();

        const bool active = kw0 < n_k && (!CAUSAL || q0 + BQ - 1 >= kw0);
        if (active) {
            // S = Q K^T and dP = dO V^T (rows = queries, columns = keys).
            f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8 aq = *(const bf16x8*)(&Qs[r * QSTR + 16 * kk + 8 * g]);
                const bf16x8 ad = *(const bf16x8*)(&dOs[r * QSTR + 16 * kk + 8 * g]);
                s = mfma32(aq, kreg[kk], s);
                dp = mfma32(ad, vreg[kk], dp);
            }
            // Lane holds key kw0 + r; element v is query q0 + acc_row(v, g).
            float lq[16], dq_[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 a = *(const float4*)(&Ls[8 * i + 4 * g]);
                const float4 b = *(const float4*)(&Ds[8 * i + 4 * g]);
                lq[4 * i + 0] = a.x; lq[4 * i + 1] = a.y; lq[4 * i + 2] = a.z; lq[4 * i + 3] = a.w;
                dq_[4 * i + 0] = b.x; dq_[4 * i + 1] = b.y; dq_[4 * i + 2] = b.z; dq_[4 * i + 3] = b.w;
            }
            const int key = kw0 + r;
            const bool need_mask = (kw0 + 32 > n_k) || (CAUSAL && kw0 + 31 > q0);
            bf16x8 pa[2], dsa[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float p = fast_exp2(fmaf(s[v], scale2, -lq[v]));
                if (need_mask && (key >= n_k || (CAUSAL && key > q0 + acc_row(v, g)))) p = 0.0f;
                const float ds = p * (dp[v] - dq_[v]);
                pa[v >> 3][v & 7] = to_bf16(p);
                dsa[v >> 3][v & 7] = to_bf16(ds);
                dSs[acc_row(v, g) * SSTR + 32 * wave + r] = dsa[v >> 3][v & 7];
            }
            // dV += P^T dO, dK += dS^T Q (rows = keys, columns = d).
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 bdo = *(const bf16x8*)(&dOt[(32 * db + r) * TSTR + 16 * c + 8 * g]);
                    const bf16x8 bq = *(const bf16x8*)(&Qt[(32 * db + r) * TSTR + 16 * c + 8 * g]);
                    dv[db] = mfma32(pa[c], bdo, dv[db]);
                    dk[db] = mfma32(dsa[c], bq, dk[db]);
                }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) dSs[acc_row(v, g) * SSTR + 32 * wave + r] = (bf16)0.0f;
        }
        __syncthreads();

        // dQ partial = dS K over this wave's chunks, for d block dq_db.
        {
            f32x16 acc = zero_f32x16();
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const bf16x8 a = *(const bf16x8*)(&dSs[r * SSTR + 16 * (cbase + c) + 8 * g]);
                acc = mfma32(a, kdt[c], acc);
            }
            const bool any = !CAUSAL || q0 + BQ - 1 >= k0 + 16 * cbase;
            if (any) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int q = q0 + acc_row(v, g);
                    if (q < n_q)
                        __hip_atomic_fetch_add(dQh + (size_t)q * D + 32 * dq_db + r, acc[v],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        __syncthreads();
    }

    // Epilogue: dK = scale * acc; rows = keys kw0 + acc_row(v, g), column = d.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = kw0 + acc_row(v, g);
            if (key < n_k) {
                const size_t off = ((size_t)bh * n_k + key) * D + 32 * db + r;
                dK[off] = to_bf16(dk[db][v] * scale);
                dV[off] = to_bf16(dv[db][v]);
            }
        }
}

// --------------------------------------------------------------------------
// 3. dQ = scale * accumulator, to bf16.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void bwd_dq_convert_kernel(
    const float* __restrict__ acc, bf16* __restrict__ dq, long long n8, float scale) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n8) return;
    const float4 a = *(const float4*)(acc + 8 * i), b = *(const float4*)(acc + 8 * i + 4);
    bf16x8 o;
    o[0] = to_bf16(a.x * scale); o[1] = to_bf16(a.y * scale);
    o[2] = to_bf16(a.z * scale); o[3] = to_bf16(a.w * scale);
    o[4] = to_bf16(b.x * scale); o[5] = to_bf16(b.y * scale);
    o[6] = to_bf16(b.z * scale); o[7] = to_bf16(b.w * scale);
    *(bf16x8*)(dq + 8 * i) = o;
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t st) {
    const int n_ktiles = (a.n_k + 127) / 128;
    const long long nwg = (long long)a.bh * n_ktiles;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.d_o,
                       a.lse, a.drow, (bf16*)a.dk, (bf16*)a.dv, a.dq_acc,
                       a.n_q, a.n_k, n_ktiles, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
hipError_t launch_all(const BwdArgs& a, hipStream_t st) {
    const long long rows = (long long)a.bh * a.n_q;
    constexpr int RPB = kThreads / (D / 8);
    const long long nb = (rows + RPB - 1) / RPB;
    if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.o_f32)
        hipLaunchKernelGGL((bwd_pre_kernel<D, float>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const float*)a.o, (const bf16*)a.d_o, a.drow, a.dq_acc, rows);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<D, bf16>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const bf16*)a.o, (const bf16*)a.d_o, a.drow, a.dq_acc, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = a.causal ? launch_dkdv<D, true>(a, st) : launch_dkdv<D, false>(a, st);
    if (e != hipSuccess) return e;
    const long long n8 = rows * D / 8;
    const long long nc = (n8 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)nc), dim3(kThreads), 0, st,
                       (const float*)a.dq_acc, (bf16*)a.dq, n8, a.scale);
    return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void zero_kernel(unsigned* __restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (long long)gridDim.x * kThreads)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
    const long long n = (long long)(bytes / 4);
    if (n == 0) return hipSuccess;
    long long nb = (n + kThreads - 1) / kThreads;
    if (nb > 65536) nb = 65536;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)nb), dim3(kThreads), 0, st, (unsigned*)p, n);
    return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 64: return launch_all<64>(a, st);
        case 128: return launch_all<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
