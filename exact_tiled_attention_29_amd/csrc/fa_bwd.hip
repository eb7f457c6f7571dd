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
    float* __restrict__ dq_acc, long long rows, int n_q, int n_q_pad) {
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
        // accumulator rows are padded per head to n_q_pad
        const long long arow = (row / n_q) * n_q_pad + row % n_q;
        float* a = dq_acc + (size_t)arow * D + 8 * sub;
        *(float4*)(a) = make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(a + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && sub == 0) drow[row] = acc;
}

// --------------------------------------------------------------------------
// 2. dK, dV (and dQ partial sums) per key tile.
// --------------------------------------------------------------------------
// Layout per workgroup (4 waves, 128 keys; wave w owns keys k0 + 32w ..):
//  * K and V rows of the wave's keys live in registers as MFMA B operands of
//    S = Q K^T and dP = dO V^T; dK and dV accumulate in fp32 registers.
//  * Query tiles of 32 rows (Q, dO row-major with swizzled 16-byte chunks,
//    L in the exp2 domain, D) are double-buffered in LDS. The next tile is
//    loaded into registers at the top of an iteration and written to the
//    other buffer at its end, so the global latency overlaps the MFMAs.
//  * dV += P^T dO and dK += dS^T Q take the transposed dO / Q operands with
//    ds_read_b64_tr_b16 straight from the row-major tiles.
//  * dS^T (keys x queries) goes to a double-buffered LDS tile with 8-byte
//    writes; dQ = dS K for a tile is formed one iteration later (reading it
//    with transpose reads) and added to the fp32 accumulator with float
//    atomics, so the atomics overlap the next tile's work.
//  * One barrier per iteration, waiting on LDS traffic only.
// dS^T tile rows (one per key) hold 32 queries as 8 slots of 4; slot s of
// row key sits at s ^ ((key >> 2) & 7), spreading both the accumulator-order
// writes and the transpose reads over all banks.
__device__ __forceinline__ int dst_off(int key, int q) {
    return key * 32 + 4 * ((q >> 2) ^ ((key >> 2) & 7)) + (q & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ Lse, const float* __restrict__ drow,
    bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dq_acc,
    int n_q, int n_k, int n_q_pad, int n_ktiles, float scale, float scale2) {
    constexpr int BKV = 128;           // keys per workgroup (32 per wave)
    constexpr int BQ = 32;             // query rows per step (n_q_pad is a multiple)
    constexpr int KK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int KSPLIT = 4 / NDB;    // waves sharing one d block of dQ
    constexpr int CPW = (BKV / 16) / KSPLIT;  // 16-key chunks of dQ per wave
    constexpr int CQ = BQ * D / 8 / kThreads; // 16-byte chunks per thread per tile
    static_assert(CQ >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) bf16 Qs[2][BQ * D];
    __shared__ __attribute__((aligned(16))) bf16 dOs[2][BQ * D];
    __shared__ __attribute__((aligned(16))) bf16 dSt[2][BKV * BQ];
    __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
    __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;   // transpose-read lane roles

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
    float* dQh = dq_acc + (size_t)bh * n_q_pad * D;
    // Offsets inside one head fit in 32 bits (n * d < 2^31 is checked on the host).

    // K, V rows of this wave's keys as B operands (column = key, k = d).
    bf16x8 kreg[KK], vreg[KK];
    {
        const int key = kw0 + r;
        const int kc = min(key, n_k - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 kx = *(const bf16x8*)(Kh + kc * D + 16 * kk + 8 * g);
            const bf16x8 vx = *(const bf16x8*)(Vh + kc * D + 16 * kk + 8 * g);
            kreg[kk] = key < n_k ? kx : zero_bf16x8();
            vreg[kk] = key < n_k ? vx : zero_bf16x8();
        }
    }
    // K as the B operand of dQ = dS K (column = d, k-slot (g, e) = key
    // 16c + 8g + e), for d block dq_db and this wave's chunks.
    const int dq_db = wave % NDB;
    const int cbase = (wave / NDB) * CPW;
    bf16x8 kdt[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = k0 + 16 * (cbase + c) + 8 * g + e;
            const bf16 x = Kh[min(key, n_k - 1) * D + 32 * dq_db + r];
            kdt[c][e] = key < n_k ? x : (bf16)0.0f;
        }

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero_f32x16();

    const int nqt = (n_q + BQ - 1) / BQ;
    const int t_begin = CAUSAL ? k0 / BQ : 0;

    // ---- prefetch registers for one query tile ----
    // Loads are unconditional (rows clamped to n_q - 1) and the raw values are
    // kept until the stash; rows past n_q are replaced only there. With no
    // branches around them the compiler can count the memory operations in
    // flight and never has to drain the dQ atomics to wait for a tile.
    bf16x8 pq[CQ], pdo[CQ];
    float pld = 0.0f;
    auto fetch = [&](int t) {
        const int q0 = t * BQ;
#pragma unroll
        for (int i = 0; i < CQ; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), cc = c % (D / 8);
            const int off = min(q0 + row, n_q - 1) * D + 8 * cc;
            pq[i] = *(const bf16x8*)(Qh + off);
            pdo[i] = *(const bf16x8*)(dOh + off);
        }
        pld = ((tid & BQ) ? Dh : Lh)[min(q0 + (tid & (BQ - 1)), n_q - 1)];
    };
    auto stash = [&](int buf, int t) {
        const int q0 = t * BQ;
#pragma unroll
        for (int i = 0; i < CQ; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), cc = c % (D / 8);
            const bool ok = q0 + row < n_q;
            *(bf16x8*)(&Qs[buf][tile_off<D>(row, 8 * cc)]) = ok ? pq[i] : zero_bf16x8();
            *(bf16x8*)(&dOs[buf][tile_off<D>(row, 8 * cc)]) = ok ? pdo[i] : zero_bf16x8();
        }
        // Rows past n_q get L = +inf so their P is exactly 0, and D = 0.
        const bool ok = q0 + (tid & (BQ - 1)) < n_q;
        if (tid < BQ) Ls[buf][tid] = ok ? pld * kLog2e : __builtin_huge_valf();
        else if (tid < 2 * BQ) Ds[buf][tid - BQ] = ok ? pld : 0.0f;
    };

    // dQ of the tile held in dS^T buffer `buf` (query rows from q0).
    auto dq_step = [&](int buf, int q0) {
        f32x16 acc = zero_f32x16();
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int kc = 16 * (cbase + c) + 8 * g + (s16 >> 2);
            const int qc = 16 * half + 4 * (s16 & 3);
            const bf16x4 lo = lds_read_tr(&dSt[buf][dst_off(kc, qc)]);
            const bf16x4 hi = lds_read_tr(&dSt[buf][dst_off(kc + 4, qc)]);
            acc = mfma32(concat(lo, hi), kdt[c], acc);
        }
        // lane holds d column 32*dq_db + r, query rows acc_row(v, g); the
        // accumulator has n_q_pad rows, so no row guard is needed.
        float* base = dQh + (q0 + 4 * g) * D + 32 * dq_db + r;
#pragma unroll
        for (int v = 0; v < 16; ++v)
            __hip_atomic_fetch_add(base + (8 * (v >> 2) + (v & 3)) * D, acc[v], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    };

    // S, dP, P, dS, dV, dK for tile t, and dS^T to LDS buffer `buf`.
    auto tile_step = [&](int buf, int q0) {
        const bool active = kw0 < n_k && (!CAUSAL || q0 + BQ - 1 >= kw0);
        if (active) {
            // S = Q K^T and dP = dO V^T (rows = queries, columns = keys).
            f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8 aq = *(const bf16x8*)(&Qs[buf][tile_off<D>(r, 16 * kk + 8 * g)]);
                const bf16x8 ad = *(const bf16x8*)(&dOs[buf][tile_off<D>(r, 16 * kk + 8 * g)]);
                s = mfma32(aq, kreg[kk], s);
                dp = mfma32(ad, vreg[kk], dp);
            }
            // Lane holds key kw0 + r; element v is query q0 + acc_row(v, g).
            float lq[16], dq_[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 a = *(const float4*)(&Ls[buf][8 * i + 4 * g]);
                const float4 b = *(const float4*)(&Ds[buf][8 * i + 4 * g]);
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
            }
            // dS^T rows: 4 consecutive queries per 8-byte write.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x4 w4;
#pragma unroll
                for (int j = 0; j < 4; ++j) w4[j] = dsa[i >> 1][4 * (i & 1) + j];
                *(bf16x4*)(&dSt[buf][dst_off(32 * wave + r, 8 * i + 4 * g)]) = w4;
            }
            // dV += P^T dO, dK += dS^T Q (rows = keys, columns = d). The B
            // operands carry queries 16c + 8*(e/4) + 4g + e%4 in slot (g, e),
            // matching the accumulator order of P and dS.
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int col = 32 * db + 16 * half + 4 * (s16 & 3);
                    const int row0 = 16 * c + 4 * g + (s16 >> 2);
                    const bf16x8 bdo = concat(lds_read_tr(&dOs[buf][tile_off<D>(row0, col)]),
                                              lds_read_tr(&dOs[buf][tile_off<D>(row0 + 8, col)]));
                    const bf16x8 bq = concat(lds_read_tr(&Qs[buf][tile_off<D>(row0, col)]),
                                             lds_read_tr(&Qs[buf][tile_off<D>(row0 + 8, col)]));
                    dv[db] = mfma32(pa[c], bdo, dv[db]);
                    dk[db] = mfma32(dsa[c], bq, dk[db]);
                }
        } else {
            bf16x4 z;
#pragma unroll
            for (int j = 0; j < 4; ++j) z[j] = (bf16)0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) *(bf16x4*)(&dSt[buf][dst_off(32 * wave + r, 8 * i + 4 * g)]) = z;
        }
    };

    if (t_begin < nqt) {
        // First tile (peeled: no dQ of a previous tile yet).
        fetch(t_begin);
        stash(t_begin & 1, t_begin);
        lds_barrier();
        fetch(min(t_begin + 1, nqt - 1));
        tile_step(t_begin & 1, t_begin * BQ);
        if (t_begin + 1 < nqt) stash((t_begin + 1) & 1, t_begin + 1);
        // Steady state: one barrier per tile; the tile-(t+1) loads and the
        // tile-(t-1) dQ atomics are in flight while tile t is computed.
        for (int t = t_begin + 1; t < nqt; ++t) {
            const int buf = t & 1;
            lds_barrier();  // tile t staged; dS^T of tile t-1 written; tile t-1 reads done
            fetch(min(t + 1, nqt - 1));
            dq_step(buf ^ 1, (t - 1) * BQ);
            tile_step(buf, t * BQ);
            if (t + 1 < nqt) stash(buf ^ 1, t + 1);
        }
        lds_barrier();
        dq_step((nqt - 1) & 1, (nqt - 1) * BQ);
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
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_convert_kernel(
    const float* __restrict__ acc, bf16* __restrict__ dq, long long n8, int n_q, int n_q_pad,
    float scale) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n8) return;
    constexpr int CPR = D / 8;  // 8-element chunks per row
    const long long row = i / CPR;
    const long long arow = (row / n_q) * n_q_pad + row % n_q;
    const float* a_ = acc + (size_t)arow * D + 8 * (i % CPR);
    const float4 a = *(const float4*)(a_), b = *(const float4*)(a_ + 4);
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
                       a.n_q, a.n_k, dq_rows_padded(a.n_q), n_ktiles, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
hipError_t launch_all(const BwdArgs& a, hipStream_t st) {
    const long long rows = (long long)a.bh * a.n_q;
    constexpr int RPB = kThreads / (D / 8);
    const long long nb = (rows + RPB - 1) / RPB;
    if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e = record_stage(a, 0, st);
    if (e != hipSuccess) return e;
    if (a.o_f32)
        hipLaunchKernelGGL((bwd_pre_kernel<D, float>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const float*)a.o, (const bf16*)a.d_o, a.drow, a.dq_acc, rows, a.n_q,
                           dq_rows_padded(a.n_q));
    else
        hipLaunchKernelGGL((bwd_pre_kernel<D, bf16>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const bf16*)a.o, (const bf16*)a.d_o, a.drow, a.dq_acc, rows, a.n_q,
                           dq_rows_padded(a.n_q));
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 1, st);
    if (e != hipSuccess) return e;
    e = a.causal ? launch_dkdv<D, true>(a, st) : launch_dkdv<D, false>(a, st);
    if (e == hipSuccess) e = record_stage(a, 2, st);
    if (e != hipSuccess) return e;
    const long long n8 = rows * D / 8;
    const long long nc = (n8 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((bwd_dq_convert_kernel<D>), dim3((unsigned)nc), dim3(kThreads), 0, st,
                       (const float*)a.dq_acc, (bf16*)a.dq, n8, a.n_q, dq_rows_padded(a.n_q), a.scale);
    e = hipGetLastError();
    return e == hipSuccess ? record_stage(a, 3, st) : e;
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
