// Forward attention kernel for bf16 inputs on gfx950 (MFMA 32x32x16 bf16).
//
// Algorithm: the tiled forward with online softmax of page 1
// ("05_flash_attention.py", section 2, flash_attention_forward): per query
// tile, walk the key tiles left to right keeping a running max m and running
// sum l per row; rescale the output accumulator by exp(m_old - m_new); finish
// with O / l and L = m + log(l). Key tiles that lie wholly in the causal
// future are skipped (same section). The running-statistics recurrence is
// the one of page 1, section 1 and page 3 ("Flash Attention"), section 1.1.
//
// MI355X mapping (not from the pages):
//  * one workgroup = 4 waves = 128*QB query rows of one (batch, head);
//    each wave owns 32*QB rows and keeps its Q rows in registers as the
//    B operand of S^T = K Q^T, so every per-row quantity (m, l, the O
//    accumulator column) lives in one lane pair (l, l^32);
//  * K tiles (64 keys, row-major) and V^T tiles (keys contiguous, permuted
//    so each MFMA A operand is one 16-byte LDS read) are double-buffered in
//    LDS; the next tile's global loads are in flight during the MFMAs;
//  * scores are kept in the exp2 domain (scale * log2 e folded in), the
//    row max needs one cross-lane step (v_permlane32_swap), l sums the fp32
//    probabilities and only the PV operand is rounded to bf16 (RNE);
//  * workgroups are renumbered so each XCD works through whole heads
//    (K/V reuse in that XCD's L2), longest causal tiles first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBC = 64;  // keys per tile

// V^T rows hold each 16-key chunk permuted: position 8*h + 4*i + j holds key
// 8*i + 4*h + j (h, i in {0,1}, j in 0..3). Lane-half g of the PV MFMA needs
// the keys its S^T accumulator rows cover, {4g..4g+3, 8+4g..8+4g+3}, and
// finds them at positions 8g..8g+7: one 16-byte LDS read.

template <int D, int QB, bool CAUSAL, bool OF32>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ Lse,
    int n_q, int n_k, int n_qtiles, float scale2) {
    constexpr int RW = 32 * QB;          // query rows per wave
    constexpr int BR = 4 * RW;           // query rows per workgroup
    constexpr int KK = D / 16;           // MFMA k-steps over d
    constexpr int NDB = D / 32;          // 32-wide d blocks of the output
    constexpr int KSTR = D + 8;          // K tile row stride (elements)
    constexpr int VSTR = kBC + 8;        // V^T tile row stride (elements)
    constexpr int CK = kBC * D / 8 / kThreads;  // 16-byte K chunks per thread
    constexpr int DPT = D / 32;          // d columns per thread in the V^T stage
    static_assert(CK >= 1 && DPT >= 2, "tile shape");

    __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBC * KSTR];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * VSTR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;

    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    const int bh = logical / n_qtiles;
    const int qt = n_qtiles - 1 - logical % n_qtiles;
    const int q0 = qt * BR;
    const int qw = q0 + wave * RW;

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* Kh = K + (size_t)bh * n_k * D;
    const bf16* Vh = V + (size_t)bh * n_k * D;

    // Q rows as MFMA B operands: lane (r, g) holds d = 16*kk + 8*g .. +7.
    bf16x8 qreg[QB][KK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw + 32 * qb + r;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[qb][kk] = row < n_q ? *(const bf16x8*)(Qh + (size_t)row * D + 16 * kk + 8 * g)
                                     : zero_bf16x8();
    }

    int kend = n_k;
    if (CAUSAL) kend = min(n_k, min(q0 + BR, n_q));  // keys <= last row of the tile
    const int ntiles = (kend + kBC - 1) / kBC;

    // ---- tile staging (registers -> LDS) ----
    uint4 kst[CK];
    typedef __attribute__((ext_vector_type(DPT / 2))) unsigned vword_t;
    vword_t vst[8];
    const int vdg = tid & 31;   // d group of DPT columns
    const int voct = tid >> 5;  // key octet: chunk voct/2, half voct%2

    auto load_tile = [&](int ks) {
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), cc = c % (D / 8);
            const int key = ks + row;
            kst[i] = key < n_k ? *(const uint4*)(Kh + (size_t)key * D + 8 * cc) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = ks + 16 * (voct >> 1) + 8 * (e >> 2) + 4 * (voct & 1) + (e & 3);
            if (key < n_k) {
                vst[e] = *(const vword_t*)(Vh + (size_t)key * D + DPT * vdg);
            } else {
#pragma unroll
                for (int w = 0; w < DPT / 2; ++w) vst[e][w] = 0u;
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CK; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), cc = c % (D / 8);
            *(uint4*)(&Ks[buf][row * KSTR + 8 * cc]) = kst[i];
        }
        // Transpose 8 keys x DPT columns into DPT rows of 8 keys.
#pragma unroll
        for (int dd = 0; dd < DPT; ++dd) {
            const int w = dd >> 1, sh = 16 * (dd & 1);
            unsigned h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (vst[e][w] >> sh) & 0xffffu;
            uint4 pk = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                  h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            *(uint4*)(&Vt[buf][(DPT * vdg + dd) * VSTR + 16 * (voct >> 1) + 8 * (voct & 1)]) = pk;
        }
    };

    float m_run[QB], l_run[QB];
    f32x16 o[QB][NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = kNegInf;
        l_run[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qb][db] = zero_f32x16();
    }

    const int wave_last_row = min(qw + RW, n_q) - 1;  // < qw when the wave has no rows

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int ks = t * kBC;
        const bool has_next = t + 1 < ntiles;
        if (has_next) load_tile(ks + kBC);

        const bool active = wave_last_row >= qw && (!CAUSAL || ks <= wave_last_row);
        if (active) {
            // S^T (keys x queries) for two 32-key blocks.
            f32x16 s[QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][0] = s[qb][1] = zero_f32x16();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *(const bf16x8*)(&Ks[buf][(32 * kb + r) * KSTR + 16 * kk + 8 * g]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qreg[qb][kk], s[qb][kb]);
                }
            }
            // Mask: keys past n_k, and (causal) keys after the query.
            const bool need_mask = (ks + kBC > n_k) || (CAUSAL && ks + kBC - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int row = qw + 32 * qb + r;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int key = ks + 32 * kb + acc_row(v, g);
                            if (key >= n_k || (CAUSAL && key > row)) s[qb][kb][v] = kNegInf;
                        }
                }
            }
            // Online softmax; P packed as bf16 B operands, 4 chunks of 16 keys.
            bf16x8 pb[QB][4];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = kNegInf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[qb][kb][v]);
                mx = halves_max(mx);
                const float m_new = fmaxf(m_run[qb], mx * scale2);
                const float m_use = m_new == kNegInf ? 0.0f : m_new;
                const float corr = fast_exp2(m_run[qb] - m_use);
                float rs = 0.0f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float p = fast_exp2(fmaf(s[qb][kb][v], scale2, -m_use));
                        rs += p;
                        pb[qb][2 * kb + (v >> 3)][v & 7] = to_bf16(p);
                    }
                l_run[qb] = l_run[qb] * corr + rs;
                m_run[qb] = m_new;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[qb][db][v] *= corr;
            }
            // O^T (d x queries) += V^T P^T.
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 a = *(const bf16x8*)(&Vt[buf][(32 * db + r) * VSTR + 16 * c + 8 * g]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(a, pb[qb][c], o[qb][db]);
                }
            }
        }
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O / l, L = ln 2 * (m + log2 l).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const int row = qw + 32 * qb + r;
        if (row < n_q) {
            const float inv = 1.0f / l;
            const size_t obase = ((size_t)bh * n_q + row) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int d0 = 32 * db + 8 * i + 4 * g;
                    const float x0 = o[qb][db][4 * i + 0] * inv, x1 = o[qb][db][4 * i + 1] * inv;
                    const float x2 = o[qb][db][4 * i + 2] * inv, x3 = o[qb][db][4 * i + 3] * inv;
                    if (OF32) {
                        *(float4*)((float*)Out + obase + d0) = make_float4(x0, x1, x2, x3);
                    } else {
                        bf16x4 pk;
                        pk[0] = to_bf16(x0); pk[1] = to_bf16(x1); pk[2] = to_bf16(x2); pk[3] = to_bf16(x3);
                        *(bf16x4*)((bf16*)Out + obase + d0) = pk;
                    }
                }
            if (g == 0) Lse[(size_t)bh * n_q + row] = kLn2 * (m_run[qb] + fast_log2(l));
        }
    }
}

template <int D, int QB, bool CAUSAL, bool OF32>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
    constexpr int BR = 128 * QB;
    const int n_qtiles = (a.n_q + BR - 1) / BR;
    const long long nwg = (long long)a.bh * n_qtiles;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, CAUSAL, OF32>), dim3((unsigned)nwg), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.o, a.lse,
                       a.n_q, a.n_k, n_qtiles, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, int QB>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t st) {
    if (a.causal)
        return a.o_f32 ? launch<D, QB, true, true>(a, st) : launch<D, QB, true, false>(a, st);
    return a.o_f32 ? launch<D, QB, false, true>(a, st) : launch<D, QB, false, false>(a, st);
}

}  // namespace

int fwd_bf16_rows_per_wg(const FwdArgs& a) {
    // Two 32-row blocks per wave halve the LDS operand traffic per MFMA but
    // need enough tiles to fill 256 CUs.
    const int qb = fwd_bf16_qb_override();
    if (qb == 1 || qb == 2) return 128 * qb;
    const long long wg2 = (long long)a.bh * ((a.n_q + 255) / 256);
    return wg2 >= 512 ? 256 : 128;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
    const bool two = fwd_bf16_rows_per_wg(a) == 256;
    switch (a.d) {
        case 64: return two ? dispatch_mask<64, 2>(a, st) : dispatch_mask<64, 1>(a, st);
        case 128: return two ? dispatch_mask<128, 2>(a, st) : dispatch_mask<128, 1>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
