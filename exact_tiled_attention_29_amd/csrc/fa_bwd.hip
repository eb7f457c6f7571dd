// Backward attention kernels for bf16 inputs on gfx950.
//
// Algorithm: the recomputation backward of page 1 ("05_flash_attention.py",
// section 3, flash_attention_backward): P is rebuilt tile by tile from the
// saved logsumexp as exp(S - L); dV += P^T dO; dP = dO V^T; dS = P * (dP - D)
// with D = rowsum(dO * O); dQ += scale * dS K; dK += scale * dS^T Q. Tiles
// wholly in the causal future are skipped. The derivative rules are those of
// page 3 ("Flash Attention"), section 1.5.
//
// Three kernels on one stream:
//  1. bwd_pre:  D = rowsum(dO * O) and L2 = L * log2(e) into per-head arrays
//     padded to a multiple of 32 rows (padding: L2 = +inf, D = 0, so padded
//     query rows get P = 0 and dS = 0 without any masking);
//  2. bwd_dkdv: key-stationary. One workgroup per 128 keys of one (batch,
//     head); each of its 4 waves keeps 32 keys' K and V rows in registers as
//     MFMA operands and their dK, dV in fp32 accumulators, and walks the
//     32-row query tiles (S, dP, dV, dK: 4 products per tile pair);
//  3. bwd_dq:   query-stationary, shaped like the forward kernel. One
//     workgroup per 128 queries; each wave keeps 32 queries' Q and dO rows in
//     registers and their dQ in fp32 accumulators, and walks the 64-key tiles
//     (S, dP recomputed, then dQ: 3 products per tile pair).
// Splitting dQ from dK/dV costs two extra products per tile pair but needs
// no atomics and no dS round trip through memory, keeps each kernel within a
// register budget that lets the hardware overlap waves, and makes every
// gradient deterministic.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBQ = 32;   // query rows per tile of the dK/dV kernel
constexpr int kBC = 64;   // keys per tile of the dQ kernel

// --------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and L2 = L * log2(e), padded per head.
// --------------------------------------------------------------------------
template <int D, typename OT>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const OT* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ Lse,
    float* __restrict__ l2p, float* __restrict__ dp, long long rows_pad, int n_q, int n_q_pad) {
    constexpr int LPR = D / 8;               // lanes per row, 8 elements each
    constexpr int RPB = kThreads / LPR;      // rows per block
    const int tid = threadIdx.x;
    const long long prow = (long long)blockIdx.x * RPB + tid / LPR;
    const int sub = tid % LPR;
    const long long bh = prow / n_q_pad;
    const int q = (int)(prow % n_q_pad);
    const bool valid = prow < rows_pad && q < n_q;
    float acc = 0.0f;
    if (valid) {
        const size_t base = ((size_t)bh * n_q + q) * D + 8 * sub;
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
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (prow < rows_pad && sub == 0) {
        dp[prow] = valid ? acc : 0.0f;
        l2p[prow] = valid ? Lse[(size_t)bh * n_q + q] * kLog2e : __builtin_huge_valf();
    }
}

// --------------------------------------------------------------------------
// 2. dK, dV: key-stationary, software-pipelined.
// --------------------------------------------------------------------------
// One wave per SIMD (the K/V operands and dK/dV accumulators take most of
// the register file), so the wave overlaps its own work: while the matrix
// core computes S and dP of query tile t+1, the wave's VALU turns S, dP of
// tile t into P and dS; then dV, dK of tile t follow. Query tiles stream
// through a ring of three LDS buffers: t (read by the dV/dK products), t+1
// (read by the S/dP products) and t+2 (being copied).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ l2p, const float* __restrict__ dp,
    bf16* __restrict__ dK, bf16* __restrict__ dV,
    int n_q, int n_k, int n_q_pad, int n_ktiles, float scale, float scale2) {
    constexpr int BKV = 128;           // keys per workgroup (32 per wave)
    constexpr int KK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int TILE = kBQ * D;      // elements per Q or dO tile
    constexpr int LPW = TILE * 2 / 1024 / 4;  // 1 KB direct copies per wave per tile

    // One LDS object per ring slot, holding the slot's Q tile, dO tile
    // (row-major, swizzled 16-byte chunks) and the L2, D values of its rows.
    // Distinct objects let the compiler tell a slot being copied from slots
    // being read (it tracks only a few copy targets, so the slot's three
    // parts share one object).
    constexpr int SLOT = 2 * TILE + 4 * kBQ;   // bf16 elements per slot
    __shared__ __attribute__((aligned(16))) bf16 Sl0[SLOT];
    __shared__ __attribute__((aligned(16))) bf16 Sl1[SLOT];
    __shared__ __attribute__((aligned(16))) bf16 Sl2[SLOT];
    auto q_of = [](bf16* sl) { return sl; };
    auto do_of = [](bf16* sl) { return sl + TILE; };
    auto ld_of = [](bf16* sl) { return (float*)(sl + 2 * TILE); };

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;

    int bh, kt;   // rank = key tile, ascending: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_ktiles, n_ktiles, &bh, &kt);
    const int k0 = kt * BKV;
    const int kw0 = k0 + 32 * wave;      // this wave's first key
    const int key = kw0 + r;             // this lane's key (column of S, dP)

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* dOh = dO + (size_t)bh * n_q * D;
    const bf16* Kh = K + (size_t)bh * n_k * D;
    const bf16* Vh = V + (size_t)bh * n_k * D;
    const float* l2h = l2p + (size_t)bh * n_q_pad;
    const float* dph = dp + (size_t)bh * n_q_pad;

    // K, V rows of this wave's keys as B operands (column = key, k = d).
    bf16x8 kreg[KK], vreg[KK];
    {
        const int kc = min(key, n_k - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 kx = *(const bf16x8*)(Kh + kc * D + 16 * kk + 8 * g);
            const bf16x8 vx = *(const bf16x8*)(Vh + kc * D + 16 * kk + 8 * g);
            kreg[kk] = key < n_k ? kx : zero_bf16x8();
            vreg[kk] = key < n_k ? vx : zero_bf16x8();
        }
    }

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = zero_f32x16();

    // Copy query tile t (rows q0 .. q0+31; rows past n_q fall outside the
    // buffer and read as zeros, and their L2 = +inf padding makes P = 0) and
    // its L2, D values into LDS.
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, n_q * D * 2);
    const __amdgpu_buffer_rsrc_t dors = make_rsrc(dOh, n_q * D * 2);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(l2h, n_q_pad * 4);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dph, n_q_pad * 4);
    auto issue_tile = [&](bf16* Qd, bf16* dOd, float* LDd, int t) {
        const int q0 = t * kBQ;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int b = 4 * i + wave;
            const int p = 64 * b + lane;
            const int row = p / (D / 8), pc = p % (D / 8);
            const int chunk = pc ^ tile_swz<D>(row);
            const int boff = ((q0 + row) * D + 8 * chunk) * 2;
            load_lds16(qrs, boff, Qd + 512 * b);
            load_lds16(dors, boff, dOd + 512 * b);
        }
        // lanes 0-7: 8 x 16 B of L2 into LDd[0..31]; lanes 8-15: D into
        // LDd[32..63] (q0 is a multiple of 32 < n_q_pad)
        if (wave == 0) {
            if (lane < 8) load_lds16(lrs, (q0 + 4 * lane) * 4, LDd);
            else if (lane < 16) load_lds16(drs, (q0 + 4 * (lane - 8)) * 4, LDd);
        }
    };

    // Per-lane byte offsets of the LDS operand reads, the same for every
    // buffer. Each step passes them through an empty asm so that the
    // buffer's base is added inside the step and folds into the read's
    // immediate offset (otherwise every buffer/offset pair is hoisted out of
    // the loop into a register of its own).
    //  soff[kk]:       Q / dO row r, k-step kk (A operands of S and dP);
    //  troff[c][j][h]: transpose reads for dV / dK, B operand of product
    //                  (c, db = j), rows 16c + 4g + s16/4 + 8h.
    int soff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) soff[kk] = 2 * tile_off<D>(r, 16 * kk + 8 * g);
    int troff[2][NDB][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                troff[c][db][h] = 2 * tile_off<D>(16 * c + 4 * g + (s16 >> 2) + 8 * h,
                                                  32 * db + 16 * half + 4 * (s16 & 3));
    auto at = [](const bf16* base, int byte_off) {
        return (const bf16*)((const char*)base + byte_off);
    };
    auto launder_offsets = [&]() {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(soff[kk]));
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(troff[c][db][h]));
    };

    // S = Q K^T and dP = dO V^T of one staged tile (rows = queries, columns
    // = keys). Lane holds key kw0 + r; element v is query q0 + acc_row(v, g).
    // The Q, dO operands are read kLookS k-steps ahead of their MFMAs.
    constexpr int kLookS = 3;
    auto scores = [&](const bf16* Qb, const bf16* dOb, f32x16& s, f32x16& dpv) {
        s = zero_f32x16();
        dpv = zero_f32x16();
        bf16x8 aq[kLookS + 1], ad[kLookS + 1];
#pragma unroll
        for (int kk = 0; kk < kLookS && kk < KK; ++kk) {
            aq[kk] = *(const bf16x8*)at(Qb, soff[kk]);
            ad[kk] = *(const bf16x8*)at(dOb, soff[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + kLookS < KK) {
                aq[(kk + kLookS) % (kLookS + 1)] = *(const bf16x8*)at(Qb, soff[kk + kLookS]);
                ad[(kk + kLookS) % (kLookS + 1)] = *(const bf16x8*)at(dOb, soff[kk + kLookS]);
            }
            s = mfma32(aq[kk % (kLookS + 1)], kreg[kk], s);
            dpv = mfma32(ad[kk % (kLookS + 1)], vreg[kk], dpv);
        }
    };

    // L2 and D of the 16 queries this lane's accumulator elements hold:
    // element v = 4i + j is query q0 + 8i + 4g + j.
    auto read_ld = [&](const float* LDb, float* lq, float* dq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 l4 = *(const float4*)(&LDb[8 * i + 4 * g]);
            const float4 d4 = *(const float4*)(&LDb[kBQ + 8 * i + 4 * g]);
            lq[4 * i] = l4.x; lq[4 * i + 1] = l4.y; lq[4 * i + 2] = l4.z; lq[4 * i + 3] = l4.w;
            dq[4 * i] = d4.x; dq[4 * i + 1] = d4.y; dq[4 * i + 2] = d4.z; dq[4 * i + 3] = d4.w;
        }
    };

    // Element v of P = exp2(S * scale * log2(e) - L2) and dS = P * (dP - D)
    // into the bf16 A operands of the dV, dK products (k = query), without
    // the mask (apply_mask follows on tiles that need it).
    auto softmax_elem = [&](int v, const f32x16& s, const f32x16& dpv, const float* lq,
                            const float* dq, bf16x8* pa, bf16x8* dsa) {
        const float p = fast_exp2(fmaf(s[v], scale2, -lq[v]));
        pa[v >> 3][v & 7] = to_bf16(p);
        dsa[v >> 3][v & 7] = to_bf16(p * (dpv[v] - dq[v]));
    };

    // Zero P and dS where the key is past n_k or (causal) after the query:
    // element v (query offset 8*(v/4) + v%4 from q0 + 4g) is masked iff that
    // offset is below lim. Works on the packed bf16 pairs with bit masks, so
    // whatever an unmasked element held there (even inf or NaN) is cleared.
    auto apply_mask = [&](int lim, bf16x8* pa, bf16x8* dsa) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            auto pw = __builtin_bit_cast(uint4, pa[c]);
            auto dw = __builtin_bit_cast(uint4, dsa[c]);
            unsigned keep[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int v = 8 * c + 2 * w;   // elements v, v + 1 in word w
                const int off = 8 * (v >> 2) + (v & 3);
                keep[w] = (off < lim ? 0u : 0x0000ffffu) | (off + 1 < lim ? 0u : 0xffff0000u);
            }
            pw.x &= keep[0]; pw.y &= keep[1]; pw.z &= keep[2]; pw.w &= keep[3];
            dw.x &= keep[0]; dw.y &= keep[1]; dw.z &= keep[2]; dw.w &= keep[3];
            pa[c] = __builtin_bit_cast(bf16x8, pw);
            dsa[c] = __builtin_bit_cast(bf16x8, dw);
        }
    };

    // dV += P^T dO, dK += dS^T Q of one tile (rows = keys, columns = d) from
    // its P, dS operands; the B operands carry queries 16c + 8*(e/4) + 4g +
    // e%4 in slot (g, e), matching the accumulator order of P and dS, and
    // are read kLookG products ahead. With `with_softmax`, the (unmasked)
    // softmax of the tile after it (s, dpv -> pa_n, dsa_n) is computed
    // between the MFMAs, EPM elements after each.
    constexpr int NJ = 2 * NDB;                // (c, db) products of dV and of dK
    constexpr int EPM = 16 / (2 * NJ);         // softmax elements per MFMA
    constexpr int kLookG = 3;
    auto grads = [&](auto with_softmax, const bf16* Qb, const bf16* dOb, const bf16x8* pa,
                     const bf16x8* dsa, const f32x16& s, const f32x16& dpv, const float* lq,
                     const float* dq, bf16x8* pa_n, bf16x8* dsa_n) {
        bf16x8 bdo[kLookG + 1], bq[kLookG + 1];
        auto load = [&](int j) {
            const int c = j / NDB, db = j % NDB, slot = j % (kLookG + 1);
            bdo[slot] = concat(lds_read_tr(at(dOb, troff[c][db][0])), lds_read_tr(at(dOb, troff[c][db][1])));
            bq[slot] = concat(lds_read_tr(at(Qb, troff[c][db][0])), lds_read_tr(at(Qb, troff[c][db][1])));
        };
#pragma unroll
        for (int j = 0; j < kLookG && j < NJ; ++j) load(j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = j / NDB, db = j % NDB;
            if (j + kLookG < NJ) load(j + kLookG);
            dv[db] = mfma32(pa[c], bdo[j % (kLookG + 1)], dv[db]);
            if constexpr (decltype(with_softmax)::value) {
#pragma unroll
                for (int e = 0; e < EPM; ++e)
                    softmax_elem(2 * EPM * j + e, s, dpv, lq, dq, pa_n, dsa_n);
            }
            dk[db] = mfma32(dsa[c], bq[j % (kLookG + 1)], dk[db]);
            if constexpr (decltype(with_softmax)::value) {
#pragma unroll
                for (int e = 0; e < EPM; ++e)
                    softmax_elem(2 * EPM * j + EPM + e, s, dpv, lq, dq, pa_n, dsa_n);
            }
        }
    };

    const int nqt = (n_q + kBQ - 1) / kBQ;
    const int t_begin = CAUSAL ? k0 / kBQ : 0;
    const std::true_type yes{};
    const std::false_type no{};
    auto mask_limit = [&](int q0) { return key >= n_k ? 64 : (CAUSAL ? key - q0 - 4 * g : -1); };
    auto needs_mask = [&](int q0) { return (kw0 + 32 > n_k) || (CAUSAL && kw0 + 31 > q0); };

    // P and dS of the previous tile (A operands of its dV, dK products).
    bf16x8 pa_p[2], dsa_p[2];

    // One step for tile t: slots c (tile t), p (tile t-1), f (tile t+1,
    // copied during the step). S, dP of tile t on the matrix core; then the
    // dV, dK products of tile t-1 on the matrix core with the softmax of
    // tile t on the VALU between them.
    auto step = [&](bf16* Sc, bf16* Sp, bf16* Sf, int t) {
        copies_barrier();  // tile t landed; every wave is done with tile t-2's slot (f)
        if (t + 1 < nqt) issue_tile(q_of(Sf), do_of(Sf), ld_of(Sf), t + 1);
        launder_offsets();
        float lq[16], dq[16];
        read_ld(ld_of(Sc), lq, dq);
        f32x16 s, dpv;
        scores(q_of(Sc), do_of(Sc), s, dpv);
        bf16x8 pa[2], dsa[2];
        grads(yes, q_of(Sp), do_of(Sp), pa_p, dsa_p, s, dpv, lq, dq, pa, dsa);
        const int q0 = t * kBQ;
        if (needs_mask(q0)) apply_mask(mask_limit(q0), pa, dsa);
#pragma unroll
        for (int c = 0; c < 2; ++c) { pa_p[c] = pa[c]; dsa_p[c] = dsa[c]; }
    };

    if (t_begin < nqt) {
        // Tile t_begin + i is staged in slot i % 3.
        issue_tile(q_of(Sl0), do_of(Sl0), ld_of(Sl0), t_begin);
        copies_barrier();
        if (t_begin + 1 < nqt) issue_tile(q_of(Sl1), do_of(Sl1), ld_of(Sl1), t_begin + 1);
        {
            launder_offsets();
            float lq[16], dq[16];
            read_ld(ld_of(Sl0), lq, dq);
            f32x16 s, dpv;
            scores(q_of(Sl0), do_of(Sl0), s, dpv);
#pragma unroll
            for (int v = 0; v < 16; ++v) softmax_elem(v, s, dpv, lq, dq, pa_p, dsa_p);
            if (needs_mask(t_begin * kBQ)) apply_mask(mask_limit(t_begin * kBQ), pa_p, dsa_p);
        }
        // Unrolled by three so each step names its slots at compile time;
        // the loop has a single exit, which keeps the dK/dV accumulators in
        // the same registers across the steps.
        for (int t = t_begin + 1; t < nqt; t += 3) {
            step(Sl1, Sl0, Sl2, t);
            if (t + 1 < nqt) step(Sl2, Sl1, Sl0, t + 1);
            if (t + 2 < nqt) step(Sl0, Sl2, Sl1, t + 2);
        }
        // dV, dK of the last tile (already staged; no copy is in flight, so
        // its slot may be picked at run time).
        const int slot = (nqt - 1 - t_begin) % 3;
        bf16* Sll = slot == 0 ? Sl0 : (slot == 1 ? Sl1 : Sl2);
        const bf16* Ql = q_of(Sll);
        const bf16* dOl = do_of(Sll);
        launder_offsets();
        {
            const f32x16 z = zero_f32x16();
            float lz[16];
            bf16x8 unused[2];
            grads(no, Ql, dOl, pa_p, dsa_p, z, z, lz, lz, unused, unused);
        }
    }

    // Epilogue: dK = scale * acc; rows = keys kw0 + acc_row(v, g), column = d.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int kr = kw0 + acc_row(v, g);
            if (kr < n_k) {
                const size_t off = ((size_t)bh * n_k + kr) * D + 32 * db + r;
                dK[off] = to_bf16(dk[db][v] * scale);
                dV[off] = to_bf16(dv[db][v]);
            }
        }
}

// --------------------------------------------------------------------------
// 3. dQ: query-stationary.
// --------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ l2p, const float* __restrict__ dp,
    bf16* __restrict__ dQ, int n_q, int n_k, int n_q_pad, int n_qtiles, float scale, float scale2) {
    constexpr int RW = 32;               // query rows per wave
    constexpr int BR = 4 * RW;           // query rows per workgroup
    constexpr int KK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int TILE = kBC * D;        // elements per K or V tile
    constexpr int LPW = TILE * 2 / 1024 / 4;

    __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs1[TILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;

    int bh, rank;   // rank 0 = last query tile: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_qtiles, n_qtiles, &bh, &rank);
    const int qt = n_qtiles - 1 - rank;
    const int q0 = qt * BR;
    const int qw = q0 + wave * RW;

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* dOh = dO + (size_t)bh * n_q * D;
    const bf16* Kh = K + (size_t)bh * n_k * D;
    const bf16* Vh = V + (size_t)bh * n_k * D;

    // Q and dO rows as B operands (column = query, k = d); L2 and D of the
    // lane's query (both halves of the lane pair hold the same row).
    const int row = qw + r;
    bf16x8 qreg[KK], doreg[KK];
    {
        const int rc = min(row, n_q - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 x = *(const bf16x8*)(Qh + rc * D + 16 * kk + 8 * g);
            const bf16x8 y = *(const bf16x8*)(dOh + rc * D + 16 * kk + 8 * g);
            qreg[kk] = row < n_q ? x : zero_bf16x8();
            doreg[kk] = row < n_q ? y : zero_bf16x8();
        }
    }
    const float l2 = row < n_q ? l2p[(size_t)bh * n_q_pad + row] : __builtin_huge_valf();
    const float drw = row < n_q ? dp[(size_t)bh * n_q_pad + row] : 0.0f;

    int kend = n_k;
    if (CAUSAL) kend = min(n_k, min(q0 + BR, n_q));
    const int ntiles = (kend + kBC - 1) / kBC;

    // K, V tiles straight to LDS; rows past n_k read as zeros (masked keys).
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh, n_k * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vh, n_k * D * 2);
    auto issue_tile = [&](bf16* Kd, bf16* Vd, int ks) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int b = 4 * i + wave;
            const int p = 64 * b + lane;
            const int rw = p / (D / 8), pc = p % (D / 8);
            const int chunk = pc ^ tile_swz<D>(rw);
            const int boff = ((ks + rw) * D + 8 * chunk) * 2;
            load_lds16(krs, boff, Kd + 512 * b);
            load_lds16(vrs, boff, Vd + 512 * b);
        }
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();
    const int wave_last_row = min(qw + RW, n_q) - 1;

    auto tile_step = [&](const bf16* Kb, const bf16* Vb, int ks) {
        const bool active = wave_last_row >= qw && (!CAUSAL || ks <= wave_last_row);
        if (!active) return;
        const bool need_mask = (ks + kBC > n_k) || (CAUSAL && ks + kBC - 1 > qw);
        // Two 32-key halves, one after the other, to keep fewer values live.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mfma_priority(true);
            // S^T = K Q^T and dP^T = V dO^T (rows = keys, columns = queries);
            // K and V operands are read one k-step ahead of their MFMAs.
            f32x16 s = zero_f32x16(), dpt = zero_f32x16();
            bf16x8 ak[2], av[2];
            ak[0] = *(const bf16x8*)(&Kb[tile_off<D>(32 * kb + r, 8 * g)]);
            av[0] = *(const bf16x8*)(&Vb[tile_off<D>(32 * kb + r, 8 * g)]);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (kk + 1 < KK) {
                    ak[(kk + 1) & 1] = *(const bf16x8*)(&Kb[tile_off<D>(32 * kb + r, 16 * (kk + 1) + 8 * g)]);
                    av[(kk + 1) & 1] = *(const bf16x8*)(&Vb[tile_off<D>(32 * kb + r, 16 * (kk + 1) + 8 * g)]);
                }
                s = mfma32(ak[kk & 1], qreg[kk], s);
                dpt = mfma32(av[kk & 1], doreg[kk], dpt);
            }
            sched_reads_ahead_of_mfma<KK>();
            mfma_priority(false);
            // key of element v: ks + 32kb + 4g + 8*(v/4) + v%4 (see the forward)
            const int lim = (CAUSAL ? min(n_k, row + 1) : n_k) - ks - 32 * kb - 4 * g;
            bf16x8 dsb[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float p = fast_exp2(fmaf(s[v], scale2, -l2));
                if (need_mask && 8 * (v >> 2) + (v & 3) >= lim) p = 0.0f;
                dsb[v >> 3][v & 7] = to_bf16(p * (dpt[v] - drw));
            }
            // dQ^T (d x queries) += K^T dS^T; K^T operands by transpose reads.
            mfma_priority(true);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int col = 32 * db + 16 * half + 4 * (s16 & 3);
                    const int row0 = 32 * kb + 16 * c + 4 * g + (s16 >> 2);
                    const bf16x8 a = concat(lds_read_tr(&Kb[tile_off<D>(row0, col)]),
                                            lds_read_tr(&Kb[tile_off<D>(row0 + 8, col)]));
                    acc[db] = mfma32(a, dsb[c], acc[db]);
                }
            mfma_priority(false);
        }
    };

    issue_tile(Ks0, Vs0, 0);
    copies_barrier();
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) issue_tile(Ks1, Vs1, (t + 1) * kBC);
        tile_step(Ks0, Vs0, t * kBC);
        copies_barrier();
        if (t + 1 >= ntiles) break;
        if (t + 2 < ntiles) issue_tile(Ks0, Vs0, (t + 2) * kBC);
        tile_step(Ks1, Vs1, (t + 1) * kBC);
        copies_barrier();
    }

    if (row < n_q) {
        const size_t obase = ((size_t)bh * n_q + row) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = to_bf16(acc[db][4 * i + j] * scale);
                *(bf16x4*)(dQ + obase + 32 * db + 8 * i + 4 * g) = pk;
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_kernels(const BwdArgs& a, hipStream_t st) {
    const int n_q_pad = dq_rows_padded(a.n_q);
    const long long rows_pad = (long long)a.bh * n_q_pad;
    constexpr int RPB = kThreads / (D / 8);
    const long long nb = (rows_pad + RPB - 1) / RPB;
    const int n_ktiles = (a.n_k + 127) / 128;
    const int n_qtiles = (a.n_q + 127) / 128;
    if (nb > 0x7fffffffLL || (long long)a.bh * n_ktiles > 0x7fffffffLL ||
        (long long)a.bh * n_qtiles > 0x7fffffffLL)
        return hipErrorInvalidValue;
    hipError_t e = record_stage(a, 0, st);
    if (e != hipSuccess) return e;
    if (a.o_f32)
        hipLaunchKernelGGL((bwd_pre_kernel<D, float>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const float*)a.o, (const bf16*)a.d_o, a.lse, a.l2pad, a.drow, rows_pad,
                           a.n_q, n_q_pad);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<D, bf16>), dim3((unsigned)nb), dim3(kThreads), 0, st,
                           (const bf16*)a.o, (const bf16*)a.d_o, a.lse, a.l2pad, a.drow, rows_pad,
                           a.n_q, n_q_pad);
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 1, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * n_ktiles)), dim3(kThreads), 0,
                       st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.d_o,
                       (const float*)a.l2pad, (const float*)a.drow, (bf16*)a.dk, (bf16*)a.dv,
                       a.n_q, a.n_k, n_q_pad, n_ktiles, a.scale, a.scale * kLog2e);
    e = hipGetLastError();
    if (e == hipSuccess) e = record_stage(a, 2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * n_qtiles)), dim3(kThreads), 0,
                       st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.d_o,
                       (const float*)a.l2pad, (const float*)a.drow, (bf16*)a.dq,
                       a.n_q, a.n_k, n_q_pad, n_qtiles, a.scale, a.scale * kLog2e);
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
        case 64: return a.causal ? launch_kernels<64, true>(a, st) : launch_kernels<64, false>(a, st);
        case 128: return a.causal ? launch_kernels<128, true>(a, st) : launch_kernels<128, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
