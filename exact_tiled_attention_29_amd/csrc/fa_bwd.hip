// Backward attention kernels for bf16 inputs on gfx950.
//
// Algorithm: the recomputation backward of page 1 ("05_flash_attention.py",
// section 3, flash_attention_backward): P is rebuilt tile by tile from the
// saved logsumexp as exp(S - L); dV += P^T dO; dP = dO V^T; dS = P * (dP - D)
// with D = rowsum(dO * O); dQ += scale * dS K; dK += scale * dS^T Q. Tiles
// wholly in the causal future are skipped. The derivative rules are those of
// page 3 ("Flash Attention"), section 1.5. The causal diagonal is a runtime
// offset coff (key j visible to query i iff j <= i + coff), as in the forward;
// a query row that sees no key (L = -inf) gets L2 = +inf, so its P, dS and
// dQ are 0 and it adds nothing to dK, dV.
//
// Three kernels on one stream:
//  1. bwd_pre:  -D = -rowsum(dO * O) and L2 = L * log2(e) into per-head
//     arrays padded to a multiple of 32 rows (padding and rows with L = -inf:
//     L2 = +inf, D = 0, so those query rows get P = 0 and dS = 0 without any
//     masking); -D is where the dP accumulators of both later kernels start,
//     so their MFMAs deliver dP - D;
//  2. bwd_dkdv: key-stationary. One workgroup per 128 keys of one (batch,
//     head) (64 at d = 256), as 4 wave pairs of 32 keys each: one wave of a
//     pair keeps the keys' K rows as MFMA operands and their dV in fp32
//     accumulators, the other their V rows and dK; the workgroup walks the
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
// Lanes that share one row of the row pass: the largest power of two (at
// most 16) that divides the row's D/8 chunks of 8 elements.
constexpr int pre_lanes_per_row(int chunks) {
    int l = 1;
    while (l < 16 && chunks % (2 * l) == 0) l *= 2;
    return l;
}

template <int D, typename OT>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const OT* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ Lse,
    float* __restrict__ l2p, float* __restrict__ dp, long long rows_pad, int n_q, int n_q_pad) {
    constexpr int LPR = pre_lanes_per_row(D / 8);  // lanes per row
    constexpr int CPL = D / 8 / LPR;               // chunks of 8 elements per lane
    constexpr int RPB = kThreads / LPR;            // rows per block
    const int tid = threadIdx.x;
    const long long prow = (long long)blockIdx.x * RPB + tid / LPR;
    const int sub = tid % LPR;
    const long long bh = prow / n_q_pad;
    const int q = (int)(prow % n_q_pad);
    const bool valid = prow < rows_pad && q < n_q;
    float acc = 0.0f;
    if (valid) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const size_t base = ((size_t)bh * n_q + q) * D + 8 * (sub + LPR * c);
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
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (prow < rows_pad && sub == 0) {
        const float lse = valid ? Lse[(size_t)bh * n_q + q] : kNegInf;
        const bool live = lse > kNegInf;
        dp[prow] = live ? -acc : 0.0f;   // stored negated: the dP accumulators start from it
        l2p[prow] = live ? lse * kLog2e : __builtin_huge_valf();
    }
}

// --------------------------------------------------------------------------
// 2. dK, dV: key-stationary, two waves per group of keys.
// --------------------------------------------------------------------------
// One workgroup of 2 * NP waves per 32 * NP keys of one (batch, head), as NP
// groups of 32 keys (NP = 4; NP = 2 at d = 256, where a wave needs more than
// 256 registers, so only one wave may share each SIMD). A group is handled
// by a pair of waves that share its work:
//   wave A (waves 0 .. NP-1) keeps the group's K rows as MFMA operands and
//     the dV accumulator: S = Q K^T, P = exp2(S * scale * log2(e) - L2),
//     dV += P^T dO;
//   wave B (waves NP .. 2NP-1) keeps the group's V rows and the dK accumulator:
//     dP = dO V^T, dS = P * (dP - D), dK += dS^T Q.
// Wave A hands P to wave B through LDS as the bf16 values it feeds its own
// dV product (in the accumulator layout both waves use), so dS is formed
// from the same rounded P; dS is rounded to bf16 for the dK product anyway.
// Splitting the group this way halves each wave's registers,
// so (for NP = 4) two waves share each SIMD and one issues while the other
// waits.
// Query tiles of 32 rows stream through a ring of three LDS slots; a slot
// also holds the P that wave A computed from its tile, which wave B uses one
// step later. Within a step each wave overlaps its VALU work (A: the softmax
// of this tile; B: dS of the previous one) with its MFMAs.
// Wave pairs per dK/dV workgroup.
template <int D>
constexpr int dkdv_pairs() { return D >= 256 ? 2 : 4; }

// Query split (nsplit > 1, grids with few key blocks): virtual head
// bhv = bh * nsplit + s takes query rows [s * qchunk, (s + 1) * qchunk) only
// (qchunk a multiple of 32) and writes its fp32 partials of dK and dV at bhv
// in part_k / part_v; split_reduce_kernel adds them (both are sums over the
// queries).
template <int D, bool CAUSAL, int NP>
__global__ __launch_bounds__(128 * NP, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ l2p, const float* __restrict__ dp,
    bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ part_k,
    float* __restrict__ part_v, int n_q_all, int n_k, int coff, int n_q_pad, int n_ktiles,
    float scale, float scale2, int nsplit, int qchunk) {
    constexpr int NW = 2 * NP;         // waves
    constexpr int BKV = 32 * NP;       // keys per workgroup
    constexpr int KK = D / 16;
    constexpr int NDB = D / 32;
    constexpr int NJ = 2 * NDB;        // (c, db) products of a dV or dK update
    constexpr int TILE = kBQ * D;      // elements per Q or dO tile
    constexpr int NCH = TILE * 2 / 1024;  // 1 KB copies per tensor and tile
    static_assert(NCH * 1024 == TILE * 2, "whole 1 KB copies");
    constexpr int CPW = (2 * NCH + NW - 1) / NW;   // copies per wave and tile (at most)
    constexpr bool kEvenCopies = 2 * NCH % NW == 0;
    constexpr int XB = 64 * 16 * 2;    // bytes of P (bf16) per wave pair

    // One LDS object per ring slot: Q tile, dO tile (row-major, swizzled
    // 16-byte chunks), L2 and D of the tile's rows, and the NP pairs' P
    // (at byte 2 * (2 * TILE + 4 * kBQ); see exoff below).
    // Distinct objects let the compiler tell a slot being copied from slots
    // being read (it tracks only a few copy targets).
    constexpr int SLOT = 2 * TILE + 4 * kBQ + NP * XB / 2;   // bf16 units
    __shared__ __attribute__((aligned(16))) bf16 Sl0[SLOT];
    __shared__ __attribute__((aligned(16))) bf16 Sl1[SLOT];
    __shared__ __attribute__((aligned(16))) bf16 Sl2[SLOT];
    auto q_of = [](bf16* sl) { return sl; };
    auto do_of = [](bf16* sl) { return sl + TILE; };
    auto ld_of = [](bf16* sl) { return (float*)(sl + 2 * TILE); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;
    const bool role_a = wave < NP;
    const int pair = wave & (NP - 1);

    int bhv, kt;   // rank = key tile, ascending: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_ktiles, n_ktiles, &bhv, &kt);
    const int k0 = kt * BKV;
    const int kw0 = k0 + 32 * pair;      // the pair's first key
    const int key = kw0 + r;             // this lane's key (column of S, dP)
    // this workgroup's queries: rows [q_lo, q_lo + n_q) of head bh, with the
    // causal diagonal moved to those local row indices
    const int bh = bhv / nsplit;
    const int q_lo = (bhv - bh * nsplit) * qchunk;
    const int n_q = max(0, min(n_q_all, q_lo + qchunk) - q_lo);
    coff += q_lo;

    const bf16* Qh = Q + ((size_t)bh * n_q_all + q_lo) * D;
    const bf16* dOh = dO + ((size_t)bh * n_q_all + q_lo) * D;
    const float* l2h = l2p + (size_t)bh * n_q_pad + q_lo;
    const float* dph = dp + (size_t)bh * n_q_pad + q_lo;

    // K (wave A) or V (wave B) rows of the pair's keys as B operands
    // (column = key, k = d).
    bf16x8 kv[KK];
    {
        const bf16* src = (role_a ? K : V) + (size_t)bh * n_k * D;
        const int kc = min(key, n_k - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 x = *(const bf16x8*)(src + kc * D + 16 * kk + 8 * g);
            kv[kk] = key < n_k ? x : zero_bf16x8();
        }
    }

    // dV (wave A) or dK (wave B) accumulators, transposed: block db holds
    // rows = d (32 db ..), columns = the pair's keys, so each lane keeps its
    // own key's row (4 adjacent columns per 4 elements; see the epilogue).
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();

    // Copy query tile t (rows q0 .. q0+31; rows past n_q fall outside the
    // buffer and read as zeros, and their L2 = +inf padding makes P = 0) and
    // its L2, D values into a slot. Copy b of the tile (Q chunks, then dO
    // chunks) is issued by wave b % NW.
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qh, n_q * D * 2);
    const __amdgpu_buffer_rsrc_t dors = make_rsrc(dOh, n_q * D * 2);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(l2h, (n_q_pad - q_lo) * 4);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dph, (n_q_pad - q_lo) * 4);
    auto issue_tile = [&](bf16* Sd, int t) {
        const int q0 = t * kBQ;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int b = NW * i + wave;
            if (!kEvenCopies && b >= 2 * NCH) break;
            const bool is_q = b < NCH;
            const int chunk = is_q ? b : b - NCH;
            const int p = 64 * chunk + lane;
            const int row = p / (D / 8), pc = p % (D / 8);
            // unsigned: (n_q rounded up to the tile) * D * 2 may pass 2^31 - 1
            const unsigned boff = ((unsigned)(q0 + row) * D + 8u * (unsigned)(pc ^ tile_swz<D>(row))) * 2u;
            if (is_q) load_lds16(qrs, boff, q_of(Sd) + 512 * chunk);
            else load_lds16(dors, boff, do_of(Sd) + 512 * chunk);
        }
        // lanes 0-7: 8 x 16 B of L2 into LD[0..31]; lanes 8-15: D into
        // LD[32..63] (q0 is a multiple of 32 < n_q_pad)
        if (wave == 0) {
            if (lane < 8) load_lds16(lrs, (q0 + 4 * lane) * 4, ld_of(Sd));
            else if (lane < 16) load_lds16(drs, (q0 + 4 * (lane - 8)) * 4, ld_of(Sd));
        }
    };

    // Per-lane byte offsets of the LDS operand reads, the same for every
    // slot. Each step passes them through an empty asm so that the slot's
    // base is added inside the step and folds into the read's immediate
    // offset (otherwise every slot/offset pair is hoisted out of the loop
    // into a register of its own).
    //  soff[kk]:     tile row r, k-step kk (A operands of S and dP);
    //  troff[db][h]: transpose reads (B operands of dV and dK) of product
    //                (c, db), rows 16c + 4g + s16/4 + 8h; c = 1 adds 16
    //                rows, which keeps the swizzle, so it is a constant.
    int soff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) soff[kk] = 2 * tile_off<D>(r, 16 * kk + 8 * g);
    int troff[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            troff[db][h] = 2 * tile_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * half + 4 * (s16 & 3));
    static_assert(tile_swz<D>(16) == tile_swz<D>(0) && tile_swz<D>(17) == tile_swz<D>(1) &&
                      tile_swz<D>(18) == tile_swz<D>(2) && tile_swz<D>(19) == tile_swz<D>(3),
                  "16 rows down keeps the swizzle");
    //  ldoff:        L2 / D values of the lane's queries, 4g floats in;
    //  exoff:        the lane's P words in the exchange area.
    int ldoff = 2 * 2 * TILE + 4 * 4 * g;
    int exoff = 2 * (2 * TILE + 4 * kBQ) + pair * XB + 16 * lane;
    auto launder_offsets = [&]() {
        asm volatile("" : "+v"(ldoff));
        asm volatile("" : "+v"(exoff));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(soff[kk]));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(troff[db][h]));
    };
    auto at = [](const bf16* base, int byte_off) {
        return (const bf16*)((const char*)base + byte_off);
    };

    // Scheduling: the operand loops below are each a region of their own
    // (sched_barrier), with the order of reads, MFMAs and the VALU work
    // handed in pinned by group barriers: left to itself the scheduler
    // moves every LDS read next to the MFMA that uses it, which exposes the
    // read's latency on every MFMA.
    constexpr int kDsRead = 0x100, kMfma = 0x008, kValu = 0x402;  // VALU incl. transcendental

    // acc_s = T kv^T for a staged Q or dO tile T: rows = queries, columns =
    // the pair's keys; lane holds key kw0 + r, element v is query
    // q0 + acc_row(v, g). Tile operands are read kLookS k-steps ahead;
    // extra(kk) runs after the MFMA of k-step kk and issues about NV VALU
    // instructions.
    constexpr int kLookS = 3;
    auto rows_times_keys = [&](const bf16* Tb, f32x16& acc_s, auto&& extra, auto nv, const f32x16& init) {
        constexpr int NV = decltype(nv)::value;
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 a[kLookS + 1];
#pragma unroll
        for (int kk = 0; kk < kLookS && kk < KK; ++kk) a[kk] = *(const bf16x8*)at(Tb, soff[kk]);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + kLookS < KK)
                a[(kk + kLookS) % (kLookS + 1)] = *(const bf16x8*)at(Tb, soff[kk + kLookS]);
            // the first k-step reads init directly (no copy into acc_s)
            acc_s = mfma32(a[kk % (kLookS + 1)], kv[kk], kk == 0 ? init : acc_s);
            extra(kk);
        }
        __builtin_amdgcn_sched_group_barrier(kDsRead, kLookS < KK ? kLookS : KK, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            if (NV > 0) __builtin_amdgcn_sched_group_barrier(kValu, NV, 0);
            if (kk + kLookS < KK) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // acc[db] += T^T X for a staged Q or dO tile T (acc rows = d, columns =
    // keys), X = P or dS as B operands (k = query). The A operands carry
    // queries 16c + 8*(e/4) + 4g + e%4 in slot (g, e), matching the
    // accumulator order of P and dS, and are read kLookG products ahead;
    // extra(j) runs after product j and issues about NV VALU instructions.
    constexpr int kLookG = 3;
    auto keys_times_tile = [&](const bf16* Tb, const bf16x8* xa, auto&& extra, auto nv) {
        constexpr int NV = decltype(nv)::value;
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 b[kLookG + 1];
        auto load = [&](int j) {
            const int cb = (j / NDB) * 16 * D * 2, db = j % NDB;
            b[j % (kLookG + 1)] = concat(lds_read_tr(at(Tb, troff[db][0] + cb)),
                                         lds_read_tr(at(Tb, troff[db][1] + cb)));
        };
#pragma unroll
        for (int j = 0; j < kLookG && j < NJ; ++j) load(j);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (j + kLookG < NJ) load(j + kLookG);
            acc[j % NDB] = mfma32(b[j % (kLookG + 1)], xa[j / NDB], acc[j % NDB]);
            extra(j);
        }
        __builtin_amdgcn_sched_group_barrier(kDsRead, 2 * (kLookG < NJ ? kLookG : NJ), 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            if (NV > 0) __builtin_amdgcn_sched_group_barrier(kValu, NV, 0);
            if (j + kLookG < NJ) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // 16 fp32 values of this lane's queries (element v = 4i + j is query
    // q0 + 8i + 4g + j) from slot Sd's L2 (part 0) or D (part 1) array.
    auto read_rows = [&](bf16* Sd, int part, float* x) {
        const float* ld = (const float*)at(Sd, ldoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = *(const float4*)(ld + kBQ * part + 8 * i);
            x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
        }
    };
    // P exchange (bf16, the A operands wave A already holds): 16-byte word i
    // of lane l of pair p at byte p*XB + 1024i + 16l, so each 16-byte access
    // of a wave covers 1 KB contiguously.
    auto write_p = [&](bf16* Sd, const bf16x8* pa) {
        char* ex = (char*)Sd + exoff;
        *(bf16x8*)ex = pa[0];
        *(bf16x8*)(ex + 1024) = pa[1];
    };
    auto read_p = [&](bf16* Sd, float* p) {
        const char* ex = (const char*)Sd + exoff;
        const bf16x8 a = *(const bf16x8*)ex, b = *(const bf16x8*)(ex + 1024);
#pragma unroll
        for (int e = 0; e < 8; ++e) { p[e] = bf2f(a[e]); p[8 + e] = bf2f(b[e]); }
    };

    // One step's MFMAs of a wave as a single operand stream: KK products
    // acc1 = T1 kv^T (operands read from tile T1 by rows), then NJ products
    // acc[db] += T2^T X (operands read from tile T2 by transpose). Operands
    // are read kLook stream positions ahead, across the change of tile, so
    // the second phase starts with its operands in registers. pre() issues
    // NPRE other LDS reads first; extra1(kk) / extra2(j) run after the MFMAs
    // of the two phases with about NV1 / NV2 VALU instructions each.
    constexpr int kLook = 3;   // with the raised priority, 3 beat 2, 4 and 5 (measured)
    auto stream = [&](const bf16* T1, f32x16& acc1, const f32x16& init1, const bf16* T2,
                      const bf16x8* X, auto&& pre, auto npre, auto&& extra1, auto nv1, auto&& extra2,
                      auto nv2) {
        constexpr int NPRE = decltype(npre)::value;
        constexpr int NV1 = decltype(nv1)::value, NV2 = decltype(nv2)::value;
        constexpr int NS = KK + NJ;
        __builtin_amdgcn_sched_barrier(0);
        // Raised issue priority for the stream (both waves): MFMAs and their
        // operand reads go first, the other wave's VALU work fills the gaps.
        mfma_priority(true);
        pre();
        bf16x8 op[kLook + 1];
        auto load = [&](int i) {
            if (i < KK) {
                op[i % (kLook + 1)] = *(const bf16x8*)at(T1, soff[i]);
            } else {
                const int j = i - KK, cb = (j / NDB) * 16 * D * 2, db = j % NDB;
                op[i % (kLook + 1)] = concat(lds_read_tr(at(T2, troff[db][0] + cb)),
                                             lds_read_tr(at(T2, troff[db][1] + cb)));
            }
        };
#pragma unroll
        for (int i = 0; i < kLook; ++i) load(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + kLook < NS) load(i + kLook);
            if (i < KK) {
                // the first product reads init1 directly (no copy into acc1)
                acc1 = mfma32(op[i % (kLook + 1)], kv[i], i == 0 ? init1 : acc1);
                extra1(i);
            } else {
                const int j = i - KK;
                acc[j % NDB] = mfma32(op[i % (kLook + 1)], X[j / NDB], acc[j % NDB]);
                extra2(j);
            }
        }
        // DS read instructions per stream position: 1 (row read), 2 (transpose)
        constexpr int FIRST = NPRE + (kLook <= KK ? kLook : KK + 2 * (kLook - KK));
        __builtin_amdgcn_sched_group_barrier(kDsRead, FIRST, 0);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            if (i < KK && NV1 > 0) __builtin_amdgcn_sched_group_barrier(kValu, NV1, 0);
            if (i >= KK && NV2 > 0) __builtin_amdgcn_sched_group_barrier(kValu, NV2, 0);
            if (i + kLook < KK) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
            else if (i + kLook < NS) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_priority(false);
    };

    const int nqt = (n_q + kBQ - 1) / kBQ;
    // first query tile with a row that sees key k0 (rows >= k0 - coff)
    const int t_begin = CAUSAL ? max(0, k0 - coff) / kBQ : 0;
    auto noop = [](int) {};
    const std::integral_constant<int, 0> nv0{};
    auto none = []() {};
    // VALU instructions per MFMA of wave A's softmax (fma, exp per element).
    // Softmax elements per product of the dV update (the last product may
    // get fewer when NJ does not divide 16).
    constexpr int EPM = (16 + NJ - 1) / NJ;
    const std::integral_constant<int, 2 * EPM> nv_softmax{};
    const std::integral_constant<int, 4> n_row_reads{};

    // Wave A's P of tile t (q0 = t * kBQ): zero where the key is past n_k or
    // (causal) after the query (element v's query offset 8*(v/4) + v%4 from
    // q0 + 4g is masked iff below lim), round them to bf16 (A operands of
    // dV) and hand those to wave B through slot Sd.
    auto finish_p = [&](int q0, float* p, bf16* Sd, bf16x8* pa) {
        if ((kw0 + 32 > n_k) || (CAUSAL && kw0 + 31 > q0 + coff)) {
            const int lim = key >= n_k ? 64 : (CAUSAL ? key - coff - q0 - 4 * g : -1);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (8 * (v >> 2) + (v & 3) < lim) p[v] = 0.0f;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) pa[v >> 3][v & 7] = to_bf16(p[v]);
        write_p(Sd, pa);
    };

    if (t_begin < nqt) {
        // Tile t_begin + i is staged in slot i % 3.
        issue_tile(Sl0, t_begin);
        copies_barrier();
        if (t_begin + 1 < nqt) issue_tile(Sl1, t_begin + 1);
        launder_offsets();
        const int t_last = nqt - 1;
        const int s_last = (t_last - t_begin) % 3;
        if (role_a) {
            // P of the previous tile (A operands of its dV update).
            bf16x8 pa_p[2];
            {
                float lq[16], p[16];
                read_rows(Sl0, 0, lq);
                f32x16 s;
                rows_times_keys(q_of(Sl0), s, noop, nv0, zero_f32x16());
#pragma unroll
                for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(s[v], scale2, -lq[v]));
                finish_p(t_begin * kBQ, p, Sl0, pa_p);
            }
            // Step for tile t: slots c (tile t), p (t-1), f (t+1, copied
            // during the step). S of tile t, then dV of tile t-1 with the
            // softmax of tile t between its MFMAs.
            auto step = [&](bf16* Sc, bf16* Sp, bf16* Sf, int t) {
                copies_barrier();  // tile t landed; everyone is done with slot f (tile t-2)
                if (t + 1 < nqt) issue_tile(Sf, t + 1);
                launder_offsets();
                float lq[16], p[16];
                f32x16 s;
                stream(q_of(Sc), s, zero_f32x16(), do_of(Sp), pa_p, [&]() { read_rows(Sc, 0, lq); }, n_row_reads,
                       noop, nv0, [&](int j) {
#pragma unroll
                    for (int e = 0; e < EPM; ++e) {
                        const int v = EPM * j + e;
                        if (v < 16) p[v] = fast_exp2(fmaf(s[v], scale2, -lq[v]));
                    }
                }, nv_softmax);
                finish_p(t * kBQ, p, Sc, pa_p);
            };
            // Unrolled by three so each step names its slots at compile
            // time; a single loop exit keeps the accumulators in place.
            for (int t = t_begin + 1; t < nqt; t += 3) {
                step(Sl1, Sl0, Sl2, t);
                if (t + 1 < nqt) step(Sl2, Sl1, Sl0, t + 1);
                if (t + 2 < nqt) step(Sl0, Sl2, Sl1, t + 2);
            }
            copies_barrier();  // pairs with wave B's wait for the last P
            bf16* Sl = s_last == 0 ? Sl0 : (s_last == 1 ? Sl1 : Sl2);
            launder_offsets();
            keys_times_tile(do_of(Sl), pa_p, noop, nv0);
        } else {
            // dP - D of the previous tile (its dS is formed one step later):
            // the accumulators start from -D of the tile's queries (element
            // v's query is the one of element v of read_rows).
            auto neg_d_of = [&](bf16* Sd) {
                float nd[16];
                read_rows(Sd, 1, nd);
                f32x16 x;
#pragma unroll
                for (int v = 0; v < 16; ++v) x[v] = nd[v];
                return x;
            };
            // dP - D alternates between two register sets (dp_x, dp_y): a
            // step forms dS from one and writes the next tile's dP into the
            // other, which is dead at that point. (With one loop-carried set
            // the compiler put the new dP elsewhere and copied it back after
            // every step.)
            f32x16 dp_x, dp_y;
            rows_times_keys(do_of(Sl0), dp_x, noop, nv0, neg_d_of(Sl0));
            // Step for tile t: dS = P * (dP - D) of tile t-1 (from wave A's
            // P, dP - D in dp_in), dP - D of tile t (into dp_out), then dK
            // of tile t-1. The dS work runs while wave A of the same SIMD
            // keeps the matrix core busy.
            auto step = [&](bf16* Sc, bf16* Sp, bf16* Sf, int t, const f32x16& dp_in, f32x16& dp_out) {
                copies_barrier();  // tile t landed; P of tile t-1 written
                if (t + 1 < nqt) issue_tile(Sf, t + 1);
                launder_offsets();
                float p[16];
                const f32x16 nd = neg_d_of(Sc);
                read_p(Sp, p);
                bf16x8 dsa[2];
#pragma unroll
                for (int v = 0; v < 16; ++v) dsa[v >> 3][v & 7] = to_bf16(p[v] * dp_in[v]);
                stream(do_of(Sc), dp_out, nd, q_of(Sp), dsa, none, nv0, noop, nv0, noop, nv0);
            };
            // Unrolled by six: three ring slots times two dP sets.
            for (int t = t_begin + 1; t < nqt; t += 6) {
                step(Sl1, Sl0, Sl2, t, dp_x, dp_y);
                if (t + 1 < nqt) step(Sl2, Sl1, Sl0, t + 1, dp_y, dp_x);
                if (t + 2 < nqt) step(Sl0, Sl2, Sl1, t + 2, dp_x, dp_y);
                if (t + 3 < nqt) step(Sl1, Sl0, Sl2, t + 3, dp_y, dp_x);
                if (t + 4 < nqt) step(Sl2, Sl1, Sl0, t + 4, dp_x, dp_y);
                if (t + 5 < nqt) step(Sl0, Sl2, Sl1, t + 5, dp_y, dp_x);
            }
            copies_barrier();  // P of the last tile written
            bf16* Sl = s_last == 0 ? Sl0 : (s_last == 1 ? Sl1 : Sl2);
            launder_offsets();
            // the last tile's dP - D: in dp_x after an even number of steps
            const bool in_x = ((t_last - t_begin) & 1) == 0;
            float p[16];
            read_p(Sl, p);
            bf16x8 dsa[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) dsa[v >> 3][v & 7] = to_bf16(p[v] * (in_x ? dp_x[v] : dp_y[v]));
            keys_times_tile(q_of(Sl), dsa, noop, nv0);
        }
    }

    // Epilogue: wave A stores dV, wave B stores dK = scale * acc (lane (r, g)
    // holds the row of key kw0 + r). Under the query split the fp32 partials
    // of virtual head bhv go out directly, 16 bytes per (db, i); otherwise
    // each wave stages its bf16 rows in the (now idle) ring and stores them
    // whole (store_rows_via_lds).
    const float f = role_a ? 1.0f : scale;
    if (part_k) {
        if (key < n_k) {
            float* out = (role_a ? part_v : part_k) + ((size_t)bhv * n_k + key) * D + 4 * g;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *(float4*)(out + 32 * db + 8 * i) =
                        make_float4(acc[db][4 * i] * f, acc[db][4 * i + 1] * f, acc[db][4 * i + 2] * f,
                                    acc[db][4 * i + 3] * f);
        }
    } else {
        constexpr int SB = 32 * D * 2;              // staging bytes per wave
        constexpr int WPS = SLOT * 2 / SB;          // waves staged per slot
        static_assert(3 * WPS >= NW, "the staging blocks fit the ring");
        copies_barrier();   // every wave is done with the ring, no copy in flight
        bf16* sl = wave / WPS == 0 ? Sl0 : (wave / WPS == 1 ? Sl1 : Sl2);
        store_rows_via_lds<D>((char*)sl + (wave % WPS) * SB, (role_a ? dV : dK) + ((size_t)bh * n_k + kw0) * D,
                              n_k - kw0, [&](int db, int v) { return acc[db][v] * f; });
    }
}

// --------------------------------------------------------------------------
// 3. dQ: query-stationary.
// --------------------------------------------------------------------------
// Key split (nsplit > 1, grids with few query tiles): virtual head
// bhv = bh * nsplit + s sums dS K over keys [s * kchunk, (s + 1) * kchunk)
// only and writes that fp32 partial of dQ at bhv in `part`; dq_reduce_kernel
// adds the partials (dQ is linear in the keys' terms).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D >= 256 ? 1 : 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ l2p, const float* __restrict__ dp,
    bf16* __restrict__ dQ, float* __restrict__ part, int n_q, int n_k_all, int coff, int n_q_pad,
    int n_qtiles, float scale, float scale2, int nsplit, int kchunk) {
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

    static_assert(32 * D * 4 <= TILE * 2, "a wave's fp32 rows fit one tile buffer");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;

    int bhv, rank;   // rank 0 = last query tile: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_qtiles, n_qtiles, &bhv, &rank);
    const int qt = n_qtiles - 1 - rank;
    const int q0 = qt * BR;
    const int qw = q0 + wave * RW;
    // this workgroup's keys: [k_lo, k_lo + n_k) of head bh, with the causal
    // diagonal moved to those local key indices
    const int bh = bhv / nsplit;
    const int k_lo = (bhv - bh * nsplit) * kchunk;
    const int n_k = max(0, min(n_k_all, k_lo + kchunk) - k_lo);
    coff -= k_lo;

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* dOh = dO + (size_t)bh * n_q * D;
    const bf16* Kh = K + ((size_t)bh * n_k_all + k_lo) * D;
    const bf16* Vh = V + ((size_t)bh * n_k_all + k_lo) * D;

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
    const float ndrw = row < n_q ? dp[(size_t)bh * n_q_pad + row] : 0.0f;   // -D
    // Every element of a lane's dP^T accumulator belongs to the lane's query,
    // so the accumulator starts at -D and the MFMAs deliver dP - D directly.
    f32x16 neg_d;
#pragma unroll
    for (int v = 0; v < 16; ++v) neg_d[v] = ndrw;

    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + BR, n_q) + coff));
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
            const unsigned boff = ((unsigned)(ks + rw) * D + 8u * (unsigned)chunk) * 2u;   // see above
            load_lds16(krs, boff, Kd + 512 * b);
            load_lds16(vrs, boff, Vd + 512 * b);
        }
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();
    const int wave_last_row = min(qw + RW, n_q) - 1;

    // Per-lane byte offsets of the LDS operand reads, the same for both
    // buffers and both 32-key halves (32 and 16 rows down keep the
    // swizzle, so those are constants); passed through an empty asm in each
    // tile step so the buffer's base folds into the reads' immediate offsets.
    //  soff[kk]:     K / V row r, k-step kk (A operands of S^T and dP^T);
    //  troff[db][h]: transpose reads of K (A operands of dQ^T), rows
    //                4g + s16/4 + 8h (+ 16c + 32kb), columns of block db.
    int soff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) soff[kk] = 2 * tile_off<D>(r, 16 * kk + 8 * g);
    int troff[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            troff[db][h] = 2 * tile_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * half + 4 * (s16 & 3));
    static_assert(tile_swz<D>(16) == tile_swz<D>(0) && tile_swz<D>(17) == tile_swz<D>(1) &&
                      tile_swz<D>(18) == tile_swz<D>(2) && tile_swz<D>(19) == tile_swz<D>(3),
                  "16 rows down keeps the swizzle");
    auto at = [](const bf16* base, int byte_off) {
        return (const bf16*)((const char*)base + byte_off);
    };

    // Zero dS^T where the key is past n_k or (causal) after the query:
    // element v (key offset 8*(v/4) + v%4 from ks + 32kb + 4g) is masked iff
    // that offset is >= lim. Works on the packed bf16 pairs with bit masks.
    auto apply_mask = [&](int lim, bf16x8* ds) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            auto w = __builtin_bit_cast(uint4, ds[c]);
            unsigned keep[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = 8 * c + 2 * i;   // elements v, v + 1 in word i
                const int off = 8 * (v >> 2) + (v & 3);
                keep[i] = (off >= lim ? 0u : 0x0000ffffu) | (off + 1 >= lim ? 0u : 0xffff0000u);
            }
            w.x &= keep[0]; w.y &= keep[1]; w.z &= keep[2]; w.w &= keep[3];
            ds[c] = __builtin_bit_cast(bf16x8, w);
        }
    };

    auto tile_step = [&](const bf16* Kb, const bf16* Vb, int ks) {
        const bool active = wave_last_row >= qw && (!CAUSAL || ks <= wave_last_row + coff);
        if (!active) return;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(soff[kk]));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(troff[db][h]));
        const bool need_mask = (ks + kBC > n_k) || (CAUSAL && ks + kBC - 1 > qw + coff);
        // Two 32-key halves, one after the other, to keep fewer values live.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int rb = kb * 32 * D * 2;   // byte offset of the half's rows
            mfma_priority(true);
            // S^T = K Q^T and dP^T - D = V dO^T - D (rows = keys, columns =
            // queries); K and V operands are read one k-step ahead.
            f32x16 s = zero_f32x16(), dpt = neg_d;
            bf16x8 ak[2], av[2];
            ak[0] = *(const bf16x8*)at(Kb, soff[0] + rb);
            av[0] = *(const bf16x8*)at(Vb, soff[0] + rb);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (kk + 1 < KK) {
                    ak[(kk + 1) & 1] = *(const bf16x8*)at(Kb, soff[kk + 1] + rb);
                    av[(kk + 1) & 1] = *(const bf16x8*)at(Vb, soff[kk + 1] + rb);
                }
                s = mfma32(ak[kk & 1], qreg[kk], s);
                dpt = mfma32(av[kk & 1], doreg[kk], dpt);
            }
            sched_reads_ahead_of_mfma<KK>();
            mfma_priority(false);
            // key of element v: ks + 32kb + 4g + 8*(v/4) + v%4 (see the forward)
            bf16x8 dsb[2];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(fmaf(s[v], scale2, -l2));
                dsb[v >> 3][v & 7] = to_bf16(p * dpt[v]);
            }
            if (need_mask)
                apply_mask((CAUSAL ? min(n_k, row + 1 + coff) : n_k) - ks - 32 * kb - 4 * g, dsb);
            // dQ^T (d x queries) += K^T dS^T; K^T operands by transpose reads.
            mfma_priority(true);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int cb = rb + c * 16 * D * 2;
                    const bf16x8 a = concat(lds_read_tr(at(Kb, troff[db][0] + cb)),
                                            lds_read_tr(at(Kb, troff[db][1] + cb)));
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

    // Epilogue: dQ = scale * acc (lane (r, g) holds the row of query qw + r),
    // or, under the key split, its fp32 partial at virtual head bhv; each
    // wave stages its 32 rows in one of the (now idle) tile buffers and
    // stores them whole (store_rows_via_lds; 32 * D * 4 bytes fit a buffer).
    copies_barrier();   // every wave is done with the tile buffers
    char* st = (char*)(wave == 0 ? Ks0 : (wave == 1 ? Ks1 : (wave == 2 ? Vs0 : Vs1)));
    auto value = [&](int db, int v) { return acc[db][v] * scale; };
    if (part) store_rows_via_lds<D>(st, part + ((size_t)bhv * n_q + qw) * D, n_q - qw, value);
    else store_rows_via_lds<D>(st, dQ + ((size_t)bh * n_q + qw) * D, n_q - qw, value);
}

// A gradient as the sum of its split partials ([bh, nsplit, n, D] fp32), in
// split order (deterministic), rounded once to bf16 into [bh, n, D]; one
// thread per 4 columns of a row. Used for dQ (key split) and dK, dV (query
// split).
template <int D>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(const float* __restrict__ part,
                                                                bf16* __restrict__ out, long long rows,
                                                                int n, int nsplit) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= rows * (D / 4)) return;
    const long long row = i / (D / 4);
    const int c = (int)(i - row * (D / 4)) * 4;
    const long long bh = row / n;
    const size_t first = ((size_t)bh * nsplit * n + (size_t)(row - bh * n)) * D + c;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s = 0; s < nsplit; ++s) {
        const float4 x = *(const float4*)(part + first + (size_t)s * n * D);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    bf16x4 pk;
    pk[0] = to_bf16(acc.x); pk[1] = to_bf16(acc.y); pk[2] = to_bf16(acc.z); pk[3] = to_bf16(acc.w);
    *(bf16x4*)(out + (size_t)row * D + c) = pk;
}

template <int D>
hipError_t launch_split_reduce(const float* part, void* out, long long rows, int n, int nsplit,
                               hipStream_t st) {
    const long long nb = (rows * (D / 4) + kThreads - 1) / kThreads;
    if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((split_reduce_kernel<D>), dim3((unsigned)nb), dim3(kThreads), 0, st, part,
                       (bf16*)out, rows, n, nsplit);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_kernels(const BwdArgs& a, hipStream_t st) {
    const int n_q_pad = dq_rows_padded(a.n_q);
    const long long rows_pad = (long long)a.bh * n_q_pad;
    constexpr int RPB = kThreads / pre_lanes_per_row(D / 8);   // as in bwd_pre_kernel
    const long long nb = (rows_pad + RPB - 1) / RPB;
    constexpr int NP = dkdv_pairs<D>();
    const int n_ktiles = (a.n_k + 32 * NP - 1) / (32 * NP);
    const int n_qtiles = (a.n_q + 127) / 128;
    const int nsplit = a.dq_part ? a.dq_nsplit : 1;
    const int kv_split = a.kv_part ? a.kv_nsplit : 1;
    if (nb > 0x7fffffffLL || (long long)a.bh * kv_split * n_ktiles > 0x7fffffffLL ||
        (long long)a.bh * nsplit * n_qtiles > 0x7fffffffLL)
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
    float* part_k = kv_split > 1 ? a.kv_part : nullptr;
    float* part_v = kv_split > 1 ? a.kv_part + (size_t)kv_split * a.bh * a.n_k * D : nullptr;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, NP>), dim3((unsigned)((long long)a.bh * kv_split * n_ktiles)),
                       dim3(128 * NP), 0, st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (const bf16*)a.d_o, (const float*)a.l2pad, (const float*)a.drow, (bf16*)a.dk,
                       (bf16*)a.dv, part_k, part_v, a.n_q, a.n_k, a.coff, n_q_pad, n_ktiles, a.scale,
                       a.scale * kLog2e, kv_split, kv_split > 1 ? a.kv_chunk : a.n_q);
    e = hipGetLastError();
    if (e == hipSuccess && kv_split > 1) {
        const long long krows = (long long)a.bh * a.n_k;
        e = launch_split_reduce<D>(part_k, a.dk, krows, a.n_k, kv_split, st);
        if (e == hipSuccess) e = launch_split_reduce<D>(part_v, a.dv, krows, a.n_k, kv_split, st);
    }
    if (e == hipSuccess) e = record_stage(a, 2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((long long)a.bh * nsplit * n_qtiles)),
                       dim3(kThreads), 0, st, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (const bf16*)a.d_o, (const float*)a.l2pad, (const float*)a.drow, (bf16*)a.dq,
                       nsplit > 1 ? a.dq_part : nullptr, a.n_q, a.n_k, a.coff, n_q_pad, n_qtiles,
                       a.scale, a.scale * kLog2e, nsplit, nsplit > 1 ? a.dq_chunk : a.n_k);
    e = hipGetLastError();
    if (e == hipSuccess && nsplit > 1)
        e = launch_split_reduce<D>(a.dq_part, a.dq, (long long)a.bh * a.n_q, a.n_q, nsplit, st);
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

// Key split of the dQ kernel (128-row workgroups, two resident per CU, one
// at d = 256; chunks of whole 64-key tiles) and query split of the dK/dV
// kernel (one workgroup per CU; chunks of 256-row multiples), by the shared
// rule of plan_split.
Split dq_split_plan(long long bh, int n_q, int n_k, int d) {
    const long long slots = (long long)device_cu_count() * (d >= 256 ? 1 : 2);
    return plan_split(bh * ((n_q + 127) / 128), slots, n_k, kBC);
}

size_t dq_part_bytes(const Split& sp, long long bh, int n_q, int d) {
    return sp.nsplit > 1 ? (size_t)sp.nsplit * (size_t)bh * (size_t)n_q * (size_t)d * sizeof(float) : 0;
}

Split kv_split_plan(long long bh, int n_q, int n_k, int d) {
    const int bkv = 32 * (d >= 256 ? 2 : 4);
    return plan_split(bh * ((n_k + bkv - 1) / bkv), device_cu_count(), n_q, 256);
}

size_t kv_part_bytes(const Split& sp, long long bh, int n_k, int d) {
    return sp.nsplit > 1 ? 2 * (size_t)sp.nsplit * (size_t)bh * (size_t)n_k * (size_t)d * sizeof(float) : 0;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 32: return a.causal ? launch_kernels<32, true>(a, st) : launch_kernels<32, false>(a, st);
        case 64: return a.causal ? launch_kernels<64, true>(a, st) : launch_kernels<64, false>(a, st);
        case 96: return a.causal ? launch_kernels<96, true>(a, st) : launch_kernels<96, false>(a, st);
        case 128: return a.causal ? launch_kernels<128, true>(a, st) : launch_kernels<128, false>(a, st);
        case 256: return a.causal ? launch_kernels<256, true>(a, st) : launch_kernels<256, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
