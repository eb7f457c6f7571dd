// Forward attention for bf16 inputs on gfx950, phase-locked "ping-pong"
// form (head dims 64 and 128).
//
// Algorithm: the tiled forward with online softmax of page 1
// ("05_flash_attention.py", section 2, flash_attention_forward), as in
// fa_fwd.hip: per query row a running max m and running sum l over the key
// tiles, the output accumulator rescaled by exp(m_old - m_new), O / l and
// L = m + log(l) at the end; key tiles wholly in the causal future are
// skipped. The recurrence is the one of page 1, section 1 and page 3
// ("Flash Attention"), section 1.1.
//
// MI355X mapping (not from the pages):
//  * one workgroup = 8 waves = 256 query rows of one (batch, head), one
//    workgroup per CU. Waves w and w + 4 run on the same SIMD; they form the
//    two groups G = w / 4, whose rows are adjacent 32-row blocks.
//  * every key tile (64 keys) is processed in two half-steps separated by
//    workgroup barriers. In each half-step one group issues only matrix
//    work (O += V P for the previous tile and S = K Q^T for this one, raised
//    issue priority) while the other group does only the softmax of its
//    scores and the tile copies, so on every SIMD one wave keeps the matrix
//    core busy while the other's VALU work fills the issue slots between
//    its MFMAs; then the groups swap.
//  * K and V tiles go global -> LDS without registers through a ring of four
//    stages. The group in its matrix half-step copies tile t + 2 (group 0
//    the K tile, group 1 the V tile), one chunk every few MFMAs, so the
//    copies use issue slots the matrix stream leaves free and have two
//    steps to land; the tile read path carries half the bytes of two
//    independent 128-row workgroups per CU.
//  * scores in the exp2 domain, the PV operand is P rounded to bf16 (RNE);
//    l sums the fp32 probabilities (for L), and O is divided by the sum of
//    the bf16 values the PV product applied, so the rounding of a dominant
//    weight cancels between numerator and denominator (with the reference
//    max up to 2^8 below the row max, that weight's rounding reaches 2^-8
//    and would show in O at 1e-2 on peaked rows). The VALU is the scarce unit here (while
//    the other wave streams MFMAs it issues at about half rate), so a tile
//    first takes its exponentials against the current reference max without
//    computing its own max; only when that lets a value exceed 2^8 (or on
//    the first tile) does it compute the true max, rescale O and l and redo
//    the exponentials. Exact either way: O and l share the reference.
#include <atomic>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kPPThreads = 512;
constexpr int kPPRows = 256;   // query rows per workgroup
constexpr int kPPBC = 64;      // keys per tile

// s_waitcnt immediate for gfx9: vmcnt(vm), expcnt(7), lgkmcnt(lgkm).
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Key split (nsplit > 1): the grid holds nsplit "virtual heads" per head;
// virtual head bhv = bh * nsplit + s attends head bh's queries to keys
// [s * kchunk, (s + 1) * kchunk) only and writes its partial result at bhv:
// O (fp32, normalised over those keys), L from the fp32 probability sum and,
// in Lb, the same logsumexp taken over the bf16 weights the PV product
// applied (what the merge weights O by; see fwd_merge_kernel).
template <int D, bool CAUSAL, bool OF32>
__global__ __launch_bounds__(kPPThreads, 1) void fwd_pp_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ Lse, float* __restrict__ Lb,
    int n_q, int n_k_all, int coff, int n_qtiles, float scale2, int nsplit, int kchunk) {
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int KK = D / 16;            // MFMA k-steps over d
    constexpr int NDB = D / 32;           // 32-wide d blocks of the output
    constexpr int TILE = kPPBC * D;       // elements per K or V tile
    constexpr int CPT = TILE * 2 / 1024;  // 1 KB copies per tile and tensor
    constexpr int CPW = CPT / 4;          // ... per wave of one group
    static_assert(CPW * 4 == CPT && CPT % 8 == 0, "whole copies per wave");

    // Ring of four K and four V stages, one LDS object each so the compiler
    // can tell the stage being filled from the ones being read.
    __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Ks2[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Ks3[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs2[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs3[TILE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;
    const int grp = wave >> 2, sub = wave & 3;

    int bhv, rank;   // rank 0 = last query tile: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_qtiles, n_qtiles, &bhv, &rank);
    const int qt = n_qtiles - 1 - rank;
    const int q0 = qt * kPPRows;
    const int qw = q0 + 32 * (2 * sub + grp);   // this wave's first row
    // this workgroup's keys: [k_lo, k_lo + n_k) of head bh, with the causal
    // diagonal moved to those local key indices
    const int bh = bhv / nsplit;
    const int k_lo = (bhv - bh * nsplit) * kchunk;
    const int n_k = max(0, min(n_k_all, k_lo + kchunk) - k_lo);
    coff -= k_lo;

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* Kh = K + ((size_t)bh * n_k_all + k_lo) * D;
    const bf16* Vh = V + ((size_t)bh * n_k_all + k_lo) * D;

    // Q rows as MFMA B operands: lane (r, g) holds d = 16*kk + 8*g .. +7.
    bf16x8 qreg[KK];
    {
        const int row = qw + r;
        const int rc = min(row, n_q - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 x = *(const bf16x8*)(Qh + (size_t)rc * D + 16 * kk + 8 * g);
            qreg[kk] = row < n_q ? x : zero_bf16x8();
        }
    }

    // Keys the workgroup needs and the keys this wave needs (causal: keys
    // <= last row + coff).
    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + kPPRows, n_q) + coff));
    const int ntiles = (kend + kPPBC - 1) / kPPBC;
    const int wave_last_row = min(qw + 32, n_q) - 1;   // < qw when the wave has no rows
    int wend = wave_last_row >= qw ? n_k : 0;
    if (CAUSAL) wend = max(0, min(wend, wave_last_row + 1 + coff));
    const int wtiles = (wend + kPPBC - 1) / kPPBC;     // tiles 0 .. wtiles-1 are active

    // Tile copies (rows past n_k read as zeros through the buffer bounds).
    // Byte offsets are unsigned: (n_k + 63) * D * 2 < 2^32.
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh, n_k * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vh, n_k * D * 2);
    // Chunk b (1 KB) of the tile of keys ks.. into LDS tile dst. With
    // valid == false the offset lies past the end of any tensor (the host
    // keeps n_k * D * 2 < 2^31), so the load fetches nothing and writes zeros.
    auto copy_chunk = [&](__amdgpu_buffer_rsrc_t rs, bf16* dst, int ks, int b, bool valid) __attribute__((always_inline)) {
        const int p = 64 * b + lane;
        const int row = p / (D / 8), pc = p % (D / 8);
        const unsigned boff = ((unsigned)(ks + row) * D + 8u * (unsigned)(pc ^ tile_swz<D>(row))) * 2u;
        load_lds16(rs, valid ? boff : 0x80000000u, dst + 512 * b);
    };
    // The same copy during the loop, where this wave always copies chunks
    // 4c + sub: the lane's part of the offset is computed once (cpart[c]),
    // and the tile's part is a wave-uniform base, 0x80000000 for an invalid
    // copy, so each chunk costs one vector add.
    unsigned cpart[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int p = 64 * (4 * c + sub) + lane;
        const int row = p / (D / 8), pc = p % (D / 8);
        cpart[c] = ((unsigned)row * D + 8u * (unsigned)(pc ^ tile_swz<D>(row))) * 2u;
    }
    auto copy_share = [&](__amdgpu_buffer_rsrc_t rs, bf16* dst, int ks, int c, bool valid) __attribute__((always_inline)) {
        const unsigned base = valid ? (unsigned)ks * D * 2u : 0x80000000u;
        load_lds16(rs, base + cpart[c], dst + 512 * (4 * c + sub));
    };
    // One tensor tile copied by all eight waves.
    auto copy_by_all = [&](__amdgpu_buffer_rsrc_t rs, bf16* dst, int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < CPT / 8; ++i) copy_chunk(rs, dst, ks, 8 * i + wave, true);
    };

    // Per-lane LDS byte offsets (see fa_fwd.hip): K rows r (+32 for the second
    // 32-key block), V transpose reads rows 4g + s16/4 + 8h (+16c).
    // A read's immediate offset reaches 64 KB past its address register. At
    // d = 128 the eight stages take 128 KB and the V stages lie past the
    // first 64 KB, so the V offsets carry a bias of 64 KB that each read
    // takes off again: the stage's address minus the bias then fits the
    // immediate, instead of costing an add per read. (Any placement of the
    // stages stays correct; only the folding depends on it.)
    constexpr int kVBias = 8 * TILE * 2 > 65536 ? 4 * TILE * 2 : 0;
    int soff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) soff[kk] = 2 * tile_off<D>(r, 16 * kk + 8 * g);
    int troff[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            troff[db][h] = 2 * tile_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * half + 4 * (s16 & 3)) + kVBias;
    auto launder = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(soff[kk]));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(troff[db][h]));
    };
    auto at = [](const bf16* base, int byte_off) __attribute__((always_inline)) {
        return (const bf16*)((const char*)base + byte_off);
    };

    // l_run: sum of the fp32 probabilities (for L); lb_run: sum of their
    // bf16 roundings, the weights the PV product actually applied (for O).
    float m_ref = kNegInf, l_run = 0.0f, lb_run = 0.0f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero_f32x16();
    f32x16 s[2];
    s[0] = s[1] = zero_f32x16();
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pb[c] = zero_bf16x8();

    // Matrix half-step: O^T += V^T P^T of the previous tile (V stage Vb) and
    // S^T = K Q^T of this tile (K stage Kb). The two products alternate MFMA
    // by MFMA (independent accumulators); operands are read kLook MFMAs
    // ahead. The wave's share of one tile copy (CPW chunks of tensor crs into
    // stage cdst, keys from cks) is spread over the stream, one chunk every
    // NT / CPW MFMAs; when !cvalid the chunks point past the tensor's end,
    // so they fetch nothing and write zeros into a stage nobody reads again.
    auto mfma_phase = [&](const bf16* Kb, const bf16* Vb, __amdgpu_buffer_rsrc_t crs, bf16* cdst,
                          int cks, bool cvalid) __attribute__((always_inline)) {
        constexpr int NSM = 2 * KK;     // S MFMAs
        constexpr int NPV = 4 * NDB;    // PV MFMAs
        constexpr int NT = NSM + NPV;
        // Slot i: S (kind 0) and PV (kind 1) alternate while both remain;
        // index = position within its own kind.
        constexpr int MBOTH = NSM < NPV ? NSM : NPV;
        auto kind = [](int i) __attribute__((always_inline)) -> int {
            if (i < 2 * MBOTH) return i & 1;
            return NSM > NPV ? 0 : 1;
        };
        auto index = [](int i) __attribute__((always_inline)) -> int {
            return i < 2 * MBOTH ? i >> 1 : i - MBOTH;
        };
        // copy chunk c goes after the MFMA of slot copy_slot(c)
        auto copy_slot = [](int c) __attribute__((always_inline)) -> int {
            return c * (NT / CPW) + NT / (2 * CPW);
        };
        launder();
        constexpr int kLook = 3;
        bf16x8 op[kLook + 1];
        auto load = [&](int i) __attribute__((always_inline)) {
            const int j = index(i);
            if (kind(i) == 0) {
                const int kb = j / KK, kk = j % KK;
                op[i % (kLook + 1)] = *(const bf16x8*)at(Kb, soff[kk] + kb * 32 * D * 2);
            } else {
                const int c = j / NDB, db = j % NDB;
                const int cb = c * 16 * D * 2 - kVBias;
                op[i % (kLook + 1)] = concat(lds_read_tr(at(Vb, troff[db][0] + cb)),
                                             lds_read_tr(at(Vb, troff[db][1] + cb)));
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        mfma_priority(true);
#pragma unroll
        for (int i = 0; i < kLook; ++i) load(i);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            if (i + kLook < NT) load(i + kLook);
            const int j = index(i);
            if (kind(i) == 0) {
                const int kb = j / KK, kk = j % KK;
                // the first k-step starts from zero (an inline constant)
                s[kb] = mfma32(op[i % (kLook + 1)], qreg[kk], kk == 0 ? zero_f32x16() : s[kb]);
            } else {
                const int c = j / NDB, db = j % NDB;
                o[db] = mfma32(op[i % (kLook + 1)], pb[c], o[db]);
            }
#pragma unroll
            for (int c = 0; c < CPW; ++c)
                if (i == copy_slot(c)) copy_share(crs, cdst, cks, c, cvalid);
        }
        // Pin the order: the reads of slot i + kLook and any copy chunk
        // follow the MFMA of slot i (one ds_read_b128 for a K operand, two
        // transpose reads for a V operand).
        auto pin_reads = [&](int i) __attribute__((always_inline)) {
            if (kind(i) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        };
#pragma unroll
        for (int i = 0; i < kLook; ++i) pin_reads(i);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
            for (int c = 0; c < CPW; ++c)
                if (i == copy_slot(c)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (i + kLook < NT) pin_reads(i + kLook);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_priority(false);
    };

    // Softmax half-step on this wave's scores of tile t (keys ks ..): P
    // and the running statistics.
    // P (bf16, the B operands of the next PV product) of the lane's 32
    // scores against reference max m_use; returns their fp32 sum (four
    // independent chains: one serial chain leaves the VALU waiting).
    auto exp_tile = [&](float m_use) __attribute__((always_inline)) -> float {
        float rq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = fast_exp2(fmaf(s[kb][v], scale2, -m_use));
                rq[v & 3] += p;
                pb[2 * kb + (v >> 3)][v & 7] = to_bf16(p);
            }
        return (rq[0] + rq[1]) + (rq[2] + rq[3]);
    };
    // Move the reference max to the row's true running max and rescale O and
    // l by exp2(m_old - m_new) where it grew.
    auto rebase = [&]() __attribute__((always_inline)) {
        float mq[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mq[v & 3] = fmaxf(mq[v & 3], s[kb][v]);
        const float mx = halves_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * scale2;
        if (__any(mx > m_ref)) {
            const float m_new = fmaxf(m_ref, mx);
            const float corr = fast_exp2(m_ref - (m_new == kNegInf ? 0.0f : m_new));
            l_run *= corr;
            lb_run *= corr;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[db][v] *= corr;
            m_ref = m_new;
        }
    };
    auto softmax_phase = [&](int ks) __attribute__((always_inline)) {
        const bool need_mask = (ks + kPPBC > n_k) || (CAUSAL && ks + kPPBC - 1 > qw + coff);
        if (need_mask) {
            const int lim = (CAUSAL ? min(n_k, qw + r + 1 + coff) : n_k) - ks - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * kb + 8 * (v >> 2) + (v & 3) >= lim) s[kb][v] = kNegInf;
        }
        // Speculative pass: exponentials against the current reference max
        // m_ref without computing this tile's max. The lane's 32 values
        // sum to at most 256 unless one of them exceeds 8 (its score is
        // over m_ref + 3), and every value is at most 256 (2^8 above m_ref)
        // when the sum is; so a sum <= 256 in every lane keeps the
        // accumulation exactly as safe as a rescale at 2^8 would. Otherwise
        // (or on the first tile, m_ref = -inf) the tile takes the full
        // pass: true row max, rescale of O and l, exponentials again.
        float rs = 0.0f;
        bool full = __any(m_ref == kNegInf);
        if (!full) {
            rs = exp_tile(m_ref);
            full = __any(!(rs <= 256.0f));
        }
        if (full) {
            rebase();
            rs = exp_tile(m_ref == kNegInf ? 0.0f : m_ref);
        }
        l_run += rs;
        // (two chains for the bf16 sum of the P operands)
        lb_run += sum_bf16x8(pb[0], sum_bf16x8(pb[1], 0.0f)) + sum_bf16x8(pb[2], sum_bf16x8(pb[3], 0.0f));
    };

    auto mid_barrier = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
    // End of a step: the wave's copies from earlier steps have landed, then
    // the barrier makes every wave's copies visible. A wave issues its CPW
    // copies of tile t + 2 in step t (or none, past its own work when there
    // is no tile t + 2): vmcnt(CPW) leaves just this step's copies in flight;
    // after a step without copies everything is waited for.
    auto step_barrier = [&](bool issued) __attribute__((always_inline)) {
        if (issued) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(CPW, 0));
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(CPW) : "memory");
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };

    // Prologue: tiles 0 and 1 by all waves. Step 0's matrix half-step runs
    // O += V P on V stage 3 with P = 0 before any tile has landed there, and
    // LDS keeps whatever an earlier workgroup left (an fp32 +inf from the
    // backward's padded rows reads as a bf16 +inf): 0 times Inf or NaN would
    // make O NaN, so stage 3 starts as zeros.
    {
        constexpr int N16 = TILE * 2 / 16;   // 16-byte words of a stage
#pragma unroll
        for (int i = 0; i < (N16 + kPPThreads - 1) / kPPThreads; ++i) {
            const int w = i * kPPThreads + tid;
            if (w < N16) *(bf16x8*)(Vs3 + 8 * w) = zero_bf16x8();
        }
    }
    copy_by_all(krs, Ks0, 0);
    copy_by_all(vrs, Vs0, 0);
    if (ntiles > 1) {
        copy_by_all(krs, Ks1, kPPBC);
        copy_by_all(vrs, Vs1, kPPBC);
    }
    copies_barrier();

    // Step t (t = 0 .. ntiles): tile t is in stage t % 4, the previous tile
    // in stage (t - 1) % 4, and tile t + 2 goes to stage (t + 2) % 4. Each
    // group runs its own loop with the same barriers: group 0 does its matrix
    // work (and the K copy) in the first half-step and its softmax in the
    // second, group 1 the other way round (softmax of the previous tile
    // first, then its matrix work and the V copy).
    // The matrix half-step always runs both products, so the accumulators
    // keep their registers on every path: at t = 0 the P operands are still
    // zero (O += V 0), and at t = wtiles the scores are computed but unused.
    // Past t = wtiles the wave has nothing left to do.
    // Its copy share (tile t + 2: K by group 0, V by group 1) is issued also
    // when the products are not, so every wave's copies stay in step.
    // Returns whether this step issued copies (see step_barrier).
    auto matrix = [&](const bf16* Kc, const bf16* Vp, __amdgpu_buffer_rsrc_t crs, bf16* cdst, int t)
                      __attribute__((always_inline)) -> bool {
        const bool cvalid = t + 2 < ntiles;
        if (t <= wtiles) mfma_phase(Kc, Vp, crs, cdst, (t + 2) * kPPBC, cvalid);
        // (two separate branches: an if/else here makes the compiler move the
        // accumulators through a second register set)
        if (t > wtiles && cvalid) {
#pragma unroll
            for (int c = 0; c < CPW; ++c) copy_share(crs, cdst, (t + 2) * kPPBC, c, true);
        }
        return t <= wtiles || cvalid;
    };
    if (grp == 0) {
        auto step = [&](const bf16* Kc, const bf16* Vp, bf16* Kn, int t) __attribute__((always_inline)) {
            const bool issued = matrix(Kc, Vp, krs, Kn, t);
            mid_barrier();
            if (t < wtiles) softmax_phase(t * kPPBC);
            step_barrier(issued);
        };
        // Unrolled by four so every step names its stages at compile time;
        // one loop exit keeps the accumulators in place.
        for (int t = 0; t <= ntiles; t += 4) {
            step(Ks0, Vs3, Ks2, t);
            if (t + 1 > ntiles) break;
            step(Ks1, Vs0, Ks3, t + 1);
            if (t + 2 > ntiles) break;
            step(Ks2, Vs1, Ks0, t + 2);
            if (t + 3 > ntiles) break;
            step(Ks3, Vs2, Ks1, t + 3);
        }
    } else {
        auto step = [&](const bf16* Kc, const bf16* Vp, bf16* Vn, int t) __attribute__((always_inline)) {
            if (t >= 1 && t - 1 < wtiles) softmax_phase((t - 1) * kPPBC);
            mid_barrier();
            const bool issued = matrix(Kc, Vp, vrs, Vn, t);
            step_barrier(issued);
        };
        for (int t = 0; t <= ntiles; t += 4) {
            step(Ks0, Vs3, Vs2, t);
            if (t + 1 > ntiles) break;
            step(Ks1, Vs0, Vs3, t + 1);
            if (t + 2 > ntiles) break;
            step(Ks2, Vs1, Vs0, t + 2);
            if (t + 3 > ntiles) break;
            step(Ks3, Vs2, Vs1, t + 3);
        }
    }

    // Epilogue: O / l, L = ln 2 * (m + log2 l); a row that saw no key gets
    // O = 0, L = -inf. Lane (r, g) holds the row of query qw + r; each wave
    // stages its 32 rows of O in one of the eight (now idle) ring stages and
    // stores them whole (store_rows_via_lds). The barrier also waits for the
    // zero-filling copies the last step may still have in flight into the
    // stages.
    static_assert(32 * D * 4 <= TILE * 2, "a wave's fp32 rows fit one stage");
    const float l = halves_sum(l_run), lb = halves_sum(lb_run);
    const int row = qw + r;
    const float inv = lb > 0.0f ? 1.0f / lb : 0.0f;
    copies_barrier();
    bf16* stg = wave < 4 ? (wave < 2 ? (wave == 0 ? Ks0 : Ks1) : (wave == 2 ? Ks2 : Ks3))
                         : (wave < 6 ? (wave == 4 ? Vs0 : Vs1) : (wave == 6 ? Vs2 : Vs3));
    char* st = (char*)stg;
    auto value = [&](int db, int v) { return o[db][v] * inv; };
    if (OF32) store_rows_via_lds<D>(st, (float*)Out + ((size_t)bhv * n_q + qw) * D, n_q - qw, value);
    else store_rows_via_lds<D>(st, (bf16*)Out + ((size_t)bhv * n_q + qw) * D, n_q - qw, value);
    if (row < n_q && g == 0) {
        Lse[(size_t)bhv * n_q + row] = kLn2 * (m_ref + fast_log2(l));
        if (Lb) Lb[(size_t)bhv * n_q + row] = kLn2 * (m_ref + fast_log2(lb));
    }
}

// Merge of the key-split partials of one row (one wave per row, four rows
// per workgroup): with the partial logsumexps L_s (fp32 probability sums)
// and B_s (bf16 weight sums), L = log sum_s exp(L_s) and
// O = sum_s exp(B_s - B) O_s, B = log sum_s exp(B_s) (the online-softmax
// merge of page 1, section 2, applied across workgroups instead of key
// tiles). Weighting by the bf16 sums keeps O the quotient of the bf16-weighted
// sum of V rows by the sum of those weights, as without the split. A row
// with no visible key in any split gets O = 0, L = -inf.
template <int D, bool OF32>
__global__ __launch_bounds__(256) void fwd_merge_kernel(
    const float* __restrict__ po, const float* __restrict__ pl, const float* __restrict__ plb,
    void* __restrict__ Out, float* __restrict__ Lse, long long rows, int n_q, int nsplit) {
    constexpr int PL = D / 64;   // values per lane
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const long long bh = row / n_q;
    const int r = (int)(row - bh * n_q);
    const size_t first = (size_t)bh * nsplit * n_q + r;   // split s at first + s * n_q
    float ml = kNegInf, mb = kNegInf;
    for (int s = 0; s < nsplit; ++s) {
        ml = fmaxf(ml, pl[first + (size_t)s * n_q]);
        mb = fmaxf(mb, plb[first + (size_t)s * n_q]);
    }
    float sl = 0.0f, sb = 0.0f;
    if (mb != kNegInf) {
        for (int s = 0; s < nsplit; ++s) {
            sl += fast_exp2((pl[first + (size_t)s * n_q] - ml) * kLog2e);
            sb += fast_exp2((plb[first + (size_t)s * n_q] - mb) * kLog2e);
        }
    }
    float acc[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) acc[i] = 0.0f;
    if (mb != kNegInf) {
        const float b = mb + kLn2 * fast_log2(sb);
        for (int s = 0; s < nsplit; ++s) {
            const float w = fast_exp2((plb[first + (size_t)s * n_q] - b) * kLog2e);
            const float* o = po + (first + (size_t)s * n_q) * D;
#pragma unroll
            for (int i = 0; i < PL; ++i) acc[i] = fmaf(w, o[64 * i + lane], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        if (OF32) ((float*)Out)[(size_t)row * D + 64 * i + lane] = acc[i];
        else ((bf16*)Out)[(size_t)row * D + 64 * i + lane] = to_bf16(acc[i]);
    }
    if (lane == 0) Lse[row] = mb != kNegInf ? ml + kLn2 * fast_log2(sl) : kNegInf;
}

template <int D, bool CAUSAL, bool OF32>
hipError_t launch_pp(const FwdArgs& a, hipStream_t st) {
    const int n_qtiles = (a.n_q + kPPRows - 1) / kPPRows;
    const long long nwg = (long long)a.bh * n_qtiles;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, OF32>), dim3((unsigned)nwg), dim3(kPPThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.o, a.lse, (float*)nullptr,
                       a.n_q, a.n_k, a.coff, n_qtiles, a.scale * kLog2e, 1, a.n_k);
    return hipGetLastError();
}

// Key-split forward: partials of every split into the workspace (fp32 O,
// then L, then the bf16-weight logsumexp), then the merge into O and L.
template <int D, bool CAUSAL, bool OF32>
hipError_t launch_pp_split(const FwdArgs& a, const Split& sp, float* ws, hipStream_t st) {
    const int n_qtiles = (a.n_q + kPPRows - 1) / kPPRows;
    const long long nwg = (long long)a.bh * sp.nsplit * n_qtiles;
    const long long rows = (long long)a.bh * a.n_q;
    if (nwg > 0x7fffffffLL || (rows + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidValue;
    float* po = ws;
    float* pl = po + (size_t)sp.nsplit * rows * D;
    float* plb = pl + (size_t)sp.nsplit * rows;
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, true>), dim3((unsigned)nwg), dim3(kPPThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (void*)po, pl, plb,
                       a.n_q, a.n_k, a.coff, n_qtiles, a.scale * kLog2e, sp.nsplit, sp.chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_merge_kernel<D, OF32>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const float*)po, (const float*)pl, (const float*)plb, a.o, a.lse, rows, a.n_q,
                       sp.nsplit);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_pp(const FwdArgs& a, hipStream_t st) {
    if (a.causal)
        return a.o_f32 ? launch_pp<D, true, true>(a, st) : launch_pp<D, true, false>(a, st);
    return a.o_f32 ? launch_pp<D, false, true>(a, st) : launch_pp<D, false, false>(a, st);
}

template <int D>
hipError_t dispatch_pp_split(const FwdArgs& a, const Split& sp, float* ws, hipStream_t st) {
    if (a.causal)
        return a.o_f32 ? launch_pp_split<D, true, true>(a, sp, ws, st)
                       : launch_pp_split<D, true, false>(a, sp, ws, st);
    return a.o_f32 ? launch_pp_split<D, false, true>(a, sp, ws, st)
                   : launch_pp_split<D, false, false>(a, sp, ws, st);
}

}  // namespace

int device_cu_count() {
    // zero until first asked for on that device; threads that race on the
    // first call store the same value
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int q = 0;
        if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && q > 0) {
            cus[dev].store(q, std::memory_order_relaxed);
            n = q;
        }
    }
    return n;
}

// One 256-row workgroup per CU: used when its workgroups fill the CUs in
// whole rounds or come in enough rounds that the last one matters little
// (else the 128-row kernel, two workgroups per CU, balances better).
bool fwd_pp_supports(const FwdArgs& a) {
    if (a.d != 128 && a.d != 64) return false;
    return fills_cus((long long)a.bh * ((a.n_q + kPPRows - 1) / kPPRows));
}

hipError_t launch_fwd_pp(const FwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 64: return dispatch_pp<64>(a, st);
        case 128: return dispatch_pp<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// Key split for grids that leave most CUs idle (one 256-row workgroup per
// CU; chunks of whole 64-key tiles), by the shared rule of plan_split.
// Measured: one head of 4096 (16 workgroups) 1.8x faster split; the
// cross-attention workload (384 workgroups, 3000 keys) 1.5x slower split in
// two, and one head of 1024 keys slower too (the merge and the partials
// cost more than the idle CUs): those stay unsplit. Head dims 64 and 128
// only.
Split fwd_split_plan(const FwdArgs& a) {
    if (a.d != 128 && a.d != 64) return Split{1, a.n_k};
    return plan_split((long long)a.bh * ((a.n_q + kPPRows - 1) / kPPRows), device_cu_count(), a.n_k, kPPBC);
}

size_t fwd_split_workspace_bytes(const FwdArgs& a, const Split& sp) {
    if (sp.nsplit <= 1) return 0;
    const size_t rows = (size_t)a.bh * (size_t)a.n_q * (size_t)sp.nsplit;
    return rows * ((size_t)a.d + 2) * sizeof(float);
}

hipError_t launch_fwd_split(const FwdArgs& a, const Split& sp, float* ws, hipStream_t st) {
    switch (a.d) {
        case 64: return dispatch_pp_split<64>(a, sp, ws, st);
        case 128: return dispatch_pp_split<128>(a, sp, ws, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
