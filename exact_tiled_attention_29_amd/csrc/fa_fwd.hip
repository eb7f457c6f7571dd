// Forward attention kernel for bf16 inputs on gfx950 (MFMA 32x32x16 bf16).
//
// Algorithm: the tiled forward with online softmax of page 1
// ("05_flash_attention.py", section 2, flash_attention_forward): per query
// tile, walk the key tiles left to right keeping a running max m and running
// sum l per row; rescale the output accumulator by exp(m_old - m_new); finish
// with O / l and L = m + log(l). Key tiles that lie wholly in the causal
// future are skipped (same section). The causal diagonal is a runtime offset
// coff (key j visible to query i iff j <= i + coff): 0 is the pages' top-left
// mask, n_k - n_q the bottom-right one, under which a query may see no key
// at all; such a row gets O = 0 and L = -inf. The running-statistics recurrence is
// the one of page 1, section 1 and page 3 ("Flash Attention"), section 1.1.
//
// MI355X mapping (not from the pages):
//  * one workgroup = 4 waves = 128 query rows of one (batch, head), two
//    workgroups per CU (one at d = 256, where the wave needs more than 256
//    registers and the K/V buffers take 128 KB of LDS); each wave owns 32 rows and keeps its Q rows in
//    registers as the B operand of S^T = K Q^T, so every per-row quantity
//    (m, l, the O accumulator column) lives in one lane pair (l, l^32);
//  * K and V tiles (64 keys, row-major, swizzled 16-byte chunks) are copied
//    global -> LDS without registers and double-buffered; the V^T operand of
//    O^T += V^T P^T comes from transpose reads of the row-major V tile;
//  * scores are kept in the exp2 domain (scale * log2 e folded in), the
//    row max needs one cross-lane step (v_permlane32_swap), l sums the fp32
//    probabilities (for L) and only the PV operand is rounded to bf16 (RNE);
//    O is divided by the sum of those bf16 weights, so the rounding of a
//    dominant weight cancels between O and its divisor; O and both sums are
//    rescaled only when a row max grows by more than 2^8 (exact: they share
//    the reference max, and the quotients do not depend on it);
//  * workgroups are renumbered so each XCD works through whole heads
//    (K/V reuse in that XCD's L2), longest causal tiles first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBC = 64;  // keys per tile

template <int D, bool CAUSAL, bool OF32>
__global__ __launch_bounds__(kThreads, D >= 256 ? 1 : 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ Lse,
    int n_q, int n_k, int coff, int n_qtiles, float scale2) {
    constexpr int RW = 32;               // query rows per wave
    constexpr int BR = 4 * RW;           // query rows per workgroup
    constexpr int KK = D / 16;           // MFMA k-steps over d
    constexpr int NDB = D / 32;          // 32-wide d blocks of the output
    constexpr int TILE = kBC * D;        // elements per K or V tile
    constexpr int LPW = TILE * 2 / 1024 / 4;  // 1 KB direct loads per wave per tile
    constexpr float kTau = 8.0f;         // rescale O only when the max grows by > 2^kTau

    // One LDS object per buffer, so the compiler can tell the tile being
    // read from the one being filled and need not wait for the copies.
    __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs0[TILE];
    __shared__ __attribute__((aligned(16))) bf16 Vs1[TILE];

    static_assert(32 * D * 4 <= TILE * 2, "a wave's fp32 rows fit one tile buffer");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, half = (lane >> 4) & 1;

    int bh, rank;   // rank 0 = last query tile: longest causal work first
    work_item(blockIdx.x, gridDim.x / n_qtiles, n_qtiles, &bh, &rank);
    const int qt = n_qtiles - 1 - rank;
    const int q0 = qt * BR;
    const int qw = q0 + wave * RW;

    const bf16* Qh = Q + (size_t)bh * n_q * D;
    const bf16* Kh = K + (size_t)bh * n_k * D;
    const bf16* Vh = V + (size_t)bh * n_k * D;

    // Q rows as MFMA B operands: lane (r, g) holds d = 16*kk + 8*g .. +7.
    bf16x8 qreg[KK];
    {
        const int row = qw + r;
        const int rc = min(row, n_q - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 x = *(const bf16x8*)(Qh + rc * D + 16 * kk + 8 * g);
            qreg[kk] = row < n_q ? x : zero_bf16x8();
        }
    }

    int kend = n_k;
    if (CAUSAL) kend = max(0, min(n_k, min(q0 + BR, n_q) + coff));  // keys <= last row + coff
    const int ntiles = (kend + kBC - 1) / kBC;

    // K and V tiles go straight from global memory to LDS (no registers),
    // row-major with swizzled 16-byte chunks. Each wave copies LPW blocks of
    // 1 KB: lane l of block b fills chunk position 64*b + l. Rows past n_k
    // fall outside the buffer resource and read as zeros (those keys are
    // masked).
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kh, n_k * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vh, n_k * D * 2);
    auto issue_tile = [&](bf16* Kd, bf16* Vd, int ks) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int b = 4 * i + wave;
            const int p = 64 * b + lane;
            const int row = p / (D / 8), pc = p % (D / 8);
            const int chunk = pc ^ tile_swz<D>(row);
            // unsigned: (n_k rounded up to the tile) * D * 2 may pass 2^31 - 1
            const unsigned boff = ((unsigned)(ks + row) * D + 8u * (unsigned)chunk) * 2u;
            load_lds16(krs, boff, Kd + 512 * b);
            load_lds16(vrs, boff, Vd + 512 * b);
        }
    };

    // l_run: sum of the fp32 probabilities (for L); lb_run: sum of their
    // bf16 roundings, the weights the PV product actually applied (for O),
    // so the rounding of a dominant weight cancels in O / lb.
    float m_ref = kNegInf, l_run = 0.0f, lb_run = 0.0f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero_f32x16();

    const int wave_last_row = min(qw + RW, n_q) - 1;  // < qw when the wave has no rows

    // Per-lane byte offsets of the LDS operand reads, the same for both
    // buffers; 32 and 16 rows down keep the swizzle, so the second 32-key
    // block and the 16-key groups of the PV product are immediates. Passed
    // through an empty asm in each tile step so the buffer's base folds into
    // the reads' immediate offsets (otherwise every buffer/offset pair is
    // hoisted out of the loop into a register of its own).
    //  soff[kk]:     K row r, k-step kk (A operands of S^T);
    //  troff[db][h]: transpose reads of V (A operands of O^T), rows
    //                4g + s16/4 + 8h (+ 16c), columns of block db.
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

    // Compute on one staged tile (K rows in Kb, V rows in Vb).
    auto tile_step = [&](const bf16* Kb, const bf16* Vb, int ks) {
        const bool active = wave_last_row >= qw && (!CAUSAL || ks <= wave_last_row + coff);
        if (active) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(soff[kk]));
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(troff[db][h]));
            // S^T (keys x queries) for two 32-key blocks. K operands are read
            // kLook k-steps ahead of their MFMAs (order pinned below: the
            // scheduler would otherwise move each read next to its MFMA).
            constexpr int kLook = 2;
            f32x16 s[2];
            s[0] = s[1] = zero_f32x16();
            bf16x8 ka[kLook + 1][2];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < kLook; ++kk)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    ka[kk][kb] = *(const bf16x8*)at(Kb, soff[kk] + kb * 32 * D * 2);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (kk + kLook < KK) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        ka[(kk + kLook) % (kLook + 1)][kb] =
                            *(const bf16x8*)at(Kb, soff[kk + kLook] + kb * 32 * D * 2);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(ka[kk % (kLook + 1)][kb], qreg[kk], s[kb]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLook, 0);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if (kk + kLook < KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // Mask keys past n_k and (causal) keys after the query: the key of
            // element v is ks + 32*kb + 4g + 8*(v/4) + v%4, so one compare of a
            // constant against a per-lane limit decides it.
            const bool need_mask = (ks + kBC > n_k) || (CAUSAL && ks + kBC - 1 > qw + coff);
            if (need_mask) {
                const int lim = (CAUSAL ? min(n_k, qw + r + 1 + coff) : n_k) - ks - 4 * g;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (32 * kb + 8 * (v >> 2) + (v & 3) >= lim) s[kb][v] = kNegInf;
            }
            // Online softmax in the exp2 domain against a reference max m_ref
            // that only moves when the row max exceeds it by more than 2^kTau;
            // O and l are rescaled only then (a wave-wide decision).
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
            mx = halves_max(mx) * scale2;
            if (__any(mx > m_ref + kTau)) {
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
            const float m_use = m_ref == kNegInf ? 0.0f : m_ref;
            bf16x8 pb[4];
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = fast_exp2(fmaf(s[kb][v], scale2, -m_use));
                    rs += p;
                    pb[2 * kb + (v >> 3)][v & 7] = to_bf16(p);
                }
            l_run += rs;
            lb_run += sum_bf16x8(pb[0], sum_bf16x8(pb[1], 0.0f)) + sum_bf16x8(pb[2], sum_bf16x8(pb[3], 0.0f));
            // O^T (d x queries) += V^T P^T; V^T operands by transpose reads.
            // Raised issue priority for these MFMAs, so they go first and the
            // other wave's softmax fills the gaps (around the S^T MFMAs a
            // raised priority was slower).
            mfma_priority(true);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int cb = c * 16 * D * 2;
                    const bf16x8 a = concat(lds_read_tr(at(Vb, troff[db][0] + cb)),
                                            lds_read_tr(at(Vb, troff[db][1] + cb)));
                    o[db] = mfma32(a, pb[c], o[db]);
                }
            }
            mfma_priority(false);
        }
    };

    issue_tile(Ks0, Vs0, 0);
    copies_barrier();
    // Unrolled by two so each step names its buffers at compile time.
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) issue_tile(Ks1, Vs1, (t + 1) * kBC);
        tile_step(Ks0, Vs0, t * kBC);
        copies_barrier();  // tile t+1 landed (each wave waited for its copies); tile t reads done
        if (t + 1 >= ntiles) break;
        if (t + 2 < ntiles) issue_tile(Ks0, Vs0, (t + 2) * kBC);
        tile_step(Ks1, Vs1, (t + 1) * kBC);
        copies_barrier();
    }

    // Epilogue: O / l, L = ln 2 * (m + log2 l). A row that saw no key has
    // l = 0 and m = -inf: O = 0 and L = -inf. Lane (r, g) holds the row of
    // query qw + r; each wave stages its 32 rows of O in one of the (now
    // idle) tile buffers and stores them whole (store_rows_via_lds).
    const float l = halves_sum(l_run), lb = halves_sum(lb_run);
    const int row = qw + r;
    const float inv = lb > 0.0f ? 1.0f / lb : 0.0f;
    copies_barrier();   // every wave is done with the tile buffers
    char* st = (char*)(wave == 0 ? Ks0 : (wave == 1 ? Ks1 : (wave == 2 ? Vs0 : Vs1)));
    auto value = [&](int db, int v) { return o[db][v] * inv; };
    if (OF32) store_rows_via_lds<D>(st, (float*)Out + ((size_t)bh * n_q + qw) * D, n_q - qw, value);
    else store_rows_via_lds<D>(st, (bf16*)Out + ((size_t)bh * n_q + qw) * D, n_q - qw, value);
    if (row < n_q && g == 0) Lse[(size_t)bh * n_q + row] = kLn2 * (m_ref + fast_log2(l));
}

template <int D, bool CAUSAL, bool OF32>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
    constexpr int BR = 128;
    const int n_qtiles = (a.n_q + BR - 1) / BR;
    const long long nwg = (long long)a.bh * n_qtiles;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OF32>), dim3((unsigned)nwg), dim3(kThreads), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.o, a.lse,
                       a.n_q, a.n_k, a.coff, n_qtiles, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t st) {
    if (a.causal)
        return a.o_f32 ? launch<D, true, true>(a, st) : launch<D, true, false>(a, st);
    return a.o_f32 ? launch<D, false, true>(a, st) : launch<D, false, false>(a, st);
}

}  // namespace

int fwd_bf16_rows_per_wg(const FwdArgs& a) { return fwd_pp_supports(a) ? 256 : 128; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
    if (fwd_pp_supports(a)) return launch_fwd_pp(a, st);
    switch (a.d) {
        case 32: return dispatch_mask<32>(a, st);
        case 64: return dispatch_mask<64>(a, st);
        case 96: return dispatch_mask<96>(a, st);
        case 128: return dispatch_mask<128>(a, st);
        case 256: return dispatch_mask<256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
