// Device-side building blocks shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.
// A: lane l holds row (l % 32), 8 consecutive k-slots of half (l / 32).
// B: lane l holds column (l % 32), the same 8 k-slots as A.
// D: lane l holds column (l % 32); element v is row 8*(v/4) + 4*(l/32) + v%4.
// Only the row/column placement matters to the callers: a contraction sums
// over all k-slots, so any bijection of keys onto slots works as long as A
// and B use the same one.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in element v by lane-half g.
__device__ __forceinline__ constexpr int acc_row(int v, int g) {
    return 8 * (v >> 2) + 4 * g + (v & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by the lane 32 positions away
// (l <-> l ^ 32). v_permlane32_swap with the same register as both operands
// leaves, in every lane, its own value in one result and its partner's in
// the other, so max / sum of the two results is the pairwise reduction
// whichever half each lands in.
__device__ __forceinline__ float halves_max(float x) {
    unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
    unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// acc + the sum of the 8 bf16 values of x (as fp32), with two-element dot
// products against (1, 1) (v_dot2c_f32_bf16): the exact sum of the rounded
// values that an MFMA operand carries.
__device__ __forceinline__ float sum_bf16x8(bf16x8 x, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t pr = {x[2 * i], x[2 * i + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
}

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// Issue priority of this wave on its SIMD: raised around blocks of MFMAs so
// they issue as soon as the matrix core is free, while the other wave on
// the SIMD fills the gaps with its VALU work.
__device__ __forceinline__ void mfma_priority(bool high) {
    if (high) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads and atomics still in flight are not waited for (a __syncthreads()
// would also drain every outstanding global store and atomic).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier after direct global -> LDS copies: each wave first waits
// for its own copies (vmcnt) and LDS writes (lgkmcnt), so after the barrier
// every wave sees every wave's data. Written out because the compiler orders
// a wave's copy only against that wave's own later reads of the same buffer.
// The wait is also issued through the builtin (encoding 0x70: vmcnt(0)
// lgkmcnt(0)), which the compiler's wait insertion sees: it then knows no
// copy is pending after the barrier and adds no waits of its own for them.
__device__ __forceinline__ void copies_barrier() {
    __builtin_amdgcn_s_waitcnt(0x70);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ds_read_b64_tr_b16: within each 16-lane group, the lane with local index
// 4*a + e receives element e of the 8-byte chunks addressed by the lanes
// a, 4 + a, 8 + a, 12 + a (in that order). When lane s of the group points
// at row k0 + s/4, column n0 + 4*(s%4) of a row-major bf16 tile, lane t
// therefore receives column n0 + t, rows k0 .. k0 + 3: an MFMA operand with
// the contraction index along the registers, read from an untransposed tile.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    typedef __bf16 lds_bf16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile with rows of D
// elements (D/8 chunks): row rho keeps logical chunk c at physical chunk
// c ^ tile_swz<D>(rho). The LDS has 64 banks of 4 bytes, i.e. 16 groups of
// 16 bytes; chunk k of the tile sits in group k % 16. Chosen so that (a) 16
// consecutive rows read at one logical chunk (an MFMA operand read with
// ds_read_b128) hit 16 different groups, and (b) 4 consecutive rows (aligned
// to 4) read over an aligned quad of chunks (a transpose read) hit disjoint
// groups. The swizzle only permutes chunks within aligned quads (values
// < 4) or aligned groups of 16 (values < 16, for rows of 16 or 32 chunks),
// so every physical chunk stays inside its row.
//  D = 128, 256 (16 or 32 chunks a row): the row's own offset is a multiple
//    of 16 groups, so the swizzle alone spreads rows: 4*(rho%4) separates
//    the 4 rows of a quad, (rho/4)%4 the 4 quads of 16 rows.
//  D = 64 (8 chunks): two rows share the 16 groups; 4*((rho/2)%2) separates
//    them, (rho/4)%4 the quads.
//  D = 32, 96 (4 or 12 chunks): the row offsets 4*rho or 12*rho mod 16
//    already take the 4 multiples of 4 over a quad of rows, so only the
//    quads of 16 rows need separating: (rho/4)%4.
template <int D>
__host__ __device__ constexpr int tile_swz(int rho) {
    static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dim");
    if constexpr (D == 128 || D == 256) return (4 * (rho & 3)) ^ ((rho >> 2) & 3);
    else if constexpr (D == 64) return (4 * ((rho >> 1) & 1)) ^ ((rho >> 2) & 3);
    else return (rho >> 2) & 3;
}

// Element offset of (row, col) in a swizzled row-major tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
    return row * D + 8 * ((col >> 3) ^ tile_swz<D>(row)) + (col & 7);
}

// Scheduling hint for an unrolled loop of STEPS steps, each with 2 LDS reads
// (for the next step) and 2 MFMAs: keep the reads one step ahead of the
// MFMAs that consume them instead of clustering or serialising them.
template <int STEPS>
__device__ __forceinline__ void sched_reads_ahead_of_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads of steps 0 and 1
#pragma unroll
    for (int i = 0; i < STEPS - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMAs of step i
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads of step i + 2
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMAs of the last two steps
}

// Buffer resource over `bytes` bytes from `base` (raw, 32-bit data format):
// buffer loads at byte offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16-byte global -> LDS copy that bypasses registers (buffer_load_dwordx4 ...
// lds): lane l's 16 bytes, read at byte offset `voff` of the resource, land at
// lds_base + 16*l; lds_base must be wave-uniform. A buffer (not a flat/global)
// load, so the compiler keeps precise waits on the LDS reads that follow.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, unsigned voff, void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds_base),
                                             16, (int)voff, 0, 0, 0);
}

// Work order of a grid of n_bh * n_tiles workgroups (one per (head, tile)).
// Workgroups go round-robin to the 8 XCDs (id % 8). When the heads split
// evenly over the XCDs, each XCD gets its own heads (their K/V re-reads stay
// in that XCD's L2) and runs its work by rank: rank 0 first for all its heads,
// then rank 1, and so on, so the longest causal tiles (rank 0) start first and
// the short ones fill the end. Otherwise ranks are interleaved over all
// heads. Returns the head in *bh and the rank in *rank.
__device__ __forceinline__ void work_item(int bid, int n_bh, int n_tiles, int* bh, int* rank) {
    const int n = n_bh * n_tiles;
    if ((n_bh & 7) == 0) {
        const int hpx = n_bh >> 3;                 // heads per XCD
        const int xcd = bid & 7, slot = bid >> 3;  // slot < hpx * n_tiles
        *bh = xcd * hpx + slot % hpx;
        *rank = slot / hpx;
    } else {
        const int l = bid < n ? bid : n - 1;
        *bh = l % n_bh;
        *rank = l / n_bh;
    }
}

// Store a wave's block of 32 rows x D columns that it holds as the
// transposed accumulators of 32x32 MFMAs (lane (r, g) owns row r; element
// 4i + j of block db is column 32 db + 8i + 4g + j) as whole rows, with
// 16-byte stores: the values go through the wave's own LDS area `st`
// (32 * D * sizeof(T) bytes, 16-byte aligned, idle meanwhile; rows of
// D * sizeof(T) bytes whose 16-byte chunks are XOR-swizzled by row, which
// spreads the staging writes over the banks and keeps each row's read-back
// conflict-free), then row p goes to out + p * D for p < nrows. Stored
// directly, each lane's four adjacent columns would make every store
// instruction touch 32 rows. value(db, v) is element v of block db.
template <int D, typename T, typename F>
__device__ __forceinline__ void store_rows_via_lds(char* st, T* out, int nrows, F&& value) {
    static_assert(sizeof(T) == 2 || sizeof(T) == 4, "bf16 or fp32 rows");
    constexpr int E = 16 / sizeof(T);          // elements per 16-byte chunk
    constexpr int CH = D / E;                  // chunks per row
    constexpr int LOW = CH & -CH;
    constexpr int SWM = (LOW < 32 ? LOW : 32) - 1;   // XOR mask: stays in the row
    constexpr int RB = D * (int)sizeof(T);     // bytes per row
    constexpr int NK = 32 * CH / 64;           // 16-byte stores per lane
    static_assert(32 * CH % 64 == 0, "whole 16-byte stores per lane");
    // The lane index passes an empty asm so that none of the address
    // arithmetic is hoisted above the caller's main loop, where it would
    // hold registers through it.
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    const int r = ln & 31, g = ln >> 5;
    const int rs = r & SWM;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                bf16x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = (bf16)value(db, 4 * i + j);
                const int c = 4 * db + i;      // columns 8c .. 8c + 7, half g
                *(bf16x4*)(st + r * RB + 16 * (c ^ rs) + 8 * g) = pk;
            } else {
                const int c = 8 * db + 2 * i + g;   // columns 4c .. 4c + 3
                *(float4*)(st + r * RB + 16 * (c ^ rs)) =
                    make_float4(value(db, 4 * i), value(db, 4 * i + 1), value(db, 4 * i + 2),
                                value(db, 4 * i + 3));
            }
        }
    if constexpr (64 % CH == 0) {
        // Store k covers rows RPI k .. RPI k + RPI - 1 (lane: row RPI k + rb,
        // chunk c). rb < RPI and RPI is a power of two, so the row's swizzle
        // bits are rb's plus those of RPI k: the LDS address is one lane
        // value XOR a constant, plus a constant the read folds into its
        // offset, and the global address a lane pointer plus a constant.
        constexpr int RPI = 64 / CH;
        const int rb = ln / CH, c = ln % CH;
        const int a0 = rb * RB + 16 * (c ^ (rb & SWM));
        T* o0 = out + (size_t)rb * D + E * c;
        auto row_addr = [&](int k) __attribute__((always_inline)) {
            return st + RPI * k * RB + (a0 ^ (16 * ((RPI * k) & SWM)));
        };
        if (nrows >= 32) {
#pragma unroll
            for (int k = 0; k < NK; ++k)
                *(uint4*)(o0 + (size_t)RPI * k * D) = *(const uint4*)row_addr(k);
        } else {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const uint4 x = *(const uint4*)row_addr(k);
                if (RPI * k + rb < nrows) *(uint4*)(o0 + (size_t)RPI * k * D) = x;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int p = 64 * k + ln;
            const int row = p / CH, c = p % CH;
            const uint4 x = *(const uint4*)(st + row * RB + 16 * (c ^ (row & SWM)));
            if (row < nrows) *(uint4*)(out + (size_t)row * D + E * c) = x;
        }
    }
}

}  // namespace fa
