// Row softmax / logsumexp on gfx950: the one-pass running statistics of
// page 1 ("05_flash_attention.py", section 1) and page 3 ("Flash
// Attention", section 1.1) as a standalone, HBM-bound kernel.
//
// One wave per row. Each lane walks its share of the row once, keeping a
// running max m and a sum l of exponentials rebased to m (exp2 domain, with
// scale * log2(e) folded into one FMA per element); the 64 lanes' (m, l)
// pairs are merged with the same rebasing rule in a butterfly, which gives
// L = ln 2 * (m + log2 l). If a softmax output is asked for, a second pass
// reads the row again and writes exp2(x * c - m) / l. A row whose entries
// are all -inf gets L = -inf and a zero softmax row.
//
// Rows are read with 16-byte vector loads when every row starts 16-byte
// aligned (cols a multiple of 16 / sizeof(T), x and y 16-byte aligned),
// otherwise element by element.
// A row of at most 64 lanes x kHold vectors (4096 bf16 or 2048 fp32
// elements) is held in registers between the two passes, so the softmax
// reads it from HBM once; longer rows stream twice, four loads in flight per
// lane.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kRowThreads = 256;  // 4 waves, one row each
constexpr int kUnroll = 4;        // vector loads in flight per lane (streaming)
constexpr int kHold = 8;          // vectors per lane held in registers

__device__ __forceinline__ float to_f(bf16 v) { return bf2f(v); }
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ void from_f(float v, bf16* p) { *p = to_bf16(v); }
__device__ __forceinline__ void from_f(float v, float* p) { *p = v; }

// (m, l) <- merge of (m, l) and (m2, l2), both in the exp2 domain. An empty
// side has m = -inf, l = 0; two empty sides stay empty.
__device__ __forceinline__ void merge(float& m, float& l, float m2, float l2) {
    const float mn = fmaxf(m, m2);
    if (mn == kNegInf) return;
    l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
    m = mn;
}

// Fold V consecutive elements into the running (m, l).
template <int V>
__device__ __forceinline__ void fold(const float* v, float cs, float& m, float& l) {
    float mx = v[0];
#pragma unroll
    for (int i = 1; i < V; ++i) mx = fmaxf(mx, v[i]);
    const float mn = fmaxf(m, mx * cs);
    if (mn == kNegInf) return;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) acc += fast_exp2(fmaf(v[i], cs, -mn));
    l = l * fast_exp2(m - mn) + acc;
    m = mn;
}

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
    static constexpr int N = 8;
    typedef bf16x8 raw;
    __device__ static raw ld(const bf16* p) { return *(const bf16x8*)p; }
    __device__ static void cvt(raw x, float* out) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = bf2f(x[i]);
    }
    __device__ static void load(const bf16* p, float* out) { cvt(ld(p), out); }
};
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    typedef float4 raw;
    __device__ static raw ld(const float* p) { return *(const float4*)p; }
    __device__ static void cvt(raw x, float* out) {
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
    __device__ static void load(const float* p, float* out) { cvt(ld(p), out); }
};

// Store V softmax values.
template <int V, typename YT>
__device__ __forceinline__ void store_y(YT* p, const float* y) {
#pragma unroll
    for (int i = 0; i < V; ++i) from_f(y[i], p + i);
}

// MODE 0: element by element; 1: vector loads, two streaming passes;
// 2: vector loads, row held in registers (cols <= 64 * V * kHold).
template <typename T, typename YT, int MODE>
__global__ __launch_bounds__(kRowThreads) void row_softmax_kernel(
    const T* __restrict__ X, long long rows, int cols, float cs, float* __restrict__ Lse,
    YT* __restrict__ Y) {
    constexpr int V = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * (kRowThreads / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave
    const T* xr = X + row * (long long)cols;

    float m = kNegInf, l = 0.0f;
    typename Vec16<T>::raw held[MODE == 2 ? kHold : 1];
    if (MODE == 2) {
#pragma unroll
        for (int u = 0; u < kHold; ++u) {
            const int c = (lane + 64 * u) * V;
            if (c < cols) held[u] = Vec16<T>::ld(xr + c);
        }
#pragma unroll
        for (int u = 0; u < kHold; ++u) {
            const int c = (lane + 64 * u) * V;
            if (c < cols) {
                float v[V];
                Vec16<T>::cvt(held[u], v);
                fold<V>(v, cs, m, l);
            }
        }
    } else if (MODE == 1) {
        constexpr int STEP = 64 * V;
        for (int c0 = lane * V; c0 < cols; c0 += kUnroll * STEP) {
            float v[kUnroll][V];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (c0 + u * STEP < cols) Vec16<T>::load(xr + c0 + u * STEP, v[u]);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (c0 + u * STEP < cols) fold<V>(v[u], cs, m, l);
        }
    } else {
        for (int c = lane; c < cols; c += 64) {
            const float v = to_f(xr[c]);
            fold<1>(&v, cs, m, l);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
        merge(m, l, m2, l2);
    }
    if (lane == 0) Lse[row] = m == kNegInf ? kNegInf : kLn2 * (m + fast_log2(l));
    if (Y == nullptr) return;

    // Second pass: y = exp2(x * c - m) / l (zero for an all -inf row).
    YT* yr = Y + row * (long long)cols;
    const bool empty = m == kNegInf;
    const float inv = empty ? 0.0f : 1.0f / l;
    const float mm = empty ? 0.0f : m;
    if (MODE == 2) {
#pragma unroll
        for (int u = 0; u < kHold; ++u) {
            const int c = (lane + 64 * u) * V;
            if (c < cols) {
                float v[V], y[V];
                Vec16<T>::cvt(held[u], v);
#pragma unroll
                for (int i = 0; i < V; ++i) y[i] = empty ? 0.0f : fast_exp2(fmaf(v[i], cs, -mm)) * inv;
                store_y<V>(yr + c, y);
            }
        }
    } else if (MODE == 1) {
        for (int c = lane * V; c < cols; c += 64 * V) {
            float v[V], y[V];
            Vec16<T>::load(xr + c, v);
#pragma unroll
            for (int i = 0; i < V; ++i) y[i] = empty ? 0.0f : fast_exp2(fmaf(v[i], cs, -mm)) * inv;
            store_y<V>(yr + c, y);
        }
    } else {
        for (int c = lane; c < cols; c += 64) {
            const float v = to_f(xr[c]);
            from_f(empty ? 0.0f : fast_exp2(fmaf(v, cs, -mm)) * inv, yr + c);
        }
    }
}

template <typename T, typename YT>
hipError_t launch_typed(const RowArgs& a, hipStream_t st) {
    const long long nb = (a.rows + 3) / 4;
    if (nb > 0x7fffffffLL) return hipErrorInvalidValue;
    constexpr int V = Vec16<T>::N;
    const float cs = a.scale * kLog2e;
    // Vector loads and stores need every row 16-byte aligned: cols a multiple
    // of the vector and both buffers starting 16-byte aligned.
    const bool aligned = a.cols % V == 0 && ((uintptr_t)a.x & 15) == 0 && ((uintptr_t)a.y & 15) == 0;
    if (!aligned)
        hipLaunchKernelGGL((row_softmax_kernel<T, YT, 0>), dim3((unsigned)nb), dim3(kRowThreads), 0, st,
                           (const T*)a.x, a.rows, a.cols, cs, a.lse, (YT*)a.y);
    else if (a.cols <= 64 * V * kHold)
        hipLaunchKernelGGL((row_softmax_kernel<T, YT, 2>), dim3((unsigned)nb), dim3(kRowThreads), 0, st,
                           (const T*)a.x, a.rows, a.cols, cs, a.lse, (YT*)a.y);
    else
        hipLaunchKernelGGL((row_softmax_kernel<T, YT, 1>), dim3((unsigned)nb), dim3(kRowThreads), 0, st,
                           (const T*)a.x, a.rows, a.cols, cs, a.lse, (YT*)a.y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_softmax(const RowArgs& a, hipStream_t st) {
    if (a.x_f32) return a.y_f32 ? launch_typed<float, float>(a, st) : launch_typed<float, bf16>(a, st);
    return a.y_f32 ? launch_typed<bf16, float>(a, st) : launch_typed<bf16, bf16>(a, st);
}

}  // namespace fa
