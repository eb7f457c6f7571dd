/*
 * fa.h - exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfa.so. Every tensor argument is a HIP device pointer to a
 * contiguous row-major array; sizes are plain ints; the stream is a
 * hipStream_t passed as void* (NULL = the default stream). No call allocates
 * or frees device memory. Apart from the static scratch of fa_bwd_noalloc
 * the library keeps no global state but a per-device cache of the
 * compute-unit count (read on first use, safe from any thread), so the other
 * calls may run concurrently on different streams and host threads.
 *
 * Layout: Q, O, dO, dQ are [batch, heads, n_q, d]; K, V, dK, dV are
 * [batch, heads, n_k, d]; L is [batch, heads, n_q]. Offsets are 64-bit.
 * Q, K, V, O, dO, dQ, dK and dV must start 16-byte aligned (the kernels
 * move them in 16-byte pieces), else FA_E_ALIGN.
 *
 * Errors: every argument is checked on the host before any HIP call. On a
 * failed check nothing is launched, no output is touched and a status code
 * is returned. A failed launch returns FA_E_HIP. Calls are asynchronous: a
 * fault inside a kernel surfaces at the caller's next synchronisation.
 *
 * Supported: dtype FA_BF16 with d in {32, 64, 96, 128, 256}; dtype FA_F32
 * with d in {16, 32, 64, 96, 128}. n_k >= 1 whenever there is work (a softmax over zero
 * keys is undefined). One head's Q, K or V must be under 2 GiB
 * (max(n_q, n_k) * d * element size < 2^31), else FA_E_SHAPE. batch, heads
 * or n_q equal to 0 is an empty call: the forward does nothing; the backward
 * zeroes dK and dV when n_q == 0.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_BF16 = 0, /* bfloat16 storage; products on bf16 MFMA, accumulation in fp32 */
    FA_F32 = 1   /* float32 storage and arithmetic */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_E_NULLPTR = 1,   /* a required pointer is NULL                         */
    FA_E_SHAPE = 2,     /* negative size, n_k == 0 with work to do, or too big */
    FA_E_DTYPE = 3,     /* unknown dtype / o_dtype, or an unsupported pairing  */
    FA_E_HEADDIM = 4,   /* d not supported for this dtype                      */
    FA_E_SCALE = 5,     /* scale not finite or not > 0                         */
    FA_E_WORKSPACE = 6, /* backward workspace NULL or smaller than required    */
    FA_E_HIP = 7,       /* a HIP launch or runtime call failed                 */
    FA_E_CAUSAL = 8,    /* causal is not one of the fa_mask values             */
    FA_E_SCRATCH = 9,   /* fa_bwd_noalloc: the problem needs more scratch than
                           FA_BWD_NOALLOC_SCRATCH_BYTES                        */
    FA_E_ALIGN = 10     /* a tensor pointer is not 16-byte aligned             */
} fa_status;

/* The `causal` argument of fa_fwd / fa_bwd. */
typedef enum {
    FA_NO_MASK = 0,             /* every key visible                            */
    FA_CAUSAL_TOP_LEFT = 1,     /* key j visible to query i iff j <= i          */
    FA_CAUSAL_BOTTOM_RIGHT = 2  /* key j visible to query i iff j <= i + n_k - n_q */
} fa_mask;

/*
 * Forward pass: O = softmax(scale * Q K^T [+ causal mask]) V and
 * L = logsumexp of each masked, scaled score row (natural log), without
 * ever forming the n_q x n_k score matrix in memory.
 *
 * Defined by: the attention formula on page 2 ("FlashAttention：深度学习中的
 * 高效注意力机制", section 公式推导); the tiled forward with running max m and
 * running sum l, O rescaled by exp(m_old - m_new) per key tile, and the
 * outputs O / l and L = m + log(l), on page 1 ("05_flash_attention.py",
 * section 2, flash_attention_forward).
 *
 * q      [B,H,n_q,d] dtype       k, v  [B,H,n_k,d] dtype
 * o      [B,H,n_q,d] o_dtype     (o_dtype: FA_BF16 or FA_F32; FA_F32 inputs
 *                                 require FA_F32 output). A bf16 O is the
 *                                 round-to-nearest-even rounding of the fp32
 *                                 result.
 * lse    [B,H,n_q] float32, natural-log logsumexp L.
  * causal FA_NO_MASK (0): every key visible.
 *        FA_CAUSAL_TOP_LEFT (1): key j visible to query i iff j <= i, also
 *        when n_q != n_k (page 1, section 2, standard_attention masks the
 *        strict upper triangle).
 *        FA_CAUSAL_BOTTOM_RIGHT (2): key j visible to query i iff
 *        j <= i + n_k - n_q, so the last query sees every key (queries are
 *        the newest n_q positions of an n_k-long sequence; not on the pages,
 *        which define only the top-left mask). Same as 1 when n_q == n_k.
 *        When n_q > n_k the first n_q - n_k queries see no key: their O is
 *        0 and their L is -inf.
 *        Any other value: FA_E_CAUSAL.
 * scale  multiplies Q K^T; the usual value is 1/sqrt(d). Finite, > 0.
 * Outputs are written for every row < n_q and nothing else is written.
 */
int fa_fwd(const void* q, const void* k, const void* v,
           void* o, int o_dtype, float* lse,
           int batch, int heads, int n_q, int n_k, int d, int dtype,
           int causal, float scale, void* stream);

/*
 * Bytes of device workspace that let fa_fwd_ws split the keys of each query
 * tile over several workgroups for these sizes; 0 when it would not split
 * (the grid of query tiles already fills the GPU's compute units, or the
 * head dim is not 64 or 128, or float32, or fewer than 512 keys, or an empty
 * call). The answer depends on the current device's compute-unit count.
 * Returns SIZE_MAX for arguments fa_fwd would reject.
 */
size_t fa_fwd_workspace_bytes(int batch, int heads, int n_q, int n_k, int d,
                              int dtype, int causal);

/*
 * fa_fwd with a workspace: the same arguments, outputs and definition, for
 * grids with few query tiles (few heads, short query ranges, decoding-like
 * bottom-right calls). When fa_fwd_workspace_bytes(...) > 0 the keys of each
 * query tile are split into chunks of whole 64-key tiles, one workgroup per
 * chunk computes O and L over its keys into the workspace, and a second
 * kernel merges the chunks row by row: L = ln sum_s exp(L_s), O = sum_s
 * w_s O_s with w_s = exp(B_s - B), where B_s is the logsumexp of the bf16
 * weights chunk s applied in its PV product (the rescaling that merges the
 * running (m, l) of two key tiles on page 1, "05_flash_attention.py",
 * section 2, applied across workgroups). Otherwise it runs exactly fa_fwd.
 * Results equal fa_fwd's up to rounding, not bitwise; they are
 * deterministic.
 * workspace: device memory of at least fa_fwd_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored; may be
 * NULL when that size is 0. Too small (or NULL when needed): FA_E_WORKSPACE
 * with nothing launched. Calls that overlap in time must not share it.
 */
int fa_fwd_ws(const void* q, const void* k, const void* v,
              void* o, int o_dtype, float* lse,
              int batch, int heads, int n_q, int n_k, int d, int dtype,
              int causal, float scale,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (0 for an empty
 * call). bf16: the fp32 row term -D and L * log2(e), each [B,H,ceil(n_q/32)*32]
 * and 256-byte aligned, and, for grids with few query tiles (the dQ
 * kernel's 128-row workgroups would fill at most half of the GPU and there
 * are at least 2048 keys), the fp32 partials of dQ over key chunks
 * [chunks, B,H,n_q,d], and for grids with few key blocks (at least 2048
 * queries) those of dK and dV over query chunks [2, chunks, B,H,n_k,d];
 * float32: D [B,H,n_q]. The answer depends on the
 * current device's compute-unit count. Returns SIZE_MAX for arguments
 * fa_bwd would reject (so 0 always means an empty call).
 */
size_t fa_bwd_workspace_bytes(int batch, int heads, int n_q, int n_k, int d,
                              int dtype, int causal);

/*
 * Backward pass by recomputation: from Q, K, V, the forward's O and L and the
 * upstream gradient dO, computes dQ, dK, dV. P is rebuilt tile by tile as
 * exp(scale * Q K^T - L); D = rowsum(dO * O); dV = P^T dO; dP = dO V^T;
 * dS = P * (dP - D); dQ = scale * dS K; dK = scale * dS^T Q.
 *
 * Defined by: page 1 ("05_flash_attention.py", section 3,
 * flash_attention_backward and its docstring: the two tricks of rebuilding
 * P from the saved logsumexp and of D = rowsum(dO * O)); page 3 ("Flash
 * Attention", section 1.5, the derivatives of O = PV and of P = softmax(S)).
 *
 * o, lse are the outputs of fa_fwd for the same q, k, v, causal and scale
 * (o in o_dtype). A query row with no visible key (L = -inf, bottom-right
 * mask with n_q > n_k) gets dQ = 0 and adds nothing to dK or dV. d_o [B,H,n_q,d] dtype. dq [B,H,n_q,d], dk, dv [B,H,n_k,d]
 * in dtype; every element is overwritten.
 * workspace: device memory of at least fa_bwd_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored. Calls
 * that overlap in time must not share a workspace.
 * Results are deterministic: the same inputs give bitwise the same outputs.
 * With few query tiles (see fa_bwd_workspace_bytes) the dQ kernel splits
 * the keys over several workgroups, each summing dS K over its chunk in
 * fp32, and a second kernel adds the chunks in a fixed order and rounds dQ
 * once to bf16; with few key blocks the dK/dV kernel splits the queries
 * the same way.
 * Accuracy (bf16): dS is rounded to bf16 for the dQ and dK products; dQ's
 * error relative to each row's norm was about 2.4e-3 (median) at every
 * context length measured, 32K to 512K keys (causal, d = 128): it does not
 * grow with the number of keys summed.
 */
int fa_bwd(const void* q, const void* k, const void* v,
           const void* o, int o_dtype, const float* lse, const void* d_o,
           void* dq, void* dk, void* dv,
           int batch, int heads, int n_q, int n_k, int d, int dtype,
           int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd with per-kernel timing: identical arguments and results, plus
 * `events`, NULL or an array of 4 hipEvent_t (passed as void*) created by
 * the caller with timing enabled. They are recorded on `stream` before the
 * row-term kernel (D = rowsum(dO * O)), before the dK/dV kernel, after it
 * (= before the dQ kernel), and after the dQ kernel, so hipEventElapsedTime
 * gives each stage's duration. Not recorded for an empty call. For the callers that need the dominant kernel's own time (the
 * benchmark); the computation is the one fa_bwd documents.
 */
int fa_bwd_timed(const void* q, const void* k, const void* v,
                 const void* o, int o_dtype, const float* lse, const void* d_o,
                 void* dq, void* dk, void* dv,
                 int batch, int heads, int n_q, int n_k, int d, int dtype,
                 int causal, float scale,
                 void* workspace, size_t workspace_bytes, void* stream,
                 void* const* events);

/* Size of the static per-GPU scratch behind fa_bwd_noalloc (16 MiB). */
#define FA_BWD_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as fa_bwd, without the workspace. Its scratch
 * is a static array of FA_BWD_NOALLOC_SCRATCH_BYTES in the library's code
 * object, one per GPU, held from the first call on that GPU until the
 * process ends; the call itself allocates nothing. It serves problems whose
 * row arrays fit in the scratch (the bf16 -D and L * log2(e), or the float32
 * D, that fa_bwd_workspace_bytes counts; bf16: about 2 million query rows
 * over all batches and heads) and returns FA_E_SCRATCH beyond that, with
 * nothing launched. Where fa_bwd would split a kernel and the partials do
 * not fit in the scratch as well, it runs that kernel unsplit (the same
 * gradients up to rounding); otherwise its results equal fa_bwd's bitwise. Calls on one
 * GPU share that GPU's scratch: calls that overlap in time on the same GPU (other streams,
 * other host threads) race and give undefined results. The first call on a
 * GPU looks the scratch address up (hipGetSymbolAddress); a failure there
 * returns FA_E_HIP.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v,
                   const void* o, int o_dtype, const float* lse, const void* d_o,
                   void* dq, void* dk, void* dv,
                   int batch, int heads, int n_q, int n_k, int d, int dtype,
                   int causal, float scale, void* stream);

/*
 * Row softmax and logsumexp of a plain matrix: for every row r of scale * X,
 * lse[r] = ln sum_c exp(scale * X[r,c]) and, when y is not NULL,
 * y[r,c] = exp(scale * X[r,c] - lse[r]).
 *
 * Defined by: the softmax of a score row and its logsumexp, computed in one
 * pass with a running max m and a sum l rebased to it (page 1,
 * "05_flash_attention.py", section 1, online softmax; page 3, "Flash
 * Attention", section 1.1); lse = m + ln l.
 *
 * x      [rows, cols] dtype (FA_BF16 or FA_F32), read once for lse and once
 *        more for y.
 * lse    [rows] float32 (required).
 * y      NULL (lse only) or [rows, cols] y_dtype (FA_BF16, rounded to
 *        nearest even, or FA_F32).
 * rows   >= 0 (0 is an empty call); cols >= 1 when rows > 0.
 * scale  finite, > 0.
 * A row whose entries are all -inf gets lse = -inf and a zero y row. NaN or
 * +inf entries give undefined results for their row.
 */
int fa_row_softmax(const void* x, int dtype, long long rows, int cols, float scale,
                   float* lse, void* y, int y_dtype, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_str(int status);

/* ABI version of this header: 5 (2 added FA_CAUSAL_BOTTOM_RIGHT and
   FA_E_CAUSAL; 3 added fa_bwd_noalloc and FA_E_SCRATCH, and
   fa_bwd_workspace_bytes returns SIZE_MAX instead of 0 for rejected
   arguments; 4 added fa_fwd_workspace_bytes and fa_fwd_ws; 5 added the
   16-byte alignment check of the tensor pointers and FA_E_ALIGN). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
