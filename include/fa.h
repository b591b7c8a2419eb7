/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library, libfa.so.
 *
 * The operation is standard scaled dot-product attention computed without ever
 * writing the N x N score or probability matrices to memory:
 *
 *     S = scale * Q K^T,   P = softmax(S) (row-wise),   O = P V,
 *     LSE_i = m_i + ln(l_i),  m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i).
 *
 * The problem statement is the one in "FlashAttention 硬件感知计算剖析" (section 一.2,
 * the three formulas of standard attention); tensors are laid out as
 * [Batch, Heads, Seq_Len, Head_Dim] as in that page's section 五.1; the running
 * row statistics m (max) and l (exp-sum) and the rescale by exp(m_old - m_new) are
 * the online softmax of "从零理解Flash Attention中的online softmax" (section 3.1) and
 * of the two-block merge in "FlashAttention 硬件感知计算剖析" (section 二).  The saved
 * statistic is the log-sum-exp m + ln l, which is what a recompute-based backward
 * ("从原理出发理解 Flash Attention Part2", section 2.4) needs to rebuild P.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a HIP device pointer owned by the caller.  The
 *     library allocates nothing in these calls and keeps no pointer after return.
 *     Buffers must stay alive until the work queued on `stream` has completed.
 *   - Layout: contiguous [B, H, N, d]; element (b, h, n, k) is at index
 *     ((b*H + h)*N + n)*d + k.  LSE / D are contiguous fp32 [B, H, N].
 *   - Q, K, V, O (and dO, dQ, dK, dV) share one element type `dtype`; O has the
 *     input dtype.  LSE is always fp32, natural log.
 *   - `stream` is a hipStream_t (NULL = the default stream).  The header declares the
 *     type as HIP does, an opaque pointer, so it needs no HIP header of its own.
 *     Calls are asynchronous: validation errors return synchronously before any
 *     work is queued; device faults surface at the caller's next synchronisation.
 *   - Outputs must not alias inputs.  Tensor pointers must be 16-byte aligned,
 *     LSE/D 4-byte aligned.
 *   - Non-finite inputs propagate to the outputs; finite inputs of any magnitude
 *     give finite outputs.
 *   - Validation order: shapes, head dim / dtype; then an empty problem
 *     (B*H*N == 0) returns FA_OK and queues nothing (its pointers may be NULL);
 *     then null pointers, alignment, scale, and finally the device.
 *   - Environment (read on every call, host only):
 *       FA_TILE=Br,Bc,W  replaces the tile chooser's plan for fa_fwd, fa_fwd_causal and
 *                        fa_fwd_plan (and split-KV calls that run as one split) with Br
 *                        query rows per workgroup, Bc keys per K/V tile and W waves, for
 *                        measuring tile choices ("从零理解Flash Attention中的online softmax",
 *                        section 6.1, picks tiles by measurement per GPU).  It must name a
 *                        compiled kernel for the call's dtype and head dim -- bf16/fp16:
 *                        d = 128: 256,128,8  128,64,4  128,32,4;  d = 64: 256,128,8
 *                        128,128,4  128,64,4;  fp32: 32,32,4 -- else those calls return
 *                        FA_ERR_TILE.  Unset or empty: the chooser decides.
 *       FA_LOG=1         prints each call's plan (tiles, waves, grid, LDS, splits) to
 *                        stderr as soon as it is chosen, before the device check.
 *   - Thread safety: calls may be made concurrently from several host threads;
 *     the only global state is a read-only per-device property cache and the
 *     static scratch buffer of fa_fwd_splitkv_qk_noalloc (whose own calls must not
 *     overlap on one GPU).
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared exactly as hip_runtime_api.h declares it (an identical
 * typedef may appear twice), so that callers without HIP headers can still pass one. */
typedef struct ihipStream_t* hipStream_t;

/* Compiled as C++, the enumerations take int as their fixed underlying type, so any int a
 * C caller passes (an unknown dtype, an unknown status) is a valid value for the library to
 * receive and reject; the layout is the C enum's either way. */
#ifdef __cplusplus
#define FA_ENUM_INT : int
#else
#define FA_ENUM_INT
#endif

typedef enum FA_ENUM_INT {
    FA_F32 = 0,
    FA_F16 = 1,
    FA_BF16 = 2
} fa_dtype;

typedef enum FA_ENUM_INT {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
    FA_ERR_SHAPE = 2,       /* B, H or N negative, or sizes overflow the index math */
                            /* or a launch's 2^31 workgroup ids                       */
    FA_ERR_UNSUPPORTED = 3, /* head dim not in {64, 128}, or unknown dtype           */
    FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte (LSE: 4-byte) aligned */
    FA_ERR_SCALE = 5,       /* scale is not finite or not > 0                        */
    FA_ERR_DEVICE = 6,      /* no HIP device, or the current device is not gfx950    */
    FA_ERR_LAUNCH = 7,      /* the kernel launch was rejected by the runtime          */
    FA_ERR_WORKSPACE = 8,   /* workspace missing or smaller than required             */
    FA_ERR_SCRATCH = 9,     /* the call needs more than the library's static scratch  */
    FA_ERR_TILE = 10        /* FA_TILE names no compiled kernel for this problem      */
} fa_status;

/* Bytes of the per-device static scratch buffer behind fa_fwd_splitkv_qk_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Launch plan the tile/occupancy chooser picks for a forward problem. */
typedef struct {
    int32_t block_q;        /* Br: query rows per workgroup                            */
    int32_t block_k;        /* Bc: keys per K/V tile streamed through LDS              */
    int32_t waves;          /* wavefronts (64 lanes) per workgroup                     */
    int32_t rows_per_wave;  /* query rows each wave computes                           */
    int32_t lds_bytes;      /* LDS per workgroup (its K and V tile buffers)            */
    int64_t grid;           /* workgroups launched = B*H*ceil(N/Br) (*splits); with    */
                            /* tail first (below) B*H*floor(N/Br)                      */
    int32_t kv_splits;      /* >1: key range split across workgroups, then merged      */
    int32_t wave_kv_splits; /* >1: a workgroup's waves share its query rows and split  */
                            /*     the key tiles among themselves, merged in LDS       */
    int32_t tail_kv_splits; /* >1: the last query block of each head (at most 32 rows; */
                            /*     128 on 8 waves) has its keys split.  4 waves: over  */
                            /*     the block's waves, merged in LDS (whole grid        */
                            /*     resident at once).                                  */
                            /*     8 waves ("tail first"): those rows are computed     */
                            /*     ahead of the main launch by tail_kv_splits          */
                            /*     workgroups per head, their partials parked in the   */
                            /*     head's first O rows; the main launch covers the     */
                            /*     full blocks and merges them first (not used when O  */
                            /*     overlaps Q, K, V or LSE)                            */
} fa_plan;

/*
 * Forward attention.  Q, K, V: [B,H,N,d] of `dtype`; O: [B,H,N,d] of `dtype`;
 * LSE: [B,H,N] fp32 (natural log).  `scale` multiplies Q K^T (1/sqrt(d) for the
 * usual attention).  Supported: d in {64, 128}; dtype FA_BF16 / FA_F16 (matrix
 * products on bf16/fp16 MFMA with fp32 accumulation and fp32 softmax statistics)
 * or FA_F32 (fp32 MFMA throughout).  Any N >= 0 (tails are masked).  O may also hold
 * intermediate values while the call's work runs (see fa_plan.tail_kv_splits): read it only
 * after the stream has passed the call.  O may coincide with Q (computed in place).
 */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                 fa_dtype dtype, hipStream_t stream);

/*
 * Causal forward: as fa_fwd, but query i attends only to keys j <= i (the
 * lower-triangular mask of "FlashAttention 硬件感知计算剖析", section 五.3).  Key
 * tiles strictly above the diagonal are skipped, not masked.
 */
fa_status fa_fwd_causal(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        fa_dtype dtype, hipStream_t stream);

/*
 * The plan fa_fwd / fa_fwd_causal would launch for this problem on a gfx950
 * device (pure host computation: no HIP call, usable without a GPU).
 * Returns the same validation status fa_fwd would (pointer checks excepted).
 */
fa_status fa_fwd_plan(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype,
                      int causal, fa_plan* plan);

/*
 * Split-KV forward ("从零理解Flash Attention中的online softmax", section 8.1: two-level
 * blocking; "FlashAttention 硬件感知计算剖析", section 二: merging blocks by their
 * maximum and sum).  The key range of every query block is cut into `splits` ranges of
 * whole key tiles, each computed by its own workgroup into normalised fp32 partials
 * (O_s, LSE_s) in `workspace`; a merge pass writes LSE = ln sum_s e^{LSE_s} and
 * O = sum_s e^{LSE_s - LSE} O_s.  For problems whose plain grid does not fill the chip
 * (small B*H*N).  Same inputs, outputs, layouts and validation as fa_fwd (non-causal),
 * bf16/fp16 only (FA_F32 -> FA_ERR_UNSUPPORTED).  splits: 0 = the library's choice
 * (fa_fwd_splitkv_splits), else 1..64 (more than the key tiles is clamped to them;
 * outside -> FA_ERR_SHAPE).  With one split it is fa_fwd and needs no workspace.
 * workspace: device memory of at least fa_fwd_splitkv_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller, contents on entry ignored; NULL, short or
 * misaligned -> FA_ERR_WORKSPACE.
 */
size_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype,
                                      int32_t splits);
/* The split count fa_fwd_splitkv uses for splits = 0 (1: splitting would not pay). */
int32_t fa_fwd_splitkv_splits(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype);
fa_status fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                         void* workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, fa_dtype dtype, int32_t splits, hipStream_t stream);

/*
 * The same with Nq query rows and Nk keys per head (Q, O [B,H,Nq,d]; K, V [B,H,Nk,d]; LSE
 * [B,H,Nq]): every query attends to all Nk keys -- a chunk of new queries against a longer
 * key/value history, or one query per head when decoding.  It is the split-KV forward
 * above with the two lengths apart (fa_fwd_splitkv is this call with Nq = Nk = N); the
 * split count and workspace refer to Nk's key tiles and Nq's rows.  Nq > 0 with Nk = 0 is
 * FA_ERR_SHAPE (no keys to attend to); Nq = 0 is an empty problem.
 */
size_t fa_fwd_splitkv_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                         fa_dtype dtype, int32_t splits);
int32_t fa_fwd_splitkv_qk_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype);
fa_status fa_fwd_splitkv_qk(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            void* workspace, size_t ws_bytes, int64_t B, int64_t H, int64_t Nq,
                            int64_t Nk, int64_t d, float scale, fa_dtype dtype, int32_t splits,
                            hipStream_t stream);

/*
 * fa_fwd_splitkv_qk without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split partials go to a static device buffer of
 * FA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it runs on until
 * the process ends; its address is looked up once per device, on the first call there.
 * Same arguments (minus workspace / ws_bytes), layouts, results and errors as
 * fa_fwd_splitkv_qk; a call whose split partials need more than the static buffer
 * (fa_fwd_splitkv_qk_workspace_bytes(...) > FA_NOALLOC_SCRATCH_BYTES) returns
 * FA_ERR_SCRATCH before queuing anything.  Every call on one GPU shares that GPU's
 * buffer: calls that can overlap on one GPU (different streams, or host threads without
 * ordering) race on it and must be serialised by the caller.  Calls on one stream are
 * ordered and safe.  With one split (the chooser's answer for full grids) no scratch is
 * used at all.
 */
fa_status fa_fwd_splitkv_qk_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                    int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                    fa_dtype dtype, int32_t splits, hipStream_t stream);

/*
 * Workspace the backward needs, in bytes: two fp32 values per row (B*H*N rows).
 * Returns 0 for invalid or empty shapes.
 */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype);

/*
 * Recompute-based backward of fa_fwd ("从原理出发理解 Flash Attention Part2", section
 * 2.4; "从零理解Flash Attention中的online softmax", section 5.1): P is rebuilt from the
 * saved LSE, never stored.  With D_i = sum_k dO_ik O_ik:
 *     dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * Inputs: Q, K, V, O, dO [B,H,N,d] of `dtype`; LSE [B,H,N] fp32 exactly as fa_fwd wrote
 * them.  Outputs dQ, dK, dV [B,H,N,d] of `dtype` (overwritten, not accumulated).
 * `workspace` is device memory of at least fa_bwd_workspace_bytes(...) bytes, 256-byte
 * aligned, owned by the caller; its contents on entry are ignored.  Supported: dtype
 * FA_BF16 / FA_F16, d in {64, 128} (FA_F32 returns FA_ERR_UNSUPPORTED).  Deterministic
 * (no atomics).  Validation as fa_fwd, plus FA_ERR_WORKSPACE for a NULL, misaligned or
 * short workspace.
 */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t ws_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                 hipStream_t stream);

/* Backward of fa_fwd_causal (keys after the query row get P = 0). */
fa_status fa_bwd_causal(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t ws_bytes,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale, fa_dtype dtype,
                        hipStream_t stream);

/*
 * Block-scaled fp8 mode (opt-in; changes the numerics).  "从零理解Flash Attention中的online
 * softmax" (section 9.1) keeps K and V in 8 bits with a scale and dequantises each tile on
 * load; "FlashAttention 硬件感知计算剖析" (its FlashAttention-3 summary) names native FP8
 * with block-wise scale factors.  The reading taken here:
 *   - codes are OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
 *     finite 448; S.1111.111 is NaN), one byte per element;
 *   - every 64 consecutive rows of a (batch, head) share one scale 2^e, the smallest power
 *     of two with max|x| <= 448 * 2^e (e in [-126, 127]; an all-zero block takes -126);
 *     a code c stands for value(c) * 2^e;
 *   - the forward is attention of the dequantised Q, K, V; it also rounds the
 *     probabilities to E4M3 for the P V product (fp32 accumulation throughout), so O
 *     carries that rounding on top of the quantisation of the inputs.
 * Scales are fp32 [B, H, nb] with nb = fa_fp8_scale_blocks(N); block k covers rows
 * 64k .. 64k+63.  V is passed transposed, V^T [B, H, d, Np] with Np = fa_fp8_padded_len(N),
 * keys contiguous; the padding keys N..Np-1 must hold code 0 (fa_quantize_fp8 writes it).
 */
/* Np: N rounded up to the forward's key tile (128); 0 for N < 0 or N > INT64_MAX - 128. */
int64_t fa_fp8_padded_len(int64_t N);
/* nb = ceil(N / 64): scale blocks per (batch, head); 0 for N < 0. */
int64_t fa_fp8_scale_blocks(int64_t N);
/*
 * Quantise X [B,H,N,d] (FA_BF16 / FA_F16) into codes and block scales.  transpose = 0:
 * X8 is [B,H,N,d]; transpose = 1: X8 is V^T [B,H,d,Np] including its zero padding.
 * scales: fp32 [B,H,nb].  Deterministic; rounding to nearest, ties to even.  Non-finite
 * elements give a scale of 1 for their block and NaN codes.  Errors: as fa_fwd for
 * shapes, dtype (FA_F32 -> FA_ERR_UNSUPPORTED) and pointers (X, X8 16-byte, scales
 * 4-byte aligned); transpose not 0/1 -> FA_ERR_UNSUPPORTED.
 */
fa_status fa_quantize_fp8(const void* X, void* X8, float* scales, int64_t B, int64_t H, int64_t N,
                          int64_t d, fa_dtype dtype, int32_t transpose, hipStream_t stream);
/*
 * Attention forward on block-scaled E4M3 inputs: Q8, K8 [B,H,N,d] codes, Vt8 [B,H,d,Np]
 * codes, their scales [B,H,nb]; writes O [B,H,N,d] of out_dtype (FA_BF16 / FA_F16) and
 * LSE [B,H,N] fp32 (natural log of the dequantised scores' exp-sum, scale included).
 * Non-causal.  Errors: as fa_fwd (code pointers and O 16-byte aligned, scales and LSE
 * 4-byte aligned; out_dtype FA_F32 -> FA_ERR_UNSUPPORTED).
 */
fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale,
                     const float* k_scale, const float* v_scale, void* O, float* LSE, int64_t B,
                     int64_t H, int64_t N, int64_t d, float scale, fa_dtype out_dtype, hipStream_t stream);
/*
 * fa_fwd_fp8 with the causal mask of fa_fwd_causal: query row i attends to keys 0..i.
 * Same arguments, layouts and errors.
 */
fa_status fa_fwd_fp8_causal(const void* Q8, const void* K8, const void* Vt8, const float* q_scale,
                            const float* k_scale, const float* v_scale, void* O, float* LSE, int64_t B,
                            int64_t H, int64_t N, int64_t d, float scale, fa_dtype out_dtype, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
