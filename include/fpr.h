/*
 * fpr.h -- C interface of libfpr.so: the packed FP8 QKV projection with
 * reduced-width Q/K heads, forward and backward, on one MI355X (gfx950);
 * and the FP8 ReLU^2 MLP of the same block (the mlp_* calls below).
 *
 * The method ("96 is enough: shrinking attention's routing vectors",
 * section "The change"): Q and K heads are d_qk = 96 wide while V stays
 * d_v = 128 wide; the three projections are packed into one weight
 * W_packed = [W_q | W_k | W_v] (320 columns per head instead of 384), and a
 * single FP8 product of x with W_packed gives all three; q, k, v are split
 * off, q and k are RMS-normalised and rotated with RoPE.  The PR #344 page,
 * section "Changes", adds: both FP8 layouts of W_packed (row-major and
 * transposed) are cached per optimizer update and come from one weight
 * read; the logical Q/K and V packs are quantised without materialising the
 * concatenation; norm, RoPE and layout conversion are fused; the backward
 * pass runs in FP8 too.  "Where the eight seconds were hiding", section
 * "The inventory": the transposed view is reused, not rebuilt, by backward.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or synchronises, and keeps no mutable
 *    global state apart from the optional per-thread profiling trace and
 *    qkv_forward_noalloc's fixed per-device scratch.  Every call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL means the default
 *    stream) and returns.
 *  - Inputs are read-only.  Outputs are fully overwritten (dW is written,
 *    not accumulated).
 *  - bf16 tensors are passed as uint16_t bit patterns.  FP8 is OCP E4M3
 *    ("e4m3fn": max 448, no infinities), round to nearest even, saturating.
 *  - Per-tensor scales: s = amax/448 and inv = 448/amax in fp32 (IEEE
 *    division); codes are e4m3(v * inv).  amax == 0 (or 448/amax overflowing)
 *    gives s = inv = 1.  One scale covers the whole W_packed, one covers x,
 *    one covers the packed gradient dQKV (over its bf16 values).
 *  - T = n_seq * seq_len tokens; token t = b*seq_len + s has RoPE position s.
 *  - Packed column order: [Q heads | K heads | V heads],
 *    N = n_heads * (2*d_qk + d_v).
 *  - RMSNorm has no gain: u = a / sqrt(mean(a^2) + eps).  RoPE rotates the
 *    pairs (i, i + d_qk/2) by p * rope_base^(-2i/d_qk).
 *  - Return value: FPR_OK or an FPR_ERR_* code.  Argument errors are found
 *    before anything is launched.  A non-finite amax is reported on the
 *    device, in cache->status (see fpr_weight_cache), readable after the
 *    caller synchronises.
 *
 * Supported shapes: d_model % 64 == 0, d_qk % 16 == 0, d_v % 16 == 0,
 * N % 64 == 0, n_heads <= 64; for d_qk other than 64, 96 and 128 the
 * norm/RoPE tiles of 16 tokens must also fit 64 KiB of LDS
 * (36 * 2*n_heads*d_qk + 64*d_qk bytes); any 1 <= T <= 2^24 (ragged tails
 * are masked).
 * Alignment: every pointer 16-byte aligned; ldq/ldk/ldv multiples of 4.
 */
#ifndef FPR_H
#define FPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these calls are exported. */
#define FPR_API __attribute__((visibility("default")))

enum {
    FPR_OK = 0,
    FPR_ERR_ARG = 1,        /* null pointer, non-positive size, ld < columns */
    FPR_ERR_SHAPE = 2,      /* dimensions outside the supported set */
    FPR_ERR_ALIGN = 3,      /* pointer or leading dimension misaligned */
    FPR_ERR_WORKSPACE = 4,  /* workspace or saved buffer too small */
    FPR_ERR_LAUNCH = 5,     /* a kernel launch failed */
    FPR_ERR_SCRATCH = 6     /* qkv_forward_noalloc: the workspace the call
                               needs exceeds the fixed scratch */
};

/* Bits of *cache->status (device int32). */
enum {
    FPR_STATUS_W_NONFINITE = 1,   /* W_packed had a NaN/Inf (set by pack) */
    FPR_STATUS_X_NONFINITE = 2,   /* x had a NaN/Inf (set by forward) */
    FPR_STATUS_G_NONFINITE = 4,   /* dQKV (or the MLP's dy) had a NaN/Inf */
    FPR_STATUS_H_NONFINITE = 8    /* the MLP's h or dpre had a NaN/Inf */
};

/* Model dimensions.  The pages' setting: d_qk = 96, d_v = 128. */
typedef struct fpr_dims {
    int32_t d_model;   /* D, width of x */
    int32_t n_heads;   /* H */
    int32_t d_qk;      /* width of each q and k head */
    int32_t d_v;       /* width of each v head */
    float eps;         /* RMSNorm epsilon (inside the square root) */
    float rope_base;   /* RoPE base, e.g. 10000 */
    int32_t qk_stride; /* row stride (elements) of the q/k/dq/dk heads; 0 means
                          d_qk.  Otherwise a multiple of 8 in [d_qk, 1024]: a
                          consumer that wants equal Q/K/V head widths (an
                          attention kernel built for 128-wide heads) gets q and
                          k with d_qk values and qk_stride - d_qk zeros per
                          row, and hands dq/dk back in the same layout; their
                          padding columns are never read.  The padding for
                          FlashAttention-3 is one of the steps fused into the
                          norm/RoPE kernel in "Reduced-width QK and packed FP8
                          attention", Changes. */
    int32_t grad_format;  /* FPR_FORMAT_E4M3 (0, the default) or FPR_FORMAT_E5M2:
                          the FP8 format of the packed gradient dQKV in the
                          backward (its per-tensor scale then uses 57344, the
                          largest finite e5m2, in place of 448).  The weight
                          and x codes stay e4m3; dX and dW multiply e5m2 by
                          e4m3 codes on the matrix cores.  An attention-ready
                          variant: gradients keep e5m2's wider range. */
    int32_t bwd_passes;   /* 0 or 1 (the default): the backward writes dQK in bf16
                          to its workspace and quantises dQK and dv from there.
                          2: two passes over the forward's rows that never
                          write dQK, the fusion of the norm/RoPE backward into
                          the gradient quantiser with a two-pass amax: the
                          first pass takes dQK's amax, the second re-derives
                          every row and encodes it with the gradient scale.
                          The same codes, dX and dW bit for bit, and no dQK
                          buffer in the workspace; d_qk 64, 96 or 128 only. */
} fpr_dims;

/* FP8 formats (OCP): E4M3 (max 448, no inf) and E5M2 (max 57344, with inf;
 * encoding saturates at +-57344). */
enum { FPR_FORMAT_E4M3 = 0, FPR_FORMAT_E5M2 = 1 };

/* The cached FP8 views of W_packed, rebuilt by pack_quantize_weights after
 * every update of the fp32 weights ("invalidate on update").  All four
 * pointers are caller-owned device buffers. */
typedef struct fpr_weight_cache {
    uint8_t* w_packed;    /* [D][N] e4m3: W_packed row-major (read by dX)      */
    uint8_t* w_packed_t;  /* [N][D] e4m3: its transpose (read by the forward)  */
    float* scales;        /* [2] fp32: s_w, inv_w                              */
    int32_t* status;      /* [1] FPR_STATUS_* bits; pack resets it             */
} fpr_weight_cache;

enum { FPR_CALL_PACK = 0, FPR_CALL_FORWARD = 1, FPR_CALL_BACKWARD = 2,
       FPR_CALL_PACK_FORWARD = 3 };

/* Bytes of workspace each call needs for `tokens` = T tokens (ignored for
 * FPR_CALL_PACK; FPR_CALL_PACK_FORWARD is qkv_pack_forward's).  0 for
 * invalid dims. */
FPR_API size_t fpr_workspace_bytes(const fpr_dims* dims, int64_t tokens, int which);

/* Bytes of the buffer qkv_forward fills for qkv_backward: the FP8 x (in the
 * layout the dW GEMM reads), its scales, and one fp32 1/rms per Q and K head
 * row.  It must stay alive and unmodified from forward to backward, and so
 * must the forward's q and k outputs, which the backward reads too (no
 * pre-norm row is kept: the backward rebuilds the normalised rows from q, k
 * and the saved 1/rms). */
FPR_API size_t fpr_saved_bytes(const fpr_dims* dims, int64_t tokens);

/* Step 1 ("Changes": cache row-major and transposed FP8 weights once per
 * optimizer update, both from one weight read; no materialised
 * concatenation).  Computes amax over the logical W_packed whose pieces are
 *   wq: [D][H*d_qk] fp32, row stride ldq elements
 *   wk: [D][H*d_qk] fp32, row stride ldk
 *   wv: [D][H*d_v]  fp32, row stride ldv
 * then writes cache->w_packed, cache->w_packed_t, cache->scales and resets
 * cache->status.  Workspace: fpr_workspace_bytes(dims, 0, FPR_CALL_PACK). */
FPR_API int pack_quantize_weights(const fpr_dims* dims,
                          const float* wq, int64_t ldq,
                          const float* wk, int64_t ldk,
                          const float* wv, int64_t ldv,
                          const fpr_weight_cache* cache,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Step 2 ("96 is enough", "The change": one FP8 product of x with W_packed,
 * split, rms_norm and rope on q and k; "Reduced-width QK and packed FP8
 * attention", Changes: norm, RoPE and layout conversion fused).  For d_qk of
 * 64, 96 and 128 the norm and RoPE run inside the GEMM's epilogue and no
 * pre-norm value reaches memory; other widths pass the pre-norm Q|K rows
 * through the forward workspace.
 *   x:  [T][D] bf16 input activations
 *   q:  [n_seq][H][seq_len][qk_stride] bf16 out (normalised, rotated; the
 *       columns past d_qk written as zero)
 *   k:  [n_seq][H][seq_len][qk_stride] bf16 out, likewise
 *   v:  [n_seq][H][seq_len][d_v]  bf16 out
 *   saved: fpr_saved_bytes(dims, T) bytes, filled for qkv_backward.
 * The weight cache must have been filled by pack_quantize_weights. */
FPR_API int qkv_forward(const fpr_dims* dims, int32_t n_seq, int32_t seq_len,
                const uint16_t* x, const fpr_weight_cache* cache,
                uint16_t* q, uint16_t* k, uint16_t* v,
                void* saved, size_t saved_bytes,
                void* workspace, size_t workspace_bytes,
                void* stream);

/* pack_quantize_weights then qkv_forward, for a step that packs fresh
 * weights before its forward (the weights change every optimizer step,
 * "Reduced-width QK and packed FP8 attention", Changes): the same results
 * bit for bit (the cache with its status word, saved, q, k, v), with the
 * weight's amax and x's in one launch and both quantisers in the next, so
 * that the small weight work runs beside the activation streams instead of
 * before them.  Arguments, ownership and errors as in the two calls (every
 * check of both is made before the first launch); the workspace is
 * fpr_workspace_bytes(dims, T, FPR_CALL_PACK_FORWARD) bytes. */
FPR_API int qkv_pack_forward(const fpr_dims* dims,
                const float* wq, int64_t ldq, const float* wk, int64_t ldk,
                const float* wv, int64_t ldv, const fpr_weight_cache* cache,
                int32_t n_seq, int32_t seq_len, const uint16_t* x,
                uint16_t* q, uint16_t* k, uint16_t* v,
                void* saved, size_t saved_bytes,
                void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * as qkv_forward, with the workspace taken from a fixed device array inside
 * the library, fpr_noalloc_scratch_bytes() = 64 KiB per device, held until
 * the process ends.  No allocation happens in the call.  With the norm and
 * RoPE fused into the GEMM (d_qk 64, 96, 128) the forward needs only the x
 * amax partials (at most 1 KiB); a call that would need more (other head
 * widths, whose pre-norm rows pass through the workspace) returns
 * FPR_ERR_SCRATCH before anything is launched.  Every call on one device
 * shares that device's array, and nothing in it needs to start at zero:
 * calls that overlap on one device (other streams, other threads) race on
 * it and must be ordered by the caller.  The first call on a device looks
 * up the array's address there (hipGetSymbolAddress). */
FPR_API int qkv_forward_noalloc(const fpr_dims* dims, int32_t n_seq, int32_t seq_len,
                const uint16_t* x, const fpr_weight_cache* cache,
                uint16_t* q, uint16_t* k, uint16_t* v,
                void* saved, size_t saved_bytes, void* stream);

/* Bytes of the fixed scratch qkv_forward_noalloc uses. */
FPR_API size_t fpr_noalloc_scratch_bytes(void);

/* Step 3, the backward of step 2 ("Reduced-width QK and packed FP8
 * attention", Changes: the FP8 coverage extends to the backward GEMMs;
 * "Where the eight seconds were hiding", The inventory: the backward reads
 * the cached transposed weight view instead of rebuilding it).  The
 * norm/RoPE backward gives the packed gradient dQKV from q, k, the saved
 * 1/rms and dq, dk, dv (with u = R_{-p} q the normalised row, the pre-norm
 * gradient is rho * R_{-p}(dq - q <q,dq> / d_qk)); then dX through the
 * cached W_packed codes and dW = x^T dQKV, quantisers treated as identity.
 *   q, k:   the matching qkv_forward's q and k outputs, unmodified
 *   dq, dk: [n_seq][H][seq_len][qk_stride] bf16 upstream gradients (only
 *           the first d_qk columns of each row, of q and k too, are read)
 *   dv:     [n_seq][H][seq_len][d_v]  bf16
 *   saved:  the buffer filled by the matching qkv_forward
 *   dx:     [T][D] bf16 out
 *   dwq: [D][H*d_qk] fp32 out (row stride ldq), dwk likewise, dwv [D][H*d_v].
 * With dims->bwd_passes = 2 the norm/RoPE backward runs twice instead of
 * writing dQK (its amax first, then straight into the gradient codes), and
 * the workspace holds no dQK; the outputs are the same bit for bit. */
FPR_API int qkv_backward(const fpr_dims* dims, int32_t n_seq, int32_t seq_len,
                 const uint16_t* q, const uint16_t* k,
                 const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                 const void* saved, size_t saved_bytes,
                 const fpr_weight_cache* cache,
                 uint16_t* dx,
                 float* dwq, int64_t ldq,
                 float* dwk, int64_t ldk,
                 float* dwv, int64_t ldv,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/* Human-readable text of an FPR_* return code (static storage). */
FPR_API const char* fpr_status_string(int code);

/* ---------------------------------------------------------------------
 * Verification hooks.  Byte offsets of the intermediates inside `saved`
 * and the forward/backward workspaces, so that tests can check each stage
 * on its own.  The layout is private and may change between versions.
 * Offsets of (size_t)-1 mean "not present".
 *
 * The FP8 copies x8 and g8 are stored blocked, in the order the GEMMs
 * stream them: blocks of act_block_rows rows (tokens) x k_block bytes,
 * block (r / act_block_rows, c / k_block) at index
 * (r / act_block_rows) * ceil(C / k_block) + c / k_block, each block
 * row-major with a k_block-byte row; C is padded to k_block with zero
 * columns, tokens T..tokens_padded-1 are zero rows (the dW GEMM's K tail),
 * and rows from tokens_padded to the end of the last block are undefined.
 * ------------------------------------------------------------------- */
typedef struct fpr_layout {
    int64_t tokens;          /* T */
    int64_t tokens_padded;   /* T rounded up to k_block                     */
    /* in `saved` */
    size_t saved_x8;         /* [T][D] e4m3 blocked                         */
    size_t saved_rho;        /* [2][n_seq][H][S] fp32: 1/rms of each q head
                                row, then of each k head row               */
    size_t saved_x_scales;   /* [2] fp32: s_x, inv_x                        */
    /* in the forward workspace (besides the x amax partials) */
    size_t fwd_qk_pre;       /* [T][2*H*d_qk] bf16 pre-norm Q|K, for head
                                widths without the fused forward; -1 else  */
    /* in the backward workspace */
    size_t bwd_dqkv;         /* [T][2*H*d_qk] bf16, Q|K part of the packed
                                gradient (its V part is dv itself); -1 with
                                bwd_passes = 2, which never writes it        */
    size_t bwd_g_scales;     /* [2] fp32: s_g, inv_g                         */
    size_t bwd_g8;           /* [T][N] e4m3 blocked                          */
    size_t bwd_dw_part;      /* [dw_splits][D][N] fp32 split-K dW partials   */
    int32_t dw_splits;       /* K splits of the dW GEMM at this token count  */
    int32_t bwd_amax_partials; /* amax partials the gradient quantiser folds */
    int32_t k_block;         /* bytes of K per block (128)                   */
    int32_t act_block_rows;  /* rows per block of x8 and g8 (256)            */
} fpr_layout;

FPR_API int fpr_get_layout(const fpr_dims* dims, int64_t tokens, fpr_layout* out);

/* Profiling: while a trace is set on the calling thread, every kernel the
 * calls above launch from that thread whose stage name matches `only` (all
 * kernels when `only` is NULL) is bracketed by hipEventRecord(events[2i]) and
 * hipEventRecord(events[2i+1]) on the call's stream, and its stage name is
 * stored in names[i], for i = count, count+1, ... while count < capacity
 * (and count < FPR_TRACE_MAX).  events are caller-created hipEvent_t handles.
 * Stage names: amax_w, quantize_w, amax_x, quantize_x, amax_wx and
 * quantize_wx (qkv_pack_forward's shared launches), gemm_fwd, norm_rope_fwd,
 * amax_dv, norm_rope_bwd, quantize_g, gemm_dx, gemm_dw, dw_reduce;
 * for the MLP: mlp_amax_w, mlp_quantize_w, mlp_amax_x, mlp_quantize_x,
 * mlp_amax_wx and mlp_quantize_wx (mlp_pack_forward's shared launches),
 * mlp_gemm_up, mlp_quantize_h, mlp_gemm_down, mlp_amax_dy, mlp_quantize_dy,
 * mlp_gemm_dh, mlp_quantize_dpre, mlp_gemm_dx, mlp_gemm_dw1,
 * mlp_dw1_reduce, mlp_gemm_dw2, mlp_dw2_reduce.  fpr_trace_set(NULL) stops
 * tracing.  This is the only per-thread state the library keeps. */
#define FPR_TRACE_MAX 4096
typedef struct fpr_trace {
    void** events;
    int capacity;
    int count;
    const char* only;
    const char* names[FPR_TRACE_MAX];
} fpr_trace;

FPR_API void fpr_trace_set(fpr_trace* trace);

/* ---------------------------------------------------------------------
 * FP8 ReLU^2 MLP ("Reduced-width QK and packed FP8 attention", Changes:
 * FP8 extended to the whole ReLU-squared MLP, forward and backward, both
 * projections and all four backward GEMMs; pre is not kept, and relu(pre)
 * is recovered as sqrt(s_h * dec(h8)) from the squared activation's codes).
 *
 *   forward:  pre = x W1, h = relu(pre)^2, y = h W2
 *             (W1 [D][F], W2 [F][D] fp32; x, y [T][D] bf16)
 *   backward: dh = dy W2^T, dpre = 2 dh relu(pre), dx = dpre W1^T,
 *             dW1 = x^T dpre, dW2 = h^T dy
 *
 * Every GEMM is FP8 e4m3 x e4m3 with fp32 accumulation and one per-tensor
 * scale per operand (the convention of the QKV path): x, W1, h, W2, dy and
 * dpre.  The kept h^2 is h's e4m3 copy h8 (and s_h),
 * which the second projection and dW2 read anyway; the backward takes
 * relu(pre) = sqrt(s_h * dec(h8)).  The h and dpre that are quantised are
 * the fp32 results rounded once to bf16.  Quantisers are treated as the
 * identity in the backward.  The conventions of the QKV calls above hold
 * (caller-owned device memory, no allocation or synchronisation, outputs
 * overwritten, argument errors before any launch, 16-byte alignment).
 * Supported shapes: d_model % 64 == 0, d_ff % 64 == 0, both <= 65536, and
 * 1 <= T <= 2^24.
 * ------------------------------------------------------------------- */
typedef struct fpr_mlp_dims {
    int32_t d_model;      /* D */
    int32_t d_ff;         /* F, the hidden width (3072 for D = 768) */
    int32_t grad_format;  /* FPR_FORMAT_E4M3 (0) or FPR_FORMAT_E5M2: the format
                             of the backward's gradient codes dy8 and dpre8 */
} fpr_mlp_dims;

/* The cached FP8 views of W1 and W2, rebuilt by mlp_pack_quantize_weights
 * after every update of the fp32 weights.  Caller-owned device buffers. */
typedef struct fpr_mlp_cache {
    uint8_t* w1;       /* [D][F] e4m3 (read by dX = dpre W1^T)           */
    uint8_t* w1_t;     /* [F][D] e4m3 (read by the first projection)     */
    uint8_t* w2;       /* [F][D] e4m3 (read by dh = dy W2^T)             */
    uint8_t* w2_t;     /* [D][F] e4m3 (read by the second projection)    */
    float* scales;     /* [4] fp32: s_w1, inv_w1, s_w2, inv_w2            */
    int32_t* status;   /* [1] FPR_STATUS_* bits; pack resets it           */
} fpr_mlp_cache;

/* Bytes of workspace (FPR_CALL_PACK / _FORWARD / _BACKWARD, and
 * FPR_CALL_PACK_FORWARD for mlp_pack_forward) and of the
 * saved buffer (x8, h8 and their scales, which must stay alive and
 * unmodified from mlp_forward to mlp_backward) for T = tokens; 0 for
 * invalid dims or token counts. */
FPR_API size_t fpr_mlp_workspace_bytes(const fpr_mlp_dims* dims, int64_t tokens, int which);
FPR_API size_t fpr_mlp_saved_bytes(const fpr_mlp_dims* dims, int64_t tokens);

/* Quantise W1 [D][F] (row stride ld1 elements) and W2 [F][D] (ld2) with one
 * scale each, both layouts of each from one read of it; resets
 * cache->status, then sets FPR_STATUS_W_NONFINITE if either had a NaN/Inf. */
FPR_API int mlp_pack_quantize_weights(const fpr_mlp_dims* dims,
                              const float* w1, int64_t ld1,
                              const float* w2, int64_t ld2,
                              const fpr_mlp_cache* cache,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* x [T][D] bf16 -> y [T][D] bf16; fills `saved` for mlp_backward.  Sets
 * FPR_STATUS_X_NONFINITE for a NaN/Inf in x, FPR_STATUS_H_NONFINITE for one
 * in h. */
FPR_API int mlp_forward(const fpr_mlp_dims* dims, int64_t tokens,
                const uint16_t* x, const fpr_mlp_cache* cache, uint16_t* y,
                void* saved, size_t saved_bytes,
                void* workspace, size_t workspace_bytes,
                void* stream);

/* mlp_pack_quantize_weights then mlp_forward, for a step that packs fresh
 * weights before its forward ("Reduced-width QK and packed FP8 attention",
 * Changes: the MLP's forward and backward in FP8, its weights changing
 * every step): the same results bit for bit (the cache with its status
 * word, saved, y), with the amax of W1, W2 and x in one launch and their
 * three quantisers in the next.  Arguments, ownership and errors as in the
 * two calls (every check of both is made before the first launch); the
 * workspace is fpr_mlp_workspace_bytes(dims, T, FPR_CALL_PACK_FORWARD)
 * bytes. */
FPR_API int mlp_pack_forward(const fpr_mlp_dims* dims,
                const float* w1, int64_t ld1, const float* w2, int64_t ld2,
                const fpr_mlp_cache* cache, int64_t tokens,
                const uint16_t* x, uint16_t* y,
                void* saved, size_t saved_bytes,
                void* workspace, size_t workspace_bytes, void* stream);

/* dy [T][D] bf16 -> dx [T][D] bf16, dW1 [D][F] fp32 (row stride ld1),
 * dW2 [F][D] fp32 (ld2).  Sets FPR_STATUS_G_NONFINITE for a NaN/Inf in dy,
 * FPR_STATUS_H_NONFINITE for one in dpre. */
FPR_API int mlp_backward(const fpr_mlp_dims* dims, int64_t tokens,
                 const uint16_t* dy, const void* saved, size_t saved_bytes,
                 const fpr_mlp_cache* cache, uint16_t* dx,
                 float* dw1, int64_t ld1, float* dw2, int64_t ld2,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/* Offsets of the MLP's intermediates, for stage-wise tests (blocked FP8
 * layout as for fpr_layout). */
typedef struct fpr_mlp_layout {
    int64_t tokens, tokens_padded;
    size_t saved_x8;          /* [T][D] e4m3 blocked                     */
    size_t saved_h8;          /* [T][F] e4m3 blocked, the stored h       */
    size_t saved_x_scales;    /* [2] fp32: s_x, inv_x                    */
    size_t saved_h_scales;    /* [2] fp32: s_h, inv_h                    */
    size_t fwd_h;             /* [T][F] bf16 relu(pre)^2                 */
    size_t bwd_dy8;           /* [T][D] e4m3 blocked                     */
    size_t bwd_dy_scales;     /* [2] fp32                                */
    size_t bwd_dpre;          /* [T][F] bf16                             */
    size_t bwd_dpre8;         /* [T][F] e4m3 blocked                     */
    size_t bwd_dpre_scales;   /* [2] fp32                                */
    size_t bwd_dw_part;       /* split-K dW partials                     */
    int32_t dw1_splits, dw2_splits;
} fpr_mlp_layout;

FPR_API int fpr_mlp_get_layout(const fpr_mlp_dims* dims, int64_t tokens, fpr_mlp_layout* out);

/* Encode n fp32 values as e4m3(in[i] * inv_scale) with the library's device
 * encoder (no amax; the caller supplies the scale).  For exhaustive tests of
 * the encoder.  in/out are device pointers, 16-byte aligned, n % 16 == 0. */
FPR_API int fpr_e4m3_encode(const float* in, int64_t n, float inv_scale, uint8_t* out,
                    void* stream);

/* The same for the device's e5m2 encoder (saturating at +-57344). */
FPR_API int fpr_e5m2_encode(const float* in, int64_t n, float inv_scale, uint8_t* out,
                    void* stream);

/* ---------------------------------------------------------------------
 * Measurement hooks: the device's practical ceilings, for holding the
 * kernels above against measured limits next to the published peaks.
 * All pointers are device pointers, 16-byte aligned; `blocks` is the grid.
 *   fpr_probe_copy: streaming copy of `bytes` (multiple of 16) src -> dst
 *                   (counts 2 * bytes of HBM traffic);
 *   fpr_probe_read: streaming read of `bytes`, one word per block to out;
 *   fpr_probe_mfma: blocks of 8 waves, each `iters` rounds of 4 independent
 *                   FP8 32x32x64 MFMAs on register operands, one float per
 *                   wave to out[blocks * 8]; returns the FLOP it does (or
 *                   -FPR_ERR_* on an error).
 * ------------------------------------------------------------------- */
FPR_API int fpr_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream);
FPR_API int fpr_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks,
                           void* stream);
FPR_API int64_t fpr_probe_mfma(int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FPR_H */
