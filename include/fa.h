/*
 * fa.h -- C ABI of libfa.so: exact IO-aware softmax attention on AMD MI355X (gfx950).
 *
 * The library computes exact attention, O = softmax(scale * Q K^T [masked]) V,
 * without ever writing the N x N score or probability matrices to HBM: a
 * fused forward kernel tiles Q by rows and K/V by columns, keeps a running
 * row max and row sum (online softmax), rescales an unnormalized output
 * accumulator and divides once at the end ("FlashAttention 深度解析" sections
 * 二 and 四; "FlashAttention原理概览" section 3.1; "FlashAttention: Fast and
 * Memory-Efficient Exact Attention with IO-Awareness" sections 2.3, 2.4, 2.6).
 * The backward recomputes the scores and probabilities tile by tile from the
 * saved per-row logsumexp instead of storing them ("FlashAttention原理概览"
 * section 3.2; IO-Awareness page section 2.5).
 *
 * Definition computed (per batch b, head h, row i):
 *   S_ij  = scale * sum_c q_ic k_jc   (- alibi_slope_h |i - j| with ALiBi, see fa_variant)
 *   allowed(i, j) = (!causal || j <= i) && (blockmask == NULL || blockmask[i/128][j/128] != 0)
 *                   && (inside the local window, if one is given: see fa_variant)
 *   lse_i = log sum_{allowed j} exp(S_ij)         (natural log; -inf if no j is allowed)
 *   O_i   = sum_{allowed j} exp(S_ij - lse_i) v_j (0 if no j is allowed)
 * The causal mask is the lower triangle including the diagonal ("FlashAttention
 * 深度解析" section 五 lists it as built in).  The block mask is the
 * block-sparse variant (IO-Awareness page section 4): a zero entry removes a
 * whole 128 x 128 block and the kernels skip it; causal and block mask combine
 * by intersection.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout    q, k, v, o, dO, dq, dk, dv: [B][H][N][d], row-major, d fastest,
 *           densely packed (element (b,h,i,c) at ((b*H + h)*N + i)*d + c),
 *           base addresses 16-byte aligned (lse: 4-byte aligned).
 *           lse: float [B][H][N].  blockmask: uint8 [nb][nb], nb = ceil(N/128),
 *           row-major, one mask shared by all (b, h).
 * Types     fa_fwd / fa_bwd: bfloat16 tensors (raw 16-bit storage), fp32
 *           accumulation, fp32 softmax statistics, outputs rounded to bfloat16
 *           (round to nearest even).  fa_fwd_f32 / fa_bwd_f32: float tensors.
 * Memory    every pointer is device memory owned by the caller.  The library
 *           never allocates, frees or synchronizes and is re-entrant; its only
 *           host-side state is a per-device cache of the compute-unit count
 *           (read once with hipDeviceGetAttribute, used to size launches).
 *           Outputs must not alias inputs.
 * Streams   `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *           enqueue work and return; results are ready once the stream is
 *           synchronized.  Kernel faults surface at the caller's next sync.
 * Limits    B, H, N >= 1; the head size d a multiple of 16 ("FlashAttention
 *           原理概览" section 3.4) of at most 256 for the bf16 forward and at
 *           most 128 for the backward and the fp32 entry points ("FlashAttention
 *           深度解析" section 五 bounds it by 256; the key-outer backward's LDS
 *           ring does not fit at 256); other values return FA_ERR_UNSUPPORTED;
 *           B*H*N*d < 2^31; (N + 256) * d * 2 < 2^32 (else FA_ERR_UNSUPPORTED:
 *           the kernels address one head with 32-bit byte offsets); scale
 *           finite; with a blockmask, N <= 4194304 (forward, d <= 128),
 *           N <= 524288 (forward with d > 128, and the backward).
 * Errors    arguments are validated before anything is enqueued; on any
 *           error nothing is enqueued and the outputs are untouched.
 *           FA_ERR_HIP reports a failed kernel launch (hipGetLastError).
 * Inputs    NaN/Inf in q, k, v or dO propagate; they are not checked.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, non-finite scale, aliasing, too large */
    FA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. a head size that is not a multiple of 16) */
    FA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than the *_workspace_size() */
    FA_ERR_HIP = 4,         /* the HIP runtime reported an error while enqueueing */
    FA_ERR_SCRATCH = 5      /* fa_bwd_noalloc: B*H*N exceeds FA_NOALLOC_MAX_ROWS */
} fa_status;

#define FA_MASK_BLOCK 128 /* block-mask granularity in rows and columns */
#define FA_VERSION 7

/*
 * Local window and ALiBi, the two further built-in variants "FlashAttention
 * 深度解析" section 五 lists beside the causal mask (the pages give no formula;
 * the definition taken here):
 *   window_left, window_right: key j is allowed for query i only if
 *       i - window_left <= j <= i + window_right; a negative value leaves that
 *       side unbounded.  Intersected with causal and the block mask.
 *   alibi_slopes: device float[H] (4-byte aligned) or NULL; the scaled score of
 *       (i, j) in head h becomes S_ij - alibi_slopes[h] * |i - j|, before the
 *       softmax (lse includes it).
 * The struct itself is read on the host during the call (the caller keeps
 * ownership); passing NULL, or {-1, -1, NULL}, is the plain computation.  The
 * _ex entry points below take it; the backward must get the variant the
 * forward used.
 */
typedef struct fa_variant {
    int window_left;
    int window_right;
    const float* alibi_slopes;
} fa_variant;

/*
 * Forward, bfloat16.  q, k, v: const bf16 [B][H][N][d] (read).  o: bf16
 * [B][H][N][d] (written).  lse: float [B][H][N] (written; natural-log
 * logsumexp of the scaled, masked score row -- the saved statistic the
 * backward needs).  causal: 0 or 1.  blockmask: NULL for dense.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, const uint8_t* blockmask, void* stream);

/* Forward, float32 tensors; same semantics as fa_fwd. */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, const uint8_t* blockmask, void* stream);

/* fa_fwd / fa_fwd_f32 with a local window and/or ALiBi (variant may be NULL).
 * A misaligned alibi_slopes pointer returns FA_ERR_INVALID_ARG. */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
              int d, float scale, int causal, const uint8_t* blockmask, const fa_variant* variant,
              void* stream);
int fa_fwd_f32_ex(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                  int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
                  const fa_variant* variant, void* stream);

/*
 * Bytes of device workspace fa_bwd and fa_bwd_f32 need: two fp32 row vectors
 * per (b, h, i) -- D_i = sum_c dO_ic O_ic and lse_i in log2 units -- each
 * 256-byte aligned (O(N) memory, nothing O(N^2) and no O(N d) accumulator).
 * Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward, bfloat16.  Inputs: q, k, v, o (the forward's output), dO (gradient
 * of the loss w.r.t. o) as bf16 [B][H][N][d]; lse as written by fa_fwd.
 * Outputs: dq, dk, dv bf16 [B][H][N][d] (written, rounded to bf16).  The
 * scores and probabilities are recomputed from q, k and lse; nothing N x N is
 * stored.  workspace: device buffer of at least fa_bwd_workspace_size() bytes,
 * 256-byte aligned, contents ignored on entry and clobbered.  Every gradient is
 * accumulated in fp32 registers by exactly one workgroup (no atomics), so the
 * results are bitwise deterministic.  scale, causal and blockmask must be the
 * ones the forward used.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           int causal, const uint8_t* blockmask, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * The stages of the backward, for callers that want to schedule or time them
 * separately.  Both orders below give exactly fa_bwd's results, bit for bit,
 * on the same stream with the same workspace; fa_bwd itself enqueues the
 * second, which saves the preprocessing pass.
 *   order 1: fa_bwd_prep, fa_bwd_main, fa_bwd_dq;
 *   order 2: fa_bwd_dq_first, fa_bwd_main.
 *   fa_bwd_prep: D_i = sum_c dO_ic O_ic and lse_i * log2(e) into the
 *                workspace.  Reads o, dO, lse.
 *   fa_bwd_main: key-outer pass: recomputes S, P, dP and dS per tile from q, k,
 *                v, dO and the workspace; writes dk and dv (bf16).
 *   fa_bwd_dq:   query-outer pass: recomputes S, P, dP and dS per tile; writes
 *                dq (bf16).  Independent of fa_bwd_main (both need only the
 *                workspace as left by fa_bwd_prep).
 *   fa_bwd_dq_first: fa_bwd_dq that also does fa_bwd_prep's work for its own
 *                rows (same summation order, same bits) and leaves D and
 *                lse * log2(e) in the workspace for fa_bwd_main.  Reads q, k,
 *                v, o, dO, lse; writes dq and the workspace.
 * Validation and error codes as for fa_bwd.
 */
int fa_bwd_prep(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_main(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
                void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, void* dq, int B, int H,
              int N, int d, float scale, int causal, const uint8_t* blockmask, void* workspace,
              size_t workspace_bytes, void* stream);
int fa_bwd_dq_first(const void* q, const void* k, const void* v, const void* o, const void* dO,
                    const float* lse, void* dq, int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* blockmask, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics, kernels and results
 * (bit for bit) as fa_bwd_ex, bfloat16 only.  The backward's two fp32 row
 * vectors live in a static device array of the library (2 * FA_NOALLOC_MAX_ROWS
 * floats, 16 MiB, held on every GPU the library runs on until the process
 * ends); its address is resolved once per device with hipGetSymbolAddress on
 * the first call, which must therefore run with the stream's device current.
 * The call allocates and frees nothing.  Limit: B*H*N <= FA_NOALLOC_MAX_ROWS,
 * else FA_ERR_SCRATCH and nothing is enqueued.  Every call on one GPU shares
 * that array: calls that overlap in time on one GPU (on different streams,
 * or on one stream from several host threads interleaving their stages)
 * race and give wrong gradients; calls serialized on one stream do not.
 * The array needs no clearing: each call writes every entry it reads.
 */
#define FA_NOALLOC_MAX_ROWS 2097152
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                   int causal, const uint8_t* blockmask, const fa_variant* variant, void* stream);

/* Backward, float32 tensors; same semantics as fa_bwd (deterministic). */
int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dO,
               const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
               float scale, int causal, const uint8_t* blockmask, void* workspace,
               size_t workspace_bytes, void* stream);

/* The backward entry points with a local window and/or ALiBi (variant may be
 * NULL); the variant must be the one the forward used.  fa_bwd_prep needs none. */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
              float scale, int causal, const uint8_t* blockmask, const fa_variant* variant,
              void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_main_ex(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
                   const fa_variant* variant, void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO, void* dq, int B, int H,
                 int N, int d, float scale, int causal, const uint8_t* blockmask,
                 const fa_variant* variant, void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dq_first_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                       const float* lse, void* dq, int B, int H, int N, int d, float scale, int causal,
                       const uint8_t* blockmask, const fa_variant* variant, void* workspace,
                       size_t workspace_bytes, void* stream);
int fa_bwd_f32_ex(const float* q, const float* k, const float* v, const float* o, const float* dO,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                  float scale, int causal, const uint8_t* blockmask, const fa_variant* variant,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over a paged KV cache, bfloat16 ("FlashAttention 深度解析" section 五:
 * since version 2.5 FlashAttention reads the KV cache from the paged layout
 * PagedAttention manages; the layout below is the one taken, the pages give
 * none).  For each sequence b, its Nq new queries (the last Nq positions
 * L_b - Nq .. L_b - 1) attend to its L_b cached keys:
 *   q:           const bf16 [B][H][Nq][d]
 *   k_cache,
 *   v_cache:     const bf16 [num_pages][page_size][H_kv][d]: page p holds
 *                page_size consecutive positions of one sequence, every KV head
 *   block_table: const int32 [B][max_pages]: logical page j of sequence b (its
 *                positions j*page_size ..) is physical page block_table[b][j]
 *   seqlens:     const int32 [B]: L_b, 0 <= L_b <= max_pages * page_size
 *   o:           bf16 [B][H][Nq][d] (written); lse: float [B][H][Nq] (written,
 *                natural log; -inf and o = 0 for a query with no key)
 * Query head h reads KV head h / (H / H_kv) (grouped heads; H % H_kv == 0).
 * causal = 1: query i of sequence b sees positions <= L_b - Nq + i; causal = 0:
 * all L_b keys.  block_table and seqlens are device memory read by the
 * kernels: a length outside [0, max_pages * page_size] is clamped into it, and
 * a page index outside [0, num_pages) reads as zeros (its sequence's result is
 * then meaningless, but nothing outside the cache is touched).
 * Limits: d in {64, 128}; page_size a multiple of 32; B*H*Nq*d < 2^31;
 * max_pages * page_size < 2^31; page_size * H_kv * d * 2 < 2^32.
 * workspace: device, 256-byte aligned, at least fa_decode_workspace_size()
 * bytes (0 when one key range covers every sequence: NULL is then allowed).
 * The keys are split into ranges processed in parallel and merged exactly
 * with the running max / sum rule; the result does not depend on the split.
 */
size_t fa_decode_workspace_size(int B, int H, int H_kv, int Nq, int d, int page_size, int max_pages);
int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* seqlens, void* o, float* lse, int B, int H, int H_kv, int Nq, int d,
                    int num_pages, int page_size, int max_pages, float scale, int causal, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * FP8 forward ("FlashAttention 深度解析" section 四: FlashAttention-3's FP8
 * block quantization with incoherent processing; the pages give no formulas,
 * the definitions taken are these).  Format: FP8 E4M3 (OCP E4M3FN: bias 7,
 * largest finite 448, no infinities), the format the gfx950 matrix cores read.
 *
 * fa_fp8_quantize: x bf16 [B][H][N][d] -> codes uint8 [B][H][N][d] and block
 * exponents exps int8 [B][H][ceil(N/FA_FP8_BLOCK)].  Each (b, h) slice is cut
 * into blocks of FA_FP8_BLOCK rows; with signs (device float[d] of +-1, or
 * NULL) every row first goes through the incoherent map x -> H (signs o x), H
 * the Sylvester Hadamard matrix of order d, times 1/d when k_side = 1 (use
 * k_side = 0 for Q, 1 for K, the same signs for both and NULL for V: then
 * Q' K'^T = Q K^T).  A block gets the smallest e with max|x| / 2^e <= 448
 * (e = 0 for an all-zero block, clamped to [-127, 127]) and codes = the nearest
 * E4M3 value of x / 2^e, ties to even.  Deterministic and exact (the map is
 * computed in fp64, where these sums are exact).
 *
 * fa_fwd_fp8: exact-attention forward of the dequantized tensors
 * (code * 2^exp), with both matrix products on the FP8 matrix cores: S = Q K^T
 * from the codes (block exponents applied by the instruction), P rounded to
 * E4M3 (as 2^8 P, P <= 1) for P V; o bf16 [B][H][N][d] and lse float [B][H][N]
 * as fa_fwd.  causal 0 or 1; no block mask or window.  The result differs from
 * exact attention of the dequantized tensors by the rounding of P.
 * Limits as fa_fwd but d in {64, 128}; codes 16-byte aligned.
 */
#define FA_FP8_BLOCK 64
int fa_fp8_quantize(const void* x, uint8_t* codes, int8_t* exps, int B, int H, int N, int d, const float* signs,
                    int k_side, void* stream);
int fa_fwd_fp8(const uint8_t* q, const int8_t* q_exps, const uint8_t* k, const int8_t* k_exps, const uint8_t* v,
               const int8_t* v_exps, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
               void* stream);

/* Static text for a status code (never NULL). */
const char* fa_status_string(int status);

/* FA_VERSION of the loaded library. */
int fa_version(void);

/* Debug self-check ("FlashAttention 深度解析" section 二's invariants of the
 * online softmax): a library built with FA_DEBUG_CHECK (libfa_debug.so, built
 * beside libfa.so) has every attention kernel (bf16 and float32 forward and
 * backward, FP8 forward, paged decode and its merge) record, as bits
 * of a device flag word, a row that saw a finite score but whose sum of
 * weights is not positive (FA_DEBUG_ROW_SUM) and any output element of O,
 * lse, dQ, dK or dV that is NaN or infinite (FA_DEBUG_NON_FINITE; lse = -inf
 * for a row without allowed keys is not flagged).  fa_debug_flags synchronizes
 * the device, returns the bits accumulated since the last clear (clear != 0
 * resets them) or -1 on a HIP error.  The plain library returns 0 and checks
 * nothing.  Meant for debugging runs, not for production calls. */
#define FA_DEBUG_ROW_SUM 1
#define FA_DEBUG_NON_FINITE 2
int fa_debug_flags(int clear);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
