// C ABI of libfa.so: argument validation, workspace layout and dispatch.
// The contract (layouts, ownership, errors) is stated in include/fa.h.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxMaskN = 4194304;
constexpr int kMaxMaskNBwd = 524288;  // the backward keeps its block-row list in LDS beside its tiles
constexpr int kMaxHead = 128;         // head size limit of the backward and of the fp32 path
constexpr int kMaxHeadFwd = 256;      // ... of the bf16 forward

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Whether the product of the (positive) factors is below `limit`, computed
// without overflow: each partial product stays at most `limit`.
bool prod_below(long long limit, std::initializer_list<long long> factors) {
    long long t = 1;
    for (long long x : factors) {
        if (x <= 0) return false;
        if (t > (limit - 1) / x) return false;
        t *= x;
    }
    return t < limit;
}

// Half-open byte ranges [p, p+n) overlap?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Head sizes a path supports: a multiple of 16 up to `max_d`, or (max_d = 0)
// exactly 64 or 128.
int check_sizes(int B, int H, int N, int d, float scale, const uint8_t* mask, int max_d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!prod_below(1LL << 31, {B, H, N, d})) return FA_ERR_INVALID_ARG;
    if (max_d == 0 ? (d != 64 && d != 128) : (d % 16 != 0 || d > max_d)) return FA_ERR_UNSUPPORTED;
    if (mask && N > kMaxMaskN) return FA_ERR_UNSUPPORTED;
    // the bf16 kernels address one head with 32-bit byte offsets and may form
    // offsets up to a few hundred rows past N (reads there fall outside the
    // head's range and return zero): keep that below 2^32
    if ((long long)(N + 256) * d * 2 >= (1LL << 32)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// window / ALiBi options: NULL = none; the slopes pointer must be 4-byte aligned
int check_variant(const fa_variant* var) {
    if (var && var->alibi_slopes && ((uintptr_t)var->alibi_slopes & 3)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

template <typename Args>
void set_variant(Args& a, int H, const fa_variant* var) {
    a.H = H;
    a.wl = (var && var->window_left >= 0) ? var->window_left : -1;
    a.wr = (var && var->window_right >= 0) ? var->window_right : -1;
    a.slopes = var ? var->alibi_slopes : nullptr;
}

template <typename T>
int fwd_common(const T* q, const T* k, const T* v, T* o, float* lse, int B, int H, int N, int d, float scale,
               int causal, const uint8_t* mask, const fa_variant* var, void* stream, bool bf16) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    int st = check_sizes(B, H, N, d, scale, mask, bf16 ? kMaxHeadFwd : kMaxHead);
    if (st != FA_OK) return st;
    // the 256-wide tiles leave room for a block-row list of at most 4096 entries
    if (mask && d > kMaxHead && N > kMaxMaskNBwd) return FA_ERR_UNSUPPORTED;
    st = check_variant(var);
    if (st != FA_OK) return st;
    const size_t tb = (size_t)B * H * N * d * sizeof(T), lb = (size_t)B * H * N * sizeof(float);
    if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) || overlap(lse, lb, o, tb) ||
        overlap(lse, lb, q, tb) || overlap(lse, lb, k, tb) || overlap(lse, lb, v, tb))
        return FA_ERR_INVALID_ARG;
    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.BH = B * H; a.N = N; a.d = d;
    a.scale = scale;
    a.c = fabsf(scale) * fa::kLog2eHost;
    a.qsign = (bf16 && scale < 0.f) ? 0x80008000u : 0u;
    a.causal = causal;
    a.mask = mask;
    a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
    set_variant(a, H, var);
    a.stream = (hipStream_t)stream;
    hipError_t e = bf16 ? fa::launch_fwd_bf16(a) : fa::launch_fwd_f32(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

enum Stage { kAll = 0, kPrep = 1, kMain = 2, kDq = 3, kDqFirst = 4 };

// Validates and enqueues the backward (or one stage of it).  Tensors a stage
// does not use may be NULL and are not checked.
template <typename T>
int bwd_common(const T* q, const T* k, const T* v, const T* o, const T* dO, const float* lse, T* dq, T* dk, T* dv,
               int B, int H, int N, int d, float scale, int causal, const uint8_t* mask, const fa_variant* var,
               void* ws, size_t ws_bytes, void* stream, bool bf16, Stage stage) {
    const bool use_qkv = stage != kPrep;
    const bool use_o = stage == kAll || stage == kPrep || stage == kDqFirst;
    const bool use_lse = stage == kAll || stage == kPrep || stage == kDqFirst;
    const bool use_do = true;
    const bool use_dq = stage == kAll || stage == kDq || stage == kDqFirst;
    const bool use_dkdv = stage == kAll || stage == kMain;
    if (use_qkv && (!q || !k || !v)) return FA_ERR_INVALID_ARG;
    if (use_lse && !lse) return FA_ERR_INVALID_ARG;
    if (use_o && !o) return FA_ERR_INVALID_ARG;
    if (use_do && !dO) return FA_ERR_INVALID_ARG;
    if (use_dq && !dq) return FA_ERR_INVALID_ARG;
    if (use_dkdv && (!dk || !dv)) return FA_ERR_INVALID_ARG;
    const void* all[] = {q, k, v, o, dO, dq, dk, dv};
    for (const void* p : all)
        if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
    if (lse && ((uintptr_t)lse & 3)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    int st = check_sizes(B, H, N, d, scale, mask, kMaxHead);
    if (st != FA_OK) return st;
    st = check_variant(var);
    if (st != FA_OK) return st;
    if (mask && N > kMaxMaskNBwd) return FA_ERR_UNSUPPORTED;
    const size_t tb = (size_t)B * H * N * d * sizeof(T), lb = (size_t)B * H * N * sizeof(float);
    const void* ins[] = {q, k, v, o, dO};
    void* outs[] = {dq, dk, dv};
    for (void* x : outs) {
        if (!x) continue;
        for (const void* y : ins)
            if (y && overlap(x, tb, y, tb)) return FA_ERR_INVALID_ARG;
        if (lse && overlap(x, tb, lse, lb)) return FA_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 3; i++)
        for (int j = i + 1; j < 3; j++)
            if (outs[i] && outs[j] && overlap(outs[i], tb, outs[j], tb)) return FA_ERR_INVALID_ARG;
    const size_t need = fa_bwd_workspace_size(B, H, N, d);
    if (!ws || ws_bytes < need || ((uintptr_t)ws % kAlign) != 0) return FA_ERR_WORKSPACE;
    for (void* x : outs)
        if (x && overlap(x, tb, ws, need)) return FA_ERR_INVALID_ARG;
    for (const void* y : ins)
        if (y && overlap(ws, need, y, tb)) return FA_ERR_INVALID_ARG;
    if (lse && overlap(ws, need, lse, lb)) return FA_ERR_INVALID_ARG;
    fa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.BH = B * H; a.N = N; a.d = d;
    a.scale = scale;
    a.causal = causal;
    a.mask = mask;
    a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
    const size_t vec_bytes = align_up((size_t)B * H * N * sizeof(float));
    a.ws_D = (float*)ws;
    a.ws_lse2 = (float*)((char*)ws + vec_bytes);
    set_variant(a, H, var);
    a.stream = (hipStream_t)stream;
    hipError_t e;
    if (!bf16) e = fa::launch_bwd_f32(a);
    else if (stage == kPrep) e = fa::launch_bwd_prep_bf16(a);
    else if (stage == kMain) e = fa::launch_bwd_main_bf16(a);
    else if (stage == kDq) e = fa::launch_bwd_dq_bf16(a);
    else if (stage == kDqFirst) e = fa::launch_bwd_dq_first_bf16(a);
    else e = fa::launch_bwd_bf16(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Static scratch of fa_bwd_noalloc: the two fp32 row vectors of the backward
// (D and lse in log2 units) for at most FA_NOALLOC_MAX_ROWS rows, laid out as
// the fa_bwd workspace.  `scratch` names the host-side stand-in of the device
// array; the device address comes from hipGetSymbolAddress, once per device,
// and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = 2 * (size_t)FA_NOALLOC_MAX_ROWS * sizeof(float);
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (resolved on the
// first call on that device, with it current).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FA_ERR_HIP;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return FA_OK;
}
static_assert(2 * ((FA_NOALLOC_MAX_ROWS * sizeof(float) + kAlign - 1) / kAlign * kAlign) <= kScratchBytes,
              "the scratch must hold the backward workspace of FA_NOALLOC_MAX_ROWS rows");

}  // namespace

extern "C" {

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
              float scale, int causal, const uint8_t* blockmask, const fa_variant* variant, void* stream) {
    return fwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, B,
                                H, N, d, scale, causal, blockmask, variant, stream, true);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, const uint8_t* blockmask, void* stream) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, nullptr, stream);
}

int fa_fwd_f32_ex(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
                  float scale, int causal, const uint8_t* blockmask, const fa_variant* variant, void* stream) {
    return fwd_common<float>(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, variant, stream, false);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, const uint8_t* blockmask, void* stream) {
    return fa_fwd_f32_ex(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, nullptr, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || !prod_below(1LL << 31, {B, H, N, d})) return 0;
    const size_t rows = (size_t)B * H * N;
    return 2 * align_up(rows * sizeof(float));
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
              void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
              const fa_variant* variant, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                                (const uint16_t*)dO, lse, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, B, H, N, d,
                                scale, causal, blockmask, variant, workspace, workspace_bytes, stream, true, kAll);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
           void* workspace, size_t workspace_bytes, void* stream) {
    return fa_bwd_ex(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, blockmask, nullptr, workspace,
                     workspace_bytes, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, const fa_variant* variant, void* stream) {
    if (B >= 1 && H >= 1 && N >= 1 && !prod_below((long long)FA_NOALLOC_MAX_ROWS + 1, {B, H, N}))
        return FA_ERR_SCRATCH;
    void* ws = nullptr;
    const int st = scratch_address(&ws);
    if (st != FA_OK) return st;
    return bwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                                (const uint16_t*)dO, lse, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, B, H, N, d,
                                scale, causal, blockmask, variant, ws, kScratchBytes, stream, true, kAll);
}

int fa_bwd_prep(const void* o, const void* dO, const float* lse, int B, int H, int N, int d, void* workspace,
                size_t workspace_bytes, void* stream) {
    return bwd_common<uint16_t>(nullptr, nullptr, nullptr, (const uint16_t*)o, (const uint16_t*)dO, lse,
                                nullptr, nullptr, nullptr, B, H, N, d, 1.0f, 0, nullptr, nullptr, workspace,
                                workspace_bytes, stream, true, kPrep);
}

int fa_bwd_main_ex(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, const uint8_t* blockmask, const fa_variant* variant,
                   void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, nullptr,
                                (const uint16_t*)dO, nullptr, nullptr, (uint16_t*)dk, (uint16_t*)dv, B, H, N, d, scale,
                                causal, blockmask, variant, workspace, workspace_bytes, stream, true, kMain);
}

int fa_bwd_main(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv, int B, int H, int N,
                int d, float scale, int causal, const uint8_t* blockmask, void* workspace, size_t workspace_bytes,
                void* stream) {
    return fa_bwd_main_ex(q, k, v, dO, dk, dv, B, H, N, d, scale, causal, blockmask, nullptr, workspace,
                          workspace_bytes, stream);
}

int fa_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO, void* dq, int B, int H, int N, int d,
                 float scale, int causal, const uint8_t* blockmask, const fa_variant* variant, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return bwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, nullptr,
                                (const uint16_t*)dO, nullptr, (uint16_t*)dq, nullptr, nullptr, B, H, N, d, scale,
                                causal, blockmask, variant, workspace, workspace_bytes, stream, true, kDq);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, void* dq, int B, int H, int N, int d,
              float scale, int causal, const uint8_t* blockmask, void* workspace, size_t workspace_bytes,
              void* stream) {
    return fa_bwd_dq_ex(q, k, v, dO, dq, B, H, N, d, scale, causal, blockmask, nullptr, workspace, workspace_bytes,
                        stream);
}

int fa_bwd_dq_first_ex(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                       void* dq, int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
                       const fa_variant* variant, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_common<uint16_t>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)o,
                                (const uint16_t*)dO, lse, (uint16_t*)dq, nullptr, nullptr, B, H, N, d, scale,
                                causal, blockmask, variant, workspace, workspace_bytes, stream, true, kDqFirst);
}

int fa_bwd_dq_first(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                    void* dq, int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return fa_bwd_dq_first_ex(q, k, v, o, dO, lse, dq, B, H, N, d, scale, causal, blockmask, nullptr, workspace,
                              workspace_bytes, stream);
}

int fa_bwd_f32_ex(const float* q, const float* k, const float* v, const float* o, const float* dO, const float* lse,
                  float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* blockmask, const fa_variant* variant, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return bwd_common<float>(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, blockmask, variant,
                             workspace, workspace_bytes, stream, false, kAll);
}

int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dO, const float* lse,
               float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
               const uint8_t* blockmask, void* workspace, size_t workspace_bytes, void* stream) {
    return fa_bwd_f32_ex(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, blockmask, nullptr, workspace,
                         workspace_bytes, stream);
}

// Key ranges of the decode: about one wave per resident wave slot of the chip
// (256 CUs x 8) when every sequence is full, at least 256 keys (eight tiles)
// per range; kpp is a multiple of the 32-key tile.
static void decode_plan(int B, int H, int H_kv, int Nq, int page_size, int max_pages, int& n_parts, int& kpp) {
    const long long cap = (long long)max_pages * page_size;
    const long long groups = (long long)B * H_kv * (((long long)(H / H_kv) * Nq + 15) / 16);
    const long long want = (2048 + groups - 1) / groups;
    const long long most = (cap + 255) / 256;
    long long parts = want < 1 ? 1 : want;
    if (parts > most) parts = most;
    long long per = (cap + parts - 1) / parts;
    per = (per + 31) / 32 * 32;
    kpp = (int)per;
    n_parts = (int)((cap + per - 1) / per);
}

static int decode_check(int B, int H, int H_kv, int Nq, int d, int page_size, int max_pages) {
    if (B < 1 || H < 1 || H_kv < 1 || Nq < 1 || d < 1 || page_size < 1 || max_pages < 1) return FA_ERR_INVALID_ARG;
    if (H % H_kv != 0) return FA_ERR_INVALID_ARG;
    if (!prod_below(1LL << 31, {B, H, Nq, d})) return FA_ERR_INVALID_ARG;
    if (!prod_below(1LL << 31, {max_pages, page_size})) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (page_size % 32 != 0) return FA_ERR_UNSUPPORTED;
    if (!prod_below(1LL << 32, {page_size, H_kv, d, 2})) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

size_t fa_decode_workspace_size(int B, int H, int H_kv, int Nq, int d, int page_size, int max_pages) {
    if (decode_check(B, H, H_kv, Nq, d, page_size, max_pages) != FA_OK) return 0;
    int n_parts, kpp;
    decode_plan(B, H, H_kv, Nq, page_size, max_pages, n_parts, kpp);
    if (n_parts == 1) return 0;
    const size_t rows = (size_t)B * H * Nq * n_parts;
    return align_up(rows * d * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* seqlens, void* o, float* lse, int B, int H, int H_kv, int Nq, int d,
                    int num_pages, int page_size, int max_pages, float scale, int causal, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seqlens || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || ((uintptr_t)lse & 3) ||
        ((uintptr_t)block_table & 3) || ((uintptr_t)seqlens & 3))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || num_pages < 1) return FA_ERR_INVALID_ARG;
    int st = decode_check(B, H, H_kv, Nq, d, page_size, max_pages);
    if (st != FA_OK) return st;
    const size_t qb = (size_t)B * H * Nq * d * 2, lb = (size_t)B * H * Nq * 4;
    const size_t cb = (size_t)num_pages * page_size * H_kv * d * 2;
    const size_t tb = (size_t)B * max_pages * 4, sb = (size_t)B * 4;
    const void* ins[] = {q, k_cache, v_cache};
    const size_t in_bytes[] = {qb, cb, cb};
    for (int i = 0; i < 3; i++)
        if (overlap(o, qb, ins[i], in_bytes[i]) || overlap(lse, lb, ins[i], in_bytes[i])) return FA_ERR_INVALID_ARG;
    if (overlap(o, qb, lse, lb) || overlap(o, qb, block_table, tb) || overlap(o, qb, seqlens, sb) ||
        overlap(lse, lb, block_table, tb) || overlap(lse, lb, seqlens, sb))
        return FA_ERR_INVALID_ARG;
    fa::DecArgs a;
    decode_plan(B, H, H_kv, Nq, page_size, max_pages, a.n_parts, a.kpp);
    const size_t need = fa_decode_workspace_size(B, H, H_kv, Nq, d, page_size, max_pages);
    a.ws_o = nullptr;
    a.ws_ml = nullptr;
    if (need > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0) return FA_ERR_WORKSPACE;
        const void* all[] = {q, k_cache, v_cache, o, lse, block_table, seqlens};
        const size_t all_bytes[] = {qb, cb, cb, qb, lb, tb, sb};
        for (int i = 0; i < 7; i++)
            if (overlap(workspace, need, all[i], all_bytes[i])) return FA_ERR_INVALID_ARG;
        const size_t rows = (size_t)B * H * Nq * a.n_parts;
        a.ws_o = (float*)workspace;
        a.ws_ml = (float*)((char*)workspace + align_up(rows * d * sizeof(float)));
    }
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
    a.block_table = block_table; a.seqlens = seqlens;
    a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.Hkv = H_kv; a.Nq = Nq; a.d = d;
    a.num_pages = num_pages; a.page_size = page_size; a.max_pages = max_pages;
    a.causal = causal;
    // scale 0 would turn -inf * 0 into NaN; any c below 1e-30 gives the same fp32 probabilities
    a.c = fmaxf(fabsf(scale) * fa::kLog2eHost, 1e-30f);
    a.qsign = scale < 0.f ? 0x80008000u : 0u;
    a.stream = (hipStream_t)stream;
    return fa::launch_decode_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fp8_quantize(const void* x, uint8_t* codes, int8_t* exps, int B, int H, int N, int d, const float* signs,
                    int k_side, void* stream) {
    if (!x || !codes || !exps) return FA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(codes) || (signs && ((uintptr_t)signs & 3))) return FA_ERR_INVALID_ARG;
    if (k_side != 0 && k_side != 1) return FA_ERR_INVALID_ARG;
    const int st = check_sizes(B, H, N, d, 1.0f, nullptr, 0);
    if (st != FA_OK) return st;
    const size_t xb = (size_t)B * H * N * d * 2, cb = (size_t)B * H * N * d;
    const size_t eb = (size_t)B * H * ((N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK);
    if (overlap(codes, cb, x, xb) || overlap(exps, eb, x, xb) || overlap(exps, eb, codes, cb)) return FA_ERR_INVALID_ARG;
    if (signs && (overlap(codes, cb, signs, (size_t)d * 4) || overlap(exps, eb, signs, (size_t)d * 4)))
        return FA_ERR_INVALID_ARG;
    fa::F8QuantArgs a;
    a.x = x; a.codes = codes; a.exps = exps;
    a.BH = B * H; a.N = N; a.d = d;
    a.signs = signs; a.k_side = k_side;
    a.stream = (hipStream_t)stream;
    return fa::launch_fp8_quantize(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const uint8_t* q, const int8_t* q_exps, const uint8_t* k, const int8_t* k_exps, const uint8_t* v,
               const int8_t* v_exps, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
               void* stream) {
    if (!q || !q_exps || !k || !k_exps || !v || !v_exps || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    const int st = check_sizes(B, H, N, d, scale, nullptr, 0);
    if (st != FA_OK) return st;
    const size_t cb = (size_t)B * H * N * d, ob = cb * 2, lb = (size_t)B * H * N * 4;
    const size_t eb = (size_t)B * H * ((N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK);
    const void* ins[] = {q, k, v, q_exps, k_exps, v_exps};
    const size_t in_bytes[] = {cb, cb, cb, eb, eb, eb};
    for (int i = 0; i < 6; i++)
        if (overlap(o, ob, ins[i], in_bytes[i]) || overlap(lse, lb, ins[i], in_bytes[i])) return FA_ERR_INVALID_ARG;
    if (overlap(o, ob, lse, lb)) return FA_ERR_INVALID_ARG;
    fa::F8FwdArgs a;
    a.q = q; a.qe = q_exps; a.k = k; a.ke = k_exps; a.v = v; a.ve = v_exps;
    a.o = o; a.lse = lse;
    a.BH = B * H; a.N = N; a.d = d; a.causal = causal;
    a.c = fmaxf(fabsf(scale) * fa::kLog2eHost, 1e-30f);
    a.qsign = scale < 0.f ? 0x80808080u : 0u;
    a.stream = (hipStream_t)stream;
    return fa::launch_fwd_fp8(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_INVALID_ARG: return "invalid argument";
        case FA_ERR_UNSUPPORTED: return "unsupported configuration";
        case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case FA_ERR_HIP: return "HIP runtime error while enqueueing";
        case FA_ERR_SCRATCH: return "B*H*N exceeds the static scratch of fa_bwd_noalloc (FA_NOALLOC_MAX_ROWS rows)";
        default: return "unknown status";
    }
}

int fa_version(void) { return FA_VERSION; }

int fa_debug_flags(int clear) {
#ifdef FA_DEBUG_CHECK
    if (hipDeviceSynchronize() != hipSuccess) return -1;
    const unsigned f = fa::debug_flags_fwd_w64(clear) | fa::debug_flags_fwd_w96(clear) |
                       fa::debug_flags_fwd_w128(clear) | fa::debug_flags_fwd_w192(clear) | fa::debug_flags_fwd_w256(clear) |
                       fa::debug_flags_bwd(clear) |
                       fa::debug_flags_f32(clear) | fa::debug_flags_decode(clear) | fa::debug_flags_fp8(clear);
    return f == ~0u ? -1 : (int)f;
#else
    (void)clear;
    return 0;
#endif
}

}  // extern "C"
