// Host-side launchers of the attention kernels (internal to libfa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

constexpr float kLog2eHost = 1.4426950408889634f;

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int BH, N, d;
    float scale;      // signed softmax scale
    float c;          // |scale| * log2(e)
    uint32_t qsign;   // 0x80008000 when scale < 0 (bf16 path negates Q), else 0
    int causal;
    const uint8_t* mask;
    int nb;           // ceil(N / 128)
    // local window and ALiBi: key j allowed for query i iff i - wl <= j <= i + wr
    // (negative = unbounded); score += -slopes[h] |i - j| (slopes may be null)
    int H, wl, wr;
    const float* slopes;
    hipStream_t stream;
    bool variant() const { return wl >= 0 || wr >= 0 || slopes != nullptr; }
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int BH, N, d;
    float scale;      // signed softmax scale
    int causal;
    const uint8_t* mask;
    int nb;
    float* ws_D;      // [BH*N] fp32: D_i = rowsum(dO o O)
    float* ws_lse2;   // [BH*N] fp32: lse in log2 units (+inf for rows without keys)
    int H, wl, wr;    // local window and ALiBi, as in FwdArgs
    const float* slopes;
    hipStream_t stream;
    bool variant() const { return wl >= 0 || wr >= 0 || slopes != nullptr; }
};

// Decode over a paged KV cache (see fa_decode_paged in fa.h).
struct DecArgs {
    const void* q;          // bf16 [B][H][Nq][d]
    const void* k_cache;    // bf16 [num_pages][page_size][Hkv][d]
    const void* v_cache;
    const int* block_table; // [B][max_pages]
    const int* seqlens;     // [B]
    void* o;                // bf16 [B][H][Nq][d]
    float* lse;             // [B][H][Nq]
    int B, H, Hkv, Nq, d;
    int num_pages, page_size, max_pages;
    int causal;
    float c;                // |scale| * log2(e)
    uint32_t qsign;         // 0x80008000 when scale < 0 (Q negated), else 0
    int n_parts, kpp;       // key ranges per (sequence, KV head, query group) and keys per range
    float* ws_o;            // [B*H*Nq][n_parts][d] fp32 (n_parts > 1)
    float* ws_ml;           // [B*H*Nq][n_parts][2] fp32: max (log2 units), sum
    hipStream_t stream;
};

// FP8 block quantization (see fa_fp8_quantize in fa.h).
struct F8QuantArgs {
    const void* x;          // bf16 [BH][N][d]
    uint8_t* codes;         // [BH][N][d] E4M3
    int8_t* exps;           // [BH][ceil(N/64)] block exponents
    int BH, N, d;
    const float* signs;     // [d] +-1 or null (incoherent map)
    int k_side;             // 1: times 1/d (the K side of the map)
    hipStream_t stream;
};

// FP8 forward (see fa_fwd_fp8 in fa.h).
struct F8FwdArgs {
    const uint8_t* q;
    const int8_t* qe;
    const uint8_t* k;
    const int8_t* ke;
    const uint8_t* v;
    const int8_t* ve;
    void* o;                // bf16 [BH][N][d]
    float* lse;
    int BH, N, d, causal;
    float c;                // |scale| * log2(e)
    uint32_t qsign;         // 0x80808080 when scale < 0 (Q codes negated), else 0
    hipStream_t stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);  // dq_first then main (= prep, main, dq)
hipError_t launch_bwd_prep_bf16(const BwdArgs& a);
hipError_t launch_bwd_main_bf16(const BwdArgs& a);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a);
hipError_t launch_bwd_dq_first_bf16(const BwdArgs& a);  // dQ plus the preprocessing (needs o, lse)
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_decode_bf16(const DecArgs& a);
hipError_t launch_fp8_quantize(const F8QuantArgs& a);
hipError_t launch_fwd_fp8(const F8FwdArgs& a);

// Debug self-check flags of the bf16 kernels' translation units (always 0
// unless built with FA_DEBUG_CHECK); synchronous, `clear` resets them.
unsigned debug_flags_fwd_w64(bool clear);
unsigned debug_flags_fwd_w96(bool clear);
unsigned debug_flags_fwd_w192(bool clear);
unsigned debug_flags_f32(bool clear);
unsigned debug_flags_decode(bool clear);
unsigned debug_flags_fp8(bool clear);
unsigned debug_flags_fwd_w128(bool clear);
unsigned debug_flags_fwd_w256(bool clear);
unsigned debug_flags_bwd(bool clear);

}  // namespace fa
