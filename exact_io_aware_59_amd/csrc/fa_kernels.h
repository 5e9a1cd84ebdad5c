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

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);  // the three stages below, in order
hipError_t launch_bwd_prep_bf16(const BwdArgs& a);
hipError_t launch_bwd_main_bf16(const BwdArgs& a);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_decode_bf16(const DecArgs& a);

}  // namespace fa
