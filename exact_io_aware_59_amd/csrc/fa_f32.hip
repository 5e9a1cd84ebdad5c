// fp32 attention on gfx950: a plain, high-precision path for small problems.
//
// Same online-softmax forward and recompute backward as the bf16 kernels, but
// every product is an fp32 FMA on the vector ALUs and every row is owned by
// one thread, so results stay within a few fp32 ulps of exact attention.
// Forward: running max / running sum per key ("FlashAttention 深度解析"
// section 二).  Backward: P recomputed from the saved logsumexp
// ("FlashAttention原理概览" section 3.2), dQ by query-owning threads and
// dK/dV by key-owning threads, so no atomics and deterministic results.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

__device__ __forceinline__ bool allowed(int i, int j, int causal, const uint8_t* mask, int nb, const Variant& var) {
    if (causal && j > i) return false;
    if (mask && !mask[(size_t)(i / kMaskBlock) * nb + (j / kMaskBlock)]) return false;
    if (var.dead(i, j)) return false;
    return true;
}

// window / ALiBi parameters of head bh
__device__ __forceinline__ Variant variant_of(int bh, int H, int wl, int wr, const float* slopes) {
    return Variant{wl, wr, slopes ? slopes[bh % H] * kLog2e : 0.f};
}

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ LSE, int N, float c, int causal,
                                                     const uint8_t* __restrict__ mask, int nb, int H, int wl, int wr,
                                                     const float* __restrict__ slopes) {
    const int bh = blockIdx.y;
    const Variant var = variant_of(bh, H, wl, wr, slopes);
    const int i = blockIdx.x * 64 + threadIdx.x;
    const size_t head = (size_t)bh * N * D;
    const bool row_ok = i < N;
    float q[D], o[D];
#pragma unroll
    for (int e = 0; e < D; e++) {
        q[e] = row_ok ? Q[head + (size_t)i * D + e] : 0.f;
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int kv_end = causal ? min(N, (int)blockIdx.x * 64 + 64) : N;
    const int brow = (blockIdx.x * 64) / kMaskBlock;  // all 64 rows share one mask row
    for (int j = 0; j < kv_end; j++) {
        if (mask && (j % kMaskBlock) == 0 && !mask[(size_t)brow * nb + j / kMaskBlock]) {
            j += kMaskBlock - 1;
            continue;
        }
        const float* kj = K + head + (size_t)j * D;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; e++) s = __builtin_fmaf(q[e], kj[e], s);
        if (!row_ok || !allowed(i, j, causal, mask, nb, var)) continue;
        const float t = __builtin_fmaf(s, c, var.bias2(i, j));
        const float m_new = fmaxf(m, t);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f_hw(m - m_new);
        const float p = exp2f_hw(t - m_new);
        l = l * alpha + p;
        const float* vj = V + head + (size_t)j * D;
#pragma unroll
        for (int e = 0; e < D; e++) o[e] = __builtin_fmaf(p, vj[e], o[e] * alpha);
        m = m_new;
    }
    if (!row_ok) return;
    FA_CHECK(m == -INFINITY || l > 0.f, kDbgRowSum);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < D; e++) {
        O[head + (size_t)i * D + e] = o[e] * inv;
        FA_CHECK(!nonfinite_bits(o[e] * inv), kDbgNonFinite);
    }
    const float lse = l > 0.f ? (m + log2f_hw(l)) * kLn2 : -INFINITY;
    FA_CHECK(lse == -INFINITY || !nonfinite_bits(lse), kDbgNonFinite);
    LSE[(size_t)bh * N + i] = lse;
}

// D_i = sum_c dO_ic O_ic
template <int D>
__global__ __launch_bounds__(256) void rowdot_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                                                         float* __restrict__ Dv, long rows) {
    const long r = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    float acc = 0.f;
    for (int e = 0; e < D; e++) acc = __builtin_fmaf(O[r * D + e], dO[r * D + e], acc);
    Dv[r] = acc;
}

// dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j, one thread per query row
template <int D>
__global__ __launch_bounds__(64) void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                    const float* __restrict__ V, const float* __restrict__ dO,
                                                    const float* __restrict__ LSE, const float* __restrict__ Dv,
                                                    float* __restrict__ dQ, int N, float c, float scale, int causal,
                                                    const uint8_t* __restrict__ mask, int nb, int H, int wl, int wr,
                                                    const float* __restrict__ slopes) {
    const int bh = blockIdx.y;
    const Variant var = variant_of(bh, H, wl, wr, slopes);
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i >= N) return;
    const size_t head = (size_t)bh * N * D;
    const float lse2 = LSE[(size_t)bh * N + i] * kLog2e;
    const float Di = Dv[(size_t)bh * N + i];
    float q[D], g[D], acc[D];
#pragma unroll
    for (int e = 0; e < D; e++) {
        q[e] = Q[head + (size_t)i * D + e];
        g[e] = dO[head + (size_t)i * D + e];
        acc[e] = 0.f;
    }
    for (int j = 0; j < N; j++) {
        if (!allowed(i, j, causal, mask, nb, var)) continue;
        const float* kj = K + head + (size_t)j * D;
        const float* vj = V + head + (size_t)j * D;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; e++) {
            s = __builtin_fmaf(q[e], kj[e], s);
            dp = __builtin_fmaf(g[e], vj[e], dp);
        }
        const float p = exp2f_hw(__builtin_fmaf(s, c, -lse2) + var.bias2(i, j));
        const float ds = p * (dp - Di);
#pragma unroll
        for (int e = 0; e < D; e++) acc[e] = __builtin_fmaf(ds, kj[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < D; e++) {
        dQ[head + (size_t)i * D + e] = acc[e] * scale;
        FA_CHECK(!nonfinite_bits(acc[e] * scale), kDbgNonFinite);
    }
}

// dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij q_i, one thread per key row
template <int D>
__global__ __launch_bounds__(64) void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, const float* __restrict__ dO,
                                                      const float* __restrict__ LSE, const float* __restrict__ Dv,
                                                      float* __restrict__ dK, float* __restrict__ dV, int N, float c,
                                                      float scale, int causal, const uint8_t* __restrict__ mask,
                                                      int nb, int H, int wl, int wr, const float* __restrict__ slopes) {
    __shared__ float kv[2][64][D + 1];  // this block's k and v rows (padded against bank conflicts)
    const int bh = blockIdx.y;
    const Variant var = variant_of(bh, H, wl, wr, slopes);
    const int j0 = blockIdx.x * 64;
    const int t = threadIdx.x;
    const int j = j0 + t;
    const size_t head = (size_t)bh * N * D;
    for (int r = 0; r < 64; r++) {
        const bool ok = j0 + r < N;
        for (int e = t; e < D; e += 64) {
            kv[0][r][e] = ok ? K[head + (size_t)(j0 + r) * D + e] : 0.f;
            kv[1][r][e] = ok ? V[head + (size_t)(j0 + r) * D + e] : 0.f;
        }
    }
    __syncthreads();
    float gk[D], gv[D];
#pragma unroll
    for (int e = 0; e < D; e++) gk[e] = gv[e] = 0.f;
    const int i_start = causal ? j0 : 0;
    for (int i = i_start; i < N; i++) {
        if (j >= N || !allowed(i, j, causal, mask, nb, var)) continue;
        const float* qi = Q + head + (size_t)i * D;
        const float* gi = dO + head + (size_t)i * D;
        float s = 0.f, dp = 0.f;
        for (int e = 0; e < D; e++) {
            s = __builtin_fmaf(qi[e], kv[0][t][e], s);
            dp = __builtin_fmaf(gi[e], kv[1][t][e], dp);
        }
        const float p = exp2f_hw(__builtin_fmaf(s, c, -LSE[(size_t)bh * N + i] * kLog2e) + var.bias2(i, j));
        const float ds = p * (dp - Dv[(size_t)bh * N + i]);
#pragma unroll
        for (int e = 0; e < D; e++) {
            gv[e] = __builtin_fmaf(p, gi[e], gv[e]);
            gk[e] = __builtin_fmaf(ds, qi[e], gk[e]);
        }
    }
    if (j >= N) return;
#pragma unroll
    for (int e = 0; e < D; e++) {
        dK[head + (size_t)j * D + e] = gk[e] * scale;
        dV[head + (size_t)j * D + e] = gv[e];
        FA_CHECK(!nonfinite_bits(gk[e] * scale) && !nonfinite_bits(gv[e]), kDbgNonFinite);
    }
}

template <int D>
hipError_t fwd_f32(const FwdArgs& a) {
    dim3 grid((a.N + 63) / 64, a.BH);
    hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(64), 0, a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (float*)a.o, a.lse, a.N, a.scale * kLog2e, a.causal, a.mask, a.nb,
                       a.H, a.wl, a.wr, a.slopes);
    return hipGetLastError();
}

template <int D>
hipError_t bwd_f32(const BwdArgs& a) {
    const long rows = (long)a.BH * a.N;
    hipLaunchKernelGGL(rowdot_f32_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, a.stream,
                       (const float*)a.o, (const float*)a.dO, a.ws_D, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((a.N + 63) / 64, a.BH);
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL(dq_f32_kernel<D>, grid, dim3(64), 0, a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.dO, a.lse, a.ws_D, (float*)a.dq, a.N, c, a.scale,
                       a.causal, a.mask, a.nb, a.H, a.wl, a.wr, a.slopes);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dkdv_f32_kernel<D>, grid, dim3(64), 0, a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.dO, a.lse, a.ws_D, (float*)a.dk, (float*)a.dv, a.N, c,
                       a.scale, a.causal, a.mask, a.nb, a.H, a.wl, a.wr, a.slopes);
    return hipGetLastError();
}

// One instantiation per head size (a multiple of 16 up to 128): the per-row
// register arrays need the size at compile time.
template <template <int> class L, class Args>
hipError_t by_head_dim(const Args& a) {
    switch (a.d) {
        case 16: return L<16>::run(a);
        case 32: return L<32>::run(a);
        case 48: return L<48>::run(a);
        case 64: return L<64>::run(a);
        case 80: return L<80>::run(a);
        case 96: return L<96>::run(a);
        case 112: return L<112>::run(a);
        case 128: return L<128>::run(a);
        default: return hipErrorInvalidValue;  // excluded by the argument checks
    }
}
template <int D>
struct FwdF32 {
    static hipError_t run(const FwdArgs& a) { return fwd_f32<D>(a); }
};
template <int D>
struct BwdF32 {
    static hipError_t run(const BwdArgs& a) { return bwd_f32<D>(a); }
};

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) { return by_head_dim<FwdF32>(a); }
hipError_t launch_bwd_f32(const BwdArgs& a) { return by_head_dim<BwdF32>(a); }

unsigned debug_flags_f32(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
