// Recompute backward of exact attention for bf16 on gfx950.
//
// The forward keeps only O and the per-row logsumexp; the backward recomputes
// the scores and probabilities tile by tile from them instead of reading a
// stored N x N matrix ("FlashAttention原理概览" section 3.2; "FlashAttention:
// ... IO-Awareness" section 2.5).  With P = exp(scale*S - lse) and
// D_i = sum_c dO_ic O_ic (which equals sum_j P_ij dP_ij):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = scale dS^T Q,  dQ = scale dS K
// -- the five matrix products of "FlashAttention 深度解析" section 四.
//
// Three launches on one stream:
//   1. rowdot:  D_i = rowsum(dO o O) in fp32, and clear the fp32 dQ accumulator;
//   2. main:    one workgroup per (batch, head, block of 128 keys); its K and V
//               rows stay in registers, dK and dV accumulate in registers; it
//               sweeps the query tiles its mask allows (the K/V-outer order of
//               the IO-Awareness page section 2.3) and adds each tile's dQ
//               contribution into the fp32 accumulator with atomic adds;
//   3. dq_out:  dQ = scale * accumulator, rounded to bf16.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBck = 128;  // keys per workgroup (32 per wave) = one mask block column
constexpr int kBrq = 64;   // queries per step

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); clear the dQ accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                     float* __restrict__ Dv, float* __restrict__ dq_acc,
                                                     long rows) {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long row = gid / CPR;
    const int ch = (int)(gid % CPR);
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + ch * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + ch * 8);
        const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 8; i++) acc = __builtin_fmaf((float)x[i], (float)y[i], acc);
        f32x4* z = reinterpret_cast<f32x4*>(dq_acc + row * D + ch * 8);
        z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // reduce over the CPR lanes of the row (CPR divides 64, rows never straddle waves)
#pragma unroll
    for (int m = 1; m < CPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (row < rows && ch == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> bf16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dq_out_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                     float scale, long n8) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * i];
    const f32x4 b = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        r[e] = (bf16)(a[e] * scale);
        r[4 + e] = (bf16)(b[e] * scale);
    }
    reinterpret_cast<bf16x8*>(dq)[i] = r;
}

// Position of key k' (0..15) inside a 16-key group of the dS tile: swaps the
// middle two groups of four so that one 16-byte read returns the keys in the
// order a transposing read of K produces (see lds_read_tr_operand).
__device__ __forceinline__ int ds_pos16(int k) {
    return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

// ---------------------------------------------------------------------------
// 2. main backward kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float c,
    float scale, const uint8_t* __restrict__ mask, int nb, int nkb, int n_items) {
    constexpr int NKK = D / 16;           // k-steps over the head dimension
    constexpr int NDM = D / 32;           // 32-dim blocks
    constexpr int QT = kBrq * D;          // elements of a Q (or dO) tile
    constexpr int LDT = QT / 8 / kThreads;  // 16-byte chunks per thread per tile
    static_assert(LDT * kThreads * 8 == QT, "tile must split evenly");

    __shared__ __attribute__((aligned(16))) bf16 qdo[2 * QT];       // Q tile | dO tile (or the K block at setup)
    __shared__ __attribute__((aligned(16))) bf16 dsb[kBrq * kBck];  // dS tile, [query][key] 128 wide
    __shared__ __attribute__((aligned(16))) float lse2_s[kBrq];
    __shared__ __attribute__((aligned(16))) float dd_s[kBrq];
    __shared__ int wave_cnt[kWaves];
    extern __shared__ uint16_t rows_list[];

    bf16* qt = qdo;
    bf16* dot = qdo + QT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;

    const int item = xcd_remap(blockIdx.x, n_items);
    const int bh = item / nkb;
    const int kb = item % nkb;
    const int k0 = kb * kBck;
    const int my_key = k0 + 32 * wave + l32;
    const size_t head_off = (size_t)bh * N * D;
    const bf16* Qh = Q + head_off;
    const bf16* Kh = K + head_off;
    const bf16* Vh = V + head_off;
    const bf16* dOh = dO + head_off;
    const float* LSEh = LSE + (size_t)bh * N;
    const float* Dh = Dv + (size_t)bh * N;
    float* dqh = dq_acc + head_off;

    // ---- this wave's K and V rows as B operands (k = head dim, n = key) ----
    bf16x8 kf[NKK], vf[NKK];
    {
        const bool ok = my_key < N;
        const size_t off = (size_t)(ok ? my_key : 0) * D + 8 * h;
#pragma unroll
        for (int kk = 0; kk < NKK; kk++) {
            kf[kk] = ok ? *reinterpret_cast<const bf16x8*>(Kh + off + 16 * kk) : bf16x8{};
            vf[kk] = ok ? *reinterpret_cast<const bf16x8*>(Vh + off + 16 * kk) : bf16x8{};
        }
    }
    // ---- K block in LDS once, to read the dQ product's B operand (k = key, n = dim) ----
    // dQ work split: d=128 -> wave owns dims 32w..32w+31 of both 32-query halves;
    //                d=64  -> wave owns dim block w&1 of query half w>>1.
    constexpr int DQ_QB = (D == 128) ? 2 : 1;
    const int dq_db = (D == 128) ? wave : (wave & 1);
    const int dq_qb0 = (D == 128) ? 0 : (wave >> 1);
    bf16x8 kq[kBck / 16];
    {
        // 128 x D tile, rows = keys (swizzled D wide); fills exactly qdo
        constexpr int CH = kBck * D / 8 / kThreads;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int idx = tid + kThreads * i;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            const bool ok = k0 + row < N;
            const u32x4 val = ok ? *reinterpret_cast<const u32x4*>(Kh + (size_t)(k0 + row) * D + ch * 8)
                                 : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(&qdo[swz<D>(row, ch * 8)]) = val;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kBck / 16; t++) kq[t] = lds_read_tr_operand<D>(qdo, 16 * t, 32 * dq_db, lane);
        __syncthreads();
    }

    // ---- the query tiles to visit ----
    int nsteps;
    int q_first = 0;
    if (MASK) {
        const int lo = CAUSAL ? kb : 0;
        const int cnt = build_block_list<kWaves>(mask + kb, (size_t)nb, lo, nb - 1, rows_list, wave_cnt);
        nsteps = cnt * (kMaskBlock / kBrq);
    } else {
        q_first = CAUSAL ? k0 : 0;
        nsteps = (N - q_first + kBrq - 1) / kBrq;
    }
    auto step_q0 = [&](int st) -> int {
        if (MASK) return rows_list[st / (kMaskBlock / kBrq)] * kMaskBlock + (st % (kMaskBlock / kBrq)) * kBrq;
        return q_first + st * kBrq;
    };

    f32x16 dvacc[NDM], dkacc[NDM];
#pragma unroll
    for (int dm = 0; dm < NDM; dm++) dvacc[dm] = dkacc[dm] = f32x16{};

    // ---- staging of Q / dO tiles and the row terms ----
    u32x4 qst[LDT], dost[LDT];
    float rowv = 0.f;
    auto gload = [&](int q0) {
#pragma unroll
        for (int i = 0; i < LDT; i++) {
            const int idx = tid + kThreads * i;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            const bool ok = q0 + row < N;
            const size_t off = (size_t)(ok ? q0 + row : 0) * D + ch * 8;
            qst[i] = ok ? *reinterpret_cast<const u32x4*>(Qh + off) : u32x4{0, 0, 0, 0};
            dost[i] = ok ? *reinterpret_cast<const u32x4*>(dOh + off) : u32x4{0, 0, 0, 0};
        }
        if (tid < 2 * kBrq) {
            const int r = tid & (kBrq - 1);
            const bool ok = q0 + r < N;
            if (tid < kBrq) {
                // log2-domain lse; rows past N or without any key get +inf so P = 0
                const float l = ok ? LSEh[q0 + r] : -INFINITY;
                rowv = (l == -INFINITY) ? INFINITY : l * kLog2e;
            } else {
                rowv = ok ? Dh[q0 + r] : 0.f;
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < LDT; i++) {
            const int idx = tid + kThreads * i;
            const int row = idx / (D / 8), ch = idx % (D / 8);
            const int off = swz<D>(row, ch * 8);
            *reinterpret_cast<u32x4*>(&qt[off]) = qst[i];
            *reinterpret_cast<u32x4*>(&dot[off]) = dost[i];
        }
        if (tid < kBrq) lse2_s[tid] = rowv;
        else if (tid < 2 * kBrq) dd_s[tid - kBrq] = rowv;
    };

    if (nsteps > 0) {
        gload(step_q0(0));
        lstore();
    }
    __syncthreads();

    for (int st = 0; st < nsteps; st++) {
        const int q0 = step_q0(st);
        if (st + 1 < nsteps) gload(step_q0(st + 1));

        // Keys of this wave vs queries of this tile: all masked when causal and
        // the wave's first key is past the tile's last query.
        const int wk0 = k0 + 32 * wave;
        const bool wave_skip = CAUSAL && wk0 > q0 + kBrq - 1;
        const bool need_mask = (CAUSAL && wk0 + 31 > q0) || (k0 + kBck > N);

        if (!wave_skip) {
            // ---- S = Q K^T and dP = dO V^T (queries x keys) ----
            f32x16 s[2], dp[2];
            s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NKK; kk++) {
#pragma unroll
                for (int qb = 0; qb < 2; qb++) {
                    const bf16x8 aq = lds_read8(qt, swz<D>(32 * qb + l32, 16 * kk + 8 * h));
                    s[qb] = mfma32(aq, kf[kk], s[qb]);
                    const bf16x8 ad = lds_read8(dot, swz<D>(32 * qb + l32, 16 * kk + 8 * h));
                    dp[qb] = mfma32(ad, vf[kk], dp[qb]);
                }
            }
            // ---- P = 2^(c*s - lse2), dS = P (dP - D) ----
#pragma unroll
            for (int qb = 0; qb < 2; qb++) {
#pragma unroll
                for (int a = 0; a < 4; a++) {
                    const int rbase = 32 * qb + 8 * a + 4 * h;
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2_s[rbase]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dd_s[rbase]);
#pragma unroll
                    for (int b = 0; b < 4; b++) {
                        const int r = 4 * a + b;
                        float p = exp2f_hw(__builtin_fmaf(s[qb][r], c, -l4[b]));
                        if (need_mask) {
                            const int qi = q0 + rbase + b;
                            const bool dead = (CAUSAL && my_key > qi) || my_key >= N;
                            p = dead ? 0.f : p;
                        }
                        s[qb][r] = p;
                        dp[qb][r] = p * (dp[qb][r] - d4[b]);
                    }
                }
            }
            // ---- dV^T += dO^T P and dK^T += Q^T dS (dims x keys) ----
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int qb = t >> 1;
                const bf16x8 pb = (t & 1) ? pack8<8>(s[qb]) : pack8<0>(s[qb]);
                const bf16x8 sb = (t & 1) ? pack8<8>(dp[qb]) : pack8<0>(dp[qb]);
#pragma unroll
                for (int dm = 0; dm < NDM; dm++) {
                    const bf16x8 ad = lds_read_tr_operand<D>(dot, 16 * t, 32 * dm, lane);
                    dvacc[dm] = mfma32(ad, pb, dvacc[dm]);
                    const bf16x8 aq = lds_read_tr_operand<D>(qt, 16 * t, 32 * dm, lane);
                    dkacc[dm] = mfma32(aq, sb, dkacc[dm]);
                }
            }
            // ---- dS tile to LDS (bf16, [query][key]) for the dQ product ----
            const int kcol = ds_pos16(32 * wave + l32);
#pragma unroll
            for (int qb = 0; qb < 2; qb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int row = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                    dsb[swz<kBck>(row, kcol)] = (bf16)dp[qb][r];
                }
        } else {
            // this wave's keys see none of these queries: its dS columns are zero
            const int kcol = ds_pos16(32 * wave + l32);
#pragma unroll
            for (int qb = 0; qb < 2; qb++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int row = 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                    dsb[swz<kBck>(row, kcol)] = (bf16)0.f;
                }
        }
        __syncthreads();

        // ---- dQ (queries x dims) += dS K over the 128 keys; atomic fp32 adds ----
#pragma unroll
        for (int qq = 0; qq < DQ_QB; qq++) {
            const int qb = dq_qb0 + qq;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int t = 0; t < kBck / 16; t++) {
                const bf16x8 a = lds_read8(dsb, swz<kBck>(32 * qb + l32, 16 * t + 8 * h));
                acc = mfma32(a, kq[t], acc);
            }
            const int dim = 32 * dq_db + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                if (qi < N) unsafeAtomicAdd(dqh + (size_t)qi * D + dim, acc[r]);
            }
        }

        if (st + 1 < nsteps) lstore();
        __syncthreads();
    }

    // ---- epilogue: dK = scale * acc, dV = acc, bf16 ----
    if (my_key < N) {
        bf16* dkp = dK + head_off + (size_t)my_key * D;
        bf16* dvp = dV + head_off + (size_t)my_key * D;
#pragma unroll
        for (int dm = 0; dm < NDM; dm++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                bf16x4 a, b;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    a[e] = (bf16)(dkacc[dm][4 * g + e] * scale);
                    b[e] = (bf16)dvacc[dm][4 * g + e];
                }
                *reinterpret_cast<bf16x4*>(dkp + 32 * dm + 8 * g + 4 * h) = a;
                *reinterpret_cast<bf16x4*>(dvp + 32 * dm + 8 * g + 4 * h) = b;
            }
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_main(const BwdArgs& a) {
    const int nkb = (a.N + kBck - 1) / kBck;
    const int n_items = a.BH * nkb;
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = bwd_bf16_kernel<D, CAUSAL, MASK>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads), dyn, a.stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (const bf16*)a.dO, a.lse, a.ws_D, a.ws_dq, (bf16*)a.dk, (bf16*)a.dv, a.N,
                       a.scale * kLog2e, a.scale, a.mask, a.nb, nkb, n_items);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const BwdArgs& a) {
    const long rows = (long)a.BH * a.N;
    const long nthr = rows * (D / 8);
    hipLaunchKernelGGL(rowdot_kernel<D>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, a.stream,
                       (const bf16*)a.o, (const bf16*)a.dO, a.ws_D, a.ws_dq, rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_main_all(const BwdArgs& a) {
    const bool m = a.mask != nullptr;
    if (a.causal) return m ? launch_main<D, true, true>(a) : launch_main<D, true, false>(a);
    return m ? launch_main<D, false, true>(a) : launch_main<D, false, false>(a);
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const BwdArgs& a) {
    return a.d == 128 ? launch_prep<128>(a) : launch_prep<64>(a);
}

hipError_t launch_bwd_main_bf16(const BwdArgs& a) {
    return a.d == 128 ? launch_main_all<128>(a) : launch_main_all<64>(a);
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) {
    const long n8 = (long)a.BH * a.N * a.d / 8;
    hipLaunchKernelGGL(dq_out_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, a.stream, a.ws_dq,
                       (bf16*)a.dq, a.scale, n8);
    return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
    hipError_t e = launch_bwd_prep_bf16(a);
    if (e != hipSuccess) return e;
    e = launch_bwd_main_bf16(a);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_bf16(a);
}

}  // namespace fa
