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
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBck = 128;  // keys per workgroup (32 per wave) = one mask block column
constexpr int kBrq = 64;   // queries per step

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); lse in log2 units; clear the dQ accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE, float* __restrict__ Dv,
                                                     float* __restrict__ lse2, float* __restrict__ dq_acc,
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
    if (row < rows && ch == 0) {
        Dv[row] = acc;
        // a row without any allowed key (lse = -inf) gets +inf, so its P = 2^(c s - lse2) = 0
        const float l = LSE[row];
        lse2[row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
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

// ---------------------------------------------------------------------------
// 2. main backward kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
    static constexpr int NKK = D / 16;          // k-steps over the head dimension
    static constexpr int NDM = D / 32;          // 32-dim blocks
    static constexpr int QS = D + 40;           // Q / dO / K tile row stride: 16-row b128 reads conflict-free,
                                                // 4-row transposing reads at most 2-way
    static constexpr int QTILE = kBrq * QS;     // elements of one Q (or dO) tile
    static constexpr int QSEGS = QTILE / 512;   // 1 KB DMA segments
    static constexpr int KTILE = kBck * QS;     // the workgroup's K rows
    static constexpr int KSEGS = KTILE / 512;
    static constexpr int DSS = kBck + 8;        // dS tile: 64 rows (queries) x 128 keys, padded
    static_assert(QSEGS * 512 == QTILE && KSEGS * 512 == KTILE, "tiles must be whole 1 KB segments");
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// HBM -> LDS copy of `rows` rows (r0 ..) of a [N][D] tensor into a padded tile
// (row stride QS); untracked, see dma16_untracked.
template <int D, int SEGS>
__device__ __forceinline__ void dma_rows(int32x4_t srd, const bf16* tile, int r0, int wave, int lane) {
    using C = BwdCfg<D>;
    const uint32_t base = lds_addr_of(tile);
#pragma unroll
    for (int i = 0; i < (SEGS + kWaves - 1) / kWaves; i++) {
        const int s = i * kWaves + wave;
        if (s < SEGS) {
            const int el = s * 512 + lane * 8;
            const int row = el / C::QS;
            int col = el - row * C::QS;
            col = col < D ? col : 0;  // padding slot: harmless re-read of the row's first chunk
            dma16_untracked(srd, base + s * 1024, ((uint32_t)(r0 + row) * D + col) * 2);
        }
    }
}

// Position of key k (within the workgroup's 128) in a dS row: swaps the middle
// two groups of four in every 16 keys, so that one 16-byte read returns keys in
// the order a transposing read of the K tile produces (lds_tr_operand_pad).
__device__ __forceinline__ int ds_pos(int k) {
    return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float c,
    float scale, const uint8_t* __restrict__ mask, int nb, int nkb, int BH) {
    using C = BwdCfg<D>;
    __shared__ __attribute__((aligned(1024))) bf16 qbuf[2][C::QTILE];
    __shared__ __attribute__((aligned(1024))) bf16 obuf[2][C::QTILE];
    __shared__ __attribute__((aligned(1024))) bf16 ktile[C::KTILE];
    __shared__ __attribute__((aligned(16))) bf16 dsb[kBrq * C::DSS];
    __shared__ __attribute__((aligned(16))) float lvec[2][kBrq];
    __shared__ __attribute__((aligned(16))) float dvec[2][kBrq];
    __shared__ int wave_cnt[kWaves];
    extern __shared__ uint16_t rows_list[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;

    // heaviest key blocks first (causal), heads fastest: with B*H a multiple of 8
    // every workgroup of a head lands on the same XCD
    const int kb = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int k0 = kb * kBck;
    const int my_key = k0 + 32 * wave + l32;
    const size_t head_off = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const int32x4_t sq = make_srd(Q + head_off, head_bytes);
    const int32x4_t sdo = make_srd(dO + head_off, head_bytes);
    const int32x4_t sl = make_srd(LSE2 + (size_t)bh * N, (uint32_t)N * 4);
    const int32x4_t sdv = make_srd(Dv + (size_t)bh * N, (uint32_t)N * 4);
    const rsrc_t racc = make_rsrc(dq_acc + head_off, (uint32_t)N * D * 4);

    // ---- K rows of the block to LDS (S operand and dQ operand); this wave's V rows to registers ----
    dma_rows<D, C::KSEGS>(make_srd(K + head_off, head_bytes), ktile, k0, wave, lane);
    bf16x8 vf[C::NKK];
    {
        const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
        const uint32_t off = (uint32_t)(my_key * D + 8 * h) * 2;
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) vf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, off + 32 * kk));
    }
    // dQ work split: d=128 -> wave owns dims 32w..32w+31 of both 32-query halves;
    //                d=64  -> wave owns dim block w&1 of query half w>>1.
    constexpr int DQ_QB = (D == 128) ? 2 : 1;
    const int dq_db = (D == 128) ? wave : (wave & 1);
    const int dq_qb0 = (D == 128) ? 0 : (wave >> 1);

    // ---- the query tiles to visit ----
    int nsteps, n_masked;
    int q_first = 0;
    const bool key_tail = k0 + kBck > N;
    if (MASK) {
        const int lo = CAUSAL ? kb : 0;
        const int cnt = build_block_list<kWaves>(mask + kb, (size_t)nb, lo, nb - 1, rows_list, wave_cnt);
        nsteps = cnt * (kMaskBlock / kBrq);
        n_masked = key_tail ? nsteps : ((CAUSAL && cnt > 0 && rows_list[0] == kb) ? kMaskBlock / kBrq : 0);
    } else {
        q_first = CAUSAL ? k0 : 0;
        nsteps = (N - q_first + kBrq - 1) / kBrq;
        n_masked = key_tail ? nsteps : (CAUSAL ? min(nsteps, kBck / kBrq) : 0);
    }
    auto step_q0 = [&](int st) -> int {
        if (MASK) return rows_list[st / (kMaskBlock / kBrq)] * kMaskBlock + (st % (kMaskBlock / kBrq)) * kBrq;
        return q_first + st * kBrq;
    };

    f32x16 dvacc[C::NDM], dkacc[C::NDM];
#pragma unroll
    for (int dm = 0; dm < C::NDM; dm++) dvacc[dm] = dkacc[dm] = f32x16{};

    auto issue_loads = [&](int q0, int buf) {
        dma_rows<D, C::QSEGS>(sq, qbuf[buf], q0, wave, lane);
        dma_rows<D, C::QSEGS>(sdo, obuf[buf], q0, wave, lane);
        if (wave == 0 && lane < 16) dma16_untracked(sl, lds_addr_of(lvec[buf]), (uint32_t)(q0 + 4 * lane) * 4);
        if (wave == 1 && lane < 16) dma16_untracked(sdv, lds_addr_of(dvec[buf]), (uint32_t)(q0 + 4 * lane) * 4);
    };

    if (nsteps > 0) issue_loads(step_q0(0), 0);
    wait_vmem();
    __syncthreads();

    const int q_lane = l32 * C::QS + 8 * h;                 // b128 operand offset in a Q/dO/K tile
    const int tr_lane = lane_tr_offset<C::QS>(lane);        // transposing-read offset in a Q/dO/K tile
    const int ds_lane = l32 * C::DSS + 8 * h;               // b128 operand offset in the dS tile
    const int kcol = ds_pos(32 * wave + l32);               // this lane's key column in the dS tile
    const bf16* kf_base = ktile + 32 * wave * C::QS + q_lane;

    // One step over 64 queries.  MASKED adds the element mask (diagonal tiles, keys past N).
    auto step = [&](auto masked, int st) {
        constexpr bool MASKED = decltype(masked)::value;
        const int buf = st & 1;
        const bf16* qt = qbuf[buf];
        const bf16* ot = obuf[buf];
        const float* lv = lvec[buf];
        const float* dvv = dvec[buf];
        const int q0 = step_q0(st);
        if (st + 1 < nsteps) issue_loads(step_q0(st + 1), buf ^ 1);

        bf16x8 dsp[4];  // dS of the four 16-query k-steps, bf16
#pragma unroll
        for (int qb = 0; qb < 2; qb++) {
            // ---- S = Q K^T and dP = dO V^T for 32 queries (queries x keys) ----
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                s = mfma32(lds_read8(qt + q_lane, 32 * qb * C::QS + 16 * kk), lds_read8(kf_base, 16 * kk), s);
                dp = mfma32(lds_read8(ot + q_lane, 32 * qb * C::QS + 16 * kk), vf[kk], dp);
            }
            // ---- P = 2^(c s - lse2), dS = P (dP - D) ----
#pragma unroll
            for (int a = 0; a < 4; a++) {
                const int rbase = 32 * qb + 8 * a + 4 * h;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lv + rbase);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(dvv + rbase);
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int r = 4 * a + b;
                    float p = exp2f_hw(__builtin_fmaf(s[r], c, -l4[b]));
                    if (MASKED) {
                        const int qi = q0 + rbase + b;
                        p = ((CAUSAL && my_key > qi) || my_key >= N) ? 0.f : p;
                    }
                    s[r] = p;
                    dp[r] = p * (dp[r] - d4[b]);
                }
            }
            // ---- dV^T += dO^T P, dK^T += Q^T dS (dims x keys) ----
#pragma unroll
            for (int half = 0; half < 2; half++) {
                const int t = 2 * qb + half;
                const bf16x8 pb = half ? pack8<8>(s) : pack8<0>(s);
                dsp[t] = half ? pack8<8>(dp) : pack8<0>(dp);
#pragma unroll
                for (int dm = 0; dm < C::NDM; dm++) {
                    dvacc[dm] = mfma32(lds_tr_operand_pad<C::QS>(ot + tr_lane, 16 * t, 32 * dm), pb, dvacc[dm]);
                    dkacc[dm] = mfma32(lds_tr_operand_pad<C::QS>(qt + tr_lane, 16 * t, 32 * dm), dsp[t], dkacc[dm]);
                }
            }
        }
        // ---- dS tile to LDS ([query][key], key-permuted), once every wave is done with the previous one ----
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int row = 16 * t + 8 * (i >> 2) + 4 * h + (i & 3);
                dsb[row * C::DSS + kcol] = dsp[t][i];
            }
        wait_vmem();  // this wave's copies for the next step have landed
        __syncthreads();

        // ---- dQ (queries x dims) += dS K over the 128 keys; fp32 atomics (rows >= N dropped) ----
#pragma unroll
        for (int qq = 0; qq < DQ_QB; qq++) {
            const int qb = dq_qb0 + qq;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int t = 0; t < kBck / 16; t++)
                acc = mfma32(lds_read8(dsb + ds_lane, 32 * qb * C::DSS + 16 * t),
                             lds_tr_operand_pad<C::QS>(ktile + tr_lane, 16 * t, 32 * dq_db), acc);
            const int dim = 32 * dq_db + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], racc, (uint32_t)(qi * D + dim) * 4, 0, 0);
            }
        }
    };

    int st = 0;
    for (; st < n_masked; st++) step(std::true_type{}, st);
    for (; st < nsteps; st++) step(std::false_type{}, st);

    // ---- epilogue: dK = scale * acc, dV = acc, bf16 (rows >= N dropped) ----
    const rsrc_t rdk = make_rsrc(dK + head_off, head_bytes);
    const rsrc_t rdv = make_rsrc(dV + head_off, head_bytes);
#pragma unroll
    for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            bf16x4 a, b;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                a[e] = (bf16)(dkacc[dm][4 * g + e] * scale);
                b[e] = (bf16)dvacc[dm][4 * g + e];
            }
            const uint32_t off = (uint32_t)(my_key * D + 32 * dm + 8 * g + 4 * h) * 2;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, a), rdk, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), rdv, off, 0, 0);
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
                       (const bf16*)a.v, (const bf16*)a.dO, a.ws_lse2, a.ws_D, a.ws_dq, (bf16*)a.dk, (bf16*)a.dv,
                       a.N, a.scale * kLog2e, a.scale, a.mask, a.nb, nkb, a.BH);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const BwdArgs& a) {
    const long rows = (long)a.BH * a.N;
    const long nthr = rows * (D / 8);
    hipLaunchKernelGGL(rowdot_kernel<D>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, a.stream,
                       (const bf16*)a.o, (const bf16*)a.dO, a.lse, a.ws_D, a.ws_lse2, a.ws_dq, rows);
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
