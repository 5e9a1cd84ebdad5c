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
//   1. rowdot:  D_i = rowsum(dO o O) and lse_i * log2(e), fp32;
//   2. main:    one workgroup per (batch, head, block of 128 keys); dK and dV
//               accumulate in registers while it sweeps the query tiles its mask
//               allows (the K/V-outer order of the IO-Awareness page section 2.3);
//   3. dq:      one workgroup per (batch, head, block of 128 queries) sweeping
//               the key tiles (Q-outer), recomputing S and dP and accumulating
//               dQ = dS K in registers.
// Splitting dQ off costs two extra tile products (S and dP are recomputed) but
// replaces fp32 atomic accumulation of dQ, which measured slower than the
// extra matrix work on this part; every output is deterministic ("FlashAttention
// 深度解析" section 五 notes the deterministic backward as a trade-off).
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
// 1. D = rowsum(dO * O); lse in log2 units.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE, float* __restrict__ Dv,
                                                     float* __restrict__ lse2, long rows) {
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
    static_assert(QSEGS * 512 == QTILE && KSEGS * 512 == KTILE, "tiles must be whole 1 KB segments");
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// HBM -> LDS copy of rows r0 .. of a [N][D] tensor into a padded tile (row
// stride QS); untracked, see dma16_untracked.  The tile is cut into 1 KB
// segments dealt round-robin to the waves; `lane_off[i]` is this lane's byte
// offset of segment i relative to row r0 (precomputed once, dma_lane_offsets).
template <int D, int SEGS>
struct DmaPlan {
    static constexpr int PER_WAVE = (SEGS + kWaves - 1) / kWaves;
    uint32_t lane_off[PER_WAVE];
};

template <int D, int SEGS>
__device__ __forceinline__ DmaPlan<D, SEGS> dma_plan(int wave, int lane) {
    using C = BwdCfg<D>;
    DmaPlan<D, SEGS> p;
#pragma unroll
    for (int i = 0; i < DmaPlan<D, SEGS>::PER_WAVE; i++) {
        const int el = (i * kWaves + wave) * 512 + lane * 8;
        const int row = el / C::QS;
        int col = el - row * C::QS;
        col = col < D ? col : 0;  // padding slot: harmless re-read of the row's first chunk
        p.lane_off[i] = (uint32_t)(row * D + col) * 2;
    }
    return p;
}

template <int D, int SEGS>
__device__ __forceinline__ void dma_rows(int32x4_t srd, const bf16* tile, int r0, const DmaPlan<D, SEGS>& p,
                                         int wave) {
    const uint32_t base = lds_addr_of(tile);
    const uint32_t row_bytes = (uint32_t)r0 * D * 2;
#pragma unroll
    for (int i = 0; i < DmaPlan<D, SEGS>::PER_WAVE; i++) {
        const int s = i * kWaves + wave;
        if (s < SEGS) dma16_untracked(srd, base + s * 1024, row_bytes + p.lane_off[i]);
    }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float c, float scale,
    const uint8_t* __restrict__ mask, int nb, int nkb, int BH) {
    using C = BwdCfg<D>;
    __shared__ __attribute__((aligned(1024))) bf16 qbuf[2][C::QTILE];
    __shared__ __attribute__((aligned(1024))) bf16 obuf[2][C::QTILE];
    __shared__ __attribute__((aligned(1024))) bf16 ktile[C::KTILE];
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

    // ---- K rows of the block to LDS (S operand); this wave's V rows to registers ----
    dma_rows<D, C::KSEGS>(make_srd(K + head_off, head_bytes), ktile, k0, dma_plan<D, C::KSEGS>(wave, lane), wave);
    bf16x8 vf[C::NKK];
    {
        const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
        const uint32_t off = (uint32_t)(my_key * D + 8 * h) * 2;
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) vf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, off + 32 * kk));
    }
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

    const DmaPlan<D, C::QSEGS> qplan = dma_plan<D, C::QSEGS>(wave, lane);
    auto issue_loads = [&](int q0, int buf) {
        dma_rows<D, C::QSEGS>(sq, qbuf[buf], q0, qplan, wave);
        dma_rows<D, C::QSEGS>(sdo, obuf[buf], q0, qplan, wave);
        if (wave == 0 && lane < 16) dma16_untracked(sl, lds_addr_of(lvec[buf]), (uint32_t)(q0 + 4 * lane) * 4);
        if (wave == 1 && lane < 16) dma16_untracked(sdv, lds_addr_of(dvec[buf]), (uint32_t)(q0 + 4 * lane) * 4);
    };

    if (nsteps > 0) issue_loads(step_q0(0), 0);
    wait_vmem();
    __syncthreads();

    const int q_lane = l32 * C::QS + 8 * h;                 // b128 operand offset in a Q/dO/K tile
    const int tr_lane = lane_tr_offset<C::QS>(lane);        // transposing-read offset in a Q/dO/K tile
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

        // Two 32-query halves, software-pipelined: the matrix cores compute
        // S/dP of half 1 while the vector ALUs turn half 0 into P/dS, and the
        // dV/dK products of half 0 run while half 1's P/dS are computed.
        f32x16 s[2], dp[2];
        auto scores = [&](int qb) {
            s[qb] = f32x16{};
            dp[qb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                s[qb] = mfma32(lds_read8(qt + q_lane, 32 * qb * C::QS + 16 * kk), lds_read8(kf_base, 16 * kk), s[qb]);
                dp[qb] = mfma32(lds_read8(ot + q_lane, 32 * qb * C::QS + 16 * kk), vf[kk], dp[qb]);
            }
        };
        bf16x8 pb[2][2], sb[2][2];
        auto probs = [&](int qb) {  // P = 2^(c s - lse2), dS = P (dP - D), packed to bf16
#pragma unroll
            for (int a = 0; a < 4; a++) {
                const int rbase = 32 * qb + 8 * a + 4 * h;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(lv + rbase);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(dvv + rbase);
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const int r = 4 * a + b;
                    float p = exp2f_hw(__builtin_fmaf(s[qb][r], c, -l4[b]));
                    if (MASKED) {
                        const int qi = q0 + rbase + b;
                        p = ((CAUSAL && my_key > qi) || my_key >= N) ? 0.f : p;
                    }
                    s[qb][r] = p;
                    dp[qb][r] = p * (dp[qb][r] - d4[b]);
                }
            }
            pb[qb][0] = pack8<0>(s[qb]);
            pb[qb][1] = pack8<8>(s[qb]);
            sb[qb][0] = pack8<0>(dp[qb]);
            sb[qb][1] = pack8<8>(dp[qb]);
        };
        auto grads = [&](int qb) {  // dV^T += dO^T P, dK^T += Q^T dS (dims x keys)
#pragma unroll
            for (int half = 0; half < 2; half++) {
                const int t = 2 * qb + half;
#pragma unroll
                for (int dm = 0; dm < C::NDM; dm++) {
                    dvacc[dm] = mfma32(lds_tr_operand_pad<C::QS>(ot + tr_lane, 16 * t, 32 * dm), pb[qb][half], dvacc[dm]);
                    dkacc[dm] = mfma32(lds_tr_operand_pad<C::QS>(qt + tr_lane, 16 * t, 32 * dm), sb[qb][half], dkacc[dm]);
                }
            }
        };
        scores(0);
        scores(1);
        probs(0);
#pragma unroll
        for (int i = 0; i < 2 * C::NKK; i++) {
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
        }
        grads(0);
        probs(1);
#pragma unroll
        for (int i = 0; i < 4 * C::NDM; i++) {
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
        }
        grads(1);
        wait_vmem();  // this wave's copies for the next step have landed
        __syncthreads();
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

// ---------------------------------------------------------------------------
// 3. dQ kernel (query-outer): recompute S and dP per key tile, dQ += dS K.
// One workgroup (4 waves x 32 queries) per 128-query block, like the forward:
// the lane owns one query, so lse and D are per-lane scalars.  Deterministic.
// ---------------------------------------------------------------------------
template <int D>
struct DqCfg {
    static constexpr int BC = 64;               // keys per tile
    static constexpr int NKK = D / 16;
    static constexpr int NDM = D / 32;
    static constexpr int KS = D + 40;           // K tile: 16-row b128 reads and 4-row transposing reads
    static constexpr int VS = PadK<D>::STRIDE;  // V tile: 16-row b128 reads only
    static constexpr int KTILE = BC * KS;
    static constexpr int VTILE = BC * VS;
    static constexpr int KSEGS = KTILE / 512;
    static constexpr int VSEGS = VTILE / 512;
    static_assert(KSEGS * 512 == KTILE && VSEGS * 512 == VTILE, "tiles must be whole 1 KB segments");
};
constexpr int kDqBr = 128;  // queries per workgroup

template <int D, int STRIDE, int SEGS>
__device__ __forceinline__ void dq_load_tile(rsrc_t r, bf16* tile, int kv0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (SEGS + kWaves - 1) / kWaves; i++) {
        const int s = i * kWaves + wave;
        if (s < SEGS) {
            const int el = s * 512 + lane * 8;
            const int row = el / STRIDE;
            int col = el - row * STRIDE;
            col = col < D ? col : 0;
            buf_load16_lds(r, tile + s * 512, ((uint32_t)(kv0 + row) * D + col) * 2);
        }
    }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
    bf16* __restrict__ dQ, int N, float c, float scale, const uint8_t* __restrict__ mask, int nb, int nqb,
    int n_items) {
    using C = DqCfg<D>;
    __shared__ __attribute__((aligned(1024))) bf16 kbuf0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 kbuf1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf1[C::VTILE];
    __shared__ int wave_cnt[kWaves];
    extern __shared__ uint16_t mask_cols[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int k_lane = l32 * C::KS + 8 * h;           // K rows as the A operand of S^T
    const int v_lane = l32 * C::VS + 8 * h;           // V rows as the A operand of dP^T
    const int kt_lane = lane_tr_offset<C::KS>(lane);  // K^T via transposing reads (A operand of dQ^T)

    const int item = xcd_remap(blockIdx.x, n_items);
    int bh, qblk[2], nblk;
    if (CAUSAL) {
        const int npair = (nqb + 1) / 2;
        bh = item / npair;
        const int p = item % npair;
        qblk[0] = nqb - 1 - p;
        qblk[1] = p;
        nblk = (qblk[1] == qblk[0]) ? 1 : 2;
    } else {
        bh = item / nqb;
        qblk[0] = item % nqb;
        qblk[1] = -1;
        nblk = 1;
    }
    const size_t head_off = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const rsrc_t rq = make_rsrc(Q + head_off, head_bytes);
    const rsrc_t rdo = make_rsrc(dO + head_off, head_bytes);
    const rsrc_t rk = make_rsrc(K + head_off, head_bytes);
    const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
    const rsrc_t rdq = make_rsrc(dQ + head_off, head_bytes);
    const rsrc_t rl = make_rsrc(LSE2 + (size_t)bh * N, (uint32_t)N * 4);
    const rsrc_t rd = make_rsrc(Dv + (size_t)bh * N, (uint32_t)N * 4);

    for (int bi = 0; bi < nblk; bi++) {
        const int qb = qblk[bi];
        const int q0 = qb * kDqBr;
        const int qw = q0 + wave * 32;
        const int my_q = qw + l32;

        int ntiles;
        const uint16_t* cols = nullptr;
        const int q_end = min(N, q0 + kDqBr);
        if (MASK) {
            const int max_col = CAUSAL ? (q_end - 1) / kMaskBlock : nb - 1;
            const int cnt = build_block_list<kWaves>(mask + (size_t)qb * nb, 1, 0, max_col, mask_cols, wave_cnt);
            cols = mask_cols;
            ntiles = cnt * (kMaskBlock / C::BC);
        } else {
            ntiles = ((CAUSAL ? q_end : N) + C::BC - 1) / C::BC;
        }
        auto kv0_of = [&](int it) -> int {
            if (MASK) return cols[it / (kMaskBlock / C::BC)] * kMaskBlock + (it % (kMaskBlock / C::BC)) * C::BC;
            return it * C::BC;
        };

        // this lane's query: Q and dO fragments (B operands, k = head dim, n = query), lse2 and D
        bf16x8 qf[C::NKK], of[C::NKK];
        {
            const uint32_t off = (uint32_t)(my_q * D + 8 * h) * 2;
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, off + 32 * kk));
                of[kk] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off + 32 * kk));
            }
        }
        const float l2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)my_q * 4, 0, 0));
        const float dd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (uint32_t)my_q * 4, 0, 0));
        const float ml2 = (my_q < N) ? -l2 : -INFINITY;  // rows past N get P = 0

        f32x16 acc[C::NDM];
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) acc[dm] = f32x16{};

        if (ntiles > 0) {
            dq_load_tile<D, C::KS, C::KSEGS>(rk, kbuf0, kv0_of(0), wave, lane);
            dq_load_tile<D, C::VS, C::VSEGS>(rv, vbuf0, kv0_of(0), wave, lane);
        }
        wait_vmem();
        __syncthreads();

        auto step = [&](auto parity, int it) {
            constexpr int P = decltype(parity)::value;
            const bf16* kt = P ? kbuf1 : kbuf0;
            const bf16* vt = P ? vbuf1 : vbuf0;
            const int kv0 = kv0_of(it);
            if (it + 1 < ntiles) {
                dq_load_tile<D, C::KS, C::KSEGS>(rk, P ? kbuf0 : kbuf1, kv0_of(it + 1), wave, lane);
                dq_load_tile<D, C::VS, C::VSEGS>(rv, P ? vbuf0 : vbuf1, kv0_of(it + 1), wave, lane);
            }
            const bool need_mask = (CAUSAL && kv0 + C::BC - 1 > qw) || (kv0 + C::BC > N);
            // two 32-key halves, software-pipelined as in the key-outer kernel
            f32x16 s[2], dp[2];
            auto scores = [&](int kb) {  // S^T and dP^T for 32 keys (keys x queries)
                s[kb] = f32x16{};
                dp[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < C::NKK; kk++) {
                    s[kb] = mfma32(lds_read8(kt + k_lane, 32 * kb * C::KS + 16 * kk), qf[kk], s[kb]);
                    dp[kb] = mfma32(lds_read8(vt + v_lane, 32 * kb * C::VS + 16 * kk), of[kk], dp[kb]);
                }
            };
            bf16x8 sb[2][2];
            auto probs = [&](int kb) {  // P = 2^(c s - lse2), dS = P (dP - D)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    float p = exp2f_hw(__builtin_fmaf(s[kb][r], c, ml2));
                    if (need_mask) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        p = ((CAUSAL && key > my_q) || key >= N) ? 0.f : p;
                    }
                    dp[kb][r] = p * (dp[kb][r] - dd);
                }
                sb[kb][0] = pack8<0>(dp[kb]);
                sb[kb][1] = pack8<8>(dp[kb]);
            };
            auto grads = [&](int kb) {  // dQ^T += K^T dS^T
#pragma unroll
                for (int half = 0; half < 2; half++)
#pragma unroll
                    for (int dm = 0; dm < C::NDM; dm++)
                        acc[dm] = mfma32(lds_tr_operand_pad<C::KS>(kt + kt_lane, 32 * kb + 16 * half, 32 * dm),
                                         sb[kb][half], acc[dm]);
            };
            scores(0);
            scores(1);
            probs(0);
            grads(0);
            probs(1);
            grads(1);
            wait_vmem();
            __syncthreads();
        };
        int it = 0;
        for (; it + 1 < ntiles; it += 2) {
            step(std::integral_constant<int, 0>{}, it);
            step(std::integral_constant<int, 1>{}, it + 1);
        }
        if (it < ntiles) step(std::integral_constant<int, 0>{}, it);

        // dQ = scale * acc -> bf16 (rows >= N dropped)
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; e++) v4[e] = (bf16)(acc[dm][4 * g + e] * scale);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v4), rdq,
                                                      (uint32_t)(my_q * D + 32 * dm + 8 * g + 4 * h) * 2, 0, 0);
            }
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_dq(const BwdArgs& a) {
    const int nqb = (a.N + kDqBr - 1) / kDqBr;
    const int per_head = CAUSAL ? (nqb + 1) / 2 : nqb;
    const int n_items = a.BH * per_head;
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = bwd_dq_kernel<D, CAUSAL, MASK>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads), dyn, a.stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (const bf16*)a.dO, a.ws_lse2, a.ws_D, (bf16*)a.dq, a.N,
                       a.scale * kLog2e, a.scale, a.mask, a.nb, nqb, n_items);
    return hipGetLastError();
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
                       (const bf16*)a.v, (const bf16*)a.dO, a.ws_lse2, a.ws_D, (bf16*)a.dk, (bf16*)a.dv,
                       a.N, a.scale * kLog2e, a.scale, a.mask, a.nb, nkb, a.BH);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const BwdArgs& a) {
    const long rows = (long)a.BH * a.N;
    const long nthr = rows * (D / 8);
    hipLaunchKernelGGL(rowdot_kernel<D>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, a.stream,
                       (const bf16*)a.o, (const bf16*)a.dO, a.lse, a.ws_D, a.ws_lse2, rows);
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
    const bool m = a.mask != nullptr;
    if (a.d == 128) {
        if (a.causal) return m ? launch_dq<128, true, true>(a) : launch_dq<128, true, false>(a);
        return m ? launch_dq<128, false, true>(a) : launch_dq<128, false, false>(a);
    }
    if (a.causal) return m ? launch_dq<64, true, true>(a) : launch_dq<64, true, false>(a);
    return m ? launch_dq<64, false, true>(a) : launch_dq<64, false, false>(a);
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
    hipError_t e = launch_bwd_prep_bf16(a);
    if (e != hipSuccess) return e;
    e = launch_bwd_main_bf16(a);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_bf16(a);
}

}  // namespace fa
