// Fused exact-attention forward for bf16 on gfx950.
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head) and sweeps
// the K/V tiles that its mask allows: the Q-outer loop order of
// FlashAttention-2 with the grid spread over batch x heads x query blocks
// ("FlashAttention 深度解析" section 四; "FlashAttention原理概览" section 3.1).
// Per K/V tile every wave computes S^T = K Q^T for its 32 queries on the
// matrix cores, folds the tile into a running row max and row sum (online
// softmax, "FlashAttention 深度解析" section 二), and accumulates
// O^T += V^T P^T, again on the matrix cores.  S and P live only in registers;
// K and V tiles go through LDS with the next tile's global loads in flight
// while the current one is computed ("FlashAttention原理概览" section 3.3).
// O is divided by the row sum once, after the last tile (section 四).
//
// Layout choices for CDNA4:
//  * S is computed transposed (keys x queries) so each lane owns one query:
//    the row max and row sum are in-lane reductions plus one half-wave swap.
//  * The S^T accumulator is converted in place to the B operand of the
//    O^T = V^T P^T product; V is read transposed straight from its row-major
//    LDS tile with ds_read_tr16_b64, matching the accumulator's key order.
//  * The softmax runs in the log2 domain: p = 2^(s*c - m*c) with
//    c = |scale|*log2(e) applied by one FMA; a negative scale is handled by
//    negating Q (exact in bf16).  The running max is only moved when it grows
//    by more than 8 (in log2 units), which keeps p <= 256 and skips most O
//    rescales; the result is the same exact quantity since O and l always
//    share one reference point.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPerWave = 32;
constexpr int kBr = kWaves * kQPerWave;  // 128 query rows per workgroup = one mask block row
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct FwdCfg {
    static constexpr int BC = 8192 / D;       // keys per K/V tile: 64 (d=128) or 128 (d=64)
    static constexpr int NKB = BC / 32;       // 32-key blocks per tile
    static constexpr int NKK = D / 16;        // k-steps of the S product
    static constexpr int NDM = D / 32;        // 32-dim blocks of O
    static constexpr int TILE = BC * D;       // elements of one K (or V) tile
    static constexpr int CHUNKS = TILE / 8;   // 16-byte chunks per tile
    static constexpr int LD_PER_THREAD = CHUNKS / kThreads;
    static_assert(LD_PER_THREAD * kThreads == CHUNKS, "tile must split evenly over the threads");
    static_assert(kMaskBlock % BC == 0, "a mask block must hold whole tiles");
};

// Which K/V tiles a query block visits.
struct TileList {
    int n;          // number of tiles
    int tpb;        // tiles per mask block (mask mode)
    int bc;
    const uint16_t* cols;  // mask mode: allowed mask columns (LDS)
    __device__ __forceinline__ int kv0(int it) const {
        if (cols == nullptr) return it * bc;
        return cols[it / tpb] * kMaskBlock + (it % tpb) * bc;
    }
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, float c, uint32_t qsign,
    const uint8_t* __restrict__ mask, int nb, int nqb, int n_items) {
    using C = FwdCfg<D>;
    __shared__ __attribute__((aligned(16))) bf16 kbuf[2][C::TILE];
    __shared__ __attribute__((aligned(16))) bf16 vbuf[2][C::TILE];
    __shared__ int wave_cnt[kWaves];
    extern __shared__ uint16_t mask_cols[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;

    // work item -> (bh, up to two query blocks); causal pairs block p with nqb-1-p
    const int item = xcd_remap(blockIdx.x, n_items);
    int bh, qblk[2], nblk;
    if (CAUSAL) {
        const int npair = (nqb + 1) / 2;
        bh = item / npair;
        const int p = item % npair;
        qblk[0] = nqb - 1 - p;  // longer block first
        qblk[1] = p;
        nblk = (qblk[1] == qblk[0]) ? 1 : 2;
    } else {
        bh = item / nqb;
        qblk[0] = item % nqb;
        qblk[1] = -1;
        nblk = 1;
    }
    const size_t head_off = (size_t)bh * N * D;
    const bf16* Qh = Q + head_off;
    const bf16* Kh = K + head_off;
    const bf16* Vh = V + head_off;

    for (int bi = 0; bi < nblk; bi++) {
        const int qb = qblk[bi];
        const int q0 = qb * kBr;
        const int qw = q0 + wave * kQPerWave;  // first query of this wave
        const int my_q = qw + l32;

        // ---- tile list for this query block ----
        TileList tl;
        tl.bc = C::BC;
        tl.tpb = kMaskBlock / C::BC;
        tl.cols = nullptr;
        const int q_end = min(N, q0 + kBr);  // one past the last query of the block
        if (MASK) {
            const int max_col = CAUSAL ? (q_end - 1) / kMaskBlock : nb - 1;
            const int cnt = build_block_list<kWaves>(mask + (size_t)qb * nb, 1, 0, max_col, mask_cols, wave_cnt);
            tl.cols = mask_cols;
            tl.n = cnt * tl.tpb;
        } else {
            const int kv_end = CAUSAL ? q_end : N;
            tl.n = (kv_end + C::BC - 1) / C::BC;
        }

        // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
        bf16x8 qf[C::NKK];
        {
            const bool ok = my_q < N;
            const bf16* src = Qh + (size_t)(ok ? my_q : 0) * D + 8 * h;
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 16 * kk) : u32x4{0, 0, 0, 0};
                raw ^= qsign;
                qf[kk] = __builtin_bit_cast(bf16x8, raw);
            }
        }

        f32x16 oacc[C::NDM];
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) oacc[dm] = f32x16{};
        float m_ref = -INFINITY;  // running max of raw scores (reference point)
        float l_part = 0.f;       // this lane's half of the running sum

        // ---- staging of K/V tiles: global -> registers -> swizzled LDS ----
        u32x4 kst[C::LD_PER_THREAD], vst[C::LD_PER_THREAD];
        auto gload = [&](int kv0) {
#pragma unroll
            for (int i = 0; i < C::LD_PER_THREAD; i++) {
                const int idx = tid + kThreads * i;
                const int row = idx / (D / 8), ch = idx % (D / 8);
                const bool ok = kv0 + row < N;
                const size_t off = (size_t)(ok ? kv0 + row : 0) * D + ch * 8;
                kst[i] = ok ? *reinterpret_cast<const u32x4*>(Kh + off) : u32x4{0, 0, 0, 0};
                vst[i] = ok ? *reinterpret_cast<const u32x4*>(Vh + off) : u32x4{0, 0, 0, 0};
            }
        };
        auto lstore = [&](int buf) {
#pragma unroll
            for (int i = 0; i < C::LD_PER_THREAD; i++) {
                const int idx = tid + kThreads * i;
                const int row = idx / (D / 8), ch = idx % (D / 8);
                const int off = swz<D>(row, ch * 8);
                *reinterpret_cast<u32x4*>(&kbuf[buf][off]) = kst[i];
                *reinterpret_cast<u32x4*>(&vbuf[buf][off]) = vst[i];
            }
        };

        if (tl.n > 0) {
            gload(tl.kv0(0));
            lstore(0);
        }
        __syncthreads();

        for (int it = 0; it < tl.n; it++) {
            const int buf = it & 1;
            const int kv0 = tl.kv0(it);
            if (it + 1 < tl.n) gload(tl.kv0(it + 1));

            // Does this wave see any key of the tile?  Does it need element masks?
            const bool wave_skip = CAUSAL && kv0 > qw + kQPerWave - 1;
            const bool need_mask = (CAUSAL && kv0 + C::BC - 1 > qw) || (kv0 + C::BC > N);
            if (!wave_skip) {
                const bf16* kt = kbuf[buf];
                const bf16* vt = vbuf[buf];
                // ---- S^T = K Q^T (keys x queries), fp32 accumulate ----
                f32x16 s[C::NKB];
#pragma unroll
                for (int kb = 0; kb < C::NKB; kb++) s[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < C::NKK; kk++) {
#pragma unroll
                    for (int kb = 0; kb < C::NKB; kb++) {
                        const bf16x8 a = lds_read8(kt, swz<D>(32 * kb + l32, 16 * kk + 8 * h));
                        s[kb] = mfma32(a, qf[kk], s[kb]);
                    }
                }
                // ---- masks: causal (key > query) and keys past N ----
                if (need_mask) {
#pragma unroll
                    for (int kb = 0; kb < C::NKB; kb++)
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                            const bool dead = (CAUSAL && key > my_q) || key >= N;
                            s[kb][r] = dead ? -INFINITY : s[kb][r];
                        }
                }
                // ---- online softmax: tile max, lazy rescale, exponentials ----
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < C::NKB; kb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[kb][r]);
                mx = xhalf_max(mx);
                const float m_new = fmaxf(m_ref, mx);
                const bool bump = m_new != -INFINITY && (m_ref == -INFINITY || (m_new - m_ref) * c > kRescaleThreshold);
                if (__builtin_expect(__ballot(bump) != 0, 0)) {
                    const float alpha = bump ? (m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - m_new) * c)) : 1.f;
                    if (bump) m_ref = m_new;
                    l_part *= alpha;
#pragma unroll
                    for (int dm = 0; dm < C::NDM; dm++) oacc[dm] *= alpha;
                }
                const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < C::NKB; kb++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        float p = exp2f_hw(__builtin_fmaf(s[kb][r], c, -mc));
                        if (need_mask) p = (s[kb][r] == -INFINITY) ? 0.f : p;
                        s[kb][r] = p;
                        lsum += p;
                    }
                l_part += lsum;
                // ---- O^T += V^T P^T ----
#pragma unroll
                for (int kb = 0; kb < C::NKB; kb++) {
#pragma unroll
                    for (int half = 0; half < 2; half++) {
                        const bf16x8 pb = half ? pack8<8>(s[kb]) : pack8<0>(s[kb]);
                        const int row0 = 32 * kb + 16 * half;
#pragma unroll
                        for (int dm = 0; dm < C::NDM; dm++) {
                            const bf16x8 a = lds_read_tr_operand<D>(vt, row0, 32 * dm, lane);
                            oacc[dm] = mfma32(a, pb, oacc[dm]);
                        }
                    }
                }
            }
            if (it + 1 < tl.n) lstore(buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue: one division per row, bf16 output, lse ----
        const float l = xhalf_sum(l_part);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (my_q < N) {
            bf16* dst = O + head_off + (size_t)my_q * D;
#pragma unroll
            for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    bf16x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; e++) v4[e] = (bf16)(oacc[dm][4 * g + e] * inv);
                    *reinterpret_cast<bf16x4*>(dst + 32 * dm + 8 * g + 4 * h) = v4;
                }
            if (h == 0)
                LSE[(size_t)bh * N + my_q] = l > 0.f ? (m_ref * c + log2f_hw(l)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const FwdArgs& a) {
    const int nqb = (a.N + kBr - 1) / kBr;
    const int per_head = CAUSAL ? (nqb + 1) / 2 : nqb;
    const int n_items = a.BH * per_head;
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = fwd_bf16_kernel<D, CAUSAL, MASK>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads), dyn, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.N,
                       a.c, a.qsign, a.mask, a.nb, nqb, n_items);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    const bool m = a.mask != nullptr;
    if (a.d == 128) {
        if (a.causal) return m ? launch<128, true, true>(a) : launch<128, true, false>(a);
        return m ? launch<128, false, true>(a) : launch<128, false, false>(a);
    }
    if (a.causal) return m ? launch<64, true, true>(a) : launch<64, true, false>(a);
    return m ? launch<64, false, true>(a) : launch<64, false, false>(a);
}

}  // namespace fa
