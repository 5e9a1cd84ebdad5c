// FP8 forward for gfx950: block quantization with the incoherent map, and the
// fused forward on the FP8 matrix cores ("FlashAttention 深度解析" section 四:
// FlashAttention-3 adds FP8 block quantization with incoherent processing).
//
//  1. fp8_quant_kernel: one workgroup per 64-row block of one (b, h) slice of
//     Q, K or V, a row per wave at a time in fp64 registers; with a sign
//     vector the incoherent map x -> H (sigma o x) (Sylvester Hadamard matrix,
//     a fast Walsh-Hadamard transform in log2(d) butterfly stages across the
//     lanes; times 1/d for K) is applied exactly (sums of bf16 values fit
//     fp64).  The block gets the
//     smallest power-of-two scale 2^e with amax / 2^e <= 448, and every value
//     becomes the nearest FP8 E4M3 code of x / 2^e (ties to even, computed in
//     fp64 with round-to-nearest-even).  Power-of-two scales are exactly the
//     E8M0 block scales the gfx950 matrix instructions apply.
//  2. fwd_fp8_kernel: the Q-outer forward of the bf16 kernel (4 waves x 32
//     queries, 64-key K/V tiles copied HBM -> LDS with buffer_load ... lds,
//     two stages) with both products on v_mfma_scale_f32_32x32x64_f8f6f4:
//     S^T = K Q^T with the K and Q block exponents as the instruction's scales
//     (S comes out dequantized), then O^T += V^T P^T with P = 2^(c s - c m)
//     times 2^8 rounded to E4M3 (its scale 2^-8 and the V block exponent are
//     again the instruction's scales).  The reference max trails the row max
//     by less than kF8LazyMax (log2 units): it moves only when the max grows
//     by more than that, so P < 2^0.75 and 2^8 P stays below 431, inside
//     E4M3's range (448), with 17 binades below it, while most rescales of O
//     (every growth of the max, with an exact reference) are skipped.  V^T is
//     read with ds_read_b64_tr_b8 in the key order of the S^T accumulator, so
//     P never leaves registers.  The row sum uses the fp32 probabilities.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kF8Block = 64;   // rows per quantization block = keys per tile
constexpr int kF8Waves = 4;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8Br = 32 * kF8Waves;  // queries per workgroup
constexpr int kPExp = 8;              // P is stored as 2^8 p
// the reference max moves when the row max exceeds it by more than this (log2
// units): 2^8 * 2^0.75 = 430.5 < 448, the largest finite E4M3 value
constexpr float kF8LazyMax = 0.75f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// 1. quantization
// ---------------------------------------------------------------------------

// Nearest E4M3 code of x (ties to even), saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne(double x) {
    const uint32_t sign = signbit(x) ? 0x80u : 0u;
    const double a = fabs(x);
    if (!(a < 448.0)) return sign | 0x7Eu;
    int e2;
    frexp(a, &e2);                  // a = f 2^e2, f in [0.5, 1) (a > 0)
    int E = a > 0.0 ? max(e2 - 1, -6) : -6;  // binade; subnormals share the quantum 2^-9
    double q = rint(ldexp(a, 3 - E));       // units of the binade's quantum
    if (q >= 16.0) {                         // rounded up into the next binade
        q = 8.0;
        E++;
    }
    if (E > 8 || (E == 8 && q > 14.0)) return sign | 0x7Eu;
    const uint32_t code = q < 8.0 ? (uint32_t)q : ((uint32_t)(E + 7) << 3) | (uint32_t)(q - 8.0);
    return sign | code;
}

// One workgroup per 64-row block (4 waves x 16 rows).  A wave keeps a row in
// registers, EPL = D/64 consecutive elements per lane (element c = EPL lane +
// j), so the butterfly stages of the map with stride < EPL stay in a lane and
// the others exchange fp64 values with the lane at distance stride / EPL.
template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const bf16* __restrict__ X, uint8_t* __restrict__ codes,
                                                        int8_t* __restrict__ exps, int N, int nblk,
                                                        const float* __restrict__ signs, int k_side) {
    constexpr int EPL = D / 64;
    constexpr int RPW = kF8Block / 4;  // rows per wave
    __shared__ double wmax[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int r0 = blk * kF8Block + wave * RPW;
    const int rows = max(0, min(RPW, N - r0));
    const bf16* xh = X + ((size_t)bh * N + r0) * D;
    double sg[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j++) sg[j] = signs ? (double)signs[EPL * lane + j] : 1.0;
    double v[RPW][EPL];
    double m = 0.0;
#pragma unroll
    for (int r = 0; r < RPW; r++) {
#pragma unroll
        for (int j = 0; j < EPL; j++) v[r][j] = r < rows ? (double)(float)xh[(size_t)r * D + EPL * lane + j] * sg[j] : 0.0;
        if (signs) {
            // fast Walsh-Hadamard transform of the row: (u, w) -> (u + w, u - w) for pairs at distance len
#pragma unroll
            for (int len = 1; len < D; len <<= 1) {
                if (len < EPL) {
#pragma unroll
                    for (int j = 0; j < EPL; j++)
                        if (!(j & len)) {
                            const double u = v[r][j], w = v[r][j + len];
                            v[r][j] = u + w;
                            v[r][j + len] = u - w;
                        }
                } else {
                    const int xl = len / EPL;
                    const bool upper = lane & xl;
#pragma unroll
                    for (int j = 0; j < EPL; j++) {
                        const double o = __shfl_xor(v[r][j], xl);
                        v[r][j] = upper ? o - v[r][j] : v[r][j] + o;
                    }
                }
            }
            if (k_side)
#pragma unroll
                for (int j = 0; j < EPL; j++) v[r][j] *= 1.0 / D;  // exact: D a power of two
        }
#pragma unroll
        for (int j = 0; j < EPL; j++) m = fmax(m, fabs(v[r][j]));
    }
    // block amax: wave, then workgroup
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    const double amax = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
    // smallest e with amax / 2^e <= 448, within the E8M0 range
    int e = 0;
    if (amax > 0.0) {
        int e2;
        frexp(amax / 448.0, &e2);
        e = e2;
        while (ldexp(amax, -e) > 448.0) e++;
        while (ldexp(amax, -(e - 1)) <= 448.0) e--;
    }
    e = max(-127, min(127, e));
    if (tid == 0) exps[(size_t)bh * nblk + blk] = (int8_t)e;
    // codes: EPL consecutive bytes per lane and row
    uint8_t* ch = codes + ((size_t)bh * N + r0) * D;
#pragma unroll
    for (int r = 0; r < RPW; r++) {
        if (r >= rows) break;
        if constexpr (EPL == 2) {
            const uint32_t w = e4m3_rne(ldexp(v[r][0], -e)) | (e4m3_rne(ldexp(v[r][1], -e)) << 8);
            *reinterpret_cast<uint16_t*>(ch + (size_t)r * D + 2 * lane) = (uint16_t)w;
        } else {
            ch[(size_t)r * D + lane] = (uint8_t)e4m3_rne(ldexp(v[r][0], -e));
        }
    }
}

// ---------------------------------------------------------------------------
// 2. forward
// ---------------------------------------------------------------------------
template <int D>
struct F8Cfg {
    static constexpr int RS = D + 16;                  // LDS row stride in bytes (16 * odd mod 256)
    static constexpr int TILE = kF8Block * RS;         // bytes of one padded 64-row tile
    static constexpr int SEGS = TILE / 1024;           // 1 KB copies per tile
    static constexpr int NKK = D / 64;                 // k-steps of S^T (64 dims each)
    static constexpr int NDM = D / 32;                 // 32-dim blocks of O^T
    static_assert(SEGS * 1024 == TILE, "tiles must be whole 1 KB copies");
    // one pipelined step = a fixed schedule of NSLOT matrix products
    static constexpr int NS = 2 * NKK;                 // S^T products of a tile (two 32-key blocks)
    static constexpr int NSLOT = NS + NDM;             // then the O^T products
    static constexpr int PD = 2;                       // slots between an LDS operand read and its product
    static constexpr int NDMA = (2 * SEGS + kF8Waves - 1) / kF8Waves;  // 1 KB copies per wave per step
};

// Items [spread<E, S>(j), spread<E, S>(j + 1)) of E items dealt evenly over
// slots 0 .. S-1 (none to later slots).
template <int E, int S>
constexpr int f8_spread(int j) { return ((j < S ? j : S) * E + S - 1) / S; }

template <int D>
__device__ __forceinline__ void f8_load_tile(rsrc_t r, uint8_t* tile, int kv0, int wave, int lane) {
    using C = F8Cfg<D>;
#pragma unroll
    for (int i = 0; i < (C::SEGS + kF8Waves - 1) / kF8Waves; i++) {
        const int s = i * kF8Waves + wave;
        if (s < C::SEGS) {
            const int el = s * 1024 + lane * 16;
            const int row = el / C::RS;
            int col = el - row * C::RS;
            col = col < D ? col : 0;  // padding: re-read the row's first chunk (never used)
            buf_load16_lds(r, tile + s * 1024, (uint32_t)(kv0 + row) * D + col);
        }
    }
}

__device__ __forceinline__ i32x8 lds_read32(const uint8_t* p) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (i32x2 __attribute__((address_space(3)))*)((__attribute__((address_space(3))) uint8_t*)p));
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const int8_t* __restrict__ QE, const uint8_t* __restrict__ K,
    const int8_t* __restrict__ KE, const uint8_t* __restrict__ V, const int8_t* __restrict__ VE,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, float c, uint32_t qsign, int nqb, int n_items) {
    using C = F8Cfg<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[C::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int nblk = (N + kF8Block - 1) / kF8Block;

    // work item -> (bh, up to two query blocks); causal pairs block p with nqb-1-p
    const int item = xcd_remap(blockIdx.x, n_items);
    int bh, qblk[2], nb;
    if (CAUSAL) {
        const int npair = (nqb + 1) / 2;
        bh = item / npair;
        const int p = item % npair;
        qblk[0] = nqb - 1 - p;
        qblk[1] = p;
        nb = (qblk[1] == qblk[0]) ? 1 : 2;
    } else {
        bh = item / nqb;
        qblk[0] = item % nqb;
        qblk[1] = -1;
        nb = 1;
    }
    const size_t head_off = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D;
    const rsrc_t rk = make_rsrc(K + head_off, head_bytes);
    const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
    const int8_t* ke = KE + (size_t)bh * nblk;
    const int8_t* ve = VE + (size_t)bh * nblk;

    // per-lane LDS offsets: K rows (A operand of S^T), V^T transposing reads
    const int k_lane = l32 * C::RS + 32 * h;
    int v_lane;
    {
        const int G = lane >> 4, i = lane & 15;
        const int jj = i >> 1, half = i & 1;
        const int key = 8 * (jj >> 2) + 4 * (G >> 1) + (jj & 3);   // + 16 r8 per read
        v_lane = key * C::RS + 16 * (G & 1) + 8 * half;            // + 32 dm per 32-dim block
    }

    // copies of the pipelined steps: descriptors and, for copy i of this wave,
    // its lane's byte offset from the tile's first row (1 KB segment
    // i*kF8Waves + wave of the K tile, then of the V tile; past the V tile its
    // last segment again; a lane whose bytes fall in row padding re-reads the
    // row's first chunk)
    const int32x4_t srd_k = make_srd(K + head_off, head_bytes);
    const int32x4_t srd_v = make_srd(V + head_off, head_bytes);
    uint32_t dma_rel[C::NDMA];
#pragma unroll
    for (int i = 0; i < C::NDMA; i++) {
        const int g = i * kF8Waves + wave;
        const int seg = g < C::SEGS ? g : min(g - C::SEGS, C::SEGS - 1);
        const int el = seg * 1024 + lane * 16;
        const int row = el / C::RS;
        int col = el - row * C::RS;
        col = col < D ? col : 0;
        dma_rel[i] = (uint32_t)(row * D + col);
    }

    for (int bi = 0; bi < nb; bi++) {
        const int q0 = qblk[bi] * kF8Br;
        const int qw = q0 + wave * 32;
        const int my_q = qw + l32;
        const int q_end = min(N, q0 + kF8Br);
        const int kv_hi = CAUSAL ? q_end : N;
        const int ntiles = (kv_hi + kF8Block - 1) / kF8Block;
        const int sq = 127 + QE[(size_t)bh * nblk + min(qw, N - 1) / kF8Block];

        // Q fragments (B operand of S^T): 32 bytes of this lane's query per 64 dims
        i32x8 qf[C::NKK];
        {
            const rsrc_t rq = make_rsrc(Q + head_off, head_bytes);
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                const uint32_t off = (uint32_t)my_q * D + 64 * kk + 32 * h;
                const u32x4 a = buf_load16(rq, off) ^ qsign;
                const u32x4 b = buf_load16(rq, off + 16) ^ qsign;
                qf[kk] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
            }
        }
        f32x16 oacc[C::NDM];
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) oacc[dm] = f32x16{};
        float m_ref = -INFINITY, l_part = 0.f;

        // tiles past the last one start at row N: they read as zero and are masked out
        auto kv_of = [&](int t) -> int { return t < ntiles ? t * kF8Block : N; };
        auto needs_mask = [&](int kv0) { return (CAUSAL && kv0 + kF8Block - 1 > qw) || kv0 + kF8Block > N; };
        // scores of a tile at kv0: keys past the diagonal or N to -inf, then the row max
        auto finish = [&](f32x16 (&sv)[2], int kv0) -> float {
            if (needs_mask(kv0)) {
                // a lane's keys increase with the register index: one compare of the
                // element's key offset against the lane's last live key
                const int last = CAUSAL ? min(my_q, N - 1) : N - 1;
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    const int lim = last - (kv0 + 32 * kb + 4 * h);
#pragma unroll
                    for (int r = 0; r < 16; r++) sv[kb][r] = 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : sv[kb][r];
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int r = 0; r < 16; r++) mx = fmaxf(mx, sv[kb][r]);
            return xhalf_max(mx);
        };
        auto kscale = [&](int t) -> int { return 127 + ke[min(t, nblk - 1)]; };

        // ---- prologue: K0, V0, K1 in flight; S(0) and its max ----
        f32x16 sa[2], sb[2];
        float mx_cur = -INFINITY;
        if (ntiles > 0) {
            f8_load_tile<D>(rk, kbuf0, 0, wave, lane);
            f8_load_tile<D>(rv, vbuf0, 0, wave, lane);
            if (ntiles > 1) f8_load_tile<D>(rk, kbuf1, kF8Block, wave, lane);
        }
        wait_vmem();
        __syncthreads();
        if (ntiles > 0) {
            const int sk = kscale(0);
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                sa[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < C::NKK; kk++)
                    sa[kb] = mfma_f8(lds_read32(kbuf0 + k_lane + kb * 32 * C::RS + 64 * kk), qf[kk], sa[kb], sk, sq);
            }
            mx_cur = finish(sa, 0);
        }
        __syncthreads();  // every wave is done with kbuf0 before K2 overwrites it

        // One pipelined step, a fixed schedule of NSLOT matrix products closed by
        // scheduling fences (as in the bf16 forward): slots [0, NS) compute S of
        // tile it+1 while the vector ALUs take 2^8 P of tile it and pack it to
        // E4M3; slots [NS, NSLOT) compute O^T += V^T P^T of tile it while they
        // take the row max of tile it+1.  Every slot issues the LDS operand read
        // of slot j + PD and a share of the copies (K of tile it+2, V of tile
        // it+1, into the buffers tiles it and it-1 left before the last barrier).
        // The reference max follows the exact running max (P <= 1, so 2^8 P fits
        // E4M3); scores of tile it+1 that need a mask are finished after the
        // schedule and their max taken again.
        auto step = [&](auto parity, int it, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
            constexpr int P = decltype(parity)::value;
            uint8_t* k_this = P ? kbuf1 : kbuf0;  // K(it), then K(it+2)
            const uint8_t* k_next = P ? kbuf0 : kbuf1;
            const uint8_t* v_this = P ? vbuf1 : vbuf0;
            uint8_t* v_next = P ? vbuf0 : vbuf1;
            const bool has_next = it + 1 < ntiles;
            const int kv1 = kv_of(it + 1), kv2 = kv_of(it + 2);
            const int sk1 = kscale(it + 1), sv0 = 127 + ve[it];
            // ---- reference-max update for tile it (lazy, within E4M3's range) ----
            {
                const bool bump = mx_cur != -INFINITY && (m_ref == -INFINITY || (mx_cur - m_ref) * c > kF8LazyMax);
                if (__ballot(bump) != 0) {
                    const float alpha = bump ? (m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - mx_cur) * c)) : 1.f;
                    if (bump) m_ref = mx_cur;
                    l_part *= alpha;
#pragma unroll
                    for (int dm = 0; dm < C::NDM; dm++) oacc[dm] *= alpha;
                }
            }
            // 2^8 P = 2^(c s - c m + 8): the factor rides in the exponent's addend, and
            // the running sum is of 2^8 P (divided out, exactly, at the end)
            const float mc8 = (m_ref == -INFINITY ? 0.f : m_ref * c) - (float)kPExp;
            const uint32_t k_dst = lds_addr_of(k_this), v_dst = lds_addr_of(v_next);
            const uint32_t k_src = (uint32_t)kv2 * D, v_src = (uint32_t)kv1 * D;
            i32x8 opnd[C::NSLOT];
            i32x8 pb;
            float ls[4];  // partial row sums, each started by its first term
            float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            float pw[4];
            auto read_operand = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j < C::NS) {
                    constexpr int kk = j / 2, kb = j % 2;
                    opnd[j] = lds_read32(k_next + k_lane + kb * 32 * C::RS + 64 * kk);
                } else {
                    constexpr int dm = j - C::NS;
#pragma unroll
                    for (int r8 = 0; r8 < 4; r8++) {
                        const i32x2 t2 = lds_tr8(v_this + v_lane + r8 * 16 * C::RS + 32 * dm);
                        opnd[j][2 * r8] = t2[0];
                        opnd[j][2 * r8 + 1] = t2[1];
                    }
                }
            };
            auto dma_op = [&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const int g = i * kF8Waves + wave;
                const bool isk = g < C::SEGS;
                const int seg = isk ? g : min(g - C::SEGS, C::SEGS - 1);
                dma16_untracked(isk ? srd_k : srd_v, (isk ? k_dst : v_dst) + (uint32_t)seg * 1024u,
                                dma_rel[i] + (isk ? k_src : v_src));
            };
            static_for<C::PD>([&](auto jc) { read_operand(jc); });
            static_for<C::NSLOT>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j == 0) __builtin_amdgcn_s_setprio(1);
                if constexpr (j == C::NS) __builtin_amdgcn_s_setprio(0);
                if constexpr (j + C::PD < C::NSLOT) read_operand(std::integral_constant<int, j + C::PD>{});
                if constexpr (j < C::NS) {
                    // ---- S(it+1) product; 2^8 P of tile it to E4M3 ----
                    constexpr int kk = j / 2, kb = j % 2;
                    if constexpr (kk == 0) sn[kb] = mfma_f8(opnd[j], qf[0], f32x16{}, sk1, sq);
                    else sn[kb] = mfma_f8(opnd[j], qf[kk], sn[kb], sk1, sq);
                    static_for<f8_spread<32, C::NS>(j + 1) - f8_spread<32, C::NS>(j)>([&](auto ec) {
                        constexpr int idx = f8_spread<32, C::NS>(j) + decltype(ec)::value;  // 16 kb + r
                        float p = exp2f_hw(__builtin_fmaf(sc[idx / 16][idx % 16], c, -mc8));
                        pin(p);
                        pw[idx % 4] = p;
                        if constexpr (idx < 4) ls[idx] = p;
                        else ls[idx % 4] += p;
                        pin(ls[idx % 4]);
                        if constexpr (idx % 4 == 3) {
                            // both halves of the word are written, so the first conversion's
                            // "old" operand may be any register: pw[0]'s own saves a move
                            int word = __builtin_amdgcn_cvt_pk_fp8_f32(pw[0], pw[1], __float_as_int(pw[0]), false);
                            word = __builtin_amdgcn_cvt_pk_fp8_f32(pw[2], pw[3], word, true);
                            pb[idx / 4] = word;
                        }
                    });
                } else {
                    // ---- O^T += V^T P^T of tile it; row max of S(it+1) ----
                    constexpr int dm = j - C::NS;
                    oacc[dm] = mfma_f8(opnd[j], pb, oacc[dm], sv0, 127 - kPExp);
                    static_for<f8_spread<16, C::NDM>(dm + 1) - f8_spread<16, C::NDM>(dm)>([&](auto ec) {
                        constexpr int pr = f8_spread<16, C::NDM>(dm) + decltype(ec)::value;
                        constexpr int kb = (2 * pr) / 16, r = (2 * pr) % 16;
                        mp[pr & 3] = fmaxf(mp[pr & 3], fmaxf(sn[kb][r], sn[kb][r + 1]));
                        pin(mp[pr & 3]);
                    });
                }
                static_for<f8_spread<C::NDMA, C::NSLOT>(j + 1) - f8_spread<C::NDMA, C::NSLOT>(j)>([&](auto ic) {
                    dma_op(std::integral_constant<int, f8_spread<C::NDMA, C::NSLOT>(j) + decltype(ic)::value>{});
                });
                __builtin_amdgcn_sched_barrier(0);
            });
            l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
            if (has_next && needs_mask(kv1)) mx_cur = finish(sn, kv1);
            else mx_cur = xhalf_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
            wait_vmem();
            __syncthreads();
        };
        int it = 0;
        for (; it + 1 < ntiles; it += 2) {
            step(std::integral_constant<int, 0>{}, it, sa, sb);
            step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
        }
        if (it < ntiles) step(std::integral_constant<int, 0>{}, it, sa, sb);

        // epilogue: one division per row, bf16 output (staged through the tile
        // buffers, one per wave, which every wave finished reading before the
        // last step's barrier), lse (rows >= N dropped)
        const float l = xhalf_sum(l_part) * (1.f / (float)(1 << kPExp));
        FA_CHECK(m_ref == -INFINITY || l > 0.f, kDbgRowSum);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const rsrc_t ro = make_rsrc(O + head_off, head_bytes * 2);
        static_assert(32 * (D + 8) * 2 <= C::TILE && kF8Waves == 4, "output staging: one tile buffer per wave");
        uint8_t* const stage = wave == 0 ? kbuf0 : wave == 1 ? kbuf1 : wave == 2 ? vbuf0 : vbuf1;
        store_rows_staged<D>(oacc, inv, reinterpret_cast<bf16*>(stage), ro, (uint32_t)qw * D * 2, D, lane);
        const float lse = l > 0.f ? (m_ref * c + log2f_hw(l)) * kLn2 : -INFINITY;
        FA_CHECK(lse == -INFINITY || !nonfinite_bits(lse), kDbgNonFinite);
        if (h == 0 && my_q < N) LSE[(size_t)bh * N + my_q] = lse;
        __syncthreads();  // the next query block reuses the tiles
    }
}

template <int D>
hipError_t launch_quant_d(const F8QuantArgs& a) {
    const int nblk = (a.N + kF8Block - 1) / kF8Block;
    hipLaunchKernelGGL(fp8_quant_kernel<D>, dim3(a.BH * nblk), dim3(256), 0, a.stream, (const bf16*)a.x, a.codes,
                       a.exps, a.N, nblk, a.signs, a.k_side);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd8_d(const F8FwdArgs& a) {
    const int nqb = (a.N + kF8Br - 1) / kF8Br;
    const int n_items = a.BH * (CAUSAL ? (nqb + 1) / 2 : nqb);
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(n_items), dim3(kF8Threads), 0, a.stream, a.q, a.qe, a.k,
                       a.ke, a.v, a.ve, (bf16*)a.o, a.lse, a.N, a.c, a.qsign, nqb, n_items);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const F8QuantArgs& a) {
    return a.d == 128 ? launch_quant_d<128>(a) : launch_quant_d<64>(a);
}

hipError_t launch_fwd_fp8(const F8FwdArgs& a) {
    if (a.d == 128) return a.causal ? launch_fwd8_d<128, true>(a) : launch_fwd8_d<128, false>(a);
    return a.causal ? launch_fwd8_d<64, true>(a) : launch_fwd8_d<64, false>(a);
}

unsigned debug_flags_fp8(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
