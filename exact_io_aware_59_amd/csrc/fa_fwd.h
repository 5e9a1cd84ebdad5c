// Fused exact-attention forward for bf16 on gfx950.
//
// One workgroup (4 waves; 8 in two tile groups when the launch has fewer than
// two workgroups per CU) owns 128 query rows of one (batch, head) and sweeps
// the K/V tiles its mask allows: the Q-outer loop order of FlashAttention-2
// with the grid spread over batch x heads x query blocks ("FlashAttention
// 深度解析" section 四; "FlashAttention原理概览" section 3.1).  Per K/V tile
// every wave computes S^T = K Q^T for its 32 queries on the matrix cores,
// folds the tile into a running row max and row sum (online softmax,
// "FlashAttention 深度解析" section 二) and accumulates O^T += V^T P^T, again
// on the matrix cores.  S and P live only in registers; O is divided by the
// row sum once, after the last tile (section 四).
//
// Layout and scheduling choices for CDNA4:
//  * S is computed transposed (keys x queries) so each lane owns one query:
//    the row max and row sum are in-lane reductions plus one half-wave swap.
//  * The S^T accumulator, rounded to bf16 in place, is the B operand of
//    O^T = V^T P^T; V is read transposed straight from its row-major LDS tile
//    with ds_read_tr16_b64, in the accumulator's key order.
//  * K and V tiles travel HBM -> LDS with buffer_load ... lds (no register
//    staging) into padded rows: K rows D+8 elements apart (16-row operand
//    reads hit distinct banks), V rows D+32 apart (4-row transposing reads
//    hit distinct banks).  Rows past N read as zero (buffer range check).
//  * K runs one tile ahead of V: while the exponentials of tile j are being
//    computed on the vector ALUs, the matrix cores already compute S for tile
//    j+1; the P V products of tile j then overlap the row max of tile j+1
//    ("FlashAttention原理概览" section 3.3: overlap compute with data movement).
//  * Softmax in the log2 domain: p = 2^(s*c - m*c), c = |scale|*log2(e), one
//    FMA per score; a negative scale negates Q (exact in bf16).  The reference
//    max only moves when the running max grows by more than 8 (log2 units), so
//    p <= 256 and O is rarely rescaled; O and l share one reference point, so
//    the result is the same exact quantity.
#pragma once

#include <type_traits>

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
    static constexpr int BC = 64;            // keys per K/V tile
    static constexpr int NKB = BC / 32;      // 32-key blocks per tile
    static constexpr int NKK = D / 16;       // k-steps of the S product
    static constexpr int NDM = D / 32;       // 32-dim blocks of O
    static constexpr int NT = BC / 16;       // k-steps of the PV product
    static constexpr int KS = PadK<D>::STRIDE;
    static constexpr int VS = PadV<D>::STRIDE;
    static constexpr int KTILE = BC * KS;    // elements of a padded K tile
    static constexpr int VTILE = BC * VS;
    static constexpr int KSEGS = KTILE / 512;  // 1 KB segments (one wave-wide 16 B/lane copy each)
    static constexpr int VSEGS = VTILE / 512;
    static_assert(KSEGS * 512 == KTILE && VSEGS * 512 == VTILE, "tiles must be whole 1 KB segments");
    static_assert(kMaskBlock % BC == 0, "a mask block must hold whole tiles");
    // one pipelined step = a fixed schedule of NSLOT matrix products
    static constexpr int NS = NKK * NKB;     // S^T products of a tile
    static constexpr int NP = NT * NDM;      // O^T products of a tile
    static constexpr int NSLOT = NS + NP;
    static constexpr int PD = 2;             // slots between an LDS operand read and its product
    static constexpr int NDMA = (KSEGS + VSEGS + kWaves - 1) / kWaves;  // 1 KB copies per wave per step
    static constexpr int DMA_SLOTS = NSLOT;  // the copies are spread over the whole step
};

// Items [spread<E, S>(j), spread<E, S>(j + 1)) of E items dealt evenly over
// slots 0 .. S-1 (none to later slots).
template <int E, int S>
constexpr int spread(int j) { return ((j < S ? j : S) * E + S - 1) / S; }

// Which K/V tiles a query block visits.
struct TileList {
    int n;                  // number of tiles
    int tpb;                // tiles per mask block (mask mode)
    int bc;
    int first;              // dense mode: index of the first tile
    const uint16_t* cols;   // mask mode: allowed mask columns (LDS)
    __device__ __forceinline__ int kv0(int it) const {
        if (cols == nullptr) return (first + it) * bc;
        return cols[it / tpb] * kMaskBlock + (it % tpb) * bc;
    }
};

// Issue the HBM -> LDS copy of BC rows (kv0 ..) of a [N][hd] tensor (hd <= D
// elements per row) into a padded tile of row stride STRIDE.  The tile is cut
// into 1 KB segments, dealt round-robin to the waves; a lane whose 16 bytes
// fall past the row's hd elements re-reads the row's first chunk.  Tile
// columns [hd, D) therefore hold finite copies of row data: they only meet
// zero Q / dO columns (scores) or produce output columns that are not stored.
template <int D, int STRIDE, int SEGS>
__device__ __forceinline__ void load_tile(rsrc_t r, bf16* tile, int kv0, int hd, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (SEGS + kWaves - 1) / kWaves; i++) {
        const int s = i * kWaves + wave;
        if (s < SEGS) {
            const int el = s * 512 + lane * 8;
            const int row = el / STRIDE;
            int col = el - row * STRIDE;
            col = col < hd ? col : 0;
            buf_load16_lds(r, tile + s * 512, ((uint32_t)(kv0 + row) * hd + col) * 2);
        }
    }
}


// Key of accumulator element r relative to the lane's first key (kv0 + 32 kb + 4h).
constexpr int key_in_block(int r) { return 8 * (r >> 2) + (r & 3); }

// Scores of keys past the causal diagonal or past N become -inf.  A lane's
// keys increase with the register index, so each element is one compare of
// its constant offset against a per-lane limit (no per-element key
// arithmetic for the compiler to hoist into lane masks).
template <int D, bool CAUSAL>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[FwdCfg<D>::NKB], int kv0, int my_q, int N, int h) {
    using C = FwdCfg<D>;
    const int last = CAUSAL ? min(my_q, N - 1) : N - 1;  // last live key of this lane's query
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++) {
        const int lim = last - (kv0 + 32 * kb + 4 * h);
#pragma unroll
        for (int r = 0; r < 16; r++) s[kb][r] = key_in_block(r) > lim ? -INFINITY : s[kb][r];
    }
}

// Local window / ALiBi variant: scores to log2 units with the bias added,
// z = cs * s - slope2 |i - j|, and -inf outside the causal range, the window or N.
template <int D, bool CAUSAL>
__device__ __forceinline__ void variant_scores(f32x16 (&s)[FwdCfg<D>::NKB], int kv0, int my_q, int N, int h,
                                               float cs, const Variant& var) {
    using C = FwdCfg<D>;
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool dead = (CAUSAL && key > my_q) || key >= N || var.dead(my_q, key);
            s[kb][r] = dead ? -INFINITY : __builtin_fmaf(s[kb][r], cs, var.bias2(my_q, key));
        }
}

// Window form of the variant, on tiles that reach an edge: scores outside the
// causal range, the window or N become -inf (live keys of the lane's query form
// [first, last]).  The bias is not applied here.
template <int D, bool CAUSAL>
__device__ __forceinline__ void window_mask(f32x16 (&s)[FwdCfg<D>::NKB], int kv0, int my_q, int N, int h,
                                            const Variant& var) {
    using C = FwdCfg<D>;
    int last = CAUSAL ? min(my_q, N - 1) : N - 1;
    if (var.wr >= 0) last = min(last, my_q + var.wr);
    const int first = var.wl >= 0 ? my_q - var.wl : INT32_MIN / 2;
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++) {
        const int k0 = kv0 + 32 * kb + 4 * h;
        const int hi = last - k0, lo = first - k0;
#pragma unroll
        for (int r = 0; r < 16; r++)
            s[kb][r] = (key_in_block(r) > hi || key_in_block(r) < lo) ? -INFINITY : s[kb][r];
    }
}

// Scores to log2 units with a bias linear in the key, z = cs s + slope2 (key - q),
// for tiles whose live keys all precede their query (causal) or whose slope is
// zero; off0 = slope2 (kv0 + 4h - q).  Two FMAs per score; -inf stays -inf.
template <int D>
__device__ __forceinline__ void linear_bias_scores(f32x16 (&s)[FwdCfg<D>::NKB], float cs, float off0, float slope2) {
    using C = FwdCfg<D>;
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++) {
        const float off = __builtin_fmaf(slope2, (float)(32 * kb), off0);
#pragma unroll
        for (int r = 0; r < 16; r++)
            s[kb][r] = __builtin_fmaf(s[kb][r], cs, __builtin_fmaf(slope2, (float)key_in_block(r), off));
    }
}

template <int D>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[FwdCfg<D>::NKB]) {
    using C = FwdCfg<D>;
    float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) m[r & 3] = fmaxf(m[r & 3], s[kb][r]);
    return xhalf_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])));
}

// S^T of one tile: s[kb] += K[32kb + l32][..] . Q[my_q][..]; `kl` is this lane's row base.
template <int D>
__device__ __forceinline__ void tile_scores(const bf16* kl, const bf16x8 (&qf)[D / 16], f32x16 (&s)[FwdCfg<D>::NKB]) {
    using C = FwdCfg<D>;
#pragma unroll
    for (int kb = 0; kb < C::NKB; kb++) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::NKK; kk++)
#pragma unroll
        for (int kb = 0; kb < C::NKB; kb++)
            s[kb] = mfma32(lds_read8(kl, 32 * kb * C::KS + 16 * kk), qf[kk], s[kb]);
}

// O^T += V^T P^T for one tile; `vl` is this lane's transposing-read base.
template <int D>
__device__ __forceinline__ void tile_pv(const bf16* vl, const bf16x8 (&pb)[FwdCfg<D>::NT], f32x16 (&o)[D / 32]) {
    using C = FwdCfg<D>;
#pragma unroll
    for (int t = 0; t < C::NT; t++)
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++)
            o[dm] = mfma32(lds_tr_operand_pad<C::VS>(vl, 16 * t, 32 * dm), pb[t], o[dm]);
}

// VK: 0 = plain; 1 and 2 = local window and/or ALiBi: every tile's scores are
// taken to log2 units with the bias and the kernel runs with c = 1 (`cs` is
// the true |scale| log2(e)).  With 1 the bias is linear in the key over every
// live pair (causal, or no slopes): two FMAs per score (linear_bias_scores),
// and only tiles that reach an edge of the window, the diagonal or N are
// masked; 2 handles any window and slopes (variant_scores on every tile).
//
// KS = 2 (launches with fewer than two workgroups per CU, e.g. 8 heads of a
// causal N = 8192): eight waves in two groups of four share the 128 query rows
// and split the block's K/V tiles, group g taking tiles g, g+2, ...; each
// group has its own tile buffers and copies.  This doubles the waves per SIMD
// and halves the longest chain of tiles.  At the end group 1 hands its running
// (reference max, row sum, O) to group 0 through LDS, which merges them with
// the online-softmax rescale ("FlashAttention 深度解析" section 二) and writes
// the block.
//
// D is the tile width: 64, 96, 128, 192 or 256.  The tensors' rows hold hd <= D
// elements (a multiple of 16); Q columns from hd on are zero in registers, so
// the padded columns of the K and V tiles never reach a score.  PAD = false
// when hd == D: the row length is then the compile-time D (a runtime length
// costs registers the plain kernels do not have).  D = 256 runs one
// workgroup of four waves per CU (its tiles take 141 KB of LDS).
template <int D, bool CAUSAL, bool MASK, int VK, int KS, bool PAD>
__global__ __launch_bounds__(64 * kWaves * KS, D >= 192 ? 1 : 2 / KS) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int hd_arg, float c, uint32_t qsign,
    const uint8_t* __restrict__ mask, int nb, int nqb, int n_items, int H, int wl, int wr,
    const float* __restrict__ slopes, float cs) {
    using C = FwdCfg<D>;
    const int hd = PAD ? hd_arg : D;
    constexpr bool VAR = VK != 0, LIN = VK == 1, GEN = VK == 2;
    constexpr int NW = kWaves * KS;  // waves per workgroup
    // four separate arrays (not one 2-D array) so that alias analysis can tell
    // the tile being read from the tile the DMA is filling; group g uses
    // [g * TILE, (g + 1) * TILE) of each
    __shared__ __attribute__((aligned(1024))) bf16 kbuf0s[KS * C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 kbuf1s[KS * C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf0s[KS * C::VTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf1s[KS * C::VTILE];
    __shared__ int wave_cnt[NW];
    extern __shared__ uint16_t mask_cols[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
    const int group = KS == 1 ? 0 : wave_id / kWaves;             // tile group
    const int wave = KS == 1 ? wave_id : wave_id % kWaves;        // wave within the group (its 32 queries)
    bf16* const kbuf0 = kbuf0s + group * C::KTILE;
    bf16* const kbuf1 = kbuf1s + group * C::KTILE;
    bf16* const vbuf0 = vbuf0s + group * C::VTILE;
    bf16* const vbuf1 = vbuf1s + group * C::VTILE;
    const int h = lane >> 5, l32 = lane & 31;
    const int k_lane = l32 * C::KS + 8 * h;            // this lane's K operand offset in a tile
    const int v_lane = lane_tr_offset<C::VS>(lane);    // this lane's transposing-read offset

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
    const size_t head_off = (size_t)bh * N * hd;
    const uint32_t head_bytes = (uint32_t)N * hd * 2;
    const rsrc_t rq = make_rsrc(Q + head_off, head_bytes);
    const rsrc_t rk = make_rsrc(K + head_off, head_bytes);
    const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
    const rsrc_t ro = make_rsrc(O + head_off, head_bytes);
    const rsrc_t rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
    Variant var{wl, wr, 0.f};
    if (VAR && slopes != nullptr) var.slope2 = slopes[bh % H] * kLog2e;
    // the pipelined steps' copies: descriptors and, for copy i of this wave,
    // the byte offset of its lane's 16 bytes from the tile's first row (a lane
    // whose bytes fall past the row's hd elements re-reads its first chunk)
    const int32x4_t srd_k = make_srd(K + head_off, head_bytes);
    const int32x4_t srd_v = make_srd(V + head_off, head_bytes);
    uint32_t dma_rel[C::NDMA];
#pragma unroll
    for (int i = 0; i < C::NDMA; i++) {
        const int g = i * kWaves + wave;
        const bool isk = g < C::KSEGS;
        const int seg = isk ? g : min(g - C::KSEGS, C::VSEGS - 1);  // past the V tile: its last segment again
        const int stride = isk ? C::KS : C::VS;
        const int el = seg * 512 + lane * 8;
        const int row = el / stride;
        int col = el - row * stride;
        col = col < hd ? col : 0;
        dma_rel[i] = (uint32_t)(row * hd + col) * 2;
    }

    for (int bi = 0; bi < nblk; bi++) {
        const int qb = qblk[bi];
        const int q0 = qb * kBr;
        const int qw = q0 + wave * kQPerWave;  // first query of this wave
        const int my_q = qw + l32;

        // ---- tile list for this query block ----
        TileList tl;
        tl.bc = C::BC;
        tl.tpb = kMaskBlock / C::BC;
        tl.first = 0;
        tl.cols = nullptr;
        const int q_end = min(N, q0 + kBr);  // one past the last query of the block
        int kv_lo = 0, kv_hi = CAUSAL ? q_end : N;  // keys this block can see
        if (VAR) {
            int lo, hi;
            var.key_range(q0, q_end, N, lo, hi);
            kv_lo = lo;
            kv_hi = min(kv_hi, hi);
        }
        if (MASK) {
            const int lo_col = kv_lo / kMaskBlock;
            const int max_col = kv_hi > kv_lo ? (kv_hi - 1) / kMaskBlock : lo_col - 1;
            const int cnt = max_col >= lo_col
                                ? build_block_list<NW>(mask + (size_t)qb * nb, 1, lo_col, max_col, mask_cols,
                                                           wave_cnt)
                                : 0;
            tl.cols = mask_cols;
            tl.n = cnt * tl.tpb;
        } else {
            tl.first = kv_lo / C::BC;
            tl.n = kv_hi > kv_lo ? (kv_hi + C::BC - 1) / C::BC - tl.first : 0;
        }

        // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
        bf16x8 qf[C::NKK];
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) {
            const int col = 16 * kk + 8 * h;
            u32x4 raw = buf_load16(rq, (uint32_t)(my_q * hd + (col < hd ? col : 0)) * 2);
            raw = col < hd ? (raw ^ qsign) : u32x4{0u, 0u, 0u, 0u};  // columns past hd are zero
            qf[kk] = __builtin_bit_cast(bf16x8, raw);
        }

        f32x16 oacc[C::NDM];
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) oacc[dm] = f32x16{};
        float m_ref = -INFINITY;  // reference max of raw scores (moves lazily)
        float mc = 0.f;           // m_ref * c (0 while m_ref = -inf)
        float l_part = 0.f;       // this lane's half of the running sum
        // The local window / ALiBi kernels follow the exact running max: there one
        // key often dominates a row, and a reference that trails the max leaves
        // that key's weight 2^(m - m_ref) off a power of two, so its bf16 rounding
        // (up to 2^-9 of the dominant term) reaches the output; the plain kernels
        // keep the lazy reference (about 7 % faster).
        constexpr float thr = VK != 0 ? 0.f : kRescaleThreshold;
        // Reference decision for the next tile to be exponentiated, taken as soon
        // as that tile's row max is known: its candidate reference and whether
        // this lane moves to it.
        float m_nx = -INFINITY;
        bool bump_nx = false;
        auto decide = [&](float mx) {
            m_nx = fmaxf(m_ref, mx);
            bump_nx = m_nx != -INFINITY && (m_ref == -INFINITY || (m_nx - m_ref) * c > thr);
        };

        auto needs_mask = [&](int kv0) {
            bool m = (CAUSAL && kv0 + C::BC - 1 > qw) || (kv0 + C::BC > N);
            if (LIN) m = m || (var.wl >= 0 && kv0 < qw + (kQPerWave - 1) - var.wl) ||
                         (var.wr >= 0 && kv0 + C::BC - 1 > qw + var.wr);
            return m;
        };
        // scores of the tile at kv0 -> masked in place, and their row max
        auto finish_scores = [&](f32x16 (&sv)[C::NKB], int kv0) -> float {
            if constexpr (GEN) {
                variant_scores<D, CAUSAL>(sv, kv0, my_q, N, h, cs, var);
                return tile_max<D>(sv);
            } else if constexpr (LIN) {
                if (needs_mask(kv0)) window_mask<D, CAUSAL>(sv, kv0, my_q, N, h, var);
                linear_bias_scores<D>(sv, cs, var.slope2 * (float)(kv0 + 4 * h - my_q), var.slope2);
                return tile_max<D>(sv);
            } else {
                if (needs_mask(kv0)) mask_scores<D, CAUSAL>(sv, kv0, my_q, N, h);
                return tile_max<D>(sv);
            }
        };

        // this group's m-th tile and the number of steps (the same for every
        // group, so that all waves pass the same barriers); a group's tiles past
        // the list start at row N: they read as zero and are masked out.  The
        // variant kernels (exact running max) take the tiles from the last one
        // down: with a causal ALiBi bias the largest scores sit at the diagonal,
        // so the max is found on the first tiles and O is rarely rescaled after.
        const int n_steps = (tl.n + KS - 1) / KS;
        auto kvg = [&](int m) -> int {
            const int t = KS * m + group;
            return t < tl.n ? tl.kv0(VK != 0 ? tl.n - 1 - t : t) : N;
        };

        // ---- prologue: K0, V0, K1 in flight; S(0) and its max ----
        f32x16 sa[C::NKB], sb[C::NKB];
        float mx_cur = -INFINITY;
        if (n_steps > 0) {
            load_tile<D, C::KS, C::KSEGS>(rk, kbuf0, kvg(0), hd, wave, lane);
            load_tile<D, C::VS, C::VSEGS>(rv, vbuf0, kvg(0), hd, wave, lane);
            if (n_steps > 1) load_tile<D, C::KS, C::KSEGS>(rk, kbuf1, kvg(1), hd, wave, lane);
            wait_vmem();
        }
        __syncthreads();
        if (n_steps > 0) {
            tile_scores<D>(kbuf0 + k_lane, qf, sa);
            mx_cur = finish_scores(sa, kvg(0));
            decide(mx_cur);
        }
        __syncthreads();  // every wave is done with kbuf0 before K2 overwrites it

        // One pipelined step: tile `it` (scores in sc, max mx_cur) is exponentiated
        // and multiplied into O while the scores of tile it+1 land in sn.
        // P = parity of `it`: tile it lives in kbuf<P>/vbuf<P>, tile it+1 in the other pair.
        // The step is a fixed schedule of NSLOT matrix products, each slot closed
        // by a scheduling fence: slots [0, NS) compute S(it+1) while the vector
        // ALUs take the exponentials of tile it and pack them to bf16; slots
        // [NS, NSLOT) compute O += V(it)^T P(it)^T while the vector ALUs take the
        // row max of S(it+1).  Every slot issues the LDS operand read of slot
        // j + PD, so no product waits on a read it has just issued, and a share of
        // the step's HBM -> LDS copies (K of tile it+2, V of tile it+1; their
        // buffers were last read before the previous barrier).  Scores of tile
        // it+1 that need a mask or a bias (the few tiles at the diagonal, an edge
        // of the window or N; every tile of a variant) are finished after the
        // schedule, and their max is taken again.  (One instantiation of the
        // schedule: a branch between a masked and a plain copy of it made the
        // register allocator spill.)
        auto step = [&](auto parity, int it, f32x16 (&sc)[C::NKB], f32x16 (&sn)[C::NKB]) {
            constexpr int P = decltype(parity)::value;
            bf16* k_this = P ? kbuf1 : kbuf0;   // K(it), then K(it+2)
            bf16* k_next = P ? kbuf0 : kbuf1;   // K(it+1)
            bf16* v_this = P ? vbuf1 : vbuf0;   // V(it)
            bf16* v_next = P ? vbuf0 : vbuf1;   // V(it+1)
            const bool has_next = it + 1 < n_steps;
            // tiles past the end are copied from rows >= N, which read as zero
            const int kv1 = kvg(it + 1);
            const int kv2 = kvg(it + 2);

            // ---- reference-max update for tile it (rare O rescale), decided when
            // its row max became known ----
            if (__builtin_expect(__ballot(bump_nx) != 0, 0)) {
                const float alpha = bump_nx ? (m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - m_nx) * c)) : 1.f;
                if (bump_nx) {
                    m_ref = m_nx;
                    mc = m_ref * c;
                }
                l_part *= alpha;
#pragma unroll
                for (int dm = 0; dm < C::NDM; dm++) oacc[dm] *= alpha;
            }

            const bf16* kl = k_next + k_lane;
            const bf16* vl = v_this + v_lane;
            const uint32_t k_dst = lds_addr_of(k_this), v_dst = lds_addr_of(v_next);
            const uint32_t k_src = (uint32_t)kv2 * (hd * 2), v_src = (uint32_t)kv1 * (hd * 2);
            bf16x8 opnd[C::NSLOT];
            bf16x8 pb[C::NT];
            float ls[4] = {0.f, 0.f, 0.f, 0.f};   // independent partial sums (short dependency chains)
            float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            auto read_operand = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j < C::NS)
                    opnd[j] = lds_read8(kl, 32 * (j % C::NKB) * C::KS + 16 * (j / C::NKB));
                else
                    opnd[j] = lds_tr_operand_pad<C::VS>(vl, 16 * ((j - C::NS) / C::NDM), 32 * ((j - C::NS) % C::NDM));
            };
            // copy i of this wave: 1 KB segment i*kWaves + wave of the K tile, then of the V tile
            auto dma_op = [&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const int g = i * kWaves + wave;
                const bool isk = g < C::KSEGS;
                const int seg = isk ? g : min(g - C::KSEGS, C::VSEGS - 1);
                dma16_untracked(isk ? srd_k : srd_v, (isk ? k_dst : v_dst) + (uint32_t)seg * 1024u,
                                dma_rel[i] + (isk ? k_src : v_src));
            };
            // The probabilities of tile it go through three stages, each in its own
            // slot so that no slot waits on a result it has just issued: z = c s - c m
            // (slot j-1), p = 2^z (slot j), row sum and bf16 packing (slot j+1).
            constexpr int NE = 16 * C::NKB;  // scores per lane per tile
            auto for_items = [&](auto jc, auto&& fn) {   // the scores whose exponential is in slot j
                constexpr int j = decltype(jc)::value;
                if constexpr (j >= 0 && j < C::NS)
                    static_for<spread<NE, C::NS>(j + 1) - spread<NE, C::NS>(j)>(
                        [&](auto ec) { fn(std::integral_constant<int, spread<NE, C::NS>(j) + decltype(ec)::value>{}); });
            };
            auto z_stage = [&](auto ic) {
                constexpr int idx = decltype(ic)::value;
                float z = __builtin_fmaf(sc[idx / 16][idx % 16], c, -mc);
                pin(z);
                sc[idx / 16][idx % 16] = z;
            };
            auto p_stage = [&](auto ic) {
                constexpr int idx = decltype(ic)::value;
                float p = exp2f_hw(sc[idx / 16][idx % 16]);
                pin(p);
                sc[idx / 16][idx % 16] = p;
            };
            auto sum_stage = [&](auto ic) {
                constexpr int idx = decltype(ic)::value;
                ls[idx & 3] += sc[idx / 16][idx % 16];
                pin(ls[idx & 3]);
                if constexpr (idx % 8 == 7) pb[idx / 8] = pack8<((idx / 8) & 1) * 8>(sc[idx / 16]);
            };
            static_for<C::PD>([&](auto jc) { read_operand(jc); });
            for_items(std::integral_constant<int, 0>{}, z_stage);
            static_for<C::NSLOT>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (j + C::PD < C::NSLOT) read_operand(std::integral_constant<int, j + C::PD>{});
                for_items(std::integral_constant<int, j + 1>{}, z_stage);
                for_items(std::integral_constant<int, j>{}, p_stage);
                for_items(std::integral_constant<int, j - 1>{}, sum_stage);
                // The two waves that share a SIMD (from two workgroups, or from the two
                // tile groups of an eight-wave one) drift in and out of phase: the
                // wave in its exponential half is
                // given issue priority, so its vector work goes out while the other
                // wave's O^T products keep the matrix core busy (measured: ~4 % on
                // the causal d=128 forward; no effect at one wave per SIMD).
                if constexpr (j == 0) __builtin_amdgcn_s_setprio(1);
                if constexpr (j == C::NS) __builtin_amdgcn_s_setprio(0);
                if constexpr (j < C::NS) {
                    // ---- S(it+1) product; exponentials of tile it ----
                    constexpr int kk = j / C::NKB, kb = j % C::NKB;
                    if constexpr (kk == 0) sn[kb] = mfma32(opnd[j], qf[0], f32x16{});
                    else sn[kb] = mfma32(opnd[j], qf[kk], sn[kb]);
                } else {
                    // ---- O += V(it)^T P(it)^T product; row max of S(it+1) ----
                    constexpr int jp = j - C::NS, t = jp / C::NDM, dm = jp % C::NDM;
                    oacc[dm] = mfma32(opnd[j], pb[t], oacc[dm]);
                    if constexpr (VK == 0) {
                        // row max of S(it+1) in the first NP - 3 slots, then its
                        // half-wave exchange and the reference decision, so the
                        // next step starts without that dependency chain
                        constexpr int NMX = C::NP - 3;
                        static_for<spread<8 * C::NKB, NMX>(jp + 1) - spread<8 * C::NKB, NMX>(jp)>([&](auto ec) {
                            constexpr int pr = spread<8 * C::NKB, NMX>(jp) + decltype(ec)::value;
                            constexpr int kb = (2 * pr) / 16, r = (2 * pr) % 16;
                            mp[pr & 3] = fmaxf(mp[pr & 3], fmaxf(sn[kb][r], sn[kb][r + 1]));
                            pin(mp[pr & 3]);
                        });
                        if constexpr (jp == NMX) {
                            mp[0] = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
                            pin(mp[0]);
                        } else if constexpr (jp == NMX + 1) {
                            mx_cur = xhalf_max(mp[0]);
                            pin(mx_cur);
                        } else if constexpr (jp == NMX + 2) {
                            decide(mx_cur);
                        }
                    }
                }
                static_for<spread<C::NDMA, C::DMA_SLOTS>(j + 1) - spread<C::NDMA, C::DMA_SLOTS>(j)>([&](auto ic) {
                    dma_op(std::integral_constant<int, spread<C::NDMA, C::DMA_SLOTS>(j) + decltype(ic)::value>{});
                });
                __builtin_amdgcn_sched_barrier(0);
            });
            l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
            if (VK != 0 || (has_next && needs_mask(kv1))) {
                if (has_next) {
                    mx_cur = finish_scores(sn, kv1);
                    decide(mx_cur);
                }
            }
            wait_vmem();
            __syncthreads();
        };

        int it = 0;
        for (; it + 1 < n_steps; it += 2) {
            step(std::integral_constant<int, 0>{}, it, sa, sb);
            step(std::integral_constant<int, 1>{}, it + 1, sb, sa);
        }
        if (it < n_steps) step(std::integral_constant<int, 0>{}, it, sa, sb);

        if constexpr (KS == 2) {
            // ---- group 1 hands (m_ref, l, O) of its rows to group 0 through LDS
            // (the V buffers hold O, lane-contiguous; kbuf0s the max and sum) ----
            float* xml = reinterpret_cast<float*>(kbuf0s);
            auto xo = [&](int dm, int r) -> float* {
                float* base = reinterpret_cast<float*>((dm & 1) ? vbuf1s : vbuf0s);
                return base + (((dm >> 1) * kWaves + wave) * 16 + r) * 64 + lane;
            };
            static_assert((C::NDM + 1) / 2 * kWaves * 16 * 64 * 4 <= 2 * C::VTILE * 2, "O exchange must fit");
            if (group == 1) {
#pragma unroll
                for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
                    for (int r = 0; r < 16; r++) *xo(dm, r) = oacc[dm][r];
                xml[wave * 64 + lane] = m_ref;
                xml[(kWaves + wave) * 64 + lane] = l_part;
            }
            __syncthreads();
            if (group == 0) {
                const float m1 = xml[wave * 64 + lane], l1 = xml[(kWaves + wave) * 64 + lane];
                const float mm = fmaxf(m_ref, m1);
                const float f0 = m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - mm) * c);
                const float f1 = m1 == -INFINITY ? 0.f : exp2f_hw((m1 - mm) * c);
#pragma unroll
                for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[dm][r] = oacc[dm][r] * f0 + *xo(dm, r) * f1;
                l_part = l_part * f0 + l1 * f1;
                m_ref = mm;
            }
            __syncthreads();  // the exchange buffers are the next block's tiles
        }

        // ---- epilogue: one division per row, bf16 output, lse (buffer stores drop rows >= N) ----
        // O goes out through a staging area in the tile buffers (every wave finished
        // reading them before the last step's barrier): two waves per V buffer, or
        // with 96-wide tiles one wave per K or V buffer; the barrier after it keeps
        // the next block's first copies from landing there too early.
        constexpr bool kTwoPerV = 2 * 32 * (D + 8) <= C::VTILE;
        static_assert(kTwoPerV || (KS == 1 && 32 * (D + 8) <= C::VTILE && 32 * (D + 8) <= C::KTILE),
                      "output staging must fit in the tile buffers");
        if (KS == 1 || group == 0) {
            const float l = xhalf_sum(l_part);
            const float inv = l > 0.f ? 1.f / l : 0.f;
            FA_CHECK(m_ref == -INFINITY || l > 0.f, kDbgRowSum);
            bf16* const stage = kTwoPerV ? (wave < 2 ? vbuf0s : vbuf1s) + (wave & 1) * 32 * (D + 8)
                                         : (wave == 0 ? kbuf0s : wave == 1 ? kbuf1s : wave == 2 ? vbuf0s : vbuf1s);
            store_rows_staged<D>(oacc, inv, stage, ro, (uint32_t)qw * hd * 2, hd, lane);
            if (h == 0) {
                const float lse = l > 0.f ? (m_ref * c + log2f_hw(l)) * kLn2 : -INFINITY;
                FA_CHECK(lse == -INFINITY || !nonfinite_bits(lse), kDbgNonFinite);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, (uint32_t)my_q * 4, 0, 0);
            }
        }
        if (bi + 1 < nblk) __syncthreads();
    }
}

// Compute units of the current device (cached per device).
int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int D, bool CAUSAL, bool MASK, int VK, int KS, bool PAD>
hipError_t launch_ks(const FwdArgs& a, int nqb, int n_items) {
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = fwd_bf16_kernel<D, CAUSAL, MASK, VK, KS, PAD>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    // c = 0 (scale 0) would turn -inf * 0 into NaN; any c below 1e-30 gives the
    // same fp32 probabilities (2^(s*c) == 1 for every finite score s).
    const float c = a.c < 1e-30f ? 1e-30f : a.c;
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads * KS), dyn, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.o, a.lse, a.N, a.d,
                       VK != 0 ? 1.0f : c, a.qsign, a.mask, a.nb, nqb, n_items, a.H, a.wl, a.wr, a.slopes, c);
    return hipGetLastError();
}

// Two workgroups of four waves fit on a CU; with fewer work items than that
// the tile-split eight-wave workgroup keeps two waves on every SIMD.
template <int D, bool CAUSAL, bool MASK, int VK>
hipError_t launch(const FwdArgs& a) {
    const int nqb = (a.N + kBr - 1) / kBr;
    const int per_head = CAUSAL ? (nqb + 1) / 2 : nqb;
    const int n_items = a.BH * per_head;
    const bool pad = a.d != D;
    if constexpr (D >= 192 || D == 96) {  // two tile groups: LDS (192, 256) or the O exchange (96) would not fit
        return pad ? launch_ks<D, CAUSAL, MASK, VK, 1, true>(a, nqb, n_items)
                   : launch_ks<D, CAUSAL, MASK, VK, 1, false>(a, nqb, n_items);
    } else {
        if (n_items < 2 * cu_count())
            return pad ? launch_ks<D, CAUSAL, MASK, VK, 2, true>(a, nqb, n_items)
                       : launch_ks<D, CAUSAL, MASK, VK, 2, false>(a, nqb, n_items);
        return pad ? launch_ks<D, CAUSAL, MASK, VK, 1, true>(a, nqb, n_items)
                   : launch_ks<D, CAUSAL, MASK, VK, 1, false>(a, nqb, n_items);
    }
}

template <int D, int VK>
hipError_t launch_d(const FwdArgs& a) {
    const bool m = a.mask != nullptr;
    if (a.causal) return m ? launch<D, true, true, VK>(a) : launch<D, true, false, VK>(a);
    return m ? launch<D, false, true, VK>(a) : launch<D, false, false, VK>(a);
}

// All three variant kinds of the D-wide kernels (one translation unit per D).
template <int D>
hipError_t launch_fwd_width(const FwdArgs& a) {
    if (!a.variant()) return launch_d<D, 0>(a);
    // the ALiBi bias is linear in the key over the live pairs only when they all precede their query
    return (a.slopes == nullptr || a.causal) ? launch_d<D, 1>(a) : launch_d<D, 2>(a);
}

}  // namespace
}  // namespace fa
