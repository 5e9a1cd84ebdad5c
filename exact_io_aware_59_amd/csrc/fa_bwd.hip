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
// Kernels:
//   rowdot: D_i = rowsum(dO o O) and lse_i * log2(e), fp32 (the preprocessing
//           stage on its own);
//   main:   one workgroup per (batch, head, block of 128 keys); dK and dV
//           accumulate in registers while it sweeps the query tiles its mask
//           allows (the K/V-outer order of the IO-Awareness page section 2.3);
//   dq:     one workgroup per (batch, head, block of 128 queries) sweeping the
//           key tiles (Q-outer), recomputing S and dP and accumulating
//           dQ = dS K in registers; given O and lse it also does the
//           preprocessing of its own rows.
// fa_bwd launches dq (with the preprocessing) and then main; the stages can
// also run as rowdot, main, dq, with the same bits.
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
// D (64 or 128) bounds the row length hd; chunks past hd contribute nothing.
template <int D>
constexpr int rowdot_lanes() { return D <= 64 ? 8 : 16; }  // lanes per row: chunks per row, to a power of two

template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE, float* __restrict__ Dv,
                                                     float* __restrict__ lse2, long rows, int hd) {
    constexpr int CPR = D / 8;                   // 16-byte chunks per row (at most)
    constexpr int LPR = rowdot_lanes<D>();       // lanes per row (chunks past CPR add zeros)
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long row = gid / LPR;
    const int ch = (int)(gid % LPR);
    float acc = 0.f;
    if (row < rows && ch < CPR && 8 * ch < hd) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * hd + ch * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * hd + ch * 8);
        const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 8; i++) acc = __builtin_fmaf((float)x[i], (float)y[i], acc);
    }
    // reduce over the LPR lanes of the row (LPR divides 64, rows never straddle waves)
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
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
    static constexpr int RB = 2 * D;            // bytes per tile row (no padding: rows are swizzled)
    static constexpr int QTILE = kBrq * D;      // elements of one Q (or dO) tile
    static constexpr int QSEGS = QTILE / 512;   // 1 KB DMA segments
    static constexpr int SEG_PER_WAVE = QSEGS / kWaves;
    static_assert(SEG_PER_WAVE * kWaves * 512 == QTILE, "a tile must split into whole segments per wave");
    // copies one wave issues per tile: its Q and dO segments, then one 256-byte
    // row of lse2 (waves 0, 2) or D (waves 1, 3)
    static constexpr int NDMA = 2 * SEG_PER_WAVE + 1;
    // matrix products of one 32-query half step, in issue order:
    //   NA = S and dP of the NEXT half (alternating), then NC for dV, NC for dK
    static constexpr int NA = 2 * NKK;
    static constexpr int NC = 2 * NDM;
    static constexpr int NSLOT = NA + 2 * NC;
    static constexpr int PD = 2;  // slots between an LDS operand read and its product
};

__device__ __forceinline__ bf16x8 lds_read8_b(const void* base, uint32_t byte_off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ bf16x8 lds_tr_pair_b(const void* base, uint32_t lo_off, uint32_t hi_off) {
    const bf16* b = reinterpret_cast<const bf16*>(base);
    const bf16x4 lo = lds_read_tr4(b, lo_off / 2);
    const bf16x4 hi = lds_read_tr4(b, hi_off / 2);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// S and R chains (zero start / accumulate).  The builtin lets the compiler
// see the matrix instructions and insert the hazard waits they need.
__device__ __forceinline__ void mfma32_zero(f32x16& d, bf16x8 a, bf16x8 b) { d = mfma32(a, b, f32x16{}); }
__device__ __forceinline__ void mfma32_acc(f32x16& d, bf16x8 a, bf16x8 b) { d = mfma32(a, b, d); }

// Items [first(j), first(j+1)) of E items spread evenly over S slots.
template <int E, int S>
constexpr int slot_first(int j) { return (j * E + S - 1) / S; }

// Key of accumulator element r relative to the lane's first key or query (32-row block + 4h).
constexpr int row_in_block(int r) { return 8 * (r >> 2) + (r & 3); }

// Whether any (query, key) pair of queries [q0, q0 + nq) x keys [k0, k0 + nk) is
// outside the causal range, the local window or N.
template <bool CAUSAL>
__device__ __forceinline__ bool block_has_dead(int q0, int nq, int k0, int nk, int N, const Variant& var) {
    return (CAUSAL && k0 + nk - 1 > q0) || k0 + nk > N || (var.wl >= 0 && q0 + nq - 1 - k0 > var.wl) ||
           (var.wr >= 0 && k0 + nk - 1 - q0 > var.wr);
}

// VK: 0 = plain; 1 = local window and/or an ALiBi bias linear in the key over
// the live pairs (causal, or no slopes): the S chain starts from -slope2 r'/c
// (r' = the row offset of element r) and the exponent's addend carries
// slope2 (key - 4h - q0); only steps that reach an edge of the window, the
// diagonal or N take the masked path; 2 = any window and ALiBi, every step
// masked with the bias computed per element.
template <int D, bool CAUSAL, bool MASK, int VK>
__global__ __launch_bounds__(kThreads, 1) void bwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dv,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, int hd, float c, float scale,
    const uint8_t* __restrict__ mask, int nb, int nkb, int BH, int H, int wl, int wr,
    const float* __restrict__ slopes) {
    using C = BwdCfg<D>;
    constexpr bool VAR = VK != 0, LIN = VK == 1, GEN = VK == 2;
    // three-deep ring of query tiles (Q then dO): tile t+2 streams in while t and
    // t+1 are read.  Rows are unpadded; 16-byte chunk c of row r sits at chunk
    // position c ^ swz_sigma(r), which keeps both the 16-row operand reads and
    // the 4-row transposing reads free of bank conflicts.
    __shared__ __attribute__((aligned(1024))) bf16 ring[3][2][C::QTILE];
    __shared__ __attribute__((aligned(256))) float lvec[3][kBrq];
    __shared__ __attribute__((aligned(256))) float dvec[3][kBrq];
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
    const size_t head_off = (size_t)bh * N * hd;
    const uint32_t head_bytes = (uint32_t)N * hd * 2;
    const int32x4_t sq = make_srd(Q + head_off, head_bytes);
    const int32x4_t sdo = make_srd(dO + head_off, head_bytes);
    // waves 0 and 2 copy lse2 rows, waves 1 and 3 the D rows (the second copy is
    // a duplicate of identical bytes, which keeps the issue free of branches)
    const int32x4_t svec = (wave & 1) ? make_srd(Dv + (size_t)bh * N, (uint32_t)N * 4)
                                      : make_srd(LSE2 + (size_t)bh * N, (uint32_t)N * 4);
    const uint32_t vec_lds0 = (wave & 1) ? lds_addr_of(&dvec[0][0]) : lds_addr_of(&lvec[0][0]);

    // ---- this wave's K and V rows as MFMA B operands (k = head dim, n = key);
    // columns past hd are zero, so the padded columns of the query tiles never
    // reach S or dP ----
    bf16x8 kf[C::NKK], vneg[C::NKK];
    {
        const rsrc_t rk = make_rsrc(K + head_off, head_bytes);
        const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) {
            const int col = 16 * kk + 8 * h;
            const uint32_t off = (uint32_t)(my_key * hd + (col < hd ? col : 0)) * 2;
            const u32x4 z = {0u, 0u, 0u, 0u};
            kf[kk] = __builtin_bit_cast(bf16x8, col < hd ? buf_load16(rk, off) : z);
            // -V (exact: a sign flip), so the R chain yields D - dP
            vneg[kk] = __builtin_bit_cast(bf16x8, col < hd ? (buf_load16(rv, off) ^ 0x80008000u) : z);
        }
    }
    // ---- the query tiles to visit: queries [q_lo, q_hi) can see this key block ----
    Variant var{wl, wr, 0.f};
    if (VAR && slopes != nullptr) var.slope2 = slopes[bh % H] * kLog2e;
    int q_lo = CAUSAL ? k0 : 0, q_hi = N;
    if (VAR) {
        int lo, hi;
        var.query_range(k0, min(N, k0 + kBck), N, lo, hi);
        q_lo = max(q_lo, lo);
        q_hi = min(q_hi, hi);
    }
    int nsteps, n_masked;
    int q_first = 0;
    const bool key_tail = k0 + kBck > N;
    if (MASK) {
        const int lo_blk = q_lo / kMaskBlock;
        const int hi_blk = q_hi > q_lo ? (q_hi - 1) / kMaskBlock : lo_blk - 1;
        const int cnt = hi_blk >= lo_blk
                            ? build_block_list<kWaves>(mask + kb, (size_t)nb, lo_blk, hi_blk, rows_list, wave_cnt)
                            : 0;
        nsteps = cnt * (kMaskBlock / kBrq);
        n_masked = (GEN || key_tail) ? nsteps
                                     : ((CAUSAL && cnt > 0 && rows_list[0] == kb) ? kMaskBlock / kBrq : 0);
    } else {
        q_first = q_lo;
        nsteps = q_hi > q_lo ? (q_hi - q_first + kBrq - 1) / kBrq : 0;
        n_masked = (GEN || key_tail) ? nsteps : (CAUSAL ? min(nsteps, kBck / kBrq) : 0);
    }
    // first query of step st; steps past the end map to row N, whose copies
    // fall outside the buffers and fetch nothing
    auto step_q0 = [&](int st) -> int {
        if (st >= nsteps) return N;
        if (MASK) return rows_list[st / (kMaskBlock / kBrq)] * kMaskBlock + (st % (kMaskBlock / kBrq)) * kBrq;
        return q_first + st * kBrq;
    };

    // Per-lane byte offsets of this wave's DMA segments relative to the tile's
    // first row.  Segments are dealt round-robin to the waves; lane i of a
    // segment fills LDS chunk position i, i.e. logical chunk i ^ sigma(row).
    // A chunk past the row's hd elements re-reads the row's first chunk: those
    // tile columns only meet the zero columns of K and V or produce dK / dV
    // columns that are not stored.
    uint32_t seg_off[C::SEG_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::SEG_PER_WAVE; i++) {
        constexpr int CPR = D / 8;  // chunks per row
        const int g = (i * kWaves + wave) * 64 + lane;  // chunk position in the tile
        const int row = g / CPR;
        const int col = 8 * chunk_at<D>(row, g % CPR);
        seg_off[i] = (uint32_t)(row * hd + (col < hd ? col : 0)) * 2;
    }
    // copy k (0 .. NDMA-1) of the tile starting at query q0 into ring slot `buf`
    auto dma_op = [&](auto kc, int q0, int buf) {
        constexpr int k = decltype(kc)::value;
        const uint32_t rb = (uint32_t)q0 * hd * 2;
        if constexpr (k < 2 * C::SEG_PER_WAVE) {
            constexpr int i = k % C::SEG_PER_WAVE;
            constexpr int tensor = k / C::SEG_PER_WAVE;
            const uint32_t dst = lds_addr_of(ring[buf][tensor]) + (i * kWaves + wave) * 1024;
            dma16_untracked(tensor == 0 ? sq : sdo, dst, rb + seg_off[i]);
        } else {
            dma4_untracked(svec, vec_lds0 + buf * (kBrq * 4), (uint32_t)(q0 + lane) * 4);
        }
    };
    auto dma_tile = [&](int q0, int buf) { static_for<C::NDMA>([&](auto k) { dma_op(k, q0, buf); }); };

    f32x16 dvacc[C::NDM], dkacc[C::NDM];
#pragma unroll
    for (int dm = 0; dm < C::NDM; dm++) dvacc[dm] = dkacc[dm] = f32x16{};
    // VK = 1: start of every S chain, -slope2 r' / c for row offset r' of element r
    f32x16 sinit = {};
    if constexpr (LIN) {
        const float t = -var.slope2 / c;
#pragma unroll
        for (int r = 0; r < 16; r++) sinit[r] = t * (float)row_in_block(r);
    }

    // Operand byte offsets inside a swizzled tile (loop invariant, per lane):
    //   a_off[kk]: row l32, logical chunk 2kk + h (B128 read of the S / dP A operand);
    //   tr_lo/hi[dm]: rows 4h + j and 4h + j + 8, columns 32dm + 16g + 4q (the two
    //   transposing reads of a dV / dK A operand, see lds_tr_operand_pad).
    uint32_t a_off[C::NKK], tr_lo[C::NDM], tr_hi[C::NDM];
    {
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) a_off[kk] = l32 * C::RB + (chunk_pos<D>(l32, 2 * kk + h) << 4);
        const int sl = lane & 15, j = sl >> 2, q = sl & 3, g = (lane >> 4) & 1;
        const int r = 4 * h + j;
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) {
            const int cc = 4 * dm + 2 * g + (q >> 1);
            tr_lo[dm] = r * C::RB + (chunk_pos<D>(r, cc) << 4) + (q & 1) * 8;
            tr_hi[dm] = (r + 8) * C::RB + (chunk_pos<D>(r + 8, cc) << 4) + (q & 1) * 8;
        }
    }

    // One 32-query half step g, as a fixed schedule of NSLOT matrix products.
    // Slot j issues the LDS operand read of slot j + PD, its own product and the
    // vector work assigned to it; a scheduling fence closes every slot, so the
    // products stay evenly interleaved with the vector work and the copies.
    //   products: S of half g+1 (NKK, chain from zero), then R = D - dP of half
    //             g+1 (NKK, chain from that half's D rows; V is held negated),
    //             then dV += dO^T P (NC) and dK += Q^T dS' (NC) of half g;
    //   vector:   during the S / R products dS' = P R of half g (= -dS, the
    //             sign is restored in the dK epilogue); during the dV / dK
    //             products P = 2^(c s - lse2) of half g+1, whose S is ready.
    struct HalfRegs {
        f32x16 s;   // S, then P (fp32) in place
        f32x16 r;   // R = D - dP, then dS' in place
        u32x4 pb[2];  // P as bf16 pairs, B operands of dV
    };
    HalfRegs X, Y;
    u32x4 sb[2];      // dS' as bf16 pairs, B operands of dK
    // `ta` / `tc`: ring slots of the A-phase and C-phase tiles, `ha` / `hc` the
    // 32-query halves inside them; lv_next / dv_next the lse2 / D rows and qn
    // the first query of half g+1.
    // `carry`: the first PD operands of a step's first half step, read at the
    // end of the previous step (its tile was published by that step's
    // barrier), so that half step does not start on an LDS round trip.  The
    // second half step follows the barrier and reads its own.
    bf16x8 carry[C::PD];
    auto half_step = [&](auto masked, auto with_dma, HalfRegs& cur, HalfRegs& nxt,
                         const bf16 (*ta)[C::QTILE], int ha, const bf16 (*tc)[C::QTILE], int hc,
                         const bf16 (*tn)[C::QTILE], int hn,
                         const float* lv_next, const float* dv_next, int qn, int dma_q0, int dma_buf) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr bool DMA = decltype(with_dma)::value;
        bf16x8 opnd[C::NSLOT];
        f32x4 lvn[4], dvn[4];
        auto read_operand = [&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j < C::NA) {
                opnd[j] = lds_read8_b(ta[j < C::NKK ? 0 : 1], a_off[j % C::NKK] + ha * 32 * C::RB);
            } else if constexpr (j < C::NA + C::NC) {
                constexpr int cc = j - C::NA;
                const uint32_t rows = (hc * 32 + 16 * (cc / C::NDM)) * C::RB;
                opnd[j] = lds_tr_pair_b(tc[1], tr_lo[cc % C::NDM] + rows, tr_hi[cc % C::NDM] + rows);
            } else {
                constexpr int cc = j - C::NA - C::NC;
                const uint32_t rows = (hc * 32 + 16 * (cc / C::NDM)) * C::RB;
                opnd[j] = lds_tr_pair_b(tc[0], tr_lo[cc % C::NDM] + rows, tr_hi[cc % C::NDM] + rows);
            }
        };
        // P of half g+1, element r (row 8(r/4) + 4h + r%4 of the half)
        const float kq = LIN ? var.slope2 * (float)(my_key - 4 * h - qn) : 0.f;
        auto probs = [&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int qi = qn + 8 * (r / 4) + 4 * h + (r % 4);
            float z;
            if constexpr (LIN) z = __builtin_fmaf(nxt.s[r], c, kq - lvn[r / 4][r % 4]);
            else z = __builtin_fmaf(nxt.s[r], c, -lvn[r / 4][r % 4]);
            if constexpr (GEN) z += var.bias2(qi, my_key);
            float p = exp2f_hw(z);
            if constexpr (MASKED || GEN)
                p = ((CAUSAL && my_key > qi) || my_key >= N || (VAR && var.dead(qi, my_key))) ? 0.f : p;
            nxt.s[r] = p;
            if constexpr (r % 2 == 1) nxt.pb[r / 8][(r % 8) / 2] = cvt_pk_bf16(nxt.s[r - 1], p);
        };
        // the half step with the copies is the one after the barrier
        if constexpr (DMA) static_for<C::PD>([&](auto jc) { read_operand(jc); });
        else static_for<C::PD>([&](auto jc) { opnd[decltype(jc)::value] = carry[decltype(jc)::value]; });
        static_for<C::NSLOT>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j + C::PD < C::NSLOT) read_operand(std::integral_constant<int, j + C::PD>{});
            else if constexpr (DMA)
                carry[j + C::PD - C::NSLOT] = lds_read8_b(tn[0], a_off[j + C::PD - C::NSLOT] + hn * 32 * C::RB);
            if constexpr (j < C::NA) {
                // ---- S / R of half g+1; dS' of half g; lse2 / D rows of half g+1 ----
                if constexpr (j == 0) {
                    if constexpr (LIN) nxt.s = mfma32(opnd[j], kf[0], sinit);
                    else mfma32_zero(nxt.s, opnd[j], kf[0]);
                } else if constexpr (j < C::NKK) {
                    mfma32_acc(nxt.s, opnd[j], kf[j]);
                } else if constexpr (j == C::NKK) {
                    nxt.r = f32x16{dvn[0][0], dvn[0][1], dvn[0][2], dvn[0][3], dvn[1][0], dvn[1][1], dvn[1][2],
                                   dvn[1][3], dvn[2][0], dvn[2][1], dvn[2][2], dvn[2][3], dvn[3][0], dvn[3][1],
                                   dvn[3][2], dvn[3][3]};
                    mfma32_acc(nxt.r, opnd[j], vneg[0]);
                } else {
                    mfma32_acc(nxt.r, opnd[j], vneg[j - C::NKK]);
                }
                if constexpr (j < 4) dvn[j] = *reinterpret_cast<const f32x4*>(dv_next + 8 * j + 4 * h);
                else if constexpr (j < 8) lvn[j - 4] = *reinterpret_cast<const f32x4*>(lv_next + 8 * (j - 4) + 4 * h);
                static_for<slot_first<16, C::NA>(j + 1) - slot_first<16, C::NA>(j)>([&](auto ic) {
                    constexpr int r = slot_first<16, C::NA>(j) + decltype(ic)::value;
                    const float ds = cur.s[r] * cur.r[r];
                    cur.r[r] = ds;
                    if constexpr (r % 2 == 1) sb[r / 8][(r % 8) / 2] = cvt_pk_bf16(cur.r[r - 1], ds);
                });
            } else {
                constexpr int cc = j - C::NA;  // 0 .. 2 NC - 1
                if constexpr (cc < C::NC) {
                    // ---- dV += dO^T P of half g ----
                    dvacc[cc % C::NDM] =
                        mfma32(opnd[j], __builtin_bit_cast(bf16x8, cur.pb[cc / C::NDM]), dvacc[cc % C::NDM]);
                } else {
                    // ---- dK' += Q^T dS' of half g ----
                    constexpr int ck = cc - C::NC;
                    dkacc[ck % C::NDM] =
                        mfma32(opnd[j], __builtin_bit_cast(bf16x8, sb[ck / C::NDM]), dkacc[ck % C::NDM]);
                }
                // ---- P of half g+1 ----
                static_for<slot_first<16, 2 * C::NC>(cc + 1) - slot_first<16, 2 * C::NC>(cc)>([&](auto ic) {
                    probs(std::integral_constant<int, slot_first<16, 2 * C::NC>(cc) + decltype(ic)::value>{});
                });
            }
            if constexpr (DMA) {
                static_for<slot_first<C::NDMA, C::NSLOT>(j + 1) - slot_first<C::NDMA, C::NSLOT>(j)>([&](auto kc) {
                    dma_op(std::integral_constant<int, slot_first<C::NDMA, C::NSLOT>(j) + decltype(kc)::value>{},
                           dma_q0, dma_buf);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- prologue: tile 0 resident, tile 1 in flight; S, R and P of tile 0's first half ----
    dma_tile(step_q0(0), 0);
    wait_vmem();
    __syncthreads();
    dma_tile(step_q0(1), 1);
    {
        f32x4 l4[4], d4[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            l4[e] = *reinterpret_cast<const f32x4*>(&lvec[0][8 * e + 4 * h]);
            d4[e] = *reinterpret_cast<const f32x4*>(&dvec[0][8 * e + 4 * h]);
        }
        if constexpr (LIN) X.s = mfma32(lds_read8_b(ring[0][0], a_off[0]), kf[0], sinit);
        else mfma32_zero(X.s, lds_read8_b(ring[0][0], a_off[0]), kf[0]);
#pragma unroll
        for (int kk = 1; kk < C::NKK; kk++) mfma32_acc(X.s, lds_read8_b(ring[0][0], a_off[kk]), kf[kk]);
        X.r = f32x16{d4[0][0], d4[0][1], d4[0][2], d4[0][3], d4[1][0], d4[1][1], d4[1][2], d4[1][3],
                     d4[2][0], d4[2][1], d4[2][2], d4[2][3], d4[3][0], d4[3][1], d4[3][2], d4[3][3]};
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) mfma32_acc(X.r, lds_read8_b(ring[0][1], a_off[kk]), vneg[kk]);
        const int q0 = step_q0(0);
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int qi = q0 + 8 * (r / 4) + 4 * h + (r % 4);
            float z;
            if constexpr (LIN) z = __builtin_fmaf(X.s[r], c, var.slope2 * (float)(my_key - 4 * h - q0) - l4[r / 4][r % 4]);
            else z = __builtin_fmaf(X.s[r], c, -l4[r / 4][r % 4]);
            if constexpr (GEN) z += var.bias2(qi, my_key);
            float p = exp2f_hw(z);
            p = ((CAUSAL && my_key > qi) || my_key >= N || (VAR && var.dead(qi, my_key))) ? 0.f : p;
            X.s[r] = p;
        }
#pragma unroll
        for (int i = 0; i < 8; i++) X.pb[i / 4][i % 4] = cvt_pk_bf16(X.s[2 * i], X.s[2 * i + 1]);
#pragma unroll
        for (int j = 0; j < C::PD; j++) carry[j] = lds_read8_b(ring[0][0], a_off[j] + 32 * C::RB);
    }

    // Step st uses ring slot st % 3.  Its first half step computes S / R of
    // its own second half; its second half step, after the barrier that
    // publishes tile st+1, computes S / R / P of tile st+1's first half and
    // streams tile st+2 into the slot that tile st-1 occupied (every wave
    // finished it before that barrier).  Past the last tile the next-half work
    // runs on stale LDS contents and is discarded.
    int cur = 0;
    auto step = [&](auto masked, int st) {
        const int nxt = cur == 2 ? 0 : cur + 1;
        const int nn = nxt == 2 ? 0 : nxt + 1;
        const int q0 = step_q0(st);
        half_step(masked, std::false_type{}, X, Y, ring[cur], 1, ring[cur], 0, ring[nxt], 0, &lvec[cur][32],
                  &dvec[cur][32], q0 + 32, 0, 0);
        wait_vmem();  // this wave's copies of tile st+1 have landed
        __syncthreads();
        half_step(masked, std::true_type{}, Y, X, ring[nxt], 0, ring[cur], 1, ring[nxt], 1, &lvec[nxt][0],
                  &dvec[nxt][0], step_q0(st + 1), step_q0(st + 2), nn);
        cur = nxt;
    };

    int n_plain_end = nsteps;  // steps [n_masked, n_plain_end) take the unmasked path, the rest (VK = 1) masked
    if constexpr (LIN) {
        // Steps holding a dead pair form a prefix (diagonal, upper window edge)
        // and a suffix (lower window edge) of the increasing query order.  A
        // step's P work covers its own second half and the next tile's first
        // half, so the step before a dead one is masked too.
        auto dead_at = [&](int st) { return block_has_dead<CAUSAL>(step_q0(st), kBrq, k0, kBck, N, var); };
        int a = 0;
        while (a < nsteps && dead_at(a)) a++;
        int b = nsteps;
        while (b > a && dead_at(b - 1)) b--;
        n_masked = a;
        n_plain_end = b < nsteps ? max(a, b - 1) : nsteps;
    }
    int st = 0;
    for (; st < n_masked; st++) step(std::true_type{}, st);
    for (; st < n_plain_end; st++) step(std::false_type{}, st);
    if constexpr (LIN)
        for (; st < nsteps; st++) step(std::true_type{}, st);
    wait_vmem();  // copies past the last tile fetch nothing, but must retire before exit
    __syncthreads();  // every wave is done with the ring, which now stages the outputs

    // ---- epilogue: dK = -scale * acc, dV = acc, bf16 (rows >= N dropped) ----
    static_assert(kWaves * 2 * 32 * (D + 8) <= 3 * 2 * C::QTILE, "output staging must fit in the ring");
    bf16* const stage = &ring[0][0][0] + wave * 2 * 32 * (D + 8);
    const uint32_t rows_off = (uint32_t)(k0 + 32 * wave) * hd * 2;
    store_rows_staged<D>(dkacc, -scale, stage, make_rsrc(dK + head_off, head_bytes), rows_off, hd, lane);
    store_rows_staged<D>(dvacc, 1.0f, stage + 32 * (D + 8), make_rsrc(dV + head_off, head_bytes), rows_off, hd,
                         lane);
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
    static constexpr int RB = 2 * D;            // K tile: unpadded rows, 16-byte chunks swizzled (swz_sigma)
    static constexpr int VS = PadK<D>::STRIDE;  // V tile: 16-row b128 reads only
    static constexpr int KTILE = BC * D;
    static constexpr int VTILE = BC * VS;
    static constexpr int KSEGS = KTILE / 512;
    static constexpr int VSEGS = VTILE / 512;
    static_assert(KSEGS * 512 == KTILE && VSEGS * 512 == VTILE, "tiles must be whole 1 KB segments");
};
constexpr int kDqBr = 128;  // queries per workgroup

// The K tile is read both as rows (16 rows x 16 bytes per b128 operand read)
// and as columns (4 rows x 64 bytes per half-wave transposing read); no row
// padding keeps both free of bank conflicts, the chunk swizzle of swz<D> does.
// Lane i of 1 KB segment s fills LDS chunk position i of its row and fetches
// the logical chunk that position holds.
// (Rows hold hd <= D elements; a chunk past hd re-reads the row's first one:
// those tile columns only meet the zero columns of Q and dO or produce dQ
// columns that are not stored.)
template <int D, int SEGS>
__device__ __forceinline__ void dq_load_tile_swz(rsrc_t r, bf16* tile, int kv0, int hd, int wave, int lane) {
    constexpr int CPR = D / 8;  // chunks per row
#pragma unroll
    for (int i = 0; i < (SEGS + kWaves - 1) / kWaves; i++) {
        const int s = i * kWaves + wave;
        if (s < SEGS) {
            const int g = s * 64 + lane;  // chunk position in the tile
            const int row = g / CPR;
            const int col = 8 * chunk_at<D>(row, g % CPR);
            buf_load16_lds(r, tile + s * 512, ((uint32_t)(kv0 + row) * hd + (col < hd ? col : 0)) * 2);
        }
    }
}

template <int D, int STRIDE, int SEGS>
__device__ __forceinline__ void dq_load_tile(rsrc_t r, bf16* tile, int kv0, int hd, int wave, int lane) {
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

// VK as for the key-outer kernel; with VK = 1 the bias enters the exponent's
// addend, slope2 (kv0 + 32 kb + 4h - q) per 32-key block plus slope2 r' per element.
// PAD = false when the rows hold exactly D elements (the row length is then a
// compile-time constant, as the runtime one costs registers here).
//
// With O != null the kernel runs before the key-outer one and also does the
// preprocessing: for each of its query rows it computes D = rowsum(dO o O)
// and lse2 = lse log2(e) itself and stores them in the workspace rows that
// the key-outer kernel reads.  D is summed in exactly the order of
// rowdot_kernel (an FMA chain per 8-element chunk, then the chunks pairwise:
// 0+1, 2+3, ..., then those sums pairwise, and so on), so both orders of the
// stages give the same bits.
template <int D, bool CAUSAL, bool MASK, int VK, bool PAD>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ LSE2, float* __restrict__ Dv,
    bf16* __restrict__ dQ, int N, int hd_arg, float c, float scale, const uint8_t* __restrict__ mask, int nb,
    int nqb, int n_items, int H, int wl, int wr, const float* __restrict__ slopes) {
    using C = DqCfg<D>;
    const int hd = PAD ? hd_arg : D;
    constexpr bool VAR = VK != 0, LIN = VK == 1, GEN = VK == 2;
    __shared__ __attribute__((aligned(1024))) bf16 kbuf0[C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 kbuf1[C::KTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf0[C::VTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vbuf1[C::VTILE];
    __shared__ int wave_cnt[kWaves];
    extern __shared__ uint16_t mask_cols[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int v_lane = l32 * C::VS + 8 * h;  // V rows as the A operand of dP^T
    // Byte offsets in the swizzled K tile (loop invariant, per lane; rows 16
    // apart share a swizzle, so the 32-key block and 16-row half are immediates):
    //   k_off[kk]: row l32, logical chunk 2kk + h (b128 read of the S^T A operand);
    //   kt_lo/hi[dm]: rows 4h + j and 4h + j + 8, columns 32dm + 16g + 4q (the two
    //   transposing reads of the dQ^T A operand, see lds_tr_operand_pad).
    uint32_t k_off[C::NKK], kt_lo[C::NDM], kt_hi[C::NDM];
    {
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) k_off[kk] = l32 * C::RB + (chunk_pos<D>(l32, 2 * kk + h) << 4);
        const int sl = lane & 15, j = sl >> 2, q = sl & 3, g = (lane >> 4) & 1;
        const int r = 4 * h + j;
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) {
            const int cc = 4 * dm + 2 * g + (q >> 1);
            kt_lo[dm] = r * C::RB + (chunk_pos<D>(r, cc) << 4) + (q & 1) * 8;
            kt_hi[dm] = (r + 8) * C::RB + (chunk_pos<D>(r + 8, cc) << 4) + (q & 1) * 8;
        }
    }

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
    const size_t head_off = (size_t)bh * N * hd;
    const uint32_t head_bytes = (uint32_t)N * hd * 2;
    const rsrc_t rq = make_rsrc(Q + head_off, head_bytes);
    const rsrc_t rdo = make_rsrc(dO + head_off, head_bytes);
    const rsrc_t rk = make_rsrc(K + head_off, head_bytes);
    const rsrc_t rv = make_rsrc(V + head_off, head_bytes);
    const rsrc_t rdq = make_rsrc(dQ + head_off, head_bytes);
    const rsrc_t rl = make_rsrc(LSE2 + (size_t)bh * N, (uint32_t)N * 4);
    const rsrc_t rd = make_rsrc(Dv + (size_t)bh * N, (uint32_t)N * 4);
    Variant var{wl, wr, 0.f};
    if (VAR && slopes != nullptr) var.slope2 = slopes[bh % H] * kLog2e;

    for (int bi = 0; bi < nblk; bi++) {
        const int qb = qblk[bi];
        const int q0 = qb * kDqBr;
        const int qw = q0 + wave * 32;
        const int my_q = qw + l32;

        int ntiles;
        const uint16_t* cols = nullptr;
        const int q_end = min(N, q0 + kDqBr);
        int k_lo = 0, k_hi = CAUSAL ? q_end : N;  // keys this block can see
        if (VAR) {
            int lo, hi;
            var.key_range(q0, q_end, N, lo, hi);
            k_lo = lo;
            k_hi = min(k_hi, hi);
        }
        int k_first = 0;
        if (MASK) {
            const int lo_col = k_lo / kMaskBlock;
            const int max_col = k_hi > k_lo ? (k_hi - 1) / kMaskBlock : lo_col - 1;
            const int cnt = max_col >= lo_col ? build_block_list<kWaves>(mask + (size_t)qb * nb, 1, lo_col, max_col,
                                                                        mask_cols, wave_cnt)
                                              : 0;
            cols = mask_cols;
            ntiles = cnt * (kMaskBlock / C::BC);
        } else {
            k_first = k_lo;
            ntiles = k_hi > k_lo ? (k_hi - k_first + C::BC - 1) / C::BC : 0;
        }
        auto kv0_of = [&](int it) -> int {
            if (MASK) return cols[it / (kMaskBlock / C::BC)] * kMaskBlock + (it % (kMaskBlock / C::BC)) * C::BC;
            return k_first + it * C::BC;
        };

        // this lane's query: Q and dO fragments (B operands, k = head dim, n = query), lse2 and D
        // (columns past hd are zero)
        bf16x8 qf[C::NKK], of[C::NKK];
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) {
            const int col = 16 * kk + 8 * h;
            const uint32_t off = (uint32_t)(my_q * hd + (col < hd ? col : 0)) * 2;
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[kk] = __builtin_bit_cast(bf16x8, col < hd ? buf_load16(rq, off) : z);
            of[kk] = __builtin_bit_cast(bf16x8, col < hd ? buf_load16(rdo, off) : z);
        }
        float l2, dd;
        if (O != nullptr) {
            // ---- preprocessing of this block's rows (see above) ----
            const rsrc_t ro = make_rsrc(O + head_off, head_bytes);
            float cs[C::NKK];  // chunk 2kk + h of the row: FMA chain over its 8 elements
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) {
                const int col = 16 * kk + 8 * h;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const bf16x8 ob = __builtin_bit_cast(
                    bf16x8, col < hd ? buf_load16(ro, (uint32_t)(my_q * hd + col) * 2) : z);
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < 8; i++) a = __builtin_fmaf((float)ob[i], (float)of[kk][i], a);
                cs[kk] = a;
            }
            // chunks 2kk and 2kk + 1 sit in lanes l and l ^ 32: their sum (the
            // same bits in both lanes), then the pairwise tree over kk
#pragma unroll
            for (int kk = 0; kk < C::NKK; kk++) cs[kk] = xhalf_sum(cs[kk]);
#pragma unroll
            for (int w = 1; w < C::NKK; w <<= 1)
#pragma unroll
                for (int kk = 0; kk + w < C::NKK; kk += 2 * w) cs[kk] = cs[kk] + cs[kk + w];
            dd = cs[0];
            const float l = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4),
                                                     (uint32_t)my_q * 4, 0, 0));
            // a row without any allowed key (lse = -inf) gets +inf, so its P = 2^(c s - lse2) = 0
            l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
            if (h == 0 && my_q < N) {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dd), rd, (uint32_t)my_q * 4, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l2), rl, (uint32_t)my_q * 4, 0, 0);
            }
        } else {
            l2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)my_q * 4, 0, 0));
            dd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (uint32_t)my_q * 4, 0, 0));
        }
        const float ml2 = (my_q < N) ? -l2 : -INFINITY;  // rows past N get P = 0

        f32x16 acc[C::NDM];
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) acc[dm] = f32x16{};

        if (ntiles > 0) {
            dq_load_tile_swz<D, C::KSEGS>(rk, kbuf0, kv0_of(0), hd, wave, lane);
            dq_load_tile<D, C::VS, C::VSEGS>(rv, vbuf0, kv0_of(0), hd, wave, lane);
        }
        wait_vmem();
        __syncthreads();

        auto step = [&](auto parity, int it) {
            constexpr int P = decltype(parity)::value;
            const bf16* kt = P ? kbuf1 : kbuf0;
            const bf16* vt = P ? vbuf1 : vbuf0;
            const int kv0 = kv0_of(it);
            if (it + 1 < ntiles) {
                dq_load_tile_swz<D, C::KSEGS>(rk, P ? kbuf0 : kbuf1, kv0_of(it + 1), hd, wave, lane);
                dq_load_tile<D, C::VS, C::VSEGS>(rv, P ? vbuf0 : vbuf1, kv0_of(it + 1), hd, wave, lane);
            }
            const bool need_mask = GEN || (LIN ? block_has_dead<CAUSAL>(qw, 32, kv0, C::BC, N, var)
                                               : (CAUSAL && kv0 + C::BC - 1 > qw) || (kv0 + C::BC > N));
            // two 32-key halves, software-pipelined as in the key-outer kernel
            f32x16 s[2], dp[2];
            auto scores = [&](int kb) {  // S^T and dP^T for 32 keys (keys x queries)
                s[kb] = f32x16{};
                dp[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < C::NKK; kk++) {
                    s[kb] = mfma32(lds_read8_b(kt, k_off[kk] + 32 * kb * C::RB), qf[kk], s[kb]);
                    dp[kb] = mfma32(lds_read8(vt + v_lane, 32 * kb * C::VS + 16 * kk), of[kk], dp[kb]);
                }
            };
            bf16x8 sb[2][2];
            auto probs = [&](int kb) {  // P = 2^(c s - lse2), dS = P (dP - D)
                const float mlk = LIN ? __builtin_fmaf(var.slope2, (float)(kv0 + 32 * kb + 4 * h - my_q), ml2) : ml2;
                // exponentials, then the element mask under one branch (a select per
                // element inside the loop became a branch per element), then dS
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    float z;
                    if constexpr (LIN) z = __builtin_fmaf(s[kb][r], c, __builtin_fmaf(var.slope2, (float)row_in_block(r), mlk));
                    else z = __builtin_fmaf(s[kb][r], c, ml2);
                    if constexpr (GEN) z += var.bias2(my_q, key);
                    p[r] = exp2f_hw(z);
                }
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        p[r] = ((CAUSAL && key > my_q) || key >= N || (VAR && var.dead(my_q, key))) ? 0.f : p[r];
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; r++) dp[kb][r] = p[r] * (dp[kb][r] - dd);
                sb[kb][0] = pack8<0>(dp[kb]);
                sb[kb][1] = pack8<8>(dp[kb]);
            };
            auto grads = [&](int kb) {  // dQ^T += K^T dS^T
#pragma unroll
                for (int half = 0; half < 2; half++)
#pragma unroll
                    for (int dm = 0; dm < C::NDM; dm++)
                        acc[dm] = mfma32(lds_tr_pair_b(kt, kt_lo[dm] + (32 * kb + 16 * half) * C::RB,
                                                       kt_hi[dm] + (32 * kb + 16 * half) * C::RB),
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

        // dQ = scale * acc -> bf16 (rows >= N dropped), staged in the V tiles, which
        // every wave finished reading before the last step's barrier
        static_assert(2 * 32 * (D + 8) <= C::VTILE, "output staging must fit in the V tiles");
        bf16* const stage = (wave < 2 ? vbuf0 : vbuf1) + (wave & 1) * 32 * (D + 8);
        store_rows_staged<D>(acc, scale, stage, rdq, (uint32_t)qw * hd * 2, hd, lane);
        __syncthreads();  // the staging is read before the next block's tiles land there
    }
}

template <int D, bool CAUSAL, bool MASK, int VK, bool PAD>
hipError_t launch_dq_pad(const BwdArgs& a, bool fused) {
    const int nqb = (a.N + kDqBr - 1) / kDqBr;
    const int per_head = CAUSAL ? (nqb + 1) / 2 : nqb;
    const int n_items = a.BH * per_head;
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = bwd_dq_kernel<D, CAUSAL, MASK, VK, PAD>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads), dyn, a.stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (const bf16*)a.dO, fused ? (const bf16*)a.o : nullptr, a.lse, a.ws_lse2,
                       a.ws_D, (bf16*)a.dq, a.N, a.d, a.scale * kLog2e, a.scale, a.mask, a.nb, nqb, n_items, a.H,
                       a.wl, a.wr, a.slopes);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK, int VK>
hipError_t launch_dq(const BwdArgs& a, bool fused) {
    return a.d == D ? launch_dq_pad<D, CAUSAL, MASK, VK, false>(a, fused)
                    : launch_dq_pad<D, CAUSAL, MASK, VK, true>(a, fused);
}

template <int D, bool CAUSAL, bool MASK, int VK>
hipError_t launch_main(const BwdArgs& a) {
    const int nkb = (a.N + kBck - 1) / kBck;
    const int n_items = a.BH * nkb;
    const size_t dyn = MASK ? (size_t)a.nb * sizeof(uint16_t) : 0;
    auto kern = bwd_bf16_kernel<D, CAUSAL, MASK, VK>;
    if (dyn > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(kThreads), dyn, a.stream, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (const bf16*)a.dO, a.ws_lse2, a.ws_D, (bf16*)a.dk, (bf16*)a.dv,
                       a.N, a.d, a.scale * kLog2e, a.scale, a.mask, a.nb, nkb, a.BH, a.H, a.wl, a.wr, a.slopes);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const BwdArgs& a) {
    const long rows = (long)a.BH * a.N;
    const long nthr = rows * rowdot_lanes<D>();
    hipLaunchKernelGGL(rowdot_kernel<D>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, a.stream,
                       (const bf16*)a.o, (const bf16*)a.dO, a.lse, a.ws_D, a.ws_lse2, rows, a.d);
    return hipGetLastError();
}

template <int D, int VK>
hipError_t launch_main_all(const BwdArgs& a) {
    const bool m = a.mask != nullptr;
    if (a.causal) return m ? launch_main<D, true, true, VK>(a) : launch_main<D, true, false, VK>(a);
    return m ? launch_main<D, false, true, VK>(a) : launch_main<D, false, false, VK>(a);
}

template <int D, int VK>
hipError_t launch_dq_all(const BwdArgs& a, bool fused) {
    const bool m = a.mask != nullptr;
    if (a.causal) return m ? launch_dq<D, true, true, VK>(a, fused) : launch_dq<D, true, false, VK>(a, fused);
    return m ? launch_dq<D, false, true, VK>(a, fused) : launch_dq<D, false, false, VK>(a, fused);
}

hipError_t launch_dq_any(const BwdArgs& a, bool fused);

// The tile width that holds a row: 64, 96 or 128.
template <typename F, typename... A>
hipError_t by_width(const BwdArgs& a, F w64, F w96, F w128, A... rest) {
    return a.d <= 64 ? w64(a, rest...) : a.d <= 96 ? w96(a, rest...) : w128(a, rest...);
}

// The ALiBi bias is linear in the key over the live pairs only when they all
// precede their query; the key-outer kernel also divides the slope by c.
int variant_kind(const BwdArgs& a, bool divides_by_c) {
    if (!a.variant()) return 0;
    if (a.slopes == nullptr) return 1;
    if (!a.causal) return 2;
    return (divides_by_c && fabsf(a.scale * kLog2e) < 0x1p-40f) ? 2 : 1;
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const BwdArgs& a) {
    return a.d <= 64 ? launch_prep<64>(a) : a.d <= 96 ? launch_prep<96>(a) : launch_prep<128>(a);
}

hipError_t launch_bwd_main_bf16(const BwdArgs& a) {
    switch (variant_kind(a, true)) {
        case 0: return by_width(a, launch_main_all<64, 0>, launch_main_all<96, 0>, launch_main_all<128, 0>);
        case 1: return by_width(a, launch_main_all<64, 1>, launch_main_all<96, 1>, launch_main_all<128, 1>);
        default: return by_width(a, launch_main_all<64, 2>, launch_main_all<96, 2>, launch_main_all<128, 2>);
    }
}

namespace {
hipError_t launch_dq_any(const BwdArgs& a, bool fused) {
    switch (variant_kind(a, false)) {
        case 0: return by_width(a, launch_dq_all<64, 0>, launch_dq_all<96, 0>, launch_dq_all<128, 0>, fused);
        case 1: return by_width(a, launch_dq_all<64, 1>, launch_dq_all<96, 1>, launch_dq_all<128, 1>, fused);
        default: return by_width(a, launch_dq_all<64, 2>, launch_dq_all<96, 2>, launch_dq_all<128, 2>, fused);
    }
}
}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdArgs& a) { return launch_dq_any(a, false); }

hipError_t launch_bwd_dq_first_bf16(const BwdArgs& a) { return launch_dq_any(a, true); }

unsigned debug_flags_bwd(bool clear) { return read_debug_flags(clear); }

// dQ first (it also writes D and lse2), then dK and dV: the preprocessing
// pass and its launch are saved; the results are those of prep, main, dQ.
hipError_t launch_bwd_bf16(const BwdArgs& a) {
    hipError_t e = launch_bwd_dq_first_bf16(a);
    if (e != hipSuccess) return e;
    return launch_bwd_main_bf16(a);
}

}  // namespace fa
