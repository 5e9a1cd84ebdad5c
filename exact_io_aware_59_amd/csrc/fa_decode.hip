// Decode over a paged KV cache for bf16 on gfx950.
//
// A few new queries per sequence attend to that sequence's whole KV cache,
// which lives in fixed-size pages named by a page table ("FlashAttention 深度
// 解析" section 五: since version 2.5 FlashAttention reads the paged layout
// PagedAttention manages; "FlashAttention原理概览" section 3.2: inference
// needs no score matrix, only the cache).  The work is a stream over the
// cache: every K and V byte is read once, and at a handful of queries per KV
// head the matrix work per byte is tiny, so HBM bandwidth is the bound.
//
// Split along the keys ("FlashAttention 深度解析" section 二: partial results
// over disjoint key ranges merge exactly with the running max / sum rule):
//   1. decode_kernel: one wave per (sequence, KV head, group of 32 query rows,
//      key range).  The query rows of a KV head (its grouped query heads times
//      the new positions) are the 32 columns of S^T = K Q^T; per 32-key tile
//      the wave computes S^T on the matrix cores, folds it into its running
//      max and sum and accumulates O^T += V^T P^T, like the forward kernel.
//      K tiles go from HBM straight into registers (their rows are the MFMA A
//      operand); V tiles go HBM -> LDS by buffer_load ... lds into a swizzled
//      per-wave ring of two and are read transposed; the next tile is in
//      flight while one is computed, and two workgroups (eight waves) share a
//      CU.  The wave writes (O unnormalized, max,
//      sum) for its key range, or the final O and lse when one range covers
//      the sequence.
//   2. decode_merge_kernel: per query row (one wave), O = sum_p w_p O_p /
//      sum_p w_p l_p with w_p = 2^(m_p - max_p m_p), lse = ln 2 (max + log2 sum).
// Rows past a sequence's length and pages outside the cache read as zero
// (buffer range checks), so nothing outside the caller's buffers is touched.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// Transposing pair read (A operand of O^T += V^T P^T) at two byte offsets of a swizzled tile.
__device__ __forceinline__ bf16x8 lds_tr_pair_v(const bf16* base, uint32_t lo_off, uint32_t hi_off) {
    const bf16x4 lo = lds_read_tr4(base, lo_off / 2);
    const bf16x4 hi = lds_read_tr4(base, hi_off / 2);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecBC = 32;     // keys per tile
constexpr int kDecStages = 2;  // per-wave ring: the tile being computed and the next in flight
constexpr float kDecRescale = 8.0f;

template <int D>
struct DecCfg {
    static constexpr int NKK = D / 16;          // k-steps of S^T over the head dimension
    static constexpr int NDM = D / 32;          // 32-dim blocks of O^T
    static constexpr int RB = 2 * D;            // bytes per V tile row (unpadded, swizzled)
    static constexpr int VTILE = kDecBC * D;    // elements of a V tile
    static constexpr int VSEGS = VTILE / 512;   // 1 KB copies per V tile
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static_assert(VSEGS * 512 == VTILE, "a V tile must be whole 1 KB copies");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ seqlens, bf16* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ ws_o, float* __restrict__ ws_ml, int H, int Hkv, int Nq,
    int page_size, int max_pages, int num_pages, int nqg, int n_parts, int kpp, int n_items, float c,
    uint32_t qsign) {
    using C = DecCfg<D>;
    // the two V slots are separate arrays so the compiler can tell the copy
    // in flight into one from the reads of another (it then waits for exactly
    // the copies a tile needs)
    __shared__ __attribute__((aligned(1024))) bf16 vring0[kDecWaves][C::VTILE];
    __shared__ __attribute__((aligned(1024))) bf16 vring1[kDecWaves][C::VTILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int item = blockIdx.x * kDecWaves + wave;
    if (item >= n_items) return;
    // item -> (sequence b, KV head hk, query group qg, key range part), part fastest
    const int part = item % n_parts;
    int rest = item / n_parts;
    const int qg = rest % nqg;
    rest /= nqg;
    const int hk = rest % Hkv;
    const int b = rest / Hkv;
    const int G = H / Hkv;
    const int L = max(0, min(seqlens[b], max_pages * page_size));
    const int k_begin = part * kpp;
    const int k_end = min(L, k_begin + kpp);

    // ---- this lane's query row: (grouped head g, new position qi) ----
    const int R = qg * 32 + l32;
    const bool row_ok = R < G * Nq;
    const int g = row_ok ? R / Nq : 0, qi = row_ok ? R % Nq : 0;
    const size_t row_id = ((size_t)b * H + (size_t)hk * G + g) * Nq + qi;
    if (k_begin >= k_end) {
        // an empty range: the merge does not read it; a sequence without keys
        // written directly gets O = 0 and lse = -inf
        if (n_parts == 1 && row_ok) {
            bf16* orow = O + row_id * D;
            for (int c0 = 4 * h; c0 < D; c0 += 8) *reinterpret_cast<u32x2*>(orow + c0) = u32x2{0u, 0u};
            if (h == 0) LSE[row_id] = -INFINITY;
        }
        return;
    }
    const int nt = (k_end - k_begin + kDecBC - 1) / kDecBC;
    const int last_key = CAUSAL ? L - Nq + qi : L - 1;  // keys 0 .. last_key are allowed (and < k_end here)
    bf16x8 qf[C::NKK];  // B operand of S^T = K Q^T (k = head dim, n = query)
    {
        const u32x4* qrow = reinterpret_cast<const u32x4*>(Q + row_id * D + 8 * h);
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) {
            u32x4 raw = row_ok ? qrow[2 * kk] : u32x4{0u, 0u, 0u, 0u};
            qf[kk] = __builtin_bit_cast(bf16x8, raw ^ qsign);
        }
    }

    // ---- where tile t lives: one page of the sequence, rows past k_end read as zero ----
    struct TileSrc {
        const bf16* kbase;
        const bf16* vbase;
        uint32_t bytes;
    };
    auto tile_src = [&](int t) -> TileSrc {
        const int t0 = k_begin + kDecBC * t;
        const int rows = t < nt ? min(kDecBC, k_end - t0) : 0;
        const int lp = min(t0 / page_size, max_pages - 1);
        const int pg = block_table[(size_t)b * max_pages + lp];
        const bool ok = rows > 0 && pg >= 0 && pg < num_pages;
        const size_t row0 = ok ? (size_t)pg * page_size + (t0 % page_size) : 0;
        const size_t off = (row0 * Hkv + hk) * D;
        return TileSrc{Kc + off, Vc + off, ok ? (uint32_t)rows * Hkv * D * 2 : 0u};
    };
    const uint32_t row_stride = (uint32_t)Hkv * D * 2;  // bytes between consecutive keys of one head

    // K rows as MFMA A operands: lane l holds key l32, columns 16 kk + 8h .. + 7
    bf16x8 kreg[kDecStages][C::NKK];
    // V copy: segment i of a tile, lane -> (row, logical chunk (lane % CPR) ^ sigma(row))
    uint32_t v_off[C::VSEGS];
#pragma unroll
    for (int i = 0; i < C::VSEGS; i++) {
        const int row = i * (512 / D) + lane / C::CPR;
        const int chunk = (lane % C::CPR) ^ swz_sigma<D>(row & 15);
        v_off[i] = (uint32_t)row * row_stride + (uint32_t)chunk * 16;
    }
    auto slot_of = [&](auto sc) -> bf16* {
        constexpr int s = decltype(sc)::value;
        return s == 0 ? &vring0[wave][0] : &vring1[wave][0];
    };
    auto issue = [&](auto sc, int t) {
        constexpr int s = decltype(sc)::value;
        const TileSrc src = tile_src(t);
        const rsrc_t rk = make_rsrc(src.kbase, src.bytes);
        const uint32_t koff = (uint32_t)l32 * row_stride + 16u * h;
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) kreg[s][kk] = __builtin_bit_cast(bf16x8, buf_load16(rk, koff + 32u * kk));
        const rsrc_t rv = make_rsrc(src.vbase, src.bytes);
        bf16* dst = slot_of(sc);
#pragma unroll
        for (int i = 0; i < C::VSEGS; i++) buf_load16_lds(rv, dst + 512 * i, v_off[i]);
    };

    // transposing-read offsets of V^T as the A operand of O^T += V^T P^T
    uint32_t tr_lo[C::NDM], tr_hi[C::NDM];
    {
        const int sl = lane & 15, j = sl >> 2, q = sl & 3, gq = (lane >> 4) & 1;
        const int r = 4 * h + j;
        const int slo = swz_sigma<D>(r), shi = swz_sigma<D>(r + 8);
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++) {
            const int cc = 4 * dm + 2 * gq + (q >> 1);
            tr_lo[dm] = r * C::RB + ((cc ^ slo) << 4) + (q & 1) * 8;
            tr_hi[dm] = (r + 8) * C::RB + ((cc ^ shi) << 4) + (q & 1) * 8;
        }
    }

    f32x16 oacc[C::NDM];
#pragma unroll
    for (int dm = 0; dm < C::NDM; dm++) oacc[dm] = f32x16{};
    float m_ref = -INFINITY;  // reference max of raw scores (moves lazily)
    float l_part = 0.f;       // this lane's half of the running sum

    // One tile from ring slot s (the compiler waits for exactly its loads; the
    // next tile stays in flight), then refill the slot with tile t + 2.  A tile
    // past the range (the last round of two) reads zeros, is masked out
    // completely and costs matrix work only.
    auto tile = [&](auto sc, int t) {
        constexpr int s = decltype(sc)::value;
        const int t0 = k_begin + kDecBC * t;
        f32x16 sv = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::NKK; kk++) sv = mfma32(kreg[s][kk], qf[kk], sv);
        if (t0 + kDecBC > k_end || (CAUSAL && t0 + kDecBC - 1 > L - Nq)) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int key = t0 + 8 * (r >> 2) + 4 * h + (r & 3);
                sv[r] = (key > last_key || key >= k_end) ? -INFINITY : sv[r];
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 16; r++) mx = fmaxf(mx, sv[r]);
        mx = xhalf_max(mx);
        const float m_new = fmaxf(m_ref, mx);
        const bool bump = m_new != -INFINITY && (m_ref == -INFINITY || (m_new - m_ref) * c > kDecRescale);
        if (__builtin_expect(__ballot(bump) != 0, 0)) {
            const float alpha = bump ? (m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - m_new) * c)) : 1.f;
            if (bump) m_ref = m_new;
            l_part *= alpha;
#pragma unroll
            for (int dm = 0; dm < C::NDM; dm++) oacc[dm] *= alpha;
        }
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
        u32x4 pb[2];
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2f_hw(__builtin_fmaf(sv[r], c, -mc));
            const float p1 = exp2f_hw(__builtin_fmaf(sv[r + 1], c, -mc));
            ls[0] += p0;
            ls[1] += p1;
            pb[r / 8][(r % 8) / 2] = cvt_pk_bf16(p0, p1);
        }
        l_part += ls[0] + ls[1];
        const bf16* vt = slot_of(sc);
#pragma unroll
        for (int k16 = 0; k16 < 2; k16++)
#pragma unroll
            for (int dm = 0; dm < C::NDM; dm++)
                oacc[dm] = mfma32(lds_tr_pair_v(vt, tr_lo[dm] + 16u * k16 * C::RB, tr_hi[dm] + 16u * k16 * C::RB),
                                  __builtin_bit_cast(bf16x8, pb[k16]), oacc[dm]);
        issue(sc, t + kDecStages);
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    for (int t = 0; t < nt; t += kDecStages) {
        tile(std::integral_constant<int, 0>{}, t);
        tile(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vmem();  // copies past the last tile fetch nothing but must retire before the wave ends

    // ---- epilogue ----
    const float l = xhalf_sum(l_part);
    if (n_parts == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (row_ok) {
            bf16* orow = O + row_id * D;
#pragma unroll
            for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    bf16x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; e++) v4[e] = (bf16)(oacc[dm][4 * gq + e] * inv);
                    *reinterpret_cast<bf16x4*>(orow + 32 * dm + 8 * gq + 4 * h) = v4;
                }
            if (h == 0) LSE[row_id] = l > 0.f ? (m_ref * c + log2f_hw(l)) * kLn2 : -INFINITY;
        }
    } else if (row_ok) {
        float* wo = ws_o + (row_id * n_parts + part) * D;
#pragma unroll
        for (int dm = 0; dm < C::NDM; dm++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++)
                *reinterpret_cast<f32x4*>(wo + 32 * dm + 8 * gq + 4 * h) =
                    f32x4{oacc[dm][4 * gq], oacc[dm][4 * gq + 1], oacc[dm][4 * gq + 2], oacc[dm][4 * gq + 3]};
        if (h == 0) {
            float* ml = ws_ml + (row_id * n_parts + part) * 2;
            ml[0] = m_ref == -INFINITY ? -INFINITY : m_ref * c;  // log2 units
            ml[1] = l;
        }
    }
}

// Per query row: merge the key ranges' (O, max, sum).  One wave per row: the
// lanes take the ranges' maxima in parallel (wave max), then every lane owns
// D/64 output columns and sums the ranges' partial rows with their weights.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_ml,
                                                           const int* __restrict__ seqlens, bf16* __restrict__ O,
                                                           float* __restrict__ LSE, int rows, int H, int Nq,
                                                           int n_parts, int kpp, int max_keys) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int b = row / (H * Nq);
    const int L = max(0, min(seqlens[b], max_keys));
    const int nvalid = min(n_parts, (L + kpp - 1) / kpp);
    const float* ml = ws_ml + (size_t)row * n_parts * 2;
    float M = -INFINITY;
    for (int p = lane; p < nvalid; p += 64) M = fmaxf(M, ml[2 * p]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; e++) acc[e] = 0.f;
    float lsum = 0.f;
    if (M != -INFINITY) {
        const float* src = ws_o + (size_t)row * n_parts * D + lane * PER;
        int p = 0;
        for (; p + 4 <= nvalid; p += 4) {  // four ranges' loads in flight
            float w[4], ov[4][PER];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                w[u] = ml[2 * (p + u)];
#pragma unroll
                for (int e = 0; e < PER; e++) ov[u][e] = src[(size_t)(p + u) * D + e];
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const float wu = exp2f_hw(w[u] - M);  // 0 for a range with no allowed key
                lsum += wu * ml[2 * (p + u) + 1];
#pragma unroll
                for (int e = 0; e < PER; e++) acc[e] += wu * ov[u][e];
            }
        }
        for (; p < nvalid; p++) {
            const float wu = exp2f_hw(ml[2 * p] - M);
            lsum += wu * ml[2 * p + 1];
#pragma unroll
            for (int e = 0; e < PER; e++) acc[e] += wu * src[(size_t)p * D + e];
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int e = 0; e < PER; e++) O[(size_t)row * D + lane * PER + e] = (bf16)(acc[e] * inv);
    if (lane == 0) LSE[row] = lsum > 0.f ? (M + log2f_hw(lsum)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_decode_d(const DecArgs& a) {
    const int G = a.H / a.Hkv;
    const int nqg = (G * a.Nq + 31) / 32;
    const int n_items = a.B * a.Hkv * nqg * a.n_parts;
    const int blocks = (n_items + kDecWaves - 1) / kDecWaves;
    hipLaunchKernelGGL((decode_kernel<D, CAUSAL>), dim3(blocks), dim3(kDecThreads), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.block_table, a.seqlens,
                       (bf16*)a.o, a.lse, a.ws_o, a.ws_ml, a.H, a.Hkv, a.Nq, a.page_size, a.max_pages, a.num_pages,
                       nqg, a.n_parts, a.kpp, n_items, a.c, a.qsign);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_parts == 1) return e;
    const int rows = a.B * a.H * a.Nq;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, a.stream, a.ws_o, a.ws_ml,
                       a.seqlens, (bf16*)a.o, a.lse, rows, a.H, a.Nq, a.n_parts, a.kpp, a.max_pages * a.page_size);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecArgs& a) {
    if (a.d == 128) return a.causal ? launch_decode_d<128, true>(a) : launch_decode_d<128, false>(a);
    return a.causal ? launch_decode_d<64, true>(a) : launch_decode_d<64, false>(a);
}

}  // namespace fa
