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
//   1. decode_kernel: one wave per (sequence, KV head, group of 16 query rows,
//      key range).  The query rows of a KV head (its grouped query heads times
//      the new positions) are the 16 columns of S^T = K Q^T on 16x16x32
//      products: with a handful of useful rows, the narrow shape halves the
//      matrix and softmax work per K/V byte against 32-wide products.  Per
//      32-key tile the wave computes S^T, folds it into its running max and
//      sum and accumulates O^T += V^T P^T.  K rows go from HBM straight into
//      registers (their rows are the A operand, 64 contiguous bytes per row
//      and load); V rows go HBM -> LDS by buffer_load ... lds into padded rows
//      and are read transposed in the key order of the S^T results, so P
//      never leaves registers.  The next tile is in flight while one is
//      computed; a workgroup is eight waves (one per CU).  The wave
//      writes (O unnormalized, max, sum) for its key range, or the final O
//      and lse when one range covers the sequence.
//   2. decode_merge_kernel: per query row (one wave), O = sum_p w_p O_p /
//      sum_p w_p l_p with w_p = 2^(m_p - max_p m_p), lse = ln 2 (max + log2 sum).
// Rows past a sequence's length and pages outside the cache read as zero
// (buffer range checks), so nothing outside the caller's buffers is touched.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecBC = 32;     // keys per tile (two 16-key blocks)
constexpr int kDecRows = 16;   // query rows per wave (the N of the 16x16x32 products)
constexpr int kDecStages = 2;  // per-wave ring: the tile being computed and the next in flight
constexpr float kDecRescale = 8.0f;

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int D>
struct DecCfg {
    static constexpr int NK = D / 32;           // k-steps of S^T (32 dims each)
    static constexpr int NDB = D / 16;          // 16-dim blocks of O^T
    static constexpr int VS = 2 * D + 32;       // bytes per V tile row in LDS (32 mod 256: transposing reads)
    static constexpr int VTILE = kDecBC * VS;   // bytes of a V tile
    static constexpr int VSEGS = VTILE / 1024;  // 1 KB copies per V tile
    static_assert(VSEGS * 1024 == VTILE, "a V tile must be whole 1 KB copies");
};

__device__ __forceinline__ f32x4v mfma16(bf16x8 a, bf16x8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Max / sum over the four lanes that hold the same query (l, l^16, l^32, l^48).
__device__ __forceinline__ float xquad_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float xquad_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDecThreads, 1) void decode_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ seqlens, bf16* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ ws_o, float* __restrict__ ws_ml, int H, int Hkv, int Nq,
    int page_size, int max_pages, int num_pages, int nqg, int n_parts, int kpp, int n_items, float c,
    uint32_t qsign) {
    using C = DecCfg<D>;
    // the two V slots are separate arrays so the compiler can tell the copy
    // in flight into one from the reads of another (it then waits for exactly
    // the copies a tile needs)
    __shared__ __attribute__((aligned(1024))) uint8_t vring0[kDecWaves][C::VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vring1[kDecWaves][C::VTILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gq = lane >> 4, l16 = lane & 15;  // k group of the operands / row group of the results
    const int item = blockIdx.x * kDecWaves + wave;
    if (item >= n_items) return;
    // item -> (sequence b, query group qg, key range part, KV head hk), KV head
    // fastest: the waves of a workgroup read the same cache rows' other heads
    // at the same time, which keeps the HBM accesses close together
    const int hk = item % Hkv;
    int rest = item / Hkv;
    const int part = rest % n_parts;
    rest /= n_parts;
    const int qg = rest % nqg;
    const int b = rest / nqg;
    const int G = H / Hkv;
    const int L = max(0, min(seqlens[b], max_pages * page_size));
    const int k_begin = part * kpp;
    const int k_end = min(L, k_begin + kpp);

    // ---- this lane's query row (the 16 columns; four lanes share each) ----
    const int R = qg * kDecRows + l16;
    const bool row_ok = R < G * Nq;
    const int g = row_ok ? R / Nq : 0, qi = row_ok ? R % Nq : 0;
    const size_t row_id = ((size_t)b * H + (size_t)hk * G + g) * Nq + qi;
    if (k_begin >= k_end) {
        // an empty range: the merge does not read it; a sequence without keys
        // written directly gets O = 0 and lse = -inf
        if (n_parts == 1 && row_ok) {
            bf16* orow = O + row_id * D;
            for (int c0 = 4 * gq; c0 < D; c0 += 16) *reinterpret_cast<u32x2*>(orow + c0) = u32x2{0u, 0u};
            if (gq == 0) LSE[row_id] = -INFINITY;
        }
        return;
    }
    const int nt = (k_end - k_begin + kDecBC - 1) / kDecBC;
    const int last_key = CAUSAL ? L - Nq + qi : L - 1;  // keys 0 .. last_key are allowed (and < k_end here)
    bf16x8 qf[C::NK];  // B operand of S^T = K Q^T: query l16, dims 32 kk + 8 gq .. + 7
    {
        const u32x4* qrow = reinterpret_cast<const u32x4*>(Q + row_id * D + 8 * gq);
#pragma unroll
        for (int kk = 0; kk < C::NK; kk++) {
            u32x4 raw = row_ok ? qrow[4 * kk] : u32x4{0u, 0u, 0u, 0u};
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

    // K rows as A operands of the 16x16x32 products: block mb holds keys 16 mb + l16,
    // dims 32 kk + 8 gq .. + 7 (each load: 16 rows x 64 contiguous bytes)
    bf16x8 kreg[kDecStages][2][C::NK];
    const uint32_t k_off = (uint32_t)l16 * row_stride + 16u * gq;
    // V copy into padded rows: segment i, lane -> (row, byte column); padding lanes re-read column 0
    uint32_t v_off[C::VSEGS];
#pragma unroll
    for (int i = 0; i < C::VSEGS; i++) {
        const int el = i * 1024 + lane * 16;
        const int row = el / C::VS;
        int col = el - row * C::VS;
        col = col < 2 * D ? col : 0;
        v_off[i] = (uint32_t)row * row_stride + (uint32_t)col;
    }
    auto slot_of = [&](auto sc) -> uint8_t* {
        constexpr int s = decltype(sc)::value;
        return s == 0 ? &vring0[wave][0] : &vring1[wave][0];
    };
    auto issue = [&](auto sc, int t) {
        constexpr int s = decltype(sc)::value;
        const TileSrc src = tile_src(t);
        const rsrc_t rk = make_rsrc(src.kbase, src.bytes);
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int kk = 0; kk < C::NK; kk++)
                kreg[s][mb][kk] =
                    __builtin_bit_cast(bf16x8, buf_load16(rk, k_off + 16u * row_stride * mb + 64u * kk));
        const rsrc_t rv = make_rsrc(src.vbase, src.bytes);
        uint8_t* dst = slot_of(sc);
#pragma unroll
        for (int i = 0; i < C::VSEGS; i++) buf_load16_lds(rv, dst + 1024 * i, v_off[i]);
    };
    // V^T as the A operand of O^T += V^T P^T, dims 16 db + l16: the transposing read of
    // block mb gives keys 16 mb + 4 gq + j (j = 0..3), the key order of the S^T results
    const uint32_t v_tr = (uint32_t)(4 * gq + (l16 >> 2)) * C::VS + 8u * (l16 & 3);

    f32x4v oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; db++) oacc[db] = f32x4v{};
    float m_ref = -INFINITY;  // reference max of raw scores (moves lazily)
    float l_part = 0.f;       // this lane's quarter of the running sum

    // One tile from ring slot s (the compiler waits for exactly its loads; the
    // next tile stays in flight), then refill the slot with tile t + 2.  A tile
    // past the range (the last round of two) reads zeros, is masked out
    // completely and costs matrix work only.
    auto tile = [&](auto sc, int t) {
        constexpr int s = decltype(sc)::value;
        const int t0 = k_begin + kDecBC * t;
        f32x4v sv[2];
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
            sv[mb] = f32x4v{};
#pragma unroll
            for (int kk = 0; kk < C::NK; kk++) sv[mb] = mfma16(kreg[s][mb][kk], qf[kk], sv[mb]);
        }
        // result (mb, r): key t0 + 16 mb + 4 gq + r, query l16
        if (t0 + kDecBC > k_end || (CAUSAL && t0 + kDecBC - 1 > L - Nq)) {
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int key = t0 + 16 * mb + 4 * gq + r;
                    sv[mb][r] = (key > last_key || key >= k_end) ? -INFINITY : sv[mb][r];
                }
        }
        float mx = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                         fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
        mx = xquad_max(mx);
        const float m_new = fmaxf(m_ref, mx);
        const bool bump = m_new != -INFINITY && (m_ref == -INFINITY || (m_new - m_ref) * c > kDecRescale);
        if (__builtin_expect(__ballot(bump) != 0, 0)) {
            const float alpha = bump ? (m_ref == -INFINITY ? 0.f : exp2f_hw((m_ref - m_new) * c)) : 1.f;
            if (bump) m_ref = m_new;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < C::NDB; db++) oacc[db] *= alpha;
        }
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
        u32x4 pb;  // P^T as the B operand: element 4 mb + r is key 16 mb + 4 gq + r
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; r++) p[r] = exp2f_hw(__builtin_fmaf(sv[mb][r], c, -mc));
            l_part += (p[0] + p[1]) + (p[2] + p[3]);
            pb[2 * mb] = cvt_pk_bf16(p[0], p[1]);
            pb[2 * mb + 1] = cvt_pk_bf16(p[2], p[3]);
        }
        const uint8_t* vt = slot_of(sc);
#pragma unroll
        for (int db = 0; db < C::NDB; db++) {
            const bf16x4 lo = lds_read_tr4(reinterpret_cast<const bf16*>(vt), (v_tr + 32u * db) / 2);
            const bf16x4 hi = lds_read_tr4(reinterpret_cast<const bf16*>(vt), (v_tr + 16u * C::VS + 32u * db) / 2);
            const bf16x8 va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[db] = mfma16(va, __builtin_bit_cast(bf16x8, pb), oacc[db]);
        }
        issue(sc, t + kDecStages);
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    for (int t = 0; t < nt; t += kDecStages) {
        tile(std::integral_constant<int, 0>{}, t);
        tile(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vmem();  // copies past the last tile fetch nothing but must retire before the wave ends

    // ---- epilogue: result (db, r) is dim 16 db + 4 gq + r of query l16 ----
    const float l = xquad_sum(l_part);
    if (row_ok) FA_CHECK(m_ref == -INFINITY || l > 0.f, kDbgRowSum);
    if (n_parts == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (row_ok) {
            bf16* orow = O + row_id * D;
#pragma unroll
            for (int db = 0; db < C::NDB; db++) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v4[e] = (bf16)(oacc[db][e] * inv);
                    FA_CHECK(!nonfinite_bits(oacc[db][e] * inv), kDbgNonFinite);
                }
                *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * gq) = v4;
            }
            const float lse = l > 0.f ? (m_ref * c + log2f_hw(l)) * kLn2 : -INFINITY;
            FA_CHECK(lse == -INFINITY || !nonfinite_bits(lse), kDbgNonFinite);
            if (gq == 0) LSE[row_id] = lse;
        }
    } else if (row_ok) {
        float* wo = ws_o + (row_id * n_parts + part) * D;
#pragma unroll
        for (int db = 0; db < C::NDB; db++)
            *reinterpret_cast<f32x4*>(wo + 16 * db + 4 * gq) = f32x4{oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]};
        if (gq == 0) {
            float* ml = ws_ml + (row_id * n_parts + part) * 2;
            ml[0] = m_ref == -INFINITY ? -INFINITY : m_ref * c;  // log2 units
            ml[1] = l;
        }
    }
}

// Per query row: merge the key ranges' (O, max, sum).  One wave per row: the
// lanes take the ranges' maxima in parallel (wave max) and then one range's
// weight and weighted sum each; every lane owns D/64 output columns and sums
// the ranges' partial rows, sixteen rows' loads in flight at a time, with
// the weights passed between lanes.
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
    // the ranges' maxima, a lane per range (64 at a time)
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
        for (int p0 = 0; p0 < nvalid; p0 += 64) {
            // lane q: range p0 + q's weight 2^(m - M) (0 for a range with no allowed key) and its sum
            const int pq = p0 + lane;
            const float wq = pq < nvalid ? exp2f_hw(ml[2 * pq] - M) : 0.f;
            lsum += pq < nvalid ? wq * ml[2 * pq + 1] : 0.f;
            const int n = min(64, nvalid - p0);
            for (int u0 = 0; u0 < n; u0 += 16) {
                // sixteen ranges' partial rows in flight at once, weights by lane exchange
                float ov[16][PER];
#pragma unroll
                for (int u = 0; u < 16; u++)
#pragma unroll
                    for (int e = 0; e < PER; e++)
                        ov[u][e] = u0 + u < n ? src[(size_t)(p0 + u0 + u) * D + e] : 0.f;
#pragma unroll
                for (int u = 0; u < 16; u++) {
                    const float wu = __shfl(wq, u0 + u);
#pragma unroll
                    for (int e = 0; e < PER; e++) acc[e] += wu * ov[u][e];
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    }
    FA_CHECK(M == -INFINITY || lsum > 0.f, kDbgRowSum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int e = 0; e < PER; e++) {
        O[(size_t)row * D + lane * PER + e] = (bf16)(acc[e] * inv);
        FA_CHECK(!nonfinite_bits(acc[e] * inv), kDbgNonFinite);
    }
    const float lse = lsum > 0.f ? (M + log2f_hw(lsum)) * kLn2 : -INFINITY;
    FA_CHECK(lse == -INFINITY || !nonfinite_bits(lse), kDbgNonFinite);
    if (lane == 0) LSE[row] = lse;
}

template <int D, bool CAUSAL>
hipError_t launch_decode_d(const DecArgs& a) {
    const int G = a.H / a.Hkv;
    const int nqg = (G * a.Nq + kDecRows - 1) / kDecRows;
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

unsigned debug_flags_decode(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
