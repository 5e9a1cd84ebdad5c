// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (checked on the device):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32], wave64.
//     lane l holds A[l%32][8*(l/32) + i] and B[8*(l/32) + i][l%32], i = 0..7;
//     accumulator register r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   ds_read_tr16_b64 (transposing LDS read): inside each group of 16 lanes,
//     lane s supplies the address of 4 consecutive 16-bit elements; the lane i
//     of the group receives element i%4 of the rows supplied by lanes
//     4*j + i/4, j = 0..3.  With lane s = 4*j + q pointing at row(j), column
//     c0 + 4*q, lane i obtains M[row(j)][c0 + i] for j = 0..3.
//   v_permlane32_swap exchanges the upper half-wave of its first operand with
//     the lower half-wave of its second.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaskBlock = 128;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) (v_log_f32); log2(0) = -inf.
__device__ __forceinline__ float log2f_hw(float x) { return __builtin_amdgcn_logf(x); }

// Computes x at this point of the program: an empty asm that "modifies" x.
// Scheduling fences bind only the machine scheduler; without this, earlier
// passes sink a running sum or max that is read only after a fenced loop down
// to that read, out of the slots it was placed in.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// Value of x in the other half-wave (lane l <-> lane l^32).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats to a packed pair of bf16 (RNE, one v_cvt_pk_bf16_f32); `lo` is
// the element with the lower index.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Pack registers [base, base+8) of an accumulator into MFMA bf16 operands (RNE).
template <int BASE>
__device__ __forceinline__ bf16x8 pack8(const f32x16& s) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (bf16)s[BASE + i];
    return r;
}

// ---------------------------------------------------------------------------
// Swizzled row-major tiles in LDS.
// A tile row holds D bf16 = D/8 chunks of 16 bytes.  Chunk c of row r lives at
// chunk position c ^ sigma(r).  sigma makes both access patterns the kernels
// use conflict-free on the 64-bank LDS:
//   * 16 consecutive rows, same chunk (ds_read_b128 of an MFMA operand);
//   * 4 consecutive rows, 64 contiguous bytes each (ds_read_tr16_b64 of a
//     half-wave).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz_sigma(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// Chunk position of logical 16-byte chunk c in row r of a swizzled tile, and
// its inverse.  64- and 128-wide rows XOR the chunk index with sigma(r).
// 96-wide rows (12 chunks, not a power of two) rotate it by (r >> 2) mod 4
// instead: for 16 consecutive rows and one chunk, rows r = 4a + b sit at
// 16-byte units 12r + pos = 4(3b mod 4) + (c + a) mod 12 (mod 16), which are
// all distinct; for the 4 rows 4h .. 4h+3 of a transposing read (one shared
// rotation) and 4 consecutive chunks, the 4 positions have distinct residues
// mod 4 and the rows distinct multiples of 4, again 16 distinct units.
template <int D>
__device__ __forceinline__ int chunk_pos(int r, int c) {
    if constexpr (D == 96) {
        const int p = c + ((r >> 2) & 3);
        return p >= 12 ? p - 12 : p;
    } else {
        return c ^ swz_sigma<D>(r & 15);
    }
}
template <int D>
__device__ __forceinline__ int chunk_at(int r, int p) {
    if constexpr (D == 96) {
        const int c = p - ((r >> 2) & 3);
        return c < 0 ? c + 12 : c;
    } else {
        return p ^ swz_sigma<D>(r & 15);
    }
}
// Element offset of logical (row, col) in a D-wide swizzled tile.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
    return row * D + ((((col >> 3) ^ swz_sigma<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* base, int off) {
    return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* base, int off) {
    typedef short __attribute__((address_space(3))) * lds_i16x4_ptr;
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4 __attribute__((address_space(3)))*)((__attribute__((address_space(3))) bf16*)(base + off)));
    return __builtin_bit_cast(bf16x4, v);
}

// MFMA A-operand (rows m = 32 columns of the tile starting at col0, k = 16 tile
// rows starting at row0, in the key/query order produced by the accumulator
// layout) read from a row-major swizzled tile with two transposing reads.
// Lane l obtains tile[row0 + 8*(i/4) + 4*(l/32) + i%4][col0 + l%32], i = 0..7,
// which is exactly the order in which registers 0..7 (or 8..15) of a 32x32
// accumulator hold their 16 rows.
template <int D>
__device__ __forceinline__ bf16x8 lds_read_tr_operand(const bf16* tile, int row0, int col0, int lane) {
    const int s = lane & 15, j = s >> 2, q = s & 3;
    const int g = (lane >> 4) & 1, h = lane >> 5;
    const int col = col0 + 16 * g + 4 * q;
    const bf16x4 lo = lds_read_tr4(tile, swz<D>(row0 + 4 * h + j, col));
    const bf16x4 hi = lds_read_tr4(tile, swz<D>(row0 + 8 + 4 * h + j, col));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// ---------------------------------------------------------------------------
// Buffer resources (gfx9 descriptor): loads past num_records bytes return 0
// and stores past it are dropped, which handles ragged tails without branches.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// 16 bytes per lane from global straight into LDS: lane i writes lds_base + 16*i
// (lds_base must be the same for the whole wave).
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, void* lds_base, uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, byte_off, 0,
                                             0, 0);
}

// ---------------------------------------------------------------------------
// Padded row-major tiles in LDS (row stride = D + pad elements).  A stride of
// 16*odd bytes mod 256 makes 16 consecutive rows of a 16-byte column hit 16
// distinct bank groups (operand reads with ds_read_b128); a stride of 64 mod
// 256 bytes makes 4 consecutive rows of 64 bytes disjoint (transposing reads
// by half a wave).  Every operand address is then a base plus an immediate.
// ---------------------------------------------------------------------------
template <int D>
struct PadK {  // tiles read with ds_read_b128 (16 rows x 16 B)
    static constexpr int STRIDE = D + 8;  // 272 B (d=128) or 144 B (d=64)
};
template <int D>
struct PadV {  // tiles read with ds_read_tr16_b64 (4 rows x 64 B per half-wave)
    // 320 B (d=128), 192 B (d=64), 576 B (d=256): 64 or 192 mod 256; 96-wide
    // rows are 192 B already
    static constexpr int STRIDE = D == 96 ? D : D + 32;
};

// Transposing A-operand read from a padded row-major tile (see
// lds_read_tr_operand): lane l obtains
// tile[row0 + 8*(i/4) + 4*(l/32) + i%4][col0 + l%32], i = 0..7.
// `lane_base` = tile + lane_tr_offset<STRIDE>(lane), computed once.
template <int STRIDE>
__device__ __forceinline__ int lane_tr_offset(int lane) {
    const int s = lane & 15, j = s >> 2, q = s & 3, g = (lane >> 4) & 1, h = lane >> 5;
    return (4 * h + j) * STRIDE + 16 * g + 4 * q;
}
template <int STRIDE>
__device__ __forceinline__ bf16x8 lds_tr_operand_pad(const bf16* lane_base, int row0, int col0) {
    const bf16x4 lo = lds_read_tr4(lane_base, row0 * STRIDE + col0);
    const bf16x4 hi = lds_read_tr4(lane_base, (row0 + 8) * STRIDE + col0);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgVmem = 0x020;

// The same HBM -> LDS copy issued as an opaque instruction: the compiler does
// not track it, so it inserts no wait for it before unrelated LDS reads.  The
// caller must wait (s_waitcnt vmcnt(0)) and synchronize the workgroup before
// reading what it wrote.  `srd` is a gfx9 buffer descriptor, `lds_addr` the
// wave-uniform LDS byte address of lane 0's 16 bytes.
typedef int int32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32x4_t make_srd(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return int32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, kRsrcFlags};
}

__device__ __forceinline__ void dma16_untracked(int32x4_t srd, uint32_t lds_addr, uint32_t byte_off) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_addr), "v"(byte_off), "s"(srd)
        : "memory", "m0");
}

// Four bytes per lane: lane i writes lds_addr + 4*i (one 256-byte row of a
// 64-entry fp32 vector per instruction).
__device__ __forceinline__ void dma4_untracked(int32x4_t srd, uint32_t lds_addr, uint32_t byte_off) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(lds_addr), "v"(byte_off), "s"(srd)
        : "memory", "m0");
}

// s_waitcnt vmcnt(0) through the builtin, so the compiler's wait tracking sees
// it.  An inline-asm wait is invisible to that tracking: loads issued before it
// (fragments kept in registers) would still count as outstanding, and the
// compiler would add waits of its own at their first use -- inside a loop, where
// the hardware counter also holds the next tile's untracked copies, such a wait
// stalls until those copies land.  Encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename T>
__device__ __forceinline__ uint32_t lds_addr_of(const T* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}

// ---------------------------------------------------------------------------
// Debug self-check, compiled in with -DFA_DEBUG_CHECK (libfa_debug.so): the
// kernels record violated invariants as bits of a device flag word, one per
// translation unit (device globals are not shared between code objects); the
// C ABI's fa_debug_flags() collects them.  Without the macro the checks
// compile to nothing.
// ---------------------------------------------------------------------------
constexpr unsigned kDbgRowSum = 1u;     // a row saw a finite score but its sum of weights is not > 0
constexpr unsigned kDbgNonFinite = 2u;  // an output element (O, lse, dQ, dK, dV) is NaN or infinite
// NaN or infinity, from the exponent bits (the forwards are compiled without
// NaN semantics, under which isnan / isfinite may fold to constants)
__device__ __forceinline__ bool nonfinite_bits(float x) { return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u; }
#ifdef FA_DEBUG_CHECK
namespace {
__device__ unsigned int g_debug_flags;
// Flags of this translation unit's kernels (synchronous; `clear` resets them).
inline unsigned read_debug_flags(bool clear) {
    unsigned v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return ~0u;
    if (clear) {
        const unsigned z = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &z, sizeof z, 0, hipMemcpyHostToDevice) != hipSuccess)
            return ~0u;
    }
    return v;
}
}  // namespace
// per lane: the atomic is a vector instruction on the flag's global address
#define FA_CHECK(cond, bit)                                 \
    do {                                                    \
        if (!(cond)) atomicOr(&g_debug_flags, (unsigned)(bit)); \
    } while (0)
#else
#define FA_CHECK(cond, bit) \
    do {                    \
    } while (0)
inline unsigned read_debug_flags(bool) { return 0u; }
#endif

// Store one wave's 32 x D block of a row-major bf16 tensor held in 32x32 MFMA
// accumulator layout -- acc[dm][4g + e] is element (row l32, column
// 32dm + 8g + 4h + e) -- scaled by `mul`.  Written straight from that layout
// every lane stores 8 bytes into a different row, 64 partial cache lines per
// instruction; instead the block goes through a wave-private LDS staging area
// (32 rows of D + 8 elements: 16-byte aligned rows, at most two-way bank
// conflicts on the 8-byte writes) and leaves with 16-byte stores, each
// instruction covering up to 1 KB of consecutive rows.  The tensor's rows
// hold `ld` <= D elements (a multiple of 8); columns from `ld` on are not
// stored.  `row0_off` is the byte offset of the block's first row in the
// buffer; rows past the buffer's end are dropped by its range check.  The
// caller must make sure no other wave uses `stage` meanwhile.
template <int D>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[D / 32], float mul, bf16* stage, rsrc_t r,
                                                  uint32_t row0_off, int ld, int lane) {
    constexpr int SS = D + 8;
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int dm = 0; dm < D / 32; dm++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                v4[e] = (bf16)(acc[dm][4 * g + e] * mul);
                FA_CHECK(!nonfinite_bits(acc[dm][4 * g + e] * mul), kDbgNonFinite);
            }
            *reinterpret_cast<bf16x4*>(stage + l32 * SS + 32 * dm + 8 * g + 4 * h) = v4;
        }
    // chunk 64 i + lane of the block, row-major: 16-byte chunk `ch` of row
    // `row` (when CPR divides 64 every lane stores; otherwise the last
    // instruction's spare lanes do nothing)
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int NCH = (32 * CPR + 63) / 64;   // store instructions
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int g = 64 * i + lane, row = g / CPR, ch = g % CPR;
        if (row < 32) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * SS + 8 * ch);
            if (8 * ch < ld)
                __builtin_amdgcn_raw_buffer_store_b128(v, r, row0_off + (uint32_t)(row * ld + 8 * ch) * 2, 0, 0);
        }
    }
}

// Local window and ALiBi of one head ("FlashAttention 深度解析" section 五
// names both as built-in variants beside the causal mask): key j is allowed
// for query i iff i - wl <= j <= i + wr (a negative bound is unbounded), and
// the score of (i, j) gets -slope |i - j|; `slope2` is slope * log2(e).
struct Variant {
    int wl, wr;
    float slope2;
    __device__ __forceinline__ bool dead(int i, int j) const {
        return (wl >= 0 && j < i - wl) || (wr >= 0 && j > i + wr);
    }
    // bias in log2 units
    __device__ __forceinline__ float bias2(int i, int j) const {
        return -slope2 * (float)(i > j ? i - j : j - i);
    }
    // keys [lo, hi) a block of queries [q_lo, q_hi) can see, within [0, n)
    __device__ __forceinline__ void key_range(int q_lo, int q_hi, int n, int& lo, int& hi) const {
        lo = wl >= 0 ? max(0, q_lo - wl) : 0;
        hi = wr >= 0 ? min(n, q_hi - 1 + wr + 1) : n;
    }
    // queries [lo, hi) a block of keys [k_lo, k_hi) is seen by, within [0, n)
    __device__ __forceinline__ void query_range(int k_lo, int k_hi, int n, int& lo, int& hi) const {
        lo = wr >= 0 ? max(0, k_lo - wr) : 0;
        hi = wl >= 0 ? min(n, k_hi - 1 + wl + 1) : n;
    }
};

// Workgroup id -> logical work item such that consecutive logical items land
// on the same XCD (the hardware deals workgroups round-robin over the 8 XCDs),
// so tiles of one (batch, head) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
    constexpr int kXcd = 8;
    const int x = wg % kXcd, per = n / kXcd, rem = n % kXcd;
    return x * per + (x < rem ? x : rem) + wg / kXcd;
}

// Compact, in LDS, the indices idx in [lo, hi] whose mask byte base[idx*stride]
// is nonzero (increasing order).  All threads of the workgroup must call it.
// Returns the count.  `list` needs room for hi - lo + 1 entries.
template <int WAVES>
__device__ int build_block_list(const uint8_t* __restrict__ base, size_t stride, int lo, int hi,
                                uint16_t* list, int* wave_cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int total = 0;
    for (int start = lo; start <= hi; start += 64 * WAVES) {
        const int idx = start + tid;
        const bool keep = idx <= hi && base[(size_t)idx * stride] != 0;
        const uint64_t bal = __ballot(keep);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = total, sum = 0;
        for (int w = 0; w < WAVES; w++) {
            if (w < wave) off += wave_cnt[w];
            sum += wave_cnt[w];
        }
        if (keep) list[off + __popcll(bal & ((1ull << lane) - 1))] = (uint16_t)idx;
        total += sum;
        __syncthreads();
    }
    return total;
}

}  // namespace fa
