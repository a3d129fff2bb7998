// Device-side building blocks of the gfx950 attention kernels: element
// types, matrix-core fragments, wavefront exchanges and the dropout
// generator.  Everything here is written for CDNA4 (64-lane wavefronts,
// 32x32 MFMA tiles).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- fragments
//
// A fragment is one lane's share of a 32x16 operand of a 32x32 MFMA tile:
// eight elements along the contraction dimension.  For 16-bit types it is
// one register quadruple feeding a single v_mfma_f32_32x32x16 instruction;
// for fp32 it is eight registers feeding eight v_mfma_f32_32x32x2f32.  The
// A and B operands of one product always fill their eight slots with the
// same contraction indices, so the hardware's own slot order cancels out.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct Frag<f16> { typedef f16x8 type; typedef f16x4 half; };
template <> struct Frag<float> { typedef f32x8 type; typedef f32x4 half; };

template <typename T> using frag_t = typename Frag<T>::type;
template <typename T> using half_t = typename Frag<T>::half;

// acc += A(32x16) * B(16x32) on the matrix cores.
__device__ __forceinline__ void mma(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16 &acc, const f16x8 &a, const f16x8 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16 &acc, const f32x8 &a, const f32x8 &b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
}

// Round-to-nearest-even conversions from fp32.
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Join two half-fragments (four contraction indices each) into a fragment.
template <typename T>
__device__ __forceinline__ frag_t<T> join(const half_t<T> &lo, const half_t<T> &hi) {
    frag_t<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[i + 4] = hi[i]; }
    return f;
}

// Eight fp32 values rounded into a fragment.
template <typename T>
__device__ __forceinline__ frag_t<T> pack8(const float *x) {
    frag_t<T> f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = from_f32<T>(x[i]);
    return f;
}

// Eight consecutive accumulator registers (from `off`) rounded into a fragment.
template <typename T>
__device__ __forceinline__ frag_t<T> pack8(const f32x16 &x, int off) {
    frag_t<T> f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = from_f32<T>(x[off + i]);
    return f;
}

// ------------------------------------------------------------ lane exchange
//
// Exchanges of one value between the two halves of a wavefront (lane ^ 32)
// go through ds_bpermute: v_permlane32_swap fed the same value as both
// operands has its two results treated as equal by this compiler, which then
// drops the partner's value.  Where two different values are traded (the
// keep-mask words, keep_masks_from_blocks) the swap is used.

__device__ __forceinline__ uint32_t lane_in_wave() { return threadIdx.x & (kWave - 1); }

// Value held by lane ^ 32.
__device__ __forceinline__ uint32_t other_half(uint32_t x) {
    return (uint32_t)__shfl_xor((int)x, 32);
}

// max(x, x of lane ^ 32), identical in both lanes.
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// x + (x of lane ^ 32), bitwise identical in both lanes.
__device__ __forceinline__ float sum_halves(float x) {
    const float y = __shfl_xor(x, 32);
    return (lane_in_wave() & 32) ? y + x : x + y;
}

// ------------------------------------------------------------------ dropout
//
// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11): a keyed
// bijection on four 32-bit words built from two 32x32->64-bit products per
// round, with the key advanced by two Weyl increments between rounds.
struct Philox4 { uint32_t x[4]; };

constexpr uint32_t kPhiloxWeylA = 0x9E3779B9u, kPhiloxWeylB = 0xBB67AE85u;

// Round r (0-based) of the generator on counter c under key (k0, k1): the
// round key is the key advanced r times by the Weyl increments.  With
// FLIP, the last round (r = 9) also flips the top bit of both 16-bit halves
// of output words 0 and 2, through its round key (a uniform value, so the
// flip costs no vector instruction); keep_masks_from_blocks and
// keep_mask2_flipped expect words drawn this way.  The forward and the dQ
// kernel draw with the flip (1.2 % and 0.6 % faster); in the dK/dV kernel
// only the B wavefronts do (with A's draws flipped too, its register
// allocation came out 3 % slower at d = 128; B alone: 1-2 % faster).
template <bool FLIP = false>
__device__ __forceinline__ void philox_round(Philox4 &c, int r, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    const uint32_t flip = (FLIP && r == 9) ? 0x80008000u : 0u;
    // One 32x32->64-bit product per word pair (v_mad_u64_u32 gives both
    // halves in a single instruction).
    const uint64_t pA = (uint64_t)kMulA * c.x[0], pB = (uint64_t)kMulB * c.x[2];
    const uint32_t hiA = (uint32_t)(pA >> 32), loA = (uint32_t)pA;
    const uint32_t hiB = (uint32_t)(pB >> 32), loB = (uint32_t)pB;
    // Three-input XORs as single v_bitop3_b32 instructions (truth table 0x96).
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hiB, c.x[1], (k0 + (uint32_t)r * kPhiloxWeylA) ^ flip, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hiA, c.x[3], (k1 + (uint32_t)r * kPhiloxWeylB) ^ flip, 0x96);
    c.x[0] = n0; c.x[1] = loB; c.x[2] = n2; c.x[3] = loA;
}

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
    Philox4 c;
    c.x[0] = c0; c.x[1] = c1; c.x[2] = c2; c.x[3] = c3;
#pragma unroll
    for (int r = 0; r < 10; ++r) philox_round(c, r, k0, k1);
    return c;
}

// Keep bits of the eight columns 8*grp .. 8*grp+7 of one row: bit e is set
// when column 8*grp+e survives (its 16-bit lane >= threshold).
__device__ __forceinline__ uint32_t keep_byte(uint32_t grp, uint32_t row, uint32_t h, uint32_t b,
                                              uint32_t seed_lo, uint32_t seed_hi,
                                              uint32_t threshold) {
    const Philox4 r = philox4x32_10(grp, row, h, b, seed_lo, seed_hi);
    uint32_t bits = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        bits |= (uint32_t)((r.x[w] & 0xFFFFu) >= threshold) << (2 * w);
        bits |= (uint32_t)((r.x[w] >> 16) >= threshold) << (2 * w + 1);
    }
    return bits;
}

// Keep masks of the two 16-bit lanes of a generator word: 0xFFFF in each half
// whose lane value is at least the threshold T, 0 elsewhere, for both halves
// at once.  Flipping the top bits maps the unsigned order of the lanes onto
// the signed one; then lane >= T exactly when the saturating 16-bit difference
// (T' - 1) - lane' is negative (T', lane': flipped), and an arithmetic shift
// spreads its sign over the half.  kc2 = keep_cmp_const(T), 1 <= T <= 65535.
// keep_mask2_flipped takes a word whose halves are already flipped.
typedef short i16x2 __attribute__((ext_vector_type(2)));
__host__ __device__ constexpr uint32_t keep_cmp_const(uint32_t T) {
    return (((T ^ 0x8000u) - 1u) & 0xFFFFu) * 0x00010001u;
}
__device__ __forceinline__ uint32_t keep_mask2_flipped(uint32_t wf, uint32_t kc2) {
    const i16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(i16x2, kc2), __builtin_bit_cast(i16x2, wf));
    return __builtin_bit_cast(uint32_t, d >> (i16x2){15, 15});
}
__device__ __forceinline__ uint32_t keep_mask2(uint32_t w, uint32_t kc2) {
    return keep_mask2_flipped(w ^ 0x80008000u, kc2);
}

// Keep masks (keep_mask2 layout) of the eight probability pairs one lane
// holds in a 32x32 accumulator with one query row per lane, from blocks
// drawn with philox_round<true> (words 0 and 2 flipped): pair i is
// registers 2i, 2i+1, keys 8(i/2) + 4g + 2(i%2) + {0, 1} of the 32-key block
// (g = lane / 32).  Lane (row, g) draws 8-key blocks 2g (b0) and 2g+1 (b1)
// of the row; pair i takes word 2g + i%2 of block i/2.  So the lower half
// of the wavefront needs words 0, 1 and the upper half words 2, 3 of every
// block, and one v_permlane32_swap per (block, word) pair -- the upper half
// of the first operand traded for the lower half of the second -- hands
// each half the words the other half drew.
__device__ __forceinline__ void keep_masks_from_blocks(const Philox4 &b0, const Philox4 &b1, uint32_t kc2,
                                                       uint32_t (&m)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const Philox4 &b = h ? b1 : b0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            // e = 0 trades words 0 and 2 (drawn flipped), e = 1 words 1 and 3
            const auto r = __builtin_amdgcn_permlane32_swap(b.x[e], b.x[2 + e], false, false);
            m[2 * h + e] = e ? keep_mask2(r[0], kc2) : keep_mask2_flipped(r[0], kc2);         // block h: pairs 2h + e
            m[4 + 2 * h + e] = e ? keep_mask2(r[1], kc2) : keep_mask2_flipped(r[1], kc2);     // block 2 + h: pairs 4 + 2h + e
        }
    }
}

// Keep bits of the sixteen keys one lane holds in a 32x32 accumulator that
// has one query row per lane (register r <-> key kbase + 8(r/4) + 4g +
// r%4, g = lane / 32): bit r of the result.  Each half-wavefront draws two
// of the row's four 8-key Philox blocks (keys kbase + 16g .. + 15) and the
// halves exchange the nibbles the other one needs.
__device__ __forceinline__ uint32_t keep_bits_row(uint32_t kbase, uint32_t row, uint32_t h,
                                                  uint32_t b, uint32_t seed_lo, uint32_t seed_hi,
                                                  uint32_t threshold) {
    const uint32_t g = lane_in_wave() >> 5;
    const uint32_t grp = (kbase >> 3) + 2 * g;
    const uint32_t bits = keep_byte(grp, row, h, b, seed_lo, seed_hi, threshold) |
                          (keep_byte(grp + 1, row, h, b, seed_lo, seed_hi, threshold) << 8);
    const uint32_t mine = g ? 4 : 0, theirs = g ? 0 : 4;
    const uint32_t own = ((bits >> mine) & 0xFu) | (((bits >> (8 + mine)) & 0xFu) << 4);
    const uint32_t send = ((bits >> theirs) & 0xFu) | (((bits >> (8 + theirs)) & 0xFu) << 4);
    const uint32_t recv = other_half(send);
    return g ? (recv | (own << 8)) : (own | (recv << 8));
}

// ------------------------------------------------------------ memory moves
//
// Eight (a fragment) or four (a half-fragment) consecutive elements moved
// with 16-byte (or 8-byte) vector accesses.  Addresses are multiples of the
// access size.
template <typename T>
__device__ __forceinline__ frag_t<T> load_frag(const T *p) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(frag_t<T>, *reinterpret_cast<const uint4 *>(p));
    } else {
        struct Two { uint4 a, b; } t;
        t.a = reinterpret_cast<const uint4 *>(p)[0];
        t.b = reinterpret_cast<const uint4 *>(p)[1];
        return __builtin_bit_cast(frag_t<T>, t);
    }
}

template <typename T>
__device__ __forceinline__ void store_half(T *p, const half_t<T> &x) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, x);
    } else {
        *reinterpret_cast<uint4 *>(p) = __builtin_bit_cast(uint4, x);
    }
}

// Four fp32 values rounded to T and stored as one vector.
template <typename T>
__device__ __forceinline__ void store4(T *p, float a, float b, float c, float d) {
    half_t<T> x;
    x[0] = from_f32<T>(a); x[1] = from_f32<T>(b); x[2] = from_f32<T>(c); x[3] = from_f32<T>(d);
    store_half<T>(p, x);
}

// ---------------------------------------------------------- transposed reads
//
// Half-fragment of a transposed fp32 operand read from a row-major LDS tile
// (the generic fp32 kernels): lane l (i = l % 32, g = l / 32) receives
// tile[rbase + 4g + k][c0 + i] for k = 0..3.  Two such reads (rbase and
// rbase + 8) give the eight slots of a fragment whose contraction index runs
// along the tile's rows in the order rbase + 4g + {0..3}, rbase + 8 + 4g +
// {0..3} -- the order in which a 32x32 accumulator holds the same rows
// (register r -> row 8(r/4) + 4g + r%4), so a rounded accumulator is the
// matching other operand.  (The 16-bit kernels read their swizzled tiles
// with ds_read_b64_tr_b16 through lds_half_tr.)
template <typename T>
__device__ __forceinline__ half_t<T> load_half_tr(const T *tile, int ld, int rbase, int c0) {
    static_assert(sizeof(T) == 4, "element-wise transposed reads serve fp32 tiles");
    const int lane = (int)lane_in_wave();
    const int i = lane & 31, g = lane >> 5;
    half_t<T> h;
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = tile[(rbase + 4 * g + k) * ld + c0 + i];
    return h;
}

template <typename T>
__device__ __forceinline__ frag_t<T> load_frag_tr(const T *tile, int ld, int rbase, int c0) {
    return join<T>(load_half_tr<T>(tile, ld, rbase, c0), load_half_tr<T>(tile, ld, rbase + 8, c0));
}

// ------------------------------------------------------------- tile copies
//
// Cooperative copy of ROWS consecutive rows (from row r0) of a row-major
// [N, D] matrix into a row-major LDS tile of pitch LD, staged through
// registers so that the global loads of the next tile can be in flight
// while the current one is consumed.  Rows at or past N read as zero.
template <typename T, int ROWS, int D, int THREADS>
struct TileCopy {
    static constexpr int CH = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int CPR = D / CH;                 // chunks per row
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PER = (CHUNKS + THREADS - 1) / THREADS;
    uint4 r[PER];

    __device__ __forceinline__ void load(const T *g, int64_t r0, int64_t N, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * THREADS;
            const int row = c / CPR, col = (c % CPR) * CH;
            r[i] = uint4{0, 0, 0, 0};
            if ((CHUNKS % THREADS == 0 || c < CHUNKS) && r0 + row < N)
                r[i] = *reinterpret_cast<const uint4 *>(g + (r0 + row) * D + col);
        }
    }

    template <int LD>
    __device__ __forceinline__ void store(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * THREADS;
            if (CHUNKS % THREADS == 0 || c < CHUNKS) {
                const int row = c / CPR, col = (c % CPR) * CH;
                *reinterpret_cast<uint4 *>(lds + row * LD + col) = r[i];
            }
        }
    }
};

// ------------------------------------------------------ swizzled LDS tiles
//
// A tile of 16-bit elements with D columns is stored with a row pitch of
// exactly 2D bytes; the 16-byte chunks of row r are permuted, logical chunk
// x sitting at position x ^ f(r).  On gfx950 the LDS serves a 16-byte read
// for 16 lanes (or an 8-byte read for 32 lanes) per cycle across 64 banks of
// 4 bytes.  f is chosen so that both access patterns of the attention
// kernels are free of bank conflicts: 16 lanes reading the same logical
// chunk of 16 consecutive rows (matrix-core operands taken along a row), and
// 32 lanes reading 64 contiguous bytes of 4 consecutive rows (transposed
// reads).  An unpadded pitch also lets whole rows be filled by direct
// global-to-LDS loads, which write 16 bytes per lane contiguously.  At
// d = 96 (12 chunks, a 192-byte pitch whose bank offset repeats every four
// rows) and d = 32 (4 chunks, 64-byte pitch) f is the row's bits 2-3, which keeps every permutation inside an
// aligned group of four chunks and gives the four rows of each bank class
// distinct groups; the transposed reads then need no permutation at all.
#define FA_LDS __attribute__((address_space(3)))

template <int D>
struct Swz {
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int ROW_BYTES = D * 2;
    __device__ static constexpr uint32_t f(uint32_t r) {
        return D == 128  ? (((r & 3u) << 2) | ((r >> 2) & 3u))
               : (D == 96 || D == 32) ? ((r >> 2) & 3u)
                         : ((((r >> 1) & 1u) << 2) | ((r >> 2) & 3u));
    }
    // Byte offset of element column `col` (a multiple of 4) of row r.
    __device__ static constexpr uint32_t off(uint32_t r, uint32_t col) {
        return r * ROW_BYTES + ((((col >> 3) ^ f(r))) << 4) + (col & 7u) * 2;
    }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef FA_LDS char lds_char;

// 16-byte LDS read (the compiler folds constant parts of the address into
// the instruction's offset field).  LDS tiles are addressed through
// pointers derived from distinct __shared__ arrays, so that the compiler
// can tell a direct global-to-LDS load into one buffer from a read of
// another and need not wait for the load before the read.
template <typename T>
__device__ __forceinline__ frag_t<T> lds_frag(const lds_char *p) {
    return __builtin_bit_cast(frag_t<T>, *(const FA_LDS u32x4 *)p);
}

// Transposed half-fragment read (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane i receives element i%4 of the 8-byte rows addressed by lanes
// 4k + i/4 (k = 0..3).
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ half_t<T> lds_half_tr(const lds_char *p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4 *)p);
    return __builtin_bit_cast(half_t<T>, r);
}

// Buffer resource over `bytes` bytes from `p` (raw, unswizzled).  Loads
// through it whose 16 bytes lie past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane at byte offset voff + soff of the buffer straight into
// LDS at base + 16 l; lanes past the buffer end write zeros.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          lds_char *base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void *)base, 16, voff, soff, 0, 0);
}

// Register-class hint: the value is placed in accumulation registers (AGPRs)
// at this point.  The statement emits no instruction; matrix-core
// instructions read their operands and accumulators from AGPRs directly,
// which keeps long-lived operands (the query block, the output
// accumulators) out of the VGPRs that the softmax arithmetic needs.
template <typename V>
__device__ __forceinline__ void pin_agpr(V &x) { asm volatile("" : "+a"(x)); }
// Same for the vector registers (values the VALU works on).
template <typename V>
__device__ __forceinline__ void pin_vgpr(V &x) { asm volatile("" : "+v"(x)); }

// ------------------------------------------------------ packed 16-bit pairs

// Two fp32 values rounded (RNE) into a packed pair of 16-bit values.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef T t2 __attribute__((ext_vector_type(2)));
    t2 v;
    v[0] = from_f32<T>(lo);
    v[1] = from_f32<T>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed pair of 16-bit values, in fp32 (the halves are
// widened exactly).  Plain VALU adds: the dot-product instructions that
// could do this in one step do not co-issue with the matrix products of the
// same wavefront (measured: each costs about ten cycles of the product
// pipeline), the widening and the adds do.
template <typename T>
__device__ __forceinline__ float sum2(uint32_t pair, float acc);
// (The widened halves pass through an empty register constraint so that the
// compiler does not fold the adds back into a dot-product instruction.)
template <>
__device__ __forceinline__ float sum2<bf16>(uint32_t pair, float acc) {
    float lo = __builtin_bit_cast(float, pair << 16);
    float hi = __builtin_bit_cast(float, pair & 0xFFFF0000u);
    asm("" : "+v"(lo), "+v"(hi));
    return (acc + lo) + hi;
}
template <>
__device__ __forceinline__ float sum2<f16>(uint32_t pair, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_bit_cast(h2, pair);
    float lo = (float)h[0], hi = (float)h[1];
    asm("" : "+v"(lo), "+v"(hi));
    return (acc + lo) + hi;
}

// The same sum as one dot-product instruction (v_dot2c_f32_bf16 / _f16):
// no extra registers, but no co-issue with matrix products.
template <typename T>
__device__ __forceinline__ float sum2_dot(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float sum2_dot<bf16>(uint32_t pair, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, pair), one, acc, false);
}
template <>
__device__ __forceinline__ float sum2_dot<f16>(uint32_t pair, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pair), one, acc, false);
}

// --------------------------------------------------------------- utilities

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
