// Forward of fused exact attention with FP8 (e4m3) inputs on gfx950.
//
// The pages name FP8 precision as part of the FlashAttention-3 speed-up
// ("FlashAttention-3 (2024)", chipfoundryservices.com page); the method is
// the one of the 16-bit forward: Q, K, V tiled into on-chip blocks, the
// online-softmax recurrence over key tiles, only O and the per-row
// log-sum-exp written back ("Tiling" and "Recomputation",
// mrodiduger.github.io page).
//
// Inputs are OCP e4m3 bytes with one fp32 descale factor per (b, h) for
// each of Q, K and V: the real inputs are q8 * dq, k8 * dk, v8 * dv.  Both
// products run on the FP8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4
// with unit block scales, fp32 accumulation):
//   S^T = K Q^T            (exact products of e4m3 values; dq dk and the
//                           softmax scale fold into the exponent scale),
//   O^T += V^T P8^T        (P8: the probabilities times 2^6 rounded to e4m3,
//                           round to nearest even; dv and 2^-6 fold into
//                           the final normalisation).
// The row sums and the log-sum-exp use the unrounded fp32 probabilities, so
// O differs from the exact result only by the rounding of P8:
// |O - O_exact| <= (2^-4 + n 2^-16) max_j |v_j| per element (n visible keys;
// the second term covers probabilities small enough to be e4m3 subnormals).
// The reference maximum of a row moves when a tile exceeds it by more than
// 2^2, so every probability is at most 4 and P * 2^6 <= 256 stays below the
// e4m3 maximum (448).
//
// Layout: as in the 16-bit forward -- 32 query rows per wavefront, four
// wavefronts (128 rows) per workgroup and two workgroups per CU, so the two
// wavefronts of a SIMD come from different workgroups; 64-key tiles in LDS
// by direct buffer loads, two K and two V buffers, loaded one step ahead.
// A tile row is 128 bytes (d = 128), stored with the XOR swizzle of 128-byte
// rows.  K operands (32 bytes of a key row per lane) are two 16-byte reads;
// V^T operands are four ds_read_b64_tr_b8 reads, addressed so that byte p of
// a lane holds the key that byte p of the rounded P^T operand holds.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct FwdFp8Tile {
    static constexpr int D = 128;
    static constexpr int NW = 4;
    static constexpr int WG_PER_CU = 2;
    static constexpr int BQ = 32 * NW;            // query rows per workgroup
    static constexpr int BC = 64;                 // keys per tile (two 32-key blocks)
    static constexpr int NBUF = 2;                // K and V buffers each
    static constexpr int RB = D;                  // bytes per tile row
    static constexpr int TILE_BYTES = BC * RB;    // 8 KB
    static constexpr int CHUNK_BYTES = kWave * 16;
    static constexpr int CHUNKS = TILE_BYTES / CHUNK_BYTES;   // 8 load instructions per tile
    static constexpr int RPC = CHUNK_BYTES / RB;              // 8 rows per load instruction
    static constexpr int LPT = CHUNKS / NW;                   // per wavefront per tile
    static constexpr int LOADS = 2 * LPT;                     // per wavefront per step (K and V)
    static constexpr int THREADS = NW * kWave;
};

constexpr int kF8Threads = FwdFp8Tile::THREADS;
constexpr int kF8WgPerCu = FwdFp8Tile::WG_PER_CU;

// Rescale threshold (log2 units) and the power of two the probabilities are
// scaled by before rounding to e4m3 (4 * 2^6 = 256 < 448).
constexpr float kF8RescaleLog2 = 2.0f;
constexpr float kF8PScaleLog2 = 6.0f;

// 128-byte rows: logical 16-byte chunk x of row r at position x ^ f(r) (the
// 16-bit kernels' swizzle for 128-byte rows).  It keeps both reads of this
// kernel free of bank conflicts: 16 lanes reading one chunk of 16
// consecutive rows, and the transposed reads (rows {0..3, 8..11} + 16 t +
// 4 g, 32 bytes of each).
__device__ constexpr uint32_t f8_swz(uint32_t r) { return Swz<64>::f(r); }
__device__ constexpr uint32_t f8_off(uint32_t r, uint32_t byte) {
    return r * 128u + ((((byte >> 4) ^ f8_swz(r))) << 4) + (byte & 15u);
}

__device__ __forceinline__ void mma8(f32x16 &acc, const i32x8 &a, const i32x8 &b) {
    // e4m3 (format 0) for both operands, unit block scales (e8m0 127 = 2^0)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

template <bool CAUSAL>
__global__ void __launch_bounds__(kF8Threads, kF8WgPerCu) fwd_fp8_kernel(const FwdArgs a) {
    using TL = FwdFp8Tile;
    constexpr int D = TL::D, BQ = TL::BQ, BC = TL::BC, NW = TL::NW, NBUF = TL::NBUF;
    constexpr int TB = TL::TILE_BYTES, CB = TL::CHUNK_BYTES, RPC = TL::RPC, LPT = TL::LPT;
    constexpr float kNegInf = -__builtin_huge_valf();

    __shared__ __attribute__((aligned(1024))) char ks0[TB], ks1[TB], vs0[TB], vs1[TB];
    static_assert(NBUF == 2, "two K and two V buffers");

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lq = lane & 31, g = lane >> 5;

    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)nqb, a.group);
    const int64_t bh = un.bh;
    const int64_t qb = CAUSAL ? (nqb - 1 - un.rank) : un.rank;
    const int N = (int)a.N, Nk = (int)a.Nk;
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const uint8_t *__restrict__ Q = reinterpret_cast<const uint8_t *>(a.q) + head;
    const uint8_t *__restrict__ K = reinterpret_cast<const uint8_t *>(a.k) + head_kv;
    const uint8_t *__restrict__ V = reinterpret_cast<const uint8_t *>(a.v) + head_kv;

    const int q0 = (int)qb * BQ;
    const int q0w = q0 + 32 * wave;
    const int qrow = q0w + lq;
    // causal: query i sees keys j <= i + off (all index arithmetic fits in 32 bits: N, Nk < 2^31)
    const int off = Nk - N;

    // exponent scale of the scores (log2 units), and the output factor
    const float sl2 = a.scale_log2 * a.descale_q[bh] * a.descale_k[bh];
    const float vsc = a.descale_v[bh];

    // Q^T operands: 32 bytes of this lane's query row per 64-wide chunk c of
    // d (bytes 64 c + 32 g ..), rows clamped into range.
    i32x8 qf[2];
    {
        const int r = qrow < N ? qrow : N - 1;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint4 *p = reinterpret_cast<const uint4 *>(Q + (size_t)r * D + 64 * c + 32 * g);
            const uint4 x0 = p[0], x1 = p[1];
            qf[c] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
    }

    // LDS offsets.  K operand of chunk c: the two 16-byte halves of bytes
    // 64 c + 32 g .. + 31 of key row lq (key block kb adds 32 rows = 4 KB).
    uint32_t koff[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) koff[c][h] = f8_off((uint32_t)lq, (uint32_t)(64 * c + 32 * g + 16 * h));
    // V^T operand of d block db: transposed read t (t = 0..3, 2 KB apart)
    // gives bytes 8 t + j, j = 0..7, of the lane, byte j coming from the
    // 8-byte row addressed by lane 2 j + i / 8 of the lane's group of 16 (i:
    // lane within the group), element i % 8.  Byte p of every operand holds
    // key 32 (p / 16) + 8 ((p % 16) / 4) + 4 g + p % 4 -- the register order
    // of the S^T accumulators -- so this lane addresses key row
    // 16 t + 8 (j / 4) + 4 g + j % 4 with j = (lane % 16) / 2, at the 8 bytes
    // from column 32 db + 16 ((lane / 16) % 2) + 8 (lane % 2).
    uint32_t voff[4];
    {
        const uint32_t j = (uint32_t)(lane & 15) >> 1;
        const uint32_t row = 8 * (j >> 2) + 4 * (uint32_t)g + (j & 3);
#pragma unroll
        for (int db = 0; db < 4; ++db)
            voff[db] = f8_off(row, (uint32_t)(32 * db + 16 * ((lane >> 4) & 1) + 8 * (lane & 1)));
    }

    // Tile loads: chunk c of a tile is 8 rows; lane l loads the logical
    // 16-byte chunk that the swizzle places at position l % 8 of its row.
    uint32_t lboff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const uint32_t r = (uint32_t)(RPC * (wave + i * NW) + lane / 8);
        lboff[i] = r * 128u + ((((uint32_t)lane % 8u) ^ f8_swz(r)) << 4);
    }
    const uint32_t head_bytes = (uint32_t)Nk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, head_bytes), vrs = make_rsrc(V, head_bytes);
    auto kbuf = [&](int m) { return m == 0 ? (lds_char *)ks0 : (lds_char *)ks1; };
    auto vbuf = [&](int m) { return m == 0 ? (lds_char *)vs0 : (lds_char *)vs1; };
    auto load_kv = [&](int tk, int kbm, int tv, int vbm) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = wave + i * NW;
            buf2lds16(krs, lboff[i], (uint32_t)(tk * BC) * (uint32_t)D, kbuf(kbm) + c * CB);
            buf2lds16(vrs, lboff[i], (uint32_t)(tv * BC) * (uint32_t)D, vbuf(vbm) + c * CB);
        }
    };

    // (q0 + BQ + off and q0w + 32 + off stay below N + BQ + Nk; clamped by Nk first)
    auto tiles_to = [&](int end) {
        end = end < Nk ? end : Nk;
        return end > 0 ? (end + BC - 1) / BC : 0;
    };
    const int NT = tiles_to(CAUSAL ? (q0 + BQ < N ? q0 + BQ : N) + off : Nk);
    const int Tw = q0w < N ? tiles_to(CAUSAL ? (q0w + 32 < N ? q0w + 32 : N) + off : Nk) : 0;
    const int edge_k = CAUSAL ? q0w + off : Nk;   // tiles reaching past this key need masks

    auto is_edge = [&](int t) {
        const int k0 = t * BC;
        return (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > edge_k);
    };
    // Register r of key block kb holds key k0 + 4g + 8(r/4) + r%4.
    auto apply_mask = [&](f32x16 &s, int t, int kb) {
        const int k0 = t * BC + 32 * kb;
        int lim = Nk - 1 - (k0 + 4 * g);
        if (CAUSAL) {
            const int c = qrow + off - (k0 + 4 * g);
            lim = c < lim ? (c > -64 ? c : -64) : lim;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r / 4) + (r % 4);
            if (kk > lim) s[r] = kNegInf;
        }
    };

    float m_run = kNegInf;   // reference row maximum (log2 units of the scaled scores)
    float l_run = 0.f;       // sum of 2^6 P over this lane's half of the keys (unrounded)
    f32x16 o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};
    f32x16 s[2];             // scores of the tile the vector phase works on next
    uint32_t pp[8];          // 2^6 P of that tile in e4m3, byte p = 16 kb + r

    auto vec_phase = [&](int t) {
        if (is_edge(t)) {
            apply_mask(s[0], t, 0);
            apply_mask(s[1], t, 1);
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
        if (__builtin_expect(__ballot(mx * sl2 > m_run + kF8RescaleLog2) != 0, 0)) {
            const float m_new = fmaxf(m_run, max_halves(mx) * sl2);
            const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
            m_run = m_new;
        }
        const float mu = (m_run == kNegInf ? 0.f : m_run) - kF8PScaleLog2;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[kb][4 * i + e], sl2, -mu));
                acc0 = (acc0 + p[0]) + p[1];
                acc1 = (acc1 + p[2]) + p[3];
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                pp[4 * kb + i] = (uint32_t)w;
            }
        }
        l_run += acc0 + acc1;
    };

    // Matrix phase of tile t (M = t % NBUF): O^T += V^T P8^T (V_t) and S^T of
    // tile t + 1 (K_{t+1}), four products each, alternating.
    auto mat_phase = [&](auto m_c) {
        constexpr int M = decltype(m_c)::value;
        constexpr int MK = (M + 1) % NBUF;
        const lds_char *kb_ = MK == 0 ? (lds_char *)ks0 : (lds_char *)ks1;
        const lds_char *vb = M == 0 ? (lds_char *)vs0 : (lds_char *)vs1;
        // S product j: key block j / 2, chunk j % 2 of d.
        auto kfrag = [&](int j) {
            const lds_char *base = kb_ + (j / 2) * 32 * 128;
            const u32x4 x0 = *(const FA_LDS u32x4 *)(base + koff[j % 2][0]);
            const u32x4 x1 = *(const FA_LDS u32x4 *)(base + koff[j % 2][1]);
            return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        };
        // O product db: all 64 keys of the tile, d block db.
        auto vfrag = [&](int db) {
            i32x8 f;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (FA_LDS i32x2 *)(vb + voff[db] + 2048 * t4));
                f[2 * t4] = x[0];
                f[2 * t4 + 1] = x[1];
            }
            return f;
        };
        const i32x8 pf = i32x8{(int)pp[0], (int)pp[1], (int)pp[2], (int)pp[3],
                               (int)pp[4], (int)pp[5], (int)pp[6], (int)pp[7]};
        __builtin_amdgcn_s_setprio(1);
        s[0] = f32x16{};
        s[1] = f32x16{};
        i32x8 kf[2], vf[2];
        kf[0] = kfrag(0);
        vf[0] = vfrag(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j + 1 < 4) {
                kf[(j + 1) & 1] = kfrag(j + 1);
                vf[(j + 1) & 1] = vfrag(j + 1);
            }
            mma8(s[j / 2], kf[j & 1], qf[j % 2]);
            mma8(o[j], vf[j & 1], pf);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Loads run one step ahead (as in the 16-bit forward): the end of step
    // t waits for every load in flight, passes a bare barrier and brings
    // K_{t+3} and V_{t+2}.
    auto end_step = [&](auto m_c, int t) {
        constexpr int M = decltype(m_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_kv(t + 3, (M + 1) % 2, t + 2, M);
    };
    load_kv(0, 0, 0, 0);
    load_kv(1, 1, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (Tw > 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const lds_char *base = (lds_char *)ks0 + kb * 32 * 128;
                const u32x4 x0 = *(const FA_LDS u32x4 *)(base + koff[c][0]);
                const u32x4 x1 = *(const FA_LDS u32x4 *)(base + koff[c][1]);
                mma8(s[kb], i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                  (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]}, qf[c]);
            }
        }
    }
    __syncthreads();
    load_kv(2, 0, 1, 1);   // K_2, V_1

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto step = [&](auto m_c, int t) {
        constexpr int M = decltype(m_c)::value;
        vec_phase(t);
        if (t > 0) end_step(std::integral_constant<int, (M + 1) % 2>{}, t - 1);
        mat_phase(m_c);
    };
    auto end_step_rt = [&](int t) {
        if (t % 2 == 0) end_step(I0{}, t);
        else end_step(I1{}, t);
    };
    for (int t = 0; t < Tw; t += 2) {
        step(I0{}, t);
        if (t + 1 < Tw) step(I1{}, t + 1);
    }
    if (Tw > 0) end_step_rt(Tw - 1);
    for (int t = Tw; t < NT; ++t) end_step_rt(t);
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: O = dv acc / l, LSE = (m + log2 l - 6) ln 2.
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? vsc / l_tot : 0.f;
    if (qrow < N) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float x0 = o[db][4 * rr + 0] * inv, x1 = o[db][4 * rr + 1] * inv;
                const float x2 = o[db][4 * rr + 2] * inv, x3 = o[db][4 * rr + 3] * inv;
                if (a.out_f32) {
                    float *O = reinterpret_cast<float *>(a.o) + head;
                    store4<float>(O + (size_t)qrow * D + col, x0, x1, x2, x3);
                } else {
                    bf16 *O = reinterpret_cast<bf16 *>(a.o) + head;
                    store4<bf16>(O + (size_t)qrow * D + col, x0, x1, x2, x3);
                }
            }
        if (g == 0)
            a.lse[(size_t)bh * (size_t)N + qrow] =
                l_tot > 0.f ? (m_run + __log2f(l_tot) - kF8PScaleLog2) * 0.69314718055994530942f : kNegInf;
    }
}

template <bool CAUSAL>
static hipError_t launch_fwd_fp8_k(const FwdArgs &a, hipStream_t stream) {
    using TL = FwdFp8Tile;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    FwdArgs b = a;
    b.group = unit_group(a.B * a.H, nqb, TL::WG_PER_CU);
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL>), dim3((unsigned)units), dim3(TL::THREADS), 0, stream, b);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(int d, bool causal, const FwdArgs &a, hipStream_t stream) {
    if (d != 128 || a.kv_splits != 1) return hipErrorInvalidValue;
    return causal ? launch_fwd_fp8_k<true>(a, stream) : launch_fwd_fp8_k<false>(a, stream);
}

}  // namespace fa
