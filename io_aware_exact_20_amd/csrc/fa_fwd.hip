// Forward of fused exact attention for gfx950.
//
// One workgroup (four 64-lane wavefronts) owns one (batch, head, block of
// 128 query rows); each wavefront owns 32 query rows.  The key/value
// sequence is streamed through LDS in tiles of 64 keys, double-buffered:
// the next tile is fetched into registers while the matrix cores work on
// the current one ("Tiling", mrodiduger.github.io page; steps 1-2 of
// "Architecture, step by step", interviewsvector.com page).  The running row
// maximum, normaliser and rescaled output accumulator implement the online
// softmax ("Tiling", same page; step 3), and only O and the per-row
// log-sum-exp are written back ("Recomputation" and step 4).
//
// Layout of the products.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the accumulator then gives every lane ONE query row
// (lane % 32) and sixteen of the tile's keys, so the row maximum and row sum
// are in-lane reductions plus one exchange between the two wavefront halves.
// The same registers, rounded to the input type, are directly the B operand
// of O^T += V^T P^T, whose accumulator again holds one query row per lane;
// the online rescaling factor is therefore a per-lane scalar.  K and V sit
// row-major in LDS; the transposed V operand is read with
// ds_read_b64_tr_b16.
//
// Dropout keeps the undropped probabilities in the normaliser and feeds
// keep * P to the product; the keep scale 1/(1-p) multiplies the output
// once at the end, so no rounded copy of p * 1/(1-p) enters the products.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

#ifndef FA_FWD_NW
#define FA_FWD_NW 4   // wavefronts per workgroup of the 16-bit forward
#endif

namespace fa {

template <typename T, int D>
struct FwdTile {
    static constexpr int NW = 4;                  // wavefronts per workgroup
    static constexpr int THREADS = NW * kWave;
    static constexpr int BQ = 32 * NW;            // query rows per workgroup
    static constexpr int BC = 64;                 // keys per LDS tile
    static constexpr int CH = 16 / sizeof(T);     // elements per 16-byte access
    static constexpr int LD = D + CH;             // K and V row pitch in LDS (elements)
    static constexpr int MIN_WG_PER_CU = sizeof(T) == 4 ? 1 : 2;
};

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, (FwdTile<T, D>::MIN_WG_PER_CU))
fwd_kernel(const FwdArgs a) {
    using TL = FwdTile<T, D>;
    constexpr int BQ = TL::BQ, BC = TL::BC, LD = TL::LD, THREADS = TL::THREADS;
    constexpr int NDC = D / 16;   // 16-wide contraction chunks of a row
    constexpr int NDB = D / 32;   // 32-wide column blocks of the output
    constexpr int NKB = BC / 32;  // 32-key blocks of a tile
    constexpr float kNegInf = -__builtin_huge_valf();

    __shared__ __attribute__((aligned(16))) T Ks[2][BC * LD];
    __shared__ __attribute__((aligned(16))) T Vs[2][BC * LD];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int lq = lane % 32, g = lane / 32;

    // Work unit: causal units are visited longest first.
    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int64_t qb = CAUSAL ? (nqb - 1 - u / BH) : (u / BH);
    const int64_t N = a.N;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T *__restrict__ Q = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ K = reinterpret_cast<const T *>(a.k) + head;
    const T *__restrict__ V = reinterpret_cast<const T *>(a.v) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int64_t q0 = qb * BQ;
    const int64_t qrow = q0 + wave * 32 + lq;   // this lane's query row

    // Q stays in registers for the whole key loop: B operand of S^T = K Q^T.
    frag_t<T> qf[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
        if (qrow < N) qf[c] = load_frag<T>(Q + qrow * D + 16 * c + 8 * g);
        else qf[c] = frag_t<T>{};
    }

    const int64_t kend = CAUSAL ? (q0 + BQ < N ? q0 + BQ : N) : N;
    const int ntiles = (int)((kend + BC - 1) / BC);

    TileCopy<T, BC, D, THREADS> kcopy, vcopy;

    float m_run = kNegInf;   // running row maximum, log2 units of scaled scores
    float l_run = 0.f;       // running normaliser (this lane's half of the keys)
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    kcopy.load(K, 0, N, tid);
    vcopy.load(V, 0, N, tid);
    kcopy.template store<LD>(Ks[0], tid);
    vcopy.template store<LD>(Vs[0], tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const T *ks = Ks[buf];
        const T *vs = Vs[buf];
        if (t + 1 < ntiles) {
            kcopy.load(K, (int64_t)(t + 1) * BC, N, tid);
            vcopy.load(V, (int64_t)(t + 1) * BC, N, tid);
        }

        // S^T for the tile's 32-key blocks.
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                const frag_t<T> kf = load_frag<T>(ks + (kb * 32 + lq) * LD + 16 * c + 8 * g);
                mma(s[kb], kf, qf[c]);
            }
        }

        // Causal and sequence-end masking (only tiles that reach them).
        const int64_t k0 = (int64_t)t * BC;
        const bool edge = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
        if (edge) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = k0 + kb * 32 + 8 * (r / 4) + 4 * g + (r % 4);
                    if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = kNegInf;
                }
        }

        // Online softmax update (scores scaled by scale * log2(e); exp2).
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rowsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], a.scale_log2, -m_use));
                s[kb][r] = p;
                rowsum += p;
            }
        l_run = l_run * alpha + rowsum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

        // Dropout: dropped probabilities leave the product (not the normaliser).
        if (DROPOUT) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const uint32_t keep = keep_bits_row((uint32_t)(k0 + kb * 32), (uint32_t)qrow, h_idx,
                                                    b_idx, a.seed_lo, a.seed_hi, a.drop_T);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((keep >> r) & 1u)) s[kb][r] = 0.f;
            }
        }

        // O^T += V^T P^T; V^T fragments come straight from the row-major tile.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const frag_t<T> pf = pack8<T>(s[kb], 8 * cc);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const frag_t<T> vf = load_frag_tr<T>(vs, LD, kb * 32 + 16 * cc, 32 * db);
                    mma(acc[db], vf, pf);
                }
            }

        if (t + 1 < ntiles) {
            kcopy.template store<LD>(Ks[buf ^ 1], tid);
            vcopy.template store<LD>(Vs[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue: O = c * acc / l and LSE = ln(l) + max; rows past N are not stored.
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? (DROPOUT ? a.drop_c : 1.f) / l_tot : 0.f;
    if (qrow < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float x0 = acc[db][4 * rr + 0] * inv, x1 = acc[db][4 * rr + 1] * inv;
                const float x2 = acc[db][4 * rr + 2] * inv, x3 = acc[db][4 * rr + 3] * inv;
                if (a.out_f32) {
                    float *O = reinterpret_cast<float *>(a.o) + head;
                    store4<float>(O + qrow * D + col, x0, x1, x2, x3);
                } else {
                    T *O = reinterpret_cast<T *>(a.o) + head;
                    store4<T>(O + qrow * D + col, x0, x1, x2, x3);
                }
            }
        if (g == 0) {
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f
                                          : kNegInf;
            a.lse[(size_t)bh * (size_t)N + qrow] = lse;
        }
    }
}

// ===================================================================
// 16-bit forward: 64 query rows per wavefront.
//
// Each wavefront holds 64 query rows (two 32-row column blocks of the S^T
// accumulators), so every K and V fragment read from LDS feeds two matrix
// products.  This halves the LDS traffic per flop against 32-row
// wavefronts, which matters on gfx950: the transposed reads that give the
// V^T operand (ds_read_b64_tr_b16) stream at about 85 bytes/clk/CU, well
// below the plain 16-byte reads.  With one wavefront per SIMD (about 350
// registers per lane), the matrix cores and the softmax arithmetic overlap
// within the wavefront.
//
// K and V tiles of 64 keys sit in swizzled LDS tiles filled by direct
// global-to-LDS loads, double-buffered; every LDS address is a per-lane
// constant plus an immediate offset.  The online softmax keeps a reference
// maximum per row and only moves it (rescaling the accumulator and
// normaliser) when a tile's maximum exceeds it by more than 2^8 in
// probability; otherwise the tile's probabilities are formed against the
// stale reference, which is exact in real arithmetic and keeps every
// probability below 256.  Row sums are taken on the rounded probabilities
// that enter the product (v_dot2c_f32_bf16), so the output is a convex
// combination of V rows with exactly the weights used.
template <typename T, int D, int NW>
struct Fwd16Tile {
    static constexpr int RW = 64;                 // query rows per wavefront
    static constexpr int NB = RW / 32;            // 32-row blocks per wavefront
    static constexpr int BQ = NW * RW;            // query rows per workgroup
    static constexpr int BC = 64;                 // keys per tile
    static constexpr int THREADS = NW * kWave;
    static constexpr int TILE_BYTES = BC * D * 2;
    static constexpr int LOADS = TILE_BYTES / (kWave * 16) / NW;   // per wave per tile
};

// Threshold (log2 units) by which a tile's maximum must exceed the
// reference maximum before the accumulator is rescaled.
constexpr float kRescaleLog2 = 8.0f;

template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef T t2 __attribute__((ext_vector_type(2)));
    t2 v;
    v[0] = from_f32<T>(lo);
    v[1] = from_f32<T>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// acc += lo + hi of a packed pair of 16-bit values (exact products with 1).
template <typename T>
__device__ __forceinline__ float sum2(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float sum2<bf16>(uint32_t pair, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, pair), one, acc, false);
}
template <>
__device__ __forceinline__ float sum2<f16>(uint32_t pair, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pair), one, acc, false);
}

template <typename T, int D, int NW, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(NW * 64, 4 / NW) fwd16_kernel(const FwdArgs a) {
    using TL = Fwd16Tile<T, D, NW>;
    using SW = Swz<D>;
    constexpr int NB = TL::NB, BQ = TL::BQ, BC = TL::BC, RW = TL::RW;
    constexpr int TB = TL::TILE_BYTES, LOADS = TL::LOADS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;   // contraction chunks of S
    constexpr int NDB = D / 32;   // 32-column blocks of O
    constexpr int NKB = BC / 32;  // 32-key blocks of a tile
    constexpr float kNegInf = -__builtin_huge_valf();

    // LDS: K buffers at [0, 2TB), V buffers at [2TB, 4TB).
    __shared__ __attribute__((aligned(1024))) char smem[4 * TB];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(FA_LDS char *)smem;

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lq = lane & 31, g = lane >> 5;

    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int64_t qb = CAUSAL ? (nqb - 1 - u / BH) : (u / BH);
    const int N = (int)a.N;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T *__restrict__ Q = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ K = reinterpret_cast<const T *>(a.k) + head;
    const T *__restrict__ V = reinterpret_cast<const T *>(a.v) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int q0 = (int)qb * BQ;             // first query row of the workgroup
    const int q0w = q0 + wave * RW;           // first query row of this wavefront

    // ---- Q fragments (B operand of S^T = K Q^T), rows clamped into range.
    frag_t<T> qf[NB][NDC];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        int r = q0w + 32 * nb + lq;
        r = r < N ? r : N - 1;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            qf[nb][c] = load_frag<T>(Q + (size_t)r * D + 16 * c + 8 * g);
            pin_agpr(qf[nb][c]);
        }
    }

    // ---- per-lane LDS read offsets (bytes, relative to a tile buffer).
    uint32_t koff[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) koff[c] = SW::off(lq, 16 * c + 8 * g);
    uint32_t voff[2][NDB];
    {
        const int G = lane >> 4, k = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                voff[hf][db] = SW::off(8 * hf + 4 * (G >> 1) + k, 32 * db + 16 * (G & 1) + 4 * j);
    }
    // ---- per-lane global offsets (elements) of the direct tile loads.
    uint32_t grow[LOADS], gcol[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int L = (i * NW + wave) * kWave + lane;     // 16-byte chunk of the tile
        const int R = L / SW::CPR, pos = L % SW::CPR;
        grow[i] = (uint32_t)R;
        gcol[i] = (uint32_t)((pos ^ (int)SW::f(R)) * 8);
    }

    const int kend = CAUSAL ? (q0 + BQ < N ? q0 + BQ : N) : N;
    const int ntiles = (kend + BC - 1) / BC;
    // Tiles this wavefront needs (causal: up to its own last row).
    const int wend = CAUSAL ? (q0w + RW < N ? q0w + RW : N) : N;
    const int wtiles = (wend + BC - 1) / BC;

    auto load_tile = [&](int t, int buf) {
        const int k0 = t * BC;
        const uint32_t kb_lds = lds0 + buf * TB + wave * (kWave * 16);
        const uint32_t vb_lds = lds0 + 2 * TB + buf * TB + wave * (kWave * 16);
        if (k0 + BC <= N) {
            const T *Kt = K + (size_t)k0 * D, *Vt = V + (size_t)k0 * D;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const uint32_t e = grow[i] * D + gcol[i];
                g2lds16(Kt + e, kb_lds + i * NW * (kWave * 16));
                g2lds16(Vt + e, vb_lds + i * NW * (kWave * 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                int r = k0 + (int)grow[i];
                r = r < N ? r : N - 1;
                const size_t e = (size_t)r * D + gcol[i];
                g2lds16(K + e, kb_lds + i * NW * (kWave * 16));
                g2lds16(V + e, vb_lds + i * NW * (kWave * 16));
            }
        }
    };

    const float sl2 = a.scale_log2;
    float m_run[NB], l_run[NB];
    f32x16 o[NDB][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = kNegInf;
        l_run[nb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            o[db][nb] = f32x16{};
            pin_agpr(o[db][nb]);
        }
    }

    // One key tile: K in buffer BUF of the K area, V in buffer BUF of the V
    // area (BUF is a compile-time constant so that every LDS address is a
    // per-lane register plus an immediate).
    auto tile = [&](auto buf_c, int t) {
        constexpr int BUF = decltype(buf_c)::value;
        constexpr uint32_t KB = BUF * TB, VB = 2 * TB + BUF * TB;
        const int k0 = t * BC;

        // ---- S^T = K Q^T: s[kb][nb] register r <-> key k0 + 32kb + 8(r/4) + 4g + r%4,
        // query q0w + 32nb + lq.
        f32x16 s[NKB][NB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[kb][nb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                const frag_t<T> kf = lds_frag<T>(lds0 + KB + kb * 32 * RB + koff[c]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) mma(s[kb][nb], kf, qf[nb][c]);
            }
        }

        // ---- causal and sequence-end masks (edge tiles only).
        const bool edge = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0w);
        if (edge) {
            const int rel = k0 + 4 * g - (q0w + lq);   // key - query at kb = nb = r = 0
            const int kmax = N - 1 - (k0 + 4 * g);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = 32 * kb + 8 * (r / 4) + (r % 4);
                        const bool masked = (kk > kmax) || (CAUSAL && rel + kk - 32 * nb > 0);
                        if (masked) s[kb][nb][r] = kNegInf;
                    }
        }

        // ---- row maxima of the tile (this lane's half of the keys).
        float mx[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float x = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) x = fmaxf(x, fmaxf(s[kb][nb][r], s[kb][nb][r + 1]));
            mx[nb] = x;
        }
        bool need = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) need |= mx[nb] * sl2 > m_run[nb] + kRescaleLog2;
        if (__builtin_expect(__ballot(need) != 0, 0)) {
            // Move the reference maxima to the exact row maxima.
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float m_new = fmaxf(m_run[nb], max_halves(mx[nb]) * sl2);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run[nb] - m_new);
                l_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    pin_agpr(o[db][nb]);
                    o[db][nb] *= alpha;
                    pin_agpr(o[db][nb]);
                }
                m_run[nb] = m_new;
            }
        }

        // ---- probabilities against the reference maxima; row sums of the
        // rounded values; dropout; O^T += V^T P^T.
        uint32_t pp[NKB][NB][8];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float mu = m_run[nb] == kNegInf ? 0.f : m_run[nb];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p0 = fast_exp2(fmaf(s[kb][nb][2 * i], sl2, -mu));
                    const float p1 = fast_exp2(fmaf(s[kb][nb][2 * i + 1], sl2, -mu));
                    pp[kb][nb][i] = pack2<T>(p0, p1);
                }
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    acc0 = sum2<T>(pp[kb][nb][i], acc0);
                    acc1 = sum2<T>(pp[kb][nb][i + 1], acc1);
                }
            l_run[nb] += acc0 + acc1;
        }
        if (DROPOUT) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const uint32_t keep = keep_bits_row((uint32_t)(k0 + 32 * kb),
                                                        (uint32_t)(q0w + 32 * nb + lq), h_idx,
                                                        b_idx, a.seed_lo, a.seed_hi, a.drop_T);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t m0 = ((keep >> (2 * i)) & 1u) ? 0x0000FFFFu : 0u;
                        const uint32_t m1 = ((keep >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u;
                        pp[kb][nb][i] &= (m0 | m1);
                    }
                }
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t kc_off = (uint32_t)((32 * kb + 16 * cc) * RB);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const frag_t<T> vf = join<T>(lds_half_tr<T>(lds0 + VB + kc_off + voff[0][db]),
                                                 lds_half_tr<T>(lds0 + VB + kc_off + voff[1][db]));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        u32x4 pv;
                        pv[0] = pp[kb][nb][4 * cc + 0];
                        pv[1] = pp[kb][nb][4 * cc + 1];
                        pv[2] = pp[kb][nb][4 * cc + 2];
                        pv[3] = pp[kb][nb][4 * cc + 3];
                        mma(o[db][nb], vf, __builtin_bit_cast(frag_t<T>, pv));
                    }
                }
            }
    };

    // Tile loop, two tiles per trip (buffers 0 and 1).  Tile t+1 is fetched
    // while tile t is consumed; one barrier per tile frees the buffer the
    // next fetch overwrites.
    load_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0): this wave's tile loads have landed
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) load_tile(t + 1, 1);
        if (t < wtiles) tile(std::integral_constant<int, 0>{}, t);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 >= ntiles) break;
        if (t + 2 < ntiles) load_tile(t + 2, 0);
        if (t + 1 < wtiles) tile(std::integral_constant<int, 1>{}, t + 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: O = c * acc / l, LSE = (m + log2 l) ln 2.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int qrow = q0w + 32 * nb + lq;
        const float l_tot = sum_halves(l_run[nb]);
        const float inv = l_tot > 0.f ? (DROPOUT ? a.drop_c : 1.f) / l_tot : 0.f;
        if (qrow < N) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr + 4 * g;
                    const float x0 = o[db][nb][4 * rr + 0] * inv, x1 = o[db][nb][4 * rr + 1] * inv;
                    const float x2 = o[db][nb][4 * rr + 2] * inv, x3 = o[db][nb][4 * rr + 3] * inv;
                    if (a.out_f32) {
                        float *O = reinterpret_cast<float *>(a.o) + head;
                        store4<float>(O + (size_t)qrow * D + col, x0, x1, x2, x3);
                    } else {
                        T *O = reinterpret_cast<T *>(a.o) + head;
                        store4<T>(O + (size_t)qrow * D + col, x0, x1, x2, x3);
                    }
                }
            if (g == 0) {
                const float lse = l_tot > 0.f ? (m_run[nb] + __log2f(l_tot)) * 0.69314718055994530942f
                                              : kNegInf;
                a.lse[(size_t)bh * (size_t)N + qrow] = lse;
            }
        }
    }
}

template <typename T, int D, int NW>
static hipError_t launch_fwd16_t(bool causal, bool dropout, const FwdArgs &a, hipStream_t stream) {
    using TL = Fwd16Tile<T, D, NW>;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((fwd16_kernel<T, D, NW, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fwd16_kernel<T, D, NW, true, false>), grid, block, 0, stream, a);
    } else {
        if (dropout) hipLaunchKernelGGL((fwd16_kernel<T, D, NW, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fwd16_kernel<T, D, NW, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_t(bool causal, bool dropout, const FwdArgs &a, hipStream_t stream) {
    constexpr int BQ = FwdTile<T, D>::BQ;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const int64_t units = a.B * a.H * nqb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(FwdTile<T, D>::THREADS);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((fwd_kernel<T, D, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fwd_kernel<T, D, true, false>), grid, block, 0, stream, a);
    } else {
        if (dropout) hipLaunchKernelGGL((fwd_kernel<T, D, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fwd_kernel<T, D, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_fwd(Elem e, int d, bool causal, bool dropout, const FwdArgs &a,
                      hipStream_t stream) {
    switch (e) {
    case Elem::BF16:
        return d == 64 ? launch_fwd16_t<bf16, 64, FA_FWD_NW>(causal, dropout, a, stream)
                       : launch_fwd16_t<bf16, 128, FA_FWD_NW>(causal, dropout, a, stream);
    case Elem::F16:
        return d == 64 ? launch_fwd16_t<f16, 64, FA_FWD_NW>(causal, dropout, a, stream)
                       : launch_fwd16_t<f16, 128, FA_FWD_NW>(causal, dropout, a, stream);
    case Elem::F32:
        return d == 64 ? launch_fwd_t<float, 64>(causal, dropout, a, stream)
                       : launch_fwd_t<float, 128>(causal, dropout, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
