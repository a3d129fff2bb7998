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
#include "fa_device.hpp"
#include "fa_kernels.hpp"

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
        return d == 64 ? launch_fwd_t<bf16, 64>(causal, dropout, a, stream)
                       : launch_fwd_t<bf16, 128>(causal, dropout, a, stream);
    case Elem::F16:
        return d == 64 ? launch_fwd_t<f16, 64>(causal, dropout, a, stream)
                       : launch_fwd_t<f16, 128>(causal, dropout, a, stream);
    case Elem::F32:
        return d == 64 ? launch_fwd_t<float, 64>(causal, dropout, a, stream)
                       : launch_fwd_t<float, 128>(causal, dropout, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
