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

namespace fa {

// The generic forward serves fp32 inputs (16-bit inputs take fa_fwd_pp.hip).
template <typename T, int D>
struct FwdTile {
    static_assert(sizeof(T) == 4, "generic forward: fp32 inputs");
    static constexpr int NW = 4;                  // wavefronts per workgroup
    static constexpr int THREADS = NW * kWave;
    static constexpr int BQ = 32 * NW;            // query rows per workgroup
    static constexpr int BC = 64;                 // keys per LDS tile
    static constexpr int CH = 16 / sizeof(T);     // elements per 16-byte access
    static constexpr int LD = D + CH;             // K and V row pitch in LDS (elements)
    static constexpr int MIN_WG_PER_CU = 1;
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

    // Work unit: (batch, head), query block, key chunk; causal query blocks
    // longest first.
    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)(nqb * a.kv_splits), a.group);
    const int64_t bh = un.bh;
    const int64_t qi = un.rank / (uint32_t)a.kv_splits;
    const int split = (int)(un.rank % (uint32_t)a.kv_splits);
    const int64_t qb = CAUSAL ? (nqb - 1 - qi) : qi;
    const int64_t N = a.N, Nk = a.Nk;
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Q = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ K = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ V = reinterpret_cast<const T *>(a.v) + head_kv;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int64_t q0 = qb * BQ;
    const int64_t qrow = q0 + wave * 32 + lq;   // this lane's query row
    // Keys of this unit: [klo, khi); causal rows see keys up to row + off.
    const int64_t klo = (int64_t)split * a.kv_chunk;
    const int64_t khi = klo + a.kv_chunk < Nk ? klo + a.kv_chunk : Nk;
    const int64_t off = Nk - N;

    // Q stays in registers for the whole key loop: B operand of S^T = K Q^T.
    frag_t<T> qf[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
        if (qrow < N) qf[c] = load_frag<T>(Q + qrow * D + 16 * c + 8 * g);
        else qf[c] = frag_t<T>{};
    }

    int64_t kend = CAUSAL ? q0 + BQ + off : Nk;
    kend = kend < khi ? kend : khi;
    const int ntiles = kend > klo ? (int)((kend - klo + BC - 1) / BC) : 0;

    TileCopy<T, BC, D, THREADS> kcopy, vcopy;

    float m_run = kNegInf;   // running row maximum, log2 units of scaled scores
    float l_run = 0.f;       // running normaliser (this lane's half of the keys)
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    kcopy.load(K, klo, Nk, tid);
    vcopy.load(V, klo, Nk, tid);
    kcopy.template store<LD>(Ks[0], tid);
    vcopy.template store<LD>(Vs[0], tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const T *ks = Ks[buf];
        const T *vs = Vs[buf];
        if (t + 1 < ntiles) {
            kcopy.load(K, klo + (int64_t)(t + 1) * BC, Nk, tid);
            vcopy.load(V, klo + (int64_t)(t + 1) * BC, Nk, tid);
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

        // Causal and key-end masking (only tiles that reach them).
        const int64_t k0 = klo + (int64_t)t * BC;
        const bool edge = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0 + off);
        if (edge) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = k0 + kb * 32 + 8 * (r / 4) + 4 * g + (r % 4);
                    if (key >= Nk || (CAUSAL && key > qrow + off)) s[kb][r] = kNegInf;
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

    // Epilogue: O = c * acc / l and LSE = ln(l) + max -- of the chunk, in
    // fp32 to the partial buffers, when the keys are split; rows past N are
    // not stored.
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? (DROPOUT ? a.drop_c : 1.f) / l_tot : 0.f;
    const bool part = a.kv_splits > 1;
    const size_t prow = ((size_t)split * (size_t)BH + (size_t)bh) * (size_t)N;
    if (qrow < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float x0 = acc[db][4 * rr + 0] * inv, x1 = acc[db][4 * rr + 1] * inv;
                const float x2 = acc[db][4 * rr + 2] * inv, x3 = acc[db][4 * rr + 3] * inv;
                if (part) {
                    store4<float>(a.part_o + (prow + qrow) * D + col, x0, x1, x2, x3);
                } else if (a.out_f32) {
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
            if (part) a.part_lse[prow + qrow] = lse;
            else a.lse[(size_t)bh * (size_t)N + qrow] = lse;
        }
    }
}

template <typename T, int D>
static hipError_t launch_fwd_t(bool causal, bool dropout, const FwdArgs &a, hipStream_t stream) {
    constexpr int BQ = FwdTile<T, D>::BQ;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const int64_t units = a.B * a.H * nqb * a.kv_splits;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(FwdTile<T, D>::THREADS);
    FwdArgs b = a;
    b.group = unit_group(a.B * a.H, nqb * a.kv_splits, FwdTile<T, D>::MIN_WG_PER_CU);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((fwd_kernel<T, D, true, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((fwd_kernel<T, D, true, false>), grid, block, 0, stream, b);
    } else {
        if (dropout) hipLaunchKernelGGL((fwd_kernel<T, D, false, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((fwd_kernel<T, D, false, false>), grid, block, 0, stream, b);
    }
    return hipGetLastError();
}

// ===================================================================
// Merge of the key-chunk results of a split forward.  Chunk s holds, per
// query row, O_s normalised over its own keys and LSE_s; the row's result is
// LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, the same
// rescaling the online softmax applies between key tiles ("Tiling",
// mrodiduger.github.io page).  A row that no chunk sees gets O = 0,
// LSE = -inf.  One thread per four columns of a row.
template <typename TO, int D>
__global__ void __launch_bounds__(256) fwd_merge_kernel(const FwdArgs a, int64_t rows) {
    constexpr int CPR = D / 4;
    constexpr float kNegInf = -__builtin_huge_valf();
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = idx / CPR;
    const int col = (int)(idx % CPR) * 4;
    if (row >= rows) return;
    const int S = a.kv_splits;
    float m = kNegInf;
    for (int s = 0; s < S; ++s) m = fmaxf(m, a.part_lse[(size_t)s * rows + row]);
    float l = 0.f, x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    if (m != kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float ls = a.part_lse[(size_t)s * rows + row];
            const float w = ls == kNegInf ? 0.f : expf(ls - m);
            const float4 x = *reinterpret_cast<const float4 *>(a.part_o + ((size_t)s * rows + row) * D + col);
            l += w;
            x0 = fmaf(w, x.x, x0);
            x1 = fmaf(w, x.y, x1);
            x2 = fmaf(w, x.z, x2);
            x3 = fmaf(w, x.w, x3);
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    store4<TO>(reinterpret_cast<TO *>(a.o) + (size_t)row * D + col, x0 * inv, x1 * inv, x2 * inv, x3 * inv);
    if (col == 0) a.lse[row] = l > 0.f ? m + logf(l) : kNegInf;
}

template <typename T, int D>
static hipError_t launch_merge_t(const FwdArgs &a, hipStream_t stream) {
    const int64_t rows = a.B * a.H * a.N;
    const int64_t threads = rows * (D / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.out_f32 || sizeof(T) == 4)
        hipLaunchKernelGGL((fwd_merge_kernel<float, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
    else
        hipLaunchKernelGGL((fwd_merge_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_merge_d(int d, const FwdArgs &a, hipStream_t stream) {
    switch (d) {
    case 32: return launch_merge_t<T, 32>(a, stream);
    case 64: return launch_merge_t<T, 64>(a, stream);
    case 96: return launch_merge_t<T, 96>(a, stream);
    case 128: return launch_merge_t<T, 128>(a, stream);
    case 256: return launch_merge_t<T, 256>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_merge(Elem e, int d, const FwdArgs &a, hipStream_t stream) {
    switch (e) {
    case Elem::BF16: return launch_merge_d<bf16>(d, a, stream);
    case Elem::F16: return launch_merge_d<f16>(d, a, stream);
    case Elem::F32: return launch_merge_d<float>(d, a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(Elem e, int d, bool causal, bool dropout, const FwdArgs &a,
                      hipStream_t stream) {
    // 16-bit inputs take the kernel of fa_fwd_pp.hip; fp32 inputs the generic
    // one (32 rows per wavefront).
    switch (e) {
    case Elem::BF16:
        switch (d) {
        case 32: case 64: case 96: case 128: case 256: return launch_fwd_pp(e, d, causal, dropout, a, stream);
        }
        break;
    case Elem::F16:
        switch (d) {
        case 32: case 64: case 96: case 128: case 256: return launch_fwd_pp(e, d, causal, dropout, a, stream);
        }
        break;
    case Elem::F32:
        switch (d) {
        case 32: return launch_fwd_t<float, 32>(causal, dropout, a, stream);
        case 64: return launch_fwd_t<float, 64>(causal, dropout, a, stream);
        case 96: return launch_fwd_t<float, 96>(causal, dropout, a, stream);
        case 128: return launch_fwd_t<float, 128>(causal, dropout, a, stream);
        }
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
