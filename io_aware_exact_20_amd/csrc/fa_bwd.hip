// Backward of fused exact attention for gfx950.
//
// Nothing of the forward's N x N intermediates is stored: the scores and
// probabilities are recomputed from Q, K and the stored log-sum-exp
// ("Recomputation", mrodiduger.github.io page).  With
//
//   S = scale Q K^T,  P = exp(S - LSE),  P~ = P * keep * c,
//   dP = (dO V^T) * keep * c,  D_i = dO_i . O_i,  dS = P o (dP - D),
//
// the gradients are dV = P~^T dO, dK = scale dS^T Q and dQ = scale dS K.
// Three kernels run in order on the caller's stream:
//
//   bwd_pre   D_i in fp32 (16 lanes per row);
//   bwd_dkdv  one workgroup per (batch, head, block of 32*NW keys); each
//             wavefront keeps its 32 keys' K and V rows in registers and
//             walks the query tiles, recomputing S, P and dP and
//             accumulating dV^T and dK^T in registers; the keys sit along
//             the accumulator columns, so every lane holds one key and the
//             rounded S / dS registers are directly the B operands of the
//             dV and dK products;
//   bwd_dq    one workgroup per (batch, head, block of 128 query rows),
//             shaped like the forward: recomputes S^T and dP^T with one
//             query row per lane and accumulates dQ^T += K^T dS^T.
//
// dQ is thus produced without atomics and without storing dS: the price is
// recomputing S and dP a second time (seven block products instead of
// five).  Q, dO, K and V tiles sit row-major in LDS; their transposed
// operands are read with ds_read_b64_tr_b16.  Products run on
// v_mfma_f32_32x32x16 (fp32 inputs: v_mfma_f32_32x32x2f32) with fp32
// accumulation.  The dropout keep scale c multiplies dP in fp32 and dV once
// at the end; the products see keep * P, not a rounded P * c.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr float kLog2e = 1.44269504088896340736f;

// ------------------------------------------------------------- preprocess

// Row statistics of the backward, one value per query row in fp32:
// D_i / c with D_i = sum_c dO_ic O_ic and c the dropout keep scale (1
// without dropout), and -lse_i log2(e).  With D_i / c the dS of every
// kernel is dS / c = P o (keep dP - D / c), and c joins the scale of dK and
// dQ.  16 lanes per row, kPreRows rows per 16-lane group: every lane issues
// the loads of all its rows before it uses any, so that a wavefront keeps
// 2 kPreRows loads per lane in flight.  Against one row per group: d = 32
// 23 % and 2048-row heads 8 % faster, the training shape 1-3 %; at d = 256
// (32-byte pieces already) four rows were 6 % slower, so it keeps one.
template <int D>
constexpr int kPreRows = D >= 256 ? 1 : 4;

template <typename T, typename TO, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdArgs a, int64_t rows) {
    constexpr int PER = D / 16;
    constexpr int R = kPreRows<D>;
    const int sub = threadIdx.x % 16;
    // group k of the workgroup takes rows base + 16 r + k, r < R
    const int64_t base = (int64_t)blockIdx.x * 16 * R + threadIdx.x / 16;
    TO ov[R][PER];
    T dv[R][PER];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = base + 16 * r;
        const int64_t at = (row < rows ? row : 0) * D + sub * PER;
        const TO *o = reinterpret_cast<const TO *>(a.o) + at;
        const T *dout = reinterpret_cast<const T *>(a.dout) + at;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            ov[r][i] = o[i];
            dv[r][i] = dout[i];
        }
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[r] += to_f32(ov[r][i]) * to_f32(dv[r][i]);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += __shfl_xor(acc[r], off, 16);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = base + 16 * r;
        if (sub == r && row < rows) {
            a.dvec[row] = acc[r] / a.drop_c;
            // A row that sees no key (LSE = -inf) gets -inf, so that its P is 0.
            const float l = a.lse[row];
            a.nl2[row] = l == -__builtin_huge_valf() ? l : -l * kLog2e;
        }
    }
}

// ---------------------------------------------------------------- dK, dV

// The generic dK/dV and dQ kernels serve fp32 inputs (16-bit inputs take
// fa_dkdv16.hip and fa_dq16.hpp).
template <typename T, int D>
struct DkdvTile {
    static_assert(sizeof(T) == 4, "generic dK/dV: fp32 inputs");
    static constexpr int NW = 2;                        // wavefronts per workgroup
    static constexpr int THREADS = NW * kWave;
    static constexpr int BK = 32 * NW;                  // keys per workgroup
    static constexpr int BQ = 32;                       // query rows per tile
    static constexpr int CH = 16 / sizeof(T);
    static constexpr int LD = D + CH;                   // row pitch of Q and dO tiles
};

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_kernel(const BwdArgs a) {
    using TL = DkdvTile<T, D>;
    constexpr int NW = TL::NW, BK = TL::BK, BQ = TL::BQ, LD = TL::LD, THREADS = TL::THREADS;
    constexpr int NDC = D / 16, NDB = D / 32, NQB = BQ / 32;

    __shared__ __attribute__((aligned(16))) T Qs[2][BQ * LD];
    __shared__ __attribute__((aligned(16))) T dOs[2][BQ * LD];
    __shared__ float lse2_s[2][BQ];
    __shared__ float dvec_s[2][BQ];
    __shared__ __attribute__((aligned(16))) uint32_t keep_s[NW][BQ];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int lq = lane % 32, g = lane / 32;

    const int64_t BH = a.B * a.H;
    const int64_t nkb = (a.Nk + BK - 1) / BK;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)nkb, a.group);
    const int64_t bh = un.bh;
    const int64_t kblk = un.rank;                 // causal: low key blocks (most work) first
    const int64_t N = a.N, Nk = a.Nk;
    const int64_t off = Nk - N;                   // causal: query i sees keys j <= i + off
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head_kv;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const float *__restrict__ lse_g = a.lse + (size_t)bh * (size_t)N;
    const float *__restrict__ dvec_g = a.dvec + (size_t)bh * (size_t)N;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int64_t k0 = kblk * BK;                 // first key of the workgroup
    const int64_t kw0 = k0 + wave * 32;           // first key of this wavefront
    const int64_t key = kw0 + lq;                 // this lane's key

    // K and V rows of the lane's key: B operands of S = Q K^T and dP~ = dO V^T.
    frag_t<T> kf[NDC], vf[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
        if (key < Nk) {
            kf[c] = load_frag<T>(Kg + key * D + 16 * c + 8 * g);
            vf[c] = load_frag<T>(Vg + key * D + 16 * c + 8 * g);
        } else {
            kf[c] = frag_t<T>{};
            vf[c] = frag_t<T>{};
        }
    }

    f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dv_acc[db] = f32x16{}; dk_acc[db] = f32x16{}; }

    TileCopy<T, BQ, D, THREADS> qcopy, dcopy;
    float lse_r = 0.f, dvec_r = 0.f;
    auto load_rows = [&](int64_t q0) {
        qcopy.load(Qg, q0, N, tid);
        dcopy.load(dOg, q0, N, tid);
        if (tid < BQ) {
            const int64_t q = q0 + tid;
            // Rows past N get P = exp2(-inf) = 0.
            // (and rows that see no key, LSE = -inf)
            lse_r = q < N && lse_g[q] != -__builtin_huge_valf() ? lse_g[q] * kLog2e
                                                                : __builtin_huge_valf();
            dvec_r = q < N ? dvec_g[q] : 0.f;
        }
    };
    auto store_rows = [&](int buf) {
        qcopy.template store<LD>(Qs[buf], tid);
        dcopy.template store<LD>(dOs[buf], tid);
        if (tid < BQ) { lse2_s[buf][tid] = lse_r; dvec_s[buf][tid] = dvec_r; }
    };

    const int64_t qstart = CAUSAL ? (k0 - off > 0 ? (k0 - off) / BQ * BQ : 0) : 0;
    const int ntiles = N > qstart ? (int)((N - qstart + BQ - 1) / BQ) : 0;
    load_rows(qstart);
    store_rows(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int64_t q0 = qstart + (int64_t)t * BQ;
        const T *qs = Qs[buf];
        const T *dos = dOs[buf];
        if (t + 1 < ntiles) load_rows(q0 + BQ);

        const bool edge = (q0 + BQ > N) || (k0 + BK > Nk) || (CAUSAL && k0 + BK - 1 > q0 + off);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            // ---- S = Q K^T and dP~ = dO V^T for this wavefront's 32 keys;
            // register r holds query row q0 + 32qb + 8(r/4) + 4g + r%4.
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                const frag_t<T> qa = load_frag<T>(qs + (32 * qb + lq) * LD + 16 * c + 8 * g);
                mma(s, qa, kf[c]);
                const frag_t<T> da = load_frag<T>(dos + (32 * qb + lq) * LD + 16 * c + 8 * g);
                mma(dp, da, vf[c]);
            }

            // ---- keep bits of the 32 rows x 32 keys block, transposed through LDS:
            // lane (row lq, half g) draws the row's key groups 2g, 2g+1 and
            // writes them as one half of the row's 32-bit word.
            uint32_t keepw[16];
            if (DROPOUT) {
                const uint32_t grp = (uint32_t)(kw0 >> 3) + 2 * g;
                const uint32_t row = (uint32_t)(q0 + 32 * qb + lq);
                const uint32_t lo = keep_byte(grp, row, h_idx, b_idx, a.seed_lo, a.seed_hi, a.drop_T);
                const uint32_t hi = keep_byte(grp + 1, row, h_idx, b_idx, a.seed_lo, a.seed_hi, a.drop_T);
                reinterpret_cast<uint16_t *>(&keep_s[wave][lq])[g] = (uint16_t)(lo | (hi << 8));
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 w4 = *reinterpret_cast<const uint4 *>(&keep_s[wave][8 * i + 4 * g]);
                    keepw[4 * i + 0] = w4.x; keepw[4 * i + 1] = w4.y;
                    keepw[4 * i + 2] = w4.z; keepw[4 * i + 3] = w4.w;
                }
                __builtin_amdgcn_wave_barrier();
            }

            // ---- P, keep * P and dS.
            float pk[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = 32 * qb + 8 * (r / 4) + 4 * g + (r % 4);
                float p = fast_exp2(fmaf(s[r], a.scale_log2, -lse2_s[buf][qi]));
                if (edge) {
                    const int64_t q = q0 + qi;
                    if (q >= N || key >= Nk || (CAUSAL && key > q + off)) p = 0.f;
                }
                float dpv = dp[r];
                float pkv = p;
                if (DROPOUT) {
                    const bool kept = (keepw[r] >> lq) & 1u;
                    pkv = kept ? p : 0.f;
                    dpv = kept ? dpv : 0.f;
                }
                pk[r] = pkv;
                ds[r] = p * (dpv - dvec_s[buf][qi]);
            }

            // ---- dV^T += dO^T (keep*P) and dK^T += Q^T dS over the 32 rows.
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const frag_t<T> pf = pack8<T>(&pk[8 * cc]);
                const frag_t<T> sf = pack8<T>(&ds[8 * cc]);
                const int rbase = 32 * qb + 16 * cc;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    mma(dv_acc[db], load_frag_tr<T>(dos, LD, rbase, 32 * db), pf);
                    mma(dk_acc[db], load_frag_tr<T>(qs, LD, rbase, 32 * db), sf);
                }
            }
        }

        if (t + 1 < ntiles) store_rows(buf ^ 1);
        __syncthreads();
    }

    // ---- dK = scale c (dK/c)^T^T, dV = c dV^T^T.  Register r of block db is
    // column 32 db + 8(r/4) + 4g + r%4 of the lane's key row.
    const float vscale = DROPOUT ? a.drop_c : 1.f;
    const float kscale = DROPOUT ? a.scale * a.drop_c : a.scale;
    if (key < Nk) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float v0 = vscale * dv_acc[db][4 * rr], v1 = vscale * dv_acc[db][4 * rr + 1];
                const float v2 = vscale * dv_acc[db][4 * rr + 2], v3 = vscale * dv_acc[db][4 * rr + 3];
                const float s0 = kscale * dk_acc[db][4 * rr], s1 = kscale * dk_acc[db][4 * rr + 1];
                const float s2 = kscale * dk_acc[db][4 * rr + 2], s3 = kscale * dk_acc[db][4 * rr + 3];
                if (a.out_f32) {
                    store4<float>(reinterpret_cast<float *>(a.dv) + head_kv + key * D + col, v0, v1, v2, v3);
                    store4<float>(reinterpret_cast<float *>(a.dk) + head_kv + key * D + col, s0, s1, s2, s3);
                } else {
                    store4<T>(reinterpret_cast<T *>(a.dv) + head_kv + key * D + col, v0, v1, v2, v3);
                    store4<T>(reinterpret_cast<T *>(a.dk) + head_kv + key * D + col, s0, s1, s2, s3);
                }
            }
    }
}

// -------------------------------------------------------------------- dQ

template <typename T, int D>
struct DqTile {
    static_assert(sizeof(T) == 4, "generic dQ: fp32 inputs");
    static constexpr int NW = 4;
    static constexpr int THREADS = NW * kWave;
    static constexpr int BQ = 32 * NW;           // query rows per workgroup
    static constexpr int BC = 64;                // keys per LDS tile
    static constexpr int CH = 16 / sizeof(T);
    static constexpr int LD = D + CH;
    static constexpr int MIN_WG_PER_CU = 1;
};

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, (DqTile<T, D>::MIN_WG_PER_CU)) bwd_dq_kernel(const BwdArgs a) {
    using TL = DqTile<T, D>;
    constexpr int BQ = TL::BQ, BC = TL::BC, LD = TL::LD, THREADS = TL::THREADS;
    constexpr int NDC = D / 16, NDB = D / 32, NKB = BC / 32;

    __shared__ __attribute__((aligned(16))) T Ks[2][BC * LD];
    __shared__ __attribute__((aligned(16))) T Vs[2][BC * LD];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int lq = lane % 32, g = lane / 32;

    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)nqb, a.group);
    const int64_t bh = un.bh;
    const int64_t qb = CAUSAL ? (nqb - 1 - un.rank) : un.rank;
    const int64_t N = a.N, Nk = a.Nk;
    const int64_t off = Nk - N;                   // causal: query i sees keys j <= i + off
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head_kv;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int64_t q0 = qb * BQ;
    const int64_t qrow = q0 + wave * 32 + lq;

    // Q and dO rows of the lane's query: B operands of S^T and dP~^T.
    frag_t<T> qf[NDC], df[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
        if (qrow < N) {
            qf[c] = load_frag<T>(Qg + qrow * D + 16 * c + 8 * g);
            df[c] = load_frag<T>(dOg + qrow * D + 16 * c + 8 * g);
        } else {
            qf[c] = frag_t<T>{};
            df[c] = frag_t<T>{};
        }
    }
    const float lse_q = qrow < N ? a.lse[(size_t)bh * (size_t)N + qrow] : -__builtin_huge_valf();
    // rows past N and rows that see no key (LSE = -inf): P = exp2(-inf) = 0
    const float lse2 = lse_q != -__builtin_huge_valf() ? lse_q * kLog2e
                                : __builtin_huge_valf();
    const float dvec = qrow < N ? a.dvec[(size_t)bh * (size_t)N + qrow] : 0.f;

    int64_t kend = CAUSAL ? q0 + BQ + off : Nk;
    kend = kend < Nk ? kend : Nk;
    const int ntiles = kend > 0 ? (int)((kend + BC - 1) / BC) : 0;

    TileCopy<T, BC, D, THREADS> kcopy, vcopy;
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    kcopy.load(Kg, 0, Nk, tid);
    vcopy.load(Vg, 0, Nk, tid);
    kcopy.template store<LD>(Ks[0], tid);
    vcopy.template store<LD>(Vs[0], tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const T *ks = Ks[buf];
        const T *vs = Vs[buf];
        if (t + 1 < ntiles) {
            kcopy.load(Kg, (int64_t)(t + 1) * BC, Nk, tid);
            vcopy.load(Vg, (int64_t)(t + 1) * BC, Nk, tid);
        }
        const int64_t k0 = (int64_t)t * BC;
        const bool edge = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0 + off);

#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                mma(s, load_frag<T>(ks + (kb * 32 + lq) * LD + 16 * c + 8 * g), qf[c]);
                mma(dp, load_frag<T>(vs + (kb * 32 + lq) * LD + 16 * c + 8 * g), df[c]);
            }
            uint32_t keep = 0xFFFFu;
            if (DROPOUT)
                keep = keep_bits_row((uint32_t)(k0 + kb * 32), (uint32_t)qrow, h_idx, b_idx,
                                     a.seed_lo, a.seed_hi, a.drop_T);
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(s[r], a.scale_log2, -lse2));
                if (edge) {
                    const int64_t kk = k0 + kb * 32 + 8 * (r / 4) + 4 * g + (r % 4);
                    if (kk >= Nk || (CAUSAL && kk > qrow + off)) p = 0.f;
                }
                float dpv = dp[r];
                if (DROPOUT) dpv = ((keep >> r) & 1u) ? dpv : 0.f;
                ds[r] = p * (dpv - dvec);
            }
            // dQ^T += K^T dS^T; K^T fragments come from the row-major K tile.
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const frag_t<T> sf = pack8<T>(&ds[8 * cc]);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    mma(acc[db], load_frag_tr<T>(ks, LD, kb * 32 + 16 * cc, 32 * db), sf);
            }
        }

        if (t + 1 < ntiles) {
            kcopy.template store<LD>(Ks[buf ^ 1], tid);
            vcopy.template store<LD>(Vs[buf ^ 1], tid);
        }
        __syncthreads();
    }

    const float qscale = DROPOUT ? a.scale * a.drop_c : a.scale;
    if (qrow < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float x0 = qscale * acc[db][4 * rr + 0], x1 = qscale * acc[db][4 * rr + 1];
                const float x2 = qscale * acc[db][4 * rr + 2], x3 = qscale * acc[db][4 * rr + 3];
                if (a.out_f32) store4<float>(reinterpret_cast<float *>(a.dq) + head + qrow * D + col, x0, x1, x2, x3);
                else store4<T>(reinterpret_cast<T *>(a.dq) + head + qrow * D + col, x0, x1, x2, x3);
            }
    }
}

// ---------------------------------------------------------------- launch

template <typename T, int D>
static hipError_t launch_pre_t(const BwdArgs &a, hipStream_t stream) {
    const int64_t rows = a.B * a.H * a.N;
    dim3 grid((unsigned)((rows + 16 * kPreRows<D> - 1) / (16 * kPreRows<D>))), block(256);
    if (a.out_f32) hipLaunchKernelGGL((bwd_pre_kernel<T, float, D>), grid, block, 0, stream, a, rows);
    else hipLaunchKernelGGL((bwd_pre_kernel<T, T, D>), grid, block, 0, stream, a, rows);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dkdv_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = DkdvTile<T, D>;
    const int64_t nkb = (a.Nk + TL::BK - 1) / TL::BK;
    const int64_t units = a.B * a.H * nkb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    BwdArgs b = a;
    b.group = unit_group(a.B * a.H, nkb, 1);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, false>), grid, block, 0, stream, b);
    } else {
        if (dropout) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, false>), grid, block, 0, stream, b);
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dq_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = DqTile<T, D>;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    BwdArgs b = a;
    b.group = unit_group(a.B * a.H, nqb, TL::MIN_WG_PER_CU);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((bwd_dq_kernel<T, D, true, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((bwd_dq_kernel<T, D, true, false>), grid, block, 0, stream, b);
    } else {
        if (dropout) hipLaunchKernelGGL((bwd_dq_kernel<T, D, false, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((bwd_dq_kernel<T, D, false, false>), grid, block, 0, stream, b);
    }
    return hipGetLastError();
}

// Head dimensions: 32, 64, 96, 128 for every type; 256 for 16-bit types.
#define FA_DISPATCH_D(T, d, FN, ...)                   \
    switch (d) {                                       \
    case 32: return FN<T, 32>(__VA_ARGS__);            \
    case 64: return FN<T, 64>(__VA_ARGS__);            \
    case 96: return FN<T, 96>(__VA_ARGS__);            \
    case 128: return FN<T, 128>(__VA_ARGS__);          \
    }
#define FA_DISPATCH_ELEM_D(e, d, FN, ...)                                  \
    switch (e) {                                                           \
    case Elem::BF16:                                                       \
        if (d == 256) return FN<bf16, 256>(__VA_ARGS__);                   \
        FA_DISPATCH_D(bf16, d, FN, __VA_ARGS__)                            \
        break;                                                             \
    case Elem::F16:                                                        \
        if (d == 256) return FN<f16, 256>(__VA_ARGS__);                    \
        FA_DISPATCH_D(f16, d, FN, __VA_ARGS__)                             \
        break;                                                             \
    case Elem::F32:                                                        \
        FA_DISPATCH_D(float, d, FN, __VA_ARGS__)                           \
        break;                                                             \
    }                                                                      \
    return hipErrorInvalidValue;

hipError_t launch_bwd_pre(Elem e, int d, const BwdArgs &a, hipStream_t stream) {
    FA_DISPATCH_ELEM_D(e, d, launch_pre_t, a, stream)
}

// The generic dK/dV and dQ kernels serve fp32 inputs; 16-bit inputs take
// the kernels of fa_dkdv16.hip and fa_bwd16.hip (so no generic 16-bit
// instance is built).
#define FA_DISPATCH_GENERIC(e, d, FN, ...)                                 \
    if (e == Elem::F32) {                                                  \
        FA_DISPATCH_D(float, d, FN, __VA_ARGS__)                           \
    }                                                                      \
    return hipErrorInvalidValue;

hipError_t launch_bwd_dkdv(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                           hipStream_t stream) {
    if (e != Elem::F32) return launch_bwd_dkdv16(e, d, causal, dropout, a, stream);
    FA_DISPATCH_GENERIC(e, d, launch_dkdv_t, causal, dropout, a, stream)
}

hipError_t launch_bwd_dq(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                         hipStream_t stream) {
    if (e != Elem::F32) return launch_bwd_dq16(e, d, causal, dropout, a, stream);
    FA_DISPATCH_GENERIC(e, d, launch_dq_t, causal, dropout, a, stream)
}

// ---------------------------------------------------------- dropout probe

// keep mask of one (b, h) plane: thread -> (row, 8-column group).
__global__ void __launch_bounds__(256) dropout_mask_kernel(int64_t N, uint32_t T, uint32_t seed_lo,
                                                           uint32_t seed_hi, uint32_t b, uint32_t h,
                                                           uint8_t *mask) {
    const int64_t groups = (N + 7) / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * groups) return;
    const int64_t row = i / groups, grp = i % groups;
    const uint32_t bits = keep_byte((uint32_t)grp, (uint32_t)row, h, b, seed_lo, seed_hi, T);
    for (int e = 0; e < 8; ++e) {
        const int64_t col = grp * 8 + e;
        if (col < N) mask[row * N + col] = (uint8_t)((bits >> e) & 1u);
    }
}

hipError_t launch_dropout_mask(int64_t N, uint32_t T, uint32_t seed_lo, uint32_t seed_hi,
                               int64_t b, int64_t h, uint8_t *mask, hipStream_t stream) {
    const int64_t work = N * ((N + 7) / 8);
    const int64_t blocks = (work + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, N, T,
                       seed_lo, seed_hi, (uint32_t)b, (uint32_t)h, mask);
    return hipGetLastError();
}

}  // namespace fa
