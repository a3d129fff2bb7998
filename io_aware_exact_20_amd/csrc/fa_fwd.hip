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

#ifndef FA_FWD_KH0
#define FA_FWD_KH0 (2 * SB + SC)   // generator rounds over the second half of the PV products
#endif

#ifndef FA_FWD_PP
#define FA_FWD_PP 1   // d = 128, 16-bit: two wavefronts per SIMD in opposite phases
#endif

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
    static constexpr int MIN_WG_PER_CU = (sizeof(T) == 4 || D > 128) ? 1 : 2;
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
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int64_t qi = (u / BH) / a.kv_splits;
    const int split = (int)((u / BH) % a.kv_splits);
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
// that enter the product, so the output is a convex combination of V rows
// with exactly the weights used.
template <typename T, int D, int NW>
struct Fwd16Tile {
    static constexpr int RW = 64;                 // query rows per wavefront
    static constexpr int NB = RW / 32;            // 32-row blocks per wavefront
    static constexpr int BQ = NW * RW;            // query rows per workgroup
    static constexpr int BC = 32;                 // keys per tile
    static constexpr int THREADS = NW * kWave;
    static constexpr int TILE_BYTES = BC * D * 2;
    static constexpr int LOADS = TILE_BYTES / (kWave * 16) / NW;   // per wave per tile
};

// Threshold (log2 units) by which a tile's maximum must exceed the
// reference maximum before the accumulator is rescaled.
constexpr float kRescaleLog2 = 8.0f;

template <typename T, int D, int NW, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(NW * 64, 1) fwd16_kernel(const FwdArgs a) {
    using TL = Fwd16Tile<T, D, NW>;
    using SW = Swz<D>;
    constexpr int NB = TL::NB, BQ = TL::BQ, BC = TL::BC, RW = TL::RW;
    constexpr int TB = TL::TILE_BYTES, LOADS = TL::LOADS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;   // contraction chunks of S (K fragments per tile)
    constexpr int NDB = D / 32;   // 32-column blocks of O
    constexpr float kNegInf = -__builtin_huge_valf();
    static_assert(BC == 32 && NB == 2, "the step schedule below assumes 32-key tiles, 2 row blocks");

    // LDS: three K buffers (tile t in buffer t % 3) and two V buffers (t & 1).
    __shared__ __attribute__((aligned(1024))) char ks0[TB], ks1[TB], ks2[TB], vs0[TB], vs1[TB];

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lq = lane & 31, g = lane >> 5;

    // Work unit: (batch, head), query block, key chunk; causal query blocks
    // longest first.
    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int64_t qi = (u / BH) / a.kv_splits;
    const int split = (int)((u / BH) % a.kv_splits);
    const int64_t qb = CAUSAL ? (nqb - 1 - qi) : qi;
    const int N = (int)a.N, Nk = (int)a.Nk;
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Q = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ K = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ V = reinterpret_cast<const T *>(a.v) + head_kv;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int q0 = (int)qb * BQ;             // first query row of the workgroup
    const int q0w = q0 + wave * RW;           // first query row of this wavefront
    // Keys of this unit: [klo, khi); causal rows see keys up to row + off.
    const int klo = split * a.kv_chunk;
    const int khi = (int)((int64_t)klo + a.kv_chunk < (int64_t)Nk ? klo + a.kv_chunk : Nk);
    const int64_t off = (int64_t)Nk - N;

    // ---- Q fragments (B operand of S^T = K Q^T), rows clamped into range.
    frag_t<T> qf[NB][NDC];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        int r = q0w + 32 * nb + lq;
        r = r < N ? r : N - 1;
#pragma unroll
        for (int c = 0; c < NDC; ++c) qf[nb][c] = load_frag<T>(Q + (size_t)r * D + 16 * c + 8 * g);
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
    // ---- direct tile loads: wave-instruction i of this wave fills tile rows
    // R0 + i * RSTEP (R0 = first row of instruction 0 for this lane).  The
    // swizzle repeats every 16 rows, so the lane's swizzled column takes
    // NPAT values over i.  Loads go through buffer resources bounded by the
    // head's end, so the rows of the last tile past N arrive as zeros
    // (masked scores, zero values).
    constexpr int RSTEP = NW * kWave / SW::CPR;
    constexpr int NPAT = RSTEP % 16 == 0 ? 1 : 16 / RSTEP;
    static_assert(16 % RSTEP == 0 || RSTEP % 16 == 0, "tile rows per load instruction");
    const int R0 = (wave * kWave + lane) / SW::CPR;
    uint32_t lane_boffs[NPAT];
#pragma unroll
    for (int i = 0; i < NPAT; ++i)
        lane_boffs[i] = ((uint32_t)R0 * D + (uint32_t)(((lane % SW::CPR) ^ (int)SW::f(R0 + i * RSTEP)) * 8)) * 2;
    const uint32_t head_bytes = (uint32_t)Nk * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, head_bytes), vrs = make_rsrc(V, head_bytes);

    // Tiles (of BC keys from klo) the workgroup streams, and the ones this
    // wavefront needs (causal: up to its own last row).
    auto tiles_to = [&](int64_t end) {
        end = end < khi ? end : khi;
        return end > klo ? (int)((end - klo + BC - 1) / BC) : 0;
    };
    const int NT = tiles_to(CAUSAL ? (int64_t)q0 + BQ + off : (int64_t)Nk);
    const int Tw = tiles_to(CAUSAL ? (int64_t)q0w + RW + off : (int64_t)Nk);

    // Load i of this wave's share of tile t of K (or V) into a buffer.
    auto load_part = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf_lds, int i) {
        buf2lds16(rs, lane_boffs[i % NPAT], (uint32_t)((klo + t * BC + i * RSTEP) * D * 2),
                  buf_lds + (wave + i * NW) * (kWave * 16));
    };
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf_lds) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) load_part(rs, t, buf_lds, i);
    };
    auto kbuf = [&](int buf) {
        return buf == 0 ? (lds_char *)ks0 : buf == 1 ? (lds_char *)ks1 : (lds_char *)ks2;
    };
    auto vbuf = [&](int buf) { return buf ? (lds_char *)vs1 : (lds_char *)vs0; };

    // A tile needs masking if it reaches past the last key or, causal, past
    // what this wavefront's first query row sees.
    auto is_edge = [&](int t) {
        const int64_t k0 = (int64_t)klo + t * BC;
        return (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w + off);
    };
    // Scores of tile t set to -inf where the key is masked for the query.
    auto apply_mask = [&](f32x16 (&s)[NB], int t) {
        const int k0 = klo + t * BC;
        // Register r of block nb holds key k0 + 4g + kk(r) for query
        // q0w + 32nb + lq, kk(r) = 8(r/4) + r%4.  Masked: key >= Nk, or
        // (causal) key > query + off, i.e. kk(r) > lim[nb].
        int lim[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            int l = Nk - 1 - (k0 + 4 * g);
            if (CAUSAL) {
                const int64_t c = (int64_t)q0w + 32 * nb + lq + off - (k0 + 4 * g);
                l = c < l ? (int)(c > -64 ? c : -64) : l;
            }
            lim[nb] = l;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r / 4) + (r % 4);
                if (kk > lim[nb]) s[nb][r] = kNegInf;
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
        for (int db = 0; db < NDB; ++db) o[db][nb] = f32x16{};
    }

    // ---- building blocks.
    // Keep decisions of tile t for score block nb, in the sign layout of
    // keep_signs_from_blocks (pair i of the block in bits 15 - i, 31 - i).
    const uint32_t kc2 = keep_cmp_const(a.drop_T);
    auto draw_keep = [&](uint32_t (&keep)[NB], int t) {
        const uint32_t grp = (uint32_t)((klo + t * BC) >> 3) + 2 * (uint32_t)g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t row = (uint32_t)(q0w + 32 * nb + lq);
            const Philox4 b0 = philox4x32_10(grp, row, h_idx, b_idx, a.seed_lo, a.seed_hi);
            const Philox4 b1 = philox4x32_10(grp + 1, row, h_idx, b_idx, a.seed_lo, a.seed_hi);
            keep[nb] = keep_signs_from_blocks(b0, b1, kc2);
        }
    };
    // The same draw split into its 40 generator rounds (four blocks of ten),
    // so that the rounds of tile t+1 can ride between the products of step t.
    struct KeepDraw { Philox4 c[2 * NB]; };
    auto keep_begin = [&](KeepDraw &k, int t) {
        const uint32_t grp = (uint32_t)((klo + t * BC) >> 3) + 2 * (uint32_t)g;
#pragma unroll
        for (int s = 0; s < 2 * NB; ++s) {
            k.c[s].x[0] = grp + (s & 1);
            k.c[s].x[1] = (uint32_t)(q0w + 32 * (s >> 1) + lq);
            k.c[s].x[2] = h_idx;
            k.c[s].x[3] = b_idx;
        }
    };
    auto keep_rounds = [&](KeepDraw &k, int u0, int u1) {
#pragma unroll
        for (int u = u0; u < u1; ++u) philox_round(k.c[u % (2 * NB)], u / (2 * NB), a.seed_lo, a.seed_hi);
        if (u1 > u0) {
#pragma unroll
            for (int s = 0; s < 2 * NB; ++s)
#pragma unroll
                for (int q = 0; q < 4; ++q) pin_vgpr(k.c[s].x[q]);
        }
    };
    // Move the reference maxima when a tile exceeds them by the threshold.
    auto maybe_rescale = [&](const float (&mx)[NB]) {
        bool need = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) need |= mx[nb] * sl2 > m_run[nb] + kRescaleLog2;
        if (__builtin_expect(__ballot(need) != 0, 0)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float m_new = fmaxf(m_run[nb], max_halves(mx[nb]) * sl2);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run[nb] - m_new);
                l_run[nb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db][nb] *= alpha;
                m_run[nb] = m_new;
            }
        }
    };

    // One pipelined step for tile t (scores sc, maxima mx).  Matrix-core
    // work: S of tile t+1 (NDC K fragments x 2 products, from K buffer
    // (t+1)&1) and O^T += V^T P^T of tile t (2 NDB V fragments x 2 products,
    // V buffer t&1).  The VALU work -- tile t's 16 probability pairs and row
    // sums, tile t+1's maxima -- is spread over the products so that no gap
    // between two products holds more than about four VALU instructions (a
    // single wavefront co-issues that many with a 32x32x16 product; more
    // stall the matrix core).  The next tiles' loads are spread over the
    // same groups.  LDS fragments are read two groups ahead of their use.
    //   B (S of t+1):  pairs 0..11 (key chunk 0 complete, chunk 1 half);
    //   C (PV of t):   pairs 12..15 in the first half (before chunk 1's
    //                  products), row sums and the maxima of tile t+1.
    constexpr int SB = NDC;                  // K fragment groups (2 products each)
    constexpr int SC = 2 * NDB;              // V fragment groups (2 products each)
    static_assert(SB == 8 || SB == 4, "group plan for d = 128 or 64");
    constexpr int PB = 10;                   // pairs computed in B
    constexpr int PC = 16 - PB;              // pairs computed in C
    static_assert(PB >= 8, "chunk 0's pairs must be complete before C's first product");
    // Half-groups that carry the generator rounds of the next tile's keep
    // decisions (NKR rounds in all).
    constexpr int NKR = 10 * 2 * NB;
    constexpr int KH0 = FA_FWD_KH0, KH1 = 2 * SB + 2 * SC;
    uint32_t keep_cur[NB];
    // kp: the first two K fragments of tile t+1, read during the previous
    // step (K tiles are loaded three steps ahead, so tile t+1 is complete
    // before step t begins and its buffer is not refilled before step t+1).
    auto step = [&](auto kb_c, auto par_c, f32x16 (&sc)[NB], f32x16 (&sn)[NB], float (&mx)[NB],
                    frag_t<T> (&kp)[2], int t) {
        constexpr int KB = decltype(kb_c)::value;   // K buffer of tile t+1: (t+1) % 3
        constexpr int VB = decltype(par_c)::value;  // V buffer of tile t: t & 1
        constexpr bool HN = true;
        const lds_char *kbl = KB == 0 ? (lds_char *)ks0 : KB == 1 ? (lds_char *)ks1 : (lds_char *)ks2;
        constexpr int KQ = (KB + 1) % 3;            // K buffer of tile t+2
        const lds_char *kql = KQ == 0 ? (lds_char *)ks0 : KQ == 1 ? (lds_char *)ks1 : (lds_char *)ks2;
        constexpr int KL = (KB + 2) % 3;            // K buffer refilled with tile t+3: t % 3
        const lds_char *vbl = VB ? (lds_char *)vs1 : (lds_char *)vs0;

        maybe_rescale(mx);
        float mu[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mu[nb] = m_run[nb] == kNegInf ? 0.f : m_run[nb];
        if (HN) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sn[nb] = f32x16{};
        }

        auto kfrag = [&](int j) { return lds_frag<T>(kbl + koff[j]); };
        auto vfrag = [&](int j) {
            const int cc = j / NDB, db = j % NDB;
            const uint32_t kc_off = (uint32_t)(16 * cc * RB);
            return join<T>(lds_half_tr<T>(vbl + kc_off + voff[0][db]),
                           lds_half_tr<T>(vbl + kc_off + voff[1][db]));
        };
        uint32_t pp[NB][8];
        auto pfrag = [&](int nb, int cc) {
            u32x4 pv;
            pv[0] = pp[nb][4 * cc + 0];
            pv[1] = pp[nb][4 * cc + 1];
            pv[2] = pp[nb][4 * cc + 2];
            pv[3] = pp[nb][4 * cc + 3];
            return __builtin_bit_cast(frag_t<T>, pv);
        };
        float acc[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) { acc[nb][0] = 0.f; acc[nb][1] = 0.f; }
        // Keep decisions of tile t+1: the 40 generator rounds are spread over
        // the half-groups [KH0, KH1) of this step (B: 0 .. 2 SB - 1, C: 2 SB
        // .. 2 SB + 2 SC - 1).
        KeepDraw kd;
        if (DROPOUT) keep_begin(kd, t + 1);
        auto spread = [&](int hg) {
            if (DROPOUT && hg >= KH0 && hg < KH1)
                keep_rounds(kd, (NKR * (hg - KH0)) / (KH1 - KH0), (NKR * (hg - KH0 + 1)) / (KH1 - KH0));
        };
        // Pair p = (row block p & 1, registers 2i, 2i+1 with i = p >> 1).
        auto pair = [&](int p) {
            const int nb = p & 1, i = p >> 1;
            const float p0 = fast_exp2(fmaf(sc[nb][2 * i], sl2, -mu[nb]));
            const float p1 = fast_exp2(fmaf(sc[nb][2 * i + 1], sl2, -mu[nb]));
            pp[nb][i] = pack2<T>(p0, p1);
            // Row sums of the fp32 probabilities (dropped ones included):
            // two adds that co-issue with the products and need no
            // registers beyond p0, p1.
            acc[nb][i & 1] = (acc[nb][i & 1] + p0) + p1;
            if (DROPOUT) {
                // decisions of the pair in the sign bits of the two halves
                const i16x2 sg = __builtin_bit_cast(i16x2, keep_cur[nb] << i);
                pp[nb][i] &= __builtin_bit_cast(uint32_t, sg >> (i16x2){15, 15});
            }
            pin_vgpr(pp[nb][i]);   // keeps the work in its group (no sinking)
        };
        float mxp[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mxp[nb] = kNegInf;
        auto maxpair = [&](int w) {   // registers 2w, 2w+1 (of 16) of both row blocks
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                mxp[nb] = fmaxf(mxp[nb], fmaxf(sn[nb][2 * w], sn[nb][2 * w + 1]));
        };

        // ---- B: S of tile t+1 | pairs 0..11 | K loads of tile t+3, V loads of t+1.
        frag_t<T> kf[3], vf[3];
        kf[0] = kp[0];
        kf[1] = kp[1];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            // Half-group 2j: product with row block 0, then its share of the
            // PB pairs (spread over the 2 SB products in order).
            if (HN) {
                if (j + 2 < SB) kf[(j + 2) % 3] = kfrag(j + 2);
                mma(sn[0], kf[j % 3], qf[0][j]);
            }
#pragma unroll
            for (int p = (2 * j * PB) / (2 * SB); p < ((2 * j + 1) * PB) / (2 * SB); ++p) pair(p);
            spread(2 * j);
            __builtin_amdgcn_sched_barrier(0);
            // Half-group 2j+1: row block 1.
            if (HN) mma(sn[1], kf[j % 3], qf[1][j]);
#pragma unroll
            for (int p = ((2 * j + 1) * PB) / (2 * SB); p < ((2 * j + 2) * PB) / (2 * SB); ++p) pair(p);
            spread(2 * j + 1);
            if (j < LOADS) load_part(krs, t + 3, kbuf(KL), j);
            if (j >= LOADS && j < 2 * LOADS) load_part(vrs, t + 1, vbuf(VB ^ 1), j - LOADS);
            if (j == SB - 2) vf[0] = vfrag(0);
            if (j == SB - 1) vf[1] = vfrag(1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (HN && is_edge(t + 1)) apply_mask(sn, t + 1);

        // ---- C: PV of tile t | pairs 12..15, row sums, maxima of t+1.
        // Work of half-group k (one product each, k = 0 .. 2 SC - 1): pairs
        // 12..15 over the first SC halves (before chunk 1's products), the
        // 16 row sums and the 8 maxima spread over all of them.
        auto cwork = [&](int k) {
            if (k < SC) {
#pragma unroll
                for (int p = PB + (k * PC) / SC; p < PB + ((k + 1) * PC) / SC; ++p) pair(p);
            }
            if (HN) {
#pragma unroll
                for (int w = (k * 8) / (2 * SC); w < ((k + 1) * 8) / (2 * SC); ++w) maxpair(w);
            }
        };
#pragma unroll
        for (int j = 0; j < SC; ++j) {
            if (j + 2 < SC) vf[(j + 2) % 3] = vfrag(j + 2);
            const int cc = j / NDB, db = j % NDB;
            mma(o[db][0], vf[j % 3], pfrag(0, cc));
            cwork(2 * j);
            spread(2 * SB + 2 * j);
            __builtin_amdgcn_sched_barrier(0);
            mma(o[db][1], vf[j % 3], pfrag(1, cc));
            cwork(2 * j + 1);
            spread(2 * SB + 2 * j + 1);
            if (j == SC - 2) kp[0] = lds_frag<T>(kql + koff[0]);
            if (j == SC - 1) kp[1] = lds_frag<T>(kql + koff[1]);
            if (j == SC - 1) {
                // Keep the row sums and maxima in this group (no sinking).
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    pin_vgpr(acc[nb][0]);
                    pin_vgpr(acc[nb][1]);
                    if (HN) pin_vgpr(mxp[nb]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) l_run[nb] += acc[nb][0] + acc[nb][1];
        if (HN) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) mx[nb] = mxp[nb];
            if (DROPOUT) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    keep_cur[nb] = keep_signs_from_blocks(kd.c[2 * nb], kd.c[2 * nb + 1], kc2);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of K_{t+3}, V_{t+1} landed
        __syncthreads();                 // ... everyone's; buffers of K_{t+1}, V_t free
    };

    // ---- prologue: K_0, K_1, K_2, V_0; S and maxima of tile 0.
    f32x16 sA[NB], sB[NB];
    float mx[NB];
    frag_t<T> kp[2];
    load_tile(krs, 0, kbuf(0));
    load_tile(krs, 1, kbuf(1));
    load_tile(krs, 2, kbuf(2));
    load_tile(vrs, 0, vbuf(0));
    // Q into AGPRs once all loads are in flight (a pin waits for its load).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int c = 0; c < NDC; ++c) pin_agpr(qf[nb][c]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (Tw > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sA[nb] = f32x16{};
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            const frag_t<T> kf = lds_frag<T>(kbuf(0) + koff[c]);
            mma(sA[0], kf, qf[0][c]);
            mma(sA[1], kf, qf[1][c]);
        }
        if (is_edge(0)) apply_mask(sA, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float x = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; r += 2) x = fmaxf(x, fmaxf(sA[nb][r], sA[nb][r + 1]));
            mx[nb] = x;
        }
        if (DROPOUT) draw_keep(keep_cur, 0);
    }
    kp[0] = lds_frag<T>((lds_char *)ks1 + koff[0]);
    kp[1] = lds_frag<T>((lds_char *)ks1 + koff[1]);
    __syncthreads();   // K buffer 0 is refilled in the first step

    // ---- steady state, six steps per trip (buffer indices are constants).
    // The last step also forms S of tile Tw (never used: masked or
    // zero-filled keys), so every step has one shape and the accumulators
    // keep their registers across the loop exit.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int t = 0; t < Tw; t += 6) {
        step(I1{}, I0{}, sA, sB, mx, kp, t);
        if (t + 1 < Tw) step(I2{}, I1{}, sB, sA, mx, kp, t + 1);
        if (t + 2 < Tw) step(I0{}, I0{}, sA, sB, mx, kp, t + 2);
        if (t + 3 < Tw) step(I1{}, I1{}, sB, sA, mx, kp, t + 3);
        if (t + 4 < Tw) step(I2{}, I0{}, sA, sB, mx, kp, t + 4);
        if (t + 5 < Tw) step(I0{}, I1{}, sB, sA, mx, kp, t + 5);
    }
    int t = Tw > 0 ? Tw : 0;
    // Tiles beyond this wavefront's rows: keep the workgroup's loads and
    // barriers in step.
    for (; t < NT; ++t) {
        load_tile(krs, t + 3, kbuf(t % 3));
        load_tile(vrs, t + 1, vbuf((t + 1) & 1));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: O = c * acc / l, LSE = (m + log2 l) ln 2 -- of the
    // chunk, in fp32 to the partial buffers, when the keys are split.
    const bool part = a.kv_splits > 1;
    const size_t prow = ((size_t)split * (size_t)BH + (size_t)bh) * (size_t)N;
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
                    if (part) {
                        store4<float>(a.part_o + (prow + qrow) * D + col, x0, x1, x2, x3);
                    } else if (a.out_f32) {
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
                if (part) a.part_lse[prow + qrow] = lse;
                else a.lse[(size_t)bh * (size_t)N + qrow] = lse;
            }
        }
    }
}

template <typename T, int D, int NW>
static hipError_t launch_fwd16_t(bool causal, bool dropout, const FwdArgs &a, hipStream_t stream) {
    using TL = Fwd16Tile<T, D, NW>;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb * a.kv_splits;
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
    const int64_t units = a.B * a.H * nqb * a.kv_splits;
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
    // 16-bit inputs: d = 64 and 128 take the two-wavefronts-per-SIMD kernel
    // (fa_fwd_pp.hip; the 64-rows-per-wavefront kernel when built with
    // FA_FWD_PP=0); every other case the generic one (32 rows per wavefront).
    switch (e) {
    case Elem::BF16:
        switch (d) {
        case 32: return launch_fwd_t<bf16, 32>(causal, dropout, a, stream);
        case 64:
            if (FA_FWD_PP) return launch_fwd_pp(e, d, causal, dropout, a, stream);
            return launch_fwd16_t<bf16, 64, FA_FWD_NW>(causal, dropout, a, stream);
        case 96: return launch_fwd_t<bf16, 96>(causal, dropout, a, stream);
        case 128:
            if (FA_FWD_PP) return launch_fwd_pp(e, d, causal, dropout, a, stream);
            return launch_fwd16_t<bf16, 128, FA_FWD_NW>(causal, dropout, a, stream);
        case 256: return launch_fwd_t<bf16, 256>(causal, dropout, a, stream);
        }
        break;
    case Elem::F16:
        switch (d) {
        case 32: return launch_fwd_t<f16, 32>(causal, dropout, a, stream);
        case 64:
            if (FA_FWD_PP) return launch_fwd_pp(e, d, causal, dropout, a, stream);
            return launch_fwd16_t<f16, 64, FA_FWD_NW>(causal, dropout, a, stream);
        case 96: return launch_fwd_t<f16, 96>(causal, dropout, a, stream);
        case 128:
            if (FA_FWD_PP) return launch_fwd_pp(e, d, causal, dropout, a, stream);
            return launch_fwd16_t<f16, 128, FA_FWD_NW>(causal, dropout, a, stream);
        case 256: return launch_fwd_t<f16, 256>(causal, dropout, a, stream);
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
