// Forward of fused exact attention for 16-bit inputs at d = 32, 64, 96, 128
// and 256 on gfx950, with two wavefronts per SIMD (one at d = 256).
//
// The method is the one of the other forward kernels: Q, K, V tiled into
// on-chip blocks, the online-softmax recurrence (running row maximum,
// normaliser, rescaled output accumulator) over key tiles, and only O and
// the per-row log-sum-exp written back ("Tiling" and "Recomputation",
// mrodiduger.github.io page; steps 1-4 of "Architecture, step by step",
// interviewsvector.com page).
//
// Schedule.  Each wavefront owns 32 query rows; K and V tiles are shared
// through LDS.  A step of a wavefront has a matrix phase -- S of the next
// tile (S^T = K Q^T) and O^T += V^T P^T of the current one, eight 32x32x16
// products each per 32 keys -- and a vector phase -- masking, row maxima,
// the lazy rescale, exponentials, row sums, rounding and dropout of the
// next tile's scores.  Two wavefronts share every SIMD, so that one keeps
// the matrix core busy while the other does its softmax arithmetic on the
// vector ALU (the overlap of softmax with the matrix products that the
// flash-attention-4 page describes, applied to wavefronts sharing a SIMD;
// within one wavefront a product hides only a few vector instructions).
// A workgroup has four wavefronts (128 rows) and two workgroups share a CU,
// so the two wavefronts of a SIMD come from different workgroups and one
// runs while the other waits at its step barrier.  Steps cover 64 keys
// without dropout and 32 keys with it (d = 32 and 96: 64 keys also with
// dropout).  The translation unit is compiled with matrix-core results in
// VGPRs: Q, the output accumulator and the scores all sit in VGPRs (at
// d = 128 202-213 of a wavefront's 256), so the vector phase reads the
// scores without a copy out of AGPRs.
//
// At d = 256 the output accumulator (128 registers) and Q (64) leave no room
// for a second wavefront per SIMD: one workgroup per CU, one wavefront per
// SIMD, 32-key steps.  There each softmax element costs twice the matrix
// work of d = 128, so the vector phase is short against the products of
// its own wavefront.

// Layout of the products: scores are
// formed transposed, S^T = K Q^T, so a lane owns one query row and sixteen
// keys of a tile; the rounded scores are directly the B operand of
// O^T += V^T P^T; V^T comes from the row-major LDS tile through
// ds_read_b64_tr_b16.  Tiles reach LDS by direct buffer loads (XOR-swizzled
// 16-byte chunks, zeros past the last key).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <typename T, int D, bool DROPOUT>
struct FwdPPTile {
    // Four wavefronts and two workgroups per CU: the two wavefronts of a SIMD
    // come from different workgroups, so one workgroup's wavefronts run while
    // the other's wait at their step barrier (measured faster than eight
    // wavefronts of one workgroup in opposite phases at every size: 9 % with
    // dropout, 1-2 % without).
    static constexpr int NW = 4;
    static constexpr int WG_PER_CU = D == 256 ? 1 : 2;
    static constexpr int BQ = 32 * NW;                    // query rows per workgroup
    // 32-key blocks per tile: two without dropout (one barrier per 64 keys);
    // one with it (two measured no faster there and need the vector phase
    // inlined by force to stay out of scratch memory).
    // (d = 96 and 32: always two, a 32-key tile being six or two load
    // instructions for four wavefronts)
    static constexpr int NKB = (D == 96 || D == 32) ? 2 : (DROPOUT || D == 256) ? 1 : 2;
    // K and V buffers each (two workgroups share the LDS); tiles are loaded
    // one step ahead.
    static constexpr int NBUF = 2;
    static constexpr int BC = 32 * NKB;                   // keys per tile
    static constexpr int THREADS = NW * kWave;
    static constexpr int TILE_BYTES = BC * D * 2;         // one K or V tile
    static constexpr int CHUNK_BYTES = kWave * 16;        // one wavefront load instruction
    static constexpr int CHUNKS = TILE_BYTES / CHUNK_BYTES;   // per tile
    static constexpr int LOADS = 2 * CHUNKS / NW;         // per wavefront per step (K and V)
};

// Launch bounds (single template arguments: the attribute macro splits at commas).
constexpr int kPPThreads = FwdPPTile<bf16, 128, false>::THREADS;
template <int D>
constexpr int kPPWgPerCu = D == 256 ? 1 : 2;
static_assert(kPPWgPerCu<128> == FwdPPTile<bf16, 128, false>::WG_PER_CU &&
                  kPPWgPerCu<256> == FwdPPTile<bf16, 256, false>::WG_PER_CU, "launch bounds");

// Lazy-rescale threshold (log2 units), as in the other forward kernels.
constexpr float kPPRescaleLog2 = 8.0f;

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(kPPThreads, kPPWgPerCu<D>) fwd_pp_kernel(const FwdArgs a) {
    using TL = FwdPPTile<T, D, DROPOUT>;
    using SW = Swz<D>;
    constexpr int BQ = TL::BQ, BC = TL::BC, NW = TL::NW, NKB = TL::NKB, NBUF = TL::NBUF;
    constexpr int TB = TL::TILE_BYTES, CB = TL::CHUNK_BYTES, CHUNKS = TL::CHUNKS, LOADS = TL::LOADS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;       // contraction chunks of S
    constexpr int NDB = D / 32;       // 32-column blocks of O
    constexpr float kNegInf = -__builtin_huge_valf();
    static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "tile plan for d = 32 ... 256");
    static_assert(2 * NDB == NDC, "one V^T product per K product");

    // LDS: K tile t in buffer t % 2, V tile t in buffer t % 2.
    __shared__ __attribute__((aligned(1024))) char ks0[TB], ks1[TB], vs0[TB], vs1[TB];
    static_assert(NBUF == 2, "two K and two V buffers");

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lq = lane & 31, g = lane >> 5;

    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)(nqb * a.kv_splits), a.group);
    const int64_t bh = un.bh;
    const int64_t qi = un.rank / (uint32_t)a.kv_splits;
    const int split = (int)(un.rank % (uint32_t)a.kv_splits);
    const int64_t qb = CAUSAL ? (nqb - 1 - qi) : qi;
    const int N = (int)a.N, Nk = (int)a.Nk;
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Q = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ K = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ V = reinterpret_cast<const T *>(a.v) + head_kv;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int q0 = (int)qb * BQ;
    const int q0w = q0 + 32 * wave;                    // first query row of this wavefront
    const int qrow = q0w + lq;                         // this lane's query row
    const int klo = split * a.kv_chunk;
    const int khi = (int)((int64_t)klo + a.kv_chunk < (int64_t)Nk ? klo + a.kv_chunk : Nk);
    const int64_t off = (int64_t)Nk - N;

    // Q fragments (B operand of S^T = K Q^T), rows clamped into range.
    frag_t<T> qf[NDC];
    {
        const int r = qrow < N ? qrow : N - 1;
#pragma unroll
        for (int c = 0; c < NDC; ++c) qf[c] = load_frag<T>(Q + (size_t)r * D + 16 * c + 8 * g);
    }

    // LDS read offsets: K fragments along a key row; V^T by transposed reads.
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

    // Tile loads.  A tile is CHUNKS load instructions of 1 KB; this
    // wavefront issues chunks c = wave + i NW (i < LPT) of both the K and the
    // V tile of a step.  Lane l of chunk c fills 16-byte position p = 64 c + l
    // of the tile (row p / CPR, position p % CPR: rows need not align with
    // chunks, d = 96) with the logical chunk the swizzle places there.
    constexpr int LPT = CHUNKS / NW;   // chunks per tile per wavefront
    static_assert(LPT * NW == CHUNKS && 2 * LPT == LOADS, "load split");
    uint32_t lboff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        if constexpr ((CB / 16) % SW::CPR == 0) {   // whole rows per chunk
            const int r = CB / RB * (wave + i * NW) + lane / SW::CPR;
            lboff[i] = ((uint32_t)r * D + (uint32_t)(((lane % SW::CPR) ^ (int)SW::f((uint32_t)r)) * 8)) * 2;
        } else {
            const int pos = (wave + i * NW) * (CB / 16) + lane;
            const int r = pos / SW::CPR;
            lboff[i] = ((uint32_t)r * D + (uint32_t)(((pos % SW::CPR) ^ (int)SW::f((uint32_t)r)) * 8)) * 2;
        }
    }
    const uint32_t head_bytes = (uint32_t)Nk * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, head_bytes), vrs = make_rsrc(V, head_bytes);
    // Buffers by tile index mod 3 (compile-time wherever tiles are read, so
    // that the compiler can tell the loads into one buffer from reads of
    // another).
    auto kbuf = [&](int m) { return m == 0 ? (lds_char *)ks0 : (lds_char *)ks1; };
    auto vbuf = [&](int m) { return m == 0 ? (lds_char *)vs0 : (lds_char *)vs1; };
    // This wavefront's share of the loads of K tile tk and V tile tv into
    // K buffer kbm and V buffer vbm.
    auto load_kv = [&](int tk, int kbm, int tv, int vbm) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int c = wave + i * NW;
            // (byte offsets of up to 2^31 + 3 tiles: unsigned arithmetic)
            buf2lds16(krs, lboff[i], (uint32_t)(klo + tk * BC) * (uint32_t)(D * 2), kbuf(kbm) + c * CB);
            buf2lds16(vrs, lboff[i], (uint32_t)(klo + tv * BC) * (uint32_t)(D * 2), vbuf(vbm) + c * CB);
        }
    };

    auto tiles_to = [&](int64_t end) {
        end = end < khi ? end : khi;
        return end > klo ? (int)((end - klo + BC - 1) / BC) : 0;
    };
    const int NT = tiles_to(CAUSAL ? (int64_t)q0 + BQ + off : (int64_t)Nk);   // workgroup
    // Tiles this wavefront works on (none when all its rows are past the
    // last query, e.g. the tail of a short decoding block).
    const int Tw = q0w < N ? tiles_to(CAUSAL ? (int64_t)q0w + 32 + off : (int64_t)Nk) : 0;

    // Tile t needs masking if it reaches past the last key or, causal, past
    // what the wavefront's first row sees.
    auto is_edge = [&](int t) {
        const int64_t k0 = (int64_t)klo + t * BC;
        return (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > q0w + off);
    };
    // Register r of key block kb holds key k0 + 4g + kk(r), k0 = first key
    // of the block, kk(r) = 8(r/4) + r%4, for query row qrow; masked: key >=
    // Nk, or (causal) key > qrow + off.
    auto apply_mask = [&](f32x16 &s, int t, int kb) {
        const int k0 = klo + t * BC + 32 * kb;
        int lim = Nk - 1 - (k0 + 4 * g);
        if (CAUSAL) {
            const int64_t c = (int64_t)qrow + off - (k0 + 4 * g);
            lim = c < lim ? (int)(c > -64 ? c : -64) : lim;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r / 4) + (r % 4);
            if (kk > lim) s[r] = kNegInf;
        }
    };

    const float sl2 = a.scale_log2;
    const uint32_t kc2 = keep_cmp_const(a.drop_T);
    float m_run = kNegInf;   // running row maximum (log2 units of scaled scores)
    float l_run = 0.f;       // running normaliser, this lane's half of the keys
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    f32x16 s[NKB];           // scores of the tile the vector phase works on next
    uint32_t pp[8 * NKB];    // rounded (kept) probabilities of the tile the matrix phase multiplies

    // Keep-bit draw of a tile (two Philox blocks per 32-key block, see
    // keep_masks_from_blocks).  With eight or more product pairs per matrix
    // phase (d >= 96) it is staged: counters, then the block-rounds spread
    // over the products of the matrix phase before the tile's vector phase
    // (where a wavefront's own products hide a few vector instructions
    // each), then the masks in the vector phase (d = 256 3 %, non-causal
    // d = 128 3.5 % faster; neutral on causal d = 128).  With four (d = 32,
    // 64) the rounds would crowd the products (measured 3 % slower), and the
    // whole draw stays in the vector phase.
    constexpr int NB2 = 2 * NKB, KU = 10 * NB2;   // blocks; block-rounds
    constexpr bool STAGED = DROPOUT && NKB * NDC >= 8;
    Philox4 kd[NB2];
    auto keep_begin = [&](int t) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const uint32_t grp = (uint32_t)((klo + t * BC + 32 * kb) >> 3) + 2 * (uint32_t)g;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                kd[2 * kb + h].x[0] = grp + h;
                kd[2 * kb + h].x[1] = (uint32_t)qrow;
                kd[2 * kb + h].x[2] = h_idx;
                kd[2 * kb + h].x[3] = b_idx;
            }
        }
    };
    // block-rounds u0 .. u1-1: unit u is round u / NB2 of block u % NB2
    auto keep_rounds = [&](int u0, int u1) {
#pragma unroll
        for (int u = u0; u < u1; ++u) philox_round<true>(kd[u % NB2], u / NB2, a.seed_lo, a.seed_hi);
        if (u1 > u0) {
#pragma unroll
            for (int h = 0; h < NB2; ++h)
                // not after a block's first generator round: two of its words are then
                // loop-invariant, and a pin would copy them into every
                // block's registers (0.5-1.3 % slower forward)
                if ((u1 + NB2 - 1 - h) / NB2 >= 2)
#pragma unroll
                    for (int q = 0; q < 4; ++q) pin_vgpr(kd[h].x[q]);
        }
    };

    // Vector phase for tile t: scores s -> probabilities pp.
    auto vec_phase = [&](int t) __attribute__((always_inline)) {
        if (is_edge(t)) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) apply_mask(s[kb], t, kb);
        }
        // Keep masks of each 32-key block's probability pairs, from the
        // finished draw of tile t.
        uint32_t keep_m[NKB][8];
        if (DROPOUT && !STAGED) {
            keep_begin(t);
            keep_rounds(0, KU);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            if (DROPOUT) keep_masks_from_blocks(kd[2 * kb], kd[2 * kb + 1], kc2, keep_m[kb]);
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
        // Move the reference maximum when the tile exceeds it by the threshold.
        if (__builtin_expect(__ballot(mx * sl2 > m_run + kPPRescaleLog2) != 0, 0)) {
            const float m_new = fmaxf(m_run, max_halves(mx) * sl2);
            const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            m_run = m_new;
        }
        const float mu = m_run == kNegInf ? 0.f : m_run;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = fast_exp2(fmaf(s[kb][2 * i], sl2, -mu));
                const float p1 = fast_exp2(fmaf(s[kb][2 * i + 1], sl2, -mu));
                // row sums keep the dropped probabilities
                if (i & 1) acc1 = (acc1 + p0) + p1;
                else acc0 = (acc0 + p0) + p1;
                uint32_t w = pack2<T>(p0, p1);
                if (DROPOUT) w &= keep_m[kb][i];
                pp[8 * kb + i] = w;
            }
        }
        l_run += acc0 + acc1;
    };

    // Matrix phase of tile t (M = t % NBUF): O^T += V^T P^T (V_t, pp) and S of
    // tile t + 1 (K_{t+1}) into s.  The last tile's phase also forms the
    // scores of the tile after it, which are never used: every phase has one
    // shape.  The S chain and the O products alternate, so no product waits
    // for the one just issued; fragments are read two product pairs ahead.
    auto mat_phase = [&](auto m_c, int t) {
        constexpr int M = decltype(m_c)::value;
        constexpr int NJ = NKB * NDC;   // products of each kind (S: key block x d chunk; O: key chunk x d block)
        constexpr int MK = (M + 1) % NBUF;
        const lds_char *kb_ = MK == 0 ? (lds_char *)ks0 : (lds_char *)ks1;  // K_{t+1}
        const lds_char *vb = M == 0 ? (lds_char *)vs0 : (lds_char *)vs1;      // V_t
        // S product j: key block j / NDC, contraction chunk j % NDC.
        auto kfrag = [&](int j) { return lds_frag<T>(kb_ + (j / NDC) * 32 * RB + koff[j % NDC]); };
        // O product j: key chunk (16 keys) j / NDB, output block j % NDB.
        auto vfrag = [&](int j) {
            const int cc = j / NDB, db = j % NDB;
            const uint32_t kc_off = (uint32_t)(16 * cc * RB);
            return join<T>(lds_half_tr<T>(vb + kc_off + voff[0][db]),
                           lds_half_tr<T>(vb + kc_off + voff[1][db]));
        };
        auto pfrag = [&](int cc) {
            u32x4 pv;
            pv[0] = pp[4 * cc + 0];
            pv[1] = pp[4 * cc + 1];
            pv[2] = pp[4 * cc + 2];
            pv[3] = pp[4 * cc + 3];
            return __builtin_bit_cast(frag_t<T>, pv);
        };
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
        if (STAGED) keep_begin(t + 1);
        frag_t<T> kf[3], vf[3];
        kf[0] = kfrag(0);
        vf[0] = vfrag(0);
        kf[1] = kfrag(1);
        vf[1] = vfrag(1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (j + 2 < NJ) {
                kf[(j + 2) % 3] = kfrag(j + 2);
                vf[(j + 2) % 3] = vfrag(j + 2);
            }
            mma(s[j / NDC], kf[j % 3], qf[j % NDC]);
            if (STAGED) keep_rounds((KU * j) / NJ, (KU * (j + 1)) / NJ);
            mma(o[j % NDB], vf[j % 3], pfrag(j / NDB));
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Loads run one step ahead: the end of step t brings K_{t+3} and V_{t+2}
    // (into the buffers of K_{t+1} and V_t, read for the last time in step
    // t) after waiting for every load in flight (K_{t+2}, V_{t+1}, which step
    // t+1 reads).  Loads past the end read zeros (or keys no row uses), so
    // every step issues the same number.  The barrier is the bare
    // instruction after explicit counts; no memory operation is moved across
    // it (scheduling barriers on both sides, and the hardware barrier is an
    // unmodelled side effect for the compiler).  (The buffer indices of the
    // loads are compile-time constants too, so that the compiler sees which
    // buffer each direct load writes.)
    auto end_step = [&](auto m_c, int t) {   // m_c: t % 2
        constexpr int M = decltype(m_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");   // no memory operation crosses this point in the IR either
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_kv(t + 3, (M + 1) % 2, t + 2, M);   // K_{t+3}, V_{t+2}
    };
    // ---- prologue: K_0, K_1, V_0, then S of tile 0; then the loads of step
    // 0 (K_2, V_1).
    load_kv(0, 0, 0, 0);
    load_kv(1, 1, 0, 0);   // (V_0 loaded twice: same data, same place)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (Tw > 0) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) mma(s[kb], lds_frag<T>((lds_char *)ks0 + kb * 32 * RB + koff[c]), qf[c]);
        }
    }
    __syncthreads();   // K buffer 0 is refilled before step 0
    load_kv(2, 0, 1, 1);   // K_2, V_1
    if (STAGED) {          // keep bits of tile 0
        keep_begin(0);
        keep_rounds(0, KU);
    }

    // ---- steps.  Every wavefront runs the phase sequence vec(0) mat(0)
    // vec(1) mat(1) ... mat(Tw-1), with the barrier of step t-1 between
    // vec(t) and mat(t); the other wavefront on its SIMD belongs to the other
    // workgroup on the CU, so whichever is not waiting keeps the SIMD busy.
    // Step t reads K_{t+1} and V_t.  Two steps per trip, so buffer indices
    // are constants.  Wavefronts past their last tile keep the loads and
    // barriers of the workgroup going.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto step = [&](auto m_c, int t) {
        constexpr int M = decltype(m_c)::value;
        vec_phase(t);
        if (t > 0) end_step(std::integral_constant<int, (M + 1) % 2>{}, t - 1);
        mat_phase(m_c, t);
    };
    auto end_step_rt = [&](int t) {   // run-time t % 2 (no LDS reads follow)
        if (t % 2 == 0) end_step(I0{}, t);
        else end_step(I1{}, t);
    };
    for (int t = 0; t < Tw; t += 2) {
        step(I0{}, t);
        if (t + 1 < Tw) step(I1{}, t + 1);
    }
    if (Tw > 0) end_step_rt(Tw - 1);
    for (int t = Tw; t < NT; ++t) end_step_rt(t);
    __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the workgroup

    // ---- epilogue: O = c acc / l, LSE = (m + log2 l) ln 2 (of the chunk,
    // in fp32 to the partial buffers, when the keys are split).
    const bool part = a.kv_splits > 1;
    const size_t prow = ((size_t)split * (size_t)BH + (size_t)bh) * (size_t)N;
    const float l_tot = sum_halves(l_run);
    const float inv = l_tot > 0.f ? (DROPOUT ? a.drop_c : 1.f) / l_tot : 0.f;
    if (!part && !a.out_f32) {
        // 16-bit O through LDS: a lane's registers hold 4-column pieces of
        // its row, so each wavefront writes its 32 rows into a tile buffer of
        // its own (swizzled like the tiles, conflict-free) and stores them
        // back as whole rows, 16 bytes per lane.  The barrier makes sure every
        // direct load has landed and every tile read is done.
        __syncthreads();
        lds_char *ob = wave == 0 ? (lds_char *)ks0 : wave == 1 ? (lds_char *)ks1
                     : wave == 2 ? (lds_char *)vs0 : (lds_char *)vs1;
        static_assert(TB >= 32 * D * 2, "a tile buffer holds a wavefront's output rows");
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                u32x2 w;
                w[0] = pack2<T>(o[db][4 * rr + 0] * inv, o[db][4 * rr + 1] * inv);
                w[1] = pack2<T>(o[db][4 * rr + 2] * inv, o[db][4 * rr + 3] * inv);
                *(FA_LDS u32x2 *)(ob + SW::off((uint32_t)lq, (uint32_t)col)) = w;
            }
        T *O = reinterpret_cast<T *>(a.o) + head;
        constexpr int NP = 32 * SW::CPR;          // 16-byte pieces of the wavefront's rows
#pragma unroll
        for (int i = 0; i < (NP + kWave - 1) / kWave; ++i) {
            const int pc = i * kWave + lane;
            const int r = pc / SW::CPR, x = pc % SW::CPR;
            if ((NP % kWave == 0 || pc < NP) && q0w + r < N) {
                const u32x4 v = *(const FA_LDS u32x4 *)(ob + SW::off((uint32_t)r, (uint32_t)(8 * x)));
                *(u32x4 *)(O + (size_t)(q0w + r) * D + 8 * x) = v;
            }
        }
        if (qrow < N && g == 0)
            a.lse[(size_t)bh * (size_t)N + qrow] =
                l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : kNegInf;
    } else if (qrow < N) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int col = 32 * db + 8 * rr + 4 * g;
                const float x0 = o[db][4 * rr + 0] * inv, x1 = o[db][4 * rr + 1] * inv;
                const float x2 = o[db][4 * rr + 2] * inv, x3 = o[db][4 * rr + 3] * inv;
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
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : kNegInf;
            if (part) a.part_lse[prow + qrow] = lse;
            else a.lse[(size_t)bh * (size_t)N + qrow] = lse;
        }
    }
}

template <typename T, int D, bool CAUSAL, bool DROPOUT>
static hipError_t launch_fwd_pp_k(const FwdArgs &a, hipStream_t stream) {
    using TL = FwdPPTile<T, D, DROPOUT>;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb * a.kv_splits;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    FwdArgs b = a;
    b.group = unit_group(a.B * a.H, nqb * a.kv_splits, TL::WG_PER_CU);
    hipLaunchKernelGGL((fwd_pp_kernel<T, D, CAUSAL, DROPOUT>), grid, block, 0, stream, b);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_pp_c(bool dropout, const FwdArgs &a, hipStream_t stream) {
    return dropout ? launch_fwd_pp_k<T, D, CAUSAL, true>(a, stream)
                   : launch_fwd_pp_k<T, D, CAUSAL, false>(a, stream);
}

template <typename T, int D>
static hipError_t launch_fwd_pp_t(bool causal, bool dropout, const FwdArgs &a, hipStream_t stream) {
    return causal ? launch_fwd_pp_c<T, D, true>(dropout, a, stream)
                  : launch_fwd_pp_c<T, D, false>(dropout, a, stream);
}

hipError_t launch_fwd_pp(Elem e, int d, bool causal, bool dropout, const FwdArgs &a,
                         hipStream_t stream) {
    if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return hipErrorInvalidValue;
    if (e == Elem::BF16)
        return d == 32    ? launch_fwd_pp_t<bf16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_fwd_pp_t<bf16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_fwd_pp_t<bf16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_fwd_pp_t<bf16, 128>(causal, dropout, a, stream)
                          : launch_fwd_pp_t<bf16, 256>(causal, dropout, a, stream);
    if (e == Elem::F16)
        return d == 32    ? launch_fwd_pp_t<f16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_fwd_pp_t<f16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_fwd_pp_t<f16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_fwd_pp_t<f16, 128>(causal, dropout, a, stream)
                          : launch_fwd_pp_t<f16, 256>(causal, dropout, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
