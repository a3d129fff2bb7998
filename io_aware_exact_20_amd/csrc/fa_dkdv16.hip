// Backward of fused exact attention for 16-bit inputs on gfx950: the dK /
// dV pass.
//
// The scores and probabilities are recomputed from Q, K and the stored
// log-sum-exp ("Recomputation", mrodiduger.github.io page).  With
//
//   S = scale Q K^T,  P = exp(S - LSE),  dP = (dO V^T) * keep * c,
//   D_i = dO_i . O_i,  dS = P o (dP - D),
//
// this kernel produces dV = (keep c P)^T dO and dK = scale dS^T Q for one
// block of keys per workgroup, streaming the query sequence.
//
// Register files: the K or V operands of a wavefront are pinned to AGPRs
// (the accumulation registers); this file is compiled with matrix-product
// results in VGPRs, so the softmax and dS arithmetic reads the scores and dP
// without v_accvgpr_read copies (the compiler places what does not fit, the
// long-lived dV / dK accumulators first, in the remaining AGPRs).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// One workgroup owns 128 keys (64 at d = 256): two pairs of wavefronts,
// each pair 64 keys (32).  The four products of the backward are split
// between the two wavefronts of a pair, so that each holds only one d x 64
// (d x 32) accumulator (dV^T or dK^T, keys along the lanes) besides its
// operands:
//   A: S = Q K^T (K of its keys in AGPRs), P = exp(S - LSE) and the keep
//      bits, then dV^T += dO^T (keep P);
//   B: dP = dO V^T (V in AGPRs), dS = P o (dP keep c - D) with P taken from
//      A, then dK^T += Q^T dS.
// Both products of a wavefront contract over the 32 query rows of a step
// with the keys on the accumulator columns, so the rounded S / dS
// registers are directly their B operands; the transposed A operands (dO^T,
// Q^T) are read from the row-major LDS tiles with ds_read_b64_tr_b16.
//
// A hands P over through LDS in fp32 (the register image of its
// accumulator, lane for lane).  Dropout keep decisions are drawn once per
// tile, a quarter by A and three quarters by B (A carries the
// exponentials, so this evens out the vector work of the two), as 16-bit
// masks in a row-major LDS block; the transposed 16-bit LDS read hands
// every lane the masks of its own (key, rows) registers, already paired as
// the products need them.
// Per 32-row step t:
//   A: S of tile t+1 | P of tile t (to LDS);  dV += dO^T (keep P) of tile t;
//   B: dP of tile t | dS of tile t-1;         dK += Q^T dS of tile t-1;
// ("x | y": products x on the matrix cores while the VALU does y), so B
// reads A's P one step after it was written (one barrier per step).  Tile
// t's Q is read by A in step t-1 and by B in step t+1 (four LDS buffers);
// dO tiles are read in one step (two buffers).
template <typename T, int D>
struct Dkdv16Tile {
    static constexpr int NW = 4;                       // 2 pairs x (A, B)
    // 32-key blocks per pair: two, one at d = 256 (where a d x 64 fp32
    // accumulator and the 64 keys' operands would not fit the registers)
    static constexpr int NKP = D == 256 ? 1 : 2;
    static constexpr int KP = 32 * NKP;                // keys per pair
    static constexpr int BK = 2 * KP;                  // keys per workgroup
    static constexpr int BQ = 32;                      // query rows per step
    static constexpr int THREADS = NW * kWave;
    static constexpr int TB = BQ * D * 2;              // bytes of a Q or dO tile
    static constexpr int CHUNKS = TB / (kWave * 16);        // 1 KB load instructions per tile
    static constexpr int LOADS = (CHUNKS + NW - 1) / NW;    // per wavefront (d = 96: 2 or 1)
};

// 4 bytes per lane at byte offset voff + soff straight into LDS at base + 4 l.
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         lds_char *base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void *)base, 4, voff, soff, 0, 0);
}

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, 1) dkdv16_kernel(const BwdArgs a) {
    using TL = Dkdv16Tile<T, D>;
    using SW = Swz<D>;
    constexpr int NW = TL::NW, NKP = TL::NKP, KP = TL::KP, BK = TL::BK, BQ = TL::BQ;
    constexpr int TB = TL::TB, LOADS = TL::LOADS, CHUNKS = TL::CHUNKS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;
    constexpr int NDB = D / 32;
    constexpr float kNegInf = -__builtin_huge_valf();
    static_assert(LOADS >= 1, "tile load split");

    __shared__ __attribute__((aligned(1024))) char qs0[TB], qs1[TB], qs2[TB], qs3[TB], os0[TB], os1[TB];
    __shared__ __attribute__((aligned(256))) float nl_s[2][64];
    __shared__ __attribute__((aligned(256))) float dv_s[4][64];
    __shared__ __attribute__((aligned(1024))) float pex[2][2][16 * NKP * 64];   // [slot][pair][regs x lanes]
    // Dropout keep masks: 16-bit 0x0000 / 0xFFFF per (row, key) of a pair's
    // 32 x KP block, row-major with a row pitch of 2 KP + 64 bytes (192 at
    // KP = 64: conflict-free for the transposed reads); four tiles in flight.
    constexpr int MP = 2 * KP + 64;
    __shared__ __attribute__((aligned(1024))) char mk[DROPOUT ? 4 : 1][2][32 * MP];
    auto qbuf = [&](int s) {
        return s == 0 ? (lds_char *)qs0 : s == 1 ? (lds_char *)qs1 : s == 2 ? (lds_char *)qs2 : (lds_char *)qs3;
    };
    auto obuf = [&](int s) { return s == 0 ? (lds_char *)os0 : (lds_char *)os1; };

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int role = wave >> 1, pair = wave & 1;          // role 0: A, 1: B
    const int lq = lane & 31, g = lane >> 5;

    const int64_t BH = a.B * a.H;
    const int64_t nkb = (a.Nk + BK - 1) / BK;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)nkb, a.group);
    const int64_t bh = un.bh;
    const int kblk = (int)un.rank;                        // causal: low key blocks (most work) first
    const int N = (int)a.N, Nk = (int)a.Nk;
    const int off = Nk - N;                  // causal: query i sees keys j <= i + off
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head_kv;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int k0 = kblk * BK;                 // first key of the workgroup
    const int kp0 = k0 + pair * KP;           // first key of this pair
    // first query tile (causal: the first row that sees key k0 is k0 - off)
    const int j0 = CAUSAL ? (k0 - off > 0 ? (k0 - off) / BQ : 0) : 0;
    const int NTQ = (N + BQ - 1) / BQ - j0;   // query tiles streamed

    // ---- the pair's K (A) or V (B) rows: B operands, one key per lane, in AGPRs.
    frag_t<T> kv[NKP][NDC];
    {
        const T *src = role == 0 ? Kg : Vg;
#pragma unroll
        for (int kb = 0; kb < NKP; ++kb) {
            int key = kp0 + 32 * kb + lq;
            key = key < Nk ? key : Nk - 1;
#pragma unroll
            for (int c = 0; c < NDC; ++c) kv[kb][c] = load_frag<T>(src + (size_t)key * D + 16 * c + 8 * g);
        }
    }

    // ---- LDS offsets: row fragments of a Q / dO tile (row = query lq) and
    // transposed reads (rows = queries, columns = d).
    uint32_t roff[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) roff[c] = SW::off(lq, 16 * c + 8 * g);
    uint32_t toff[2][NDB];
    {
        const int G = lane >> 4, k = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                toff[hf][db] = SW::off(8 * hf + 4 * (G >> 1) + k, 32 * db + 16 * (G & 1) + 4 * j);
    }

    // ---- loads: Q and dO tiles (all four wavefronts, LOADS instructions
    // each), -LSE log2(e) rows (the A wavefronts) and D/c rows (the B
    // wavefronts).
    // Load instruction i of a wavefront is the tile's 1 KB chunk c = wave +
    // i NW, lane l filling 16-byte position p = 64 c + l (row p / CPR).
    // Where chunks hold whole rows, instruction i fills rows R0 + i RSTEP;
    // the swizzle repeats every 16 rows, so where RSTEP is a multiple of 16
    // every instruction uses the lane offset of R0 (the row step goes into
    // the scalar offset); otherwise (d = 96, 256) each has its own.  At
    // d = 96 a tile is six chunks: waves 0 and 1 issue two, waves 2 and 3 one.
    constexpr bool ALIGNED = kWave % SW::CPR == 0;
    constexpr int RSTEP = ALIGNED ? NW * kWave / SW::CPR : 0;
    constexpr bool ONE_OFF = ALIGNED && RSTEP % 16 == 0;
    uint32_t lane_boff[ONE_OFF ? 1 : LOADS];
#pragma unroll
    for (int i = 0; i < (ONE_OFF ? 1 : LOADS); ++i) {
        if constexpr (ALIGNED) {
            const uint32_t r = (uint32_t)((wave * kWave + lane) / SW::CPR + i * RSTEP);
            lane_boff[i] = (r * D + (((uint32_t)lane % SW::CPR) ^ SW::f(r)) * 8) * 2;
        } else {
            const uint32_t pos = (uint32_t)((wave + i * NW) * kWave + lane);
            const uint32_t r = pos / SW::CPR;
            lane_boff[i] = (r * D + ((pos % SW::CPR) ^ SW::f(r)) * 8) * 2;
        }
    }
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, head_bytes), ors = make_rsrc(dOg, head_bytes);
    const __amdgpu_buffer_rsrc_t rrs =
        role == 0 ? make_rsrc(a.nl2 + (size_t)bh * (size_t)N, (uint32_t)N * 4)
                  : make_rsrc(a.dvec + (size_t)bh * (size_t)N, (uint32_t)N * 4);
    auto load_tile_part = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf, int i) {
        if (CHUNKS % NW != 0 && wave + i * NW >= CHUNKS) return;   // (wave-uniform)
        if constexpr (ONE_OFF)
            buf2lds16(rs, lane_boff[0], (uint32_t)((j0 + t) * BQ + i * RSTEP) * (uint32_t)(D * 2),
                      buf + (wave + i * NW) * (kWave * 16));
        else
            buf2lds16(rs, lane_boff[i], (uint32_t)((j0 + t) * BQ) * (uint32_t)(D * 2),
                      buf + (wave + i * NW) * (kWave * 16));
    };
    auto load_rows = [&](int t, lds_char *buf) {   // 64 fp32 rows from the tile's first row
        buf2lds4(rrs, (uint32_t)lane * 4, (uint32_t)((j0 + t) * BQ) * 4, buf);
    };
    // Loads issued during step s: Q of tile s+2; dO and row statistics of tile s+1.
    auto issue_loads = [&](int s, int qsl, int osl, int rsl2, int rsl4) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            load_tile_part(qrs, s + 2, qbuf(qsl), i);
            load_tile_part(ors, s + 1, obuf(osl), i);
        }
        if (role == 0) load_rows(s + 1, (lds_char *)nl_s[rsl2]);
        else load_rows(s + 1, (lds_char *)dv_s[rsl4]);
    };

    const float sl2 = a.scale_log2, dc = a.drop_c;
    f32x16 acc[NDB][NKP];        // dV^T (A) or dK^T (B): [d block][key block]
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < NKP; ++kb) acc[db][kb] = f32x16{};

    // Masking of tile t for this pair: key > query (causal), key >= N, row >= N.
    auto is_edge = [&](int t) {
        const int qt0 = (j0 + t) * BQ;
        return (qt0 + BQ > N) || (kp0 + KP > Nk) || (CAUSAL && kp0 + KP - 1 > qt0 + off);
    };
    auto apply_mask = [&](f32x16 (&s)[NKP], int t) {
        const int qt0 = (j0 + t) * BQ;
#pragma unroll
        for (int kb = 0; kb < NKP; ++kb) {
            const int key = kp0 + 32 * kb + lq;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = qt0 + 8 * (r / 4) + 4 * g + (r % 4);
                if ((CAUSAL && key > q + off) || key >= Nk || q >= N) s[kb][r] = kNegInf;
            }
        }
    };

    // Keep masks of this pair's tile t: its 32 rows x KP keys are 4 NKP
    // Philox blocks of 8 keys per row (block j: keys 8j .. 8j+7), drawn by
    // the four lanes of a row -- A lane (row lq, half g) block g, B lane
    // (row lq, half g) the NBB blocks from 2 + NBB g -- and stored as 16-bit
    // masks.
    // The draw is staged (counters, then the block-rounds in order, then the
    // masks): the rounds of tile s+2 are spread over the second product
    // phase of step s and its masks are formed and stored during the first
    // phase of step s+1, so no part of the draw waits at the end of a step.
    constexpr int NBA = 1, NBB = 4 * NKP / 2 - 1;   // blocks per lane: A, B
    struct MaskDraw { Philox4 c[NBB]; };
    const int jb0 = role == 0 ? g : 2 + NBB * g;  // first block of this lane
    auto mask_begin = [&](MaskDraw &m, int t) {
        const uint32_t grp = (uint32_t)(kp0 >> 3) + (uint32_t)jb0;
        const uint32_t row = (uint32_t)((j0 + t) * BQ + lq);
#pragma unroll
        for (int h = 0; h < NBB; ++h) {
            m.c[h].x[0] = grp + h;
            m.c[h].x[1] = row;
            m.c[h].x[2] = h_idx;
            m.c[h].x[3] = b_idx;
        }
    };
    // Block-rounds u0 .. u1-1 of 10 NB: unit u is round u / NB of block
    // u % NB (NB = NBA or NBB, a compile-time constant at every call).  The
    // state is pinned afterwards so that the rounds stay in the group that
    // issues them.
    struct CNB : std::integral_constant<int, NBB> {};   // a type of its own even when NBB == NBA
    auto mask_rounds = [&](auto nb_c, MaskDraw &m, int u0, int u1) {
        constexpr int NB = decltype(nb_c)::value;
        // B's draws end with the folded flip of words 0 and 2 (its masks
        // are formed with keep_mask2_flipped for them); A's are plain.
        constexpr bool FLIP = std::is_same<decltype(nb_c), CNB>::value;
#pragma unroll
        for (int u = u0; u < u1; ++u) philox_round<FLIP>(m.c[u % NB], u / NB, a.seed_lo, a.seed_hi);
        if (u1 > u0) {
#pragma unroll
            for (int h = 0; h < NB; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) pin_vgpr(m.c[h].x[q]);
        }
    };
    // Masks of block h of a finished draw: word q of the block holds keys 2q
    // (low half) and 2q + 1 (high half).
    const uint32_t kc2 = keep_cmp_const(a.drop_T);
    auto mask_end_blk = [&](MaskDraw &m, int slot, int h) {
        FA_LDS char *p = (FA_LDS char *)mk[slot & (DROPOUT ? 3 : 0)][pair] + lq * MP + 16 * (jb0 + h);
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = (role != 0 && !(q & 1)) ? keep_mask2_flipped(m.c[h].x[q], kc2) : keep_mask2(m.c[h].x[q], kc2);
        *(FA_LDS u32x4 *)p = w;
    };
    MaskDraw pend;   // draw whose masks are stored in the first phase of the next step
    // Per-lane byte offset of the transposed mask read: lane receives the
    // masks of rows 8 q4 + 4g + 0..3 (its registers 4 q4 .. 4 q4 + 3) of key
    // 32 kb + lq, with q4 and kb added as immediates.
    const uint32_t mtr = (uint32_t)((4 * ((lane >> 5)) + ((lane >> 2) & 3)) * MP +
                                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
    auto read_masks = [&](int slot, int kb, int q4) {
        const half_t<T> m = lds_half_tr<T>((lds_char *)mk[slot & (DROPOUT ? 3 : 0)][pair] + mtr +
                                           (uint32_t)(8 * q4 * MP + 32 * kb * 2));
        return __builtin_bit_cast(u32x2, m);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using CNA = std::integral_constant<int, NBA>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using YES = std::true_type;
    using NO = std::false_type;

    // ---- prologue loads: Q_0, Q_1, dO_0, rows of tile 0.
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        load_tile_part(qrs, 0, qbuf(0), i);
        load_tile_part(qrs, 1, qbuf(1), i);
        load_tile_part(ors, 0, obuf(0), i);
    }
    if (role == 0) load_rows(0, (lds_char *)nl_s[0]);
    else load_rows(0, (lds_char *)dv_s[0]);
    // K or V into AGPRs once all loads are in flight (a pin waits for its load).
#pragma unroll
    for (int kb = 0; kb < NKP; ++kb)
#pragma unroll
        for (int c = 0; c < NDC; ++c) pin_agpr(kv[kb][c]);
    if (DROPOUT) {
        MaskDraw m0;                     // tile 0: complete
        mask_begin(m0, 0);
        mask_begin(pend, 1);             // tile 1: stored during step 0
        if (role == 0) {
            mask_rounds(CNA{}, m0, 0, 10 * NBA);
            mask_end_blk(m0, 0, 0);
            mask_rounds(CNA{}, pend, 0, 10 * NBA);
        } else {
            mask_rounds(CNB{}, m0, 0, 10 * NBB);
#pragma unroll
            for (int h = 0; h < NBB; ++h) mask_end_blk(m0, 0, h);
            mask_rounds(CNB{}, pend, 0, 10 * NBB);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Work of one step is laid out in groups of two matrix products each
    // (sched_barrier between groups), with the VALU work of the group
    // placed between its two products and every LDS read issued two groups
    // before the group that uses it.
    if (role == 0) {
        // ============================== A: S, P, dV ==============================
        // Step s: S of tile s+1 (Q slot (s+1)%4) on the matrix cores while
        // the VALU exponentiates tile s; then dV of tile s (dO slot s%2).
        f32x16 sA[NKP], sB[NKP];
        auto a_step = [&](auto r_c, f32x16 (&sc)[NKP], f32x16 (&sn)[NKP], int s) {
            constexpr int R = decltype(r_c)::value;
            lds_char *qb = qbuf((R + 1) & 3);
            lds_char *ob = obuf(R & 1);
            const FA_LDS float *nlp = (const FA_LDS float *)nl_s[R & 1];
            FA_LDS float *px = (FA_LDS float *)pex[R & 1][pair];
            issue_loads(s, (R + 2) & 3, (R + 1) & 1, (R + 1) & 1, 0);

            frag_t<T> qf[3], of[3];
            qf[0] = lds_frag<T>(qb + roff[0]);
            qf[1] = lds_frag<T>(qb + roff[1]);
            f32x4 l4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) l4[q4] = *(const FA_LDS f32x4 *)(nlp + 8 * q4 + 4 * g);
            u32x2 mw[NKP][4];
            if (DROPOUT) {
#pragma unroll
                for (int kb = 0; kb < NKP; ++kb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) mw[kb][q4] = read_masks(R, kb, q4);
            }
            uint32_t pp[NKP][8];
            // P of register group (kb, q4) of tile s: handed to B in fp32,
            // and rounded (and kept) at once for dV, so that no fp32 copy of
            // P stays live (measured: d = 32 3 %, d = 64 1.5 % faster dK/dV
            // than rounding pairs of groups later; d = 128 unchanged).
            auto pgroup = [&](int kb, int q4) {
                f32x4 xo;
#pragma unroll
                for (int e = 0; e < 4; ++e) xo[e] = fast_exp2(fmaf(sc[kb][4 * q4 + e], sl2, l4[q4][e]));
                *(FA_LDS f32x4 *)(px + ((4 * kb + q4) * kWave + lane) * 4) = xo;
                pp[kb][2 * q4] = pack2<T>(xo[0], xo[1]);
                pp[kb][2 * q4 + 1] = pack2<T>(xo[2], xo[3]);
                if (DROPOUT) {
                    pp[kb][2 * q4] &= mw[kb][q4][0];
                    pp[kb][2 * q4 + 1] &= mw[kb][q4][1];
                }
                pin_vgpr(pp[kb][2 * q4]);
                pin_vgpr(pp[kb][2 * q4 + 1]);
            };
            auto ofrag = [&](int j) {
                const int cc = j / NDB, db = j % NDB;
                const uint32_t kc_off = (uint32_t)(16 * cc * RB);
                return join<T>(lds_half_tr<T>(ob + kc_off + toff[0][db]),
                               lds_half_tr<T>(ob + kc_off + toff[1][db]));
            };

            // ---- phase 1: S of tile s+1 | P of tile s.
#pragma unroll
            for (int kb = 0; kb < NKP; ++kb) sn[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                if (c + 2 < NDC) qf[(c + 2) % 3] = lds_frag<T>(qb + roff[c + 2]);
                if (c == NDC - 2) of[0] = ofrag(0);
                if (c == NDC - 1) of[1] = ofrag(1);
                mma(sn[0], qf[c % 3], kv[0][c]);
                if constexpr (NKP == 2) {
                    if (NDC == 8) {
                        if (c < 6) pgroup(c & 1, c >> 1);     // q4 = 0, 1, 2
                    } else if (NDC == 2) {                    // d = 32: two row groups per product
                        pgroup(0, 2 * c);
                        pgroup(1, 2 * c);
                        pgroup(0, 2 * c + 1);
                        pgroup(1, 2 * c + 1);
                    } else if (c < 4) {                       // d = 64, 96
                        pgroup(0, c);
                        pgroup(1, c);
                    }
                } else {
                    if (c < 4) pgroup(0, c);
                }
                if (DROPOUT && c == 1) mask_end_blk(pend, R + 1, 0);
                if constexpr (NKP == 2) mma(sn[1], qf[c % 3], kv[1][c]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- phase 2: dV^T += dO^T (keep P) of tile s | keep masks of
            // tile s+2 (block-rounds, cumulative count before group j: UA[j];
            // none in the first groups, which finish P of tile s).
            constexpr int UA[9] = {0, 0, 0, 1, 2, 4, 6, 8, 10};
            constexpr int UA64[5] = {0, 1, 4, 7, 10};
            static_assert(UA[8] == 10 * NBA && UA64[4] == 10 * NBA, "A draws NBA blocks");
            MaskDraw md;
            if (DROPOUT) mask_begin(md, s + 2);
#pragma unroll
            for (int j = 0; j < 2 * NDB; ++j) {
                const int cc = j / NDB, db = j % NDB;
                if (j + 2 < 2 * NDB) of[(j + 2) % 3] = ofrag(j + 2);
                if (DROPOUT) {
                    if constexpr (NDB == 4) mask_rounds(CNA{}, md, UA[j], UA[j + 1]);
                    else if constexpr (NDB == 2) mask_rounds(CNA{}, md, UA64[j], UA64[j + 1]);
                    else   // d = 256 (P finished in phase 1): spread evenly
                        mask_rounds(CNA{}, md, (10 * NBA * j) / (2 * NDB), (10 * NBA * (j + 1)) / (2 * NDB));
                }
                if constexpr (NKP == 2 && NDC == 8) {
                    if (j == 0) pgroup(0, 3);
                    if (j == 1) pgroup(1, 3);
                }
#pragma unroll
                for (int kb = 0; kb < NKP; ++kb) {
                    u32x4 p4;
                    p4[0] = pp[kb][4 * cc + 0];
                    p4[1] = pp[kb][4 * cc + 1];
                    p4[2] = pp[kb][4 * cc + 2];
                    p4[3] = pp[kb][4 * cc + 3];
                    mma(acc[db][kb], of[j % 3], __builtin_bit_cast(frag_t<T>, p4));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (is_edge(s + 1)) apply_mask(sn, s + 1);
            if (DROPOUT) pend = md;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };

        // prologue: S of tile 0 (Q slot 0).
        if (NTQ > 0) {
#pragma unroll
            for (int kb = 0; kb < NKP; ++kb) sA[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                const frag_t<T> qfr = lds_frag<T>(qbuf(0) + roff[c]);
#pragma unroll
                for (int kb = 0; kb < NKP; ++kb) mma(sA[kb], qfr, kv[kb][c]);
            }
            if (is_edge(0)) apply_mask(sA, 0);
        }
        // The last step also computes S of tile NTQ (zero-filled rows past
        // the end, never used), which keeps a single step shape.
        for (int s = 0; s < NTQ; s += 4) {
            a_step(I0{}, sA, sB, s);
            if (s + 1 < NTQ) a_step(I1{}, sB, sA, s + 1);
            if (s + 2 < NTQ) a_step(I2{}, sA, sB, s + 2);
            if (s + 3 < NTQ) a_step(I3{}, sB, sA, s + 3);
        }
        // step NTQ: B finishes the last tile; keep the barrier count.
        __syncthreads();
    } else {
        // ============================== B: dP, dS, dK ============================
        // Step s: dP of tile s (dO slot s%2) on the matrix cores while the
        // VALU forms dS of tile s-1 from its dP, A's P (P slot (s-1)%2) and D
        // (D slot (s-1)%4); then dK of tile s-1 (Q slot (s-1)%4).
        f32x16 dA[NKP], dB[NKP];
        // dS register groups ("items") i = (key block i % NKP, rows q4 = i / NKP);
        // item i is formed in phase-1 group ig(i), its P and masks fetched
        // two groups earlier.
        constexpr int NI = 4 * NKP;
        auto ig = [](int i) { return (i * NDC) / NI; };
        auto b_step = [&](auto r_c, auto hp_c, f32x16 (&dcur)[NKP], f32x16 (&dprv)[NKP], int s) {
            constexpr int R = decltype(r_c)::value;
            constexpr bool HP = decltype(hp_c)::value;
            lds_char *ob = obuf(R & 1);
            lds_char *qb = qbuf((R + 3) & 3);
            const FA_LDS float *dvp = (const FA_LDS float *)dv_s[(R + 3) & 3];
            const FA_LDS float *px = (const FA_LDS float *)pex[(R + 1) & 1][pair];
            issue_loads(s, (R + 2) & 3, (R + 1) & 1, 0, (R + 1) & 3);

            frag_t<T> of[3], qt[3];
            of[0] = lds_frag<T>(ob + roff[0]);
            of[1] = lds_frag<T>(ob + roff[1]);
            f32x4 d4[4], x4[NI];
            u32x2 mw[NI];
            auto fetch = [&](int i) {
                x4[i] = *(const FA_LDS f32x4 *)(px + ((4 * (i % NKP) + i / NKP) * kWave + lane) * 4);
                if (DROPOUT) mw[i] = read_masks(R + 3, i % NKP, i / NKP);
            };
            if (HP) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) d4[q4] = *(const FA_LDS f32x4 *)(dvp + 8 * q4 + 4 * g);
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    if (ig(i) < 2) fetch(i);
            }
            uint32_t sp[NKP][8];
            auto dsitem = [&](int i) {
                const int kb = i % NKP, q4 = i / NKP;
                const f32x4 x = x4[i];
                float ds[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dpv = dprv[kb][4 * q4 + e];
                    if (DROPOUT) {
                        // dP * keep: the 16-bit mask sign-extended to 32 bits.
                        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)mw[i][e >> 1], 16 * (e & 1), 16);
                        const float kd = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, dpv) & m);
                        ds[e] = x[e] * (kd - d4[q4][e]);
                    } else {
                        ds[e] = x[e] * (dpv - d4[q4][e]);
                    }
                }
                sp[kb][2 * q4] = pack2<T>(ds[0], ds[1]);
                sp[kb][2 * q4 + 1] = pack2<T>(ds[2], ds[3]);
                pin_vgpr(sp[kb][2 * q4]);
                pin_vgpr(sp[kb][2 * q4 + 1]);
            };
            auto qfrag = [&](int j) {
                const int cc = j / NDB, db = j % NDB;
                const uint32_t kc_off = (uint32_t)(16 * cc * RB);
                return join<T>(lds_half_tr<T>(qb + kc_off + toff[0][db]),
                               lds_half_tr<T>(qb + kc_off + toff[1][db]));
            };

            // ---- phase 1: dP of tile s | dS of tile s-1.
#pragma unroll
            for (int kb = 0; kb < NKP; ++kb) dcur[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                if (c + 2 < NDC) of[(c + 2) % 3] = lds_frag<T>(ob + roff[c + 2]);
                if (HP) {
#pragma unroll
                    for (int i = 0; i < NI; ++i)
                        if (ig(i) == c + 2) fetch(i);
                    if (c == NDC - 2) qt[0] = qfrag(0);
                    if (c == NDC - 1) qt[1] = qfrag(1);
                }
                mma(dcur[0], of[c % 3], kv[0][c]);
                if (HP) {
#pragma unroll
                    for (int i = 0; i < NI; ++i)
                        if (ig(i) == c) dsitem(i);
                }
                // masks of the pending draw: block h after product c = 2h + 1
                // (d >= 128), h + 1 (d = 64, 96), all after product 1 (d = 32)
                if (DROPOUT && NDC == 2 && c == 1) {
#pragma unroll
                    for (int h = 0; h < NBB; ++h) mask_end_blk(pend, R + 1, h);
                } else if (DROPOUT && NDC > 2 &&
                           (NDC >= 8 ? (c & 1) && (c >> 1) < NBB : c >= 1 && c - 1 < NBB)) {
                    mask_end_blk(pend, R + 1, NDC >= 8 ? c >> 1 : c - 1);
                }
                if constexpr (NKP == 2) mma(dcur[1], of[c % 3], kv[1][c]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- phase 2: dK^T += Q^T dS of tile s-1 | keep masks of tile
            // s+2 (block-rounds, cumulative count before group j: UB[j]).
            constexpr int UB[9] = {0, 4, 8, 12, 16, 19, 22, 26, 30};
            constexpr int UB64[5] = {0, 8, 15, 23, 30};
            static_assert(NKP == 1 || (UB[8] == 10 * NBB && UB64[4] == 10 * NBB), "B draws NBB blocks");
            MaskDraw md;
            if (DROPOUT) mask_begin(md, s + 2);
            if (HP) {
#pragma unroll
                for (int j = 0; j < 2 * NDB; ++j) {
                    const int cc = j / NDB, db = j % NDB;
                    if (j + 2 < 2 * NDB) qt[(j + 2) % 3] = qfrag(j + 2);
                    if (DROPOUT) {
                        if constexpr (NDB == 4) mask_rounds(CNB{}, md, UB[j], UB[j + 1]);
                        else if constexpr (NDB == 2) mask_rounds(CNB{}, md, UB64[j], UB64[j + 1]);
                        else   // d = 256: spread evenly
                            mask_rounds(CNB{}, md, (10 * NBB * j) / (2 * NDB), (10 * NBB * (j + 1)) / (2 * NDB));
                    }
#pragma unroll
                    for (int kb = 0; kb < NKP; ++kb) {
                        u32x4 p4;
                        p4[0] = sp[kb][4 * cc + 0];
                        p4[1] = sp[kb][4 * cc + 1];
                        p4[2] = sp[kb][4 * cc + 2];
                        p4[3] = sp[kb][4 * cc + 3];
                        mma(acc[db][kb], qt[j % 3], __builtin_bit_cast(frag_t<T>, p4));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (DROPOUT) {
                if (!HP) mask_rounds(CNB{}, md, 0, 10 * NBB);
                pend = md;
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };

        // Steps 0 .. NTQ.  Step NTQ finishes tile NTQ-1; its dP half runs on
        // the zero-filled rows past the last tile (harmless, never used).
        if (NTQ > 0) {
            b_step(I0{}, NO{}, dA, dB, 0);
            for (int s = 1; s <= NTQ; s += 4) {
                b_step(I1{}, YES{}, dB, dA, s);
                if (s + 1 <= NTQ) b_step(I2{}, YES{}, dA, dB, s + 1);
                if (s + 2 <= NTQ) b_step(I3{}, YES{}, dB, dA, s + 2);
                if (s + 3 <= NTQ) b_step(I0{}, YES{}, dA, dB, s + 3);
            }
        } else {
            __syncthreads();
        }
    }

    // ---- epilogue: dV = c * acc (A), dK = scale * acc (B); keys past N not stored.
    const float osc = DROPOUT ? (role == 0 ? dc : a.scale * dc) : (role == 0 ? 1.f : a.scale);
    void *dst = role == 0 ? a.dv : a.dk;
#pragma unroll
    for (int kb = 0; kb < NKP; ++kb) {
        const int key = kp0 + 32 * kb + lq;
        if (key < Nk) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr + 4 * g;
                    const float x0 = osc * acc[db][kb][4 * rr + 0], x1 = osc * acc[db][kb][4 * rr + 1];
                    const float x2 = osc * acc[db][kb][4 * rr + 2], x3 = osc * acc[db][kb][4 * rr + 3];
                    if (a.out_f32)
                        store4<float>(reinterpret_cast<float *>(dst) + head_kv + (size_t)key * D + col, x0, x1, x2, x3);
                    else
                        store4<T>(reinterpret_cast<T *>(dst) + head_kv + (size_t)key * D + col, x0, x1, x2, x3);
                }
        }
    }
}

template <typename T, int D>
static hipError_t launch_dkdv16_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = Dkdv16Tile<T, D>;
    const int64_t nkb = (a.Nk + TL::BK - 1) / TL::BK;
    const int64_t units = a.B * a.H * nkb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    BwdArgs b = a;
    b.group = unit_group(a.B * a.H, nkb, 1);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((dkdv16_kernel<T, D, true, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((dkdv16_kernel<T, D, true, false>), grid, block, 0, stream, b);
    } else {
        if (dropout) hipLaunchKernelGGL((dkdv16_kernel<T, D, false, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((dkdv16_kernel<T, D, false, false>), grid, block, 0, stream, b);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                             hipStream_t stream) {
    switch (e) {
    case Elem::BF16:
        return d == 32    ? launch_dkdv16_t<bf16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_dkdv16_t<bf16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_dkdv16_t<bf16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_dkdv16_t<bf16, 128>(causal, dropout, a, stream)
                          : launch_dkdv16_t<bf16, 256>(causal, dropout, a, stream);
    case Elem::F16:
        return d == 32    ? launch_dkdv16_t<f16, 32>(causal, dropout, a, stream)
               : d == 64  ? launch_dkdv16_t<f16, 64>(causal, dropout, a, stream)
               : d == 96  ? launch_dkdv16_t<f16, 96>(causal, dropout, a, stream)
               : d == 128 ? launch_dkdv16_t<f16, 128>(causal, dropout, a, stream)
                          : launch_dkdv16_t<f16, 256>(causal, dropout, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fa
