// Backward of fused exact attention for 16-bit inputs on gfx950: the dQ
// pass.
//
// The scores and probabilities are recomputed from Q, K and the stored
// log-sum-exp ("Recomputation", mrodiduger.github.io page).  With
//
//   S = scale Q K^T,  P = exp(S - LSE),  dP = (dO V^T) * keep * c,
//   D_i = dO_i . O_i,  dS = P o (dP - D),
//
// this kernel produces dQ = scale dS K for one block of query rows per
// workgroup, streaming the key/value sequence.  It is shaped like the
// forward: every wavefront holds 64 query rows, so each K and V fragment
// read from LDS feeds two matrix products, and Q and dO sit in AGPRs as
// the B operands of S^T = K Q^T and dP^T = V dO^T (one query row per lane).
// dQ^T += K^T dS^T takes K^T from the row-major K tile with transposed LDS
// reads and dS^T straight from the rounded accumulator registers.
//
// Schedule of one 32-key step t (two 32-row blocks a and b per wavefront):
//   1a  S, dP of block a, tile t      | dS of block b, tile t-1
//   3b  dQ of block b += K_{t-1}^T dS  |
//   1b  S, dP of block b, tile t      | dS of block a, tile t
//   3a  dQ of block a += K_t^T dS      |
// so that the VALU work of every row block runs under another block's
// products while only two blocks' scores are ever live.  K tiles stay in
// LDS for one more step (three buffers); V tiles are needed for one step.
//
// At d = 256, where Q, dO and the dQ accumulator of 64 rows would not fit
// the registers, a wavefront holds one block of 32 rows and the overlap is
// across tiles instead:
//   1   S, dP of tile t               | dS of tile t-1
//   3   dQ += K_{t-1}^T dS             |
#pragma once

#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr float kLog2eB = 1.44269504088896340736f;

template <typename T, int D>
struct Dq16Tile {
    static constexpr int NW = 4;                  // wavefronts per workgroup
    static constexpr int NRB = D == 256 ? 1 : 2;  // 32-row blocks per wavefront
    static constexpr int RW = 32 * NRB;           // query rows per wavefront
    static constexpr int BQ = NW * RW;            // query rows per workgroup
    static constexpr int BC = 32;                 // keys per step
    static constexpr int THREADS = NW * kWave;
    static constexpr int TILE_BYTES = BC * D * 2;
    static constexpr int CHUNKS = TILE_BYTES / (kWave * 16);       // 1 KB load instructions per tile
    static constexpr int LOADS = (CHUNKS + NW - 1) / NW;           // per wave per tile (d = 96: 2 or 1)
    static constexpr int RING = 3;                // LDS buffers per tensor
};

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, 1) dq16_kernel(const BwdArgs a) {
    using TL = Dq16Tile<T, D>;
    using SW = Swz<D>;
    constexpr int NW = TL::NW, NRB = TL::NRB, RW = TL::RW, BQ = TL::BQ, BC = TL::BC;
    constexpr int TB = TL::TILE_BYTES, LOADS = TL::LOADS, CHUNKS = TL::CHUNKS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;   // contraction chunks of S, dP
    constexpr int NDB = D / 32;   // 32-column blocks of dQ
    constexpr float kNegInf = -__builtin_huge_valf();

    __shared__ __attribute__((aligned(1024))) char ks0[TB], ks1[TB], ks2[TB], vs0[TB], vs1[TB], vs2[TB];
    auto kbuf = [&](int s) { return s == 0 ? (lds_char *)ks0 : s == 1 ? (lds_char *)ks1 : (lds_char *)ks2; };
    auto vbuf = [&](int s) { return s == 0 ? (lds_char *)vs0 : s == 1 ? (lds_char *)vs1 : (lds_char *)vs2; };

    const int lane = (int)lane_in_wave();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lq = lane & 31, g = lane >> 5;

    const int64_t BH = a.B * a.H;
    const int64_t nqb = (a.N + BQ - 1) / BQ;
    const Unit un = unit_of(blockIdx.x, gridDim.x, (uint32_t)BH, (uint32_t)nqb, a.group);
    const int64_t bh = un.bh;
    const int64_t qb = CAUSAL ? (nqb - 1 - un.rank) : un.rank;
    const int N = (int)a.N, Nk = (int)a.Nk;
    const int64_t off = (int64_t)Nk - N;   // causal: row i sees keys j <= i + off
    const size_t head = (size_t)bh * (size_t)N * D, head_kv = (size_t)bh * (size_t)Nk * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head_kv;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head_kv;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int q0 = (int)qb * BQ;
    const int q0w = q0 + wave * RW;

    // ---- Q and dO fragments (B operands, one query row per lane), in AGPRs;
    // log2-scaled LSE and D of the lane's two rows (rows past N: P = 0).
    frag_t<T> qf[NRB][NDC], df[NRB][NDC];
    float lse2[NRB], dvec[NRB];
#pragma unroll
    for (int nb = 0; nb < NRB; ++nb) {
        const int row = q0w + 32 * nb + lq;
        const int r = row < N ? row : N - 1;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            qf[nb][c] = load_frag<T>(Qg + (size_t)r * D + 16 * c + 8 * g);
            df[nb][c] = load_frag<T>(dOg + (size_t)r * D + 16 * c + 8 * g);
        }
        // rows past N and rows that see no key (LSE = -inf): P = exp2(-inf) = 0
        const float l = row < N ? a.lse[(size_t)bh * (size_t)N + row] : -__builtin_huge_valf();
        lse2[nb] = l != -__builtin_huge_valf() ? l * kLog2eB : __builtin_huge_valf();
        dvec[nb] = row < N ? a.dvec[(size_t)bh * (size_t)N + row] : 0.f;
    }

    // ---- LDS read offsets: K / V fragments along a key row; K^T transposed.
    // At d = 256 the swizzle acts on the low three bits of the 16-byte chunk
    // index only, so an offset 64 columns on is the same one plus 128 bytes:
    // four K offsets and two transposed ones per half, the rest immediates
    // (fewer address registers).
    constexpr int KC = D == 256 ? 4 : NDC, TC = D == 256 ? 2 : NDB;
    uint32_t koff[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = SW::off(lq, 16 * c + 8 * g);
    auto koff_at = [&](int c) { return koff[c % KC] + (uint32_t)(c / KC) * 128u; };
    uint32_t toff[2][TC];
    {
        const int G = lane >> 4, k = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < TC; ++db)
                toff[hf][db] = SW::off(8 * hf + 4 * (G >> 1) + k, 32 * db + 16 * (G & 1) + 4 * j);
    }
    auto toff_at = [&](int hf, int db) { return toff[hf][db % TC] + (uint32_t)(db / TC) * 128u; };
    // ---- tile loads (bounded buffer loads straight into LDS).  Load
    // instruction i of a wavefront is the tile's 1 KB chunk c = wave + i NW,
    // lane l filling 16-byte position p = 64 c + l (row p / CPR).  Where
    // chunks hold whole rows, instruction i fills rows R0 + i RSTEP; the
    // swizzle repeats every 16 rows, so where RSTEP is a multiple of 16 one
    // lane offset serves every instruction (the row step goes into the scalar
    // offset), otherwise (d = 96, 256) each has its own.  At d = 96 a tile is
    // six chunks: waves 0 and 1 issue two, waves 2 and 3 one.
    constexpr bool ALIGNED = kWave % SW::CPR == 0;
    constexpr int RSTEP = ALIGNED ? NW * kWave / SW::CPR : 0;
    constexpr bool ONE_OFF = ALIGNED && RSTEP % 16 == 0;
    const int R0 = (wave * kWave + lane) / SW::CPR;
    uint32_t lane_boff[ONE_OFF ? 1 : LOADS];
#pragma unroll
    for (int i = 0; i < (ONE_OFF ? 1 : LOADS); ++i) {
        if constexpr (ALIGNED) {
            const uint32_t r = (uint32_t)(R0 + i * RSTEP);
            lane_boff[i] = (r * D + (((uint32_t)lane % SW::CPR) ^ SW::f(r)) * 8) * 2;
        } else {
            const uint32_t pos = (uint32_t)((wave + i * NW) * kWave + lane);
            const uint32_t r = pos / SW::CPR;
            lane_boff[i] = (r * D + ((pos % SW::CPR) ^ SW::f(r)) * 8) * 2;
        }
    }
    const uint32_t head_bytes = (uint32_t)Nk * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, head_bytes), vrs = make_rsrc(Vg, head_bytes);
    auto load_part = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf, int i) {
        if (CHUNKS % NW != 0 && wave + i * NW >= CHUNKS) return;   // (wave-uniform)
        if constexpr (ONE_OFF)
            buf2lds16(rs, lane_boff[0], (uint32_t)(t * BC + i * RSTEP) * (uint32_t)(D * 2),
                      buf + (wave + i * NW) * (kWave * 16));
        else
            buf2lds16(rs, lane_boff[i], (uint32_t)(t * BC) * (uint32_t)(D * 2),
                      buf + (wave + i * NW) * (kWave * 16));
    };

    auto tiles_to = [&](int64_t end) {
        end = end < Nk ? end : Nk;
        return end > 0 ? (int)((end + BC - 1) / BC) : 0;
    };
    const int NT = tiles_to(CAUSAL ? (int64_t)q0 + BQ + off : (int64_t)Nk);
    const int Tw = tiles_to(CAUSAL ? (int64_t)q0w + RW + off : (int64_t)Nk);

    const float sl2 = a.scale_log2;
    f32x16 dq[NDB][NRB];
#pragma unroll
    for (int nb = 0; nb < NRB; ++nb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db][nb] = f32x16{};

    // Scores of block nb of tile t set to -inf where masked (edge tiles).
    auto is_edge = [&](int t, int nb) {
        return (t * BC + BC > Nk) || (CAUSAL && t * BC + BC - 1 > q0w + 32 * nb + off);
    };
    auto apply_mask = [&](f32x16 &s, int t, int nb) {
        const int k0 = t * BC;
        int lim = Nk - 1 - (k0 + 4 * g);
        if (CAUSAL) {
            const int64_t c = (int64_t)q0w + 32 * nb + lq + off - (k0 + 4 * g);
            lim = c < lim ? (int)(c > -64 ? c : -64) : lim;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r / 4) + (r % 4);
            if (kk > lim) s[r] = kNegInf;
        }
    };
    // Keep masks of a row block's eight register pairs (keep_masks_from_blocks).
    struct KeepM { uint32_t m[8]; };
    // dS of pair i (registers 2i, 2i+1) of one row block, packed.
    auto ds_pair = [&](const f32x16 &s, const f32x16 &dp, const KeepM &keep, int nb, int i) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 2 * i + e;
            const float p = fast_exp2(fmaf(s[r], sl2, -lse2[nb]));
            float dpv = dp[r];
            if (DROPOUT) {
                // the 16-bit mask of register r = 2i + e (half e of pair i)
                // sign-extended to 32 bits: dP or +0.
                const uint32_t m = e ? (uint32_t)((int)keep.m[i] >> 16)
                                     : (uint32_t)__builtin_amdgcn_sbfe((int)keep.m[i], 0, 16);
                dpv = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, dpv) & m);
            }
            ds[e] = p * (dpv - dvec[nb]);
        }
        uint32_t v = pack2<T>(ds[0], ds[1]);
        pin_vgpr(v);   // keeps the work in its group (no sinking)
        return v;
    };
    // The keep decisions of block nb of tile t, drawn in stages: counters,
    // then 20 block-rounds in order (unit u: round u/2 of block u%2), then
    // the masks, so that the rounds can sit between the dQ products, which
    // have no other VALU work.
    struct KeepDraw { Philox4 c[2]; };
    auto keep_begin = [&](KeepDraw &k, int t, int nb) {
        const uint32_t grp = (uint32_t)((t * BC) >> 3) + 2 * (uint32_t)g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            k.c[h].x[0] = grp + h;
            k.c[h].x[1] = (uint32_t)(q0w + 32 * nb + lq);
            k.c[h].x[2] = h_idx;
            k.c[h].x[3] = b_idx;
        }
    };
    auto keep_rounds = [&](KeepDraw &k, int u0, int u1) {
#pragma unroll
        for (int u = u0; u < u1; ++u) philox_round<true>(k.c[u & 1], u >> 1, a.seed_lo, a.seed_hi);
        if (u1 > u0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                // d <= 128: not after a block's first generator round (two
                // of its words are then loop-invariant, and a pin would copy
                // them; 0.4-1.6 % faster); the d = 256 kernel keeps every
                // pin (1.2 % slower without)
                if (NRB == 1 || (u1 + 1 - h) / 2 >= 2)
#pragma unroll
                    for (int q = 0; q < 4; ++q) pin_vgpr(k.c[h].x[q]);
        }
    };
    const uint32_t kc2 = keep_cmp_const(a.drop_T);
    auto keep_end = [&](KeepDraw &k) {
        KeepM km;
        keep_masks_from_blocks(k.c[0], k.c[1], kc2, km.m);
        return km;
    };

    // Scores of the lane's blocks: `cur` = the block being produced, `prv`
    // = the block whose dS is being formed.
    f32x16 s_a, dp_a, s_b, dp_b;
    uint32_t dsa[8], dsb[8];
    KeepM keep_a, keep_b;
#pragma unroll
    for (int i = 0; i < 8; ++i) keep_a.m[i] = keep_b.m[i] = 0xFFFFFFFFu;

    // 1x: S and dP of block nb of tile t (slot sl), interleaved with the dS
    // pairs of another block (sp/dpp, results into dso); loads of tile
    // t + 1 are spread over the groups.
    auto phase1 = [&](auto nb_c, auto sl_c, auto ds_c, auto ld_c, f32x16 &s, f32x16 &dp,
                      const f32x16 &sp, const f32x16 &dpp, const KeepM &keep_p, int nbp, uint32_t (&dso)[8],
                      int t, auto sln_c) {
        constexpr int NB_ = decltype(nb_c)::value, SL = decltype(sl_c)::value, SLN = decltype(sln_c)::value;
        constexpr bool do_ds = decltype(ds_c)::value, do_load = decltype(ld_c)::value;
        const lds_char *kb = kbuf(SL), *vb = vbuf(SL);
        s = f32x16{};
        dp = f32x16{};
        frag_t<T> kf[2], vf[2];
        kf[0] = lds_frag<T>(kb + koff_at(0));
        vf[0] = lds_frag<T>(vb + koff_at(0));
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            if (c + 1 < NDC) {
                kf[(c + 1) & 1] = lds_frag<T>(kb + koff_at(c + 1));
                vf[(c + 1) & 1] = lds_frag<T>(vb + koff_at(c + 1));
            }
            mma(s, kf[c & 1], qf[NB_][c]);
            if (do_ds) {
#pragma unroll
                for (int i = (c * 8) / NDC; i < ((c + 1) * 8) / NDC; ++i)
                    dso[i] = ds_pair(sp, dpp, keep_p, nbp, i);
            }
            mma(dp, vf[c & 1], df[NB_][c]);
            if (do_load && c < LOADS) load_part(krs, t + 1, kbuf(SLN), c);
            if (do_load && c >= NDC - LOADS && c - (NDC - LOADS) < LOADS)
                load_part(vrs, t + 1, vbuf(SLN), c - (NDC - LOADS));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // 3x: dQ^T of block nb += K^T dS^T with K of slot sl, one product per
    // group with its K^T fragment read two groups ahead; the block-rounds of
    // a keep draw (kd, if any) are spread over the groups.
    auto phase3 = [&](auto nb_c, auto sl_c, const uint32_t (&dsv)[8], auto kd_c, KeepDraw &kd) {
        constexpr int NB_ = decltype(nb_c)::value, SL = decltype(sl_c)::value;
        constexpr bool KD = decltype(kd_c)::value;
        constexpr int NJ = 2 * NDB;
        const lds_char *kb = kbuf(SL);
        auto ktfrag = [&](int j) {
            const int cc = j / NDB, db = j % NDB;
            const uint32_t kc_off = (uint32_t)(16 * cc * RB);
            return join<T>(lds_half_tr<T>(kb + kc_off + toff_at(0, db)),
                           lds_half_tr<T>(kb + kc_off + toff_at(1, db)));
        };
        frag_t<T> kt[3];
        kt[0] = ktfrag(0);
        kt[1] = ktfrag(1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int cc = j / NDB, db = j % NDB;
            if (j + 2 < NJ) kt[(j + 2) % 3] = ktfrag(j + 2);
            if (DROPOUT && KD) keep_rounds(kd, (20 * j) / NJ, (20 * (j + 1)) / NJ);
            u32x4 pv;
            pv[0] = dsv[4 * cc + 0];
            pv[1] = dsv[4 * cc + 1];
            pv[2] = dsv[4 * cc + 2];
            pv[3] = dsv[4 * cc + 3];
            mma(dq[db][NB_], kt[j % 3], __builtin_bit_cast(frag_t<T>, pv));
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    using YES = std::true_type;
    using NO = std::false_type;

    // One step for tile t in slot SL (previous tile in slot SP, next in SN);
    // HP: there is a previous tile (t > 0).  The loads of tile t+1 are
    // unconditional: past the sequence end they read zeros, and the slot
    // they fill is free.
    auto step = [&](auto hp_c, auto sl_c, auto sp_c, auto sn_c, int t) {
        constexpr bool HP = decltype(hp_c)::value;
        // 1a: block a of tile t | dS of block b of tile t-1 | loads of tile t+1.
        phase1(I0{}, sl_c, hp_c, YES{}, s_a, dp_a, s_b, dp_b, keep_b, 1, dsb, t, sn_c);
        if (is_edge(t, 0)) apply_mask(s_a, t, 0);
        // 3b: dQ of block b with tile t-1 | keep bits of block a of tile t.
        KeepDraw kd;
        if (DROPOUT) keep_begin(kd, t, 0);
        if (HP) phase3(I1{}, sp_c, dsb, YES{}, kd);
        else if (DROPOUT) keep_rounds(kd, 0, 20);
        if (DROPOUT) keep_a = keep_end(kd);
        // 1b: block b of tile t | dS of block a of tile t.
        phase1(I1{}, sl_c, YES{}, NO{}, s_b, dp_b, s_a, dp_a, keep_a, 0, dsa, t, sn_c);
        if (is_edge(t, 1)) apply_mask(s_b, t, 1);
        // 3a: dQ of block a with tile t | keep bits of block b of tile t.
        if (DROPOUT) keep_begin(kd, t, 1);
        phase3(I0{}, sl_c, dsa, YES{}, kd);
        if (DROPOUT) keep_b = keep_end(kd);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile t+1 landed
        __syncthreads();                 // everyone's; slot of tile t-2 free
    };

    // ---- prologue: tile 0.
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        load_part(krs, 0, kbuf(0), i);
        load_part(vrs, 0, vbuf(0), i);
    }
    // Q and dO into AGPRs once all loads are in flight (a pin waits for its load).
#pragma unroll
    for (int nb = 0; nb < NRB; ++nb)
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            if constexpr (NRB == 2) {
                pin_agpr(qf[nb][c]);
                pin_agpr(df[nb][c]);
            } else {   // d = 256: the accumulators take the AGPRs
                pin_vgpr(qf[nb][c]);
                pin_vgpr(df[nb][c]);
            }
        }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    int t = 0;
    if constexpr (NRB == 2) {
        if (Tw > 0) { step(NO{}, I0{}, I2{}, I1{}, 0); t = 1; }
        for (; t + 3 <= Tw; t += 3) {
            step(YES{}, I1{}, I0{}, I2{}, t);
            step(YES{}, I2{}, I1{}, I0{}, t + 1);
            step(YES{}, I0{}, I2{}, I1{}, t + 2);
        }
        if (t < Tw) { step(YES{}, I1{}, I0{}, I2{}, t); ++t; }
        if (t < Tw) { step(YES{}, I2{}, I1{}, I0{}, t); ++t; }
        // dQ of block b of the last tile (its dS is formed here, not in a next step).
        if (Tw > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) dsb[i] = ds_pair(s_b, dp_b, keep_b, 1, i);
            const int sl = (Tw - 1) % 3;
            KeepDraw none;
            if (sl == 0) phase3(I1{}, I0{}, dsb, NO{}, none);
            else if (sl == 1) phase3(I1{}, I1{}, dsb, NO{}, none);
            else phase3(I1{}, I2{}, dsb, NO{}, none);
        }
    } else if constexpr (CAUSAL && DROPOUT) {
        // One block per wavefront, causal with dropout: step t forms S and
        // dP of tile t, then dS of tile t and dQ^T += K^T dS^T of tile t, so
        // one score buffer suffices; the keep bits of tile t+1 are drawn
        // during the dQ products.  With the extra live values of dropout and
        // the causal edge masks, a second score buffer (the overlap below)
        // spilled, and this order measured faster: 2.52 -> 2.20 ms on
        // 4 x 32 x 4096 x 256; without dropout, or non-causal, the overlap
        // is faster (1.93 against 2.05 ms, 1.88 against 1.98 ms).  Slots of
        // tiles rotate with period 3, so each step is one of three shapes,
        // picked by a scalar branch.
        KeepM keep_c = keep_a;
        if (Tw > 0) {
            KeepDraw k0;
            keep_begin(k0, 0, 0);
            keep_rounds(k0, 0, 20);
            keep_c = keep_end(k0);
        }
        // (inlined by force: as calls, the arrays they touch would live in
        // scratch memory)
        auto step1 = [&](auto sl_c, auto sn_c, int tt) __attribute__((always_inline)) {
            // 1: S, dP of tile tt | loads of tile tt+1.
            phase1(I0{}, sl_c, NO{}, YES{}, s_a, dp_a, s_a, dp_a, keep_c, 0, dsa, tt, sn_c);
            if (is_edge(tt, 0)) apply_mask(s_a, tt, 0);
            // 2: dS of tile tt.
#pragma unroll
            for (int i = 0; i < 8; ++i) dsa[i] = ds_pair(s_a, dp_a, keep_c, 0, i);
            // 3: dQ with tile tt | keep bits of tile tt+1.
            KeepDraw kd;
            keep_begin(kd, tt + 1, 0);
            phase3(I0{}, sl_c, dsa, YES{}, kd);
            keep_c = keep_end(kd);
            __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile tt+1 landed
            __syncthreads();                 // everyone's; slot of tile tt-2 free
        };
        for (; t < Tw; ++t) {
            switch (t % 3) {
            case 0: step1(I0{}, I1{}, t); break;
            case 1: step1(I1{}, I2{}, t); break;
            default: step1(I2{}, I0{}, t); break;
            }
        }
    } else {
        // One block per wavefront: step t produces the scores of tile t in
        // (s_a, dp_a) and forms dS of tile t-1 from (s_b, dp_b), then moves
        // the new scores over (alternating the two by parity as well would
        // need more registers than there are); slots of tiles rotate with
        // period 3, so each step is one of three shapes, picked by a scalar
        // branch.
        // (inlined by force: as calls, the arrays they touch would live in
        // scratch memory)
        auto step1p = [&](auto hp_c, auto sl_c, auto sp_c, auto sn_c, f32x16 &s_c, f32x16 &dp_c,
                          const f32x16 &s_p, const f32x16 &dp_p, const KeepM &keep_p, KeepM &keep_c,
                          int tt) __attribute__((always_inline)) {
            constexpr bool HP = decltype(hp_c)::value;
            // 1: tile tt | dS of tile tt-1 | loads of tile tt+1.
            phase1(I0{}, sl_c, hp_c, YES{}, s_c, dp_c, s_p, dp_p, keep_p, 0, dsa, tt, sn_c);
            if (is_edge(tt, 0)) apply_mask(s_c, tt, 0);
            // 3: dQ with tile tt-1 | keep bits of tile tt.
            KeepDraw kd;
            if (DROPOUT) keep_begin(kd, tt, 0);
            if (HP) phase3(I0{}, sp_c, dsa, YES{}, kd);
            else if (DROPOUT) keep_rounds(kd, 0, 20);
            if (DROPOUT) keep_c = keep_end(kd);
            __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile tt+1 landed
            __syncthreads();                 // everyone's; slot of tile tt-2 free
        };
        auto step1 = [&](auto hp_c, auto sl_c, auto sp_c, auto sn_c, int tt) __attribute__((always_inline)) {
            step1p(hp_c, sl_c, sp_c, sn_c, s_a, dp_a, s_b, dp_b, keep_b, keep_a, tt);
            s_b = s_a;
            dp_b = dp_a;
            keep_b = keep_a;
        };
        // tile tt: slot tt % 3
        auto step_rt = [&](int tt) {
            switch (tt % 3) {
            case 0: step1(YES{}, I0{}, I2{}, I1{}, tt); break;
            case 1: step1(YES{}, I1{}, I0{}, I2{}, tt); break;
            default: step1(YES{}, I2{}, I1{}, I0{}, tt); break;
            }
        };
        if (Tw > 0) { step1(NO{}, I0{}, I2{}, I1{}, 0); t = 1; }
        for (; t < Tw; ++t) step_rt(t);
        // dQ of the last tile (its dS is formed here, not in a next step).
        if (Tw > 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) dsa[i] = ds_pair(s_b, dp_b, keep_b, 0, i);
            const int sl = (Tw - 1) % 3;
            KeepDraw none;
            if (sl == 0) phase3(I0{}, I0{}, dsa, NO{}, none);
            else if (sl == 1) phase3(I0{}, I1{}, dsa, NO{}, none);
            else phase3(I0{}, I2{}, dsa, NO{}, none);
        }
    }
    // Tiles beyond this wavefront's rows: keep the workgroup's loads and barriers in step.
    for (; t < NT; ++t) {
        if (t + 1 < NT) {
            const int sn = (t + 1) % 3;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                load_part(krs, t + 1, kbuf(sn), i);
                load_part(vrs, t + 1, vbuf(sn), i);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: dQ = scale c (dQ/c)^T^T (c = 1 without dropout).
    const float qsc = DROPOUT ? a.scale * a.drop_c : a.scale;
#pragma unroll
    for (int nb = 0; nb < NRB; ++nb) {
        const int qrow = q0w + 32 * nb + lq;
        if (qrow < N) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr + 4 * g;
                    const float x0 = qsc * dq[db][nb][4 * rr + 0], x1 = qsc * dq[db][nb][4 * rr + 1];
                    const float x2 = qsc * dq[db][nb][4 * rr + 2], x3 = qsc * dq[db][nb][4 * rr + 3];
                    if (a.out_f32)
                        store4<float>(reinterpret_cast<float *>(a.dq) + head + (size_t)qrow * D + col, x0, x1, x2, x3);
                    else
                        store4<T>(reinterpret_cast<T *>(a.dq) + head + (size_t)qrow * D + col, x0, x1, x2, x3);
                }
        }
    }
}

template <typename T, int D>
inline hipError_t launch_dq16_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = Dq16Tile<T, D>;
    const int64_t nqb = (a.N + TL::BQ - 1) / TL::BQ;
    const int64_t units = a.B * a.H * nqb;
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    BwdArgs b = a;
    b.group = unit_group(a.B * a.H, nqb, 1);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((dq16_kernel<T, D, true, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((dq16_kernel<T, D, true, false>), grid, block, 0, stream, b);
    } else {
        if (dropout) hipLaunchKernelGGL((dq16_kernel<T, D, false, true>), grid, block, 0, stream, b);
        else hipLaunchKernelGGL((dq16_kernel<T, D, false, false>), grid, block, 0, stream, b);
    }
    return hipGetLastError();
}

}  // namespace fa
