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
#include <type_traits>

#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

namespace {
constexpr float kLog2eB = 1.44269504088896340736f;
}

template <typename T, int D>
struct Dq16Tile {
    static constexpr int NW = 4;                  // wavefronts per workgroup
    static constexpr int RW = 64;                 // query rows per wavefront
    static constexpr int BQ = NW * RW;            // query rows per workgroup
    static constexpr int BC = 32;                 // keys per step
    static constexpr int THREADS = NW * kWave;
    static constexpr int TILE_BYTES = BC * D * 2;
    static constexpr int LOADS = TILE_BYTES / (kWave * 16) / NW;   // per wave per tile
    static constexpr int RING = 3;                // LDS buffers per tensor
};

template <typename T, int D, bool CAUSAL, bool DROPOUT>
__global__ void __launch_bounds__(256, 1) dq16_kernel(const BwdArgs a) {
    using TL = Dq16Tile<T, D>;
    using SW = Swz<D>;
    constexpr int NW = TL::NW, RW = TL::RW, BQ = TL::BQ, BC = TL::BC;
    constexpr int TB = TL::TILE_BYTES, LOADS = TL::LOADS;
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
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int64_t qb = CAUSAL ? (nqb - 1 - u / BH) : (u / BH);
    const int N = (int)a.N;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int q0 = (int)qb * BQ;
    const int q0w = q0 + wave * RW;

    // ---- Q and dO fragments (B operands, one query row per lane), in AGPRs;
    // log2-scaled LSE and D of the lane's two rows (rows past N: P = 0).
    frag_t<T> qf[2][NDC], df[2][NDC];
    float lse2[2], dvec[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int row = q0w + 32 * nb + lq;
        const int r = row < N ? row : N - 1;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            qf[nb][c] = load_frag<T>(Qg + (size_t)r * D + 16 * c + 8 * g);
            df[nb][c] = load_frag<T>(dOg + (size_t)r * D + 16 * c + 8 * g);
            pin_agpr(qf[nb][c]);
            pin_agpr(df[nb][c]);
        }
        lse2[nb] = row < N ? a.lse[(size_t)bh * (size_t)N + row] * kLog2eB : __builtin_huge_valf();
        dvec[nb] = row < N ? a.dvec[(size_t)bh * (size_t)N + row] : 0.f;
    }

    // ---- LDS read offsets: K / V fragments along a key row; K^T transposed.
    uint32_t koff[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c) koff[c] = SW::off(lq, 16 * c + 8 * g);
    uint32_t toff[2][NDB];
    {
        const int G = lane >> 4, k = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                toff[hf][db] = SW::off(8 * hf + 4 * (G >> 1) + k, 32 * db + 16 * (G & 1) + 4 * j);
    }
    // ---- tile loads (bounded buffer loads straight into LDS).
    constexpr int RSTEP = NW * kWave / SW::CPR;
    const int R0 = (wave * kWave + lane) / SW::CPR;
    const uint32_t gcol = (uint32_t)(((lane % SW::CPR) ^ (int)SW::f(R0)) * 8);
    const uint32_t lane_boff = ((uint32_t)R0 * D + gcol) * 2;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kg, head_bytes), vrs = make_rsrc(Vg, head_bytes);
    auto load_part = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf, int i) {
        buf2lds16(rs, lane_boff, (uint32_t)((t * BC + i * RSTEP) * D * 2),
                  buf + (wave + i * NW) * (kWave * 16));
    };

    const int kend = CAUSAL ? (q0 + BQ < N ? q0 + BQ : N) : N;
    const int NT = (kend + BC - 1) / BC;
    const int wend = CAUSAL ? (q0w + RW < N ? q0w + RW : N) : N;
    const int Tw = (wend + BC - 1) / BC;

    const float sl2 = a.scale_log2, dc = a.drop_c;
    f32x16 dq[NDB][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db][nb] = f32x16{};

    // Scores of block nb of tile t set to -inf where masked (edge tiles).
    auto is_edge = [&](int t, int nb) {
        return (t * BC + BC > N) || (CAUSAL && t * BC + BC - 1 > q0w + 32 * nb);
    };
    auto apply_mask = [&](f32x16 &s, int t, int nb) {
        const int k0 = t * BC;
        int lim = N - 1 - (k0 + 4 * g);
        if (CAUSAL) {
            const int c = q0w + 32 * nb + lq - (k0 + 4 * g);
            lim = c < lim ? c : lim;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r / 4) + (r % 4);
            if (kk > lim) s[r] = kNegInf;
        }
    };
    // dS of pair i (registers 2i, 2i+1) of one row block, packed.
    auto ds_pair = [&](const f32x16 &s, const f32x16 &dp, uint32_t keep, int nb, int i) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 2 * i + e;
            const float p = fast_exp2(fmaf(s[r], sl2, -lse2[nb]));
            float dpv = dp[r];
            if (DROPOUT) dpv = ((keep >> r) & 1u) ? dpv * dc : 0.f;
            ds[e] = p * (dpv - dvec[nb]);
        }
        uint32_t v = pack2<T>(ds[0], ds[1]);
        pin_vgpr(v);   // keeps the work in its group (no sinking)
        return v;
    };
    auto keep_of = [&](int t, int nb) -> uint32_t {
        if (!DROPOUT) return 0xFFFFu;
        return keep_bits_row((uint32_t)(t * BC), (uint32_t)(q0w + 32 * nb + lq), h_idx, b_idx,
                             a.seed_lo, a.seed_hi, a.drop_T);
    };

    // Scores of the lane's blocks: `cur` = the block being produced, `prv`
    // = the block whose dS is being formed.
    f32x16 s_a, dp_a, s_b, dp_b;
    uint32_t dsa[8], dsb[8];
    uint32_t keep_a = 0xFFFFu, keep_b = 0xFFFFu;

    // 1x: S and dP of block nb of tile t (slot sl), interleaved with the dS
    // pairs of another block (sp/dpp, results into dso); loads of tile
    // t + 1 are spread over the groups.
    auto phase1 = [&](auto nb_c, auto sl_c, auto ds_c, auto ld_c, f32x16 &s, f32x16 &dp,
                      const f32x16 &sp, const f32x16 &dpp, uint32_t keep_p, int nbp, uint32_t (&dso)[8],
                      int t, auto sln_c) {
        constexpr int NB_ = decltype(nb_c)::value, SL = decltype(sl_c)::value, SLN = decltype(sln_c)::value;
        constexpr bool do_ds = decltype(ds_c)::value, do_load = decltype(ld_c)::value;
        const lds_char *kb = kbuf(SL), *vb = vbuf(SL);
        s = f32x16{};
        dp = f32x16{};
        frag_t<T> kf[2], vf[2];
        kf[0] = lds_frag<T>(kb + koff[0]);
        vf[0] = lds_frag<T>(vb + koff[0]);
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            if (c + 1 < NDC) {
                kf[(c + 1) & 1] = lds_frag<T>(kb + koff[c + 1]);
                vf[(c + 1) & 1] = lds_frag<T>(vb + koff[c + 1]);
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
    // 3x: dQ^T of block nb += K^T dS^T with K of slot sl.
    auto phase3 = [&](auto nb_c, auto sl_c, const uint32_t (&dsv)[8]) {
        constexpr int NB_ = decltype(nb_c)::value, SL = decltype(sl_c)::value;
        const lds_char *kb = kbuf(SL);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            u32x4 pv;
            pv[0] = dsv[4 * cc + 0];
            pv[1] = dsv[4 * cc + 1];
            pv[2] = dsv[4 * cc + 2];
            pv[3] = dsv[4 * cc + 3];
            const frag_t<T> sf = __builtin_bit_cast(frag_t<T>, pv);
            const uint32_t kc_off = (uint32_t)(16 * cc * RB);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const frag_t<T> kt = join<T>(lds_half_tr<T>(kb + kc_off + toff[0][db]),
                                             lds_half_tr<T>(kb + kc_off + toff[1][db]));
                mma(dq[db][NB_], kt, sf);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
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
        if (DROPOUT) keep_a = keep_of(t, 0);
        // 3b: dQ of block b with tile t-1.
        if (HP) phase3(I1{}, sp_c, dsb);
        // 1b: block b of tile t | dS of block a of tile t.
        phase1(I1{}, sl_c, YES{}, NO{}, s_b, dp_b, s_a, dp_a, keep_a, 0, dsa, t, sn_c);
        if (is_edge(t, 1)) apply_mask(s_b, t, 1);
        if (DROPOUT) keep_b = keep_of(t, 1);
        // 3a: dQ of block a with tile t.
        phase3(I0{}, sl_c, dsa);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile t+1 landed
        __syncthreads();                 // everyone's; slot of tile t-2 free
    };

    // ---- prologue: tile 0.
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        load_part(krs, 0, kbuf(0), i);
        load_part(vrs, 0, vbuf(0), i);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    int t = 0;
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
        if (sl == 0) phase3(I1{}, I0{}, dsb);
        else if (sl == 1) phase3(I1{}, I1{}, dsb);
        else phase3(I1{}, I2{}, dsb);
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

    // ---- epilogue: dQ = scale * dQ^T^T.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int qrow = q0w + 32 * nb + lq;
        if (qrow < N) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr + 4 * g;
                    const float x0 = a.scale * dq[db][nb][4 * rr + 0], x1 = a.scale * dq[db][nb][4 * rr + 1];
                    const float x2 = a.scale * dq[db][nb][4 * rr + 2], x3 = a.scale * dq[db][nb][4 * rr + 3];
                    if (a.out_f32)
                        store4<float>(reinterpret_cast<float *>(a.dq) + head + (size_t)qrow * D + col, x0, x1, x2, x3);
                    else
                        store4<T>(reinterpret_cast<T *>(a.dq) + head + (size_t)qrow * D + col, x0, x1, x2, x3);
                }
        }
    }
}

// ===================================================================
// dK and dV.
//
// One workgroup owns 128 keys: two pairs of wavefronts, each pair 64 keys.
// The four products of the backward are split between the two wavefronts
// of a pair, so that each holds only one 128x64 accumulator (dV^T or dK^T,
// keys along the lanes) besides its operands:
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
// tile, half by each wavefront of the pair, as 16-bit masks in a row-major
// LDS block; the transposed 16-bit LDS read hands every lane the masks of
// its own (key, rows) registers, already paired as the products need them.
// Per 32-row step t:
//   A: S of tile t, P of tile t (to LDS), dV += dO^T (keep P) of tile t;
//   B: dS of tile t-1 from its dP and A's P, dK += Q^T dS, dP of tile t;
// so B reads A's P one step after it was written (one barrier per step).
// Tile t's Q is read by A in step t and by B in step t+1 (four LDS
// buffers); dO tiles are read in one step (two buffers).
template <typename T, int D>
struct Dkdv16Tile {
    static constexpr int NW = 4;                       // 2 pairs x (A, B)
    static constexpr int KP = 64;                      // keys per pair
    static constexpr int BK = 2 * KP;                  // keys per workgroup
    static constexpr int BQ = 32;                      // query rows per step
    static constexpr int THREADS = NW * kWave;
    static constexpr int TB = BQ * D * 2;              // bytes of a Q or dO tile
    static constexpr int LOADS = TB / (kWave * 16) / NW;
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
    constexpr int NW = TL::NW, KP = TL::KP, BK = TL::BK, BQ = TL::BQ;
    constexpr int TB = TL::TB, LOADS = TL::LOADS;
    constexpr int RB = SW::ROW_BYTES;
    constexpr int NDC = D / 16;
    constexpr int NDB = D / 32;
    constexpr float kNegInf = -__builtin_huge_valf();
    static_assert(LOADS >= 1, "tile load split");

    __shared__ __attribute__((aligned(1024))) char qs0[TB], qs1[TB], qs2[TB], qs3[TB], os0[TB], os1[TB];
    __shared__ __attribute__((aligned(256))) float lse_s[2][64];
    __shared__ __attribute__((aligned(256))) float dv_s[4][64];
    __shared__ __attribute__((aligned(1024))) float pex[2][2][32 * 64];   // [slot][pair][regs x lanes]
    // Dropout keep masks: 16-bit 0x0000 / 0xFFFF per (row, key) of a pair's
    // 32 x 64 block, row-major with a 192-byte row pitch (conflict-free for
    // the transposed reads); four tiles in flight.
    constexpr int MP = 192;
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
    const int64_t u = blockIdx.x;
    const int64_t bh = u % BH;
    const int kblk = (int)(u / BH);                       // causal: low key blocks (most work) first
    const int N = (int)a.N;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T *__restrict__ Qg = reinterpret_cast<const T *>(a.q) + head;
    const T *__restrict__ Kg = reinterpret_cast<const T *>(a.k) + head;
    const T *__restrict__ Vg = reinterpret_cast<const T *>(a.v) + head;
    const T *__restrict__ dOg = reinterpret_cast<const T *>(a.dout) + head;
    const uint32_t b_idx = (uint32_t)(bh / a.H), h_idx = (uint32_t)(bh % a.H);

    const int k0 = kblk * BK;                 // first key of the workgroup
    const int kp0 = k0 + pair * KP;           // first key of this pair
    const int j0 = CAUSAL ? k0 / BQ : 0;      // first query tile
    const int NTQ = (N + BQ - 1) / BQ - j0;   // query tiles streamed

    // ---- the pair's K (A) or V (B) rows: B operands, one key per lane, in AGPRs.
    frag_t<T> kv[2][NDC];
    {
        const T *src = role == 0 ? Kg : Vg;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            int key = kp0 + 32 * kb + lq;
            key = key < N ? key : N - 1;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                kv[kb][c] = load_frag<T>(src + (size_t)key * D + 16 * c + 8 * g);
                pin_agpr(kv[kb][c]);
            }
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
    // each), LSE rows (the A wavefronts) and D rows (the B wavefronts).
    constexpr int RSTEP = NW * kWave / SW::CPR;
    const int R0 = (wave * kWave + lane) / SW::CPR;
    const uint32_t gcol = (uint32_t)(((lane % SW::CPR) ^ (int)SW::f(R0)) * 8);
    const uint32_t lane_boff = ((uint32_t)R0 * D + gcol) * 2;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qg, head_bytes), ors = make_rsrc(dOg, head_bytes);
    const __amdgpu_buffer_rsrc_t rrs =
        role == 0 ? make_rsrc(a.lse + (size_t)bh * (size_t)N, (uint32_t)N * 4)
                  : make_rsrc(a.dvec + (size_t)bh * (size_t)N, (uint32_t)N * 4);
    auto load_tile_part = [&](__amdgpu_buffer_rsrc_t rs, int t, lds_char *buf, int i) {
        buf2lds16(rs, lane_boff, (uint32_t)(((j0 + t) * BQ + i * RSTEP) * D * 2),
                  buf + (wave + i * NW) * (kWave * 16));
    };
    auto load_rows = [&](int t, lds_char *buf) {   // 64 fp32 rows from the tile's first row
        buf2lds4(rrs, (uint32_t)lane * 4, (uint32_t)((j0 + t) * BQ) * 4, buf);
    };
    // Loads issued during step s: Q, dO and LSE/D rows of tile s+1.
    auto issue_loads = [&](int s, int qsl, int osl, int rsl2, int rsl4) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            load_tile_part(qrs, s + 1, qbuf(qsl), i);
            load_tile_part(ors, s + 1, obuf(osl), i);
        }
        if (role == 0) load_rows(s + 1, (lds_char *)lse_s[rsl2]);
        else load_rows(s + 1, (lds_char *)dv_s[rsl4]);
    };

    const float sl2 = a.scale_log2, dc = a.drop_c;
    f32x16 acc[NDB][2];          // dV^T (A) or dK^T (B): [d block][key block]
#pragma unroll
    for (int db = 0; db < NDB; ++db) { acc[db][0] = f32x16{}; acc[db][1] = f32x16{}; }

    // Masking of tile t for this pair: key > query (causal), key >= N, row >= N.
    auto is_edge = [&](int t) {
        const int qt0 = (j0 + t) * BQ;
        return (qt0 + BQ > N) || (kp0 + KP > N) || (CAUSAL && kp0 + KP - 1 > qt0);
    };
    auto apply_mask = [&](f32x16 (&s)[2], int t) {
        const int qt0 = (j0 + t) * BQ;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = kp0 + 32 * kb + lq;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = qt0 + 8 * (r / 4) + 4 * g + (r % 4);
                if ((CAUSAL && key > q) || key >= N || q >= N) s[kb][r] = kNegInf;
            }
        }
    };

    // Keep masks of key block kb of this pair for tile t: lane (row lq,
    // half g) draws the 16 keys 32kb + 16g .. +15 of its row (two Philox
    // blocks) and stores them as 16-bit masks.
    auto gen_masks = [&](int t, int kb, int slot) {
        const uint32_t grp = (uint32_t)((kp0 + 32 * kb) >> 3) + 2 * g;
        const uint32_t row = (uint32_t)((j0 + t) * BQ + lq);
        FA_LDS char *p = (FA_LDS char *)mk[slot & (DROPOUT ? 3 : 0)][pair] + lq * MP + (32 * kb + 16 * g) * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Philox4 r = philox4x32_10(grp + h, row, h_idx, b_idx, a.seed_lo, a.seed_hi);
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)   // word q: keys 2q (low half), 2q + 1 (high half)
                w[q] = ((r.x[q] & 0xFFFFu) >= a.drop_T ? 0x0000FFFFu : 0u) |
                       ((r.x[q] >> 16) >= a.drop_T ? 0xFFFF0000u : 0u);
            *(FA_LDS u32x4 *)(p + 16 * h) = w;
        }
    };
    // Per-lane byte offset of the transposed mask read: lane receives the
    // masks of rows 8 q4 + 4g + 0..3 (its registers 4 q4 .. 4 q4 + 3) of key
    // 32 kb + lq, with q4 and kb added as immediates.
    const uint32_t mtr = (uint32_t)((4 * ((lane >> 5)) + ((lane >> 2) & 3)) * MP +
                                    (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
    auto read_masks = [&](int slot, int kb, int q4) {
        const half_t<T> m = lds_half_tr<T>((lds_char *)mk[slot & (DROPOUT ? 3 : 0)][pair] + mtr +
                                           (uint32_t)(8 * q4 * MP + 32 * kb * 2));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(u32x2, m);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using YES = std::true_type;
    using NO = std::false_type;
    auto dispatch4 = [&](int r, auto f) {
        switch (r & 3) {
        case 0: f(I0{}); break;
        case 1: f(I1{}); break;
        case 2: f(I2{}); break;
        default: f(I3{}); break;
        }
    };

    // ---- prologue loads: Q_0, dO_0, rows of tile 0.
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        load_tile_part(qrs, 0, qbuf(0), i);
        load_tile_part(ors, 0, obuf(0), i);
    }
    if (role == 0) load_rows(0, (lds_char *)lse_s[0]);
    else load_rows(0, (lds_char *)dv_s[0]);
    if (DROPOUT) gen_masks(0, role, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (role == 0) {
        // ============================== A: S, P, dV ==============================
        f32x16 sacc[2];
        // Step s (R = s % 4): S of tile s (Q slot s%4), P of tile s, dV of
        // tile s (dO slot s%2); loads of tile s+1.
        auto a_step = [&](auto r_c, int s) {
            constexpr int R = decltype(r_c)::value;
            lds_char *qb = qbuf(R);
            lds_char *ob = obuf(R & 1);
            const FA_LDS float *lsep = (const FA_LDS float *)lse_s[R & 1];
            FA_LDS float *px = (FA_LDS float *)pex[R & 1][pair];
            issue_loads(s, (R + 1) & 3, (R + 1) & 1, (R + 1) & 1, 0);

            // ---- S = Q K^T.
            sacc[0] = f32x16{};
            sacc[1] = f32x16{};
            {
                frag_t<T> qf[3];
                qf[0] = lds_frag<T>(qb + roff[0]);
                if (NDC > 1) qf[1] = lds_frag<T>(qb + roff[1]);
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    if (c + 2 < NDC) qf[(c + 2) % 3] = lds_frag<T>(qb + roff[c + 2]);
                    mma(sacc[0], qf[c % 3], kv[0][c]);
                    mma(sacc[1], qf[c % 3], kv[1][c]);
                }
            }
            if (is_edge(s)) apply_mask(sacc, s);

            // ---- P (and keep P) of tile s, 4 registers per group; P goes to B.
            uint32_t pp[2][8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int kb = c >> 2, q4 = c & 3;
                const f32x4 l4 = *(const FA_LDS f32x4 *)(lsep + 8 * q4 + 4 * g);
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pv[e] = fast_exp2(fmaf(sacc[kb][4 * q4 + e], sl2, -l4[e] * kLog2eB));
                f32x4 xo;
#pragma unroll
                for (int e = 0; e < 4; ++e) xo[e] = pv[e];
                pp[kb][2 * q4] = pack2<T>(pv[0], pv[1]);
                pp[kb][2 * q4 + 1] = pack2<T>(pv[2], pv[3]);
                if (DROPOUT) {
                    // keep P: the transposed mask read gives exactly these two pairs.
                    const auto mw = read_masks(R, kb, q4);
                    pp[kb][2 * q4] &= mw[0];
                    pp[kb][2 * q4 + 1] &= mw[1];
                }
                *(FA_LDS f32x4 *)(px + (c * kWave + lane) * 4) = xo;
            }

            // ---- dV^T += dO^T (keep P).
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint32_t kc_off = (uint32_t)(16 * cc * RB);
                    const frag_t<T> ot = join<T>(lds_half_tr<T>(ob + kc_off + toff[0][db]),
                                                 lds_half_tr<T>(ob + kc_off + toff[1][db]));
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        u32x4 pv;
                        pv[0] = pp[kb][4 * cc + 0];
                        pv[1] = pp[kb][4 * cc + 1];
                        pv[2] = pp[kb][4 * cc + 2];
                        pv[3] = pp[kb][4 * cc + 3];
                        mma(acc[db][kb], ot, __builtin_bit_cast(frag_t<T>, pv));
                    }
                }
            if (DROPOUT) gen_masks(s + 1, 0, R + 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };

        for (int s = 0; s < NTQ; s += 4) {
            a_step(I0{}, s);
            if (s + 1 < NTQ) a_step(I1{}, s + 1);
            if (s + 2 < NTQ) a_step(I2{}, s + 2);
            if (s + 3 < NTQ) a_step(I3{}, s + 3);
        }
        // step NTQ: B finishes the last tile; keep the barrier count.
        __syncthreads();
    } else {
        // ============================== B: dP, dS, dK ============================
        f32x16 dacc[2];   // dP of the latest tile
        // Step s (R = s % 4): dS and dK of tile s-1 (P slot (s-1)%2, D slot
        // (s-1)%4, Q slot (s-1)%4), then dP of tile s (dO slot s%2).
        auto b_step = [&](auto r_c, auto hp_c, auto hc_c, int s) {
            constexpr int R = decltype(r_c)::value;
            constexpr bool HP = decltype(hp_c)::value, HC = decltype(hc_c)::value;
            lds_char *ob = obuf(R & 1);
            lds_char *qb = qbuf((R + 3) & 3);
            const FA_LDS float *dvp = (const FA_LDS float *)dv_s[(R + 3) & 3];
            const FA_LDS float *px = (const FA_LDS float *)pex[(R + 1) & 1][pair];
            if (HC) issue_loads(s, (R + 1) & 3, (R + 1) & 1, 0, (R + 1) & 3);

            if (HP) {
                // ---- dS of tile s-1, 4 registers per group.
                uint32_t sp[2][8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int kb = c >> 2, q4 = c & 3;
                    const f32x4 d4 = *(const FA_LDS f32x4 *)(dvp + 8 * q4 + 4 * g);
                    const f32x4 x4 = *(const FA_LDS f32x4 *)(px + (c * kWave + lane) * 4);
                    float ds[4];
                    uint32_t mw2[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
                    if (DROPOUT) {
                        const auto mw = read_masks(R + 3, kb, q4);
                        mw2[0] = mw[0];
                        mw2[1] = mw[1];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dpv = dacc[kb][4 * q4 + e];
                        if (DROPOUT) {
                            // dP * keep * c: the 16-bit mask sign-extended to 32 bits.
                            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)mw2[e >> 1], 16 * (e & 1), 16);
                            const float kd = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, dpv * dc) & m);
                            ds[e] = x4[e] * (kd - d4[e]);
                        } else {
                            ds[e] = x4[e] * (dpv - d4[e]);
                        }
                    }
                    sp[kb][2 * q4] = pack2<T>(ds[0], ds[1]);
                    sp[kb][2 * q4 + 1] = pack2<T>(ds[2], ds[3]);
                }
                // ---- dK^T += Q^T dS.
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const uint32_t kc_off = (uint32_t)(16 * cc * RB);
                        const frag_t<T> qt = join<T>(lds_half_tr<T>(qb + kc_off + toff[0][db]),
                                                     lds_half_tr<T>(qb + kc_off + toff[1][db]));
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            u32x4 pv;
                            pv[0] = sp[kb][4 * cc + 0];
                            pv[1] = sp[kb][4 * cc + 1];
                            pv[2] = sp[kb][4 * cc + 2];
                            pv[3] = sp[kb][4 * cc + 3];
                            mma(acc[db][kb], qt, __builtin_bit_cast(frag_t<T>, pv));
                        }
                    }
            }
            if (HC) {
                // ---- dP of tile s = dO V^T.
                dacc[0] = f32x16{};
                dacc[1] = f32x16{};
                frag_t<T> of[3];
                of[0] = lds_frag<T>(ob + roff[0]);
                if (NDC > 1) of[1] = lds_frag<T>(ob + roff[1]);
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    if (c + 2 < NDC) of[(c + 2) % 3] = lds_frag<T>(ob + roff[c + 2]);
                    mma(dacc[0], of[c % 3], kv[0][c]);
                    mma(dacc[1], of[c % 3], kv[1][c]);
                }
                if (DROPOUT) gen_masks(s + 1, 1, R + 1);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };

        // Steps 0 .. NTQ.  Step NTQ finishes tile NTQ-1; its dP half runs on
        // the zero-filled rows past the last tile (harmless, never used).
        if (NTQ > 0) {
            b_step(I0{}, NO{}, YES{}, 0);
            for (int s = 1; s <= NTQ; s += 4) {
                b_step(I1{}, YES{}, YES{}, s);
                if (s + 1 <= NTQ) b_step(I2{}, YES{}, YES{}, s + 1);
                if (s + 2 <= NTQ) b_step(I3{}, YES{}, YES{}, s + 2);
                if (s + 3 <= NTQ) b_step(I0{}, YES{}, YES{}, s + 3);
            }
        } else {
            __syncthreads();
        }
    }

    // ---- epilogue: dV = c * acc (A), dK = scale * acc (B); keys past N not stored.
    const float osc = role == 0 ? (DROPOUT ? dc : 1.f) : a.scale;
    void *dst = role == 0 ? a.dv : a.dk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = kp0 + 32 * kb + lq;
        if (key < N) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int col = 32 * db + 8 * rr + 4 * g;
                    const float x0 = osc * acc[db][kb][4 * rr + 0], x1 = osc * acc[db][kb][4 * rr + 1];
                    const float x2 = osc * acc[db][kb][4 * rr + 2], x3 = osc * acc[db][kb][4 * rr + 3];
                    if (a.out_f32)
                        store4<float>(reinterpret_cast<float *>(dst) + head + (size_t)key * D + col, x0, x1, x2, x3);
                    else
                        store4<T>(reinterpret_cast<T *>(dst) + head + (size_t)key * D + col, x0, x1, x2, x3);
                }
        }
    }
}

template <typename T, int D>
static hipError_t launch_dkdv16_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = Dkdv16Tile<T, D>;
    const int64_t units = a.B * a.H * ((a.N + TL::BK - 1) / TL::BK);
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((dkdv16_kernel<T, D, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dkdv16_kernel<T, D, true, false>), grid, block, 0, stream, a);
    } else {
        if (dropout) hipLaunchKernelGGL((dkdv16_kernel<T, D, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dkdv16_kernel<T, D, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                             hipStream_t stream) {
    switch (e) {
    case Elem::BF16:
        return d == 64 ? launch_dkdv16_t<bf16, 64>(causal, dropout, a, stream)
                       : launch_dkdv16_t<bf16, 128>(causal, dropout, a, stream);
    case Elem::F16:
        return d == 64 ? launch_dkdv16_t<f16, 64>(causal, dropout, a, stream)
                       : launch_dkdv16_t<f16, 128>(causal, dropout, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

template <typename T, int D>
static hipError_t launch_dq16_t(bool causal, bool dropout, const BwdArgs &a, hipStream_t stream) {
    using TL = Dq16Tile<T, D>;
    const int64_t units = a.B * a.H * ((a.N + TL::BQ - 1) / TL::BQ);
    if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)units), block(TL::THREADS);
    if (causal) {
        if (dropout) hipLaunchKernelGGL((dq16_kernel<T, D, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dq16_kernel<T, D, true, false>), grid, block, 0, stream, a);
    } else {
        if (dropout) hipLaunchKernelGGL((dq16_kernel<T, D, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((dq16_kernel<T, D, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dq16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                           hipStream_t stream) {
    switch (e) {
    case Elem::BF16:
        return d == 64 ? launch_dq16_t<bf16, 64>(causal, dropout, a, stream)
                       : launch_dq16_t<bf16, 128>(causal, dropout, a, stream);
    case Elem::F16:
        return d == 64 ? launch_dq16_t<f16, 64>(causal, dropout, a, stream)
                       : launch_dq16_t<f16, 128>(causal, dropout, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace fa
