// Kernel argument blocks and host-side launchers shared between the C ABI
// layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Elem { F32 = 0, BF16 = 1, F16 = 2 };

// ------------------------------------------------------------ unit order
//
// Every kernel's grid is one workgroup per work unit (b, h, block of query
// rows or keys).  The dispatcher hands workgroup u to XCD u % 8, as that
// XCD's (u / 8)-th workgroup, and each XCD has its own L2.  unit_of()
// renumbers u so that each XCD takes a contiguous range of one order over
// all units: heads in groups of G, and within a group block rank by block
// rank (rank 0 first: the longest causal block), the group's heads
// alternating.  The heads live on an XCD at any time are then those of one
// or two groups -- their K/V (forward) or Q/dO (backward) rows stay in that
// XCD's L2 -- while the longest units still start first.  The launchers
// pick G (unit_group) as the number of heads whose blocks fill the XCD's
// resident workgroup slots twice, capped at one XCD's share of the heads.
// Any G >= 1 gives a bijection; only locality and load balance depend on it.
constexpr uint32_t kXcds = 8;

struct Unit {
    uint32_t bh;      // b * H + h
    uint32_t rank;    // block rank within the head, 0 .. nb - 1
};

__host__ __device__ inline Unit unit_of(uint32_t u, uint32_t U, uint32_t BH, uint32_t nb,
                                        uint32_t G) {
    const uint32_t per = U / kXcds, extra = U % kXcds;
    const uint32_t x = u % kXcds, s = u / kXcds;
    const uint32_t v = x * per + (x < extra ? x : extra) + s;    // position in the order
    const uint32_t gsz = G * nb;
    const uint32_t grp = v / gsz, r = v % gsz;
    const uint32_t heads = BH - grp * G < G ? BH - grp * G : G;  // the last group may be short
    return Unit{grp * G + r % heads, r / heads};
}

// Heads per group for BH heads of nb units each and `wg_per_cu` resident
// workgroups per CU (host side; the CU count is the current device's).
uint32_t unit_group(int64_t BH, int64_t nb, int wg_per_cu);

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t B, H, N;
    int64_t Nk;           // keys (and values) per head; queries see key j <= i + Nk - N when causal
    int32_t kv_splits;    // key chunks per query block (1: one pass over all keys)
    int32_t kv_chunk;     // keys per chunk, a multiple of 64
    float *part_o;        // kv_splits > 1: O of each chunk [kv_splits,B,H,N,D] fp32, normalised
    float *part_lse;      // kv_splits > 1: log-sum-exp of each chunk [kv_splits,B,H,N]
    float scale_log2;     // softmax scale times log2(e)
    float drop_c;         // keep scale 1/(1-p) rounded to float
    uint32_t drop_T;      // 16-bit drop threshold round(p * 65536)
    uint32_t seed_lo, seed_hi;
    int32_t out_f32;
    uint32_t group;       // heads per group of the unit order (unit_of)
    // FP8 inputs only: fp32 descale factor per (b, h) of Q, K and V ([B*H] each)
    const float *descale_q, *descale_k, *descale_v;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *dvec;          // workspace: D_i / c, D_i = dO_i . O_i, [B,H,N]
    float *nl2;           // workspace: -lse_i log2(e), [B,H,N]
    int64_t B, H, N;
    int64_t Nk;           // keys per head (k, v, dk, dv are [B,H,Nk,d]); causal: key j <= i + Nk - N
    float scale;          // softmax scale
    float scale_log2;     // scale * log2(e)
    float drop_c;
    uint32_t drop_T;
    uint32_t seed_lo, seed_hi;
    int32_t out_f32;      // o, dout and the gradients are fp32 when set
    uint32_t group;       // heads per group of the unit order (unit_of), set by each launcher
};

// Each launcher enqueues its kernels on `stream` and returns the status of
// the launch (hipSuccess when enqueued).
hipError_t launch_fwd(Elem e, int d, bool causal, bool dropout, const FwdArgs &a,
                      hipStream_t stream);
hipError_t launch_bwd_pre(Elem e, int d, const BwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_dkdv(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                           hipStream_t stream);
hipError_t launch_bwd_dq(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                         hipStream_t stream);
// 16-bit inputs only (bf16, f16); d = 64, 128, 256.
hipError_t launch_bwd_dq16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                           hipStream_t stream);
hipError_t launch_bwd_dq16_256(Elem e, bool causal, bool dropout, const BwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_dkdv16(Elem e, int d, bool causal, bool dropout, const BwdArgs &a,
                             hipStream_t stream);
// 16-bit inputs at d = 64, 128, 256: four wavefronts per workgroup, two
// workgroups per CU (one at d = 256).
hipError_t launch_fwd_pp(Elem e, int d, bool causal, bool dropout, const FwdArgs &a,
                         hipStream_t stream);
// e4m3 inputs at d = 128 with per-(b, h) descale factors; bf16 (or fp32) O.
hipError_t launch_fwd_fp8(int d, bool causal, const FwdArgs &a, hipStream_t stream);
// Combines the kv_splits partial results of a split forward into o and lse.
hipError_t launch_fwd_merge(Elem e, int d, const FwdArgs &a, hipStream_t stream);
hipError_t launch_dropout_mask(int64_t N, uint32_t T, uint32_t seed_lo, uint32_t seed_hi,
                               int64_t b, int64_t h, uint8_t *mask, hipStream_t stream);

}  // namespace fa
