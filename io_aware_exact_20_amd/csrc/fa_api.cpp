// C ABI of the attention library: argument validation, workspace sizing and
// dispatch to the gfx950 kernels.  Validation happens before any HIP call,
// so a rejected call never touches the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fa.h"
#include "fa_kernels.hpp"

namespace fa {

// Heads per group of the unit order: enough heads that their blocks fill
// the resident workgroup slots of one XCD (CUs / 8 times the workgroups per
// CU) twice, but no more than one XCD's share of the heads (a group spread
// over two XCDs would give one of them all the long causal blocks).
// Measured on the training shape (4 x 32 x 4096 x 128) this takes the step
// from 3.46 ms (one group per XCD's share) or 3.37 ms (slots filled once)
// to 3.29 ms.  The CU count is read once per device.
uint32_t unit_group(int64_t BH, int64_t nb, int wg_per_cu) {
    static std::atomic<int> cu_count[64];
    int n = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        n = cu_count[dev].load(std::memory_order_relaxed);
        if (n <= 0) {
            int c = 0;
            n = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0
                    ? c : 256;
            cu_count[dev].store(n, std::memory_order_relaxed);
        }
    }
    const int64_t per_xcd = n / (int)kXcds > 0 ? n / (int)kXcds : 1;
    const int64_t slots = per_xcd * (wg_per_cu > 0 ? wg_per_cu : 1);
    int64_t g = nb > 0 ? (2 * slots + nb - 1) / nb : 1;
    const int64_t share = BH / (int64_t)kXcds;
    if (g > share) g = share;
    return (uint32_t)(g < 1 ? 1 : g);
}

}  // namespace fa

namespace {

thread_local char g_last_error[256] = "";

fa_status_t fail(fa_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status_t fail(fa_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

fa_status_t ok() {
    g_last_error[0] = '\0';
    return FA_OK;
}

}  // namespace

namespace fa {

fa_status_t record_error(fa_status_t s, const char *msg) { return fail(s, "%s", msg); }

}  // namespace fa

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int32_t dtype) { return dtype == FA_F32 ? 4 : 2; }

uint32_t drop_threshold(float p) { return (uint32_t)std::llround((double)p * 65536.0); }
float keep_scale(float p) { return (float)(1.0 / (1.0 - (double)p)); }

// Checks shared by every entry point.  *empty is set when there is nothing
// to compute (a zero extent).
fa_status_t check_params(const fa_params_t *p, bool *empty) {
    if (!p) return fail(FA_EINVAL, "params is NULL");
    if (p->B < 0 || p->H < 0 || p->N < 0)
        return fail(FA_EINVAL, "negative extent B=%lld H=%lld N=%lld", (long long)p->B,
                    (long long)p->H, (long long)p->N);
    if (p->N > 0x7fffffffLL) return fail(FA_EINVAL, "N=%lld exceeds 2^31-1", (long long)p->N);
    if (p->dtype != FA_F32 && p->dtype != FA_BF16 && p->dtype != FA_F16)
        return fail(FA_EUNSUPPORTED, "dtype %d is not supported", (int)p->dtype);
    if (p->d != 32 && p->d != 64 && p->d != 96 && p->d != 128 && p->d != 256)
        return fail(FA_EUNSUPPORTED, "head dimension d=%lld is not supported (32, 64, 96, 128, 256)",
                    (long long)p->d);
    if (p->d == 256 && p->dtype == FA_F32)
        return fail(FA_EUNSUPPORTED, "head dimension 256 needs 16-bit inputs");
    if (p->causal != 0 && p->causal != 1) return fail(FA_EINVAL, "causal must be 0 or 1");
    if (!std::isfinite(p->scale) || !(p->scale > 0.f))
        return fail(FA_EINVAL, "scale must be finite and positive (got %g)", (double)p->scale);
    if (!(p->dropout_p >= 0.f && p->dropout_p < 1.f))
        return fail(FA_EINVAL, "dropout_p must be in [0, 1) (got %g)", (double)p->dropout_p);
    // The packed keep-mask compares of the 16-bit kernels represent
    // thresholds 1 .. 65536 only; T = 0 would keep every element.
    if (p->dropout_p > 0.f && drop_threshold(p->dropout_p) == 0)
        return fail(FA_EUNSUPPORTED, "dropout_p=%g rounds to a zero 16-bit threshold (p < 2^-17)",
                    (double)p->dropout_p);
    if (p->out_f32 != 0 && p->out_f32 != 1) return fail(FA_EINVAL, "out_f32 must be 0 or 1");
    if (p->Nk < 0) return fail(FA_EINVAL, "Nk=%d is negative", (int)p->Nk);
    // One head of any operand is addressed with signed 32-bit byte offsets.
    const double head_bytes = (double)(p->Nk > p->N ? p->Nk : p->N) * (double)p->d *
                              (p->dtype == FA_F32 || p->out_f32 ? 4.0 : 2.0);
    if (head_bytes >= 2147483648.0)
        return fail(FA_EUNSUPPORTED, "one head of %.3g bytes reaches 2 GiB", head_bytes);
    // B*H*N*d must be addressable; the product of the extents is bounded
    // piecewise to avoid overflow in the check itself.
    const double total = (double)p->B * (double)p->H * (double)p->N * (double)p->d;
    if (total > 9.0e15) return fail(FA_EINVAL, "problem too large (B*H*N*d = %.3g)", total);
    *empty = p->B == 0 || p->H == 0 || p->N == 0;
    return FA_OK;
}

fa_status_t check_ptr(const void *ptr, const char *name) {
    if (!ptr) return fail(FA_EINVAL, "%s is NULL", name);
    if (!aligned16(ptr)) return fail(FA_EINVAL, "%s is not 16-byte aligned", name);
    return FA_OK;
}

fa::Elem elem(int32_t dtype) {
    return dtype == FA_F32 ? fa::Elem::F32 : dtype == FA_BF16 ? fa::Elem::BF16 : fa::Elem::F16;
}


// The workspace holds two fp32 arrays of one value per query row, each
// padded to 256 bytes: D_i / c, then -lse_i log2(e).
size_t row_array_bytes(const fa_params_t *p) {
    const size_t rows = (size_t)p->B * (size_t)p->H * (size_t)p->N;
    return (rows * 4 + 255) / 256 * 256;
}

size_t workspace_bytes(const fa_params_t *p) { return 2 * row_array_bytes(p); }

// Keys per head (Nk = 0 means N).
int64_t keys(const fa_params_t *p) { return p->Nk ? (int64_t)p->Nk : p->N; }

// A split forward: key chunks of a multiple of 64 keys; the number of
// chunks actually used for `splits` requested.
int64_t split_chunk(const fa_params_t *p, int32_t splits) {
    const int64_t nk = keys(p);
    const int64_t per = (nk + splits - 1) / splits;
    return (per + 63) / 64 * 64;
}
int32_t splits_used(const fa_params_t *p, int32_t splits) {
    const int64_t chunk = split_chunk(p, splits);
    return (int32_t)((keys(p) + chunk - 1) / chunk);
}
constexpr int32_t kMaxSplits = 256;

// The split workspace: the chunks' O (fp32, [S,B,H,N,d]) then their LSE
// ([S,B,H,N]), each rounded up to 256 bytes.
size_t split_o_bytes(const fa_params_t *p, int32_t splits) {
    const size_t n = (size_t)splits * (size_t)p->B * (size_t)p->H * (size_t)p->N * (size_t)p->d;
    return (n * 4 + 255) / 256 * 256;
}
size_t split_workspace_bytes(const fa_params_t *p, int32_t splits) {
    return split_o_bytes(p, splits) + (size_t)splits * row_array_bytes(p);
}

// Forward argument block: one pass over all Nk keys (kv_splits = 1).
fa::FwdArgs fwd_args(const fa_params_t *p, const void *q, const void *k, const void *v, void *o,
                     float *lse) {
    fa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = p->B; a.H = p->H; a.N = p->N;
    a.Nk = keys(p);
    a.kv_splits = 1;
    a.kv_chunk = (int32_t)((a.Nk + 63) / 64 * 64);
    a.scale_log2 = p->scale * 1.44269504088896340736f;
    const bool dropout = p->dropout_p > 0.f;
    a.drop_T = dropout ? drop_threshold(p->dropout_p) : 0;
    a.drop_c = dropout ? keep_scale(p->dropout_p) : 1.f;
    a.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFu);
    a.seed_hi = (uint32_t)(p->seed >> 32);
    a.out_f32 = p->out_f32;
    return a;
}

fa_status_t hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(FA_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return ok();
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const fa_params_t *p, const void *q, const void *k, const void *v, void *o,
                   float *lse, void *stream) {
    bool empty = false;
    fa_status_t s = check_params(p, &empty);
    if (s != FA_OK) return s;
    if (empty) return ok();
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_ptr(lse, "lse")))
        return s;
    fa::FwdArgs a = fwd_args(p, q, k, v, o, lse);
    return hip_status(fa::launch_fwd(elem(p->dtype), (int)p->d, p->causal != 0,
                                     p->dropout_p > 0.f, a, reinterpret_cast<hipStream_t>(stream)),
                      "fa_fwd launch");
}

size_t fa_fwd_splitkv_workspace_bytes(const fa_params_t *p, int32_t num_splits) {
    bool empty = false;
    if (check_params(p, &empty) != FA_OK) return (size_t)-1;
    if (num_splits < 1 || num_splits > kMaxSplits) return (size_t)-1;
    if (empty || splits_used(p, num_splits) < 2) return 0;
    return split_workspace_bytes(p, num_splits);
}

fa_status_t fa_fwd_fp8(const fa_params_t *p, const void *q, const void *k, const void *v,
                       const float *descale_q, const float *descale_k, const float *descale_v,
                       void *o, float *lse, void *stream) {
    if (!p) return fail(FA_EINVAL, "params is NULL");
    if (p->dtype != FA_FP8_E4M3)
        return fail(FA_EINVAL, "fa_fwd_fp8 takes dtype FA_FP8_E4M3 (got %d)", (int)p->dtype);
    // The shared checks, with the output type (bf16 or fp32) standing for
    // the element size of the largest head.
    fa_params_t c = *p;
    c.dtype = FA_BF16;
    bool empty = false;
    fa_status_t s = check_params(&c, &empty);
    if (s != FA_OK) return s;
    if (p->d != 128) return fail(FA_EUNSUPPORTED, "FP8 inputs need d = 128 (got %lld)", (long long)p->d);
    if (p->dropout_p != 0.f) return fail(FA_EUNSUPPORTED, "FP8 inputs take no dropout");
    if (empty) return ok();
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_ptr(lse, "lse")))
        return s;
    const float *ds[3] = {descale_q, descale_k, descale_v};
    const char *dn[3] = {"descale_q", "descale_k", "descale_v"};
    for (int i = 0; i < 3; ++i)
        if (!ds[i] || (reinterpret_cast<uintptr_t>(ds[i]) & 3u))
            return fail(FA_EINVAL, "%s is NULL or not 4-byte aligned", dn[i]);
    fa::FwdArgs a = fwd_args(&c, q, k, v, o, lse);
    a.descale_q = descale_q;
    a.descale_k = descale_k;
    a.descale_v = descale_v;
    return hip_status(fa::launch_fwd_fp8((int)p->d, p->causal != 0, a,
                                         reinterpret_cast<hipStream_t>(stream)),
                      "fa_fwd_fp8 launch");
}

fa_status_t fa_fwd_splitkv(const fa_params_t *p, const void *q, const void *k, const void *v,
                           void *o, float *lse, int32_t num_splits, void *workspace,
                           size_t workspace_size, void *stream) {
    bool empty = false;
    fa_status_t s = check_params(p, &empty);
    if (s != FA_OK) return s;
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FA_EINVAL, "num_splits=%d outside 1..%d", (int)num_splits, (int)kMaxSplits);
    if (empty) return ok();
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_ptr(lse, "lse")))
        return s;
    fa::FwdArgs a = fwd_args(p, q, k, v, o, lse);
    const int32_t used = splits_used(p, num_splits);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (used < 2)
        return hip_status(fa::launch_fwd(elem(p->dtype), (int)p->d, p->causal != 0,
                                         p->dropout_p > 0.f, a, st), "fa_fwd_splitkv launch");
    if ((s = check_ptr(workspace, "workspace"))) return s;
    const size_t need = split_workspace_bytes(p, num_splits);
    if (workspace_size < need)
        return fail(FA_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_size, need);
    a.kv_splits = used;
    a.kv_chunk = (int32_t)split_chunk(p, num_splits);
    a.part_o = reinterpret_cast<float *>(workspace);
    a.part_lse = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) +
                                           split_o_bytes(p, num_splits));
    s = hip_status(fa::launch_fwd(elem(p->dtype), (int)p->d, p->causal != 0,
                                  p->dropout_p > 0.f, a, st), "fa_fwd_splitkv launch");
    if (s != FA_OK) return s;
    return hip_status(fa::launch_fwd_merge(elem(p->dtype), (int)p->d, a, st),
                      "fa_fwd_splitkv merge launch");
}

size_t fa_bwd_workspace_bytes(const fa_params_t *p) {
    bool empty = false;
    if (check_params(p, &empty) != FA_OK) return (size_t)-1;
    if (empty) return 0;
    return workspace_bytes(p);
}

}  // extern "C"

namespace {

// Common part of the backward entry points: parameter and workspace checks,
// and the argument block (the workspace holds the two row arrays).
fa_status_t bwd_setup(const fa_params_t *p, const void *workspace, size_t workspace_size,
                      bool *empty, fa::BwdArgs *a) {
    fa_status_t s = check_params(p, empty);
    if (s != FA_OK || *empty) return s;
    if ((s = check_ptr(workspace, "workspace"))) return s;
    const size_t need = workspace_bytes(p);
    if (workspace_size < need)
        return fail(FA_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_size, need);
    *a = fa::BwdArgs{};
    a->dvec = reinterpret_cast<float *>(const_cast<void *>(workspace));
    a->nl2 = reinterpret_cast<float *>(reinterpret_cast<char *>(const_cast<void *>(workspace)) +
                                       row_array_bytes(p));
    a->B = p->B; a->H = p->H; a->N = p->N;
    a->Nk = keys(p);
    a->scale = p->scale;
    a->scale_log2 = p->scale * 1.44269504088896340736f;
    const bool dropout = p->dropout_p > 0.f;
    a->drop_T = dropout ? drop_threshold(p->dropout_p) : 0;
    a->drop_c = dropout ? keep_scale(p->dropout_p) : 1.f;
    a->seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFu);
    a->seed_hi = (uint32_t)(p->seed >> 32);
    a->out_f32 = p->out_f32;
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_prepare(const fa_params_t *p, const void *o, const float *lse, const void *dout,
                           void *workspace, size_t workspace_size, void *stream) {
    bool empty = false;
    fa::BwdArgs a;
    fa_status_t s = bwd_setup(p, workspace, workspace_size, &empty, &a);
    if (s != FA_OK) return s;
    if (empty) return ok();
    if ((s = check_ptr(o, "o")) || (s = check_ptr(lse, "lse")) || (s = check_ptr(dout, "dout")))
        return s;
    a.o = o; a.lse = lse; a.dout = dout;
    return hip_status(fa::launch_bwd_pre(elem(p->dtype), (int)p->d, a,
                                         reinterpret_cast<hipStream_t>(stream)),
                      "fa_bwd_prepare launch");
}

fa_status_t fa_bwd_dkdv(const fa_params_t *p, const void *q, const void *k, const void *v,
                        const float *lse, const void *dout, void *dk, void *dv,
                        const void *workspace, size_t workspace_size, void *stream) {
    bool empty = false;
    fa::BwdArgs a;
    fa_status_t s = bwd_setup(p, workspace, workspace_size, &empty, &a);
    if (s != FA_OK) return s;
    if (empty) return ok();
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(lse, "lse")) || (s = check_ptr(dout, "dout")) ||
        (s = check_ptr(dk, "dk")) || (s = check_ptr(dv, "dv")))
        return s;
    a.q = q; a.k = k; a.v = v; a.lse = lse; a.dout = dout; a.dk = dk; a.dv = dv;
    return hip_status(fa::launch_bwd_dkdv(elem(p->dtype), (int)p->d, p->causal != 0,
                                          p->dropout_p > 0.f, a,
                                          reinterpret_cast<hipStream_t>(stream)),
                      "fa_bwd_dkdv launch");
}

fa_status_t fa_bwd_dq(const fa_params_t *p, const void *q, const void *k, const void *v,
                      const float *lse, const void *dout, void *dq, const void *workspace,
                      size_t workspace_size, void *stream) {
    bool empty = false;
    fa::BwdArgs a;
    fa_status_t s = bwd_setup(p, workspace, workspace_size, &empty, &a);
    if (s != FA_OK) return s;
    if (empty) return ok();
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(lse, "lse")) || (s = check_ptr(dout, "dout")) || (s = check_ptr(dq, "dq")))
        return s;
    a.q = q; a.k = k; a.v = v; a.lse = lse; a.dout = dout; a.dq = dq;
    return hip_status(fa::launch_bwd_dq(elem(p->dtype), (int)p->d, p->causal != 0,
                                        p->dropout_p > 0.f, a,
                                        reinterpret_cast<hipStream_t>(stream)),
                      "fa_bwd_dq launch");
}

fa_status_t fa_bwd(const fa_params_t *p, const void *q, const void *k, const void *v,
                   const void *o, const float *lse, const void *dout, void *dq, void *dk,
                   void *dv, void *workspace, size_t workspace_size, void *stream) {
    bool empty = false;
    fa::BwdArgs a;
    fa_status_t s = bwd_setup(p, workspace, workspace_size, &empty, &a);
    if (s != FA_OK) return s;
    if (empty) return ok();
    // Every pointer is checked before the first stage is enqueued.
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_ptr(lse, "lse")) || (s = check_ptr(dout, "dout")) ||
        (s = check_ptr(dq, "dq")) || (s = check_ptr(dk, "dk")) || (s = check_ptr(dv, "dv")))
        return s;
    if ((s = fa_bwd_prepare(p, o, lse, dout, workspace, workspace_size, stream))) return s;
    if ((s = fa_bwd_dkdv(p, q, k, v, lse, dout, dk, dv, workspace, workspace_size, stream)))
        return s;
    return fa_bwd_dq(p, q, k, v, lse, dout, dq, workspace, workspace_size, stream);
}

fa_status_t fa_dropout_mask(const fa_params_t *p, int64_t b, int64_t h, uint8_t *mask,
                            void *stream) {
    if (!p) return fail(FA_EINVAL, "params is NULL");
    if (p->B < 0 || p->H < 0 || p->N < 0) return fail(FA_EINVAL, "negative extent");
    if (p->N > 0x7fffffffLL) return fail(FA_EINVAL, "N exceeds 2^31-1");
    if (!(p->dropout_p >= 0.f && p->dropout_p < 1.f))
        return fail(FA_EINVAL, "dropout_p must be in [0, 1)");
    if (b < 0 || b >= p->B || h < 0 || h >= p->H)
        return fail(FA_EINVAL, "plane (b=%lld, h=%lld) outside B=%lld H=%lld", (long long)b,
                    (long long)h, (long long)p->B, (long long)p->H);
    if (p->N == 0) return ok();
    if (!mask) return fail(FA_EINVAL, "mask is NULL");
    const uint32_t T = p->dropout_p > 0.f ? drop_threshold(p->dropout_p) : 0;
    return hip_status(fa::launch_dropout_mask(p->N, T, (uint32_t)(p->seed & 0xFFFFFFFFu),
                                              (uint32_t)(p->seed >> 32), b, h, mask,
                                              reinterpret_cast<hipStream_t>(stream)),
                      "fa_dropout_mask launch");
}

fa_status_t fa_unit_order(int64_t BH, int64_t nb, int32_t group, uint32_t *bh, uint32_t *rank) {
    if (BH < 1 || nb < 1 || group < 1) return fail(FA_EINVAL, "BH, nb and group must be >= 1");
    if (BH * nb > 0x7fffffffLL || (int64_t)group * nb > 0x7fffffffLL)
        return fail(FA_EINVAL, "BH * nb and group * nb must stay below 2^31");
    if (!bh || !rank) return fail(FA_EINVAL, "output arrays must not be NULL");
    const uint32_t U = (uint32_t)(BH * nb);
    for (uint32_t u = 0; u < U; ++u) {
        const fa::Unit x = fa::unit_of(u, U, (uint32_t)BH, (uint32_t)nb, (uint32_t)group);
        bh[u] = x.bh;
        rank[u] = x.rank;
    }
    return ok();
}

const char *fa_status_str(fa_status_t s) {
    switch (s) {
    case FA_OK: return "FA_OK";
    case FA_EINVAL: return "FA_EINVAL: invalid argument";
    case FA_EUNSUPPORTED: return "FA_EUNSUPPORTED: unsupported configuration";
    case FA_EHIP: return "FA_EHIP: HIP runtime error";
    }
    return "unknown fa_status_t";
}

const char *fa_last_error(void) { return g_last_error; }

}  // extern "C"
