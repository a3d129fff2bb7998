"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (per tensor): fp32 inputs max-abs <= 1e-5; bf16 / fp16 inputs
max-abs <= 2e-2 and mean-abs <= 2e-3.  Integer-valued outcomes (dropout
masks, causal and tile zero patterns) must match exactly.

Storage rounding.  A bf16 output carries up to half an ulp of rounding on
top of the computation (0.0156 for |x| in [4, 8)), so the 2e-2 max-abs bar
is applied to the computed values themselves: strictly to the run whose
outputs are written in fp32 (``out_f32=1``, same kernels), and to the
16-bit-output run with half an output ulp of |exact| added per element.
The mean-abs bar applies unchanged to the 16-bit-output run.

The oracle gets the exact float64 up-cast of the same rounded inputs and the
dropout probability rounded to float32, as the library receives it.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3), "f16": (2e-2, 2e-3)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def p32(p):
    return float(np.float32(p))


MANTISSA_BITS = {torch.bfloat16: 7, torch.float16: 10, torch.float32: 23}


def half_ulp(x, torch_dtype):
    """Half a unit in the last place of |x| in the given storage type."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - MANTISSA_BITS[torch_dtype] - 1), 0.0)


def compare(name, got, exact, dtype):
    """Max/mean abs error of `got` (torch, any device) against `exact` (f64).

    16-bit outputs get half an output ulp of |exact| on top of the max-abs
    bar (the storage rounding); fp32 outputs are held to the bar itself."""
    g = got.detach().double().cpu().numpy()
    e = np.asarray(exact)
    assert np.isfinite(g).all(), "%s has non-finite values" % name
    err = np.abs(g - e)
    tmax, tmean = TOL[dtype]
    slack = half_ulp(e, got.dtype) if got.dtype != torch.float32 else 0.0
    excess = err - slack
    mx, mn = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    mx_ex = float(excess.max(initial=0.0))
    log("  %-4s max|err| %.3e (less storage %.3e) mean|err| %.3e max|x| %.2f [%s]" %
        (name, mx, mx_ex, mn, float(np.abs(e).max(initial=0)), str(got.dtype)[6:]))
    assert mx_ex <= tmax, "%s max-abs error %.3e (beyond storage rounding) > %.1e" % (
        name, mx_ex, tmax)
    if tmean is not None:
        assert mn <= tmean, "%s mean-abs error %.3e > %.1e" % (name, mn, tmean)


def run_fwd(fa, w: Workload, q, k, v, out_f32=False):
    dev = "cuda"
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), scale=w.softmax_scale, causal=w.causal,
                    dropout_p=w.dropout_p, seed=w.dropout_seed, out_f32=out_f32)
    torch.cuda.synchronize()
    return o, lse


def run_bwd(fa, w: Workload, q, k, v, do, out_f32=False):
    dev = "cuda"
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.fwd(qd, kd, vd, scale=w.softmax_scale, causal=w.causal, dropout_p=w.dropout_p,
                    seed=w.dropout_seed, out_f32=out_f32)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, scale=w.softmax_scale, causal=w.causal,
                        dropout_p=w.dropout_p, seed=w.dropout_seed, out_f32=out_f32)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def oracle_fwd(w, q, k, v, heads=None):
    return oracle.fwd(q, k, v, w.softmax_scale, w.causal, p32(w.dropout_p), w.dropout_seed,
                      heads=heads)


def oracle_bwd(w, q, k, v, do, heads=None):
    return oracle.bwd(q, k, v, do, w.softmax_scale, w.causal, p32(w.dropout_p), w.dropout_seed,
                      heads=heads)


# ------------------------------------------------------- full comparisons

SMALL = []
for dt in ("bf16", "f16", "f32"):
    for d in (64, 128):
        for causal in (False, True):
            for p in (0.0, 0.1):
                SMALL.append(Workload("small_%s_d%d_c%d_p%g" % (dt, d, causal, p), 2, 3, 300, d,
                                      dt, causal=causal, dropout_p=p, backward=True,
                                      seed=11 + d + 3 * causal, dropout_seed=0xC0FFEE + d))


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_fwd_bwd_full(gpu_lib, w):
    """Every element of O, LSE, dQ, dK, dV at N=300 (several tiles plus a
    ragged tail), both head dims, masks, dropout and all input types."""
    log("case %s" % w.name)
    q, k, v, do = workloads.draw(w)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    for out_f32 in ((False, True) if w.dtype != "f32" else (False,)):
        o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do, out_f32=out_f32)
        for name, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                                 ("dK", dk, edk), ("dV", dv, edv)):
            compare(name, got, exact, w.dtype)


HEAD_DIMS = []
for dt, dims in (("bf16", (32, 96, 256)), ("f16", (32, 96, 256)), ("f32", (32, 96))):
    for d in dims:
        for causal, p in ((False, 0.0), (True, 0.1)) if dt != "bf16" else \
                ((False, 0.0), (False, 0.1), (True, 0.0), (True, 0.1)):
            HEAD_DIMS.append(Workload("hd_%s_d%d_c%d_p%g" % (dt, d, causal, p), 1, 2, 300, d, dt,
                                      causal=causal, dropout_p=p, backward=True,
                                      seed=40 + d + causal, dropout_seed=0xD1CE + d))


@pytest.mark.parametrize("w", HEAD_DIMS, ids=[w.name for w in HEAD_DIMS])
def test_other_head_dims_fwd_bwd_full(gpu_lib, w):
    """Head dimensions 32, 96 and 256 (16-bit inputs: the tuned kernels; fp32:
    the generic ones): every element of O, LSE, dQ, dK, dV at N=300, masks,
    dropout, all input types (256: 16-bit)."""
    log("case %s" % w.name)
    q, k, v, do = workloads.draw(w)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    for name, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                             ("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got, exact, w.dtype)


# ---------------------------- queries and keys of two lengths; split keys

def compare_rows(name, got, exact, dtype):
    """compare() over the rows that see at least one key; rows that see none
    must be exactly O = 0 / LSE = -inf."""
    e = np.asarray(exact)
    g = got.detach().double().cpu().numpy()
    lse_like = e.ndim == 3
    dead = ~np.isfinite(e) if lse_like else np.zeros(e.shape, bool)
    if lse_like:
        assert np.all(g[dead] == -np.inf), "%s: rows with no visible key must be -inf" % name
        compare(name, got.detach().cpu()[torch.from_numpy(~dead)], e[~dead], dtype)
    else:
        compare(name, got, e, dtype)


CROSS = [
    # dtype, d, N (queries), Nk (keys), causal, p
    ("bf16", 128, 300, 1000, False, 0.0), ("bf16", 128, 300, 1000, True, 0.1),
    ("bf16", 128, 1, 777, True, 0.0), ("bf16", 64, 1000, 300, True, 0.1),
    ("bf16", 64, 77, 4096, False, 0.1), ("f16", 128, 130, 555, True, 0.0),
    ("bf16", 96, 50, 333, True, 0.1), ("bf16", 256, 40, 300, True, 0.0),
    ("f32", 64, 77, 200, True, 0.1), ("f32", 128, 33, 64, False, 0.0),
    # d = 128 with fewer keys than queries: whole wavefronts of rows see no key
    ("bf16", 128, 1000, 300, True, 0.1), ("bf16", 128, 700, 250, True, 0.0),
    ("f16", 128, 600, 100, True, 0.1),
    # the other head dimensions with queries and keys of two lengths
    ("bf16", 32, 300, 700, True, 0.1), ("f16", 32, 500, 200, True, 0.0),
    ("f16", 96, 400, 150, True, 0.1), ("bf16", 256, 130, 500, False, 0.1),
    # d = 256 causal with dropout (its dQ finishes each tile in one step)
    ("f16", 256, 300, 700, True, 0.1), ("bf16", 256, 500, 130, True, 0.1),
]


@pytest.mark.parametrize("case", CROSS, ids=["%s_d%d_%dx%d_c%d_p%g" % c for c in CROSS])
def test_cross_lengths_fwd_full(gpu_lib, case):
    """N != Nk (decoding, cross attention): every element of O and LSE,
    causal aligned on the last key; queries that see no key give 0 / -inf."""
    dt, d, N, Nk, causal, p = case
    w = Workload("cross", 2, 2, N, d, dt, causal=causal, dropout_p=p, seed=17 + d + N,
                 dropout_seed=0xFACE + Nk)
    log("case %s Nk=%d" % (case, Nk))
    q, k, v = workloads.draw_cross(w, Nk)
    eo, el = oracle_fwd(w, q, k, v)
    o, lse = run_fwd(gpu_lib, w, q, k, v)
    compare_rows("O", o, eo, dt)
    compare_rows("LSE", lse, el, dt)


CROSS_BWD = [
    # dtype, d, N (queries), Nk (keys), causal, p
    ("bf16", 128, 300, 1000, True, 0.1), ("bf16", 128, 1000, 300, True, 0.0),
    ("bf16", 64, 200, 777, False, 0.1), ("bf16", 64, 555, 130, True, 0.1),
    ("f16", 128, 129, 64, True, 0.0), ("bf16", 96, 70, 250, True, 0.1),
    ("bf16", 256, 40, 100, True, 0.0), ("f32", 64, 77, 200, True, 0.1),
    ("f32", 128, 100, 33, False, 0.0),
    # d = 256 causal with dropout (its dQ finishes each tile in one step)
    ("f16", 256, 300, 700, True, 0.1), ("bf16", 256, 500, 130, True, 0.1),
]


@pytest.mark.parametrize("case", CROSS_BWD, ids=["%s_d%d_%dx%d_c%d_p%g" % c for c in CROSS_BWD])
def test_cross_lengths_fwd_bwd_full(gpu_lib, case):
    """N != Nk forward and backward (cross attention): every element of O,
    LSE, dQ [N], dK and dV [Nk] against the oracle; queries that see no key
    give O = 0, LSE = -inf and dQ = 0, and add nothing to dK, dV."""
    dt, d, N, Nk, causal, p = case
    w = Workload("crossb", 2, 2, N, d, dt, causal=causal, dropout_p=p, backward=True,
                 seed=31 + d + N, dropout_seed=0xCAFE + Nk)
    log("case %s" % (case,))
    q, k, v, do = workloads.draw_cross(w, Nk, with_dout=True)
    edq, edk, edv, eo, el = oracle_bwd(w, q, k, v, do)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    compare_rows("O", o, eo, dt)
    compare_rows("LSE", lse, el, dt)
    for name, got, exact in (("dQ", dq, edq), ("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got, exact, dt)


SPLITS = [
    # dtype, d, N, Nk, causal, p, num_splits
    ("bf16", 128, 1, 4096, True, 0.0, 8), ("bf16", 128, 16, 4096, True, 0.1, 64),
    ("bf16", 128, 300, 1000, False, 0.1, 3), ("bf16", 64, 256, 2048, True, 0.0, 7),
    ("bf16", 64, 1000, 300, True, 0.1, 2), ("f16", 128, 5, 3000, False, 0.0, 256),
    ("bf16", 256, 17, 1500, True, 0.1, 5), ("f32", 64, 9, 1000, True, 0.1, 4),
    ("bf16", 128, 1024, 1024, True, 0.1, 4), ("bf16", 32, 40, 2000, True, 0.1, 6),
    ("f16", 96, 130, 1100, False, 0.0, 3),
]


@pytest.mark.parametrize("case", SPLITS, ids=["%s_d%d_%dx%d_c%d_p%g_s%d" % c for c in SPLITS])
def test_split_keys_fwd_full(gpu_lib, case):
    """fa_fwd_splitkv: key chunks on separate workgroups merged by their
    log-sum-exp; every element of O and LSE against the oracle, and close to
    the one-pass forward."""
    dt, d, N, Nk, causal, p, splits = case
    w = Workload("split", 2, 3, N, d, dt, causal=causal, dropout_p=p, seed=23 + d + N,
                 dropout_seed=0xBEEF + Nk)
    log("case %s" % (case,))
    q, k, v = workloads.draw_cross(w, Nk)
    eo, el = oracle_fwd(w, q, k, v)
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for out_f32 in ((False, True) if dt != "f32" else (False,)):
        o, lse = gpu_lib.fwd_splitkv(qd, kd, vd, splits, scale=w.softmax_scale, causal=causal,
                                     dropout_p=p, seed=w.dropout_seed, out_f32=out_f32)
        o1, lse1 = gpu_lib.fwd(qd, kd, vd, scale=w.softmax_scale, causal=causal, dropout_p=p,
                               seed=w.dropout_seed, out_f32=out_f32)
        torch.cuda.synchronize()
        compare_rows("O", o, eo, dt)
        compare_rows("LSE", lse, el, dt)
        live = torch.isfinite(lse1)
        assert torch.equal(torch.isfinite(lse), live)
        # (16-bit paths sum the rounded probabilities, so the two summation
        # orders differ at that rounding's level)
        assert float((lse - lse1)[live].abs().max()) < (2e-3 if dt != "f32" else 1e-5)
        assert float((o.float() - o1.float()).abs().max()) <= (2e-2 if dt != "f32" else 1e-5)


def test_single_head_f32_fwd_bwd(gpu_lib):
    """B=1,H=1,N=128,d=64 fp32 non-causal forward and backward: max-abs 1e-5."""
    w = workloads.WORKLOADS["single_head_f32"]
    log("case %s" % w.name)
    q, k, v, do = workloads.draw(w)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    for name, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                             ("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got, exact, "f32")


@pytest.mark.parametrize("name", ["small_fwd_bf16", "small_fwd_bf16_causal"])
def test_small_forward_all_heads(gpu_lib, name):
    """B=2,H=8,N=1024,d=64 bf16 forward, non-causal and causal, every head."""
    w = workloads.WORKLOADS[name]
    log("case %s" % w.name)
    q, k, v, _ = workloads.draw(w)
    o, lse = run_fwd(gpu_lib, w, q, k, v)
    eo, elx = oracle_fwd(w, q, k, v)
    compare("O", o, eo, w.dtype)
    compare("LSE", lse, elx, w.dtype)


# ------------------------------------------------ full-size, every head

def compare_heads(name, got, exact, dtype):
    """compare() over the whole tensor, after logging the worst head."""
    g = got.detach().double().cpu().numpy()
    e = np.asarray(exact)
    err = np.abs(g - e).reshape(e.shape[0] * e.shape[1], -1)
    worst = int(np.argmax(err.max(axis=1)))
    log("  %-4s worst head (b=%d, h=%d): max|err| %.3e mean|err| %.3e" % (
        name, worst // e.shape[1], worst % e.shape[1], float(err[worst].max()),
        float(err[worst].mean())))
    del g, err
    compare(name, got, exact, dtype)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mid_fwdbwd_causal", "train_dropout"])
def test_full_size_fwd_bwd_every_head(gpu_lib, name):
    """The mid-size causal shape (8 x 16 x 2048 x 128) and the training shape
    (4 x 32 x 4096 x 128, causal, dropout 0.1) in the benchmark's launch
    configuration: every element of O, LSE, dQ, dK, dV of every (b, h),
    for 16-bit and for fp32 outputs, against one oracle evaluation."""
    w = workloads.WORKLOADS[name]
    log("case %s (every head)" % w.name)
    q, k, v, do = workloads.draw(w)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    for out_f32 in (False, True):
        o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do, out_f32=out_f32)
        log(" out_f32=%d" % out_f32)
        for nm, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                               ("dK", dk, edk), ("dV", dv, edv)):
            compare_heads(nm, got, exact, w.dtype)
        del o, lse, dq, dk, dv
        torch.cuda.empty_cache()


LONG_HD = [Workload("long_d%d_%s" % (d, dt), 1, 8, 4096, d, dt, causal=True, dropout_p=0.1,
                    backward=True, seed=5 + d, dropout_seed=workloads.DROPOUT_SEED)
           for d in (32, 96, 256) for dt in ("bf16", "f16")]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", LONG_HD, ids=[w.name for w in LONG_HD])
def test_full_length_other_head_dims(gpu_lib, w):
    """d = 32, 96 and 256 at the training sequence length (1 x 8 x 4096, causal,
    dropout 0.1; the layouts of those head dimensions: 64-key forward steps
    with dropout at d = 96, one workgroup per CU at d = 256, 64-key dK/dV and
    32-row dQ blocks at d = 256): every element of O, LSE, dQ, dK, dV."""
    log("case %s (every head)" % w.name)
    q, k, v, do = workloads.draw(w)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    for nm, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                           ("dK", dk, edk), ("dV", dv, edv)):
        compare_heads(nm, got, exact, w.dtype)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["long_causal_4k", "long_causal_16k"])
def test_long_context_forward_every_head(gpu_lib, name):
    """Long causal forward, 1 x 32 x N x 128 at N = 4096 and 16384: every
    element of O and LSE of all 32 heads."""
    w = workloads.WORKLOADS[name]
    log("case %s (every head)" % w.name)
    q, k, v, _ = workloads.draw(w)
    o, lse = run_fwd(gpu_lib, w, q, k, v)
    eo, elx = oracle_fwd(w, q, k, v)
    compare_heads("O", o, eo, w.dtype)
    compare_heads("LSE", lse, elx, w.dtype)


@pytest.mark.parametrize("dt,causal", [("f16", True), ("f16", False), ("bf16", False)])
def test_full_size_forward_fp16_and_noncausal(gpu_lib, dt, causal):
    """1 x 32 x 4096 x 128 without dropout (64-key steps): fp16 inputs
    causal and not, and the non-causal bf16 case, two heads compared
    element by element."""
    w = Workload("full8_%s_c%d" % (dt, causal), 1, 32, 4096, 128, dt, causal=causal, seed=41 + causal)
    heads = [(0, 0), (0, 17)]
    log("case %s heads %s" % (w.name, heads))
    q, k, v, _ = workloads.draw(w)
    o, lse = run_fwd(gpu_lib, w, q, k, v)
    eo, elx = oracle_fwd(w, q, k, v, heads=heads)
    for b, h in heads:
        compare("O", o[b, h], eo[b, h], w.dtype)
        compare("LSE", lse[b, h], elx[b, h], w.dtype)


def rows_65536_sample(N, tile=1024, seed=65536):
    """Rows 0-255, every tile-boundary row +-1 at stride `tile`, the last 256
    rows and 1024 seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(0, 256)) | set(range(N - 256, N))
    for t in range(tile, N, tile):
        rows |= {t - 1, t, t + 1}
    rows |= set(int(x) for x in rng.choice(N, size=1024, replace=False))
    return sorted(rows)


@pytest.mark.timeout(900)
def test_long_context_65536_sampled_rows(gpu_lib):
    """N=65536: rows are independent in the forward, so a seeded sample of
    rows of heads 0, 13 and 31 is compared: rows 0-255, every 1024-row
    boundary +-1, the last 256 rows and 1024 random rows.  The call adds
    only O and LSE to device memory: the caching allocator grows by the two
    outputs and the device loses nothing beyond what that allocator reserved
    (the library allocates nothing), where one bf16 score matrix per head
    would take 256 GiB."""
    w = workloads.WORKLOADS["long_causal_64k"]
    log("case %s" % w.name)
    q, k, v, _ = workloads.draw(w)
    qd, kd, vd = q.to("cuda"), k.to("cuda"), v.to("cuda")
    torch.cuda.synchronize()
    free0, res0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved(), torch.cuda.memory_allocated()
    o, lse = gpu_lib.fwd(qd, kd, vd, scale=w.softmax_scale, causal=w.causal)
    torch.cuda.synchronize()
    free1, res1, alloc1 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved(), torch.cuda.memory_allocated()
    out_bytes = o.numel() * o.element_size() + lse.numel() * 4
    assert out_bytes == w.B * w.H * w.N * (w.d * 2 + 4)
    assert out_bytes <= alloc1 - alloc0 <= out_bytes + (1 << 20)
    assert free0 - free1 <= (res1 - res0) + (2 << 20)
    del qd, kd, vd
    rows = rows_65536_sample(w.N)
    log(" %d rows per head" % len(rows))
    for b, h in [(0, 0), (0, 13), (0, 31)]:
        eo, elx = oracle.fwd_rows(q, k, v, b, h, rows, w.softmax_scale, w.causal)
        log(" head (%d, %d)" % (b, h))
        compare("O", o[b, h, rows], eo, w.dtype)
        compare("LSE", lse[b, h, rows], elx, w.dtype)


# -------------------------------------------- largest head the API accepts

# One head of [MAXN, 128] bf16 is 2^31 - 16384 bytes, the largest the library
# accepts (it addresses a head with signed 32-bit byte offsets).
MAXN = 2 ** 23 - 64


class Stats:
    """Running max / mean of |got - exact| over chunks, with compare()'s bars."""

    def __init__(self, name, dtype):
        self.name, self.dtype, self.mx, self.mx_ex, self.s, self.n = name, dtype, 0.0, 0.0, 0.0, 0

    def add(self, got, exact):
        g = got.detach().double().cpu().numpy()
        e = np.asarray(exact)
        assert np.isfinite(g).all(), "%s has non-finite values" % self.name
        err = np.abs(g - e)
        slack = half_ulp(e, got.dtype) if got.dtype != torch.float32 else 0.0
        self.mx = max(self.mx, float(err.max(initial=0.0)))
        self.mx_ex = max(self.mx_ex, float((err - slack).max(initial=0.0)))
        self.s += float(err.sum())
        self.n += err.size

    def check(self):
        tmax, tmean = TOL[self.dtype]
        mean = self.s / max(1, self.n)
        log("  %-4s max|err| %.3e (less storage %.3e) mean|err| %.3e over %d elements" % (
            self.name, self.mx, self.mx_ex, mean, self.n))
        assert self.mx_ex <= tmax and mean <= tmean, self.name


@pytest.mark.timeout(900)
def test_largest_key_head_decoding(gpu_lib):
    """16 queries over MAXN keys (causal, aligned on the last key): byte
    offsets into K, V, dK and dV reach 2^31 - 16384.  Forward (one pass and
    split keys) and backward against the oracle; dK and dV compared on the
    first, last and evenly spaced key rows."""
    w = Workload("maxk", 1, 1, 16, 128, "bf16", causal=True, seed=77)
    log("case 16 queries over %d keys" % MAXN)
    q, k, v, do = workloads.draw_cross(w, MAXN, with_dout=True)
    dev = "cuda"
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = gpu_lib.fwd(qd, kd, vd, scale=w.softmax_scale, causal=True)
    os_, lses = gpu_lib.fwd_splitkv(qd, kd, vd, 64, scale=w.softmax_scale, causal=True)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o, lse, dod, scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    del kd, vd
    edq, edk, edv, eo, el = oracle.bwd(q, k, v, do, w.softmax_scale, True, 0.0, 0)
    for name, got, exact in (("O", o, eo), ("LSE", lse, el), ("O", os_, eo), ("LSE", lses, el),
                             ("dQ", dq, edq)):
        compare(name, got, exact, "bf16")
    rows = sorted(set(range(0, 512)) | set(range(MAXN - 512, MAXN)) |
                  set(np.linspace(0, MAXN - 1, 4096).astype(int).tolist()))
    for name, got, exact in (("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got[:, :, rows], exact[:, :, rows], "bf16")


@pytest.mark.timeout(900)
def test_largest_query_head(gpu_lib):
    """MAXN queries over 64 keys (not causal): byte offsets into Q, O, dO and
    dQ reach 2^31 - 16384.  Rows are independent here, so the oracle runs
    over chunks of rows (concurrently: the oracle's C calls release the
    interpreter lock): O, LSE and dQ compared with the usual bars on the
    first and last chunks and 512 seeded rows of every other chunk, dK and
    dV against the sum of every chunk's contributions.
    Each of the 64 dK, dV rows sums 8.4 million query rows (|dK| reaches a
    few hundred), so the absolute bars of the target workloads (N <= 65536)
    measure the accumulation length there, not the method: dK and dV are
    held to the accuracy of their bf16 matrix-core operands instead --
    max error <= 2^-7 max|exact|, mean error <= 2^-8 mean|exact| per tensor.
    An addressing error would show as errors of the order of the values."""
    w = Workload("maxq", 1, 1, MAXN, 128, "bf16", causal=False, seed=78)
    log("case %d queries over 64 keys" % MAXN)
    q, k, v, do = workloads.draw_cross(w, 64, with_dout=True)
    dev = "cuda"
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = gpu_lib.fwd(qd, kd, vd, scale=w.softmax_scale)
    dq, dk, dv = gpu_lib.bwd(qd, kd, vd, o, lse, dod, scale=w.softmax_scale)
    torch.cuda.synchronize()
    del qd, dod
    st = {n: Stats(n, "bf16") for n in ("O", "LSE", "dQ")}
    edk = np.zeros((1, 1, 64, 128))
    edv = np.zeros((1, 1, 64, 128))
    step = 1 << 17
    rng = np.random.default_rng(78)
    chunks = [(r0, min(MAXN, r0 + step)) for r0 in range(0, MAXN, step)]

    def run_chunk(c):
        r0, r1 = c
        return oracle.bwd(q[:, :, r0:r1], k, v, do[:, :, r0:r1], w.softmax_scale, False, 0.0, 0)

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
        for (r0, r1), (cdq, cdk, cdv, co, cl) in zip(chunks, ex.map(run_chunk, chunks)):
            edk += cdk
            edv += cdv
            if r0 == 0 or r1 == MAXN:
                sel = np.arange(r1 - r0)
            else:
                sel = np.sort(rng.choice(r1 - r0, size=512, replace=False))
            rows = torch.from_numpy(r0 + sel)
            st["O"].add(o[:, :, rows], co[:, :, sel])
            st["LSE"].add(lse[:, :, rows], cl[:, :, sel])
            st["dQ"].add(dq[:, :, rows], cdq[:, :, sel])
    for s_ in st.values():
        s_.check()
    for name, got, exact in (("dK", dk, edk), ("dV", dv, edv)):
        err = np.abs(got.double().cpu().numpy() - exact)
        mx, mean = float(np.abs(exact).max()), float(np.abs(exact).mean())
        log("  %-4s max|err| %.3e (max|x| %.2f) mean|err| %.3e (mean|x| %.2f)" % (
            name, err.max(), mx, err.mean(), mean))
        assert float(err.max()) <= 2.0 ** -7 * mx and float(err.mean()) <= 2.0 ** -8 * mean, name


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("N", [1, 2, 63, 65, 127, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.2])
def test_ragged_lengths(gpu_lib, N, causal, p):
    """Sequence lengths around the tile sizes (32-key steps with dropout,
    64-key steps without it at d = 128)."""
    w = Workload("ragged", 1, 2, N, 128, "bf16", causal=causal, dropout_p=p, backward=True,
                 seed=N, dropout_seed=N * 31 + 7)
    q, k, v, do = workloads.draw(w)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    for name, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                             ("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got, exact, w.dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 64), ("bf16", 128), ("f16", 128)])
def test_single_key_returns_value_exactly(gpu_lib, dtype, d):
    """N = 1: exp(0) = 1 and l = 1, so O must equal V bit for bit and
    LSE = scale q.k; dV = dO bit for bit and dQ = dK = 0 (to rounding)."""
    w = Workload("n1", 3, 4, 1, d, dtype, causal=True, backward=True, seed=99)
    q, k, v, do = workloads.draw(w)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    assert torch.equal(o.cpu(), v)
    assert torch.equal(dv.cpu(), do)
    # dS = P (dP - D) is zero only up to fp32 rounding of dO.V against dO.O.
    assert float(dq.abs().max()) <= 1e-5 and float(dk.abs().max()) <= 1e-5
    ref = w.softmax_scale * (q.double() * k.double()).sum(-1)
    assert float((lse.cpu().double() - ref).abs().max()) < 1e-5


def test_zero_query_gives_prefix_mean(gpu_lib):
    w = Workload("q0", 1, 2, 333, 128, "bf16", causal=True, seed=5)
    _, k, v, _ = workloads.draw(w)
    q = torch.zeros_like(k)
    o, lse = run_fwd(gpu_lib, w, q, k, v)
    vv = v.double().numpy()
    counts = np.arange(1, w.N + 1)
    expect = np.cumsum(vv, axis=2) / counts[None, None, :, None]
    compare("O", o, expect, "bf16")
    compare("LSE", lse, np.broadcast_to(np.log(counts), lse.shape), "bf16")


def test_empty_problem(gpu_lib):
    q = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = gpu_lib.fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (2, 2, 0)
    dq, dk, dv = gpu_lib.bwd(q, q, q, o, lse, q)
    assert dq.shape == q.shape


# fp32 outputs from the 16-bit kernels: every head dimension (each has its
# own epilogue instantiation; d = 256 dQ its own translation unit).
OUT_F32 = [(32, "bf16", True, 0.1), (64, "f16", True, 0.1), (96, "bf16", True, 0.1),
           (128, "bf16", True, 0.1), (256, "f16", True, 0.1), (256, "bf16", False, 0.0)]


@pytest.mark.parametrize("d,dt,causal,p", OUT_F32,
                         ids=["d%d_%s_c%d_p%g" % c for c in OUT_F32])
def test_out_f32_matches_oracle(gpu_lib, d, dt, causal, p):
    w = Workload("outf32", 1, 2, 200, d, dt, causal=causal, dropout_p=p, backward=True,
                 seed=21 + d, dropout_seed=4)
    q, k, v, do = workloads.draw(w)
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do, out_f32=True)
    assert o.dtype == torch.float32 and dq.dtype == torch.float32
    assert dk.dtype == torch.float32 and dv.dtype == torch.float32
    edq, edk, edv, eo, elx = oracle_bwd(w, q, k, v, do)
    for name, got, exact in (("O", o, eo), ("LSE", lse, elx), ("dQ", dq, edq),
                             ("dK", dk, edk), ("dV", dv, edv)):
        compare(name, got, exact, dt)


def test_runs_on_the_callers_stream(gpu_lib):
    """Work goes to the caller's current stream: inputs produced on a side
    stream (default priority) right before the calls, forward and backward
    enqueued on it, give bitwise the default-stream results (both passes
    are deterministic)."""
    w = Workload("stream", 2, 4, 640, 128, "bf16", causal=True, dropout_p=0.1, backward=True,
                 seed=12, dropout_seed=0x5EED)
    q, k, v, do = workloads.draw(w)
    ref = run_bwd(gpu_lib, w, q, k, v, do)
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        # the inputs are rewritten on the side stream just before the calls
        q2, k2, v2, do2 = (t * 1.0 for t in (qd, kd, vd, dod))
        o, lse = gpu_lib.fwd(q2, k2, v2, scale=w.softmax_scale, causal=w.causal,
                             dropout_p=w.dropout_p, seed=w.dropout_seed)
        dq, dk, dv = gpu_lib.bwd(q2, k2, v2, o, lse, do2, scale=w.softmax_scale, causal=w.causal,
                                 dropout_p=w.dropout_p, seed=w.dropout_seed)
    side.synchronize()
    for name, got, want in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), ref):
        assert torch.equal(got, want), name


def test_forward_is_deterministic(gpu_lib):
    w = workloads.WORKLOADS["train_dropout"]
    w = Workload("det", 2, 4, 1024, 128, "bf16", causal=True, dropout_p=0.1, seed=3,
                 dropout_seed=w.dropout_seed)
    q, k, v, _ = workloads.draw(w)
    o1, l1 = run_fwd(gpu_lib, w, q, k, v)
    o2, l2 = run_fwd(gpu_lib, w, q, k, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_backward_is_deterministic(gpu_lib, d):
    """No atomics anywhere: two backward runs on the same inputs agree bit for
    bit (a race between the wavefronts sharing LDS buffers would show here)."""
    w = Workload("detb", 2, 4, 1000, d, "bf16", causal=True, dropout_p=0.1, backward=True,
                 seed=11, dropout_seed=77)
    log("case detb d=%d" % d)
    q, k, v, do = workloads.draw(w)
    r1 = run_bwd(gpu_lib, w, q, k, v, do)
    r2 = run_bwd(gpu_lib, w, q, k, v, do)
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), r1, r2):
        assert torch.equal(x, y), "%s differs between two runs" % name


# ------------------------------------------------------ bit-exact probes

def test_dropout_mask_bit_exact_full_planes(gpu_lib):
    """The device generator reproduces the oracle's keep mask bit for bit on
    whole (b, h) planes of the training workload."""
    w = workloads.WORKLOADS["train_dropout"]
    for b, h in [(0, 0), (3, 31), (2, 17)]:
        got = gpu_lib.dropout_mask(w.B, w.H, w.N, w.dropout_p, w.dropout_seed, b, h).cpu().numpy()
        exact = oracle.dropout_mask(w.N, p32(w.dropout_p), w.dropout_seed, b, h)
        log("  plane (%d,%d) kept %.5f mismatches %d" % (b, h, got.mean(), int((got != exact).sum())))
        assert np.array_equal(got, exact)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_identity_values_expose_zero_pattern(gpu_lib, d, p):
    """N = d and V = I: O[i, j] = P~[i, j], which must be exactly zero iff
    key j is masked (j > i) or dropped."""
    N = d
    w = Workload("ident", 2, 2, N, d, "bf16", causal=True, dropout_p=p, seed=d,
                 dropout_seed=1234 + d)
    q, k, _, _ = workloads.draw(w)
    v = torch.eye(N, dtype=torch.bfloat16).expand(2, 2, N, N).contiguous()
    o, _ = run_fwd(gpu_lib, w, q, k, v)
    for b in range(2):
        for h in range(2):
            keep = oracle.dropout_mask(N, p32(p), w.dropout_seed, b, h).astype(bool)
            visible = np.tril(np.ones((N, N), dtype=bool)) & keep
            got = o[b, h].float().cpu().numpy() != 0.0
            assert np.array_equal(got, visible)


@pytest.mark.parametrize("p,H", [(0.1, 2), (0.0, 32)])
def test_tile_boundary_probe_at_full_shape(gpu_lib, p, H):
    """Training shape: V has one-hot columns on 128 keys at tile boundaries,
    so O[:, c] = P~[:, probe_c] and its zero pattern must equal the oracle's
    keep & causal pattern exactly; dO one-hot on the probe rows exposes rows
    of P~ through dV.  Without dropout, 32 heads (64-key steps)."""
    w0 = workloads.WORKLOADS["train_dropout"]
    B, N, d = 1, w0.N, w0.d
    w = Workload("probe", B, H, N, d, "bf16", causal=True, dropout_p=p,
                 backward=True, seed=17, dropout_seed=w0.dropout_seed)
    q, k, _, _ = workloads.draw(w)
    probes = []
    for t in np.linspace(1, N // 32 - 1, 43).astype(int) * 32:
        probes += [int(t) - 1, int(t), int(t) + 1]
    probes = sorted(set(x for x in probes if 0 <= x < N))[:d]
    assert len(probes) == d
    v = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    do = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    for c, j in enumerate(probes):
        v[:, :, j, c] = 1.0
        do[:, :, j, c] = 1.0
    o, lse, dq, dk, dv = run_bwd(gpu_lib, w, q, k, v, do)
    rows = np.arange(N)
    o_h, dv_h = o.float().cpu().numpy(), dv.float().cpu().numpy()
    for h in range(H):
        if p > 0:
            keep = oracle.dropout_mask(N, p32(w.dropout_p), w.dropout_seed, 0, h).astype(bool)
        else:
            keep = np.ones((N, N), dtype=bool)
        for c, j in enumerate(probes):
            col_expect = keep[:, j] & (rows >= j)      # P~[:, j] != 0
            col_got = o_h[0, h, :, c] != 0
            assert np.array_equal(col_got, col_expect), (h, c, j)
            row_expect = keep[j, :] & (rows <= j)      # P~[j, :] != 0
            row_got = dv_h[0, h, :, c] != 0
            assert np.array_equal(row_got, row_expect), (h, c, j)
