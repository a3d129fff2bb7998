"""fa_bwd_noalloc (the backward on the library's static device scratch)
against fa_bwd (the same backward on a caller workspace), through the C ABI:
two calls in a row, the second on a smaller problem, each bit for bit equal
to fa_bwd (the backward is deterministic and both run the same kernels), and
within the oracle tolerance.  Also: a problem beyond the scratch is refused
before any work is enqueued."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # the second call is smaller than the first (fewer rows: the scratch keeps
    # the first call's statistics beyond the second's rows)
    Workload("noalloc_big", 2, 8, 1000, 128, "bf16", causal=True, dropout_p=0.1, backward=True,
             seed=71, dropout_seed=0xA11C),
    Workload("noalloc_small", 1, 3, 257, 64, "bf16", causal=False, dropout_p=0.0, backward=True,
             seed=72),
]


def _run(fa, w):
    dev = "cuda"
    q, k, v, do = (t.to(dev) for t in workloads.draw(w))
    kw = dict(scale=w.softmax_scale, causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed)
    o, lse = fa.fwd(q, k, v, **kw)
    ref = fa.bwd(q, k, v, o, lse, do, **kw)
    out = tuple(torch.full_like(t, float("nan")) for t in ref)
    got = fa.bwd_noalloc(q, k, v, o, lse, do, out=out, **kw)
    torch.cuda.synchronize()
    assert all(g is o_ for g, o_ in zip(got, out))
    return ref, got


def test_noalloc_backward_matches_workspace_backward(gpu_lib):
    fa = gpu_lib
    assert fa.load().fa_bwd_noalloc_max_workspace_bytes() == 32 << 20
    for w in CASES:
        log("case %s B=%d H=%d N=%d d=%d causal=%d p=%g" % (w.name, w.B, w.H, w.N, w.d, w.causal,
                                                            w.dropout_p))
        ref, got = _run(fa, w)
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(r, g), "%s of fa_bwd_noalloc differs from fa_bwd" % name
        q, k, v, do = workloads.draw(w)
        edq, edk, edv, _, _ = oracle.bwd(q, k, v, do, w.softmax_scale, w.causal,
                                         float(np.float32(w.dropout_p)), w.dropout_seed)
        for name, g, e in zip(("dQ", "dK", "dV"), got, (edq, edk, edv)):
            err = np.abs(g.double().cpu().numpy() - e)
            half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(e), 1e-300))) - 8)
            log("  %s max|err| %.3e mean|err| %.3e" % (name, err.max(), err.mean()))
            assert float((err - half_ulp).max()) <= 2e-2 and float(err.mean()) <= 2e-3


def test_noalloc_refuses_a_problem_beyond_the_scratch(gpu_lib):
    fa = gpu_lib
    lib = fa.load()
    # 4,194,305 query rows need one 256-byte step more than the 32 MiB scratch
    p = fa.make_params(1, 1, 4194305, 64, fa.BF16, causal=True)
    fake = ctypes.c_void_p(0x10000)
    st = lib.fa_bwd_noalloc(ctypes.byref(p), *([fake] * 9), None)
    assert st == fa.FA_EINVAL
    assert "static scratch" in lib.fa_last_error().decode()
