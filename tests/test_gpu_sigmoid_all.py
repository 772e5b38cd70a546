"""Every finite binary32 input through the sigmoid evaluations of the routing kernels
(mep_sigmoid_eval, the device functions the kernels inline), checked once over all
2^32 - 2^24 finite bit patterns:

- the correctly rounded sigmoid, bit-exact against the oracle (oracle.sigmoid: binary64 with a
  rounding test, binary128 where that test cannot decide).  The scoring function is the logistic
  sigmoid of [TRT] RoutingKernel.cuh (sigmoid_accurate); selection keys are formed from this
  value, so every id the exact path picks rests on it;
- the binary32 filter value s~ = rcp(1 + exp2(-x log2 e)) of the certified fast selection: its
  largest |s~ - sigma| must stay within the 3.23 * 2^-23 the certificates assume (derived from
  the instruction set's 1-ulp figure for v_exp_f32 / v_rcp_f32);
- the binary64 sigmoid of the routing weights: relative error below 2^-30 wherever sigma is a
  normal binary32 number.
sigma for the two error measurements is 1 / (1 + exp(-x)) in binary64 (numpy; a few ulp of
2^-53 relative), far below the bounds tested.  The measured maxima are printed (run with -s).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from expert_dispatch_layout_amd import _binding as B  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHUNK = 1 << 24                    # bit patterns per chunk: 256 chunks
FILTER_BOUND = 3.23 * 2.0 ** -23
WEIGHT_BOUND = 2.0 ** -30


def _chunk_range(c):
    """Bit patterns [lo, hi) of chunk c without the non-finite ones (exponent field 255, the
    upper half of every chunk whose seven high exponent bits are all ones)."""
    lo = c * CHUNK
    hi = lo + CHUNK
    if (c & 0x7F) == 0x7F:
        hi = lo + CHUNK // 2
    return lo, hi


def _check_chunk(lo, hi, cr, filt, wgt):
    x = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32)
    want = oracle.sigmoid(x)
    bad = np.nonzero(cr.view(np.uint32) != want.view(np.uint32))[0]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    ferr = float(np.max(np.abs(filt.astype(np.float64) - s)))
    normal = s >= 2.0 ** -126
    werr = float(np.max(np.abs(wgt[normal] - s[normal]) / s[normal])) if normal.any() else 0.0
    first = None if bad.size == 0 else (hex(int(lo + bad[0])), float(cr[bad[0]]), float(want[bad[0]]))
    return bad.size, first, ferr, werr


def test_sigmoid_every_finite_fp32_input():
    workers = max(1, min(16, os.cpu_count() or 1))
    oracle.lib()  # loaded once here, before the worker threads call it
    xd = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    crd = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    fd = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    wd = torch.empty(CHUNK, dtype=torch.float64, device=DEV)
    bits = torch.arange(CHUNK, dtype=torch.int64, device=DEV)
    total_bad, first_bad, max_ferr, max_werr, count = 0, None, 0.0, 0.0, 0
    pending = []

    def drain(limit):
        nonlocal total_bad, first_bad, max_ferr, max_werr
        while len(pending) > limit:
            nb, fb, fe, we = pending.pop(0).result()
            total_bad += nb
            first_bad = first_bad or fb
            max_ferr = max(max_ferr, fe)
            max_werr = max(max_werr, we)

    with ThreadPoolExecutor(workers) as pool:
        for c in range((1 << 32) // CHUNK):
            lo, hi = _chunk_range(c)
            n = hi - lo
            # the bit patterns lo .. hi-1 as float32 (as signed 32-bit integers first)
            v = bits[:n] + lo
            v = torch.where(v >= (1 << 31), v - (1 << 32), v)
            xd[:n].copy_(v.to(torch.int32).view(torch.float32))
            B.mep_sigmoid_eval(xd[:n], crd[:n], fd[:n], wd[:n])
            cr, filt, wgt = crd[:n].cpu().numpy(), fd[:n].cpu().numpy(), wd[:n].cpu().numpy()
            count += n
            pending.append(pool.submit(_check_chunk, lo, hi, cr, filt, wgt))
            drain(2 * workers)
        drain(0)
    assert count == (1 << 32) - (1 << 24)
    print("\nfinite inputs %d: correctly rounded mismatches %d; filter max |s~ - sigma| = %.4g = %.4f * 2^-23;"
          " weights max relative error = %.3g = 2^%.2f" % (count, total_bad, max_ferr, max_ferr * 2.0 ** 23,
                                                           max_werr, np.log2(max_werr) if max_werr > 0 else -np.inf))
    assert total_bad == 0, first_bad
    assert max_ferr <= FILTER_BOUND, max_ferr
    assert max_werr < WEIGHT_BOUND, max_werr
