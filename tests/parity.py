"""Parity checks shared by the GPU tests: the HIP path against the fp64 oracle.

Two bars for bf16 outputs:

* the workload bar: max |dO| <= 1e-2 raw, the tolerance stated for bf16
  inputs, on every element of the five benchmark workloads (their outputs
  stay below |O| = 4, where the bf16 spacing alone would exceed it);
* the rounding bound, asserted element by element everywhere (workloads
  included).  The kernels round P~ to bf16 before the P~V product while the
  denominator sums the fp32 P~ (TileLang tutorial section 3.2; the forward
  blog's section 4), so each numerator term carries a relative error of at
  most 2^-8 (bf16 keeps 8 significant bits) and the normalised output differs
  from the exact one by at most 2^-8 A, where A_ic = sum_j P_ij |v_jc| (the
  oracle run on |V|).  2^-11 A more covers every fp32 rounding (scores,
  exp2, sums, rescale, division), which at these sizes stays far below it.
  The output format then rounds once more: half a bf16 spacing at the value.
  So |dO| <= (2^-8 + 2^-11) A + half_spacing(|O| + (2^-8 + 2^-11) A).

fp32 outputs: |dO| <= 1e-5.  LSE: |dLSE| <= 1e-3 everywhere.  A row that sees
no key must give O = 0 and LSE = -inf (or its sink) exactly.

Each check prints one ``PARITY`` line (JSON) with the raw maximum, its
position, the maximum against the bf16-rounded oracle (what the kernel adds
beyond the unavoidable output rounding), the count of elements above 1e-2,
the worst ratio to the rounding bound and the LSE maximum.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

import oracle

BF16_WORKLOAD_BAR = 1e-2
F32_BAR = 1e-5
LSE_BAR = 1e-3
P_ROUND = 2.0 ** -8      # bf16 relative rounding of P~
FP32_SLACK = 2.0 ** -11  # every fp32 rounding together


# every record of this session, for the parity tables at the end of the run
RECORDS = []       # forward: check()
GRAD_RECORDS = []  # backward: (check, gradient, max |error|, max |gradient|, relative L2 error)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_threads() -> int:
    """Oracle threads: the host's cores, at most 16 (a GPU machine allots 16 CPUs
    to each GPU)."""
    return max(1, min(16, os.cpu_count() or 1))


def bf16_half_spacing(x):
    """Half the distance between adjacent bf16 values around |x|."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - 7)


def round_bf16(x):
    """fp64 -> nearest bf16 (ties to even), returned as fp64."""
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def rounding_bound(o_ref, a_ref):
    e = (P_ROUND + FP32_SLACK) * np.asarray(a_ref, np.float64)
    return e + bf16_half_spacing(np.abs(o_ref) + e) + 1e-7


def reference(q, k, v, scale, causal, **kw):
    """The oracle's (O, LSE) and A = the oracle's O for |V| (same softmax
    weights), for the rounding bound.  q, k, v: exact fp32 arrays."""
    kw.setdefault("nthreads", oracle_threads())
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal, **kw)
    a_ref, _ = oracle.attention(q, k, np.abs(v), scale, causal, **kw)
    return o_ref, lse_ref, a_ref


def check(o, lse, o_ref, lse_ref, dtype, what="", a_ref=None, workload=False):
    """Assert parity and print the PARITY record; returns the record.

    bf16: the rounding bound needs ``a_ref``; ``workload`` adds the raw 1e-2
    bar.  fp32: 1e-5."""
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    o_ref = np.asarray(o_ref, np.float64).reshape(o.shape)
    lse_ref = np.asarray(lse_ref, np.float64).reshape(lse.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE pattern differs"
    if empty.any():
        assert np.all(o[empty] == 0.0), f"{what}: a row without keys is not 0"
    err = np.abs(o - o_ref)
    rec = {"what": what, "dtype": dtype, "elements": int(err.size)}
    if err.size:
        i = np.unravel_index(int(np.argmax(err)), err.shape)
        rec.update(max_dO=float(err[i]), argmax=[int(x) for x in i], ref_at_max=float(o_ref[i]),
                   n_over_1e2=int((err > 1e-2).sum()))
        if dtype == "bf16":
            rec["max_dO_vs_bf16_ref"] = float(np.abs(o - round_bf16(o_ref)).max())
    fin = ~empty
    if fin.any():
        lerr = np.abs(lse[fin] - lse_ref[fin])
        j = int(np.argmax(lerr))
        rec.update(max_dLSE=float(lerr[j]), argmax_lse=[int(x) for x in np.argwhere(fin)[j]])
    else:
        rec["max_dLSE"] = 0.0
    if dtype == "f32":
        bad = err > F32_BAR
        assert not bad.any(), f"{what}: max |dO| {err.max():.3g} > {F32_BAR}"
    else:
        assert a_ref is not None or workload, f"{what}: the bf16 rounding bound needs A"
        if workload:
            assert err.max(initial=0.0) <= BF16_WORKLOAD_BAR, (
                f"{what}: max |dO| {err.max():.3g} at {rec.get('argmax')} > {BF16_WORKLOAD_BAR} "
                f"(ref {rec.get('ref_at_max')})")
        if a_ref is not None:
            tol = rounding_bound(o_ref, np.asarray(a_ref, np.float64).reshape(o.shape))
            ratio = err / tol
            rec["worst_err_over_bound"] = float(ratio.max(initial=0.0))
            if err.size:
                w = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
                assert ratio[w] <= 1.0, (f"{what}: |dO| {err[w]:.3g} at {tuple(int(x) for x in w)} above the "
                                         f"rounding bound {tol[w]:.3g} (ref {o_ref[w]:.5g}, got {o[w]:.5g})")
    assert rec["max_dLSE"] <= LSE_BAR, f"{what}: max |dLSE| {rec['max_dLSE']:.3g}"
    RECORDS.append(rec)
    say("PARITY " + json.dumps(rec))
    return rec


GRAD_REL = 1e-2  # the backward bar: 1e-2 of each gradient tensor's largest magnitude


def compare_grads(got, want, what):
    """Backward parity: every element of each gradient within GRAD_REL of the
    exact tensor's largest magnitude (plus 1e-4 absolute, for a gradient that
    is exactly zero: a single visible key makes dq and dk vanish and leaves
    rounding residue), and a relative L2 error of at most GRAD_REL."""
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        scale = max(np.abs(w).max(initial=0.0), 1e-30)
        err = np.abs(g - w).max(initial=0.0)
        # relative L2 error, the measure the pages report for their backward
        # (TileLang tutorial, section 5.4: about 1 % for dQ with bf16 atomics)
        norm = np.linalg.norm(w)
        rel2 = np.linalg.norm(g - w) / norm if norm > 0 else 0.0
        say(f"  {what}: {name} max|err| {err:.3g} of max|{name}| {scale:.3g} ({err / scale:.2e}), "
            f"rel L2 {rel2:.2e}")
        GRAD_RECORDS.append((what, name, float(err), float(scale), float(rel2)))
        assert err <= GRAD_REL * scale + 1e-4, f"{what}: {name} max|err| {err:.3g} > {GRAD_REL} x {scale:.3g}"
        assert scale < 1e-6 or rel2 <= GRAD_REL, f"{what}: {name} relative L2 error {rel2:.3g}"
