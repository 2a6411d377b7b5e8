"""Helpers of the GPU parity tests: device setup and comparisons against the
oracle.  Not a test module."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O
import workloads as W


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so a crash is attributable)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    import mxfp4_quantized_moe_amd as mx

    mx.load_library()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


def oracle_inputs(case: W.MoECase):
    L = case.layer
    return (O.widen(case.x, case.act_dtype), O.widen(L.router_w, L.param_dtype), O.widen(L.router_b, L.param_dtype))


def compare_routing(case: W.MoECase, gpu_idx: np.ndarray, gpu_w: np.ndarray, tau_rel: float = 1e-4):
    """Routing parity.  Tokens whose k-th / (k+1)-th logit gap is at rounding
    level (< tau * max(1, |l_k|)) are exempt from set identity; there the GPU
    may only pick experts within tau of the k-th logit.  Returns
    (n_exempt, override) where override = (idx, w) feeds the GPU's choice
    into the oracle with float64 softmax weights."""
    x, wr, br = oracle_inputs(case)
    k = case.layer.top_k
    idx, w, logits = O.route(x, wr, br, k)
    margin = O.routing_margin(logits, k)
    T = x.shape[0]
    n_exempt = 0
    srt = -np.sort(-logits, axis=1)
    for t in range(T):
        lk = srt[t, k - 1]
        tau = tau_rel * max(1.0, abs(lk))
        g = gpu_idx[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < case.layer.E, (t, g)
        if margin[t] >= tau:
            assert sorted(g.tolist()) == sorted(idx[t].tolist()), (t, g, idx[t])
            for j in range(k):
                jj = int(np.nonzero(idx[t] == g[j])[0][0])
                assert abs(gpu_w[t, j] - w[t, jj]) <= 2e-6 * max(1.0, w[t, jj]), (t, j, gpu_w[t, j], w[t, jj])
        else:
            n_exempt += 1
            assert np.all(logits[t, g] >= lk - tau), (t, g)
    sel = np.take_along_axis(logits, gpu_idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return n_exempt, (gpu_idx.astype(np.int32), z / z.sum(axis=1, keepdims=True))


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def sub_case(case: W.MoECase, rows) -> W.MoECase:
    """The same layer on a subset of tokens (tokens are independent)."""
    return W.MoECase(case.name + "_sample", case.layer, case.x[rows].copy(), case.act_dtype, case.fp8, case.x_calib)


# Float64 oracle outputs of the full-size cases, computed once per test
# session and shared by every test that compares against them (both weight
# layouts, the routed and the dense path).
_REF_CACHE = {}


def oracle_full(case: W.MoECase, x_scale=None, h_scale=None):
    """(out, idx) of the oracle over every token of the case, with its own
    routing (cached by case name and FP8 scales)."""
    key = (case.name, case.fp8, x_scale, h_scale)
    if key not in _REF_CACHE:
        note(f"oracle over all {case.T} tokens of {case.name}")
        out, parts = O.moe_forward(case.layer, case.x, case.act_dtype, fp8=case.fp8, x_scale=x_scale,
                                   h_scale=h_scale, return_parts=True)
        _REF_CACHE[key] = (out, parts["idx"])
    return _REF_CACHE[key]


def differing_sets(gpu_idx: np.ndarray, ref_idx: np.ndarray) -> np.ndarray:
    """Tokens whose chosen expert sets differ (rounding-level near-ties)."""
    return np.array([t for t in range(gpu_idx.shape[0])
                     if set(gpu_idx[t].tolist()) != set(ref_idx[t].tolist())], dtype=np.int64)


def poison(t) -> None:
    """Fill a scratch tensor with 0xFF bytes (bf16 and e4m3 NaN) so that any
    intermediate row a kernel fails to write shows up in the output."""
    t.view(-1).view(__import__("torch").uint8).fill_(0xFF)
