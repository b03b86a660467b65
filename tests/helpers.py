"""Shared test helpers: numpy <-> torch bf16 moves and parity comparisons.

bf16 data is numpy uint16 (bit patterns) on the host and torch.bfloat16 on
the GPU; transfers reinterpret the bits, never convert values.
"""

import numpy as np


def to_dev(a, dtype=None):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t):
    import torch

    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        n = bad.shape[0]
        first = [tuple(int(i) for i in b) for b in bad[:5]]
        vals = [(hex(int(got[tuple(b)])), hex(int(want[tuple(b)]))) for b in bad[:5]]
        raise AssertionError(f"{what}: {n} of {got.size} elements differ; first at {first}: got/want {vals}")


def projection_tolerance_ok(C, Cstar, rel=1e-2):
    """The projection's bar: per layer ||C - C*||_F / ||C*||_F <= rel, and per
    element |C - C*| <= rel (|C*| + rms of the row of C*). C bf16 bits or
    float, C* float32 (the oracle's FP32 sums). Returns (ok, message)."""
    C = f32(C) if C.dtype == np.uint16 else np.asarray(C, dtype=np.float32)
    Cs = np.asarray(Cstar, dtype=np.float64)
    Cd = C.astype(np.float64)
    L = Cs.shape[0]
    for l in range(L):
        num = np.linalg.norm(Cd[l] - Cs[l])
        den = np.linalg.norm(Cs[l])
        if den > 0 and num / den > rel:
            return False, f"layer {l}: relative Frobenius error {num / den:.3e} > {rel}"
        if den == 0 and num > 0:
            return False, f"layer {l}: nonzero output for an all-zero reference"
    rms = np.sqrt(np.mean(Cs ** 2, axis=-1, keepdims=True))
    err = np.abs(Cd - Cs)
    lim = rel * (np.abs(Cs) + rms)
    if not np.all(err <= lim):
        i = tuple(int(v) for v in np.argwhere(err > lim)[0])
        return False, f"element {i}: |{Cd[i]} - {Cs[i]}| > {lim[i]}"
    return True, ""


def oracle_norms_chunked(oracle, x, hidden_w, pre_w, L, hidden_eps=1e-6, pre_eps=1e-6, chunk=1024, each=None):
    """The oracle's norms over row chunks on a thread pool (the oracle's C
    routine releases the GIL; each row is normalised on its own, so chunking
    changes nothing). Returns [L, T, 8192] bf16 bits, or, with `each`, calls
    each(r0, r1, out_chunk) per chunk instead of assembling the whole output."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    T = x.shape[0]
    starts = list(range(0, T, chunk))
    out = None if each is not None else np.empty((L, T, x.shape[1]), dtype=np.uint16)

    def one(r0):
        r1 = min(T, r0 + chunk)
        o = oracle.context_norms(np.ascontiguousarray(x[r0:r1]), hidden_w, pre_w, L, hidden_eps, pre_eps)
        if each is not None:
            each(r0, r1, o)
        else:
            out[:, r0:r1] = o

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, starts))
    return out
