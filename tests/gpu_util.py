"""Shared helpers of the GPU parity tests: oracle values on sampled outputs and the
tolerance check.  Test infrastructure only."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

G = 128


def say(*msg):
    """Name the case before a GPU step, flushed, so a failing box still tells which."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def packed_order(n, idx8):
    is8 = np.zeros(n, bool)
    is8[np.asarray(idx8, np.int64)] = True
    return np.concatenate([np.nonzero(~is8)[0], np.nonzero(is8)[0]]), is8


def sample_cols(n, idx8, rng, n4_take=160, n8_take=64):
    """4-bit and 8-bit channels, the first/last channels and the block shared by the
    two subsets (packed positions 32 * floor(n4 / 32) ..)."""
    perm, is8 = packed_order(n, idx8)
    n4 = n - len(idx8)
    four = np.nonzero(~is8)[0]
    eight = np.nonzero(is8)[0]
    pick = [0, n - 1]
    if four.size:
        pick += list(rng.choice(four, size=min(n4_take, four.size), replace=False))
    if eight.size:
        pick += list(rng.choice(eight, size=min(n8_take, eight.size), replace=False))
    b = n4 // 32
    pick += list(perm[32 * b: min(n, 32 * b + 32)])
    return np.unique(np.array(pick, dtype=np.int64))


def sample_rows(m, rng, take=12):
    pick = [0, m - 1] + list(rng.choice(m, size=min(take, m), replace=False))
    return np.unique(np.array(pick, dtype=np.int64))


def oracle_at(a16, w16, idx8, rows=None, cols=None):
    """Oracle outputs (fp64 and fp16) and partials at the given rows x cols."""
    n = w16.shape[0]
    rows = np.arange(a16.shape[0]) if rows is None else rows
    cols = np.arange(n) if cols is None else cols
    is8 = np.zeros(n, bool)
    is8[np.asarray(idx8, np.int64)] = True
    aq, sa, _ = O.quant_act(a16[rows])
    q, z, s16, _ = O.quant_weights_mixed(w16[cols], np.nonzero(is8[cols])[0])
    y64 = O.gemm_mixed(aq, sa, q, z, s16)
    return dict(aq=aq, sa=sa, q=q, z=z, s16=s16, y64=y64, y16=O.to_fp16(y64), rows=rows, cols=cols)


def partials_at(ref):
    return O.partials(ref["aq"], ref["q"], ref["z"])


def assert_y_close(y_gpu16: np.ndarray, y16: np.ndarray, what=""):
    """|Y_gpu - Y| <= 2 ulp_fp16(Y) + 1e-3 max|Y| element-wise, Y the oracle's fp16 value."""
    yg = np.asarray(y_gpu16, np.float16).astype(np.float64)
    yo = np.asarray(y16, np.float16).astype(np.float64)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite GPU output"
    tol = 2 * O.ulp_fp16(yo) + 1e-3 * np.abs(yo).max()
    err = np.abs(yg - yo)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside tolerance; worst at {i}: "
                             f"gpu {yg[i]} oracle {yo[i]} tol {tol[i]}")


def split3(x32):
    """Host-side exact three-way bf16 split of fp32 values: the words p | p << 16 of the
    pieces p0, p1, p2 (uint32), checked to sum to x exactly."""
    x32 = np.asarray(x32, np.float32)
    b0 = x32.view(np.uint32) & np.uint32(0xFFFF0000)
    r1 = (x32 - b0.view(np.float32)).astype(np.float32)
    b1 = r1.view(np.uint32) & np.uint32(0xFFFF0000)
    r2 = (r1 - b1.view(np.float32)).astype(np.float32)
    b2 = r2.view(np.uint32) & np.uint32(0xFFFF0000)
    tot = b0.view(np.float32).astype(np.float64) + b1.view(np.float32) + b2.view(np.float32)
    assert np.array_equal(tot, x32.astype(np.float64))
    return [b | (b >> np.uint32(16)) for b in (b0, b1, b2)]


def rowop_records(sa_gm, u_gm):
    """The row operand records [G][M][8] of s_a and u = fp32(S_A s_a):
    {w(s0), w(s1), w(s2), 0, w(u0), w(u1), w(u2), 0}."""
    s0, s1, s2 = split3(sa_gm)
    u0, u1, u2 = split3(u_gm)
    z = np.zeros_like(s0)
    return np.stack([s0, s1, s2, z, u0, u1, u2, z], axis=-1)
