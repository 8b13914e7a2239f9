"""Shared helpers of the GPU parity tests."""
import os
import sys

import numpy as np
import torch

import oracle

ATOL = 2e-3      # absolute bound on fp16/bf16 outputs (fp32 accumulate)
RTOL = 1e-2      # relative bound

# One entry per assert_close call: (test id, case, max_abs, max_rel, worst err/tol).
# tests/conftest.py prints the worst case per test file at the end of the run.
MARGINS = []


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """|gpu - oracle| <= max(ATOL, RTOL*|oracle|) per element, against the unrounded
    fp64 oracle; reports max abs and max rel error."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = np.abs(got - ref)
    tol = np.maximum(ATOL, RTOL * np.abs(ref))
    bad = err > tol
    rel = err / np.maximum(np.abs(ref), 1e-30)
    big = np.abs(ref) > 1e-2
    max_rel = float(rel[big].max()) if big.any() else 0.0
    max_abs = float(err.max()) if err.size else 0.0
    ratio = float((err / tol).max()) if err.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    MARGINS.append((test, what, max_abs, max_rel, ratio))
    say(f"  {what}: max_abs={max_abs:.3e} max_rel(|ref|>1e-2)={max_rel:.3e} "
        f"worst err/tol={ratio:.3f} n={got.size}")
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={ref[i]!r}")


def gpu_out(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().double().cpu().numpy()


def oracle_full(w) -> np.ndarray:
    return oracle.decode(w.q, w.key_cache, w.value_cache, w.block_tables_host, w.seq_lens_host,
                         w.scale, w.dtype)


def oracle_rows(w, rows):
    """fp64 oracle on selected (seq, head) rows of a device-resident workload, from a
    compact host copy of only the pages those sequences reference."""
    seqs = sorted({s for s, _ in rows})
    local = {s: i for i, s in enumerate(seqs)}
    kp, vp, bt, sl = w.host_pages(seqs)
    q = w.q[seqs].cpu()
    lrows = [(local[s], h) for s, h in rows]
    return oracle.decode_rows(lrows, q, kp, vp, bt, sl, w.scale, w.dtype)
