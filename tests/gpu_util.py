"""Helpers shared by the GPU tests (device buffers and error metrics)."""
import sys

import numpy as np
import torch

F16 = np.float16


def say(*a):
    """Names the case before a GPU step, flushed, so a fault report can be traced."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(F16)
    return t.cpu().numpy()


def rel_inf(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| (infinity-norm relative error)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def quantize_rows(w, chunk=8192, workers=8):
    """oracle.quantize_w4 applied to row blocks on threads. Groups run along K
    inside one row, so the result is the same as one call on the whole matrix
    (checked by test_host_lib); it only saves time on 7B-sized matrices."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    blocks = [w[i:i + chunk] for i in range(0, w.shape[0], chunk)]
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(oracle.quantize_w4, blocks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def exact_case_weights(n, k, seed):
    """w = q * 2^-e with q in [-7, 7] (every group reaching |q| = 7) and e in
    [4, 8]: the quantiser gives back exactly (q, 2^-e)."""
    rng = np.random.default_rng(seed)
    G = k // 128
    q = rng.integers(-7, 8, size=(n, k)).astype(np.int8)
    q[:, ::128] = np.where(rng.random((n, G)) < 0.5, -7, 7)
    e = rng.integers(4, 9, size=(n, G))
    s = np.power(2.0, -e)
    w = (q.astype(np.float64) * np.repeat(s, 128, axis=1)).astype(np.float32)
    return w, q, s.astype(F16)
