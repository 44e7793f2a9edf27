"""Shared helpers for the GPU parity tests: device transfer, running the
library through its C ABI, and the error statistics with their tolerances."""
import sys

import numpy as np
import torch

# Tolerances for the HIP path against the fp64 oracle.
FWD_MAX_ABS = 1e-2   # bf16 / fp16 inputs, output O
FWD_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_FRO = 2e-2  # per gradient tensor, relative Frobenius norm
F32_MAX_ABS = 1e-5   # fp32 path, output O and LSE
F32_GRAD_REL_FRO = 1e-5


def say(msg: str) -> None:
    """Name the case on stdout (flushed) before its GPU work starts."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x):
    return None if x is None else x.contiguous().cuda()


def run_fwd(inp, scale, causal, out_dtype=None):
    from exact_io_aware_07_amd import attention_forward
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    kv = dev(inp.get("kv_len"))
    o, lse = attention_forward(q, k, v, causal=causal, kv_len=kv, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


def run_bwd(inp, o, lse, scale, causal):
    from exact_io_aware_07_amd import attention_backward
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    kv = dev(inp.get("kv_len"))
    dq, dk, dv = attention_backward(q, k, v, o, do, lse, causal=causal, kv_len=kv, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def fwd_stats(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    err = np.abs(o_gpu - o_ref)
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), inf_ref), "-inf LSE rows differ"
    fin = ~inf_ref
    lse_err = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    denom = float(np.abs(o_ref).max()) or 1.0
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "lse_max_abs": lse_err,
            "max_rel": (float(err.max()) if err.size else 0.0) / denom}


def rounding_floor(o_ref: np.ndarray, dtype: torch.dtype):
    """Error of storing the exact output in ``dtype`` (round to nearest even)."""
    r = torch.from_numpy(o_ref).to(dtype).to(torch.float64).numpy()
    e = np.abs(r - o_ref)
    return float(e.max()), float(e.mean())


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    n = float(np.linalg.norm(ref))
    return float(np.linalg.norm(x - ref)) / (n if n > 0 else 1.0)
