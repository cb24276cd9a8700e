"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
bring results back to the host for comparison with the oracle."""
import numpy as np
import torch

import sparse_gradient_reduction_amd as sg


def run_topk(g: np.ndarray, r: np.ndarray, k: int, dev, workspace=None):
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(dev)
    P, N = g.shape
    need = sg.topk_ef_workspace_bytes(P, N, k)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    idx, val = sg.topk_ef(gd, rd, k, workspace=ws)
    torch.cuda.synchronize()
    paths = sg.topk_ef_paths(ws, P).cpu().numpy()
    return (idx.cpu().numpy().view(np.uint32), val.cpu().numpy(), rd.cpu().numpy(), paths)


def assert_bits_equal(a, b, msg=""):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (a.shape, b.shape, msg)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.nonzero(a != b)
    assert bad[0].size == 0, f"{msg}: {bad[0].size} mismatches, first at {tuple(x[0] for x in bad)}"


def reduce_tolerance(P: int, vals: np.ndarray) -> float:
    m = float(np.max(np.abs(vals))) if vals.size else 0.0
    return 1e-6 * P * m
