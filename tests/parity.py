"""Parity helpers shared by the GPU tests.

Tolerances (stated once, used everywhere):
* integer outputs (CSR, row windows): bit-exact;
* fp32 forward: componentwise  max |y - y*| / max(|y*|, S) <= 1e-5, where y*
  is the fp64 oracle on the same inputs and S = sum_p alpha_p |v_p| is the
  oracle's magnitude of the same sum (the relative error of a sum is bounded
  relative to the sum of magnitudes, not to the possibly cancelled result);
  destinations without in-edges must be exactly 0;
* fp16 forward: relative L2 error ||y - y*|| / ||y*|| <= 2e-3;
* bf16 forward: relative L2 error <= 8e-3.
The oracle always reads the rounded fp16 / bf16 inputs, widened exactly.
"""
import functools

import numpy as np
import torch

import oracle
import workloads as W

FP32_TOL = 1e-5
REL_L2_TOL = {"f16": 2e-3, "bf16": 8e-3}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def componentwise(y, ref, mag):
    y, ref, mag = (np.asarray(x, np.float64) for x in (y, ref, mag))
    denom = np.maximum(np.abs(ref), mag)
    zero = denom == 0
    assert np.all(y[zero] == 0.0), "destinations without in-edges must give exactly 0"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(y - ref)[~zero] / denom[~zero]).max())


def rel_l2(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        assert np.all(y == 0)
        return 0.0
    return float(np.linalg.norm(y - ref) / nr)


def check_forward(y_gpu: torch.Tensor, ref, mag, dtype: str, rows=None):
    y = y_gpu.detach().float().cpu().double().numpy()
    if rows is not None:
        y = y[rows]
    if dtype == "f32":
        err = componentwise(y, ref, mag)
        assert err <= FP32_TOL, f"fp32 componentwise error {err:.3e} > {FP32_TOL}"
    else:
        err = rel_l2(y, ref)
        assert err <= REL_L2_TOL[dtype], f"{dtype} relative L2 error {err:.3e} > {REL_L2_TOL[dtype]}"
        # zero rows stay exactly zero
        deg0 = np.all(ref == 0, axis=(1, 2))
        assert np.all(y[deg0] == 0.0)
    return err


class Case:
    """A workload with its oracle CSR and its rounded inputs on CPU and GPU."""

    def __init__(self, wl: W.Workload, device="cuda"):
        self.wl = wl
        self.n, self.h, self.d = wl.num_nodes, wl.heads, wl.head_dim
        self.rp, self.ci, self.pe = oracle.build_csr(wl.num_nodes, wl.src, wl.dst)
        tq, tk, tv = (W.cast(x, wl.dtype) for x in (wl.q(), wl.k(), wl.v()))
        self.q, self.k, self.v = (t.to(device) for t in (tq, tk, tv))
        self.q64, self.k64, self.v64 = (oracle.widen(t) for t in (tq, tk, tv))
        self.e = self.e64 = None
        if wl.has_e:
            te = W.cast(wl.e(), wl.dtype)          # drawn per CSR position
            self.e = te.to(device)
            self.e64 = oracle.widen(te)
        self.src = torch.from_numpy(wl.src).to(device)
        self.dst = torch.from_numpy(wl.dst).to(device)

    def oracle_forward(self, rows=None, threads=8):
        wl = self.wl
        return oracle.forward(self.rp, self.ci, self.q64, self.k64, self.v64, self.e64, mode=wl.mode,
                              scale=wl.scale, clip=wl.clip, eps=wl.eps, rows=rows, want_mag=True,
                              threads=threads)


@functools.lru_cache(maxsize=4)
def case(config: int) -> Case:
    return Case(W.make(config))
