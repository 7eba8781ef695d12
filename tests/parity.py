"""Parity helpers shared by the GPU tests.

Tolerances (stated once, used everywhere):
* integer outputs (CSR, row windows): bit-exact;
* fp32 forward: componentwise  max |y - y*| / max(|y*|, S) <= 1e-5, where y*
  is the fp64 oracle on the same inputs and S = sum_p alpha_p |v_p| is the
  oracle's magnitude of the same sum (the relative error of a sum is bounded
  relative to the sum of magnitudes, not to the possibly cancelled result);
  destinations without in-edges must be exactly 0;
* fp16 forward: relative L2 error ||y - y*|| / ||y*|| <= 2e-3 over the whole
  output, and per element |y - y*| <= 4 u max(|y*|, S) + f, with u = 2^-11
  the unit roundoff of fp16 and f = 2^-25 the largest rounding error in its
  subnormal range;
* bf16 forward: relative L2 error <= 8e-3, and per element the same bound
  with u = 2^-8 (f = 2^-134).
The per-element bound is twice what the arithmetic allows: the output is
rounded once to the stored format (at most u |y*|), the matrix-core path also
rounds every softmax weight to it before the P.V product (at most u S in
total, since the rounded weights multiply |v| and sum to S), and the fp32
arithmetic adds far less than u S.  A wrong row, a dropped edge or a
misplaced head is off by O(S), hundreds of times the bound, even where the
whole-tensor norm would not notice it.
The oracle always reads the rounded fp16 / bf16 inputs, widened exactly.
"""
import functools

import numpy as np
import torch

import oracle
import workloads as W

FP32_TOL = 1e-5
REL_L2_TOL = {"f16": 2e-3, "bf16": 8e-3}
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
SUBNORMAL_FLOOR = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}
HALF_ELEMENT_C = 4.0
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def componentwise(y, ref, mag):
    y, ref, mag = (np.asarray(x, np.float64) for x in (y, ref, mag))
    denom = np.maximum(np.abs(ref), mag)
    zero = denom == 0
    assert np.all(y[zero] == 0.0), "destinations without in-edges must give exactly 0"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(y - ref)[~zero] / denom[~zero]).max())


def half_elementwise(y, ref, mag, dtype):
    """Largest |y - y*| / (4 u max(|y*|, S) + f) over the elements (must be
    <= 1); elements with y* = S = 0 must be exactly 0."""
    y, ref, mag = (np.asarray(x, np.float64) for x in (y, ref, mag))
    scale = np.maximum(np.abs(ref), mag)
    zero = scale == 0
    assert np.all(y[zero] == 0.0), "destinations without in-edges must give exactly 0"
    bound = HALF_ELEMENT_C * UNIT_ROUNDOFF[dtype] * scale + SUBNORMAL_FLOOR[dtype]
    if y.size == 0:
        return 0.0
    return float((np.abs(y - ref) / bound).max())


def rel_l2(y, ref):
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        assert np.all(y == 0)
        return 0.0
    return float(np.linalg.norm(y - ref) / nr)


class ForwardCheck:
    """Parity of one output tensor, fed in row chunks (so that a large output
    can be compared in full without holding every fp64 copy at once)."""

    def __init__(self, dtype: str):
        self.dtype = dtype
        self.comp = 0.0       # fp32: componentwise error
        self.elem = 0.0       # fp16 / bf16: per-element error over its bound
        self.diff2 = 0.0
        self.ref2 = 0.0
        self.rows = 0

    def add(self, y, ref, mag):
        y = np.asarray(y, np.float64)
        ref = np.asarray(ref, np.float64)
        self.rows += y.shape[0]
        if self.dtype == "f32":
            self.comp = max(self.comp, componentwise(y, ref, mag))
            assert self.comp <= FP32_TOL, f"fp32 componentwise error {self.comp:.3e} > {FP32_TOL}"
            return
        self.elem = max(self.elem, half_elementwise(y, ref, mag, self.dtype))
        assert self.elem <= 1.0, (f"{self.dtype} element error {self.elem:.3f} of its bound "
                                  f"(4u max(|y*|, S) + f, u = {UNIT_ROUNDOFF[self.dtype]:.3g})")
        self.diff2 += float(np.sum((y - ref) ** 2))
        self.ref2 += float(np.sum(ref ** 2))

    def finish(self) -> float:
        """The whole-tensor figure: fp32 componentwise error, or fp16 / bf16
        relative L2 error (checked against its bound)."""
        if self.dtype == "f32":
            return self.comp
        if self.ref2 == 0:
            assert self.diff2 == 0
            return 0.0
        err = (self.diff2 / self.ref2) ** 0.5
        assert err <= REL_L2_TOL[self.dtype], f"{self.dtype} relative L2 error {err:.3e} > {REL_L2_TOL[self.dtype]}"
        return err


def check_forward(y_gpu: torch.Tensor, ref, mag, dtype: str, rows=None):
    y = y_gpu.detach().float().cpu().double().numpy()
    if rows is not None:
        y = y[rows]
    chk = ForwardCheck(dtype)
    chk.add(y, ref, mag)
    return chk.finish()


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
