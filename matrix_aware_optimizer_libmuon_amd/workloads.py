"""Seeded synthetic workloads for the Muon step.

This module only draws inputs: matrix shapes, gradients, parameters and
momentum buffers with the distributions of the five standard workloads.  It
contains none of the optimizer's arithmetic, does not import the HIP binding
and does not import the oracle, so the tests can feed the very same values to
both sides.

Seeding: every array is drawn from numpy's PCG64 seeded with
``SeedSequence([workload, step, matrix_index, role])``, so any single matrix
can be regenerated on its own (the streaming oracle relies on that).

bf16 gradients are drawn in float64, rounded to float32 by numpy and then to
bf16 by round-to-nearest-even on the bit pattern.  They are carried as uint16
bit patterns (``grad_bits``) plus their exact float32 widening (``grad``).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Iterator

import numpy as np

# roles in the seed sequence
ROLE_GRAD, ROLE_PARAM, ROLE_PREV_GRAD, ROLE_SPIKE_U, ROLE_SPIKE_V, ROLE_SHAPES, ROLE_MOM, ROLE_COL = range(8)


# --------------------------------------------------------------------------
# bf16 helpers (input quantisation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the 16-bit patterns.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the standard workloads.  ``shapes`` lists (rows, cols) of every
    matrix; ``grad_dtype`` is "f32" or "bf16"."""
    key: int
    name: str
    shapes: tuple
    grad_dtype: str
    steps: int
    lr: float = 0.02
    mu: float = 0.95
    wd: float = 0.01
    ns_steps: int = 5
    eps: float = 1e-7
    rms_mode: str | None = None

    @property
    def n_mats(self) -> int:
        return len(self.shapes)

    def ns_flops(self) -> int:
        """Nominal Newton-Schulz flops of one step over all matrices: per
        iteration 4 m^2 n + 2 m^3 (m the short side)."""
        tot = 0
        for r, c in self.shapes:
            m, n = min(r, c), max(r, c)
            tot += 4 * m * m * n + 2 * m ** 3
        return tot * self.ns_steps

    def elements(self) -> int:
        return sum(r * c for r, c in self.shapes)


def _cfg4_shapes(count: int = 2048) -> tuple:
    rng = _rng(4, 0, 0, ROLE_SHAPES)
    sizes = np.array([64, 128, 256, 512])
    r = sizes[rng.integers(0, 4, size=count)]
    c = sizes[rng.integers(0, 4, size=count)]
    return tuple((int(a), int(b)) for a, b in zip(r, c))


def _mamba_shapes(layers: int = 24, d: int = 768) -> tuple:
    # per layer: in_proj d x 4d, x_proj 2d x 80, dt_proj 48 x 2d, out_proj 2d x d
    one = ((d, 4 * d), (2 * d, 80), (48, 2 * d), (2 * d, d))
    return tuple(s for _ in range(layers) for s in one)


def _transformer_shapes(layers: int = 32, d: int = 4096, ff: int = 14336) -> tuple:
    one = ((d, d),) * 4 + ((d, ff), (d, ff), (ff, d))
    return tuple(s for _ in range(layers) for s in one)


WORKLOADS = {
    1: Workload(1, "single fp32 gradient 256x768", ((256, 768),), "f32", 1, wd=0.0),
    2: Workload(2, "mamba block d768 x24 layers (96 matrices), 3 steps", _mamba_shapes(), "bf16", 3),
    3: Workload(3, "transformer hidden set d4096 x32 layers (224 matrices)", _transformer_shapes(), "bf16", 1),
    4: Workload(4, "ragged 2048 matrices rows,cols in {64..512}", _cfg4_shapes(), "bf16", 1),
    5: Workload(5, "single 8192x28672 bf16 gradient, t(3) entries", ((8192, 28672),), "bf16", 1,
                rms_mode="sqrt_max1"),
}


def layer_subset(w: Workload, layers) -> list:
    """Indices of the matrices of the given transformer layers (7 per layer)."""
    if w.key != 3:
        raise ValueError("layer subsets are defined for the transformer workload")
    return [7 * l + j for l in layers for j in range(7)]


# --------------------------------------------------------------------------
# per-matrix draws
# --------------------------------------------------------------------------
def _normal(rng, shape, std) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _grad_f64(w: Workload, step: int, idx: int) -> np.ndarray:
    r, c = w.shapes[idx]
    rng = _rng(w.key, step, idx, ROLE_GRAD)
    if w.key == 1:
        return rng.standard_normal((r, c))                 # float64 draw
    if w.key == 2:
        return _normal(rng, (r, c), 0.02)
    if w.key == 3:
        g = _normal(rng, (r, c), 1e-3).astype(np.float64)
        k = 8
        u, _ = np.linalg.qr(_rng(w.key, step, idx, ROLE_SPIKE_U).standard_normal((r, k)))
        v, _ = np.linalg.qr(_rng(w.key, step, idx, ROLE_SPIKE_V).standard_normal((c, k)))
        sigma = 1e-3 * np.sqrt(r * c)
        g += sigma * (u @ v.T)
        return g
    if w.key == 4:
        return rng.standard_normal((r, c), dtype=np.float32)
    if w.key == 5:
        return (1e-3 * rng.standard_t(3, size=(r, c))).astype(np.float32)
    raise KeyError(w.key)


def grad(w: Workload, step: int, idx: int):
    """Gradient of matrix ``idx`` at ``step`` (steps count from 0).

    Returns (values_f32, bits_u16_or_None): float32 exact values, and for bf16
    workloads the bf16 bit patterns those values come from."""
    g = _grad_f64(w, step, idx).astype(np.float32)
    if w.grad_dtype == "f32":
        return np.ascontiguousarray(g), None
    bits = f32_to_bf16_bits(g)
    return bf16_bits_to_f32(bits), bits


def param(w: Workload, idx: int) -> np.ndarray:
    """Initial fp32 parameter, N(0, 0.02)."""
    r, c = w.shapes[idx]
    return _normal(_rng(w.key, 0, idx, ROLE_PARAM), (r, c), 0.02)


def momentum(w: Workload, idx: int) -> np.ndarray:
    """Initial fp32 momentum buffer.  Zero, except for the single large
    gradient workload, which starts warm: the buffer holds 0.05 times a prior
    gradient drawn from the same 1e-3 * t(3) law under another seed (the state
    a first step from zero with momentum 0.95 would leave)."""
    r, c = w.shapes[idx]
    if w.key != 5:
        return np.zeros((r, c), dtype=np.float32)
    prev = 1e-3 * _rng(w.key, 0, idx, ROLE_PREV_GRAD).standard_t(3, size=(r, c))
    prev = f32_to_bf16_bits(prev.astype(np.float32))       # prior grad was bf16 too
    return (0.05 * bf16_bits_to_f32(prev).astype(np.float64)).astype(np.float32)


@dataclasses.dataclass
class MatrixInputs:
    rows: int
    cols: int
    grad: np.ndarray            # float32 exact values (bf16-exact for bf16 workloads)
    grad_bits: np.ndarray | None  # uint16 bf16 bit patterns, or None for fp32 grads
    param: np.ndarray           # float32
    mom: np.ndarray             # float32


def matrix_inputs(w: Workload, idx: int, step: int = 0, with_state: bool = True) -> MatrixInputs:
    g, bits = grad(w, step, idx)
    r, c = w.shapes[idx]
    p = param(w, idx) if with_state else None
    m = momentum(w, idx) if with_state else None
    return MatrixInputs(r, c, g, bits, p, m)


def iter_inputs(w: Workload, indices=None, step: int = 0, threads: int = 8,
                with_state: bool = True) -> Iterator[tuple[int, MatrixInputs]]:
    """Yield (index, inputs) in order, drawing a few matrices ahead on a thread
    pool (numpy releases the GIL while drawing)."""
    if indices is None:
        indices = range(w.n_mats)
    indices = list(indices)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        futs = {}
        ahead = max(1, threads)
        for j, idx in enumerate(indices[:ahead]):
            futs[j] = ex.submit(matrix_inputs, w, idx, step, with_state)
        for j, idx in enumerate(indices):
            nxt = j + ahead
            if nxt < len(indices):
                futs[nxt] = ex.submit(matrix_inputs, w, indices[nxt], step, with_state)
            yield idx, futs.pop(j).result()


def adhoc_inputs(rows: int, cols: int, grad_dtype: str, seed: int, grad_std: float = 1.0,
                 mom_std: float = 0.0, param_std: float = 0.02,
                 col_offset: float = 0.0) -> MatrixInputs:
    """Seeded inputs of any shape (edge-case tests): N(0, grad_std) gradient
    plus, when col_offset > 0, an N(0, col_offset) offset per column (rounded
    to bf16 when asked), N(0, mom_std) momentum, N(0, param_std) parameter.
    Seeds live in their own range (workload key 1000)."""
    g = _normal(_rng(1000, seed, rows, cols, ROLE_GRAD), (rows, cols), grad_std)
    if col_offset > 0:
        g = (g + _normal(_rng(1000, seed, rows, cols, ROLE_COL), (1, cols), col_offset)).astype(np.float32)
    bits = None
    if grad_dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        g = bf16_bits_to_f32(bits)
    m = (_normal(_rng(1000, seed, rows, cols, ROLE_MOM), (rows, cols), mom_std)
         if mom_std > 0 else np.zeros((rows, cols), dtype=np.float32))
    p = _normal(_rng(1000, seed, rows, cols, ROLE_PARAM), (rows, cols), param_std)
    return MatrixInputs(rows, cols, np.ascontiguousarray(g), bits, p, m)


@dataclasses.dataclass
class AdamWInputs:
    numel: int
    grads: list           # float32 arrays (exact values; bf16-representable when bits given)
    grad_bits: list       # uint16 arrays or None, one per step
    param: np.ndarray     # float32
    exp_avg: np.ndarray   # float32
    exp_avg_sq: np.ndarray


def adamw_inputs(numel: int, steps: int, grad_dtype: str, seed: int, grad_std: float = 1.0,
                 param_std: float = 0.02, warm: bool = False) -> AdamWInputs:
    """Seeded inputs of one AdamW tensor (flattened): ``steps`` gradients
    N(0, grad_std) (rounded to bf16 when asked), an N(0, param_std) parameter,
    and zero moments -- or, with ``warm``, moments of a prior gradient history
    (first moment N(0, 0.1 grad_std), second |N(0, grad_std^2)|).  Seeds live
    in their own range (workload key 2000)."""
    grads, bits = [], []
    for t in range(steps):
        g = _normal(_rng(2000, seed, numel, t, ROLE_GRAD), (numel,), grad_std)
        b = None
        if grad_dtype == "bf16":
            b = f32_to_bf16_bits(g)
            g = bf16_bits_to_f32(b)
        grads.append(np.ascontiguousarray(g))
        bits.append(b)
    p = _normal(_rng(2000, seed, numel, 0, ROLE_PARAM), (numel,), param_std)
    if warm:
        m = _normal(_rng(2000, seed, numel, 0, ROLE_MOM), (numel,), 0.1 * grad_std)
        v = np.abs(_normal(_rng(2000, seed, numel, 1, ROLE_MOM), (numel,), grad_std * grad_std))
    else:
        m = np.zeros(numel, dtype=np.float32)
        v = np.zeros(numel, dtype=np.float32)
    return AdamWInputs(numel, grads, bits, p, m, v.astype(np.float32))


# --------------------------------------------------------------------------
# device-side draws (benchmark inputs): the same laws as above, drawn by
# torch's seeded device generator so that the 7.8 G-element workloads do not
# spend minutes on the host.  Values differ from the host recipe (another
# random stream); shapes, dtypes, laws and structure are the same.
# --------------------------------------------------------------------------
def device_inputs(w: Workload, idx: int, device, gen, step: int = 0):
    """(param fp32, grad fp32/bf16, mom fp32) torch tensors for matrix idx."""
    import torch
    r, c = w.shapes[idx]

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    if w.key == 1:
        g = randn(r, c)
    elif w.key == 2:
        g = randn(r, c).mul_(0.02)
    elif w.key == 3:
        g = randn(r, c).mul_(1e-3)
        # rank-8 spike: orthonormal factors from a seeded host QR (tiny)
        u, _ = np.linalg.qr(_rng(w.key, step, idx, ROLE_SPIKE_U).standard_normal((r, 8)))
        v, _ = np.linalg.qr(_rng(w.key, step, idx, ROLE_SPIKE_V).standard_normal((c, 8)))
        ut = torch.from_numpy(u.astype(np.float32)).to(device)
        vt = torch.from_numpy(v.astype(np.float32)).to(device)
        g.addmm_(ut, vt.t().contiguous(), alpha=float(1e-3 * np.sqrt(r * c)))
    elif w.key == 4:
        g = randn(r, c)
    elif w.key == 5:
        g = _student_t3(randn, r, c).mul_(1e-3)
    else:
        raise KeyError(w.key)
    if w.grad_dtype == "bf16":
        g = g.to(torch.bfloat16)
    p = randn(r, c).mul_(0.02)
    if w.key == 5:
        m = _student_t3(randn, r, c).mul_(1e-3).to(torch.bfloat16).float().mul_(0.05)
    else:
        m = torch.zeros(r, c, device=device, dtype=torch.float32)
    return p, g, m


def _student_t3(randn, r, c):
    """t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3), chi2_3 a sum of
    three squared standard normals."""
    z = randn(r, c)
    chi = randn(r, c).square_()
    chi.add_(randn(r, c).square_()).add_(randn(r, c).square_())
    return z.div_(chi.div_(3.0).sqrt_())
