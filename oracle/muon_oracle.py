"""Plain, slow, fp64 CPU oracle of one Muon optimizer step over a group of
2-D matrices.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it exists so that tests, the smoke check and the
benchmark's CPU-baseline leg can check the HIP library against an independent
definition of what the step computes.  It shares no code with the library
(no kernels, headers, tables or helpers) and imports nothing from it.

Sources, cited by page title and section (the pages give the method in prose;
the numeric definition of the step is the plain reading of that prose):

* "Support Muon in BF16_Optimizer with FP32 gradient accumulation"
  (DeepSpeed PR 8526), description: Muon runs on the original (full-shape)
  matrices of the accumulated FP32 gradient, momentum is FP32, and only each
  rank's owned intersection of the update is copied into that rank's FP32
  flat partition, alignment padding excluded.
* "Run Muon once per optimizer step under ZeRO-3, not once per micro-batch"
  (DeepSpeed PR 8600), "The problem" and "The change": Muon runs once per
  optimizer step on the accumulated gradient, so momentum advances once per
  step and Newton-Schulz runs once per matrix per step; each rank's slice of
  the update is written back into its partition.  Review thread: the update
  routine takes the momentum, beta, the Newton-Schulz method ('standard' or
  'gram', default 'gram') and a per-parameter head count.
* "Fix Muon optimizer under ZeRO CPU offload and bound gather buffers"
  (DeepSpeed PR 8464), commit message on momentum dtype: momentum lives in the
  fp32 master dtype.
* Commit "ZeRO-1/2 reduce-scatter fix for Muon matrices split across
  partitions": Newton-Schulz runs on the full reduced gradient of a matrix
  that spans several partitions; each owner keeps its local slice.

Readings taken where the pages are silent:
momentum is the lerp m <- beta*m + (1-beta)*G started from zero; the update
fed to Newton-Schulz is the Nesterov blend (1-beta)*G + beta*m_new; each
Newton-Schulz block is divided by (Frobenius norm + eps) in the wide
orientation (transposed iff rows > cols); the quintic iteration
X <- a X + (b A + c A^2) X with A = X X^T and the same (a, b, c) at every
step; the Gram form iterates on R = X X^T and applies the accumulated
polynomial to the normalised input once at the end; per-head splitting cuts
the matrix into equal contiguous row blocks; the result is multiplied by the
shape scale sqrt(max(1, rows/cols)) of the source matrix (rounded to fp32);
matrices are laid out back to back in a flat index space that is cut into
equal partitions.

Parity pins: every function here is pinned by a test under tests/ that checks
it against something other than itself, and a planted mistake in a copy of it
is caught (tests/test_oracle_mutations.py):
  bf16 decoding        known bit patterns (1, -5, the smallest subnormal and
                       normal, the largest finite, -0, +-inf)
  rel_frobenius        hand values, including 0/0, x/0 and which argument is
                       the reference
  Newton-Schulz forms  SVD closed form U f^T(S) V^T, rank-one and
                       orthonormal-row inputs, Gram = standard, invariances
  momentum, blend      scalar closed forms under a constant gradient
  muon_step            one step from a warm momentum rebuilt by hand (fp32
                       momentum, Nesterov blend, normalisation, SVD closed
                       form, shape scale), so the blend, not the momentum, is
                       what reaches Newton-Schulz
  layout, writeback    per-element brute force of the flat index map, padding
                       sentinels, the Newton-Schulz call count PR 8600 prints
  norm, clip, apply    hand values and closed forms
No function is parity-unpinned.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Quintic Newton-Schulz coefficients and step count of the workloads.
NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NORM_EPS = 1e-7
BETA = 0.95


# ---------------------------------------------------------------- dtype glue


def fp32(x) -> float:
    """Round a Python float to the nearest fp32 value (returned as float)."""
    return float(np.float32(x))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to fp64 values exactly."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Input array in its storage form ('fp32' float32 or 'bf16' uint16 bits)
    to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(np.asarray(x))
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------ accumulation (a0 row)


def accumulate(micro_grads) -> np.ndarray:
    """FP32 gradient accumulation over micro-batches, as PR 8526 (description)
    and PR 8600 ("The change": the partitions accumulate the raw gradient)
    describe: the step sees the plain sum, added in micro-batch order.
    Reading: sum, not mean (a caller that wants a mean pre-scales)."""
    total = None
    for g in micro_grads:
        g = np.asarray(g, dtype=np.float64)
        total = g.copy() if total is None else total + g
    if total is None:
        raise ValueError("no micro-batches")
    return total


# ------------------------------------------------ momentum and Nesterov blend


def momentum_update(m: np.ndarray, g: np.ndarray, beta: float, nesterov: bool):
    """FP32 momentum (PR 8526 description; PR 8464 momentum-dtype commit) and
    the Nesterov blend.

    m_new = beta*m + (1-beta)*g, stored as fp32.  The update handed to the
    orthogonalisation is u = (1-beta)*g + beta*m_new (Nesterov), or m_new
    itself without Nesterov.  Arithmetic in fp64 on the fp32 state; u uses the
    stored (fp32-rounded) m_new, since that value is the method's state.
    Returns (m_new as float32 array, u as fp64 array)."""
    beta = float(beta)
    m = np.asarray(m, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m_new = (beta * m + (1.0 - beta) * g).astype(np.float32)
    if nesterov:
        u = (1.0 - beta) * g + beta * m_new.astype(np.float64)
    else:
        u = m_new.astype(np.float64)
    return m_new, u


# ------------------------------------------------------- Newton-Schulz forms


def normalise(x: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """Divide by the Frobenius norm plus eps."""
    return x / (np.linalg.norm(x) + eps)


def ns_standard(x: np.ndarray, steps: int = NS_STEPS, coeffs=NS_COEFFS) -> np.ndarray:
    """'standard' Newton-Schulz (PR 8526 validation table; ZeRO-1/2 commit;
    PR 8600 review thread names the method): repeated quintic step on a wide
    matrix X (rows <= cols):  A = X X^T,  B = b A + c A A,  X <- a X + B X."""
    a, b, c = coeffs
    x = np.array(x, dtype=np.float64)
    for _ in range(steps):
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x


def ns_gram(x0: np.ndarray, steps: int = NS_STEPS, coeffs=NS_COEFFS) -> np.ndarray:
    """'gram' Newton-Schulz (named in the same places; the default method in
    PR 8600's review thread).  Reading: the same quintic, carried on the small
    side's Gram matrix.  With R = X0 X0^T and Q = I, each step forms
    P = a I + b R + c R R, accumulates Q <- P Q, and (except after the last
    step) advances R <- P R P; the output is Q X0.  In exact arithmetic this
    equals the standard form, since every X_k is Q_k X0 with Q_k a polynomial
    in X0 X0^T."""
    a, b, c = coeffs
    x0 = np.array(x0, dtype=np.float64)
    m = x0.shape[0]
    eye = np.eye(m)
    R = x0 @ x0.T
    Q = eye.copy()
    for k in range(1, steps + 1):
        P = a * eye + b * R + c * (R @ R)
        Q = P @ Q
        if k < steps:
            R = P @ R @ P
    return Q @ x0


def orthogonalise_block(block: np.ndarray, method: str, steps: int = NS_STEPS,
                        coeffs=NS_COEFFS, eps: float = NORM_EPS) -> np.ndarray:
    """One Newton-Schulz block: transpose to the wide orientation iff it has
    more rows than columns, normalise, iterate, transpose back."""
    tall = block.shape[0] > block.shape[1]
    x = np.ascontiguousarray(block.T if tall else block, dtype=np.float64)
    x = normalise(x, eps)
    if method == "standard":
        y = ns_standard(x, steps, coeffs)
    elif method == "gram":
        y = ns_gram(x, steps, coeffs)
    else:
        raise ValueError(f"unknown Newton-Schulz method {method!r}")
    return y.T if tall else y


def split_heads(u: np.ndarray, num_heads) -> list:
    """Per-head split (PR 8600 review thread: the head count belongs to the
    parameter; per-head changes q and k and leaves untagged matrices alone).
    Reading: num_heads equal contiguous row blocks; None, 0 or 1 = unsplit."""
    h = int(num_heads or 1)
    rows = u.shape[0]
    if h < 1 or rows % h:
        raise ValueError(f"{h} heads do not divide {rows} rows")
    hr = rows // h
    return [u[i * hr:(i + 1) * hr] for i in range(h)]


def shape_scale(rows: int, cols: int) -> float:
    """Shape scale sqrt(max(1, rows/cols)) of the source matrix, computed in
    fp64 and rounded to fp32 (the value the writeback multiplies by)."""
    return fp32(math.sqrt(max(1.0, rows / cols)))


def muon_matrix_update(u: np.ndarray, method: str, num_heads=None,
                       steps: int = NS_STEPS, coeffs=NS_COEFFS,
                       eps: float = NORM_EPS):
    """Orthogonalised update of one matrix, before the shape scale: per-head
    blocks, each orthogonalised on its own, restacked in row order."""
    blocks = split_heads(np.asarray(u, dtype=np.float64), num_heads)
    outs = [orthogonalise_block(b, method, steps, coeffs, eps) for b in blocks]
    return np.concatenate(outs, axis=0)


# ---------------------------------------------------------- flat writeback


def partition_runs(flat_offset: int, numel: int, partition_numel: int):
    """Owned intersections of one matrix with each partition.

    Element j of the flattened (row-major) matrix sits at flat index
    f = flat_offset + j, i.e. partition f // P at local offset f % P.  The
    contiguous runs of that map are returned as (partition, local_offset,
    first_element, length)."""
    runs = []
    j = 0
    while j < numel:
        f = flat_offset + j
        r, off = divmod(f, partition_numel)
        n = min(numel - j, partition_numel - off)
        runs.append((r, off, j, n))
        j += n
    return runs


def scatter_f32(update_f32: np.ndarray, flat_offset: int, partitions) -> None:
    """Copy one matrix's flattened fp32 update into the flat partitions at its
    owned intersections (PR 8526 description: owned intersections only,
    padding never written).  `partitions` is a list of float32 arrays of equal
    length, modified in place."""
    flat = np.ascontiguousarray(update_f32, dtype=np.float32).reshape(-1)
    P = partitions[0].shape[0]
    for r, off, j, n in partition_runs(flat_offset, flat.size, P):
        if r >= len(partitions):
            raise ValueError("matrix extends past the last partition")
        partitions[r][off:off + n] = flat[j:j + n]


def scaled_update_f32(ns_out, rows: int, cols: int) -> np.ndarray:
    """The bit-exact writeback value: the Newton-Schulz output converted to
    fp32, times the fp32 shape scale, one IEEE round-to-nearest multiply."""
    s = np.float32(shape_scale(rows, cols))
    return (np.asarray(ns_out, dtype=np.float32) * s).astype(np.float32)


def pack_layout(shapes, num_partitions: int, align: int = 16, interior_align: bool = False):
    """Flat layout of a group (reading of "alignment padding", PR 8526
    description and PR 8464 commit on padded final partitions): matrices
    packed back to back in order (or each start rounded up to `align` with
    interior_align), the total padded at the tail so that the partition size
    is a multiple of `align`.  Returns (offsets, partition_numel)."""
    offsets = []
    f = 0
    for r, c in shapes:
        if interior_align:
            f = -(-f // align) * align
        offsets.append(f)
        f += r * c
    per = -(-f // (num_partitions * align)) * align
    return offsets, per


# --------------------------------------------------------------- the step


@dataclass
class MuonOptions:
    beta: float = BETA
    nesterov: bool = True
    method: str = "standard"
    steps: int = NS_STEPS
    coeffs: tuple = NS_COEFFS
    eps: float = NORM_EPS


@dataclass
class MuonState:
    """Caller-side state the oracle carries between steps: fp32 momentum per
    matrix and the Newton-Schulz invocation counter."""
    momenta: list
    ns_invocations: int = 0
    steps: int = 0


def init_state(shapes) -> MuonState:
    return MuonState(momenta=[np.zeros(s, dtype=np.float32) for s in shapes])


@dataclass
class StepResult:
    updates: list = field(default_factory=list)      # fp64, scaled, original orientation
    ns_out: list = field(default_factory=list)       # fp64, unscaled
    partitions: list = field(default_factory=list)   # float32 arrays


def muon_step(grads, state: MuonState, shapes, heads, offsets, num_partitions,
              partition_numel, opt: MuonOptions, partitions=None, grad_scale: float = 1.0,
              skip: bool = False) -> StepResult:
    """One optimizer step of Muon over a group, on the accumulated gradient
    (PR 8600 "The change": once per step, after accumulation).

    grads: fp64 (or castable) arrays in original orientation.  The momentum in
    `state` is updated in place; the Newton-Schulz counter advances by one per
    matrix (PR 8600 table: calls = matrices x steps).  The fp32 partitions are
    written at each matrix's owned intersections with the fp32 value
    fp32(update); padding is left as given.

    grad_scale multiplies every gradient element before the momentum blend:
    gradients produced under a loss scale S come in with grad_scale = 1/S, so
    the momentum holds unscaled gradients and the step does not depend on S
    (the PR 8464 commits validate clipping equivalence across loss scales).
    skip = True is a step the overflow check discarded: it touches neither
    momentum nor partitions and counts nothing (PR 8600 "The change": the
    update runs after the overflow check, so a discarded step leaves the
    momentum alone)."""
    res = StepResult()
    if partitions is None:
        partitions = [np.zeros(partition_numel, dtype=np.float32)
                      for _ in range(num_partitions)]
    res.partitions = partitions
    if skip:
        return res
    for i, (rows, cols) in enumerate(shapes):
        g = np.asarray(grads[i], dtype=np.float64).reshape(rows, cols) * float(grad_scale)
        m_new, u = momentum_update(state.momenta[i], g, opt.beta, opt.nesterov)
        state.momenta[i] = m_new
        y = muon_matrix_update(u, opt.method, heads[i], opt.steps, opt.coeffs, opt.eps)
        state.ns_invocations += 1
        upd = y * shape_scale(rows, cols)
        res.ns_out.append(y)
        res.updates.append(upd)
        scatter_f32(upd.astype(np.float32), offsets[i], partitions)
    state.steps += 1
    return res


# ------------------------------------- after the path: norm, clip, apply


CLIP_EPS = 1e-6


def update_norm(partitions, shapes, offsets) -> float:
    """L2 norm of the Muon update as the partitions hold it (PR 8600 "The
    change": the gradient norm is taken over the Muon update): the square
    root of the sum of squares of every owned element of every matrix, each
    element counted once, padding excluded."""
    P = partitions[0].shape[0]
    total = 0.0
    for (rows, cols), off in zip(shapes, offsets):
        for r, o, _j, n in partition_runs(off, rows * cols, P):
            v = partitions[r][o:o + n].astype(np.float64)
            total += float(np.dot(v, v))
    return math.sqrt(total)


def clip_coefficient(norm: float, max_norm: float) -> float:
    """Global-norm clipping factor applied to every update element.  Reading
    (the pages keep the clipping semantics unchanged without spelling them
    out): the common convention min(1, max_norm / (norm + 1e-6)), and no
    clipping when max_norm <= 0."""
    if max_norm <= 0.0:
        return 1.0
    return min(1.0, float(max_norm) / (float(norm) + CLIP_EPS))


def apply_update(params, partitions, shapes, offsets, lr: float, weight_decay: float,
                 max_norm: float, skip: bool = False):
    """Parameter update from the Muon update in the partitions, on the fp32
    master partitions `params` (same flat layout).  Reading (the pages stop
    at the update): decoupled weight decay and a step of size lr along the
    clipped update,
        p <- p * (1 - lr * weight_decay) - lr * clip * u,
    on owned elements only; padding untouched.  Computed in fp64, stored as
    fp32.  skip = True (a discarded step) leaves params as given.
    Returns (new params as float32 arrays, norm, clip)."""
    out = [np.array(p, dtype=np.float32, copy=True) for p in params]
    if skip:
        return out, 0.0, 1.0
    norm = update_norm(partitions, shapes, offsets)
    clip = clip_coefficient(norm, max_norm)
    P = partitions[0].shape[0]
    decay = 1.0 - float(lr) * float(weight_decay)
    for (rows, cols), off in zip(shapes, offsets):
        for r, o, _j, n in partition_runs(off, rows * cols, P):
            p = out[r][o:o + n].astype(np.float64)
            u = partitions[r][o:o + n].astype(np.float64)
            out[r][o:o + n] = (p * decay - float(lr) * clip * u).astype(np.float32)
    return out, norm, clip


def gather_from_partitions(partitions, flat_offset: int, rows: int, cols: int) -> np.ndarray:
    """Read one matrix back out of the flat partitions (inverse of the
    writeback's index map), as float32 rows x cols."""
    P = partitions[0].shape[0]
    out = np.empty(rows * cols, dtype=np.float32)
    for r, off, j, n in partition_runs(flat_offset, rows * cols, P):
        out[j:j + n] = partitions[r][off:off + n]
    return out.reshape(rows, cols)


def rel_frobenius(got, want) -> float:
    """Relative Frobenius error ||got - want|| / ||want|| (0/0 -> 0)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)
