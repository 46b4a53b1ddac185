"""Helpers of the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, read results back."""

from __future__ import annotations

import numpy as np

SENTINEL = 0x7FBADBAD


def torch_mod():
    import torch
    return torch


def to_device(arr: np.ndarray, dtype: str):
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda:0")


def sentinel_partitions(R: int, P: int):
    torch = torch_mod()
    bits = np.full(P, SENTINEL, dtype=np.uint32).view(np.int32)
    return [torch.from_numpy(bits.copy()).to("cuda:0").view(torch.float32) for _ in range(R)]


def workspace(nbytes: int):
    torch = torch_mod()
    ws = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device="cuda:0")
    off = (-ws.data_ptr()) % 256
    return ws, ws.data_ptr() + off


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def run_steps(group, micro_grads, micro_dtype: str, momenta0=None, use_accumulate=True):
    """micro_grads[step][micro][matrix] host arrays (storage form).  Returns
    (partitions as float32 arrays, momenta as float32 arrays)."""
    torch = torch_mod()
    shapes = group.shapes
    ws_t, ws = workspace(group.workspace_bytes)
    if momenta0 is None:
        moms = [torch.zeros(r, c, dtype=torch.float32, device="cuda:0") for r, c in shapes]
    else:
        moms = [to_device(m, "fp32").reshape(r, c) for m, (r, c) in zip(momenta0, shapes)]
    parts = sentinel_partitions(group.num_partitions, group.partition_numel)
    accs = [torch.empty(r, c, dtype=torch.float32, device="cuda:0") for r, c in shapes]
    for step in micro_grads:
        if use_accumulate:
            for k, mb in enumerate(step):
                dev = [to_device(g, micro_dtype) for g in mb]
                group.accumulate(accs, dev, micro_dtype, k == 0, ws)
                torch.cuda.synchronize()
            group.step(accs, moms, parts, ws)
        else:
            assert len(step) == 1
            dev = [to_device(g, micro_dtype) for g in step[0]]
            group.step(dev, moms, parts, ws)
        torch.cuda.synchronize()
    del ws_t
    return [host(p) for p in parts], [host(m) for m in moms]


def tile_errors(got, want, tile: int = 256):
    """Error of every tile x tile block of a matrix (the last row and column
    of blocks are the ragged edge strips), as (err, allowed) arrays of shape
    (ceil(rows/tile), ceil(cols/tile)).

    err is the block's error norm over the norm a block of its size has at
    the matrix's RMS magnitude, ||d_block|| / (rms(want) sqrt(N_block)): for a
    block of typical magnitude it is the block's relative Frobenius error.
    allowed(tol) = tol (1 + 3 / sqrt(N_block)): a block's error ratio
    fluctuates around the matrix-level one by about 1/sqrt(N_block) of it, so
    a whole 256 x 256 block gets tol within 1.2% while a one-element corner
    block gets 4 tol; a wrong tile or strip (errors the size of the values
    themselves) exceeds either by orders of magnitude."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    r, c = want.shape
    tr, tc = -(-r // tile), -(-c // tile)
    pr, pc = tr * tile - r, tc * tile - c

    def blocks(x):
        x = np.pad(x, ((0, pr), (0, pc)))
        return (x * x).reshape(tr, tile, tc, tile).sum(axis=(1, 3))

    num = blocks(got - want)
    cnt = blocks(np.ones_like(want))
    rms2 = float(np.sum(want * want)) / want.size
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.sqrt(num / (rms2 * cnt))
    if rms2 == 0.0:
        err = np.where(num == 0, 0.0, np.inf)
    slack = 1.0 + 3.0 / np.sqrt(cnt)
    return err, slack


def assert_tiles_within(got, want, tol: float, label: str, tile: int = 256) -> float:
    """Every block of the matrix within tol (1 + 3/sqrt(N_block)) by the
    measure of tile_errors; returns the worst block's error ratio."""
    err, slack = tile_errors(got, want, tile)
    over = err > tol * slack
    if over.any():
        i, j = np.unravel_index(int(np.argmax(err / slack)), err.shape)
        raise AssertionError(f"{label}: block ({i}, {j}) of {tile}x{tile} (rows {i * tile}.., cols {j * tile}..) "
                             f"error {err[i, j]:.3e} > {tol * slack[i, j]:.3e}; {int(over.sum())} of {err.size} "
                             f"blocks over")
    return float(err.max())
