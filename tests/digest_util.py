"""Per-row neighbour fingerprints of GPU pair lists, computed on the device
with torch integer arithmetic, in the form the oracle's digest files use
(tests/golden/make_digests.py): count c_i, fingerprint h_i = sum of
mix64(j) over the row's neighbours mod 2^64 (mix64: the splitmix64 output
function), and the block fold sum of mix64(h_i + mix64(c_i + i * 2^32)) over
blocks of consecutive rows.  int64 tensors hold the uint64 bit patterns;
their additions and multiplications wrap modulo 2^64."""
import torch

_M64 = 1 << 64


def _s64(v):
    return v - _M64 if v >= 1 << 63 else v


GOLDEN = _s64(0x9e3779b97f4a7c15)
MUL1 = _s64(0xbf58476d1ce4e5b9)
MUL2 = _s64(0x94d049bb133111eb)


def _lsr(z, k):
    return (z >> k) & ((1 << (64 - k)) - 1)


def mix64(v):
    """splitmix64 output function of an int64 tensor (uint64 bit patterns)."""
    z = v + GOLDEN
    z = (z ^ _lsr(z, 30)) * MUL1
    z = (z ^ _lsr(z, 27)) * MUL2
    return z ^ _lsr(z, 31)


def u32(t):
    return t.to(torch.int64) & 0xffffffff


def row_digests(parts, n_rows, rows=None, chunk=1 << 27):
    """(count, fingerprint) int64 tensors per query row (rows: an int64 tensor
    of selected rows; their order gives the output order), from per-batch
    [m, 2] int32 pair tensors (query id, point id)."""
    dev = parts[0].device if parts else torch.device("cuda")
    pos = None
    m = n_rows
    if rows is not None:
        pos = torch.full((n_rows,), -1, dtype=torch.int64, device=dev)
        pos[rows.to(dev)] = torch.arange(rows.numel(), dtype=torch.int64, device=dev)
        m = rows.numel()
    cnt = torch.zeros(m, dtype=torch.int64, device=dev)
    dig = torch.zeros(m, dtype=torch.int64, device=dev)
    for p in parts:
        for s in range(0, p.shape[0], chunk):
            blk = p[s:s + chunk]
            q, x = u32(blk[:, 0]), u32(blk[:, 1])
            if pos is not None:
                r = pos[q]
                sel = r >= 0
                q, x = r[sel], x[sel]
            cnt.index_add_(0, q, torch.ones_like(q))
            dig.index_add_(0, q, mix64(x))
    return cnt, dig


def block_fold(cnt, dig, block):
    """Per block of `block` rows: the count sum and the fold of the row fingerprints."""
    n = cnt.numel()
    i = torch.arange(n, dtype=torch.int64, device=cnt.device)
    t = mix64(dig + mix64(cnt + (i << 32)))
    nblk = (n + block - 1) // block
    pad = nblk * block - n
    z = torch.zeros(pad, dtype=torch.int64, device=cnt.device)
    fp = torch.cat([t, z]).view(nblk, block).sum(dim=1)
    bc = torch.cat([cnt, z]).view(nblk, block).sum(dim=1)
    return bc, fp
