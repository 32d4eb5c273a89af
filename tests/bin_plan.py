"""The backward's binning plan as the library chooses it (test infrastructure).

The value-gradient path bins points into pixel tiles with one of two bin
kernels: a register-cached one (a block keeps at most 8 points per thread in
registers for both of its passes) or a plain one (each pass loads the points
again). ``plan`` restates the library's choice so that a parity test can show
which kernel it exercised; ``workspace_bytes`` restates the resulting
workspace size, which a CPU test compares with msda_backward_workspace_size
to keep this restatement honest.
"""
BLOCK = 256          # threads per bin block
UNROLL = 8           # points per thread a cached block keeps
MAX_SLABS = 256      # bin blocks per (b, m) at most
BIN_SLABS = 64       # the same unless the points then fit in registers
MIN_QUERIES = 64     # queries per bin block at least
COUNTERS = 8 * 64 * 4
ALIGN = 256


def _up(x, a):
    return (x + a - 1) // a * a


def plan(B, M, Nq, L, K, Nv):
    """(bin blocks per (b, m), queries per block, cached, tall tiles)."""
    BM = B * M
    nW = (4096 + BM - 1) // BM
    nW = max(1, min(nW, BIN_SLABS))
    nW_q = (Nq + MIN_QUERIES - 1) // MIN_QUERIES
    if nW > nW_q:
        nW = max(nW_q, 1)
    LK = L * K
    cached = False
    q_fit = (UNROLL * BLOCK) // LK if LK > 0 else 0
    if q_fit >= 1 and Nq > 0:
        nW_fit = (Nq + q_fit - 1) // q_fit
        if nW_fit <= MAX_SLABS and nW_fit <= 3 * nW:
            nW = max(nW, nW_fit)
            cached = True
    Qc = (Nq + nW - 1) // nW if Nq > 0 else 0
    nW = (Nq + Qc - 1) // Qc if Qc > 0 else 1
    tall = Nq * L * K < Nv
    return nW, Qc, cached, tall


def workspace_bytes(B, M, Nq, L, K, Nv, planes=None):
    """Workspace of `planes` (b, m) planes per pass (all of them: one pass)."""
    BM = B * M
    if BM == 0:
        return 0
    planes = BM if planes is None else planes
    nW, Qc, _, _ = plan(B, M, Nq, L, K, Nv)
    t_stride = (Nv + 3) // 4 + L + 1          # tile boundaries per (b, m)
    slab_per_block = _up(4 * Qc * L * K, 64)
    table = planes * nW * t_stride * 4        # one slab offset per boundary and bin block
    slab = planes * nW * slab_per_block * 16
    return _up(COUNTERS, ALIGN) + _up(table, ALIGN) + _up(slab, ALIGN)
