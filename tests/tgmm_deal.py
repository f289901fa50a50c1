"""Host model of the tgmm GEMM's work-item deal (host logic, not the method's
arithmetic): which GEMM block takes each (expert, output tile) item.

Expert g's item j goes to block (offset[g] + j) mod nb.  Each expert's items
fill per_g // nb whole rounds plus per_g % nb items on consecutive (cyclic)
blocks from offset[g].  Experts are taken by decreasing modelled cost (ties
by index) and each one's remainder window starts where the blocks' modelled
load over the window is smallest (ties: the smallest offset).  The cost
model, in integer ticks and then units of 256 ticks, is the one the library's
prep pass uses: per 32-row sub-step, per ring stage, per pair-end rescale,
per output tile.  The library writes the same offsets into its workspace; a
GPU test compares them with these.
"""
import numpy as np

COST_SUB, COST_STAGE, COST_PAIR, COST_ITEM = 730, 1300, 1100, 5930
TILE_M, SUB = 512, 32
MAX_GROUPS, MAX_BLOCKS = 256, 512


def geometry(G, K, N, cus):
    """(k-tile rows, ring-stage rows, items per expert, blocks) of the GEMM launch."""
    bmk = 256 if K % 256 == 0 else 128
    chunk = 128 if bmk == 256 else 64
    per_cu = 1 if bmk == 256 else 2
    per_g = (K // bmk) * (N // 128)
    return bmk, chunk, per_g, min(G * per_g, per_cu * cus)


def expert_costs(group_sizes, M, chunk):
    """Modelled cost of one item of each expert, in units of 256 ticks
    (sizes clamped to the buffer as the library's pair table does)."""
    costs, start = [], 0
    for raw in group_sizes:
        sz = min(max(int(raw), 0), M)
        st, en = min(start, M), min(start + sz, M)
        start += sz
        c = COST_ITEM
        if en > st:
            for t in range(st // TILE_M, (en - 1) // TILE_M + 1):
                rows = min(en, (t + 1) * TILE_M) - max(st, t * TILE_M)
                sub = -(-rows // SUB)
                c += COST_SUB * sub + COST_STAGE * (-(-(sub * SUB) // chunk)) + COST_PAIR
        costs.append((c + 255) >> 8)
    return costs


def deal(group_sizes, M, K, N, cus):
    """Block offsets [G] the library computes (None where it deals round-robin)."""
    G = len(group_sizes)
    _, chunk, per_g, nb = geometry(G, K, N, cus)
    if G > MAX_GROUPS or nb > MAX_BLOCKS:
        return None
    costs = expert_costs(group_sizes, M, chunk)
    extra = per_g % nb
    load = np.zeros(nb, np.int64)
    offsets = [0] * G
    for g in sorted(range(G), key=lambda h: (-costs[h], h)):
        if extra == 0:
            continue
        twice = np.concatenate([load, load])
        windows = np.convolve(twice, np.ones(extra, np.int64), "valid")[:nb]
        o = int(np.argmin(windows))
        load[(o + np.arange(extra)) % nb] += costs[g]
        offsets[g] = o
    return offsets


def round_robin(G, per_g, nb):
    """The plain deal over the item index g * per_g + j."""
    return [g * per_g % nb for g in range(G)]


def block_loads(group_sizes, M, K, N, cus, offsets):
    """Modelled load of every block under a deal (whole rounds included)."""
    G = len(group_sizes)
    _, chunk, per_g, nb = geometry(G, K, N, cus)
    costs = expert_costs(group_sizes, M, chunk)
    load = np.zeros(nb, np.int64)
    for g in range(G):
        blocks = (offsets[g] + np.arange(per_g)) % nb
        np.add.at(load, blocks, costs[g])
    return load
