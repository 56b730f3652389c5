"""A plain model of the packed-batch plan the chunked kernels build on the
device, for the host tests of the workspace bound and the GPU test that reads
the device plan back.

A packed batch of B sequences (lengths n_b) with H heads runs as blocks of
one (sequence, head, segment) each.  Sequence b has c_b = ceil(n_b / 64)
chunks; every segment holds C = ceil(H sum_b c_b / 256) chunks but a
sequence's last, so sequence b has S_b = max(1, ceil(c_b / C)) segments.
The blocks run the full segments first, in (b, h, seg) order, then the last
segments of the sequences ordered by their size, longest first (ties by b;
batches of up to 256 sequences, else in b order), heads innermost.
Sequences with more than FOLD_MAX segments have their carries chained by a
separate kernel (the carry list)."""
from __future__ import annotations

L = 64
FOLD_MAX = 4
PLAN_HEAD = 4
SORT_MAX = 256
END_STATES = 256


def blocks_max(B: int, H: int) -> int:
    return 256 + B * H


def carry_cap(H: int) -> int:
    return 256 // (FOLD_MAX * H) + 1


def plan_ints(B: int, H: int) -> int:
    return PLAN_HEAD + 6 * B + 1 + carry_cap(H)


def plan(lens, H: int) -> dict:
    """The plan of a valid table (lengths >= 0)."""
    B = len(lens)
    c = [-(-n // L) for n in lens]
    C = max(1, -(-H * sum(c) // 256))
    S = [max(1, -(-x // C)) for x in c]
    last = [c[b] - (S[b] - 1) * C for b in range(B)]
    order = sorted(range(B), key=lambda b: (-last[b], b)) if B <= SORT_MAX else list(range(B))
    starts = [0]
    for n in lens:
        starts.append(starts[-1] + n)
    coff, soff = [0], [0]
    for b in range(B):
        coff.append(coff[-1] + c[b])
        soff.append(soff[-1] + S[b] - 1)
    carry = [b for b in range(B) if S[b] > FOLD_MAX]
    full = H * soff[-1]
    # block -> (b, h, seg, chunks)
    work = []
    for b in range(B):
        for h in range(H):
            for seg in range(S[b] - 1):
                work.append((b, h, seg, C))
    for b in order:
        for h in range(H):
            work.append((b, h, S[b] - 1, last[b]))
    return {"C": C, "blocks": full + H * B, "full": full, "S": S, "chunks": c, "start": starts[:-1],
            "len": list(lens), "coff": coff[:-1], "soff": soff, "order": order, "carry": carry,
            "end_states": full, "chunk_slots": H * coff[-1], "work": work}


def plan_array(lens, H: int) -> list:
    """The int32 array the device writes: [C, blocks, carry count, F, start[B],
    len[B], S[B], chunk offset[B], end-state offset[B + 1], order[B], carry
    list (its first carry-count entries)]."""
    p = plan(lens, H)
    cap = carry_cap(H)
    head = [p["C"], p["blocks"], min(len(p["carry"]), cap), p["full"]]
    return head + p["start"] + p["len"] + p["S"] + p["coff"] + p["soff"] + p["order"] + p["carry"][:cap]


# ---------------------------------------------------------------- dense batches
CUS = 256
BLOCK_COST = 1.5  # fixed work of a workgroup, in chunk times


def dense_makespan(P: int, c: int, C: int) -> float:
    """Chunk times to run P sequences of c chunks in segments of C chunks on
    256 units, one workgroup each at a time, full segments first and the
    shorter last segments after them, each next workgroup on the unit that
    frees first (a plain simulation)."""
    import heapq
    S = -(-c // C)
    r = c - (S - 1) * C
    loads = [0.0] * CUS
    for size in [C] * (P * (S - 1)) + [r] * P:
        t = heapq.heappop(loads)
        heapq.heappush(loads, t + size + BLOCK_COST)
    return max(loads)


def dense_plan(B: int, H: int, N: int) -> tuple:
    """(S, C): the segment count and size in chunks of a dense batch: the C
    with the least makespan among sizes from half to twice the even split
    (at most 512 of them, evenly spaced), ties to fewer segments."""
    P, c = B * H, -(-N // L)
    if c <= 1:
        return 1, 1
    even = -(-P * c // CUS)
    lo, hi = max(1, even // 2), min(2 * even, c)
    lo = min(lo, hi)
    step = (hi - lo) // 512 + 1
    best, best_t = c, dense_makespan(P, c, c)
    C = hi
    while C >= lo:
        t = dense_makespan(P, c, C)
        if t < best_t - 1e-9:
            best, best_t = C, t
        C -= step
    return -(-c // best), best
