"""CPU model of the GEMM kernels' LDS-DMA issue / wait schedules (the
vector-memory counter is the only synchronisation between a wave's DMA and
its reads of LDS, so the wait immediates must be exact).

Model: a wave's vector-memory operations complete in issue order, and
``s_waitcnt vmcnt(n)`` returns once at most the n most recently issued ones are
outstanding.  Each test replays the kernel's issue order and checks, at every
wait, that the tile about to be read has landed and that no DMA still in
flight targets a stage that is being read.

gemm_kernel (csrc/gemm_kernel.h): two LDS rings of SA (A) and SB >= SA (B)
stages; a prologue issues virtual steps -SB..-1 (A tile s + SA when >= 0, B
tile s + SB); step kt waits with vmcnt(kNewer) for tile kt + 1 and then issues
A tile kt + SA and B tile kt + SB into the stages tile kt released (B before A
when SB == SA, after it when SB > SA); tiles past the end reload tile KT - 1.
The one-barrier schedule of gemm_kernel (dense 16-bit products on two-stage
rings): the prologue issues step 0 into stage 0 and waits for it; step kt
reads stage kt % 2, issues step kt + 1 (past the end: a reload of step KT - 1)
into the other stage and ends with vmcnt(0) and the barrier.
wgrad_kernel (csrc/wgrad_kernel.h): the A strip in two halves (each waited for
and read before the next), then B(0); per column tile t: wait for B(t), issue
B(t+1) into the other buffer, multiply, stage, 8 stores.

The tail split of the dense 256 x 256 products (gemm_kernel's tsplit,
tail_split_plan and tail_reduce_kernel in csrc/lmoe_host.h and
csrc/gemm_kernel.h) is modelled the same way: its workgroup -> (tile, K slice)
numbering must cover every tile exactly once (whole, or as all of its slices),
keep every slice non-empty, and stay inside the reserved partial blocks.
"""
import pytest


def gemm_schedule(SA, SB, KT, A_W, B_W, wait_delta=0):
    """Replays gemm_kernel's issue order; wait_delta shifts its vmcnt immediates
    (0: the kernel's own).  Raises AssertionError on a read of a tile that may
    not have landed or of a stage a DMA still in flight writes."""
    k_a_first = SB > SA
    NI = A_W + B_W
    k_newer = (B_W if k_a_first else 0) + (SA - 2) * NI + wait_delta
    k_newer0 = k_newer + NI
    issued = []  # (operand, nominal tile, stage) in issue order
    last = {}    # (operand, nominal tile) -> index of its last instruction

    def issue(op, t):  # nominal tile t (past the end: a reload of tile KT - 1 into t's stage)
        S = SA if op == "A" else SB
        for _ in range(A_W if op == "A" else B_W):
            issued.append((op, t, t % S))
        last[(op, t)] = len(issued) - 1

    def step_dma(ta, tb):
        if not k_a_first:
            issue("B", tb)
        if ta is not None:
            issue("A", ta)
        if k_a_first:
            issue("B", tb)

    def check_landed(t, n):
        for op in "AB":
            assert last[(op, t)] < len(issued) - n, (SA, SB, KT, t, op)

    for s in range(-SB, 0):
        step_dma(s + SA if s + SA >= 0 else None, s + SB)
    check_landed(0, k_newer0)  # tile 0 before the loop
    for kt in range(KT):
        if kt + 1 < KT:  # barrier of step kt: tile kt + 1 must have landed ...
            check_landed(kt + 1, k_newer)
            for op, t, st in issued[len(issued) - k_newer:] if k_newer > 0 else []:
                # ... and nothing still in flight writes its stages
                assert not (op == "A" and st == (kt + 1) % SA), (SA, SB, KT, kt)
                assert not (op == "B" and st == (kt + 1) % SB), (SA, SB, KT, kt)
        step_dma(kt + SA, kt + SB)  # phase 2: DMA into the stages tile kt released
    assert k_newer0 < 64  # the vmcnt field


RINGS = [(2, 2), (3, 3), (4, 4), (2, 3), (3, 5), (2, 4), (3, 6), (4, 6)]
WIDTHS = [(1, 1), (2, 4), (3, 4), (4, 4), (6, 8), (1, 8), (2, 2)]


@pytest.mark.parametrize("SA,SB", RINGS)
def test_gemm_vmcnt_schedule_is_exact(SA, SB):
    for KT in range(1, 70):
        for A_W, B_W in WIDTHS:
            gemm_schedule(SA, SB, KT, A_W, B_W)


@pytest.mark.parametrize("SA,SB", RINGS)
def test_a_wait_one_operation_too_shallow_is_caught(SA, SB):
    with pytest.raises(AssertionError):
        gemm_schedule(SA, SB, 16, 2, 4, wait_delta=1)


def onebar_schedule(KT, A_W, B_W, wait_delta=0):
    """Replays the one-barrier schedule's issue order (A then B each step, as
    dma_step issues them with SA == SB); wait_delta shifts its vmcnt(0)."""
    issued, last = [], {}  # issued: stage written, in issue order

    def issue_step(t, stage):
        for op, w in (("A", A_W), ("B", B_W)):
            issued.extend([stage] * w)
            last[(op, t)] = len(issued) - 1

    def landed(t, n):
        return all(last[(op, t)] < len(issued) - n for op in "AB")

    issue_step(0, 0)
    assert landed(0, wait_delta), (KT, "step 0")
    for kt in range(KT):
        reading = kt % 2
        issue_step(min(kt + 1, KT - 1) if kt + 1 < KT else KT, (kt + 1) % 2)
        # nothing issued since the last barrier writes the stage this step reads
        assert all(st != reading for st in issued[len(issued) - (A_W + B_W):]), (KT, kt)
        if kt + 1 < KT:  # the barrier that ends step kt: step kt + 1 has landed
            assert landed(kt + 1, wait_delta), (KT, kt)


def wgrad_schedule(KG, NT, wait_delta=0, stores=8, nwave=4):
    """Replays wgrad_kernel's issue order per wave: the A strip's two 128-column
    halves in turn (each into the space of both B buffers, waited for with
    vmcnt(0) and read into registers before the next is issued), B tile 0
    (into B buffer 0); per column tile t: wait for B(t), B tile t+1 into
    buffer (t+1) % 2, multiply from buffer t % 2, stage, the stores of tile t.
    Also checks that no DMA still in flight targets a buffer being read or
    staged into."""
    dma = KG * (4 // nwave)  # DMA instructions per B tile per wave (an A half: 2 dma)
    issued, last = [], {}    # issued: (tag, target buffer or None)

    def issue(tag, n, buf=None):
        issued.extend([(tag, buf)] * n)
        last[tag] = len(issued) - 1

    def in_flight(n):  # what may still be outstanding after vmcnt(n)
        return issued[len(issued) - n:] if n > 0 else []

    for h in range(2):
        issue(("A", h), 2 * dma, "AB")
        n = wait_delta
        assert last[("A", h)] < len(issued) - n, (KG, NT, h)  # the half is read
    issue(("B", 0), dma, 0)
    for t in range(NT):
        n = (0 if t == 0 else stores) + wait_delta
        assert last[("B", t)] < len(issued) - n, (KG, NT, t)
        flying = in_flight(n)
        if t + 1 < NT:
            issue(("B", t + 1), dma, (t + 1) % 2)
            flying = flying + issued[-dma:]
        # the MFMAs read buffer t % 2 and the staging writes "S"
        assert all(b not in (t % 2, "S", "AB") for _, b in flying), (KG, NT, t)
        issue(("S", t), stores)


def test_one_barrier_schedule_is_exact():
    for KT in range(1, 70):
        for A_W, B_W in WIDTHS:
            onebar_schedule(KT, A_W, B_W)
    with pytest.raises(AssertionError):
        onebar_schedule(8, 4, 4, wait_delta=1)


@pytest.mark.parametrize("KG", [2, 4, 6])
def test_wgrad_vmcnt_schedule_is_exact(KG):
    for NT in range(1, 30):
        wgrad_schedule(KG, NT)
    with pytest.raises(AssertionError):
        wgrad_schedule(KG, 4, wait_delta=1)


def tail_plan(m_tiles, n_tiles, steps, cus):
    """tail_split_plan: (S, whole tiles per XCD, kslice) or None."""
    per = m_tiles * n_tiles
    if per <= 0 or per % 8 or cus < 2:
        return None
    P = per // 8
    rem = P % cus
    if rem == 0:
        return None
    S = min(cus // rem, 4)
    if S < 2 or steps // S < 8:
        return None
    kslice = -(-steps // S)
    return -(-steps // kslice), P - rem, kslice


def tail_tile_coords(L, m_tiles, n_tiles):
    """dense_tile_coords: raster groups of 4 M tiles."""
    g = L // (4 * n_tiles)
    first = 4 * g
    gs = min(m_tiles - first, 4)
    i = L - g * 4 * n_tiles
    return first + i % gs, i // gs


def tail_workgroups(m_tiles, n_tiles, steps, S, whole, kslice):
    """Yields (tile, slice or None, tail id, first K step, K steps) per workgroup."""
    P = m_tiles * n_tiles // 8
    for b in range(8 * (whole + (P - whole) * S)):
        x, j = b % 8, b // 8
        if j < whole:
            yield x * P + j, None, None, 0, steps
        else:
            t, sl = divmod(j - whole, S)
            kt0 = sl * kslice
            yield x * P + whole + t, sl, x * (P - whole) + t, kt0, min(kslice, steps - kt0)


@pytest.mark.parametrize("cus", [32, 16])
def test_tail_split_covers_every_tile_once(cus):
    tested = 0
    for m_tiles in range(1, 41):
        for n_tiles in range(1, 41):
            for steps in (16, 23, 56, 344, 646):
                plan = tail_plan(m_tiles, n_tiles, steps, cus)
                if plan is None:
                    continue
                S, whole, kslice = plan
                P = m_tiles * n_tiles // 8
                rem = P - whole
                assert 2 <= S <= 4 and 8 * rem * S <= 8 * cus  # within the reserved blocks
                seen = {}
                for L, sl, tid, kt0, kt in tail_workgroups(m_tiles, n_tiles, steps, S, whole, kslice):
                    assert 0 <= L < m_tiles * n_tiles and kt >= 1
                    seen.setdefault(L, []).append((sl, kt0, kt))
                    if tid is not None:
                        assert 0 <= tid * S + sl < 8 * rem * S
                        # tail_reduce_kernel's inverse of the tail id
                        assert (tid // rem) * P + whole + tid % rem == L
                assert len(seen) == m_tiles * n_tiles
                for L, parts in seen.items():
                    if parts[0][0] is None:
                        assert parts == [(None, 0, steps)]
                    else:
                        parts.sort()
                        assert [p[0] for p in parts] == list(range(S))
                        assert sum(p[2] for p in parts) == steps  # the slices tile K
                        assert all(parts[i][1] + parts[i][2] == parts[i + 1][1] for i in range(S - 1))
                coords = {tail_tile_coords(L, m_tiles, n_tiles) for L in range(m_tiles * n_tiles)}
                assert coords == {(a, b) for a in range(m_tiles) for b in range(n_tiles)}
                tested += 1
    assert tested > 100


def test_tail_split_merge_shape():
    """The merge at 8192 tokens: 32 x 28 tiles, 112 per XCD on 32 CUs; the last
    16 of each XCD run as two K slices of 172 steps."""
    assert tail_plan(32, 28, 344, 32) == (2, 96, 172)
    assert tail_plan(32, 14, 56, 32) is None  # the latent: last wave 3/4 full
