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
wgrad_kernel (csrc/wgrad_kernel.h): the A strip and B(0), then per column tile
t: wait for B(t), issue B(t+1) into the other buffer, multiply, stage, 8 stores.
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


def wgrad_schedule(KG, NT, wait_delta=0, stores=8, nwave=8):
    """Replays wgrad_kernel's issue order per wave: the A strip's two 128-row
    blocks (into B buffer 1 and the staging buffer), B tile 0 (into B buffer
    0), a wait for the strip; per column tile t: wait for B(t), B tile t+1 into
    buffer (t+1) % 2, multiply from buffer t % 2, stage, the stores of tile t.
    Also checks that no DMA still in flight targets a buffer being read or
    staged into."""
    dma = KG * (8 // nwave)  # DMA instructions per 128-row block per wave
    issued, last = [], {}    # issued: (tag, target buffer or None)

    def issue(tag, n, buf=None):
        issued.extend([(tag, buf)] * n)
        last[tag] = len(issued) - 1

    def in_flight(n):  # what may still be outstanding after vmcnt(n)
        return issued[len(issued) - n:] if n > 0 else []

    issue(("A", 0), dma, 1)
    issue(("A", 1), dma, "S")
    issue(("B", 0), dma, 0)
    n = dma + wait_delta
    assert last[("A", 1)] < len(issued) - n, (KG, NT)  # the strip is read
    assert all(b not in (1, "S") for _, b in in_flight(n))
    for t in range(NT):
        n = (0 if t == 0 else stores) + wait_delta
        assert last[("B", t)] < len(issued) - n, (KG, NT, t)
        flying = in_flight(n)
        if t + 1 < NT:
            issue(("B", t + 1), dma, (t + 1) % 2)
            flying = flying + issued[-dma:]
        # the MFMAs read buffer t % 2 and the staging writes "S"
        assert all(b not in (t % 2, "S") for _, b in flying), (KG, NT, t)
        issue(("S", t), stores)


@pytest.mark.parametrize("KG", [2, 4, 6])
def test_wgrad_vmcnt_schedule_is_exact(KG):
    for NT in range(1, 30):
        wgrad_schedule(KG, NT)
    with pytest.raises(AssertionError):
        wgrad_schedule(KG, 4, wait_delta=1)
