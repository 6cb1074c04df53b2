"""The ring mode's task stream, on the CPU, through moe_ring_schedule (the
function the persistent kernel decodes its tickets with): every task once,
the lag order of [DeepGEMM #88] "How it works", every wait pointing at a
lower ticket, and a drain simulation with any number of workers holding a
prefetched ticket each, as the kernel's workgroups do.  Also the ring
workspace arithmetic."""

import numpy as np
import pytest

import mixture_experts_ffn_moe_amd as moe

# (blocks, up tasks per block, down tasks per block, lag)
STREAMS = [(1, 1, 1, 0), (1, 16, 16, 5), (7, 2, 16, 0), (7, 2, 16, 3), (7, 2, 16, 7),
           (7, 2, 16, 30), (48, 16, 16, 36), (50, 4, 3, 9), (13, 1, 1, 1), (0, 16, 16, 4)]


def positions(kind, block, index, nb, S, NT):
    up = np.full((nb, S), -1)
    down = np.full((nb, NT), -1)
    for t, (k, b, i) in enumerate(zip(kind, block, index)):
        (up if k == 1 else down)[b, i] = t
    return up, down


@pytest.mark.parametrize("nb,S,NT,lag", STREAMS)
def test_every_task_once_in_lag_order(nb, S, NT, lag):
    kind, block, index = moe.moe_ring_schedule(nb, S, NT, lag)
    assert len(kind) == nb * (S + NT) and set(kind.tolist()) <= {1, 2}
    seen = set(zip(kind.tolist(), block.tolist(), index.tolist()))
    assert seen == {(1, b, i) for b in range(nb) for i in range(S)} | \
        {(2, b, i) for b in range(nb) for i in range(NT)}
    up, down = positions(kind, block, index, nb, S, NT)
    # each kind in block order, tasks of a block in index order
    assert (np.diff(up.ravel()) > 0).all() and (np.diff(down.ravel()) > 0).all()
    for b in range(nb):
        # between block b's last up task and its first down task lie the up
        # tasks of exactly min(lag, nb - 1 - b) later blocks
        between = [c for c in range(nb) if up[b, -1] < up[c, 0] < down[b, 0]]
        assert between == list(range(b + 1, b + 1 + min(lag, nb - 1 - b)))
    k2, _, _ = moe.moe_ring_schedule(nb, S, NT, lag, first=nb * (S + NT), count=3)
    assert (k2 == 0).all()


@pytest.mark.parametrize("nb,S,NT,lag", [c for c in STREAMS if c[0] > 0])
def test_waits_point_at_lower_tickets(nb, S, NT, lag):
    up, down = positions(*moe.moe_ring_schedule(nb, S, NT, lag), nb, S, NT)
    for ring in range(lag + 1, lag + 4):
        for b in range(nb):
            assert down[b].min() > up[b].max()               # reads after every write
            if b >= ring:
                assert up[b].min() > down[b - ring].max()    # slot reuse after every read


def simulate(nb, S, NT, lag, ring, workers, seed):
    """Workers take tickets in order, the next one as they start a task (the
    kernel's prefetch), and finish a task only once its waits are met; a
    random ready worker moves at each step.  Returns the finished count."""
    kind, block, _ = moe.moe_ring_schedule(nb, S, NT, lag)
    total = len(kind)
    rng = np.random.default_rng(seed)
    up_done, down_done = np.zeros(nb, int), np.zeros(nb, int)
    nxt = 0
    held = []
    for _ in range(workers):
        held.append([nxt, nxt + 1])
        nxt += 2
    finished = 0

    def ready(t):
        if t >= total:
            return False
        b = block[t]
        if kind[t] == 1:
            return b < ring or down_done[b - ring] == NT
        return up_done[b] == S

    while True:
        live = [w for w in range(workers) if held[w][0] < total]
        if not live:
            return finished
        cand = [w for w in live if ready(held[w][0])]
        if not cand:
            return finished    # no worker can move: a deadlock
        w = cand[rng.integers(len(cand))]
        t = held[w][0]
        (up_done if kind[t] == 1 else down_done)[block[t]] += 1
        finished += 1
        held[w] = [held[w][1], nxt]
        nxt += 1


@pytest.mark.parametrize("nb,S,NT,lag", [(9, 2, 3, 0), (9, 2, 3, 2), (20, 4, 4, 6), (6, 3, 2, 9)])
@pytest.mark.parametrize("workers", [1, 2, 5, 64])
def test_stream_drains(nb, S, NT, lag, workers):
    for ring in (lag + 1, lag + 2, 2 * lag + 2):
        for seed in range(3):
            assert simulate(nb, S, NT, lag, ring, workers, seed) == nb * (S + NT)


def test_simulation_catches_a_bad_ring():
    # a ring no larger than the lag makes a block's up tasks wait on down
    # tasks that come later in the stream: one worker stalls for good
    assert simulate(9, 2, 3, 3, 3, 1, 0) < 9 * 5


def test_schedule_errors():
    with pytest.raises(moe.MoeError):
        moe.moe_ring_schedule(4, 0, 2, 1)
    with pytest.raises(moe.MoeError):
        moe.moe_ring_schedule(4, 2, 2, -1)


@pytest.mark.parametrize("dtype,es,sb", [("bf16", 2, 0), ("fp8_blockwise", 1, 4 * 16),
                                         ("mxfp8", 1, 64), ("mxfp4", 1, 64)])
@pytest.mark.parametrize("T,bm", [(8, 16), (256, 16), (64, 32), (1, 16)])
def test_ring_workspace(dtype, es, sb, T, bm):
    K, N, E, k = 4096, 4096, 256, 6
    fixed, slot, slots = moe.moe_ring_layout(dtype, T, K, N, E, k, bm)
    I = N // 2
    assert slot == bm * (I * es + sb)
    _, blocks = moe.moe_align_capacity(T, k, E, bm)
    lag_max = -(-3 * 512 // (2 * (I // 128)))
    assert slots == min(blocks, 2 * lag_max + 2)
    total = moe.moe_workspace_size(dtype, T, K, N, E, k, bm, split=2)
    assert total == -(-(fixed + slots * slot) // 256) * 256
    R = T * k
    assert fixed >= R * K * 2 + R * 4          # per-route bf16 rows and flags come first


def test_ring_layout_rejects_large_blocks():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ring_layout("fp8_blockwise", 8, 4096, 4096, 256, 6, 64)
    assert ei.value.status == -3
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size("fp8_blockwise", 8, 4096, 4096, 256, 6, 64, split=2)
