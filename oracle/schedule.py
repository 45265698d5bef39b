"""Block schedules of the bounded cache, two derivations each.

PR-Sink (LiveAnimate page, section 方法, PR-Sink bullets; section 关键发现,
memory-and-latency bullet): the context of block m is a static sink (the
first generated block, kept for good), dynamic sink blocks retrieved by pose,
a rolling window of the last three blocks, and the current block.

Readings where the page is silent:
  * The static sink is block 0 only and never enters the window or the bank.
  * Retrievable history is a FIFO bank holding the last ``bank`` blocks that
    left the window (the page keeps "a fixed number of blocks"; all evicted
    blocks would grow without bound).
  * Block m's window is {max(S, m-W), ..., m-1} with S static blocks.

ConvKV (SoulX-LiveAct page, section 技术内核, ConvKV Memory bullet): recent
blocks keep exact KV; older frames are compressed by a stride=kernel 1D conv
into fixed-length memory.  Reading: the memory is rebuilt at every commit
from the ``kernel * memory_frames`` most recent evicted frames (grid aligned
to the newest end); it exists once at least ``kernel`` frames were evicted.

``*_schedule`` is the closed form; ``simulate_*`` steps a ring and a FIFO block
by block.  A test checks that the two agree.
"""
from __future__ import annotations

from collections import deque


def prsink_schedule(m: int, window: int = 3, bank: int = 8, static: int = 1) -> dict:
    """Closed-form PR-Sink schedule for block m (0-based stream index).

    Returns dict with ``static``, ``bank`` (oldest first), ``window`` (oldest
    first) stream ids as seen when block m is open, and ``evicted``: the id
    that leaves the window when block m is committed (or None).
    """
    static_ids = list(range(min(static, m)))
    window_ids = list(range(max(static, m - window), m))
    evicted_ids = list(range(static, m - window))            # left the window before m
    bank_ids = evicted_ids[max(0, len(evicted_ids) - bank):] if bank > 0 else []
    ev = m - window if (m >= static and m - window >= static) else None
    return {"static": static_ids, "bank": bank_ids, "window": window_ids, "evicted": ev}


def simulate_prsink(n_blocks: int, window: int = 3, bank: int = 8, static: int = 1) -> list:
    """Step-by-step PR-Sink bookkeeping: same keys as :func:`prsink_schedule`."""
    statics, win, bnk = [], deque(), deque()
    out = []
    for m in range(n_blocks):
        rec = {"static": list(statics), "bank": list(bnk), "window": list(win), "evicted": None}
        # commit block m
        if len(statics) < static:
            statics.append(m)
        else:
            win.append(m)
            if len(win) > window:
                e = win.popleft()
                rec["evicted"] = e
                if bank > 0:
                    bnk.append(e)
                    if len(bnk) > bank:
                        bnk.popleft()
        out.append(rec)
    return out


def simulate_prsink_pose_bank(n_blocks: int, pose, window: int = 3, bank: int = 8, static: int = 1) -> list:
    """PR-Sink bookkeeping with pose-aware bank replacement (same keys as
    :func:`prsink_schedule`; ``pose(b)`` gives block b's pose).

    Reading (alternative to the FIFO bank): the bank still holds a fixed
    number of blocks (LiveAnimate page, section 关键发现), but when a block
    leaves the window into a full bank, the member it makes most redundant
    leaves -- the one whose pose has the largest cosine with the entering
    block's pose, ranked exactly as retrieval ranks (section 局限: retrieval
    by pose similarity), so exact ties drop the lower stream id and a zero
    pose scores 0.  The entering block joins at the end (admission order).
    """
    it = iter_prsink_pose_bank(pose, window, bank, static)
    return [next(it) for _ in range(n_blocks)]


def iter_prsink_pose_bank(pose, window: int = 3, bank: int = 8, static: int = 1):
    """The records of :func:`simulate_prsink_pose_bank`, block by block, for
    as long as asked: record m needs the poses of blocks < m only."""
    from .retrieval import retrieve
    statics, win, bnk = [], deque(), []
    m = 0
    while True:
        rec = {"static": list(statics), "bank": list(bnk), "window": list(win), "evicted": None}
        if len(statics) < static:
            statics.append(m)
        else:
            win.append(m)
            if len(win) > window:
                e = win.popleft()
                rec["evicted"] = e
                if bank > 0:
                    if len(bnk) == bank:
                        victim = retrieve(pose(e), [(b, pose(b)) for b in bnk], 1)[0]
                        bnk.remove(victim)
                    bnk.append(e)
        yield rec
        m += 1


def convkv_schedule(m: int, frames: int, window: int = 3, kernel: int = 5,
                    memory_frames: int = 1) -> dict:
    """Closed-form ConvKV schedule for block m.

    Evicted frames are numbered in stream order: frame f of block b is
    b * frames + f.  Returns ``window`` block ids (oldest first), ``evicted_frames``
    (count E), ``memory``: list of memory frames, each the list of ``kernel``
    evicted frame numbers it combines (tap 0 = oldest), and ``frame_t0``:
    the context-relative temporal position of the first frame of every
    context part, in order memory, window blocks, current block.
    """
    window_ids = list(range(max(0, m - window), m))
    E = frames * max(0, m - window)
    n_mem = min(memory_frames, E // kernel)
    first = E - n_mem * kernel
    memory = [[first + j * kernel + i for i in range(kernel)] for j in range(n_mem)]
    t0 = {"memory": 0, "window": [n_mem + i * frames for i in range(len(window_ids))],
          "current": n_mem + len(window_ids) * frames}
    return {"window": window_ids, "evicted_frames": E, "memory": memory, "t0": t0,
            "evicted": (m - window) if m - window >= 0 else None}


def simulate_convkv(n_blocks: int, frames: int, window: int = 3, kernel: int = 5,
                    memory_frames: int = 1) -> list:
    """Step-by-step ConvKV bookkeeping: a window ring plus a list of evicted frames."""
    win = deque()
    evicted_frames = []
    out = []
    for m in range(n_blocks):
        E = len(evicted_frames)
        n_mem = min(memory_frames, E // kernel)
        tail = evicted_frames[E - n_mem * kernel:] if n_mem else []
        memory = [tail[j * kernel:(j + 1) * kernel] for j in range(n_mem)]
        t, win_t0 = n_mem, []
        for _ in win:
            win_t0.append(t)
            t += frames
        rec = {"window": list(win), "evicted_frames": E, "memory": memory,
               "t0": {"memory": 0, "window": win_t0, "current": t}, "evicted": None}
        win.append(m)
        if len(win) > window:
            e = win.popleft()
            rec["evicted"] = e
            evicted_frames.extend(e * frames + f for f in range(frames))
        out.append(rec)
    return out


def token_positions(frames: int, grid_h: int, grid_w: int):
    """(frame, y, x) of each token of a block, token index = (f * grid_h + y) * grid_w + x."""
    import numpy as np
    f, y, x = np.meshgrid(np.arange(frames), np.arange(grid_h), np.arange(grid_w), indexing="ij")
    return f.reshape(-1), y.reshape(-1), x.reshape(-1)
