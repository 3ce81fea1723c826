"""Pins of the oracle's cache append (kvcache_append_ref).

Passages: deepseek.csdn.net FlashMLA article, section 4.1 (the cache keeps
every earlier token's latent row and a step adds the new token's) and
section 4.2(1) (64-slot pages mapped through block_table).

The checks: a worked example whose destinations are listed by hand, the
decode gather of the appended cache against the concatenation of the old
rows and the new ones, every other byte unchanged, the rows that cannot be
placed, and planted mistakes that these checks catch."""
import inspect

import numpy as np
import pytest

import oracle.mla_oracle as mo
from oracle.mla_oracle import PAGE_SIZE, gather_latent_rows, kvcache_append_ref

D = 576


def _rows(rng, *shape):
    return rng.integers(1, 1 << 15, size=shape + (D,), dtype=np.uint16)


def _pins(fn):
    """Run every pin against an append function; returns the failures."""
    failed = []
    rng = np.random.default_rng(3)
    # worked example: sequence 0 holds 63 tokens in pages [2, 0], sequence 1 none
    cache = np.zeros((4, PAGE_SIZE, 1, D), np.uint16)
    bt = np.array([[2, 0], [3, 1]], np.int32)
    new = _rows(rng, 2, 2, 1)
    out, bad = fn(cache, bt, np.array([63, 0], np.int32), new)
    want = {(2, 63): new[0, 0, 0], (0, 0): new[0, 1, 0], (3, 0): new[1, 0, 0], (3, 1): new[1, 1, 0]}
    ok = bad == 0 and all(np.array_equal(out[p, s, 0], v) for (p, s), v in want.items())
    mask = np.ones((4, PAGE_SIZE), bool)
    for p, s in want:
        mask[p, s] = False
    if not (ok and not out[mask].any()):
        failed.append("worked example")
    # gather of the appended cache = old rows followed by the new ones
    B, h_kv, s_new, P = 3, 2, 3, 12
    L = np.array([0, 62, 127], np.int32)
    bt = rng.permutation(P).astype(np.int32).reshape(B, 4)
    cache = _rows(rng, P, PAGE_SIZE, h_kv)
    new = _rows(rng, B, s_new, h_kv)
    out, bad = fn(cache, bt, L, new)
    for b in range(B):
        for g in range(h_kv):
            old = gather_latent_rows(cache, bt[b], int(L[b]), g)
            got = gather_latent_rows(out, bt[b], int(L[b]) + s_new, g)
            if bad or not np.array_equal(got, np.concatenate([old, new[b, :, g].astype(np.float64)])):
                failed.append(f"gather b={b} g={g}")
    changed = np.argwhere((out != cache).any(axis=-1))
    placed = {(int(bt[b, (L[b] + i) // PAGE_SIZE]), int((L[b] + i) % PAGE_SIZE), g)
              for b in range(B) for i in range(s_new) for g in range(h_kv)}
    if not {tuple(map(int, c)) for c in changed} <= placed:
        failed.append("bytes outside the new rows changed")
    # rows that cannot be placed: past the block table, page id out of range, negative length
    cache = _rows(rng, 2, PAGE_SIZE, 1)
    bt = np.array([[0], [2], [1]], np.int32)          # page id 2 = P: out of range
    out, bad = fn(cache, bt, np.array([63, 0, -1], np.int32), _rows(rng, 3, 2, 1))
    if bad != 1 + 2 + 2 or not np.array_equal(np.delete(out.reshape(-1, D), 63, 0), np.delete(cache.reshape(-1, D), 63, 0)):
        failed.append("unplaceable rows")
    return failed


def test_append_pins():
    assert _pins(kvcache_append_ref) == []


@pytest.mark.parametrize("old,new", [
    ("out[pid, pos % PAGE_SIZE, g, :]", "out[pid, (pos + 1) % PAGE_SIZE, g, :]"),   # slot off by one
    ("pos = int(L[b]) + i", "pos = i"),                                             # length ignored
    ("blk = pos // PAGE_SIZE", "blk = pos // (PAGE_SIZE - 1)"),                     # wrong page size
    ("new[b, i, g, :]", "new[b, i, h_kv - 1 - g, :]"),                              # heads swapped
    ("if not 0 <= pid < P:", "if not 0 <= pid <= P:"),                              # bound off by one
])
def test_planted_append_mistakes_are_caught(old, new):
    src = inspect.getsource(kvcache_append_ref)
    assert src.count(old) == 1
    ns = dict(vars(mo))
    exec(src.replace(old, new), ns)
    try:
        failed = _pins(ns["kvcache_append_ref"])
    except (IndexError, AssertionError):
        failed = ["raised"]
    assert failed
