"""Pins of the whole-page allocator's oracle (pages_init_ref,
pages_reserve_ref, pages_release_ref): memory goes out and comes back only
in whole 64-token pages.  A worked example whose every step was derived by
hand, a conservation invariant over random sequences of operations (each
page of the pool is, at every moment, either on the free stack or mapped by
exactly one block-table entry, and the mapped entries are exactly the first
ceil(L_b / 64) of each row), and planted mistakes that must fail them."""
import numpy as np
import pytest

import oracle.mla_oracle as mo


def _table(rows):
    return np.array(rows, dtype=np.int64)


def test_worked_example():
    fp, cnt = mo.pages_init_ref(6)
    assert fp.tolist() == [5, 4, 3, 2, 1, 0] and cnt == 6
    bt = _table([[-1] * 3] * 3)
    # A: three empty sequences take 65 tokens each: 2 pages each, popped 0, 1, 2, ...
    fp, cnt, bt, st, n = mo.pages_reserve_ref(fp, cnt, [0, 0, 0], 65, bt)
    assert (st, n, cnt) == (0, 6, 0)
    assert bt.tolist() == [[0, 1, -1], [2, 3, -1], [4, 5, -1]]
    # B: one more token each stays inside the second page: nothing moves.
    fp2, cnt2, bt2, st, n = mo.pages_reserve_ref(fp, cnt, [65, 65, 65], 1, bt)
    assert (st, n, cnt2) == (0, 0, 0) and (bt2 == bt).all() and (fp2 == fp).all()
    # C: 64 more tokens each need a third page each, and none is free.
    fp2, cnt2, bt2, st, n = mo.pages_reserve_ref(fp, cnt, [65, 65, 65], 64, bt)
    assert (st, n, cnt2) == (1, 3, 0) and (bt2 == bt).all()
    # D: sequence 1 ends; its pages 2 and 3 go back on the stack.
    fp, cnt, bt, st, n = mo.pages_release_ref(fp, cnt, [65, 65, 65], [0, 1, 0], bt, 6)
    assert (st, n, cnt) == (0, 2, 2)
    assert fp[:2].tolist() == [2, 3] and bt.tolist() == [[0, 1, -1], [-1, -1, -1], [4, 5, -1]]
    # E: three pages wanted, two free: refused, nothing changes.
    fp2, cnt2, bt2, st, n = mo.pages_reserve_ref(fp, cnt, [65, 0, 65], 64, bt)
    assert (st, n, cnt2) == (1, 3, 2) and (bt2 == bt).all()
    # F: sequence 1 starts again with 8 tokens: it takes the top, page 3.
    fp, cnt, bt, st, n = mo.pages_reserve_ref(fp, cnt, [65, 0, 120], 8, bt)
    assert (st, n, cnt) == (0, 1, 1) and bt.tolist() == [[0, 1, -1], [3, -1, -1], [4, 5, -1]]
    # G: sequences 0 and 2 end (65 and 128 tokens: two pages each).
    fp, cnt, bt, st, n = mo.pages_release_ref(fp, cnt, [65, 8, 128], [1, 0, 1], bt, 6)
    assert (st, n, cnt) == (0, 4, 5) and fp[:5].tolist() == [2, 0, 1, 4, 5]
    assert bt.tolist() == [[-1, -1, -1], [3, -1, -1], [-1, -1, -1]]
    # H: releasing sequence 0 again finds no valid page id: refused.
    fp2, cnt2, bt2, st, n = mo.pages_release_ref(fp, cnt, [65, 8, 128], [1, 0, 0], bt, 6)
    assert (st, cnt2) == (2, 5) and (bt2 == bt).all() and (fp2[:5] == fp[:5]).all()
    # I: a length past the table row is refused.
    fp2, cnt2, bt2, st, n = mo.pages_reserve_ref(fp, cnt, [0, 8, 0], 200, bt)
    assert (st, cnt2) == (2, 5) and (bt2 == bt).all()


def check_conservation(fp, cnt, bt, L, num_pages):
    """Every page once: free (fp[:cnt]) or mapped (bt[b][:ceil(L_b/64)]);
    entries past a row's mapped blocks are -1."""
    seen = list(np.asarray(fp[:cnt]).tolist())
    for b in range(bt.shape[0]):
        n = (int(L[b]) + 63) // 64
        seen += bt[b, :n].tolist()
        assert (bt[b, n:] == -1).all(), f"row {b} maps blocks past its length"
    assert sorted(seen) == list(range(num_pages)), "a page was lost or handed out twice"


def random_walk(seed, steps=60, num_pages=40, B=5, max_pages=12, fns=None):
    """Random reserves (1..150 new tokens) and releases; returns the states."""
    fns = fns or (mo.pages_init_ref, mo.pages_reserve_ref, mo.pages_release_ref)
    init, reserve, release = fns
    rng = np.random.default_rng(seed)
    fp, cnt = init(num_pages)
    bt = np.full((B, max_pages), -1, dtype=np.int64)
    L = np.zeros(B, dtype=np.int64)
    states = []
    for _ in range(steps):
        if rng.random() < 0.7:
            s_new = int(rng.integers(1, 150))
            fp, cnt, bt, st, _ = reserve(fp, cnt, L, s_new, bt)
            if st == 0:
                L = L + s_new
        else:
            rel = (rng.random(B) < 0.4).astype(np.int64)
            fp, cnt, bt, st, _ = release(fp, cnt, L, rel, bt, num_pages)
            if st == 0:
                L = np.where(rel != 0, 0, L)
        states.append((fp.copy(), cnt, bt.copy(), L.copy()))
    return states


@pytest.mark.parametrize("seed", range(6))
def test_conservation_over_random_operations(seed):
    states = random_walk(seed)
    for fp, cnt, bt, L in states:
        check_conservation(fp, cnt, bt, L, 40)
    # the walk exercises both refusals and reuse of released pages
    assert any(cnt == 0 for _, cnt, _, _ in states) or seed > 2


def _mutant(kind):
    real_reserve, real_release = mo.pages_reserve_ref, mo.pages_release_ref

    def reserve(fp, cnt, L, s_new, bt):
        if kind == "need_ignores_mapped":          # asks for ceil(s_new / 64) pages, as if none were mapped
            L0 = np.zeros_like(np.asarray(L))
            out = list(real_reserve(fp, cnt, L0, s_new, bt))
            return tuple(out)
        if kind == "pop_from_bottom":
            fp2 = np.array(fp, copy=True)
            fp2[:cnt] = fp2[:cnt][::-1]
            return real_reserve(fp2, cnt, L, s_new, bt)
        if kind == "partial_on_failure":
            fp2, cnt2, bt2, st, n = real_reserve(fp, cnt, L, s_new, bt)
            if st == 1:   # hand out what there is
                bt2 = np.array(bt, copy=True)
                Ls = np.asarray(L)
                top = cnt
                for b in range(bt2.shape[0]):
                    for j in range((int(Ls[b]) + 63) // 64, (int(Ls[b]) + s_new + 63) // 64):
                        if top == 0:
                            break
                        top -= 1
                        bt2[b, j] = fp[top]
                return np.array(fp, copy=True), top, bt2, 0, n
            return fp2, cnt2, bt2, st, n
        return real_reserve(fp, cnt, L, s_new, bt)

    def release(fp, cnt, L, rel, bt, P):
        fp2, cnt2, bt2, st, n = real_release(fp, cnt, L, rel, bt, P)
        if kind == "release_keeps_entries" and st == 0:
            bt2 = np.array(bt, copy=True)
        return fp2, cnt2, bt2, st, n

    return mo.pages_init_ref, reserve, release


@pytest.mark.parametrize("kind", ["need_ignores_mapped", "pop_from_bottom", "partial_on_failure",
                                  "release_keeps_entries"])
def test_planted_allocator_mistakes_are_caught(kind):
    def pins_pass():
        try:
            for seed in range(4):
                for fp, cnt, bt, L in random_walk(seed, fns=_mutant(kind)):
                    check_conservation(fp, cnt, bt, L, 40)
            # the worked example's pop order
            fp, cnt = mo.pages_init_ref(6)
            _, _, bt, _, _ = _mutant(kind)[1](fp, cnt, [0, 0, 0], 65, _table([[-1] * 3] * 3))
            assert bt.tolist() == [[0, 1, -1], [2, 3, -1], [4, 5, -1]]
        except AssertionError:
            return False
        return True
    assert not pins_pass(), f"planted mistake {kind!r} slipped through"
