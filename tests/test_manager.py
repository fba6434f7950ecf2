"""The decode-time block manager (kvq_manager_*, host code): slots of new
tokens per layer group, block tables, ring retention of sliding layers,
release and exhaustion, checked as properties of what it hands out."""
import random

import pytest

import workloads as W


@pytest.fixture(scope="module")
def kvq():
    import quantized_fp8_int4_amd as kvq
    return kvq


BS = 16


def _model(kvq, wins=(0, 32, 0, 32, 64)):
    modes = [W.FP8_PER_TOKEN_HEAD if w == 0 else W.BF16 for w in wins]
    return kvq.ModelConfig(BS, 2, 64, modes, list(wins))


def _check(kvq, m, wins, nblocks, hist):
    """hist[seq] = {group: [slot of token 0, 1, ...]} for the live sequences."""
    groups = sorted(set(wins), key=list(wins).index)
    for g, w in enumerate(groups):
        live = []
        for seq, per in hist.items():
            sl = per[g]
            keep = sl[-w:] if w else sl
            live += keep
            assert all(0 <= s < nblocks[g] * BS for s in keep)
            if w:
                for t in range(len(sl) - w):
                    # token t + W reuses token t's ring position (either may
                    # have been displaced within its own call and not stored)
                    assert sl[t] == sl[t + w] or -1 in (sl[t], sl[t + w])
            bt, lens = m.tables(g, [seq])
            assert lens[0] == len(keep)
            view = {bt[0][j // BS] * BS + j % BS for j in range(lens[0])}
            assert view == set(keep)
        assert len(live) == len(set(live)), f"group {g}: two live tokens share a slot"


def test_random_appends_and_releases(kvq):
    wins = (0, 32, 0, 32, 64)
    groups = [0, 32, 64]
    nblocks = {0: 40, 1: 12, 2: 16}
    per_layer = [nblocks[groups.index(w)] for w in wins]
    m = kvq.SeqManager(_model(kvq, wins), per_layer, max_blocks_per_seq=20)
    assert m.num_groups == 3 and [m.layer_group(l) for l in range(5)] == [0, 1, 0, 1, 2]
    rng = random.Random(0)
    hist = {}
    for step in range(300):
        if hist and rng.random() < 0.08:
            seq = rng.choice(sorted(hist))
            m.release(seq)
            del hist[seq]
        else:
            seq = rng.randrange(6)
            n = rng.choice([0, 1, 1, 1, 3, 17, 40])
            try:
                slots = m.append(seq, n)
            except kvq.KVQError as e:
                assert e.status in (kvq.ERR_NO_SPACE, kvq.ERR_INVALID_ARG)
                continue
            h = hist.setdefault(seq, {g: [] for g in range(3)})
            for g in range(3):
                stored = [x for x in slots[g] if x >= 0]
                assert len(stored) == len(set(stored))          # one call never repeats a slot
                assert slots[g].count(-1) == max(0, n - groups[g]) if groups[g] else slots[g].count(-1) == 0
                h[g] += slots[g]
        _check(kvq, m, groups, [nblocks[g] for g in range(3)], hist)
    m.close()


def test_exhaustion_changes_nothing_and_release_restores(kvq):
    m = kvq.SeqManager(_model(kvq, (0, 32)), [4, 4], max_blocks_per_seq=8)
    a = m.append(0, 40)                       # 3 full blocks, 2 ring blocks
    before = m.tables(0, [0]), m.tables(1, [0])
    with pytest.raises(kvq.KVQError) as e:
        m.append(1, 17)                        # needs 2 full blocks, only 1 left
    assert e.value.status == kvq.ERR_NO_SPACE
    assert (m.tables(0, [0]), m.tables(1, [0])) == before
    with pytest.raises(kvq.KVQError) as e:
        m.tables(0, [1])                       # the failed append created nothing
    assert e.value.status == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as e:
        m.append(0, 8 * BS)                    # past max_blocks_per_seq
    assert e.value.status == kvq.ERR_INVALID_ARG
    m.release(0)
    b = m.append(1, 64)                        # all 4 blocks of each group again
    assert sorted(set(s // BS for s in b[0])) == [0, 1, 2, 3]
    assert len(set(s // BS for s in b[1] if s >= 0)) == 2 and b[1].count(-1) == 64 - 32
    assert sorted(set(s // BS for s in a[0])) == [0, 1, 2]
    m.close()


def test_planned_blocks_hold_exactly_the_planned_sequences(kvq):
    """The planner's block counts, given to the manager, admit exactly
    max_sequences sequences of the planned context."""
    model = _model(kvq, (0, 32, 0, 32))
    context = 100
    plan, blocks = kvq.kvq_plan_capacity(model, context, 3 << 20)
    n = plan["max_sequences"]
    assert n > 1
    m = kvq.SeqManager(model, blocks, max_blocks_per_seq=-(-context // BS))
    for s in range(n):
        m.append(s, context)
    with pytest.raises(kvq.KVQError) as e:
        m.append(n, context)
    assert e.value.status == kvq.ERR_NO_SPACE
    m.close()


def test_manager_argument_checks(kvq):
    model = _model(kvq, (0, 32))
    with pytest.raises(kvq.KVQError):
        kvq.SeqManager(model, [4, 4], 0)
    with pytest.raises(kvq.KVQError):                           # a ring wider than the table
        kvq.SeqManager(model, [4, 4], 1)
    with pytest.raises(kvq.KVQError):                           # one group, two block counts
        kvq.SeqManager(_model(kvq, (0, 0)), [4, 5], 4)
    with pytest.raises(kvq.KVQError):
        kvq.SeqManager(kvq.ModelConfig(BS, 2, 64, [W.BF16], [24]), [4], 4)   # window not whole blocks
    m = kvq.SeqManager(model, [4, 4], 4)
    for bad in (lambda: m.append(-1, 1), lambda: m.append(0, -1), lambda: m.release(9),
                lambda: m.layer_group(2), lambda: m.tables(2, [0])):
        with pytest.raises(kvq.KVQError):
            bad()
    m.close()
