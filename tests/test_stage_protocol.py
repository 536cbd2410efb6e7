"""CPU model of the attention kernel's LDS stage protocol.

The kernel (masked_attention_hn_amd/csrc/attn_fwd.hip, seg_attn_fwd_kernel)
keeps two LDS stages.  In every step it stages the next tile into one stage
while the waves compute the current tile from the other, then all waves wait
for their loads and meet at a barrier.  Blocks whose span list starts with
INT8 history tiles run them first with fp16 staging and math (phase 1), then
the segment's own bf16 tiles (phase 2); a history tile whose scales leave
fp16's range restarts the block with every tile staged in bf16.

This model replays that control flow step by step on tile sequences and
checks the invariants the kernel's correctness rests on:
  * a step never stages into the stage it computes from;
  * every tile is computed from the stage that holds it, staged in the type
    its math expects (fp16 math only on fp16-staged tiles);
  * a stage is overwritten only in the step after the one that computed it
    (the barrier between them orders the reads before the writes);
  * after the last step, every tile has been computed exactly once since the
    last restart, in span order.
"""
import itertools

import pytest
from hypothesis import given, settings, strategies as st

INT8, BF16 = "i8", "bf16"


def run_block(tiles, honor_odd=True):
    """tiles: list of (kind, ok16).  Returns the tiles computed since the last
    restart, asserting the invariants.  honor_odd=False plants a slip (phase 2
    ignoring which stage phase 1 left the current tile in)."""
    stage = [None, None]          # (tile index, staging type) held by each stage
    computed = []                 # tile indices computed since the last restart
    last_read = [None, None]      # step in which each stage was last computed from
    step_no = [0]
    it = iter(range(len(tiles)))

    def next_tile():
        return next(it, None)

    def stage_into(sn, idx, mode):
        # mode: 1 = phase-1 staging (INT8 in fp16), 2 = bf16 staging
        assert last_read[sn] is None or last_read[sn] < step_no[0], "stage overwritten before its reads"
        kind = tiles[idx][0]
        typ = "bf16" if kind == BF16 else ("f16" if mode == 1 else "bf16")
        stage[sn] = (idx, typ)

    def compute(sc, cur, f16_math):
        assert stage[sc] is not None and stage[sc][0] == cur, "computed from the wrong stage"
        typ = stage[sc][1]
        assert typ == ("f16" if f16_math else "bf16"), "math type differs from staging type"
        last_read[sc] = step_no[0]
        computed.append(cur)

    def step(sc, sn, cur, mode):
        # one pipeline step: stage the next tile into sn, compute cur from sc
        assert sc != sn
        nxt = next_tile()
        if nxt is not None:
            stage_into(sn, nxt, mode)
        compute(sc, cur, mode == 1)
        step_no[0] += 1           # waits + barrier: the step's reads and writes are done
        return nxt

    cur = next_tile()
    odd = False
    if cur is not None and tiles[cur][0] == INT8:
        stage_into(0, cur, 1)
        step_no[0] += 1
        redo = False
        while cur is not None and tiles[cur][0] == INT8:
            if not tiles[cur][1]:
                redo = True
                break
            cur = step(0, 1, cur, 1)
            if cur is None or tiles[cur][0] != INT8:
                odd = True
                break
            if not tiles[cur][1]:
                redo = True
                odd = True
                break
            cur = step(1, 0, cur, 1)
        if redo:
            computed.clear()
            it = iter(range(len(tiles)))
            cur = next_tile()
            odd = False
            stage_into(0, cur, 2)
            step_no[0] += 1
    elif cur is not None:
        stage_into(0, cur, 2)
        step_no[0] += 1
    if cur is not None and odd and honor_odd:
        cur = step(1, 0, cur, 2)
    while cur is not None:
        cur = step(0, 1, cur, 2)
        if cur is None:
            break
        cur = step(1, 0, cur, 2)
    return computed


def check(tiles):
    computed = run_block(tiles)
    assert computed == list(range(len(tiles)))


@pytest.mark.parametrize("n_i8,n_bf", list(itertools.product(range(5), range(5))))
def test_every_small_plan(n_i8, n_bf):
    for bad in range(n_i8 + 1):                      # bad == n_i8: every history tile in range
        tiles = [(INT8, i != bad) for i in range(n_i8)] + [(BF16, True)] * n_bf
        check(tiles)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 40), st.integers(0, 40), st.lists(st.booleans(), max_size=40))
def test_random_plans(n_i8, n_bf, oks):
    flags = [oks[i] if i < len(oks) else True for i in range(n_i8)]
    check([(INT8, f) for f in flags] + [(BF16, True)] * n_bf)


def test_model_catches_a_parity_slip():
    """The model fails if phase 2 ignored the stage phase 1 left the current
    tile in: one history tile then own tiles computes from the wrong stage."""
    with pytest.raises(AssertionError, match="wrong stage"):
        run_block([(INT8, True), (BF16, True), (BF16, True)], honor_odd=False)
