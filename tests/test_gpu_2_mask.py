"""GPU parity of hn_attn_mask_build: the dense expansion of the tile plan must
equal the oracle's explicit mask bit for bit (in the canonical key order), and
every key absent from the cache state must be invisible in the oracle mask."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_attention_hn_amd as hn
    import _gpu as G

_DATA = {}


def data_of(name):
    if name not in _DATA:
        _DATA[name] = W.generate(W.config(name))
    return _DATA[name]


@pytest.mark.parametrize("name,rows_env", [(n, "auto") for n in
                                           ("c1", "c1_evict", "c1_future", "m1", "m2", "m3", "m4",
                                            "c2", "c3", "c4", "c5")] +
                         [(n, "128") for n in ("c1", "m1", "m2", "m4", "c2")])
def test_dense_mask_matches_oracle(name, rows_env):
    # the spans are built per plan tile; both tile heights must expand to the oracle mask
    print(f"[mask] {name} rows={rows_env}", flush=True)
    opts = None if rows_env == "auto" else hn.PlanOpts(tile_rows=int(rows_env))
    w = W.config(name)
    d = data_of(name)
    run = G.Run(w, d, opts=opts)
    nq = w.current.video_len
    rows = np.arange(nq) if nq <= 2048 else G.sample_rows(nq)
    csr = d.get("csr") if w.sparse_keep is not None else None
    ref_full = oracle.mask(w, rows, csr)
    cols = G.canonical_columns(w)
    absent = np.ones(ref_full.shape[1], bool)
    absent[cols] = False
    assert not ref_full[:, absent].any()
    ref = ref_full[:, cols]
    # contiguous row blocks through the DENSE mode
    got = np.zeros_like(ref)
    i = 0
    while i < len(rows):
        j = i
        while j + 1 < len(rows) and rows[j + 1] == rows[j] + 1 and j + 1 - i < 512:
            j += 1
        got[i:j + 1] = run.dense(int(rows[i]), j + 1 - i)
        i = j + 1
    assert np.array_equal(got, ref)


def test_plan_visible_pairs_equal_oracle_count():
    for name in ("c1", "m1", "m2", "c3"):
        w = W.config(name)
        run = G.Run(w, data_of(name))
        assert run.plan.visible_pairs * 4 * 128 * w.heads == oracle.effective_flops(w)
