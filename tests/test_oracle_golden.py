"""Pins of the oracle against numbers the pages print (tests/golden/).

The receptive field and the token budget are measured by sensitivity: a key
or value row belongs to a query's receptive field exactly when perturbing it
changes that query's output.
"""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_parameters.json")))


def _sensitive_rows(fn, V, i_row):
    base = fn(V)
    hits = []
    for j in range(V.shape[2]):
        V2 = V.copy()
        V2[:, :, j] += 1.0
        if not np.array_equal(fn(V2), base):
            hits.append(j)
    return hits


def test_hsa_receptive_field_is_topk_times_chunk_size():
    g = GOLDEN["hsa"]
    S, K_ = g["chunk_size"], g["top_k"]
    L, d, t = 12 * S, 8, 11 * S + 5  # 11 chunks lie fully before t
    Q = synth.normal((1, 1, L, d), synth.F32, 21, synth.TID_Q)
    K = synth.normal((1, 1, L, d), synth.F32, 21, synth.TID_K)
    V = synth.normal((1, 1, L, d), synth.F32, 21, synth.TID_V)

    def fn(Vx):
        return oracle.hsa_prefill(Q, K, Vx, S=S, topk=K_, rows=[t])["out"]

    hits = _sensitive_rows(fn, V, t)
    assert len(hits) == g["receptive_field_tokens"] == K_ * S
    sel = oracle.hsa_prefill(Q, K, V, S=S, topk=K_, rows=[t])["sel"][0, 0, 0]
    assert sorted(hits) == sorted(j for c in sel for j in range(c * S, (c + 1) * S))
    assert max(hits) < (t // S) * S  # nothing from the chunk holding t


def test_dhsa_each_query_keeps_its_token_budget():
    budgets = GOLDEN["dhsa"]["token_budgets"]
    L, d = 700, 8
    Q = synth.normal((1, 1, L, d), synth.F32, 22, synth.TID_Q)
    K = synth.normal((1, 1, L, d), synth.F32, 22, synth.TID_K)
    V = synth.normal((1, 1, L, d), synth.F32, 22, synth.TID_V)
    offs = synth.chunk_offsets(L, 16, 128, seed=22)
    for nb in budgets:
        for i in (L - 1, 400):
            def fn(Vx):
                return oracle.dhsa_prefill(Q, K, Vx, offs, budget=nb, rows=[i])["out"]
            hits = _sensitive_rows(fn, V, i)
            assert len(hits) == min(nb, i + 1) and max(hits) <= i
