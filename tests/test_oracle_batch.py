"""Pins for request classification and the [decode:extend:prefill] reorder
against the page's iteration table (CPU only)."""
import json
import os

from oracle import batch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_iteration_table_paths_and_order():
    g = json.load(open(os.path.join(GOLD, "iteration_table.json")))
    names = {"decode": batch.DECODE, "extend": batch.EXTEND, "prefill": batch.PREFILL}
    for it in g["iterations"]:
        reqs = it["requests"]
        for r in reqs:
            assert batch.classify(r["query_len"], r["ctx_len"], g["threshold"]) == names[r["path"]], (it["it"], r)
        if "order" in it:
            perm, counts = batch.reorder([r["query_len"] for r in reqs],
                                         [r["ctx_len"] for r in reqs], g["threshold"])
            assert [reqs[i]["id"] for i in perm] == it["order"]
            assert sum(counts) == len(reqs)
    # R3: 100 of its 280 prompt tokens under a budget of 100, 180 left
    r3 = [r for it in g["iterations"] for r in it["requests"] if r["id"] == "R3"]
    assert r3[0]["query_len"] == g["token_budget"] and r3[1]["query_len"] == 280 - g["token_budget"]


def test_reorder_is_stable_and_grouped():
    q = [5, 1, 300, 1, 7, 1]
    c = [0, 10, 0, 99, 4, 0]
    perm, counts = batch.reorder(q, c)
    assert perm == [1, 3, 5, 4, 0, 2]
    assert counts == (3, 1, 2)
    # single-token prompt with no context counts as a decode (threshold rule)
    assert batch.classify(1, 0) == batch.DECODE
