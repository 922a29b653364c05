"""The host encoder against the oracle over the seeded parity sweep
(workloads.sweep_cases: random shapes, weight recipes, K, L and G): the
library writes the oracle's bytes for every configuration, and the oracle
decodes them back to the original bits."""
import numpy as np
import pytest

import workloads
from oracle import blob as oblob

import decode_gemv_canonical_amd as uw

CASES = workloads.sweep_cases()


def _id(c):
    return f"{c['id']}-{c['recipe']}-{c['rows']}x{c['cols']}-K{c['K']}L{c['L']}G{c['G']}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_sweep_encoder_matches_oracle(case):
    w = workloads.sweep_weights(case).numpy().view(np.uint16)
    lib = uw.uw_encode(w, K=case["K"], L=case["L"], G=case["G"])
    ora = oblob.encode(w, K=case["K"] or 16, L=case["L"] or 6, G=case["G"] or None)
    assert lib == ora
    assert np.array_equal(oblob.decode(lib), w)


def test_sweep_covers_every_family():
    # the sweep reaches raw groups, plain mode, the single-code table, blocks
    # that end mid-row and ragged last blocks
    infos = []
    for c in CASES:
        w = workloads.sweep_weights(c).numpy().view(np.uint16)
        infos.append((c, uw.uw_blob_info(uw.uw_encode(w, K=c["K"], L=c["L"], G=c["G"]))))
    coded = [(c, i) for c, i in infos if not i["plain"]]
    assert any(i["plain"] for _, i in infos)
    assert any(i["n_raw_groups"] > 0 for _, i in coded)
    assert any(i["L"] > 6 for _, i in coded)
    assert any(i["G"] > c["cols"] // 64 and i["G"] % (c["cols"] // 64) for c, i in coded)
    assert any((c["rows"] * c["cols"] // 64) % i["G"] for c, i in coded)
