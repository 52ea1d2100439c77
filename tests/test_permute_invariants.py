"""The host-side grouping invariant checker (applied to every grouping the GPU tests copy back)
accepts the oracle's groupings and rejects planted mistakes. CPU only."""
import numpy as np
import pytest

import oracle as O
from parity_util import check_permute_invariants


def _case(N=37, k=3, E=7, seed=0):
    rng = np.random.default_rng(seed)
    experts = np.stack([rng.choice(E, k, replace=False) for _ in range(N)])
    counts, offsets, _, token_of, slot_pos = O.permute(experts, E)
    return experts, counts, offsets, token_of, slot_pos, E, k


def test_accepts_oracle_groupings():
    for seed, (N, k, E) in enumerate([(37, 3, 7), (1, 1, 1), (200, 8, 128), (64, 10, 512)]):
        check_permute_invariants(*_case(N, k, E, seed))


def test_accepts_dropped_ids():
    experts, counts, offsets, token_of, slot_pos, E, k = _case()
    bad = np.zeros(experts.size, bool)
    bad[[4, 17, 50]] = True
    ex = experts.reshape(-1).copy()
    ex[bad] = [-1, E, 99]
    c, o, _, t, s = O.permute(np.where(bad, E, ex).reshape(experts.shape), E + 1)   # bad ids: an extra expert past the end
    s = np.where(bad, -1, s)
    check_permute_invariants(ex, c[:E], o[:E + 1], t, s, E, k)


@pytest.mark.parametrize("plant", ["swap_rows", "offset", "count", "token", "unstable", "bad_id_kept"])
def test_rejects_planted_mistakes(plant):
    experts, counts, offsets, token_of, slot_pos, E, k = _case()
    counts, offsets, token_of, slot_pos = counts.copy(), offsets.copy(), token_of.copy(), slot_pos.copy()
    flat = experts.reshape(-1)
    if plant == "swap_rows":            # two assignments of different experts exchange rows
        a, b = 0, int(np.nonzero(flat != flat[0])[0][0])
        slot_pos[[a, b]] = slot_pos[[b, a]]
    elif plant == "offset":
        offsets[3] += 1
    elif plant == "count":
        counts[2] += 1
    elif plant == "token":
        token_of[5] = (token_of[5] + 1) % (flat.size // k)
    elif plant == "unstable":           # two rows of one expert out of assignment order
        e = flat[0]
        a, b = np.nonzero(flat == e)[0][:2]
        slot_pos[[a, b]] = slot_pos[[b, a]]
        token_of[slot_pos[a]], token_of[slot_pos[b]] = a // k, b // k
    elif plant == "bad_id_kept":        # an out-of-range id left holding a row
        experts = experts.copy()
        experts.reshape(-1)[0] = E
    with pytest.raises(AssertionError):
        check_permute_invariants(experts, counts, offsets, token_of, slot_pos, E, k)
