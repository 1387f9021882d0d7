"""Checks of the seeded input generators (structure only; no attention math)."""
import numpy as np
import pytest

from workloads import SPECS, Spec, make_host_batch, make_layout


@pytest.mark.parametrize("name", ["tiny_decode", "tiny_extend", "decode_bf16", "extend_bf16",
                                  "long_decode_bf16", "decode_fp8"])
def test_layouts_follow_their_spec(name):
    spec = SPECS[name]
    lay, _ = make_layout(spec, 0)
    P = spec.page_size
    assert lay.seq_lens.shape == (spec.batch,)
    assert np.all(lay.seq_lens == lay.prefix_lens + lay.new_lens)
    for b in range(spec.batch):
        L = int(lay.seq_lens[b])
        row = lay.req_to_token[b, :L].astype(np.int64)
        assert np.all(row >= 0) and np.all(lay.req_to_token[b, L:] == -1)
        j = np.arange(L)
        # slots inside a page are consecutive; page starts are page-aligned
        assert np.all(row == row[j - j % P] + j % P)
        assert np.all(row[j % P == 0] % P == 0)
    used = lay.req_to_token[lay.req_to_token >= 0]
    assert len(np.unique(used)) == len(used)  # no two positions share a slot
    assert used.max() < lay.pool_slots
    if isinstance(spec.prefix, tuple):
        lo, hi = spec.prefix
        assert lay.prefix_lens.min() >= lo and lay.prefix_lens.max() <= hi
    if spec.pool == "2x":
        assert lay.pool_slots == 2 * int(((lay.seq_lens + P - 1) // P).sum()) * P


def test_same_seed_same_batch_and_poisoning():
    spec = Spec("w", "extend", 3, 4, 2, 16, 4, (0, 20), (1, 9))
    a = make_host_batch(spec, 5)
    b = make_host_batch(spec, 5)
    c = make_host_batch(spec, 6)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.layout.req_to_token, b.layout.req_to_token)
    assert not np.array_equal(a.q, c.q)
    used = a.layout.slot_owner >= 0
    assert np.all(np.isnan(a.k_pool[~used])) and np.all(np.isfinite(a.k_pool[used]))
    # bf16 values are exactly representable in bfloat16
    bits = a.q.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_tiny_tables_are_a_permutation_of_256_slots():
    lay, _ = make_layout(SPECS["tiny_extend"], 0)
    assert lay.pool_slots == 256
    assert list(lay.seq_lens) == [42, 112] and list(lay.cu_seqlens_q) == [0, 5, 17]
