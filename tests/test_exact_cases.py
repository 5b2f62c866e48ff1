"""The exact GEMM cases (tests/test_gpu_exact.py) can see the mistakes they
are there for (CPU only, oracle arithmetic): with one-hot A rows, taking the
scale of the neighbouring K block of A or of B, or B's element one position
along K, changes the oracle's result on (nearly) every output, so a GPU
result equal to the unshifted reference bit for bit rules those slips out."""
import numpy as np

import oracle
from test_gpu_exact import one_hot_a, random_b


def _ref(qa, sa, qb, sb):
    return oracle.gemm(qa, sa, qb, sb, oracle.BKIND_ROW, want_bound=False)[0]


def test_one_hot_outputs_are_exact_nonzero_products():
    qa, sa = one_hot_a(64, 2048, 1)
    qb, sb = random_b(96, 2048, 2)
    ref = _ref(qa, sa, qb, sb)
    assert (ref != 0).all() and np.isfinite(ref).all()
    f32 = ref.astype(np.float32)
    assert (f32.astype(np.float64) == ref).all()
    assert ((f32.view(np.uint32) & 0xFFFF) == 0).all()     # BF16 holds every output exactly
    assert (np.count_nonzero(qa, axis=1) == 1).all()
    assert len(np.unique(np.argmax(qa != 0, axis=1) // 32)) == 64   # one K block per row


def test_neighbouring_scale_or_position_changes_the_outputs():
    qa, sa = one_hot_a(64, 2048, 3)
    qb, sb = random_b(96, 2048, 4)
    ref = _ref(qa, sa, qb, sb)
    # A's scale of the previous block: neighbouring blocks always differ
    assert (_ref(qa, np.roll(sa, 1, axis=1), qb, sb) != ref).all()
    # B's scale of the previous block: random bytes, equal 1 time in 15
    assert (_ref(qa, sa, qb, np.roll(sb, 1, axis=1)) != ref).mean() > 0.85
    # B's element one position along K
    assert (_ref(qa, sa, np.roll(qb, 1, axis=1), sb) != ref).mean() > 0.95
    # a whole K step (128 elements) late
    assert (_ref(qa, sa, np.roll(qb, 128, axis=1), np.roll(sb, 4, axis=1)) != ref).mean() > 0.95
