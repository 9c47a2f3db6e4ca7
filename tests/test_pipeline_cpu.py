"""Host logic of the layer pipeline that needs no GPU: the GDN layer's slot
bookkeeping under eager and deferred rollback (the slots are CPU tensors;
rollback only selects one, through the library's host-only sdv_gdn_rollback)."""

import pytest
import torch

from speculative_decode_verification_amd import pipeline


def _layer(k=4):
    layer = pipeline.GdnLayer(torch.zeros((2, 8, 8)), k)
    layer.snap_ids = [i for i in range(k + 1) if i != layer.live][:k]  # as a verify call leaves them
    return layer


def test_rollback_selects_the_snapshot_slot():
    layer = _layer()
    assert layer.rollback(3) is layer.slots[3]
    assert layer.live == 3 and layer.snap_ids is None
    layer.snap_ids = [0, 1, 2, 4]
    layer.rollback(0)  # nothing accepted: the live slot stays
    assert layer.live == 3


def test_deferred_rollback_applies_once_at_the_next_use():
    layer = _layer()
    layer.rollback_later(2)
    assert layer.live == 0 and layer._pending == 2
    with pytest.raises(RuntimeError, match="pending"):
        layer.rollback_later(1)
    with pytest.raises(RuntimeError, match="pending"):
        layer.rollback(1)
    assert layer.state is layer.slots[2]  # reading the state applies it
    assert layer._pending is None and layer.live == 2
    layer.apply_rollback()  # nothing pending: no change
    assert layer.live == 2


def test_deferred_rollback_checks_the_prefix_first():
    from speculative_decode_verification_amd import ops
    layer = _layer(k=4)
    with pytest.raises(ops.SdvError):
        layer.rollback_later(5)
    assert layer._pending is None
