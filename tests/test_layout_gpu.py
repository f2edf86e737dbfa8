"""Layout builder on the GPU vs the oracle: bit-exact document ids, tile
classes, per-q-tile lists, q-tile order and status word."""
import numpy as np
import pytest

import oracle
from packed_masked_attention_amd import synth
from tests.helpers import say

pytestmark = pytest.mark.gpu


def _check(lay, tm, tn):
    from packed_masked_attention_amd import binding as B
    dl = B.pma_layout_build(lay, tile_m=tm, tile_n=tn)
    bits, row = B.pma_layout_read_status(dl)
    assert (bits, row) == oracle.layout_status(lay)
    got = B.layout_arrays(dl)
    cls, count, lst, order = oracle.layout_tiles(lay["tags"], tm, tn)
    assert np.array_equal(got["doc"], oracle.layout_doc(lay["tags"]))
    assert np.array_equal(got["cls"], cls)
    assert np.array_equal(got["count"], count)
    assert np.array_equal(got["list"], lst)
    assert np.array_equal(got["order"], order)


@pytest.mark.parametrize("tm,tn", [(64, 64), (128, 64), (256, 64), (128, 128), (256, 256)])
@pytest.mark.parametrize("seed", range(4))
def test_random_layouts_bit_exact(seed, tm, tn):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 3000))
    lay = synth.random_layout(rng, L, pad_frac=[0.0, 0.07, 0.5, 1.0][seed], T=3,
                              scattered=seed % 2 == 0)
    say(f"layout seed={seed} L={L} tiles={tm}x{tn}")
    _check(lay, tm, tn)


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_layouts_bit_exact(name):
    from packed_masked_attention_amd import binding as B
    lay = synth.make_layout(synth.workload(name))
    tm, tn = B.pma_attention_tiles()
    say(f"layout {name} tiles={tm}x{tn}")
    _check(lay, tm, tn)
    if name == "masked_L16384":
        _check(lay, 128, 128)


def test_bad_layouts_status_bits():
    from packed_masked_attention_amd import binding as B
    base = synth.layout_from_counts(40, (2, 5, 7), 30, 20, T=2)

    def run(fn):
        lay = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
        fn(lay)
        dl = B.pma_layout_build(lay)
        got = B.pma_layout_read_status(dl)
        assert got == oracle.layout_status(lay), fn.__name__
        return got

    assert run(lambda l: None) == (0, -1)

    def bad_tag(l): l["tags"][77] = 3
    def bad_ts(l): l["ts_idx"][5] = -1
    def bad_pos(l): l["pos"][100, 1] = -(1 << 24)
    def unsorted(l): l["video_idx"][[3, 4]] = l["video_idx"][[4, 3]]
    def oob(l): l["text_idx"][0] = 10 ** 6
    def wrong_tag(l): l["audio_idx"][0] = 0
    def short(l): l["text_idx"] = l["text_idx"][1:].copy()
    for fn in (bad_tag, bad_ts, bad_pos, unsorted, oob, wrong_tag, short):
        assert run(fn)[0] != 0, fn.__name__
