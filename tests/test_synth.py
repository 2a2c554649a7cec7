"""The seeded generators are deterministic, counter-based (any record regenerates
on its own) and have the requested statistics."""
import numpy as np

import synth
from synth.configs import ALL


def test_record_regenerates_alone():
    pool, ts = synth.pool_numpy(7, 2, 8, 64, 128, synth.FMT_NVFP4, nthreads=3)
    for flat in (0, 5, 13):
        rec, t = synth.record(7, 8, flat // 8, flat % 8, 64, 128, synth.FMT_NVFP4)
        assert np.array_equal(rec, pool[flat]) and np.array_equal(t, ts[flat])
    assert not np.array_equal(pool[0], pool[1])


def test_weight_statistics():
    w = synth.weights_f32(1, 8, 0, 0, 0, 512, 256)
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
    x = synth.activations(1, 0, 0, 4, 2048).reshape(-1)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.std() - 1.0) < 0.05


def test_trace_zipf_overlap():
    # adjacent tokens share about a quarter of a layer's experts (Edge0 summary, "전제와 한계")
    E, K = 256, 8
    lg = synth.trace_logits(3, 0, E, 1.1, 0, 400)
    sets = synth.gumbel_topk_sets(lg, K)
    ov = np.mean([len(set(sets[t]) & set(sets[t + 1])) / K for t in range(399)])
    assert 0.15 < ov < 0.35


def test_spec_ids_keep_rate():
    E, K = 512, 10
    lg = synth.trace_logits(5, 1, E, 1.2, 0, 300)
    truth = synth.gumbel_topk_sets(lg, K)
    kept = []
    for t in range(300):
        p = synth.spec_ids(5, 1, E, 1.2, t, truth[t], 0.65)
        assert len(set(p)) == K and all(0 <= v < E for v in p)
        kept.append(len(set(p) & set(truth[t])) / K)
    assert 0.58 < np.mean(kept) < 0.72


def test_configs_shapes():
    for w in ALL:
        assert w.H % 64 == 0 and w.I % 64 == 0 and w.K <= w.E
