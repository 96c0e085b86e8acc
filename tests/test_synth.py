"""The seeded input generators: shapes, dtypes, seeds and the loop-axis statistics."""
import numpy as np

import synth


def test_configs_shapes():
    tiny = synth.config_by_name("C0")
    assert (tiny.G, tiny.K, tiny.n_groups, tiny.row_bytes) == (8, 16, 32, 16)
    c1 = synth.config_by_name("layer1p4b")
    assert (c1.G, c1.K, c1.row_bytes) == (16, 256, 32)
    c3 = synth.config_by_name("C3")
    assert (c3.G, c3.row_bytes, c3.group_size) == (32, 16, 4)
    c4 = synth.config_by_name("C4")
    assert c4.n_blocks == 8 and len(c4.rhos) == 31
    assert abs(c4.rhos[0] - 0.7) < 1e-12 and abs(c4.rhos[-1] - 0.95) < 1e-12


def test_loop_correlation_follows_rho():
    rng = np.random.default_rng(0)
    x = synth.loop_correlated(rng, 4, (200000,), (0.7, 0.8, 0.9))
    for t, r in enumerate((0.7, 0.8, 0.9)):
        emp = np.corrcoef(x[t], x[t + 1])[0, 1]
        assert abs(emp - r) < 0.01
        assert abs(x[t + 1].std() - 1.0) < 0.01


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.3e-5, 65504.0], dtype=np.float32)
    r = synth.round_to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0078125)
    u = r.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)


def test_kv_is_deterministic_and_rounded():
    cfg = synth.config_by_name("C1")
    a = synth.make_kv(cfg, 8)
    b = synth.make_kv(cfg, 8)
    np.testing.assert_array_equal(a[0], b[0])
    assert a[0].shape == (4, 8, 16, 128)
    assert np.all(a[0].view(np.uint32) & 0xFFFF == 0)
    sub = synth.make_kv(cfg, 8, heads=[5])
    np.testing.assert_array_equal(sub[1][:, :, 0], a[1][:, :, 5])


def test_codebooks_distinct_fp16():
    cfg = synth.config_by_name("C0")
    cb = synth.make_codebooks(cfg)
    assert cb.shape == (1, 1, 2, 16, 8) and cb.dtype == np.float16
    for kv in range(2):
        assert len(np.unique(cb[0, 0, kv].view(np.uint16), axis=0)) == 16


def test_ragged_lengths_and_block_table():
    cfg = synth.config_by_name("C3")
    lens = synth.make_seq_lens(cfg)
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 16384
    bt, n = synth.make_block_table(cfg, lens)
    used = np.concatenate([bt[b, :(l + 63) // 64] for b, l in enumerate(lens)])
    assert sorted(used.tolist()) == list(range(n))


def test_window_split_and_pages():
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1000, 1003, 5, 0, 72, 71])
    ns, ws, pt, npg = synth.make_window(cfg, lens, 8, 64)
    np.testing.assert_array_equal(ns, [8, 8, 5, 0, 8, 8])
    np.testing.assert_array_equal(ws, [936, 936, 5, 0, 8, 8])
    # the window holds n_recent to n_recent + 7 tokens where the sink leaves room
    assert all(64 <= l - w <= 71 for l, w in zip(lens[:2], ws[:2]))
    nbf = ns + lens - ws
    used = np.concatenate([pt[b, :(n + 7) // 8] for b, n in enumerate(nbf)])
    assert len(np.unique(used)) == len(used) == npg      # every physical page used once
    pages = synth.fill_window_pages(npg, pt, ns, ws, lens,
                                    lambda b, pos: np.broadcast_to((b * 10000 + pos)[:, None, None], (len(pos), 2, 4)),
                                    lambda b, pos: -np.broadcast_to((b * 10000 + pos)[:, None, None], (len(pos), 2, 4)),
                                    2, 4)
    for b in range(len(lens)):
        pos = synth.window_positions(int(ns[b]), int(ws[b]), int(lens[b]))
        for u, p in enumerate(pos):
            assert pages[pt[b, u // 8], 1, 0, u % 8, 3] == b * 10000 + p
            assert pages[pt[b, u // 8], 0, 1, u % 8, 0] == -(b * 10000 + p)


def test_per_group_codebooks_hold_their_groups_vectors():
    cfg = synth.config_by_name("tiny").replace(bits=8, n_calib=300)
    cb = synth.make_codebooks_per_group(cfg)
    assert cb.shape == (cfg.n_blocks, cfg.H_kv, 2, cfg.n_groups, cfg.K, cfg.G) and cb.dtype == np.float16
    for g in (0, cfg.n_groups - 1):
        e = cb[0, 0, 0, g].view(np.uint16)
        assert len(np.unique(e, axis=0)) == cfg.K
    assert not np.array_equal(cb[0, 0, 0, 0], cb[0, 0, 0, 1])
