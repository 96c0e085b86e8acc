"""GPU decode parity for every (head dim D, channels per code c, code bits) shape
the library compiles, with bf16 queries and output, against the fp64 oracle.

Each shape runs a ragged batch of 16 requests on two KV heads (eight duos per
head: the workgroup-shared RoPE rows) and one of 6 requests (three duos: rows
per wave), both with 64-token pages and caches of random codes.  Same bars as
the other decode tests: outputs within 2e-3 max-abs plus half a bf16 ulp of
the reference, lse within 1e-4.
"""
import numpy as np
import pytest

import synth
from gpu_util import GpuLayer, compare, ref_decode

pytestmark = pytest.mark.gpu

SHAPES = [(128, 4, 8), (128, 8, 8), (128, 2, 8), (128, 4, 4), (128, 8, 4), (128, 2, 4),
          (64, 2, 4), (64, 4, 4), (64, 2, 8), (64, 4, 8), (64, 8, 8)]


@pytest.mark.parametrize("D,c,bits", SHAPES)
@pytest.mark.parametrize("lens", [
    [700, 1, 64, 65, 300, 0, 129, 511, 16, 17, 640, 200, 33, 450, 128, 2],
    [513, 64, 9, 700, 1, 300],
])
def test_decode_shape(D, c, bits, lens):
    cfg = synth.config_by_name("layer1p4b").replace(D=D, c=c, bits=bits, H_kv=2, H_q=2, n_calib=300)
    if cfg.G == 8:
        cfg = cfg.replace(x_dtype="f32")    # 8-element coupled vectors are coded from fp32 data only
    lens = np.array(lens)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 71 + D + c + bits)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    for t in (1, 4):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, cache, bt, lens)
        ref = ref_decode(cfg, t, q, cache, bt, lens, cb)
        err, ratio = compare(cfg, o, lse, ref, lens)
        print(f"D={D} c={c} bits={bits} B={len(lens)} t={t}: max err {err:.2e} (bound ratio {ratio:.2f})",
              flush=True)
        assert ratio <= 1.0
