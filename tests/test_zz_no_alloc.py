"""The decode entry point that allocates nothing (loopvq_decode_attn_noalloc)
against loopvq_decode_attn on the same inputs.

Both run the same kernels under the same split plan, so outputs and lse must
agree bit for bit; the second of two calls in a row is a smaller batch (the
fixed scratch keeps the first call's partials, which the second must not
read), and it is also held to the oracle's bar [LoopVQ paper, section
"System implementation", attention].
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import GpuLayer, compare, io_tensor, ref_decode, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _case(cfg, lens, seed):
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, seed)
    return bt, cache


def test_noalloc_decode_equals_workspace_decode():
    cfg = synth.config_by_name("layer1p4b")
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    big = np.array([3000, 1, 2048, 700, 0, 1500, 64, 4096])
    small = np.array([129, 40])
    layer = GpuLayer(cfg, cb, int(big.max()))
    for step, (lens, seed) in enumerate(((big, 11), (small, 12))):
        bt, cache = _case(cfg, lens, seed)
        t = 2 + step
        q = synth.make_queries(cfg, len(lens), t=t)
        print(f"noalloc call {step}: B={len(lens)} lens={lens.tolist()} t={t}", flush=True)
        q_d, cache_d = io_tensor(cfg, q), to_dev(cache)
        bt_d, lens_d = to_dev(bt.astype(np.int32)), to_dev(lens.astype(np.int32))
        msl = int(lens.max())
        out_ref = torch.empty((len(lens), cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
        lse_ref = torch.empty((len(lens), cfg.H_q), dtype=torch.float32, device="cuda")
        lv.loopvq_decode_attn(layer.dims, t, q_d, cache_d, layer.slices, layer.rope, bt_d, lens_d, msl,
                              out=out_ref, lse=lse_ref, max_pos=layer.max_pos)
        out = torch.full_like(out_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        lv.loopvq_decode_attn_noalloc(layer.dims, t, q_d, cache_d, layer.slices, layer.rope, bt_d, lens_d, msl,
                                      out, lse, max_pos=layer.max_pos)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
        if step == 1:
            got = out.float().cpu().numpy().astype(np.float64)
            ref = ref_decode(cfg, t, q, cache, bt, lens, cb, heads=[0, 9, 15])
            err, ratio = compare(cfg, got, lse.cpu().numpy().astype(np.float64), ref, lens)
            print(f"noalloc second call vs oracle: max err {err:.2e} (bound ratio {ratio:.2f})", flush=True)
            assert ratio <= 1.0


def test_noalloc_decode_rejects_a_batch_beyond_its_scratch():
    cfg = synth.config_by_name("layer1p4b")
    dims = GpuLayer(cfg, synth.make_codebooks(cfg.replace(n_calib=300)), 16).dims
    B, n = 256, 65536
    assert lv.loopvq_decode_workspace_bytes(dims, B, n) > lv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    cache = torch.zeros((1, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    slices = torch.zeros((cfg.T, cfg.H_kv, 2, cfg.K, cfg.c), dtype=torch.float16, device="cuda")
    rope = torch.zeros(int(lv.lib().loopvq_rope_table_floats(n, cfg.D)), dtype=torch.float32, device="cuda")
    bt = torch.zeros((B, n // cfg.page_size), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), n, dtype=torch.int32, device="cuda")
    with pytest.raises(lv.LoopVQError) as e:
        lv.loopvq_decode_attn_noalloc(dims, 1, q, cache, slices, rope, bt, lens, n, out, max_pos=n)
    assert e.value.status == -5
