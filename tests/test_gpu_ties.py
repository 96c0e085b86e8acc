"""GPU encoder on codebooks with exact ties: the lowest index must win.

The nearest-entry rule [LoopVQ paper, section "Preliminaries", eq. (2)]
returns the lowest index among entries at the same distance.  Random
codebooks almost never hold two equal entries, so these tests plant identical
fp16 entries at chosen indices and feed vectors that land on them (some equal
to the planted entry, distance 0).  Identical entries give identical scores on
any evaluation, so the lowest index is the only correct answer and the GPU
code must equal the oracle's exactly - no near-tie allowance.  The planted
index sets put the copies

  * in one 32-entry tile, in both lane halves of a vector (rows 8q + 4*hf + s
    with hf = 0 and 1) and in one lane (adjacent rows);
  * in different tiles, in the same lane (rows r and r + 32) and in other
    lanes, with the lowest copy in either half;
  * with 4-bit codes (one 16-row tile);

and run through every encoder instance: bf16 and fp32 input, c = 2, 4, 8,
16, 32 and 64 groups per token (a unit of 32 vectors spans two tokens, one
token or half a token), eight blocks, one codebook per channel group, bf16
window pages, TaSQ keys.

A vector is compared exactly unless two *distinct* entries lie within the
oracle's near-tie band of each other (then it is left out and counted).  The
encoder's near-tie counter must count every exact tie and agree with the
oracle's band to within fp32 rounding of the scores.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuLayer, dims_for, to_dev, x_tensor

pytestmark = pytest.mark.gpu
tq = oracle.tasq_ref

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401

# index sets that receive one identical entry (disjoint within a codebook size)
TIE_SETS = {
    256: ((0, 4),                 # tile 0, q = 0, s = 0, lane halves 0 and 1
          (8, 9, 13),             # tile 0: same lane (rows 8, 9) and the other half (13)
          (5, 37, 200),           # tiles 0, 1, 6; the lowest copy in half 1
          (64, 100, 255),         # tiles 2, 3, 7; the lowest copy in half 0
          (17, 18),               # adjacent rows of one lane
          (3, 35),                # one lane, tiles 0 and 1 (strict tile compare)
          (6, 40),                # lowest copy in half 1, the other in half 0 of a later tile
          (12, 66, 130, 250),     # four tiles
          (31, 224),              # last row of tile 0, first row of tile 7
          (127, 128)),            # across the tile 3 / tile 4 boundary
    16: ((1, 5),                  # lane halves 0 and 1
         (2, 10, 14),             # q = 0 and 1, both halves
         (7, 8),                  # half 1 below half 0
         (12, 15)),               # one lane
}


def _note(msg):
    print(msg, flush=True)


def _plant(E, sets, z, rng):
    """Copy one value into every index of each set: even sets get a data vector
    (fp16), odd sets the entry already at the set's highest index."""
    E = E.copy()
    for k, s in enumerate(sets):
        v = z[rng.integers(len(z))].astype(np.float16) if k % 2 == 0 else E[max(s)].copy()
        E[list(s)] = v
    return E


def tied_codebooks(cfg, cb, xk, xv, seed):
    """cb [n_blocks][H][2][K][G] (or [..][D/c][K][G]) with TIE_SETS planted in every codebook."""
    rng = np.random.default_rng(seed)
    cb = cb.copy()
    sets = TIE_SETS[cfg.K]
    for beta in range(cfg.n_blocks):
        for h in range(cfg.H_kv):
            for kv, x in enumerate((xk, xv)):
                z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, beta)
                if cb.ndim == 6:
                    for g in range(cfg.n_groups):
                        cb[beta, h, kv, g] = _plant(cb[beta, h, kv, g], sets, z[:, g, :], rng)
                else:
                    cb[beta, h, kv] = _plant(cb[beta, h, kv], sets, z.reshape(-1, cfg.G), rng)
    return cb


class Tally:
    """Exact comparison against the oracle's lowest index, plus near-tie bounds."""

    def __init__(self):
        self.checked = self.exact = self.mism = self.left_out = 0
        self.lo = self.hi = 0          # oracle near-tie counts at 1/4 and 4 times the band

    def add(self, z, E, got):
        E64 = E.astype(np.float64)
        res = oracle.nearest_entry(z, E64, method="gemm")
        _, first, inv, counts = np.unique(E.view(np.uint16), axis=0, return_index=True, return_inverse=True,
                                          return_counts=True)
        inv = inv.reshape(-1)
        distinct = E64[np.sort(first)]
        clean = ~oracle.nearest_entry(z, distinct, method="gemm").near_tie
        # the oracle's index is the first copy of its entry (the rule the GPU must follow)
        assert np.array_equal(first[inv[res.idx]][clean], res.idx[clean])
        dup = counts[inv[res.idx]] > 1
        self.checked += int(clean.sum())
        self.exact += int((clean & dup).sum())
        self.mism += int((clean & (np.asarray(got) != res.idx)).sum())
        self.left_out += int((~clean).sum())
        gap = res.d2 - res.d1
        self.lo += int((gap < 0.25 * res.band).sum())
        self.hi += int((gap < 4.0 * res.band).sum())

    def check(self, what, gpu_ties=None):
        _note(f"{what}: {self.checked} vectors compared exactly, {self.exact} of them exact ties, "
              f"{self.mism} mismatches, {self.left_out} left out (distinct entries in the band); "
              f"near-ties oracle [{self.lo}, {self.hi}], GPU {gpu_ties}")
        assert self.exact >= 100, "too few exact ties exercised"
        assert self.mism == 0
        if gpu_ties is not None:
            assert self.lo <= gpu_ties <= self.hi


def _rows_codes(cfg, cache_blk, slots, h, kv):
    P = cfg.page_size
    rows = cache_blk[slots // P, h, kv, slots % P, :]
    return oracle.slots_to_groups(oracle.unpack_rows(rows, cfg.bits, cfg.n_groups))


def _encode_dense(cfg, dims, cb, xk, xv, slots, npg, count_ties=True):
    layer = GpuLayer(cfg, cb, 16, dims=dims)
    cache = torch.zeros((cfg.n_blocks, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8,
                        device="cuda")
    ties = torch.zeros(1, dtype=torch.int32, device="cuda") if count_ties else None
    lv.loopvq_encode(dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq,
                     to_dev(np.asarray(slots, np.int32)), cache, n_blocks=cfg.n_blocks,
                     block_stride_bytes=cache[0].numel(), near_tie_count=ties)
    plain = torch.zeros_like(cache)
    lv.loopvq_encode(dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq,
                     to_dev(np.asarray(slots, np.int32)), plain, n_blocks=cfg.n_blocks,
                     block_stride_bytes=plain[0].numel())
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    # counting near-ties must not change a single code
    assert np.array_equal(got, plain.cpu().numpy())
    return got, (None if ties is None else int(ties.item()))


@pytest.mark.parametrize("name,over,n_tok", [
    ("layer1p4b", dict(H_kv=2, H_q=2), 300),           # bf16, c = 4, G = 16, 8-bit
    ("layer1p4b", dict(H_kv=2, H_q=2, c=2, Tc=8, T=8, rhos=(0.8,) * 7), 300),   # 64 groups per token
    ("gqa_ragged", dict(H_kv=2, H_q=8), 200),          # bf16, c = 8, G = 32
    ("tiny", dict(), 256),                             # fp32, c = 2, 4-bit (one 16-row tile)
    ("tiny", dict(bits=8), 256),                       # fp32, G = 8, 8-bit
    ("deeploop", dict(H_kv=1, H_q=1), 96),             # eight blocks with their own codebooks
])
def test_exact_ties_take_the_lowest_index(name, over, n_tok):
    cfg = synth.config_by_name(name).replace(n_calib=400, **over)
    xk, xv = synth.make_kv(cfg, n_tok, seed=cfg.index + 130)
    cb = tied_codebooks(cfg, synth.make_codebooks(cfg), xk, xv, seed=cfg.index + 131)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size).astype(np.int64)
    _note(f"{name} {over}: dense encode with planted ties, n_tok={n_tok}")
    got, gpu_ties = _encode_dense(cfg, dims_for(cfg), cb, xk, xv, slots, npg)
    tally = Tally()
    for beta in range(cfg.n_blocks):
        for h in range(cfg.H_kv):
            for kv, x in enumerate((xk, xv)):
                z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, beta).reshape(-1, cfg.G)
                tally.add(z, cb[beta, h, kv], _rows_codes(cfg, got[beta], slots, h, kv).reshape(-1))
    tally.check(f"{name} {over}", gpu_ties)


def test_exact_ties_per_group_codebooks():
    cfg = synth.config_by_name("layer1p4b").replace(n_calib=400, H_kv=2, H_q=2)
    n_tok = 160
    xk, xv = synth.make_kv(cfg, n_tok, seed=140)
    cb = tied_codebooks(cfg, synth.make_codebooks_per_group(cfg), xk, xv, seed=141)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size).astype(np.int64)
    _note("per-group encode with planted ties")
    got, gpu_ties = _encode_dense(cfg, dims_for(cfg, per_group=1), cb, xk, xv, slots, npg)
    tally = Tally()
    for h in range(cfg.H_kv):
        for kv, x in enumerate((xk, xv)):
            z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, 0)
            codes = _rows_codes(cfg, got[0], slots, h, kv)
            for g in range(cfg.n_groups):
                tally.add(z[:, g, :], cb[0, h, kv, g], codes[:, g])
    tally.check("per-group", gpu_ties)


def test_exact_ties_window_pages():
    cfg = synth.config_by_name("layer1p4b").replace(n_calib=400, H_kv=2, H_q=2)
    n_tok = 200
    xk, xv = synth.make_kv(cfg, n_tok, seed=150)
    cb = tied_codebooks(cfg, synth.make_codebooks(cfg), xk, xv, seed=151)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size).astype(np.int64)
    layer = GpuLayer(cfg, cb, 16)
    rng = np.random.default_rng(152)
    n_pages = (n_tok + 7) // 8 + 2
    src = rng.permutation(n_pages * 8)[:n_tok].astype(np.int32)
    pools = np.zeros((cfg.T, n_pages, cfg.H_kv, 2, 8, cfg.D), np.float32)
    pools[:, src // 8, :, 0, src % 8, :] = np.transpose(xk, (1, 0, 2, 3))
    pools[:, src // 8, :, 1, src % 8, :] = np.transpose(xv, (1, 0, 2, 3))
    cache = torch.zeros((1, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    _note("window-page encode with planted ties")
    lv.loopvq_encode_pages(layer.dims, to_dev(pools, torch.bfloat16), to_dev(src), layer.cb, layer.hsq,
                           to_dev(slots.astype(np.int32)), cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    tally = Tally()
    for h in range(cfg.H_kv):
        for kv, x in enumerate((xk, xv)):
            z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)
            tally.add(z, cb[0, h, kv], _rows_codes(cfg, got[0], slots, h, kv).reshape(-1))
    tally.check("window pages")


def test_exact_ties_tasq_keys():
    # TaSQ keys are coded from u = P(w k / sigma) by the fp32 encoder instance;
    # ties are planted in the codebooks of u (and of the values)
    cfg = synth.config_by_name("layer1p4b").replace(n_calib=400, H_kv=2, H_q=2)
    n_tok = 200
    xk, xv = synth.make_kv(cfg, n_tok, seed=160)
    w, perm = synth.make_tasq(cfg)
    u, s16 = tq.tasq_transform(xk, w, perm, cfg.Tc)
    ck, cv = synth.make_kv(cfg, cfg.n_calib, seed=161)
    cu, _ = tq.tasq_transform(ck, w, perm, cfg.Tc)
    cb = tied_codebooks(cfg, synth.codebooks_from_vectors(cfg, cu, cv, seed=162), u, xv, seed=163)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size).astype(np.int64)
    layer = GpuLayer(cfg, cb, 16)
    sigma = torch.zeros((cfg.T, npg * cfg.page_size), dtype=torch.float16, device="cuda")
    cache = torch.zeros((1, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    _note("TaSQ encode with planted ties")
    lv.loopvq_encode_tasq(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), to_dev(w), to_dev(perm), sigma,
                          layer.cb, layer.hsq, to_dev(slots.astype(np.int32)), cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    # tokens whose sigma sits at an fp16 rounding midpoint may take the other
    # neighbour on the GPU (their u then differs); they stay out of the key check
    sig_gpu = sigma.cpu().numpy()[:, slots]
    same_sigma = np.all(sig_gpu == s16, axis=0)
    tally = Tally()
    for h in range(cfg.H_kv):
        for kv, x in enumerate((u, xv)):
            z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, 0)
            codes = _rows_codes(cfg, got[0], slots, h, kv)
            keep = same_sigma if kv == 0 else np.ones(n_tok, bool)
            tally.add(z[keep].reshape(-1, cfg.G), cb[0, h, kv], codes[keep].reshape(-1))
    tally.check("TaSQ keys and values")
