"""Compaction exactness on constructed keep masks (HIP path vs np.flatnonzero).

The log-biases are written, not computed, so the mask of every segment is
known: every entry dead or live, alternating, a single survivor first or
last, first or last entry dead, seeded coins, the first half dead (every
survivor moves), over lengths 0, 1, 255, 256, 257, 511, 512, 513 and long
segments whose look-back passes more than 64 predecessor chunks.  Kept-index
lists must equal np.flatnonzero of the mask, the moved K, V, log-bias and
key-gate rows must be bit-identical to their sources, and the new lengths
equal the popcounts (stable removal of evicted entries: paperlayer.ai
summary, section 4.2).  Both compaction workgroup sizes are covered (the
larger one is chosen for caches of more than 131072 slots), and so is the
compaction fused into the decode step, run with every decay term disabled
(the log-biases then stay as written).
"""

import math

import numpy as np
import pytest

from ua_inputs import MASK_PATTERNS, config, make_mask_cache, make_weights

pytestmark = pytest.mark.gpu

LOG_P = math.log(0.15)
SHORT = [0, 1, 255, 256, 257, 511, 512, 513]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_pruning_amd import load

    load()


def _segments(long_lens):
    """Every pattern at every short length, then the long segments."""
    lens, kinds = [], []
    for n in SHORT:
        for k in MASK_PATTERNS:
            lens.append(n)
            kinds.append(k)
    for n in long_lens:
        for k in ("front_dead", "first_dead", "random", "alt"):
            lens.append(n)
            kinds.append(k)
    return lens, kinds


def _layer(lens, kinds, d, bf16, seed, H_kv=1, terms=7):
    from kv_cache_pruning_amd.layer import layer_from_arrays

    S = len(lens)
    assert S % H_kv == 0
    B = S // H_kv
    c = make_mask_cache(lens, kinds, d, bf16, LOG_P, seed=seed, B=B)
    cfg = config("1b-decode", B=B, H_q=H_kv, H_kv=H_kv, d=d, D=64, bf16=bf16)
    w = make_weights(cfg, seed)
    return layer_from_arrays(B, H_kv, H_kv, d, 64, cfg.r, bf16, w, c, terms=terms), c


def _bits(t):
    """Raw bits of a device tensor as a numpy integer array."""
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def _check(layer, c, kept_dev, fused: bool):
    cache = layer.cache
    K1, V1, L1, G1 = (_bits(t) for t in (cache.K, cache.V, cache.logbias, cache.kgate))
    n1 = cache.seg_len.cpu().numpy()
    kb = kept_dev.cpu().numpy()
    K0 = _bits_host(c.K, layer.shape.bf16)
    V0 = _bits_host(c.V, layer.shape.bf16)
    L0, G0 = c.lam.view(np.int32), c.lk.view(np.int32)
    assert int(cache.status.item()) == 0
    for s in range(len(c.seg_len)):
        o, n0 = int(c.seg_off[s]), int(c.seg_len[s])
        keep = np.flatnonzero(c.lam[o : o + n0] >= np.float32(LOG_P))
        want = keep.size + (1 if fused else 0)
        assert n1[s] == want, f"seg {s}: length {n1[s]}, expected {want}"
        got = kb[o : o + keep.size]
        assert np.array_equal(got, keep), f"seg {s} (len {n0}): kept list differs"
        src = o + keep
        dst = slice(o, o + keep.size)
        assert np.array_equal(K1[dst], K0[src]), f"seg {s}: moved K rows differ"
        assert np.array_equal(V1[dst], V0[src]), f"seg {s}: moved V rows differ"
        assert np.array_equal(G1[dst], G0[src]), f"seg {s}: moved key gates differ"
        if not fused:  # the fused step stores every survivor's updated bias (unchanged here)
            assert np.array_equal(L1[dst], L0[src]), f"seg {s}: moved log-biases differ"
        else:
            assert np.array_equal(L1[dst], L0[src]), f"seg {s}: log-biases changed with no decay term"
            assert kb[o + keep.size] == n0, f"seg {s}: new entry's kept index"
            assert L1[o + keep.size] == 0, f"seg {s}: new entry's bias is not 0"


def _bits_host(a, bf16):
    if bf16:
        return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    return a.astype(np.float32).view(np.int32)


@pytest.mark.parametrize("d,bf16,long_lens", [
    (64, True, [20000]),          # 256-thread chunks of 256 entries; 79 chunks in the long segments
    (128, True, [9000]),          # 256-byte rows: chunks of 128 entries, 71 chunks
    (64, False, [9000]),          # fp32 rows (256 bytes)
    (64, True, [40000, 40000]),   # > 131072 slots: 512-thread chunks of 512 entries, 79 chunks
])
def test_compact_constructed_masks(d, bf16, long_lens):
    import torch

    lens, kinds = _segments(long_lens)
    layer, c = _layer(lens, kinds, d, bf16, seed=len(lens) + d)
    print(f"[compact masks] d={d} bf16={bf16} segments={len(lens)} slots={layer.cache.total_slots}", flush=True)
    kept = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
    layer.compact(LOG_P, kept)
    torch.cuda.synchronize()
    _check(layer, c, kept, fused=False)
    # a second call on the compacted cache keeps everything in place
    before = [_bits(t) for t in (layer.cache.K, layer.cache.V, layer.cache.logbias)]
    n_before = layer.cache.seg_len.cpu().numpy()
    kept.fill_(-1)
    layer.compact(LOG_P, kept)
    torch.cuda.synchronize()
    assert np.array_equal(layer.cache.seg_len.cpu().numpy(), n_before)
    kb = kept.cpu().numpy()
    for s, (o, n) in enumerate(zip(c.seg_off, n_before)):
        assert np.array_equal(kb[o : o + n], np.arange(n)), f"seg {s}: second call moved entries"
        for b0, t in zip(before, (layer.cache.K, layer.cache.V, layer.cache.logbias)):
            assert np.array_equal(_bits(t)[o : o + n], b0[o : o + n])


@pytest.mark.parametrize("d,long_lens", [(64, [20000]), (128, [9000])])
def test_fused_decode_constructed_masks(d, long_lens):
    """ua_decode_compact_step with every decay term off: the log-biases are
    not changed, so the survivors are exactly the constructed mask's, and the
    new entry lands right after them."""
    import torch

    lens, kinds = _segments(long_lens)
    lens, kinds = lens + [5] * (len(lens) % 2), kinds + ["alt"] * (len(lens) % 2)
    H_kv = 2
    layer, c = _layer(lens, kinds, d, True, seed=7 + d, H_kv=H_kv, terms=0)
    B = len(lens) // H_kv
    print(f"[fused masks] d={d} segments={len(lens)} slots={layer.cache.total_slots}", flush=True)
    rng = np.random.default_rng(d)
    from ua_inputs import bf16_exact

    q = bf16_exact(rng.standard_normal((B, H_kv, d)).astype(np.float32))
    k = bf16_exact(rng.standard_normal((B, H_kv, d)).astype(np.float32))
    v = bf16_exact(rng.standard_normal((B, H_kv, d)).astype(np.float32))
    x = bf16_exact(rng.standard_normal((B, 64)).astype(np.float32))
    kept = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
    layer.decode_compact_step(q, k, v, x, LOG_P, kept=kept)
    torch.cuda.synchronize()
    _check(layer, c, kept, fused=True)
