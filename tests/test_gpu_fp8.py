"""GPU parity of the FP8 KV rows: the quantize step (``ds4attn_quantize_fp8``)
bit-exact against ``oracle.fp8.quantize_rows``, and the attention on E4M3 rows
with per-row scales against the float64 oracle run on the dequantized rows
(``oracle.fp8.dequantize_rows``), within the attention tolerance (max-abs 1e-2,
mean-abs 1e-3).

Covered: the quantizer on float16 and float32 rows of every supported head dim,
rows of zeros, negative zeros, tiny and huge magnitudes, constant rows, strided
rows; attention on the decode workloads with FP8 rows at full size (ring
window, ratio-128 with a partly valid tail, ratio-4 indexed), the ratio-4
prefill chunk in full, heads of very different query magnitudes (the scores'
E4M3 query terms), V rows of tiny, huge and block-to-block changing scales (the
V scales folded into the weights under a running power of two), general ragged
cases through both kernels
(validity masks whose hidden rows hold NaN codes and NaN scales, windows, index
lists with unused entries, two regions), and the chain quantize -> attention.
"""

import dataclasses
import zlib

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl
from tests.parity_util import compare as _compare

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()  # fail loudly if the HIP library is missing


def _oracle_problem(w) -> ref.Problem:
    """The oracle's view of an FP8 workload: rows dequantized in float64 (logical ring order)."""

    def region(r):
        if r is None:
            return None
        k, v, valid = r.logical()
        ks, vs = r.logical_scales()
        return ref.Region(ofp8.dequantize_rows(k.numpy(), ks.numpy()),
                          ofp8.dequantize_rows(v.numpy(), vs.numpy()), int(r.n_rows),
                          None if valid is None else valid.numpy())

    idx = None if w.r1_index is None else w.r1_index.numpy()
    return ref.Problem(q=w.q.numpy(), scale=float(w.scale), r0=region(w.r0), window=int(w.window),
                       q_pos0=int(w.q_pos0), k_pos0=int(w.k_pos0), r1=region(w.r1), r1_index=idx)


_FULL = {}


def _oracle_full(name):
    """The oracle over every token of a named FP8 workload, computed once."""
    if name not in _FULL:
        _FULL[name] = ref.attention(_oracle_problem(wl.named(name)))
    return _FULL[name]


def _run(w, entry, bq):
    dp = pipeline.to_device(w, DEV)
    out = pipeline.step(dp, entry, bq, splits=1)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


# --------------------------------------------------------------------------- quantize

def _quant_rows(seed, b, n, d, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(b, n, d, generator=g) * torch.exp2(torch.randint(-12, 12, (b, n, 1), generator=g).float())
    x[0, 0] = 0.0
    if n > 1:
        x[0, 1] = -0.0
    if n > 2:
        x[0, 2] = 3.0                                  # constant row
    if n > 3:
        x[0, 3] *= 1e-6                                # tiny
    if n > 4 and dtype == torch.float32:
        x[0, 4] *= 1e25                                # huge (float32 only)
    if n > 5:
        x[0, 5, ::3] = -0.0                            # signed zeros inside a row
    if n > 7 and dtype == torch.float32:
        x[0, 6] *= 1e-28                               # scale below 2^-80 (float32 only)
        x[0, 7] *= 1e35                                # near the float32 maximum
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32], ids=["f16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_quantize_matches_oracle(dtype, d):
    x = _quant_rows(300 + d, 3, 77, d, dtype)
    codes, scales = da.quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    want_c, want_s = ofp8.quantize_rows(x.numpy())
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    got_c = codes.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, (bad[:5].tolist(), got_c[tuple(bad[0])], want_c[tuple(bad[0])])


def test_quantize_strided_rows():
    """Rows inside wider buffers; the bytes around the outputs stay untouched."""
    x = _quant_rows(310, 2, 33, 512, torch.float16)
    wide = torch.zeros(2, 40, 640, dtype=torch.float16)
    wide[:, 3:36, 64:576] = x
    xd = wide.to(DEV)[:, 3:36, 64:576]
    codes = torch.full((2, 50, 544), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((2, 64), 7.0, dtype=torch.float32, device=DEV)
    da.ds4attn_quantize_fp8(xd, codes[:, 5:38, 16:528], scales[:, 10:43])
    torch.cuda.synchronize()
    want_c, want_s = ofp8.quantize_rows(x.numpy())
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(c[:, 5:38, 16:528], want_c)
    assert np.array_equal(s[:, 10:43], want_s)
    c[:, 5:38, 16:528] = 0xAB
    s[:, 10:43] = 7.0
    assert (c == 0xAB).all() and (s == 7.0).all()


# --------------------------------------------------------------------------- attention on FP8 rows

@pytest.mark.parametrize("name", ["decode_swa_fp8", "decode_r128_fp8"])
def test_attention_fp8_decode_full(name):
    w = wl.named(name)
    out = _run(w, "decode", 1)
    _compare(out, ref.attention(_oracle_problem(w)), name)


def test_attention_fp8_decode_ratio4_full():
    w = wl.named("decode_r4_fp8")
    _compare(_run(w, "decode", 1), _oracle_full("decode_r4_fp8"), "decode_r4_fp8 full")


def test_attention_fp8_prefill_ratio4_full():
    """The 2048-token ratio-4 chunk on FP8 rows, every token against the oracle."""
    w = wl.named("prefill_r4_fp8")
    out = _run(w, "prefill", da.ds4attn_prefill_bq())
    _compare(out, _oracle_full("prefill_r4_fp8"), "prefill_r4_fp8 full")


FP8_CASES = [
    ("f8_h16_ragged", dict(batch=3, tokens=2, heads=16, head_dim=512, n0=77), "decode", 1),
    ("f8_h32_window", dict(batch=1, tokens=40, heads=32, head_dim=512, n0=100, window=24,
                           q_pos0=60, k_pos0=0), "prefill", 16),
    ("f8_h48_valid", dict(batch=2, tokens=3, heads=48, head_dim=512, n0=90, valid0_frac=0.5),
     "prefill", 1),
    ("f8_h64_two_regions", dict(batch=2, tokens=2, heads=64, head_dim=512, n0=128, n1=150,
                                r1_mode="all", valid1_frac=0.8), "decode", 1),
    ("f8_h64_index", dict(batch=1, tokens=6, heads=64, head_dim=512, n0=70, window=32, q_pos0=60,
                          k_pos0=0, n1=300, r1_mode="index", r1_k=100, idx_invalid_frac=0.1),
     "prefill", 16),
    ("f8_h64_decode_index_valid", dict(batch=2, tokens=1, heads=64, head_dim=512, n0=33, n1=64,
                                       r1_mode="index", r1_k=64, valid1_frac=0.6), "decode", 1),
    ("f8_masked_tokens", dict(batch=1, tokens=5, heads=16, head_dim=512, n0=40, window=4, q_pos0=0,
                              k_pos0=3), "prefill", 2),
]


def _poison_hidden_rows(w):
    """Rows a validity mask hides hold NaN codes and NaN scales: they must not reach O."""
    for r in (w.r0, w.r1):
        if r is None or r.valid is None:
            continue
        hidden = r.valid == 0
        r.k[hidden] = 0x7F
        r.v[hidden] = 0xFF
        r.k_scale[hidden] = float("nan")
        r.v_scale[hidden] = float("nan")


@pytest.mark.parametrize("label,kw,entry,bq", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_attention_fp8_random(label, kw, entry, bq):
    seed = zlib.crc32(label.encode()) % 1000
    w = wl.fp8_variant(wl.random_problem(seed, **kw), seed + 1)
    want = ref.attention(_oracle_problem(w))
    _poison_hidden_rows(w)
    out = _run(w, entry, bq)
    _compare(out, want, label)
    if label == "f8_masked_tokens":
        assert (out[0, :3] == 0).all()   # tokens 0..2 see no row: exact zeros


@pytest.mark.parametrize("entry,bq", [("prefill", 16), ("decode", 1)])
def test_attention_fp8_query_magnitudes(entry, bq):
    """Heads whose queries differ by many binary orders of magnitude, one of them all
    zeros.  On FP8 rows the prefill and decode kernels compute the scores on the E4M3
    matrix cores, each head's query carried as two E4M3 terms under a power-of-two
    factor of its own: no term may leave the E4M3 range (past 448 the encoding is
    NaN), and tiny queries must keep their precision down to float16's own."""
    seed = 977
    tokens = 20 if entry == "prefill" else 1
    base = wl.random_problem(seed, batch=2, tokens=tokens, heads=64, head_dim=512, n0=160, window=48,
                             q_pos0=140, k_pos0=0)
    factors = [0.0, 2.0 ** -24, 2.0 ** -14, 2.0 ** -9, 2.0 ** -8, 2.0 ** -3, 1.0, 3.0]
    f = torch.tensor([factors[h % len(factors)] for h in range(64)], dtype=torch.float32)
    q = (base.q.float() * f[None, None, :, None]).to(base.q.dtype)
    q[0, :, 9, 17] = 60000.0 * 2.0 ** -9   # one element far above the rest of its head
    w = wl.fp8_variant(dataclasses.replace(base, q=q), seed + 1)
    out = _run(w, entry, bq)
    _compare(out, ref.attention(_oracle_problem(w)), f"fp8 {entry}, query magnitudes")


def test_quantize_then_attend():
    """float16 K/V -> ds4attn_quantize_fp8 -> decode on the FP8 rows, against the
    oracle's quantization fed to the oracle's attention."""
    w = wl.named("decode_swa")
    dp = pipeline.to_device(w, DEV)
    r = dp.r0
    kc, ks = da.quantize_fp8(r.k[:, :r.n_rows])
    vc, vs = da.quantize_fp8(r.v[:, :r.n_rows])
    torch.cuda.synchronize()
    wk, wks = ofp8.quantize_rows(w.r0.k.numpy())
    wv, wvs = ofp8.quantize_rows(w.r0.v.numpy())
    assert np.array_equal(kc.cpu().numpy(), wk) and np.array_equal(vc.cpu().numpy(), wv)
    assert np.array_equal(ks.cpu().numpy(), wks) and np.array_equal(vs.cpu().numpy(), wvs)
    dp.r0 = pipeline.DeviceRegion(kc, vc, r.n_rows, None, ks, vs)
    out = pipeline.step(dp, "decode", 1)
    torch.cuda.synchronize()
    w8 = dataclasses.replace(w, r0=wl.RegionInputs(torch.from_numpy(wk), torch.from_numpy(wv), w.r0.n_rows,
                                                   None, w.r0.ring_offset, torch.from_numpy(wks),
                                                   torch.from_numpy(wvs)))
    _compare(out.cpu().double().numpy(), ref.attention(_oracle_problem(w8)), "quantize -> decode")


# --------------------------------------------------------------------------- both decode work splits

FP8_SPLITS = {"dims": da.FLAG_DECODE_DIMS, "keys": da.FLAG_DECODE_KEYS}

FP8_DECODE_CASES = [(c[0], c[1]) for c in FP8_CASES] + [
    # lists longer than a chunk of 64 entries, index lists longer than 512 entries
    ("f8_long_dense", dict(batch=1, tokens=1, heads=16, head_dim=512, n0=4500, valid0_frac=0.9)),
    ("f8_long_index", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=128, n1=3000, r1_mode="index",
                           r1_k=1500, idx_invalid_frac=0.05)),
    # lists shorter than the four blocks DIMS stages before the map arrives: the blocks
    # guessed past the end of the list are in flight while the list is consumed
    ("f8_one_block", dict(batch=2, tokens=2, heads=16, head_dim=512, n0=20)),
    ("f8_short_window", dict(batch=2, tokens=3, heads=32, head_dim=512, n0=320, window=70, q_pos0=290,
                             k_pos0=0)),
]


def _run_flags(w, flags, splits=1):
    dp = pipeline.to_device(w, DEV)
    dp.flags = flags
    out = pipeline.step(dp, "decode", 1, splits=splits)   # splits=1: unsplit
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


@pytest.mark.parametrize("split", list(FP8_SPLITS))
@pytest.mark.parametrize("label,kw", FP8_DECODE_CASES, ids=[c[0] for c in FP8_DECODE_CASES])
def test_attention_fp8_decode_splits(label, kw, split):
    """Every case through the decode kernel with each way of dividing a workgroup's
    work over its waves forced; hidden rows hold NaN codes and NaN scales."""
    seed = zlib.crc32(label.encode()) % 1000
    w = wl.fp8_variant(wl.random_problem(seed, **kw), seed + 1)
    want = ref.attention(_oracle_problem(w))
    _poison_hidden_rows(w)
    out = _run_flags(w, FP8_SPLITS[split])
    _compare(out, want, f"{label}/{split}")
    if label == "f8_masked_tokens":
        assert (out[0, :3] == 0).all()


@pytest.mark.parametrize("name", ["decode_swa_fp8", "decode_r128_fp8"])
def test_attention_fp8_wide_workloads(name):
    """The wide DIMS split (32 heads per workgroup) on the FP8 batches without index
    lists, every output element."""
    w = wl.named(name)
    _compare(_run_flags(w, da.FLAG_DECODE_WIDE), _oracle_full(name), f"{name}/wide")


FP8_WIDE_CASES = [(label, kw) for label, kw in FP8_DECODE_CASES
                  if kw["heads"] % 32 == 0 and kw.get("r1_mode") != "index"] + [
    ("f8_wide_one_block", dict(batch=2, tokens=2, heads=32, head_dim=512, n0=20)),
    ("f8_wide_masked_tokens", dict(batch=1, tokens=5, heads=64, head_dim=512, n0=40, window=4, q_pos0=0,
                                   k_pos0=3)),
]


@pytest.mark.parametrize("label,kw", FP8_WIDE_CASES, ids=[c[0] for c in FP8_WIDE_CASES])
def test_attention_fp8_decode_wide(label, kw):
    """Hidden rows hold NaN codes and NaN scales, as in the other split tests."""
    w = wl.fp8_variant(wl.random_problem(zlib.crc32(label.encode()) % 1000 + 5, **kw), 7)
    want = ref.attention(_oracle_problem(w))
    _poison_hidden_rows(w)
    _compare(_run_flags(w, da.FLAG_DECODE_WIDE), want, f"{label}/wide")


@pytest.mark.parametrize("split", list(FP8_SPLITS))
def test_attention_fp8_workloads_splits(split):
    w = wl.named("decode_r128_fp8")
    _compare(_run_flags(w, FP8_SPLITS[split]), ref.attention(_oracle_problem(w)), f"decode_r128_fp8/{split}")
    w = wl.named("decode_r4_fp8")
    _compare(_run_flags(w, FP8_SPLITS[split]), _oracle_full("decode_r4_fp8"), f"decode_r4_fp8/{split}")


@pytest.mark.parametrize("split", list(FP8_SPLITS))
def test_attention_fp8_split_over_workgroups(split):
    kw = dict(batch=1, tokens=2, heads=64, head_dim=512, n0=70, window=32, q_pos0=60, k_pos0=0, n1=900,
              r1_mode="index", r1_k=300, idx_invalid_frac=0.1)
    w = wl.fp8_variant(wl.random_problem(77, **kw), 78)
    want = ref.attention(_oracle_problem(w))
    _compare(_run_flags(w, FP8_SPLITS[split], splits=3), want, f"fp8 index/{split} x3")


@pytest.mark.parametrize("mode", ["prefill", "dims", "keys", "wide"])
@pytest.mark.parametrize("pattern", ["tiny", "huge", "rising", "falling", "top"])
def test_attention_fp8_small_and_uneven_v_scales(mode, pattern):
    """V rows whose scales are tiny or huge (as float32 rows can give), or change
    by many binary orders of magnitude from one 32-row block to the next.  The
    kernels fold the V scales into the softmax weights under a running
    power-of-two factor: the weights must keep float16's precision at any
    magnitude (without the factor, V rows of magnitude 1e-4 lose tens of percent,
    and scales past 65504 overflow), and a block whose scales outgrow the factor
    must rescale what is already summed.  "top" takes the scales to the top of
    float32's range (up to 1.9 * 2^127, with codes of magnitude at most 1 so that
    every row value is a finite float32), where the factor's exponent meets its
    limit and any sum of unnormalised partial outputs would overflow.  Errors are
    relative to the output's largest magnitude, since O scales with V."""
    tokens = 16 if mode == "prefill" else 1
    w = wl.random_problem(151, batch=2, tokens=tokens, heads=64, head_dim=512, n0=160, q_pos0=200,
                          k_pos0=0)
    g = torch.Generator().manual_seed(152)
    kc, ks = ofp8.quantize_rows(w.r0.k.numpy())
    vc, vs = ofp8.quantize_rows(torch.randn(w.r0.v.shape, generator=g).half().numpy())
    block = np.arange(vs.shape[1]) // 32
    if pattern == "top":
        # codes of |value| <= 1, scales 1.9 * 2^127 * u (u in [0.5, 1)) but in blocks
        # 0 and 2, 2^-60 and 2^-30 lower: the factor set by block 0 must rise to its
        # limit at block 1, rescaling what is summed (in a split, the parts and
        # the KEYS waves each see a different mix of the two)
        x = (torch.randn(w.r0.v.shape, generator=g) * 0.3).clamp(-1.0, 1.0).numpy().astype(np.float32)
        vc = ofp8.encode(x)
        u = 0.5 + 0.5 * torch.rand(vs.shape, generator=g).numpy()
        drop = np.array([-60.0, 0.0, -30.0, 0.0, 0.0])[np.minimum(block, 4)]
        vs = (1.9 * 2.0 ** 127 * u * 2.0 ** drop[None, :]).astype(np.float32)
        assert np.isfinite(vs).all() and float(vs.max()) > 2.0 ** 127
        f = np.ones(vs.shape[1])
    elif pattern == "tiny":
        f = np.full(vs.shape[1], 1e-5)
    elif pattern == "huge":
        f = np.full(vs.shape[1], 1e25)
    elif pattern == "rising":
        f = 2.0 ** (10.0 * block - 40.0)      # 2^-40 .. 2^0, a factor 2^10 per block
    else:
        f = 2.0 ** (-10.0 * block)            # 1 .. 2^-40
    vs = (vs * f[None, :]).astype(np.float32)
    r0 = wl.RegionInputs(torch.from_numpy(kc), torch.from_numpy(vc), w.r0.n_rows, None, None,
                         torch.from_numpy(ks), torch.from_numpy(vs))
    w8 = dataclasses.replace(w, r0=r0)
    want = ref.attention(_oracle_problem(w8))
    ref_mag = float(np.abs(want).max())
    assert ref_mag > 0.0
    # decode also in three split parts, each with a V factor of its own, whose
    # records the combine pass must take in their true units (wide DIMS, two head
    # tiles per wave whose outputs both take the factor, has no split parts); at
    # the top of the range also in 12 parts over the 5 blocks: more than one batch
    # of eight records in the combine, and empty parts beside near-maximal ones
    splits_list = (1, 3, 12) if pattern == "top" else (1, 3)
    for splits in ((1,) if mode in ("prefill", "wide") else splits_list):
        dp = pipeline.to_device(w8, DEV)
        if mode == "prefill":
            out = pipeline.step(dp, "prefill", da.ds4attn_prefill_bq(), splits=1)
        else:
            dp.flags = {"dims": da.FLAG_DECODE_DIMS, "keys": da.FLAG_DECODE_KEYS,
                        "wide": da.FLAG_DECODE_WIDE}[mode]
            out = pipeline.step(dp, "decode", 1, splits=splits)
        torch.cuda.synchronize()
        out = out.cpu().double().numpy()
        assert np.isfinite(out).all()
        _compare(out / ref_mag, want / ref_mag, f"fp8 V scales {pattern}/{mode} x{splits}")


@pytest.mark.parametrize("mode", ["prefill", "dims", "keys"])
def test_attention_fp8_values_at_the_float16_maximum(mode):
    """V rows quantized (by the oracle's quantizer) from float16 rows that reach
    +-65504, so their scale is 65504/448: no value may overflow to inf in any
    kernel.  Every V row is scaled alike (standard deviation 8000), so O scales with
    them; errors are compared after dividing both sides by 65504."""
    tokens = 16 if mode == "prefill" else 1
    w = wl.random_problem(141, batch=2, tokens=tokens, heads=64, head_dim=512, n0=70, window=48, q_pos0=60,
                          k_pos0=0)
    g = torch.Generator().manual_seed(142)
    v = torch.randn(w.r0.v.shape, generator=g) * 8000
    v[:, ::3, 5] = 65504.0
    v[:, 1::3, 9] = -65504.0
    v = v.clamp(-65504, 65504).half()
    kc, ks = ofp8.quantize_rows(w.r0.k.numpy())
    vc, vs = ofp8.quantize_rows(v.numpy())
    assert float(vs.max()) == float(np.float32(65504.0) / np.float32(448.0))
    r0 = wl.RegionInputs(torch.from_numpy(kc), torch.from_numpy(vc), w.r0.n_rows, None, None,
                         torch.from_numpy(ks), torch.from_numpy(vs))
    w8 = dataclasses.replace(w, r0=r0)
    want = ref.attention(_oracle_problem(w8))
    dp = pipeline.to_device(w8, DEV)
    if mode == "prefill":
        out = pipeline.step(dp, "prefill", da.ds4attn_prefill_bq(), splits=1)
    else:
        dp.flags = da.FLAG_DECODE_DIMS if mode == "dims" else da.FLAG_DECODE_KEYS
        out = pipeline.step(dp, "decode", 1, splits=1)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    assert np.isfinite(out).all()
    _compare(out / 65504.0, want / 65504.0, f"fp8 V rows at +-65504/{mode}")
