"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Bar: padded layout and block map bit-exact; attention output within max-abs
1e-2 and mean-abs 1e-3 of the oracle (float16 inputs, float32 output).
Inputs are the seeded workloads of ``query_flashattention_amd.workloads``.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl
from tests.parity_util import compare as _compare, oracle_full

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()  # fail loudly if the HIP library is missing


def _bits(t):
    a = t.cpu().contiguous()
    if a.dtype == torch.float16:
        return a.view(torch.int16).numpy()
    if a.dtype == torch.float32:
        return a.view(torch.int32).numpy()
    return a.numpy()


# --------------------------------------------------------------------------- pad

def _pad_check(k, v, valid, n):
    kd, vd = k.to(DEV), v.to(DEV)
    vald = None if valid is None else valid.to(DEV)
    kp, vp, vap = da.pad_region(kd, vd, n, vald)
    torch.cuda.synchronize()
    wk, wv, wva = ref.pad_layout(k.numpy(), v.numpy(), None if valid is None else valid.numpy(), n)
    itype = np.int16 if k.dtype == torch.float16 else np.int32
    assert np.array_equal(_bits(kp), wk.view(itype))
    assert np.array_equal(_bits(vp), wv.view(itype))
    assert np.array_equal(vap.cpu().numpy(), wva)


@pytest.mark.parametrize("name", ["tiny", "decode_swa", "decode_r128", "prefill_swa", "prefill_r4"])
def test_pad_bits_on_workloads(name):
    w = wl.named(name)
    for r in (w.r0, w.r1):
        if r is not None:
            _pad_check(r.k, r.v, r.valid, r.n_rows)


@pytest.mark.parametrize("n", [1, 27, 31, 32, 33, 64, 95])
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_pad_bits_edges(n, dtype):
    g = torch.Generator().manual_seed(n)
    k = torch.randn(3, n, 64, generator=g).to(dtype)
    v = torch.randn(3, n, 64, generator=g).to(dtype)
    valid = (torch.rand(3, n, generator=g) < 0.5).to(torch.uint8)
    _pad_check(k, v, None, n)
    _pad_check(k, v, valid, n)


def test_pad_in_place_zeroes_only_the_tail():
    w = wl.random_problem(3, batch=2, tokens=1, heads=4, head_dim=64, dtype=torch.float32, n0=45,
                          valid0_frac=0.5)
    dp = pipeline.to_device(w, DEV)
    dp.r0.k[:, 45:].fill_(float("nan"))
    dp.r0.valid[:, 45:].fill_(7)          # the validity tail is padded in place too
    dp.r0.pad_in_place()
    torch.cuda.synchronize()
    kp, _, vap = ref.pad_layout(w.r0.k.numpy(), w.r0.v.numpy(), w.r0.valid.numpy(), 45)
    assert np.array_equal(_bits(dp.r0.k), kp.view(np.int32))
    assert np.array_equal(dp.r0.valid.cpu().numpy(), vap)


# --------------------------------------------------------------------------- block map

def _map_check(w, bq):
    dp = pipeline.to_device(w, DEV)
    dp.r0.pad_in_place()
    if dp.r1 is not None:
        dp.r1.pad_in_place()
    got = da.blockmap(dp.args(), bq, DEV).cpu().numpy()
    want = ref.blockmap(ref.from_workload(w, logical_ring=False), bq)
    assert got.shape == want.shape and np.array_equal(got, want)
    return got


@pytest.mark.parametrize("name,bq", [("tiny", 1), ("decode_swa", 1), ("decode_r128", 1),
                                     ("decode_r128_b64", 1), ("decode_r4", 1), ("prefill_swa", 1),
                                     ("prefill_swa", 16),
                                     ("prefill_r4", 1), ("prefill_r4", 16), ("prefill_r4", 2048)])
def test_blockmap_bits_on_workloads(name, bq):
    got = _map_check(wl.named(name), bq)
    if name == "prefill_swa" and bq == 16:
        assert [int((got == s).sum()) for s in (0, 1, 2)] == [7572, 248, 372]


@pytest.mark.parametrize("seed,kw,bq", [
    (1, dict(n0=77, window=20, q_pos0=40, k_pos0=0, tokens=37), 5),
    (2, dict(n0=64, valid0_frac=0.8, window=50, q_pos0=63, k_pos0=10, tokens=9), 3),
    (3, dict(n0=40, n1=70, r1_mode="all", valid1_frac=0.5, tokens=4, batch=3), 2),
    (4, dict(n0=33, window=7, q_pos0=0, k_pos0=0, tokens=70), 64),
    (5, dict(n0=1, window=3, q_pos0=5, k_pos0=0, tokens=2), 1),
])
def test_blockmap_bits_random(seed, kw, bq):
    base = dict(batch=2, tokens=3, heads=4, head_dim=64, dtype=torch.float32)
    base.update(kw)
    _map_check(wl.random_problem(seed, **base), bq)


# --------------------------------------------------------------------------- attention, the five workloads

def _run(w, entry, bq, use_map=True, flags=0):
    dp = pipeline.to_device(w, DEV)
    dp.flags = flags
    if use_map:
        out = pipeline.step(dp, entry, bq)
    else:
        dp.r0.pad_in_place()
        if dp.r1 is not None:
            dp.r1.pad_in_place()
        fn = da.ds4attn_decode if entry == "decode" else da.ds4attn_prefill
        fn(dp.args(), dp.q, None, bq, dp.o)
        out = dp.o
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("name,entry,bq", [
    ("tiny", "decode", 1),
    ("decode_swa", "decode", 1),
    ("decode_r128", "decode", 1),
    ("decode_r128_b64", "decode", 1),
    ("prefill_swa", "prefill", 16),
])
def test_attention_workload_full(name, entry, bq):
    w = wl.named(name)
    out = _run(w, entry, bq).double().numpy()
    want = ref.attention(ref.from_workload(w))
    _compare(out, want, f"{name}/{entry}")


def test_attention_decode_ratio4_full():
    """The indexed ratio-4 decode batch at full size (64 sequences, 128 ring rows +
    top-512 of 2048 compressed rows each), every sequence against the oracle."""
    w = wl.named("decode_r4")
    out = _run(w, "decode", 1).double().numpy()
    _compare(out, oracle_full("decode_r4"), "decode_r4 full")


def test_attention_prefill_ratio4_full():
    """The indexed ratio-4 prefill chunk at full size (2048 tokens, each with its own
    top-512 list), in the launch the benchmark times; every token against the oracle."""
    w = wl.named("prefill_r4")
    out = _run(w, "prefill", 16).double().numpy()
    _compare(out, oracle_full("prefill_r4"), "prefill_r4 full")


# --------------------------------------------------------------------------- attention, general cases

RANDOM_CASES = [
    # generic vector-ALU kernel: float32 / small heads / other head sizes
    ("gen_f32_d64", dict(batch=2, tokens=5, heads=4, head_dim=64, dtype=torch.float32, n0=70,
                         window=30, q_pos0=60, k_pos0=0), "decode", 1),
    ("gen_f16_d128_h7", dict(batch=1, tokens=3, heads=7, head_dim=128, n0=50, valid0_frac=0.6,
                             n1=40, r1_mode="all", valid1_frac=0.7), "prefill", 2),
    ("gen_f32_d256_idx", dict(batch=2, tokens=4, heads=3, head_dim=256, dtype=torch.float32, n0=20,
                              n1=90, r1_mode="index", r1_k=33, idx_invalid_frac=0.2), "decode", 1),
    ("gen_f16_d512_h5", dict(batch=1, tokens=2, heads=5, head_dim=512, n0=45), "decode", 1),
    # matrix-core kernel: D = 512, float16, heads a multiple of 16
    ("mfma_h16_ragged", dict(batch=3, tokens=2, heads=16, head_dim=512, n0=77), "decode", 1),
    ("mfma_h32_window", dict(batch=1, tokens=40, heads=32, head_dim=512, n0=100, window=24,
                             q_pos0=60, k_pos0=0), "prefill", 16),
    ("mfma_h48_valid", dict(batch=2, tokens=3, heads=48, head_dim=512, n0=90, valid0_frac=0.5),
     "prefill", 1),
    ("mfma_h64_two_regions", dict(batch=2, tokens=2, heads=64, head_dim=512, n0=128, n1=150,
                                  r1_mode="all", valid1_frac=0.8), "decode", 1),
    ("mfma_h64_index", dict(batch=1, tokens=6, heads=64, head_dim=512, n0=70, window=32, q_pos0=60,
                            k_pos0=0, n1=300, r1_mode="index", r1_k=100, idx_invalid_frac=0.1),
     "prefill", 16),
    ("mfma_h128_decode_index", dict(batch=2, tokens=1, heads=128, head_dim=512, n0=33, n1=64,
                                    r1_mode="index", r1_k=64), "decode", 1),
    ("mfma_big_scores", dict(batch=1, tokens=3, heads=64, head_dim=512, n0=96, q_std=4.0), "decode", 1),
    ("mfma_empty_r0", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=0, n1=50, r1_mode="all"),
     "decode", 1),
    ("mfma_masked_tokens", dict(batch=1, tokens=5, heads=16, head_dim=512, n0=40, window=4, q_pos0=0,
                                k_pos0=3), "prefill", 2),
    ("mfma_index_all_unused", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=10, n1=20,
                                   r1_mode="index", r1_k=32, idx_invalid_frac=1.0), "decode", 1),
]


@pytest.mark.parametrize("label,kw,entry,bq", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_attention_random(label, kw, entry, bq):
    w = wl.random_problem(zlib.crc32(label.encode()) % 1000, **kw)
    out = _run(w, entry, bq).double().numpy()
    want = ref.attention(ref.from_workload(w))
    _compare(out, want, label)
    if label == "mfma_masked_tokens":
        assert (out[0, :3] == 0).all()   # tokens 0..2 see no row: exact zeros


def test_map_does_not_change_the_result():
    """Skipping blocks is exact: with the map, without it (every block masked
    pair by pair) and through the vector-ALU kernel the outputs agree."""
    w = wl.random_problem(11, batch=1, tokens=33, heads=64, head_dim=512, n0=150, window=40,
                          q_pos0=100, k_pos0=0, n1=64, r1_mode="all", valid1_frac=0.7)
    with_map = _run(w, "prefill", 16)
    no_map = _run(w, "prefill", 16, use_map=False)
    assert torch.equal(with_map, no_map)
    generic = _run(w, "prefill", 16, flags=da.FLAG_GENERIC)
    _compare(generic.double().numpy(), with_map.double().numpy(), "generic vs matrix-core")


def test_decode_and_prefill_agree():
    w = wl.random_problem(12, batch=2, tokens=3, heads=64, head_dim=512, n0=96, n1=40,
                          r1_mode="index", r1_k=40)
    a = _run(w, "decode", 1).double().numpy()
    b = _run(w, "prefill", 1).double().numpy()
    _compare(a, b, "decode vs prefill")


# --------------------------------------------------------------------------- split decode

def _run_split(w, splits, use_map=True):
    dp = pipeline.to_device(w, DEV)
    if use_map:
        out = pipeline.step(dp, "decode", 1, splits=splits)
    else:
        dp.r0.pad_in_place()
        if dp.r1 is not None:
            dp.r1.pad_in_place()
        a = dp.args()
        ws = torch.empty(da.ds4attn_decode_workspace_bytes(a, splits), dtype=torch.uint8, device=DEV)
        da.ds4attn_decode_split(a, dp.q, None, 1, dp.o, splits, ws)
        out = dp.o
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("splits", [2, 3, 12, 64])
def test_split_decode_ratio128_single_sequence(splits):
    """The ratio-128 layer at 32K for one sequence (12 key blocks) with its blocks
    divided over 2, 3, 12 and 64 workgroups per head group (64: most parts empty)."""
    w = wl.named("decode_r128")
    out = _run_split(w, splits).double().numpy()
    _compare(out, ref.attention(ref.from_workload(w)), f"decode_r128 split {splits}")


@pytest.mark.parametrize("name,splits", [("decode_swa", 2), ("decode_r4", 5), ("decode_r4_fp8", 3),
                                          ("decode_r128_fp8", 4)])
def test_split_decode_batches(name, splits):
    w = wl.named(name)
    out = _run_split(w, splits).double().numpy()
    if name.endswith("_fp8"):
        plain = _run(w, "decode", 1).double().numpy()
        _compare(out, plain, f"{name} split {splits} vs unsplit")
        return
    _compare(out, oracle_full(name), f"{name} split {splits}")


SPLIT_CASES = [
    ("split_ragged_valid", dict(batch=2, tokens=3, heads=16, head_dim=512, n0=150, valid0_frac=0.5), 4),
    ("split_window_index", dict(batch=1, tokens=4, heads=64, head_dim=512, n0=70, window=32, q_pos0=60,
                                k_pos0=0, n1=300, r1_mode="index", r1_k=100, idx_invalid_frac=0.1), 6),
    ("split_masked_tokens", dict(batch=1, tokens=5, heads=16, head_dim=512, n0=40, window=4, q_pos0=0,
                                 k_pos0=3), 3),
]


@pytest.mark.parametrize("label,kw,splits", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_decode_random(label, kw, splits):
    w = wl.random_problem(zlib.crc32(label.encode()) % 1000, **kw)
    want = ref.attention(ref.from_workload(w))
    with_map = _run_split(w, splits)
    _compare(with_map.double().numpy(), want, label)
    # without a map every block is a list entry, so the parts differ: same result up to rounding
    no_map = _run_split(w, splits, use_map=False)
    _compare(no_map.double().numpy(), want, label + " no map")
    if label == "split_masked_tokens":
        assert (with_map[0, :3] == 0).all()   # tokens 0..2 see no row in any part: exact zeros


def test_split_decode_reuses_its_workspace():
    """One workspace serves split calls of different sizes and work splits in a row
    (its contents on entry do not matter); each result matches the oracle."""
    ws = None
    for name, flags in (("decode_r128", 0), ("decode_r128_b64", da.FLAG_DECODE_DIMS), ("decode_r128", da.FLAG_DECODE_KEYS),
                        ("decode_r128", 0)):
        w = wl.named(name)
        dp = pipeline.to_device(w, DEV)
        dp.flags = flags
        dp.r0.pad_in_place()
        if dp.r1 is not None:
            dp.r1.pad_in_place()
        a = dp.args()
        need = da.ds4attn_decode_workspace_bytes(a, 4)
        if ws is None:
            # large enough for the 64-sequence batch too; filled with a byte pattern
            ws = torch.full((need * 64,), 0x7F, dtype=torch.uint8, device=DEV)
        assert need <= ws.numel()
        blk = da.blockmap(a, 1, DEV)
        da.ds4attn_decode_split(a, dp.q, blk, 1, dp.o, 4, ws)
        torch.cuda.synchronize()
        out = dp.o.cpu().double().numpy()
        _compare(out, oracle_full(name), f"{name} split 4 flags {flags}, reused workspace")
