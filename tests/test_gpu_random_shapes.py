"""Seeded random small shapes through the whole path, against the oracle.

Each case draws its head pair (group sizes 1 to 16, including the pages' pairs),
page size, batch, lengths (1 to 6,000 tokens, sometimes 0), k, split count,
block-key storage and cache storage at once, so combinations that the targeted
tests do not enumerate are covered too.  Decode cases run the step of the
separate calls, and some of them the fused single launch as well (its selection
equal to the separate calls' bit for bit); extend cases put several sequences'
new rows in one launch.
The bars are those of the targeted parity tests: the selection bit-exact on the
GPU's own fp32 scores and within the 1e-4 swap window against the oracle,
outputs and lse within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import log
from test_gpu_parity import check_decode_against_oracle, run_decode, run_extend

pytestmark = pytest.mark.gpu

HEAD_PAIRS = [(16, 2), (24, 2), (12, 1), (6, 1), (3, 1), (8, 8), (16, 1), (32, 2), (4, 2)]
PAGE_SIZES = [4, 8, 16, 64, 256]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(rng, options):
    return options[int(rng.integers(len(options)))]


def random_decode(i: int):
    rng = np.random.default_rng(7000 + i)
    Hq, Hkv = draw(rng, HEAD_PAIRS)
    B = int(rng.integers(1, 5))
    lens = rng.integers(1, 6001, size=B)
    if rng.random() < 0.2:
        lens[int(rng.integers(B))] = 0
    k = draw(rng, [1, 17, 512, 600])
    splits = draw(rng, [0, 1, 3, 16])
    case = synth.make_case(f"rnd{i}", 7000 + i, Hq, Hkv, lens.tolist(), draw(rng, PAGE_SIZES), topk=k,
                           jitter=bool(rng.integers(2)), ckey_dtype=draw(rng, ["fp32", "bf16", "fp8"]),
                           kv_dtype=draw(rng, ["bf16", "fp8"]))
    return case, k, splits


def random_extend(i: int):
    rng = np.random.default_rng(9000 + i)
    Hq, Hkv = draw(rng, HEAD_PAIRS)
    B = int(rng.integers(1, 4))
    lens = rng.integers(50, 5001, size=B)
    q_seq, q_pos = [], []
    for s in range(B):  # each sequence's newest n tokens are query rows
        n = int(rng.integers(1, min(int(lens[s]), 150) + 1))
        q_seq += [s] * n
        q_pos += list(range(int(lens[s]) - n, int(lens[s])))
    k = draw(rng, [1, 64, 512])
    case = synth.make_case(f"rndx{i}", 9000 + i, Hq, Hkv, lens.tolist(), draw(rng, PAGE_SIZES), topk=k,
                           q_seq=q_seq, q_pos=q_pos, jitter=bool(rng.integers(2)),
                           ckey_dtype=draw(rng, ["fp32", "bf16", "fp8"]), kv_dtype=draw(rng, ["bf16", "fp8"]))
    return case, k


@pytest.mark.parametrize("i", range(24))
def test_random_decode_shapes(i):
    case, k, splits = random_decode(i)
    log(f"random decode {i}: heads=({case.Hq},{case.Hkv}) page={case.page_size} lens={case.lens.tolist()} k={k} "
        f"splits={splits} keys={case.ckey_dtype} cache={case.kv_dtype}")
    res = run_decode(case, k=k, num_splits=splits)
    check_decode_against_oracle(case, *res, k)


@pytest.mark.parametrize("i", range(12))
def test_random_extend_shapes(i):
    case, k = random_extend(i)
    log(f"random extend {i}: heads=({case.Hq},{case.Hkv}) page={case.page_size} lens={case.lens.tolist()} "
        f"rows={case.R} k={k} keys={case.ckey_dtype} cache={case.kv_dtype}")
    res = run_extend(case, k=k)
    check_decode_against_oracle(case, *res, k)


@pytest.mark.parametrize("i", range(0, 24, 3))
def test_random_decode_shapes_fused(i):
    from test_gpu_fused import check_fused
    case, k, splits = random_decode(i)
    log(f"random fused {i}: heads=({case.Hq},{case.Hkv}) page={case.page_size} lens={case.lens.tolist()} k={k} "
        f"splits={splits} keys={case.ckey_dtype} cache={case.kv_dtype}")
    check_fused(case, k=k, num_splits=splits)
