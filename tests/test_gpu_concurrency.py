"""Independent calls do not interfere: two host threads, each with its own stream
and buffers, run decode steps on one shared cache at the same time, and every
result equals, bit for bit, the same step run alone.  The library keeps no state
between calls (its only statics are per thread), so this must hold."""
import threading

import pytest
import torch

import block_sparse_attention_compress_amd as qsa
import synth
from block_sparse_attention_compress_amd.pipeline import DecodeBuffers, decode_step
from gpu_harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_two_threads_two_streams():
    case = synth.config("C2", B=6, L_range=(9000, 20000))
    dev = synth.to_device(case, "cuda")
    kv = qsa.KVCache(dev["k"], dev["v"], dev["ckey"], dev["block_table"], dev["seq_lens"], case.max_len)
    qsa.qsa_compress_keys(kv)
    stride = max(case.nb(i) for i in range(case.B))
    queries = [dev["q"], (-dev["q"]).contiguous()]   # two different queries over the same cache
    bufs = [DecodeBuffers.allocate(case.B, case.Hq, case.Hkv, stride, case.topk, 0, "cuda") for _ in queries]
    # refresh off: the two threads only read the shared cache
    refs = []
    for q, buf in zip(queries, bufs):
        decode_step(kv, q, dev["q_pos"], buf, scale=case.scale, refresh_keys=False)
        torch.cuda.synchronize()
        refs.append((buf.sel_idx.clone(), buf.sel_cnt.clone(), buf.out.clone(), buf.lse.clone()))
    log("two threads, two streams, 25 decode steps each")
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()   # default priority
            with torch.cuda.stream(stream):
                for it in range(25):
                    bufs[i].out.fill_(float("nan"))
                    decode_step(kv, queries[i], dev["q_pos"], bufs[i], scale=case.scale, refresh_keys=False)
                    stream.synchronize()
                    got = (bufs[i].sel_idx, bufs[i].sel_cnt, bufs[i].out, bufs[i].lse)
                    for a, b in zip(got, refs[i]):
                        if not torch.equal(a, b):
                            errors.append(f"thread {i} step {it} differs")
                            return
        except Exception as e:  # surfaced below
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
