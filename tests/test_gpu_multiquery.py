"""GPU parity with several queries per request (qo_len > 1) against the fp64
oracle.

Query i of request b is row b * qo_len + i of q / o / lse and sees the first
L_b - (qo_len - 1 - i) tokens (the causal mask with the queries at the end of
the score matrix; "FlashMLA SM100", forward kernel notes on N_Q != N_K).  The
qo_len * H query vectors of a request are folded into the kernel's head
dimension, so these cases run every kernel width (16 to 128 query vectors per
workgroup, split into several rows per request when wider), with requests
shorter than qo_len (queries that see nothing: O = 0, LSE = -inf exactly),
chunks cut inside the masked tail, and 8-bit caches.  Tolerances as in
test_gpu_parity.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_common import check, dev, gpu_run, host, ref  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_decode_amd as mla
    mla.load_library()  # fail loudly if the HIP library is missing


LENGTHS = [1, 2, 0, 17, 64, 65, 333, 1000]

# (heads, qo_len, kv dtype): query vectors per request = heads * qo_len
CASES = [
    (16, 2, synth.KV_BF16),       # 32 wide
    (16, 3, synth.KV_BF16),       # 48: three 16-wide rows per request
    (16, 4, synth.KV_BF16),       # 64 wide
    (16, 8, synth.KV_BF16),       # 128 wide
    (32, 2, synth.KV_BF16),       # 64 wide
    (64, 2, synth.KV_BF16),       # 128 wide
    (128, 2, synth.KV_BF16),      # two 128-wide rows per request
    (16, 2, synth.KV_FP8_E4M3),   # two 16-wide rows
    (16, 8, synth.KV_FP8_E4M3),   # 128 wide, 8-bit
    (64, 2, synth.KV_INT8),       # 128 wide, 8-bit
    (128, 2, synth.KV_INT8),      # two 128-wide rows, 8-bit
    (32, 2, synth.KV_FP16),       # 64 wide, fp16
    (16, 8, synth.KV_FP16),       # 128 wide, fp16
]


@pytest.mark.parametrize("heads,q,kvd", CASES)
@pytest.mark.parametrize("page", [16, 64])
def test_multiquery_matches_oracle(heads, q, kvd, page):
    inp = synth.make_inputs(LENGTHS, heads, page, kvd, seed=500 + heads + q + page, poison=True,
                            extra_pages=3, qo_len=q)
    print("case heads=%d qo_len=%d kv=%d page=%d" % (heads, q, kvd, page), flush=True)
    o, lse = host(*gpu_run(inp))
    o_ref, lse_ref = ref(inp)
    check(o, lse, o_ref, lse_ref)
    # queries with nothing visible: request of 1 token, queries 0 .. q - 2
    assert np.all(np.isneginf(lse[0:q - 1])) and np.all(o[0:q - 1] == 0)


@pytest.mark.parametrize("heads,q,kvd", [(16, 4, synth.KV_BF16), (16, 8, synth.KV_BF16),
                                         (128, 2, synth.KV_BF16), (16, 2, synth.KV_FP8_E4M3),
                                         (16, 8, synth.KV_INT8), (32, 2, synth.KV_FP16)])
@pytest.mark.parametrize("splits", [2, 5])
def test_multiquery_forced_splits(heads, q, kvd, splits):
    # with 16-token chunks, the last chunk of the 65-token request holds one
    # token, which only the last query sees: the others get an empty partial
    inp = synth.make_inputs([65, 700, 3, 1500], heads, 16, kvd, seed=600 + splits + q,
                            poison=True, qo_len=q)
    print("case heads=%d qo_len=%d kv=%d splits=%d" % (heads, q, kvd, splits), flush=True)
    o, lse = host(*gpu_run(inp, force_splits=splits))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("heads,q,hs", [(16, 2, 2), (16, 8, 2), (16, 8, 8), (128, 2, 4)])
def test_multiquery_explicit_head_split(heads, q, hs):
    inp = synth.make_inputs([700, 1, 4096, 65, 0], heads, 32, seed=700 + hs, poison=True,
                            qo_len=q)
    print("case heads=%d qo_len=%d head_split=%d" % (heads, q, hs), flush=True)
    o, lse = host(*gpu_run(inp, head_split=hs))
    check(o, lse, *ref(inp))


def test_multiquery_reruns_bit_identical():
    inp = synth.make_inputs([900, 64, 5, 2049], 16, 64, seed=801, qo_len=4)
    t = dev(inp)
    o1, l1 = gpu_run(inp, t)
    o2, l2 = gpu_run(inp, t)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kvd", [synth.KV_BF16, synth.KV_FP8_E4M3])
def test_multiquery_full_size_every_row(kvd):
    # 64 requests of 4096 tokens, 16 heads, 2 queries each (the next-token
    # prediction shape): every (query, head) row against the oracle
    inp = synth.make_inputs([4096] * 64, 16, 64, kvd, seed=802, qo_len=2)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))
