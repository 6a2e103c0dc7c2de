"""GPU parity of the outlier-channel split ("TurboQuant của Google…"
(omelet.tech) section "Thực nghiệm: 3.5 bit…": 32 outlier channels at one bit
more than the other 96) against the oracle, through the C ABI: the encoder's
code strings and group norms, and decode attention over split caches."""
import numpy as np
import pytest
import torch

import synth
from kv_cache_vector_06_amd import torch_api as T
from gpu_util import (DEV, check_encode_split, gpu_packed_arrays, oracle_encode_split, say, split_quantizer,
                      to_gpu_x)

pytestmark = pytest.mark.gpu
D = 128


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_split_encode_parity(bits, dtype):
    q, consts = split_quantizer(bits, "k")
    n = 4096 + 37
    X = synth.split_kv(1, 1, n, D, 600 + bits, consts[0], dtype=dtype)[0, 0]
    say("split encode", bits, dtype, n)
    p = T.encode(q, to_gpu_x(X, dtype))
    st = check_encode_split(gpu_packed_arrays(p, q), oracle_encode_split(X, consts, bits), bits)
    say(st)


@pytest.mark.parametrize("bits", [2, 3])
def test_split_encode_edge_cases(bits):
    # a zero row, rows with only the outlier or only the regular channels
    # nonzero, tiny batches, and a scatter into slots
    q, consts = split_quantizer(bits, "v")
    ch = consts[0]
    reg = np.setdiff1d(np.arange(D), ch)
    X = synth.split_kv(1, 1, 50, D, 650 + bits, ch, dtype="bf16")[0, 0].copy()
    X[0] = 0.0
    X[1, reg] = 0.0
    X[2, ch] = 0.0
    X[3] = 0.0
    X[3, ch[7]] = -2.5
    ref = oracle_encode_split(X, consts, bits)
    xg = to_gpu_x(X, "bf16")
    st = check_encode_split(gpu_packed_arrays(T.encode(q, xg), q), ref, bits)
    say(st)
    for m in (1, 3, 17):
        g = gpu_packed_arrays(T.encode(q, xg[:m]), q)
        sub = {k: v[:m] for k, v in ref.items()}
        check_encode_split(g, sub, bits)
    slots = torch.tensor([7, 2, 40, 0], dtype=torch.int64, device=DEV)
    out = T.Packed(q, 41, DEV)
    T.encode(q, xg[:4], out, slots)
    g = gpu_packed_arrays(out, q)
    full = gpu_packed_arrays(T.encode(q, xg[:4]), q)
    for i, s in enumerate([7, 2, 40, 0]):
        np.testing.assert_array_equal(g["codes"][s], full["codes"][i])
        np.testing.assert_array_equal(g["norms"][s], full["norms"][i])
