"""GPU parity of decode attention over the INT8 KV cache (the cache's consumer; VARC "INT8 KV
cache quantization") through the C ABI, against the oracle's fp64 attention on the exactly
dequantized cache: bf16 output within the normwise max-abs-rel 1e-2."""
import math

import numpy as np
import pytest
import torch

from bit_post_quantized_amd import binding as B
from oracle import kv_attention as oka
from oracle import kv_int8 as okv
from oracle.numerics import bf16_to_bits, decode_bf16, round_bf16
from synthetic import make_kv
from tests.gpu_cases import dev, dev_bf16, max_abs_rel

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _cache(tokens, heads, dim, seed=0):
    kv = make_kv(seed=seed, tokens=tokens, heads=heads, dim=dim)
    out = {}
    for name in ("K", "V"):
        ref = okv.kv_int8_quant(kv[name].reshape(tokens, -1))
        out[name] = (ref["q"], ref["scale"], ref["zero"])
    return out


def _run(q_bits, cache, heads, dim, sm_scale):
    nq = q_bits.shape[0]
    (kq, ks, kz), (vq, vs, vz) = cache["K"], cache["V"]
    tokens = kq.shape[0]
    out = torch.empty(nq, heads, dim, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.kv_int8_attention_workspace_bytes(nq, tokens, heads, dim), dtype=torch.uint8,
                     device="cuda")
    B.kv_int8_attention(dev_bf16(q_bits), dev(kq), dev(ks), dev(kz), dev(vq), dev(vs), dev(vz),
                        sm_scale, out, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("tokens,heads,dim,nq", [
    (1, 2, 64, 1),          # a single token: the output is its value row
    (300, 4, 128, 2),       # one full and one ragged 256-token chunk
    (1000, 8, 64, 3),
    (257, 2, 128, 1),       # a one-token tail chunk
    (10240, 32, 128, 1),    # the cache shape of the KV workload
    (70000, 2, 64, 1),      # 274 chunks: more chunks than combine threads
    (1048576, 1, 64, 1),    # 4096 chunks, the most one call takes
])
def test_attention_matches_the_oracle(gpu_lib, tokens, heads, dim, nq):
    cache = _cache(tokens, heads, dim)
    rng = np.random.default_rng(tokens)
    q = bf16_to_bits(round_bf16(rng.standard_normal((nq, heads, dim))))
    sm = 1.0 / math.sqrt(dim)
    got = _run(q, cache, heads, dim, sm)
    ref = oka.attention(q, *cache["K"], *cache["V"], heads, dim, sm)
    assert max_abs_rel(got, ref) <= TOL


def test_sharp_softmax_and_large_scores(gpu_lib):
    # queries 40x larger: the weights concentrate on a few tokens across chunk boundaries
    tokens, heads, dim = 700, 4, 128
    cache = _cache(tokens, heads, dim, seed=1)
    rng = np.random.default_rng(5)
    q = bf16_to_bits(round_bf16(40.0 * rng.standard_normal((2, heads, dim))))
    got = _run(q, cache, heads, dim, 1.0 / math.sqrt(dim))
    ref = oka.attention(q, *cache["K"], *cache["V"], heads, dim, 1.0 / math.sqrt(dim))
    assert max_abs_rel(got, ref) <= TOL


def test_end_to_end_from_the_gpu_quantizer(gpu_lib):
    # the cache as kv_int8_quant writes it on the device, read back by the attention kernel
    tokens, heads, dim = 2048, 8, 128
    kv = make_kv(seed=2, tokens=tokens, heads=heads, dim=dim)
    C = heads * dim
    parts = {}
    for name in ("K", "V"):
        x = dev_bf16(kv[name].reshape(tokens, C))
        q8 = torch.empty(tokens, C, dtype=torch.uint8, device="cuda")
        s = torch.empty(C, dtype=torch.float32, device="cuda")
        z = torch.empty(C, dtype=torch.uint8, device="cuda")
        ws = torch.empty(B.kv_int8_workspace_bytes(tokens, C), dtype=torch.uint8, device="cuda")
        B.kv_int8_quant(x, q8, s, z, ws)
        parts[name] = (q8, s, z)
    rng = np.random.default_rng(9)
    q = bf16_to_bits(round_bf16(rng.standard_normal((1, heads, dim))))
    out = torch.empty(1, heads, dim, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.kv_int8_attention_workspace_bytes(1, tokens, heads, dim), dtype=torch.uint8,
                     device="cuda")
    B.kv_int8_attention(dev_bf16(q), *parts["K"], *parts["V"], 1.0 / math.sqrt(dim), out, ws)
    torch.cuda.synchronize()
    ref_cache = _cache(tokens, heads, dim, seed=2)
    ref = oka.attention(q, *ref_cache["K"], *ref_cache["V"], heads, dim, 1.0 / math.sqrt(dim))
    assert max_abs_rel(out.float().cpu().numpy().astype(np.float64), ref) <= TOL
    # and the attention of the unquantized bf16 cache is close too (the codes' own error)
    K = decode_bf16(kv["K"]).reshape(tokens, heads, dim)
    V = decode_bf16(kv["V"]).reshape(tokens, heads, dim)
    qd = decode_bf16(q).reshape(heads, dim)
    full = np.stack([np.exp(s - s.max()) / np.exp(s - s.max()).sum() @ V[:, h]
                     for h in range(heads) for s in [K[:, h] @ qd[h] / math.sqrt(dim)]])
    assert max_abs_rel(out.float().cpu().numpy()[0].astype(np.float64), full) <= 0.05


def test_workspace_needs_no_initialization_and_is_reusable(gpu_lib):
    # every call rewrites the partials it reads: garbage in a fresh workspace and partials left
    # by earlier calls (also of another shape) never leak into a result
    tokens, heads, dim = 900, 4, 128
    cache = _cache(tokens, heads, dim, seed=3)
    small = _cache(300, heads, dim, seed=4)
    rng = np.random.default_rng(11)
    qs = [bf16_to_bits(round_bf16(rng.standard_normal((2, heads, dim)))) for _ in range(3)]
    ws = torch.full((B.kv_int8_attention_workspace_bytes(2, tokens, heads, dim),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    outs = []
    for i, qb in enumerate(qs + qs):
        c = cache if i % 2 == 0 else small
        o = torch.empty(2, heads, dim, dtype=torch.bfloat16, device="cuda")
        (kq, ks, kz), (vq, vs, vz) = c["K"], c["V"]
        B.kv_int8_attention(dev_bf16(qb), dev(kq), dev(ks), dev(kz), dev(vq), dev(vs), dev(vz),
                            1.0 / math.sqrt(dim), o, ws)   # no synchronization between calls
        outs.append((qb, c, o))
    torch.cuda.synchronize()
    for qb, c, o in outs:
        ref = oka.attention(qb, *c["K"], *c["V"], heads, dim, 1.0 / math.sqrt(dim))
        assert max_abs_rel(o.float().cpu().numpy().astype(np.float64), ref) <= TOL
