"""The binding's buffer checks: every tensor a call reads or writes must have the dtype and
hold the bytes that the layouts in include/svdq.h give for the call's sizes, and a call with
one buffer an element short, or of another dtype, raises ValueError naming it before anything
reaches the library.

The stand-ins below carry a shape, a dtype and a byte size and claim to be device tensors;
their pointers are never dereferenced, because every call here stops in the checks."""
import math

import pytest
import torch

from bit_post_quantized_amd import binding as B


class Dev:
    """A stand-in for a contiguous device tensor of the given shape and dtype."""

    def __init__(self, shape, dtype, short=False, device="cuda:0", as_dtype=None):
        self.shape = torch.Size(shape)
        self.dtype = as_dtype or dtype
        self._n = math.prod(shape) - (1 if short else 0)
        self.device = torch.device(device)
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def data_ptr(self):
        return 0x10000


bf16, f16, f32, u8, i8, i32 = (torch.bfloat16, torch.float16, torch.float32, torch.uint8,
                               torch.int8, torch.int32)
M, K, N, R = 40, 192, 48, 16
G = K // 64


@pytest.fixture(scope="module", autouse=True)
def lib():
    return B.load()


def _cases():
    e3 = lambda rows: B.svdq_e3m2_bytes(rows, K)  # noqa: E731
    act = dict(X=([M, K], bf16), inv_lambda=([K], f32), L1p=([R, K], bf16),
               x_scales=([M, G], f16), T=([M, R], f32))
    gemm = dict(x_scales=([M, G], f16), T=([M, R], f32), w_scales=([G, N], f16),
                L2p=([N, R], bf16), bias=([N], bf16), Y=([M, N], bf16))
    kv_t, heads, dim = 70, 2, 64
    C = heads * dim
    return [
        (B.svdq_pack_weights, ["R", "wq", "w_scales"],
         dict(R=([K, N], f32), wq=([N, K // 2], u8), w_scales=([G, N], f16)), {}),
        (B.svdq_pack_weights_e3m2, ["R", "wq6", "w_scales"],
         dict(R=([K, N], f32), wq6=([e3(N)], u8), w_scales=([G, N], f16)), {}),
        (B.svdq_pack_lowrank, ["L1", "L1p"], dict(L1=([K, R], bf16), L1p=([R, K], bf16)), {}),
        (B.svdq_pack_lowrank_up, ["L2", "L2p"], dict(L2=([R, N], bf16), L2p=([N, R], bf16)), {}),
        (B.svdq_quantize_act, ["X", "inv_lambda", "L1p", "r", "xq", "x_scales", "T"],
         dict(act, xq=([M, K // 2], u8)), dict(r=R)),
        (B.svdq_quantize_act_e3m2, ["X", "inv_lambda", "L1p", "r", "xq6", "x_scales", "T"],
         dict(act, xq6=([e3(M)], u8)), dict(r=R)),
        (B.svdq_quantize_act_a8, ["X", "inv_lambda", "L1p", "r", "xq8", "x_scales", "T"],
         dict(act, xq8=([M, K], i8)), dict(r=R)),
        (B.svdq_w4a4_gemm, ["xq", "x_scales", "T", "wq", "w_scales", "L2p", "bias", "r", "Y"],
         dict(gemm, xq=([M, K // 2], u8), wq=([N, K // 2], u8)), dict(r=R)),
        (B.svdq_w4a4_gemm_e3m2,
         ["xq6", "x_scales", "T", "wq6", "w_scales", "L2p", "bias", "r", "Y"],
         dict(gemm, xq6=([e3(M)], u8), wq6=([e3(N)], u8)), dict(r=R)),
        (B.svdq_w4a8_gemm, ["xq8", "x_scales", "T", "wq", "w_scales", "L2p", "bias", "r", "Y"],
         dict(gemm, xq8=([M, K], i8), wq=([N, K // 2], u8)), dict(r=R)),
        (B.svdq_w4a4_partials, ["xq", "wq", "P"],
         dict(xq=([M, K // 2], u8), wq=([N, K // 2], u8), P=([G, M, N], i32)), {}),
        (B.svdq_w4a4_partials_e3m2, ["xq6", "wq6", "M", "N", "K", "P"],
         dict(xq6=([e3(M)], u8), wq6=([e3(N)], u8), P=([G, M, N], i32)), dict(M=M, N=N, K=K)),
        (B.svdq_w4a8_partials, ["xq8", "wq", "P"],
         dict(xq8=([M, K], i8), wq=([N, K // 2], u8), P=([G, M, N], i32)), {}),
        (B.kv_int8_quant, ["x", "q", "scale", "zero", "workspace"],
         dict(x=([kv_t, heads, dim], bf16), q=([kv_t, C], u8), scale=([C], f32),
              zero=([C], u8), workspace=([B.kv_int8_workspace_bytes(kv_t, C)], u8)), {}),
        (B.kv_int8_quant_pair, ["k", "v", "qk", "sk", "zk", "qv", "sv", "zv", "workspace"],
         dict(k=([kv_t, heads, dim], bf16), v=([kv_t, heads, dim], bf16), qk=([kv_t, C], u8),
              sk=([C], f32), zk=([C], u8), qv=([kv_t, C], u8), sv=([C], f32), zv=([C], u8),
              workspace=([B.kv_int8_workspace_bytes(kv_t, C)], u8)), {}),
        (B.kv_int8_quant_pair_noalloc, ["k", "v", "qk", "sk", "zk", "qv", "sv", "zv"],
         dict(k=([kv_t, heads, dim], bf16), v=([kv_t, heads, dim], bf16), qk=([kv_t, C], u8),
              sk=([C], f32), zk=([C], u8), qv=([kv_t, C], u8), sv=([C], f32), zv=([C], u8)), {}),
        (B.kv_int8_dequant, ["q", "scale", "zero", "x_out"],
         dict(q=([kv_t, C], u8), scale=([C], f32), zero=([C], u8), x_out=([kv_t, C], bf16)),
         {}),
        (B.kv_int8_attention,
         ["q", "k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "sm_scale", "out",
          "workspace"],
         dict(q=([3, heads, dim], bf16), k_codes=([kv_t, C], u8), k_scale=([C], f32),
              k_zero=([C], u8), v_codes=([kv_t, C], u8), v_scale=([C], f32), v_zero=([C], u8),
              out=([3, heads, dim], bf16),
              workspace=([B.kv_int8_attention_workspace_bytes(3, kv_t, heads, dim)], u8)),
         dict(sm_scale=0.125)),
    ]


def _args(order, tensors, scalars, short=None, retype=None):
    return [scalars[n] if n in scalars else
            Dev(*tensors[n], short=(n == short), as_dtype=_OTHER[tensors[n][1]] if n == retype
                else None)
            for n in order]


# A different dtype of the same width, so that only the dtype check can catch it.
_OTHER = {bf16: f16, f16: bf16, f32: i32, i32: f32, u8: i8, i8: u8}


def _call(fn, order, tensors, scalars, short=None):
    fn(*_args(order, tensors, scalars, short))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0].__name__)
def test_each_short_buffer_is_rejected_by_name(case):
    fn, order, tensors, scalars = case
    for name in tensors:
        with pytest.raises(ValueError, match="holds .* bytes") as e:
            _call(fn, order, tensors, scalars, short=name)
        assert f"{fn.__name__}: {name} holds" in str(e.value), (name, e.value)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0].__name__)
def test_each_wrong_dtype_is_rejected_by_name(case):
    fn, order, tensors, scalars = case
    for name in tensors:
        if name == "workspace":
            continue  # raw bytes: any dtype
        with pytest.raises(ValueError) as e:
            fn(*_args(order, tensors, scalars, retype=name))
        want = ("Y must be bfloat16 or float32" if name == "Y"
                else f"{name} must be {tensors[name][1]}")
        assert f"{fn.__name__}: {want}" in str(e.value), (name, e.value)


def _case(fn):
    return next(c for c in _cases() if c[0] is fn)


@pytest.mark.parametrize("fn,name,bad", [
    (B.svdq_w4a4_gemm, "x_scales", [G, M]),       # group-major instead of [M, K/64]
    (B.svdq_w4a4_gemm_e3m2, "x_scales", [G, M]),
    (B.svdq_w4a4_gemm, "L2p", [R, N]),            # the unpacked factor instead of [N, r]
    (B.svdq_w4a4_gemm_e3m2, "L2p", [R, N]),
    (B.svdq_pack_lowrank_up, "L2p", [R, N]),
    (B.svdq_w4a8_gemm, "T", [R, M]),
    (B.svdq_quantize_act, "x_scales", [G, M]),
    (B.svdq_quantize_act, "L1p", [K, R]),          # the unpacked factor
    (B.svdq_pack_lowrank, "L1p", [K, R]),
])
def test_same_size_wrong_shape_is_rejected(fn, name, bad):
    """A tensor with the right number of bytes but another layout's shape (a transposed factor,
    group-major scales) is rejected: the library could not tell the layouts apart."""
    _, order, tensors, scalars = _case(fn)
    args = _args(order, tensors, scalars)
    args[order.index(name)] = Dev(bad, tensors[name][1])
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        fn(*args)


def test_other_device_and_host_tensors_are_rejected():
    fn, order, tensors, scalars = _case(B.svdq_w4a4_gemm)
    args = _args(order, tensors, scalars)
    args[order.index("Y")] = Dev(*tensors["Y"], device="cuda:1")
    with pytest.raises(ValueError, match="Y is on cuda:1"):
        fn(*args)
    args = _args(order, tensors, scalars)
    args[order.index("bias")] = torch.zeros(N, dtype=bf16)
    with pytest.raises(ValueError, match="bias must be a device tensor"):
        fn(*args)


def test_output_dtype_must_be_bf16_or_fp32():
    fn, order, tensors, scalars = _case(B.svdq_w4a4_gemm)
    args = _args(order, tensors, scalars)
    args[order.index("Y")] = Dev([M, N], f16)
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        fn(*args)
