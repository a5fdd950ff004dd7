"""The RoPE and SwiGLU C ABIs on the CPU: every contract violation is rejected
before anything is launched (fake device addresses, never dereferenced; the
tests run only where no GPU is visible, as in ``test_abi.py``)."""
import pytest

import row_normalization_amd as rn

OK, E_NULL, E_SHAPE, E_STRIDE, E_ALIGN, E_DTYPE, E_ALIAS = 0, -1, -2, -3, -4, -5, -7
F32, BF16, F16 = 0, 1, 2
GiB = 1 << 30
Q, COS, SIN, POS, E, G, DH, H, DF, DE = (0x7F0000000000 + i * 4 * GiB for i in range(10))


@pytest.fixture(scope="module")
def L():
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")
    return rn.lib()


def rope(L, fn="rope_fwd", q=Q, T=8, H=4, D=128, stride=None, cos=COS, sin=SIN, rows=16, pos=POS, seq=16,
         dtype=BF16):
    return getattr(L, fn)(q, T, H, D, H * D if stride is None else stride, cos, sin, rows, pos, seq, dtype, None)


@pytest.mark.parametrize("fn", ["rope_fwd", "rope_bwd"])
def test_rope_rejections(L, fn):
    assert rope(L, fn, dtype=5) == E_DTYPE
    assert rope(L, fn, T=-1) == E_SHAPE
    assert rope(L, fn, H=0) == E_SHAPE
    assert rope(L, fn, D=127) == E_SHAPE          # odd head_dim
    assert rope(L, fn, D=0) == E_SHAPE
    assert rope(L, fn, D=2048) == E_SHAPE
    assert rope(L, fn, rows=0) == E_SHAPE
    assert rope(L, fn, rows=1 << 23) == E_SHAPE   # table of 2^29 floats
    assert rope(L, fn, pos=None, seq=0) == E_SHAPE
    assert rope(L, fn, pos=None, seq=17) == E_SHAPE  # seq_len beyond the table
    assert rope(L, fn, stride=4 * 128 - 1) == E_STRIDE
    assert rope(L, fn, H=(1 << 24) // 128 + 1) == E_SHAPE   # heads * head_dim > 2^24
    assert rope(L, fn, H=1 << 62, stride=1 << 40) == E_SHAPE  # no overflow in heads * head_dim
    assert rope(L, fn, stride=1 << 61) == E_SHAPE           # byte offsets beyond int64
    # one thread per (token, 4-head group, 16-byte vector): 2^29 tokens of 4
    # heads x 128 bf16 make 2^32 work items, one more than a dispatch holds
    far = dict(q=1 << 44, cos=1 << 45, sin=(1 << 45) + GiB, pos=1 << 46)
    assert rope(L, fn, T=1 << 29, **far) == E_SHAPE
    assert rope(L, fn, T=1 << 29, H=8, **far) == E_SHAPE
    for kw in ("q", "cos", "sin"):
        assert rope(L, fn, **{kw: None}) == E_NULL, kw
    assert rope(L, fn, q=Q + 1) == E_ALIGN
    assert rope(L, fn, cos=COS + 2) == E_ALIGN
    assert rope(L, fn, pos=POS + 1) == E_ALIGN
    assert rope(L, fn, cos=Q + 64) == E_ALIAS         # table inside q
    assert rope(L, fn, pos=Q + 7 * 4 * 128 * 2) == E_ALIAS
    # zero tokens: nothing to do, whatever the pointers
    assert rope(L, fn, T=0, q=None, cos=None, sin=None, pos=None) == OK


def test_swiglu_rejections(L):
    f = lambda e=E, g=G, h=H, M=4, N=8, stride=8, dtype=BF16: L.swiglu_fwd(e, g, h, M, N, stride, dtype, None)
    assert f(dtype=9) == E_DTYPE
    assert f(M=-1) == E_SHAPE
    assert f(N=0) == E_SHAPE
    assert f(N=(1 << 26) + 1, stride=(1 << 26) + 1) == E_SHAPE
    assert f(stride=7) == E_STRIDE
    for kw in ("e", "g", "h"):
        assert f(**{kw: None}) == E_NULL
    assert f(h=H + 1) == E_ALIGN
    assert f(h=E + 2) == E_ALIAS                     # partial overlap with an input
    assert f(M=0, e=None, g=None, h=None) == OK

    b = lambda dh=DH, e=E, g=G, h=H, df=DF, de=DE, M=4, N=8, stride=8, dtype=F16: L.swiglu_bwd(
        dh, e, g, h, df, de, M, N, stride, dtype, None)
    assert b(dtype=3) == E_DTYPE
    assert b(N=0) == E_SHAPE
    assert b(stride=4) == E_STRIDE
    for kw in ("dh", "e", "g", "h", "df", "de"):
        assert b(**{kw: None}) == E_NULL, kw
    assert b(de=DE + 1) == E_ALIGN
    assert b(h=DF) == E_ALIAS                        # two outputs on one buffer
    assert b(df=DE + 4) == E_ALIAS                   # outputs overlapping each other
    assert b(de=G + 2) == E_ALIAS                    # an output partly over an input
    assert b(h=DH, df=E, de=G, g=E + 6) == E_ALIAS   # in place, but g overlaps e (written as df)
    assert b(M=0) == OK


def test_python_bindings_refuse_cpu_tensors():
    import torch

    q = torch.zeros(2, 1, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.rope_fwd(q, torch.ones(4, 2), torch.zeros(4, 2))
    with pytest.raises(ValueError, match="GPU tensors only"):
        rn.swiglu_fwd(q[0], q[0], q[0])
