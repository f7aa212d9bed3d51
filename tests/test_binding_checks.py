"""The Python binding checks every tensor's shape, dtype and device against the others before it
allocates or calls the library (the C ABI takes plain pointers and cannot check sizes).  CPU only:
every case is rejected before any device memory is touched."""
import pytest
import torch

saf = pytest.importorskip("fixed_pattern_mixed_amd")

B, H, HKV, T, D = 2, 4, 2, 16, 64
BF = torch.bfloat16


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def good():
    return dict(q=t(B, H, T, D), k=t(B, HKV, T, D), v=t(B, HKV, T, D), o=t(B, H, T, D),
                dout=t(B, H, T, D), lse=t(B, H, T, dtype=torch.float32),
                a=t(H, T, dtype=torch.float32), r=t(H, T, dtype=torch.float32),
                replaced=[0, 1, 0, 1])


def call_fwd(x):
    return saf.fwd(x["q"], x["k"], x["v"], x["replaced"], x["a"], x["r"],
                   out=x.get("out"), lse=x.get("lse_out"))


def call_bwd(x):
    return saf.bwd(x["q"], x["k"], x["v"], x["o"], x["dout"], x["lse"], x["replaced"], x["a"],
                   x["r"])


FWD_BAD = [
    ("q", t(B, H, T, D, dtype=torch.float32), "dtype"),   # fp32 q with bf16 v: twice the bytes
    ("q", t(B, H, T + 1, D), "shape"),
    ("k", t(B, H, T, D), "shape"),                        # k must have Hkv heads like v
    ("k", t(B, HKV, T, D, dtype=torch.float32), "dtype"),
    ("a", t(H, T - 1, dtype=torch.float32), "pat_len"),   # pattern shorter than T
    ("a", t(H, T, dtype=BF), "dtype"),
    ("r", t(H, T + 3, dtype=torch.float32), "shape"),     # r must match a
    ("a", None, "required"),
    ("out", t(B, H, T, D, dtype=torch.float32), "dtype"), # fp32 out for bf16 inputs
    ("lse_out", t(B, H, T, dtype=BF), "dtype"),
]


@pytest.mark.parametrize("name,value,msg", FWD_BAD, ids=["%s-%s" % (c[0], c[2]) for c in FWD_BAD])
def test_forward_binding_rejects(name, value, msg):
    x = good()
    x[name] = value
    with pytest.raises(ValueError, match=msg):
        call_fwd(x)


BWD_BAD = [
    ("dout", t(B, H, T, D, dtype=torch.float32), "dtype"),
    ("o", t(B, HKV, T, D), "shape"),
    ("o", None, "required"),
    ("lse", t(B, H, T + 1, dtype=torch.float32), "shape"),
    ("lse", t(B, H, T), "dtype"),                          # bf16 lse: half the bytes
    ("q", t(B, H, T, 128), "shape"),
    ("r", t(H, T, dtype=torch.float64), "dtype"),
]


@pytest.mark.parametrize("name,value,msg", BWD_BAD, ids=["%s-%s" % (c[0], c[2]) for c in BWD_BAD])
def test_backward_binding_rejects(name, value, msg):
    x = good()
    x[name] = value
    with pytest.raises(ValueError, match=msg):
        call_bwd(x)


def test_all_replaced_forward_needs_no_q_k():
    """With every head replaced q and k may be None; the call then fails only because these CPU
    tensors are not on the GPU."""
    x = good()
    with pytest.raises(ValueError, match="GPU"):
        saf.fwd(None, None, x["v"], [1] * H, x["a"], x["r"])


def test_valid_cpu_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        call_fwd(good())
    with pytest.raises(ValueError, match="GPU"):
        call_bwd(good())


def test_pattern_gradient_and_calibrate_checks():
    x = good()
    v = t(B, H, T, D)
    with pytest.raises(ValueError, match="shape"):
        saf.bwd_pattern(v, t(B, H, T, 128), x["dout"], x["lse"], x["replaced"], x["a"], x["r"])
    with pytest.raises(ValueError, match="dtype"):
        saf.bwd_pattern(v, x["o"], x["dout"], x["lse"], x["replaced"], x["a"], x["r"],
                        da=t(H, T))
    with pytest.raises(ValueError, match="dtype"):
        saf.calibrate(t(3, H, T, D), t(3, H, T, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        saf.calibrate(t(3, H, T, D), t(2, H, T, D))
    with pytest.raises(ValueError, match="dtype"):
        saf.fit_pattern(t(H, T, T))
    with pytest.raises(ValueError, match="uint8"):
        saf.fwd(x["q"], x["k"], x["v"], x["replaced"], x["a"], x["r"], pattern=t(8))
