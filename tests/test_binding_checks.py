"""CPU: the binding rejects output buffers that do not fit what the kernels
write (a buffer with too few rows would be written past its end)."""
import pytest
import torch

from sparse_attention_token_absorb_amd import binding as B

Q, K, KI, MV = 3, 16, 4, 100


def good():
    i = lambda *s: torch.zeros(s, dtype=torch.int32)
    return B.TopK(i(Q, K), i(Q), i(Q, KI), i(Q), torch.zeros((Q, MV), dtype=torch.float32))


def test_matching_buffers_pass():
    assert B.topk_out_problem(good(), Q, K, KI, MV) is None
    o = good()
    o.idx_inner = o.count_inner = None
    assert B.topk_out_problem(o, Q, K, 0, MV) is None
    o.scores = torch.zeros((Q, MV + 7), dtype=torch.float32)  # a wider stride is fine
    assert B.topk_out_problem(o, Q, K, 0, MV) is None


@pytest.mark.parametrize("field,value", [
    ("idx", torch.zeros((Q, K - 1), dtype=torch.int32)),
    ("idx", torch.zeros((Q - 1, K), dtype=torch.int32)),
    ("idx", torch.zeros((Q, K), dtype=torch.int64)),
    ("count", torch.zeros((Q + 1,), dtype=torch.int32)),
    ("idx_inner", torch.zeros((Q, KI + 1), dtype=torch.int32)),
    ("idx_inner", torch.zeros((Q, KI), dtype=torch.float32)),
    ("idx_inner", None),
    ("count_inner", torch.zeros((Q - 1,), dtype=torch.int32)),
    ("count_inner", None),
    ("scores", torch.zeros((Q, MV - 1), dtype=torch.float32)),
    ("scores", torch.zeros((Q - 1, MV), dtype=torch.float32)),
    ("scores", torch.zeros((Q * MV,), dtype=torch.float32)),
    ("scores", torch.zeros((Q, MV), dtype=torch.float64)),
])
def test_each_mismatch_is_reported(field, value):
    o = good()
    setattr(o, field, value)
    assert B.topk_out_problem(o, Q, K, KI, MV), (field, value)
    with pytest.raises(ValueError):
        B._check_topk_out(o, Q, K, KI, MV, torch.device("cpu"))
