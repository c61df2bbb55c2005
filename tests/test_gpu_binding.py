"""The binding on a GPU: a host tensor beside device tensors, or a host tensor
with an explicit stream, is refused before any kernel sees a host address;
well-formed calls with caller-supplied outputs and workspaces run."""
import pytest
import torch

import transformer_elementwise_epilogues_amd as mb

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF, F32 = torch.bfloat16, torch.float32
T, H = 16, 128


def d(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def h(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


MIXED = [
    ("gelu host bias", lambda s: mb.mb_bias_gelu_fwd(d(T, H), h(H), stream=s)),
    ("gelu host y, explicit stream", lambda s: mb.mb_bias_gelu_fwd(h(T, H), stream=s)),
    ("gelu host out", lambda s: mb.mb_bias_gelu_fwd(d(T, H), out=h(T, H), stream=s)),
    ("gelu bwd host g", lambda s: mb.mb_bias_gelu_bwd(h(T, H), d(T, H), stream=s)),
    ("gelu bwd host dbias", lambda s: mb.mb_bias_gelu_bwd(d(T, H), d(T, H), dbias=h(H, dtype=F32), stream=s)),
    ("gelu bwd host ws", lambda s: mb.mb_bias_gelu_bwd(d(T, H), d(T, H), ws=h(1 << 20, dtype=torch.uint8),
                                                       stream=s)),
    ("noalloc host bias", lambda s: mb.mb_bias_gelu_bwd_noalloc(d(T, H), d(T, H), h(H), stream=s)),
    ("bda host residual", lambda s: mb.mb_bias_dropout_add_train(d(T, H), None, h(T, H, dtype=F32), 0.1, 1,
                                                                 stream=s)),
    ("bda infer host bias", lambda s: mb.mb_bias_dropout_add_infer(d(T, H), h(H), d(T, H), stream=s)),
    ("bda bwd host dresidual", lambda s: mb.mb_bias_dropout_add_bwd(d(T, H), 0.1, 1, dresidual=h(T, H), stream=s)),
    ("swiglu host weights", lambda s: mb.mb_bias_swiglu_fwd(d(T, 2 * H), None, h(T), stream=s)),
    ("swiglu bwd host g", lambda s: mb.mb_bias_swiglu_bwd(h(T, H), d(T, 2 * H), stream=s)),
    ("geglu host bias", lambda s: mb.mb_bias_geglu_fwd(d(T, 2 * H), h(2 * H), stream=s)),
    ("geglu bwd host din", lambda s: mb.mb_bias_geglu_bwd(d(T, H), d(T, 2 * H), din=h(T, 2 * H), stream=s)),
    ("ln host gamma", lambda s: mb.mb_add_layer_norm_fwd(d(T, H), d(T, H), h(H), stream=s)),
    ("ln bwd host rstd", lambda s: mb.mb_add_layer_norm_bwd(d(T, H), d(T, H), d(H), d(T, dtype=F32),
                                                            h(T, dtype=F32), stream=s)),
    ("srelu host weights", lambda s: mb.mb_weighted_squared_relu_fwd(d(T, H), h(T, dtype=F32), stream=s)),
    ("srelu bwd host x", lambda s: mb.mb_weighted_squared_relu_bwd(d(T, H), h(T, H), stream=s)),
]


@pytest.mark.parametrize("explicit_stream", [False, True])
@pytest.mark.parametrize("case", MIXED, ids=[c[0] for c in MIXED])
def test_host_tensor_beside_device_tensors_is_refused(case, explicit_stream):
    s = torch.cuda.current_stream(DEV) if explicit_stream else None
    with pytest.raises(ValueError):
        case[1](s)
    torch.cuda.synchronize()


def test_caller_supplied_outputs_run():
    y, g = torch.randn(T, H, device=DEV).to(BF), torch.randn(T, H, device=DEV).to(BF)
    out = d(T, H)
    assert mb.mb_bias_gelu_fwd(y, out=out).data_ptr() == out.data_ptr()
    ws = torch.empty(mb.mb_bias_gelu_bwd_workspace(T, H, BF) // 4 + 1, dtype=F32, device=DEV)
    dg, db = mb.mb_bias_gelu_bwd(g, y, dgrad=d(T, H), dbias=d(H, dtype=F32), ws=ws)
    dg2, db2 = mb.mb_bias_gelu_bwd(g, y)
    torch.cuda.synchronize()
    assert torch.equal(dg, dg2) and torch.equal(db, db2)
