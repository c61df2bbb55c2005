"""The Python binding refuses bad tensor arguments before any library call.

The C ABI only sees pointers and (tokens, hidden), so the binding must catch
what a pointer cannot carry: a host tensor handed to a kernel, a secondary
input or a caller-supplied output of the wrong shape or dtype, a
non-contiguous view. These tests need no GPU: host tensors are refused as
such, and, with the device checks stubbed to accept host tensors, every other
rule is exercised against a stand-in library that fails the test if any entry
point is reached."""
import pytest
import torch

import transformer_elementwise_epilogues_amd as mb

BF, F32 = torch.bfloat16, torch.float32
T, H = 8, 64


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


class NoEntryLib:
    """Answers workspace queries; any entry point call fails the test."""

    def __getattr__(self, name):
        if name.endswith("_workspace"):
            return lambda *a: 256
        if name == "mb_status_string":
            return lambda code: b"MB_?"

        def entry(*a):
            raise AssertionError(f"{name} reached the library with bad arguments")
        return entry


@pytest.fixture
def host_as_gpu(monkeypatch):
    """Device checks accept host tensors; the library is the stand-in."""
    monkeypatch.setattr(mb, "lib", lambda: NoEntryLib())
    monkeypatch.setattr(mb, "_gpu", lambda stream, *named: torch.device("cpu"))
    monkeypatch.setattr(mb, "_on", lambda dev, name, t: t)


# Every entry point called with well-formed host tensors: refused as host memory.
GOOD_CALLS = {
    "gelu_fwd": lambda: mb.mb_bias_gelu_fwd(z(T, H), z(H)),
    "gelu_erf_fwd": lambda: mb.mb_bias_gelu_erf_fwd(z(T, H), z(H)),
    "gelu_bwd": lambda: mb.mb_bias_gelu_bwd(z(T, H), z(T, H), z(H)),
    "gelu_erf_bwd": lambda: mb.mb_bias_gelu_erf_bwd(z(T, H), z(T, H), z(H)),
    "gelu_bwd_noalloc": lambda: mb.mb_bias_gelu_bwd_noalloc(z(T, H), z(T, H), z(H)),
    "bda_train": lambda: mb.mb_bias_dropout_add_train(z(T, H), z(H), z(T, H, dtype=F32), 0.1, 1),
    "bda_infer": lambda: mb.mb_bias_dropout_add_infer(z(T, H), z(H), z(T, H)),
    "bda_bwd": lambda: mb.mb_bias_dropout_add_bwd(z(T, H), 0.1, 1),
    "mask": lambda: mb.mb_dropout_mask(T, H, 0.1, 1, out=torch.zeros(T * H // 8, dtype=torch.uint8)),
    "mask_host_device": lambda: mb.mb_dropout_mask(T, H, 0.1, 1, device="cpu"),
    "swiglu_fwd": lambda: mb.mb_bias_swiglu_fwd(z(T, 2 * H), z(2 * H), z(T)),
    "swiglu_bwd": lambda: mb.mb_bias_swiglu_bwd(z(T, H), z(T, 2 * H), z(2 * H), z(T)),
    "geglu_fwd": lambda: mb.mb_bias_geglu_fwd(z(T, 2 * H), z(2 * H)),
    "geglu_bwd": lambda: mb.mb_bias_geglu_bwd(z(T, H), z(T, 2 * H), z(2 * H)),
    "ln_fwd": lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T, H), z(H), z(H)),
    "ln_bwd": lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32), z(T, dtype=F32)),
    "srelu_fwd": lambda: mb.mb_weighted_squared_relu_fwd(z(T, H), z(T, dtype=F32)),
    "srelu_bwd": lambda: mb.mb_weighted_squared_relu_bwd(z(T, H), z(T, H), z(T, dtype=F32)),
}


@pytest.mark.parametrize("name", sorted(GOOD_CALLS))
def test_host_tensors_are_refused(name):
    with pytest.raises(ValueError, match="GPU|cuda"):
        GOOD_CALLS[name]()


def test_every_entry_point_has_a_host_tensor_case():
    covered = {"mb_bias_gelu_fwd", "mb_bias_gelu_erf_fwd", "mb_bias_gelu_bwd", "mb_bias_gelu_erf_bwd",
               "mb_bias_gelu_bwd_noalloc", "mb_bias_dropout_add_train", "mb_bias_dropout_add_infer",
               "mb_bias_dropout_add_bwd", "mb_dropout_mask", "mb_bias_swiglu_fwd", "mb_bias_swiglu_bwd",
               "mb_bias_geglu_fwd", "mb_bias_geglu_bwd", "mb_add_layer_norm_fwd", "mb_add_layer_norm_bwd",
               "mb_weighted_squared_relu_fwd", "mb_weighted_squared_relu_bwd"}
    # (the test-only team-wait setter takes no tensor)
    entry = {n for n in mb.__all__ if n.startswith("mb_") and not n.endswith("_workspace")
             and n != "mb_set_layer_norm_team_wait"}
    assert entry == covered


# With the device checks stubbed: each bad argument is refused by the binding.
BAD_CALLS = [
    # secondary inputs: rows, columns, dtype, layout
    ("gelu bwd g rows", lambda: mb.mb_bias_gelu_bwd(z(T - 1, H), z(T, H))),
    ("gelu bwd g dtype", lambda: mb.mb_bias_gelu_bwd(z(T, H, dtype=F32), z(T, H))),
    ("gelu bias length", lambda: mb.mb_bias_gelu_fwd(z(T, H), z(H + 8))),
    ("gelu bias dtype", lambda: mb.mb_bias_gelu_fwd(z(T, H), z(H, dtype=F32))),
    ("gelu y not contiguous", lambda: mb.mb_bias_gelu_fwd(z(H, T).t())),
    ("gelu y 1-D", lambda: mb.mb_bias_gelu_fwd(z(T * H))),
    ("gelu y float64", lambda: mb.mb_bias_gelu_fwd(z(T, H, dtype=torch.float64))),
    ("bda residual rows", lambda: mb.mb_bias_dropout_add_train(z(T, H), None, z(T - 1, H), 0.1, 1)),
    ("bda residual fp16 beside bf16", lambda: mb.mb_bias_dropout_add_infer(z(T, H), None,
                                                                            z(T, H, dtype=torch.float16))),
    ("swiglu g rows", lambda: mb.mb_bias_swiglu_bwd(z(T - 1, H), z(T, 2 * H))),
    ("swiglu g columns", lambda: mb.mb_bias_swiglu_bwd(z(T, 2 * H), z(T, 2 * H))),
    ("swiglu weights length", lambda: mb.mb_bias_swiglu_fwd(z(T, 2 * H), None, z(T + 1))),
    ("swiglu weights fp16 beside bf16", lambda: mb.mb_bias_swiglu_fwd(z(T, 2 * H), None,
                                                                       z(T, dtype=torch.float16))),
    ("glu odd columns", lambda: mb.mb_bias_geglu_fwd(z(T, 2 * H + 1))),
    ("ln gamma missing", lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T, H), None)),
    ("ln residual rows", lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T + 1, H), z(H))),
    ("ln mean dtype", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T), z(T, dtype=F32))),
    ("ln rstd rows", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32),
                                                      z(T - 1, dtype=F32))),
    ("ln dh_in rows", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32),
                                                       z(T, dtype=F32), dh_in=z(T - 1, H))),
    ("srelu g rows", lambda: mb.mb_weighted_squared_relu_bwd(z(T - 1, H), z(T, H))),
    ("srelu weights rows", lambda: mb.mb_weighted_squared_relu_fwd(z(T, H), z(T - 1, dtype=F32))),
    # caller-supplied outputs and buffers
    ("gelu out dtype", lambda: mb.mb_bias_gelu_fwd(z(T, H), out=z(T, H, dtype=F32))),
    ("gelu out rows", lambda: mb.mb_bias_gelu_fwd(z(T, H), out=z(T - 1, H))),
    ("gelu dgrad rows", lambda: mb.mb_bias_gelu_bwd(z(T, H), z(T, H), dgrad=z(T - 1, H))),
    ("gelu dbias length", lambda: mb.mb_bias_gelu_bwd(z(T, H), z(T, H), dbias=z(H - 4, dtype=F32))),
    ("gelu dbias dtype", lambda: mb.mb_bias_gelu_bwd(z(T, H), z(T, H), dbias=z(H))),
    ("noalloc dbias length", lambda: mb.mb_bias_gelu_bwd_noalloc(z(T, H), z(T, H), dbias=z(H + 4, dtype=F32))),
    ("gelu ws not a tensor", lambda: mb.mb_bias_gelu_bwd(z(T, H), z(T, H), ws=bytearray(64))),
    ("bda out dtype", lambda: mb.mb_bias_dropout_add_train(z(T, H), None, z(T, H), 0.1, 1, out=z(T, H, dtype=F32))),
    ("bda bwd dx rows", lambda: mb.mb_bias_dropout_add_bwd(z(T, H), 0.1, 1, dx=z(T + 1, H))),
    ("bda bwd dresidual dtype", lambda: mb.mb_bias_dropout_add_bwd(z(T, H), 0.1, 1, residual_dtype=F32,
                                                                   dresidual=z(T, H))),
    ("bda bwd residual dtype", lambda: mb.mb_bias_dropout_add_bwd(z(T, H), 0.1, 1, residual_dtype=torch.float16)),
    ("bda bwd dbias length", lambda: mb.mb_bias_dropout_add_bwd(z(T, H), 0.1, 1, dbias=z(H + 8, dtype=F32))),
    ("mask out size", lambda: mb.mb_dropout_mask(T, H, 0.1, 1, out=torch.zeros(T * H // 8 - 1, dtype=torch.uint8))),
    ("mask out dtype", lambda: mb.mb_dropout_mask(T, H, 0.1, 1, out=z(T * H // 8))),
    ("swiglu out columns", lambda: mb.mb_bias_swiglu_fwd(z(T, 2 * H), out=z(T, 2 * H))),
    ("swiglu din columns", lambda: mb.mb_bias_swiglu_bwd(z(T, H), z(T, 2 * H), din=z(T, H))),
    ("swiglu dbias length", lambda: mb.mb_bias_swiglu_bwd(z(T, H), z(T, 2 * H), dbias=z(H, dtype=F32))),
    ("swiglu dweights length", lambda: mb.mb_bias_swiglu_bwd(z(T, H), z(T, 2 * H), None, z(T),
                                                             dweights=z(T + 1, dtype=F32))),
    ("geglu din dtype", lambda: mb.mb_bias_geglu_bwd(z(T, H), z(T, 2 * H), din=z(T, 2 * H, dtype=F32))),
    ("ln y rows", lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T, H), z(H), y=z(T - 1, H))),
    ("ln h_out dtype", lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T, H), z(H), h_out=z(T, H, dtype=F32))),
    ("ln stats rows", lambda: mb.mb_add_layer_norm_fwd(z(T, H), z(T, H), z(H),
                                                       stats=(z(T, dtype=F32), z(T + 1, dtype=F32)))),
    ("ln dx dtype", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32), z(T, dtype=F32),
                                                     dx=z(T, H, dtype=F32))),
    ("ln dresidual dtype", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32),
                                                            z(T, dtype=F32), dresidual=z(T, H, dtype=F32))),
    ("ln dgamma length", lambda: mb.mb_add_layer_norm_bwd(z(T, H), z(T, H), z(H), z(T, dtype=F32), z(T, dtype=F32),
                                                          dgamma=z(H - 1, dtype=F32))),
    ("srelu dx rows", lambda: mb.mb_weighted_squared_relu_bwd(z(T, H), z(T, H), dx=z(T - 1, H))),
    ("srelu dweights dtype", lambda: mb.mb_weighted_squared_relu_bwd(z(T, H), z(T, H), z(T, dtype=F32),
                                                                     dweights=z(T))),
]


@pytest.mark.parametrize("case", BAD_CALLS, ids=[c[0] for c in BAD_CALLS])
def test_bad_arguments_are_refused(host_as_gpu, case):
    with pytest.raises(ValueError):
        case[1]()


def test_device_rule_names_the_tensor():
    """The real device check: the first host tensor is named."""
    with pytest.raises(ValueError, match="bias must be a GPU tensor"):
        mb._gpu(None, ("bias", z(H)))
    assert mb._gpu(None, ("bias", None)) is None
