"""Host logic of the Python binding that needs no GPU: the checks of
caller-supplied output buffers and workspaces (run before any launch)."""

import pytest
import torch

import exact_io_aware_37_amd as fa


class FakeGPUTensor:
    """Stands in for a CUDA tensor: only the attributes the checks read."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True, is_cuda=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = is_cuda
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous


DEV = torch.device("cuda:0")
SHAPE = (2, 4, 100, 128)


def test_matching_buffer_passes():
    t = FakeGPUTensor(SHAPE, torch.bfloat16)
    assert fa._check_out(t, "out", SHAPE, torch.bfloat16, DEV) is t


@pytest.mark.parametrize("bad, status", [
    (dict(is_cuda=False, device="cpu"), fa.FA_ERR_NULL_PTR),
    (dict(device="cuda:1"), fa.FA_ERR_NULL_PTR),
    (dict(dtype=torch.float16), fa.FA_ERR_DTYPE),
    (dict(dtype=torch.float32), fa.FA_ERR_DTYPE),
    (dict(shape=(2, 4, 99, 128)), fa.FA_ERR_BAD_DIM),
    (dict(shape=(2, 4, 100, 64)), fa.FA_ERR_BAD_DIM),
    (dict(shape=(8, 100, 128)), fa.FA_ERR_BAD_DIM),
    (dict(contiguous=False), fa.FA_ERR_BAD_DIM),
])
def test_bad_buffer_is_rejected(bad, status):
    kw = dict(shape=SHAPE, dtype=torch.bfloat16)
    kw.update(bad)
    with pytest.raises(fa.FAError) as e:
        fa._check_out(FakeGPUTensor(**kw), "out", SHAPE, torch.bfloat16, DEV)
    assert e.value.status == status


def test_real_cpu_tensor_is_rejected():
    with pytest.raises(fa.FAError) as e:
        fa._check_out(torch.empty(SHAPE, dtype=torch.bfloat16), "out", SHAPE, torch.bfloat16,
                      DEV)
    assert e.value.status == fa.FA_ERR_NULL_PTR


def test_lse_must_be_fp32():
    lse_shape = SHAPE[:3]
    with pytest.raises(fa.FAError) as e:
        fa._check_out(FakeGPUTensor(lse_shape, torch.bfloat16), "lse", lse_shape, torch.float32,
                      DEV)
    assert e.value.status == fa.FA_ERR_DTYPE
    fa._check_out(FakeGPUTensor(lse_shape, torch.float32), "lse", lse_shape, torch.float32, DEV)


def test_workspace_checks():
    fa._check_workspace(FakeGPUTensor((4096,), torch.uint8), DEV)
    with pytest.raises(fa.FAError):
        fa._check_workspace(FakeGPUTensor((4096,), torch.uint8, device="cuda:1"), DEV)
    with pytest.raises(fa.FAError):
        fa._check_workspace(FakeGPUTensor((4096,), torch.uint8, contiguous=False), DEV)
    with pytest.raises(fa.FAError):
        fa._check_workspace(torch.empty(4096, dtype=torch.uint8), DEV)


def test_fwd_is_exported_with_keyword_only_options():
    import inspect
    sig = inspect.signature(fa.fwd)
    assert list(sig.parameters)[:3] == ["q", "k", "v"]
    for name in ("causal", "scale"):
        assert sig.parameters[name].kind is inspect.Parameter.KEYWORD_ONLY
