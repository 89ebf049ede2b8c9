"""The Python binding refuses tensors the library could not use safely, before any call
into it: host tensors, outputs of the wrong shape, dtype, layout or device, and
workspaces that are not contiguous device memory. (A host pointer or an undersized
buffer handed to a kernel would be a bad device address, not an error code.)

The first test needs no GPU; the others build GPU tensors but launch nothing, since
every case fails in Python before the library is called.
"""
import pytest
import torch

import exact_attention_forward_fwd_amd as fa


def test_host_tensors_are_refused_without_a_gpu():
    q = torch.zeros((1, 2, 8, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fwd_ex(q, q, q)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fwd_split(q, q, q, num_splits=2)
    lse = torch.zeros((1, 2, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, q, lse)
    with pytest.raises(ValueError):
        fa.bwd_ex(q, q, q, q, q, lse)


@pytest.fixture
def gpu_inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 4, 64, 64), dtype=torch.float16, device=dev)
    kv = torch.zeros((1, 2, 64, 64), dtype=torch.float16, device=dev)
    return dev, q, kv


@pytest.mark.gpu
def test_forward_outputs_are_checked(gpu_inputs):
    dev, q, _ = gpu_inputs
    cases = [
        dict(out=torch.empty_like(q).cpu()),                                   # host output
        dict(out=torch.empty_like(q, dtype=torch.bfloat16)),                   # wrong dtype
        dict(out=torch.empty((1, 4, 64, 32), dtype=q.dtype, device=dev)),      # wrong shape
        dict(out=torch.empty((1, 4, 64, 128), dtype=q.dtype, device=dev)[..., :64]),   # not contiguous
        dict(lse=torch.empty((1, 4, 63), dtype=torch.float32, device=dev)),    # wrong shape
        dict(lse=torch.empty((1, 4, 64), dtype=torch.float16, device=dev)),    # wrong dtype
        dict(lse=torch.empty((1, 4, 64), dtype=torch.float32)),                # host
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            fa.fwd(q, q, q, **kw)
    with pytest.raises(ValueError):
        fa.fwd(q, q.cpu(), q)                                                  # k on the host


@pytest.mark.gpu
def test_general_outputs_and_workspaces_are_checked(gpu_inputs):
    dev, q, kv = gpu_inputs
    for kw in (dict(out=torch.empty_like(q, dtype=torch.bfloat16)), dict(out=torch.empty_like(q).cpu()),
               dict(lse=torch.empty((1, 4, 64), dtype=torch.float16, device=dev))):
        with pytest.raises(ValueError):
            fa.fwd_ex(q, kv, kv, **kw)
        with pytest.raises(ValueError):
            fa.fwd_split(q, kv, kv, num_splits=2, **kw)
    need = fa.fa_split_workspace_bytes(1, 4, 64, 64, 2)
    with pytest.raises(ValueError):
        fa.fwd_split(q, kv, kv, num_splits=2, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fa.fwd_split(q, kv, kv, num_splits=2,
                     workspace=torch.empty(2 * need, dtype=torch.uint8, device=dev)[::2])


@pytest.mark.gpu
def test_backward_outputs_and_workspaces_are_checked(gpu_inputs):
    dev, q, kv = gpu_inputs
    lse = torch.zeros((1, 4, 64), dtype=torch.float32, device=dev)
    for kw in (dict(dq=torch.empty_like(q).cpu()), dict(dk=torch.empty((1, 4, 32, 64), dtype=q.dtype, device=dev)),
               dict(dv=torch.empty_like(q, dtype=torch.bfloat16)),
               dict(workspace=torch.empty(1 << 16, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            fa.bwd(q, q, q, q, q, lse, **kw)
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, q, lse.cpu())
    # grouped heads: dk and dv are shaped like k, not like q
    with pytest.raises(ValueError):
        fa.bwd_ex(q, kv, kv, q, q, lse, dk=torch.empty_like(q))
    with pytest.raises(ValueError):
        fa.bwd_ex(q, kv, kv, q, q, lse, dq=torch.empty_like(kv))
