"""Argument checks of the Python binding that need no GPU: misplaced or
mis-shaped tensors raise ValueError before anything reaches the C ABI (whose
device pointers the library cannot check).  Stand-in tensors carry only the
attributes the checks read."""
import pytest
import torch

import deepseek_mla_decode_amd as mla


class Fake:
    def __init__(self, shape, dtype=torch.int32, device="cuda:0", contiguous=True, strides=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contig = contiguous
        self._strides = strides or tuple(int(torch.tensor(self.shape[i + 1:]).prod()) if i + 1 < len(self.shape)
                                         else 1 for i in range(len(self.shape)))

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def stride(self, i=None):
        return self._strides if i is None else self._strides[i]


Q = Fake((4, 128, 512), torch.float16)


@pytest.mark.parametrize("name", ["q_pe", "kv_latent", "k_pe", "block_table", "cache_seqlens", "out", "lse",
                                  "workspace"])
@pytest.mark.parametrize("where", ["cpu", "cuda:1"])
def test_every_tensor_must_be_on_q_nopes_device(name, where):
    tensors = dict(q_pe=Fake((4, 128, 64), torch.float16), kv_latent=Fake((4, 64, 1, 512), torch.float16),
                   k_pe=Fake((4, 64, 1, 64), torch.float16), block_table=None, cache_seqlens=Fake((4,)),
                   out=None, lse=None, workspace=None)
    mla._check_placement(Q, tensors)   # all on cuda:0: fine
    tensors[name] = Fake((4,), device=where)
    with pytest.raises(ValueError, match=name):
        mla._check_placement(Q, tensors)


def test_cache_seqlens_must_have_one_entry_per_sequence():
    mla._check_batch_arrays(4, Fake((4,)), None)
    for bad in (Fake((3,)), Fake((5,)), Fake((4, 1)), Fake((4,), torch.int64), Fake((4,), contiguous=False)):
        with pytest.raises(ValueError):
            mla._check_batch_arrays(4, bad, None)


def test_block_table_needs_a_row_per_sequence():
    lens = Fake((4,))
    mla._check_batch_arrays(4, lens, Fake((4, 16)))
    mla._check_batch_arrays(4, lens, Fake((6, 16)))   # extra rows are never read
    for bad in (Fake((3, 16)), Fake((64,)), Fake((4, 16), torch.int64), Fake((4, 16), strides=(32, 2))):
        with pytest.raises(ValueError):
            mla._check_batch_arrays(4, lens, bad)


def test_host_queries_are_rejected_first():
    q = torch.zeros(2, 16, 512, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        mla.mla_decode(q, torch.zeros(2, 16, 64, dtype=torch.float16), None, None, None,
                       torch.zeros(2, dtype=torch.int32), 1 / 24)
