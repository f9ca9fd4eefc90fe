"""csa2_group_step_static (the group step on the library's own scratch array)
against csa2_group_step with a caller workspace, through the C ABI.

Two calls in a row on the static scratch - a Full group over two sequences,
then a smaller one (one sequence, shorter cache, fewer layers) - each compared
with csa2_group_step on the same inputs: pool, Top-K list, scores, every
layer's output and lse must be identical (same kernels, same inputs).  A
group whose workspace exceeds the scratch is refused before any work.
"""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
from tests._gpu_util import announce, dev, h, random_group as _group, t

pytestmark = pytest.mark.gpu


def _compare(outputs, label):
    g_ws, ref = outputs()
    ws = torch.zeros((csa2.csa2_group_workspace_size(g_ws),), dtype=torch.uint8, device=dev())
    announce("group step with workspace", label)
    csa2.csa2_group_step(g_ws, ws)
    g_st, got = outputs()
    announce("group step on the static scratch", label)
    csa2.csa2_group_step_static(g_st)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert np.array_equal(h(a), h(b), equal_nan=True), label


def test_static_scratch_matches_workspace_two_calls():
    _compare(_group(601, [70000, 33333], 3), "two sequences, 3 layers")
    # the second call is smaller: the scratch keeps the first call's contents
    _compare(_group(602, [9000], 2), "one sequence, 2 layers")


def test_static_scratch_refuses_oversized_group():
    outputs = _group(603, [4096], 1)
    g, _ = outputs()
    need = csa2.csa2_group_workspace_size(g)
    assert need <= csa2.CSA2_STATIC_SCRATCH_BYTES
    # a flat prefill-sized group needs more than the scratch holds: refused on the host
    lens = [65536]
    M = 4096
    kv_c = torch.zeros((8, 256), dtype=torch.uint8, device=dev())
    kv_s = torch.zeros((8, 32), dtype=torch.uint8, device=dev())
    st, ln = t(np.zeros(1, np.int64)), t(np.asarray(lens, np.int32))
    kv = csa2.fp4_cache(kv_c, kv_s, st, ln, 512, lens[0], 2)
    ik = csa2.fp4_cache(kv_c[:, :64], kv_s[:, :8], st, ln, 128, lens[0], 2)
    qs = csa2.queries(torch.zeros(M, dtype=torch.int32, device=dev()), torch.zeros(M, dtype=torch.int32, device=dev()))
    q = torch.zeros((M, 64, 512), dtype=torch.bfloat16, device=dev())
    sw = csa2.swa(torch.zeros((16, 512), dtype=torch.uint8, device=dev()), torch.ones(16, device=dev()),
                  torch.zeros(M, dtype=torch.int32, device=dev()), torch.zeros(M, dtype=torch.int32, device=dev()),
                  512, 128)
    big = csa2.Group(csa2.CSA2_MODE_FULL, kv, ik, qs, torch.zeros((M, 8, 128), dtype=torch.bfloat16, device=dev()),
                     torch.zeros((M, 8), device=dev()), 0, 512, None, None,
                     torch.zeros((M, 512), dtype=torch.int32, device=dev()), None, [q], csa2.CSA2_BF16, 64, [sw],
                     [torch.zeros((M, 64, 512), device=dev())], None, 512 ** -0.5)
    assert csa2.csa2_group_workspace_size(big) > csa2.CSA2_STATIC_SCRATCH_BYTES
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_group_step_static(big)
    assert e.value.status == -5
