"""GPU tests of the device check of a packed batch's cu_seqlens
(``gdr_validate_cu_seqlens``) and of the ``GDR_VALIDATE=1`` hook of the
binding.  Only the check kernel ever sees a broken cu_seqlens: with the hook
on, the binding raises before the forward or backward is launched."""
import pytest
import torch

from chunked_gated_delta_02_amd import _lib, ops

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _first_bad(cu, T):
    """The smallest index whose entry breaks the contract, or -1 (host)."""
    for i, c in enumerate(cu):
        if (i == 0 and c != 0) or (i > 0 and (c < cu[i - 1] or c > T)):
            return i
    return -1


def _device_result(cu, T):
    t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    res = torch.full((1,), 12345, dtype=torch.int32, device=DEV)   # overwritten unconditionally
    _lib.gdr_validate_cu_seqlens(t.data_ptr(), t.numel() - 1, T, res.data_ptr(),
                                 torch.cuda.current_stream(DEV).cuda_stream)
    return int(res.item())


@pytest.mark.parametrize("cu,T", [
    ([0, 5, 5, 100], 100),              # valid, with an empty sequence
    ([0, 100], 100),
    ([0, 0], 0),                        # one empty sequence, no tokens
    ([0, 3, 7], 100),                   # valid: the last entry may stay below T
    ([1, 5, 100], 100),                 # does not start at 0
    ([0, 50, 40, 100], 100),            # decreasing at 2
    ([0, 50, 101, 100], 100),           # an entry past T (and a decrease after it)
    ([0, 10, 20, 130], 128),            # last entry past T
    ([0, -3, 10], 10),                  # negative entry
])
def test_check_matches_the_contract(cu, T):
    assert _device_result(cu, T) == _first_bad(cu, T)


def test_largest_batch_and_a_late_violation():
    rng = torch.Generator().manual_seed(7)
    lens = torch.randint(0, 9, (8192,), generator=rng)
    cu = [0] + torch.cumsum(lens, 0).tolist()
    T = cu[-1]
    assert _device_result(cu, T) == -1
    bad = list(cu)
    bad[6000] = bad[5999] - 1 if bad[5999] > 0 else -1
    bad[7000] = T + 1
    assert _device_result(bad, T) == _first_bad(bad, T) == 6000


def test_binding_raises_with_the_hook_on(monkeypatch):
    T, H, D = 96, 2, 64
    q = torch.randn(1, T, H, D, device=DEV).to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn(1, T, H, D, device=DEV), dim=-1).to(torch.bfloat16)
    v = torch.randn(1, T, H, D, device=DEV).to(torch.bfloat16)
    beta = torch.rand(1, T, H, device=DEV)
    g = -torch.rand(1, T, H, device=DEV)
    good = torch.tensor([0, 40, 96], dtype=torch.int32, device=DEV)
    bad = torch.tensor([0, 60, 40], dtype=torch.int32, device=DEV)
    monkeypatch.setenv("GDR_VALIDATE", "1")
    o, hT, _ = ops.chunk_gdr_fwd(q, k, v, beta, g, cu_seqlens=good)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    with pytest.raises(ValueError, match=r"cu_seqlens\[2\]"):
        ops.chunk_gdr_fwd(q, k, v, beta, g, cu_seqlens=bad)
    with pytest.raises(ValueError, match=r"cu_seqlens\[2\]"):
        ops.chunk_gdr_bwd(q, k, v, beta, g, torch.randn_like(v), cu_seqlens=bad)
    with pytest.raises(ValueError, match=r"cu_seqlens\[2\]"):
        ops.validate_cu_seqlens(bad, T)
