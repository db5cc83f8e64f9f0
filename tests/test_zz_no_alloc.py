"""dit_change_score_noalloc, the change score without a workspace, against
dit_change_score (the workspace entry point whose kernels it shares), through
the C ABI: two calls in a row, the second on a smaller input, for both
element types and with and without the in-place update.  The scores must be
bitwise equal (same kernels, same fixed partition of the elements) and the
updated arrays identical.  Also the host-side argument errors (no GPU)."""

import numpy as np
import pytest
import torch

import diffusion_transformer_denoising_dit_amd as D


def _expect_einval(*args):
    with pytest.raises(D.DitError) as e:
        D.dit_change_score_noalloc(*args, stream=0)
    assert e.value.status == 1, e.value


def test_noalloc_argument_errors():
    A, B, S = 1 << 36, 1 << 37, 1 << 38
    _expect_einval(A, B, 5, 16, 0, S)                          # dtype
    _expect_einval(A, B, D.DTYPE_BF16, 0, 0, S)                # n < 1
    _expect_einval(A, B, D.DTYPE_BF16, (1 << 40) + 1, 0, S)    # n beyond the scratch's reach
    _expect_einval(A, B, D.DTYPE_BF16, 16, 2, S)               # update
    _expect_einval(None, B, D.DTYPE_BF16, 16, 0, S)
    _expect_einval(A, B, D.DTYPE_BF16, 16, 0, None)
    _expect_einval(A + 2, B, D.DTYPE_BF16, 16, 0, S)           # alignment
    _expect_einval(A, A + 16, D.DTYPE_F32, 16, 1, S)           # update overlap
    _expect_einval(A, B, D.DTYPE_F32, 16, 0, A + 32)           # score inside cur


def _arrays(n, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = torch.bfloat16 if dtype == D.DTYPE_BF16 else torch.float32
    cur = torch.randn(n, generator=g).to(t).cuda()
    prev = (torch.randn(n, generator=g) * 1.5).to(t).cuda()
    return cur, prev


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [D.DTYPE_BF16, D.DTYPE_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("update", [0, 1])
def test_noalloc_matches_workspace_entry_point_two_calls(dtype, update):
    wsb = D.dit_change_score_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    # a large call (the full grid of partial sums, ragged tail), then a smaller
    # one (fewer partials: the stale ones of the first call must not leak in)
    for i, n in enumerate((3_000_001, 1000 * 8 + 5)):
        cur, prev = _arrays(n, dtype, 100 + i)
        prev_a, prev_b = prev.clone(), prev.clone()
        s_ref = torch.full((1,), -1.0, device="cuda")
        s_new = torch.full((1,), -2.0, device="cuda")
        D.dit_change_score(cur, prev_a, dtype, n, update, s_ref, ws, wsb)
        D.dit_change_score_noalloc(cur, prev_b, dtype, n, update, s_new)
        torch.cuda.synchronize()
        a, b = float(s_ref.item()), float(s_new.item())
        assert np.float32(a).tobytes() == np.float32(b).tobytes(), (n, a, b)
        c64, p64 = cur.double().cpu().numpy(), prev.double().cpu().numpy()
        want = np.abs(c64 - p64).sum() / np.abs(p64).sum()
        assert abs(b - want) <= 1e-5 * want, (n, b, want)
        assert torch.equal(prev_a, prev_b)
        assert torch.equal(prev_b, cur if update else prev)
