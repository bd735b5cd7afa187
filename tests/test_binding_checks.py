"""The binding refuses tensors that do not match the context before any
library call: a wrong dtype, shape, device or layout would make a kernel read
or write outside the buffers it was given. These cases use CPU tensors and
never reach the library's compute calls."""

import pytest
import torch

from streaming_video_diffusion_amd import binding as B

H, D = 3, 64


@pytest.fixture()
def ctx():
    c = B.PackedContext(H, D, torch.bfloat16, 128, device="cpu")
    c.rows = 100
    return c


def q_of(n=10, dtype=torch.bfloat16, heads=H, d=D):
    return torch.zeros((n, heads, d), dtype=dtype)


def table(n, d=D):
    return torch.zeros((n, d // 2, 2), dtype=torch.float32)


@pytest.mark.parametrize("kwargs,match", [
    (dict(q=q_of(dtype=torch.float32)), "dtype"),
    (dict(q=q_of(heads=H + 1)), "shape"),
    (dict(q=q_of(d=D * 2)), "shape"),
    (dict(q=q_of(), q_rope=table(9)), "q_rope has shape"),
    (dict(q=q_of(), q_rope=table(10).to(torch.float64)), "q_rope has dtype"),
    (dict(q=q_of(), q_rope=table(10).transpose(1, 2).contiguous().transpose(1, 2)), "contiguous"),
    (dict(q=q_of(), out=torch.zeros((10, H, D), dtype=torch.float16)), "out has dtype"),
    (dict(q=q_of(), out=torch.zeros((11, H, D), dtype=torch.bfloat16)), "out has shape"),
    (dict(q=q_of(), q_norm=B.Norm(torch.ones(D + 1))), "elements"),
    (dict(q=q_of(), q_norm=B.Norm(torch.ones(H + 1, D))), "q_norm.weight has shape"),
])
@pytest.mark.parametrize("call", ["sa_forward", "sa_forward_ws"])
def test_forward_rejects(ctx, kwargs, match, call):
    kwargs = dict(kwargs)
    q = kwargs.pop("q")
    with pytest.raises(ValueError, match=match):
        getattr(B, call)(ctx, q, **kwargs)


def test_forward_rejects_other_device(ctx):
    q = q_of().to("meta")
    with pytest.raises(ValueError, match="is on meta"):
        B.sa_forward(ctx, q)


def test_forward_split_rejects(ctx):
    q = q_of()
    with pytest.raises(ValueError, match="partial has shape"):
        B.sa_forward_split(ctx, q, 4, partial=torch.zeros((4, 10, H, D - 1)))
    with pytest.raises(ValueError, match="lse has shape"):
        B.sa_forward_split(ctx, q, 4, lse=torch.zeros((4, 10, H + 1)))
    with pytest.raises(ValueError, match="partial has dtype"):
        B.sa_forward_split(ctx, q, 4, partial=torch.zeros((4, 10, H, D), dtype=torch.float64))
    with pytest.raises(ValueError, match="dtype"):
        B.sa_forward_split(ctx, q_of(dtype=torch.float32), 4)


def test_combine_rejects():
    partial = torch.zeros((4, 10, H, D))
    with pytest.raises(ValueError, match="lse has shape"):
        B.sa_combine_splits(partial, torch.zeros((4, 10, H + 1)))
    with pytest.raises(ValueError, match="partial has dtype"):
        B.sa_combine_splits(partial.double(), torch.zeros((4, 10, H)))
    with pytest.raises(ValueError, match="out has shape"):
        B.sa_combine_splits(partial, torch.zeros((4, 10, H)), out=torch.zeros((10, H, D + 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out has dtype"):
        B.sa_combine_splits(partial, torch.zeros((4, 10, H)), out=torch.zeros((10, H, D), dtype=torch.int32))


def test_pack_rejects(ctx):
    k = torch.zeros((20, H, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="segment 0 k has dtype"):
        B.sa_pack_context(ctx, [(k.float(), k, 0, None)])
    with pytest.raises(ValueError, match="segment 0 v has shape"):
        B.sa_pack_context(ctx, [(k, k[:19], 0, None)])
    with pytest.raises(ValueError, match="segment 1 k has shape"):
        B.sa_pack_context(ctx, [(k, k, 0, None), (torch.zeros((5, H - 1, D), dtype=torch.bfloat16), k[:5], 20, None)])
    with pytest.raises(ValueError, match="rope has 19 rows"):
        B.sa_pack_context(ctx, [(k, k, 0, table(19))])
    with pytest.raises(ValueError, match="rope has shape"):
        B.sa_pack_context(ctx, [(k, k, 0, table(20, D // 2))])
    with pytest.raises(ValueError, match="k_norm.weight has"):
        B.sa_pack_context(ctx, [(k, k, 0, None)], k_norm=B.Norm(torch.ones(D - 2)))
    # a pooled segment's table covers its pooled rows: 2 frames of 4x6 pooled 2x2 -> 12 rows
    kp = torch.zeros((48, H, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rope has 11 rows, the segment packs 12"):
        B.sa_pack_context(ctx, [(kp, kp, 0, table(11), None, (2, 4, 6))])


def test_rope_tables_reject():
    with pytest.raises(ValueError, match="pos has shape"):
        B.sa_make_rope_tables(torch.zeros((5, 2)), D, (16, 24, 24), 10000.0)
    with pytest.raises(ValueError, match="pos has dtype"):
        B.sa_make_rope_tables(torch.zeros((5, 3), dtype=torch.float64), D, (16, 24, 24), 10000.0)
    with pytest.raises(ValueError, match="table has shape"):
        B.sa_make_rope_tables(torch.zeros((5, 3)), D, (16, 24, 24), 10000.0, table=table(4))
