"""vs_smooth_stats_noalloc (statistics without a caller workspace) against
vs_smooth_stats with one, through the C ABI: two calls in a row on one GPU,
the second with a smaller problem, every output bit-identical."""
import pytest
import torch

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _inputs(B, S, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn(B, S, H, D, generator=g) * 2.0 + 1.0).to(torch.bfloat16)
    v = (torch.randn(B, S, H, D, generator=g) * 3.0 - 0.5).to(torch.bfloat16)
    return k, v


def _run(fn_noalloc, shape, layout, k, v):
    from bit_attention_video_smooth_amd import api
    B, S, H, D = shape
    d = dev()
    nb = (S + 127) // 128
    outs = []
    for noalloc in (False, True):
        km = torch.full((B, H, D), float("nan"), device=d)
        vb = torch.full((B, H, nb, D), float("nan"), device=d)
        vq = torch.full((B, H, D), float("nan"), device=d)
        if noalloc:
            fn_noalloc(k, v, shape, layout, km, vb, vq)
        else:
            ws = torch.empty(api.vs_smooth_stats_workspace_bytes(B, S, H, D), dtype=torch.uint8,
                             device=d)
            api.vs_smooth_stats(k, v, shape, layout, km, vb, vq, ws)
        outs.append((km, vb, vq))
    torch.cuda.synchronize(d)
    return outs


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_noalloc_stats_equal_the_workspace_form_twice(layout):
    import bit_attention_video_smooth_amd as vs
    from bit_attention_video_smooth_amd import api
    d = dev()
    # the live shape (27.9 MiB of block sums: near the 32 MiB limit), then a
    # smaller one with a ragged last block, whose sums land in the part of
    # the array the first call used
    for shape, seed in (((1, 32626, 56, 128), 1), ((2, 1000, 3, 64), 2)):
        B, S, H, D = shape
        k, v = _inputs(B, S, H, D, seed)
        lay = vs.VS_LAYOUT_BSHD
        if layout == "bhsd":
            lay = vs.VS_LAYOUT_BHSD
            k, v = (t.permute(0, 2, 1, 3).contiguous() for t in (k, v))
        k, v = k.to(d), v.to(d)
        print(f"[noalloc] {layout} shape {shape}", flush=True)
        (a_km, a_vb, a_vq), (b_km, b_vb, b_vq) = _run(api.vs_smooth_stats_noalloc, shape, lay, k, v)
        for x, y, name in ((a_km, b_km, "k_mean"), (a_vb, b_vb, "v_block_mean"),
                           (a_vq, b_vq, "v_seq_mean")):
            assert not torch.isnan(x).any(), name
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (shape, name)


def test_noalloc_rejects_problems_past_its_array():
    from bit_attention_video_smooth_amd import api
    from bit_attention_video_smooth_amd._abi import VS_ERR_WORKSPACE, VsError
    d = dev()
    k = torch.zeros(1, 128, 1, 128, dtype=torch.bfloat16, device=d)
    km = torch.empty(1, 1, 128, device=d)
    # S = 115328, H = 56: 103 MB of block sums > 32 MiB; checked on the host
    with pytest.raises(VsError) as e:
        api.vs_smooth_stats_noalloc(k, None, (1, 115328, 56, 128), 0, km, None, None)
    assert e.value.status == VS_ERR_WORKSPACE
