"""kda_chunk_fwd_cp_noalloc, the variant of kda_chunk_fwd_cp that allocates nothing, against the
workspace variant: two calls in a row on one device, the second smaller than the first, so that
the second runs over summaries the first left in the shared fixed array."""
import pytest
import torch

from linear_attention_chunkwise_amd import inputs
from test_gpu_parity import assert_close

pytestmark = pytest.mark.gpu


def _pair(binding, B, T, H, dk, dv, segments, seed, lengths=None):
    cu = None if lengths is None else inputs.cu_from_lengths(lengths)
    x = inputs.make_prefill_inputs(1 if lengths else B, sum(lengths) if lengths else T, H, dk, dv,
                                   seed=seed, device="cuda", cu_seqlens=cu)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["cu_seqlens"])
    print(f"  noalloc B={B} T={T} H={H} dk={dk} dv={dv} P={segments} lengths={lengths}", flush=True)
    ref_o, ref_S = binding.chunk_fwd_cp(*args, segments=segments, out_dtype=torch.float32)
    o, S = binding.chunk_fwd_cp_noalloc(*args, segments=segments, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("o", o.cpu().numpy(), ref_o.cpu().numpy())
    assert_close("S_T", S.cpu().numpy(), ref_S.cpu().numpy())
    # same kernels, same arguments but the summaries' address: the results agree bit for bit
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S)


def test_noalloc_cp_twice_second_smaller(gpu_lib):
    binding = gpu_lib
    need1 = binding.load().kda_chunk_fwd_cp_workspace_size(2, 4, 128, 128, 4)
    need2 = binding.load().kda_chunk_fwd_cp_workspace_size(3, 2, 64, 64, 3)
    assert 0 < need2 < need1 <= 32 << 20
    _pair(binding, 2, 1000, 4, 128, 128, 4, seed=1)
    _pair(binding, 3, 0, 2, 64, 64, 3, seed=2, lengths=[300, 45, 170])


def test_noalloc_cp_single_segment_and_too_large(gpu_lib):
    binding = gpu_lib
    _pair(binding, 1, 200, 2, 64, 128, 1, seed=3)            # one segment: no summaries at all
    x = inputs.make_prefill_inputs(1, 64, 256, 128, 128, seed=4, device="cuda")
    with pytest.raises(binding.KdaError) as e:                # 256 x 7 summaries of 128 KiB
        binding.chunk_fwd_cp_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"],
                                     segments=8)
    assert e.value.status == binding.KDA_ERR_UNSUPPORTED
