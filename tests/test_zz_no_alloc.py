"""attn_decode_noalloc: the decode entry point that allocates nothing.

Its split records live in the library's fixed device array instead of a
caller workspace.  Checked through the C ABI against attn_decode (the entry
point whose kernels it shares: outputs must agree bit for bit) and against
the fp64 oracle, on two calls in a row, the second with a smaller input, so
that the second call runs on an array that still holds the first call's
records.  Named to be collected last: it changes library state (the array
of this GPU) that no other test depends on.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_attention_close, bits, log, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
lcat = pytest.importorskip("long_context_attention_tiled_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lcat.load_library()


def _run(c, split, kv_head_base):
    args = [to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    st_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_ref, lse_ref = lcat.attn_decode(*args, kv_head_base=kv_head_base, split_tokens=split,
                                      dev_status=st_a)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    lcat.attn_decode_noalloc(*args, kv_head_base=kv_head_base, split_tokens=split, o=o, lse=lse,
                             dev_status=st_b)
    torch.cuda.synchronize()
    assert st_a.item() == 0 and st_b.item() == 0
    return o_ref, lse_ref, o, lse


@pytest.mark.parametrize("split", [0, 256])
def test_noalloc_matches_decode_on_two_calls(split):
    # first call: 9 requests, long and ragged contexts; second: 3 shorter ones
    calls = [dict(seed=700, ctx=[1, 63, 64, 65, 1000, 4097, 9000, 20000, 131], base=2),
             dict(seed=701, ctx=[5, 300, 129], base=0)]
    for i, cl in enumerate(calls):
        log(f"noalloc decode call {i + 1}: split={split} ctx={cl['ctx']}")
        c = synth.decode_cache(seed=cl["seed"], B=len(cl["ctx"]), ctx_lens=cl["ctx"], Hq=16,
                               Hkv=2, kv_head_base=cl["base"], extra_blocks=3)
        o_ref, lse_ref, o, lse = _run(c, split, cl["base"])
        # the same kernels on the same records: identical bits
        assert np.array_equal(bits(o), bits(o_ref))
        assert np.array_equal(lse.cpu().numpy().view(np.uint32),
                              lse_ref.cpu().numpy().view(np.uint32))
        ref, ref_lse = oracle.decode_attention(c["q"], c["k_seq"], c["v_seq"], c["ctx_len"],
                                               c["scale"])
        e, r = assert_attention_close(to_np64(o), ref, lse.cpu().numpy(), ref_lse,
                                      what=f"noalloc decode call {i + 1}")
        log(f"  max abs {e:.3g} rel-L2 {r:.3g}")


def test_noalloc_empty_request_and_size_limit():
    """A request with no context gives o = 0, lse = -inf, as attn_decode; a
    call needing more records than the array holds is refused up front."""
    c = synth.decode_cache(seed=702, B=3, ctx_lens=[0, 70, 2], Hq=16, Hkv=2)
    o_ref, lse_ref, o, lse = _run(c, 0, 0)
    assert np.array_equal(bits(o), bits(o_ref))
    assert not to_np64(o)[0].any() and np.isneginf(lse.cpu().numpy()[0]).all()
    args = [to_dev(c[k]) for k in ("q", "k_pool", "v_pool", "block_head", "block_table", "ctx_len")]
    with pytest.raises(lcat.AttnError) as ei:
        big = torch.zeros((2000, 16, 128), dtype=torch.bfloat16, device="cuda")
        lcat.attn_decode_noalloc(big, *args[1:3], args[3],
                                 torch.zeros((2000, 2, args[4].shape[2]), dtype=torch.int32,
                                             device="cuda"),
                                 torch.zeros(2000, dtype=torch.int32, device="cuda"))
    assert ei.value.status == 8
