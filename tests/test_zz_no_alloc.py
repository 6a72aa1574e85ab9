"""attn_decode_splitkv_noalloc (library-held scratch, no workspace) through the C ABI, against
attn_decode_splitkv with a caller workspace on the same inputs (the same kernels, so the same bits)
and against the fp64 oracle at the decode tolerances: two calls in a row, the second smaller, so
that the second reads the scratch the first one left behind."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import TOL_BF16_OUT, TOL_LSE, dev, host64, maxerr, say
from transformer_attention_02_amd import synth

pytestmark = pytest.mark.gpu

# (B, Mkv, H, D), splits, seed: 64 x 16 x 32 rows of 128 floats (16.9 MB of scratch), then a
# smaller call with uneven chunks
CASES = [((16, 4096, 32, 128), 64, 41), ((3, 1000, 8, 64), 7, 42)]


def test_noalloc_decode_twice_matches_workspace_decode_and_oracle():
    from transformer_attention_02_amd import attn as A

    for (B, Mkv, H, D), S, seed in CASES:
        say(f"case: noalloc decode B={B} Mkv={Mkv} H={H} D={D} S={S}")
        qh, kh, vh = synth.qkv(seed, (B, 1, H, D), (B, Mkv, H, D), (B, Mkv, H, D), "bf16")
        q, k, v = dev(qh, "bf16"), dev(kh, "bf16"), dev(vh, "bf16")
        out = torch.empty_like(q)
        lse = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
        A.attn_decode_splitkv_noalloc(q, k, v, S, out, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = A.attn_decode_splitkv(q, k, v, S)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "differs from the workspace decode"
        oo, ol = oracle.attention(*(synth.to_f64(x, "bf16") for x in (qh, kh, vh)))
        eo, el = maxerr(host64(out), oo), maxerr(host64(lse), ol)
        say(f"  max|dout|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= TOL_BF16_OUT and el <= TOL_LSE
        # without an lse output
        out2 = torch.empty_like(q)
        A.attn_decode_splitkv_noalloc(q, k, v, S, out2, None)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref_o)


def test_noalloc_decode_refuses_more_than_its_scratch():
    from transformer_attention_02_amd import attn as A

    B, H, D, S = 64, 64, 128, 128  # 268 MB of partials
    assert A.attn_decode_workspace_bytes(B, H, D, S) > A.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 1, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 256, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(A.AttnError, match="bytes of scratch"):
        A.attn_decode_splitkv_noalloc(q, k, k, S, out)
