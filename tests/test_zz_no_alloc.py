"""lmhead_argmax_static (the entry point that allocates nothing: its scratch is
a static device array of the library) against lmhead_argmax with a caller
workspace, through the C ABI: two calls in a row, the second smaller, every
output bit-identical, ids and accepted prefix as the oracle's."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_group_amd import ops, synth
from tests.gpu_util import assert_ids, dev_bf16, dev_i32, dev_u32

pytestmark = pytest.mark.gpu


def test_lmhead_argmax_static_matches_workspace_entry_point():
    for M, V, K, seed in ((8, 20000, 1024, 15001), (3, 3001, 512, 15002)):  # the second call is smaller
        d = synth.lm_head(M=M, V=V, K=K, seed=seed)
        logits_ref, ids_ref, gap, _ = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"])
        draft = ids_ref.copy()
        if M > 1:
            draft[M // 2] = (draft[M // 2] + 1) % V  # planted accepted prefix of M // 2
        x = dev_bf16(d["x"])
        w = (dev_u32(d["codes"]), dev_bf16(d["scales"]), dev_bf16(d["biases"]))
        dr = dev_i32(draft)
        ids_a, acc_a, lg_a = ops.lmhead_argmax(x, *w, draft=dr, want_logits=True)
        ids_b, acc_b, lg_b = ops.lmhead_argmax_static(x, *w, draft=dr, want_logits=True)
        ids_c, acc_c, _ = ops.lmhead_argmax_static(x, *w, draft=dr)  # ids-only path
        torch.cuda.synchronize()
        assert torch.equal(lg_a, lg_b), f"logits differ (M{M} V{V})"
        assert torch.equal(ids_a, ids_b) and torch.equal(ids_a, ids_c), f"ids differ (M{M} V{V})"
        assert int(acc_a.cpu()[0]) == int(acc_b.cpu()[0]) == int(acc_c.cpu()[0])
        assert_ids(ids_b.cpu().numpy(), ids_ref, gap, logits_ref, what=f"static lm head M{M} V{V}")
        lead = 0
        while lead < M and ids_b.cpu().numpy()[lead] == draft[lead]:
            lead += 1
        assert int(acc_b.cpu()[0]) == lead
