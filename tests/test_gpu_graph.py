"""HIP-graph capture of a decode step built from the library's entry points:
every replay (with other eager calls on the same stream between replays,
which reuse the stream's workspace) must reproduce the eager results bit for
bit.  The entry points launch kernels only (no memset nodes, no allocation
once the stream's workspace exists), so they can be captured."""
import pytest
import torch

from bit_quantized_decode_group_amd import ops, synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, dev_u8, dev_u32

pytestmark = pytest.mark.gpu


def _step_inputs(M, seed):
    blk = synth.mlp_block(M=M, D=1024, I=1536, seed=seed)
    moe = synth.moe_token(E=16, D=512, I=256, top_k=4, seed=seed + 1, n_logit_sets=2)
    lm = synth.lm_head(M=M, V=4000, K=512, seed=seed + 2)
    gu = ops.tile_pack(dev_u32(blk["codes_gu"]), dev_bf16(blk["scales_gu"]), dev_bf16(blk["biases_gu"]))
    dn = ops.tile_pack(dev_u32(blk["codes_d"]), dev_bf16(blk["scales_d"]), dev_bf16(blk["biases_d"]))
    lmt = ops.tile_pack(dev_u32(lm["codes"]), dev_bf16(lm["scales"]), dev_bf16(lm["biases"]))
    return {
        "x": dev_bf16(blk["x"]), "gamma": dev_bf16(blk["gamma"]), "eps": blk["eps"], "I": blk["I"], "D": blk["D"],
        "gu": gu, "dn": dn, "lm": lmt, "V": lm["V"], "xl": dev_bf16(lm["x"]), "draft": dev_i32(lm["draft"][:M]),
        "xm": dev_bf16(moe["x"]), "logits": dev_f32(moe["logits"]), "w_gu": dev_u8(moe["w_gu"]),
        "w_down": dev_u8(moe["w_down"]), "top_k": moe["top_k"],
    }


def _outputs(M, t, dev):
    return {
        "h": torch.empty((M, t["I"]), dtype=torch.bfloat16, device=dev),
        "y": torch.empty((M, t["D"]), dtype=torch.bfloat16, device=dev),
        "ym": torch.empty((1, t["xm"].shape[1]), dtype=torch.bfloat16, device=dev),
        "mids": torch.empty(t["top_k"], dtype=torch.int32, device=dev),
        "mw": torch.empty(t["top_k"], dtype=torch.float32, device=dev),
        "ids": torch.empty(M, dtype=torch.int32, device=dev),
        "acc": torch.empty(1, dtype=torch.int32, device=dev),
        "lg": torch.empty((M, t["V"]), dtype=torch.float32, device=dev),
    }


def _step(t, o, which):
    ops.rmsnorm_gateup_swiglu_tiled(t["x"], t["gamma"], t["eps"], *t["gu"], t["I"], h=o["h"])
    ops.qgemv_affine4_tiled(o["h"], *t["dn"], t["D"], y=o["y"])
    ops.moe_expert_qgemv(t["xm"], t["logits"][which], t["top_k"], t["w_gu"], t["w_down"], y=o["ym"],
                         out_ids=o["mids"], out_w=o["mw"])
    ops.lmhead_argmax_tiled(t["xl"], *t["lm"], t["V"], draft=t["draft"], logits=o["lg"], ids=o["ids"],
                            accepted=o["acc"])


@pytest.mark.parametrize("M", [8, 1])
def test_graph_replay_equals_eager(M):
    dev = torch.device("cuda:0")
    t = _step_inputs(M, 7700 + M)
    other = _step_inputs(M, 7800 + M)  # a different step run eagerly between replays
    s = torch.cuda.Stream()
    want, got, scratch = _outputs(M, t, dev), _outputs(M, t, dev), _outputs(M, t, dev)
    with torch.cuda.stream(s):
        _step(t, want, 0)  # eager reference; also puts the stream's workspace in place
        _step(other, scratch, 1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _step(t, got, 0)
    for rep in range(3):
        for v in got.values():
            v.zero_()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager step"
        with torch.cuda.stream(s):
            _step(other, scratch, rep % 2)  # eager work on the same stream and workspace
        torch.cuda.synchronize()
