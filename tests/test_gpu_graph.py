"""HIP-graph capture of a decode step built from the library's entry points,
on a fresh stream with no eager call before the capture: every replay must
reproduce the eager results bit for bit, also after other eager calls on the
same stream -- with longer K, on their own workspace or on the graph's own
workspace -- ran between the replays.  The entry points take their scratch
from the caller's workspace and launch kernels only (no allocation, no memset
node, no synchronisation), so they can be captured as a stream's first work."""
import pytest
import torch

from bit_quantized_decode_group_amd import ops, synth
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, dev_u8, dev_u32

pytestmark = pytest.mark.gpu


def _step_inputs(M, seed, D=1024, I=1536, K_lm=512):
    blk = synth.mlp_block(M=M, D=D, I=I, seed=seed)
    moe = synth.moe_token(E=16, D=512, I=256, top_k=4, seed=seed + 1, n_logit_sets=2)
    lm = synth.lm_head(M=M, V=4000, K=K_lm, seed=seed + 2)
    gu = ops.tile_pack(dev_u32(blk["codes_gu"]), dev_bf16(blk["scales_gu"]), dev_bf16(blk["biases_gu"]))
    dn = ops.tile_pack(dev_u32(blk["codes_d"]), dev_bf16(blk["scales_d"]), dev_bf16(blk["biases_d"]))
    lmt = ops.tile_pack(dev_u32(lm["codes"]), dev_bf16(lm["scales"]), dev_bf16(lm["biases"]))
    return {
        "M": M, "x": dev_bf16(blk["x"]), "gamma": dev_bf16(blk["gamma"]), "eps": blk["eps"], "I": blk["I"],
        "D": blk["D"], "gu": gu, "dn": dn, "lm": lmt, "V": lm["V"], "K_lm": K_lm, "xl": dev_bf16(lm["x"]),
        "draft": dev_i32(lm["draft"][:M]), "xm": dev_bf16(moe["x"]), "logits": dev_f32(moe["logits"]),
        "w_gu": dev_u8(moe["w_gu"]), "w_down": dev_u8(moe["w_down"]), "top_k": moe["top_k"],
    }


def _ws_bytes(t):
    M = t["M"]
    return max(ops.workspace_bytes("rmsnorm_gateup_swiglu_tiled", M, t["I"], t["D"]),
               ops.workspace_bytes("qgemv_affine4_tiled", M, t["D"], t["I"]),
               ops.workspace_bytes("moe_expert_qgemv", t["top_k"], 16, 512, 256),
               ops.workspace_bytes("lmhead_argmax_tiled", M, t["V"], t["K_lm"]))


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


def _step(t, o, which, ws):
    ops.rmsnorm_gateup_swiglu_tiled(t["x"], t["gamma"], t["eps"], *t["gu"], t["I"], h=o["h"], ws=ws)
    ops.qgemv_affine4_tiled(o["h"], *t["dn"], t["D"], y=o["y"], ws=ws)
    ops.moe_expert_qgemv(t["xm"], t["logits"][which], t["top_k"], t["w_gu"], t["w_down"], y=o["ym"],
                         out_ids=o["mids"], out_w=o["mw"], ws=ws)
    ops.lmhead_argmax_tiled(t["xl"], *t["lm"], t["V"], draft=t["draft"], logits=o["lg"], ids=o["ids"],
                            accepted=o["acc"], ws=ws)


@pytest.mark.parametrize("M", [8, 1])
def test_graph_replay_equals_eager(M):
    dev = torch.device("cuda:0")
    t = _step_inputs(M, 7700 + M)
    # a different step with a longer K everywhere (larger split-K scratch), run eagerly between replays
    other = _step_inputs(M, 7800 + M, D=2560, I=12800, K_lm=2048)
    ws_g = ops.workspace(max(_ws_bytes(t), _ws_bytes(other)))  # also serves the larger eager step
    ws_o = ops.workspace(_ws_bytes(other))
    want, got, scratch = _outputs(M, t, dev), _outputs(M, t, dev), _outputs(M, other, dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # fresh: the capture is the first work on it
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _step(t, got, 0, ws_g)
    with torch.cuda.stream(s):
        _step(t, want, 0, ws_o)  # eager reference, on another workspace
    torch.cuda.synchronize()
    for rep in range(4):
        for v in got.values():
            v.zero_()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager step"
        with torch.cuda.stream(s):  # eager work between replays: larger shapes, on either workspace
            _step(other, scratch, rep % 2, ws_o if rep % 2 else ws_g)
        torch.cuda.synchronize()
    hdr = ops.lib().qg_workspace_header_bytes()
    assert int(torch.count_nonzero(ws_g[:hdr])) == 0 and int(torch.count_nonzero(ws_o[:hdr])) == 0
