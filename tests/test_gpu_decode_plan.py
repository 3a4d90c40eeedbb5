"""GA decode work plan: the split grid cuts the key units of the whole batch
(32-key tiles of each sequence's cache plus one unit for its new token) into
balanced chunks, derived on the device from ctx_lens.  These cases aim at the
plan itself -- chunks that hold many short sequences, batches longer than the
256 threads of the in-kernel scan, contexts on tile edges, chunks longer than
the 128 pages a paged workgroup preloads at a time -- against the fp64 oracle
(model doc "MiMo-V2-Flash", MiMoV2FlashModel.forward: past_key_values, one
unprocessed token per sequence; Key features: attention sink)."""
import numpy as np
import pytest
import torch

from global_attention_mimo_amd import binding as B
from global_attention_mimo_amd import synth
from gpu_util import bits, compare, log, orc, sink_array, to_dev

pytestmark = pytest.mark.gpu
GA = 1
SCALE = float(np.float32(synth.SOFTMAX_SCALE))
DEV = "cuda"


def _decode_vs_oracle(ctx, split, seed, what, max_ctx=None):
    x = synth.decode_inputs(ctx, GA, seed=seed, headroom=2)
    d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "ctx_lens",
                                            "sink")}
    mc = max(ctx) if max_ctx is None else max_ctx
    out, lse = B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], mc, GA,
                        sink=d["sink"], kv_base=d["kv_base"], split_tokens=split)
    torch.cuda.synchronize()
    ro, rl = orc().decode(bits(x.q), bits(x.k_new), bits(x.v_new), bits(x.k_cache), bits(x.v_cache),
                          x.ctx_lens.numpy(), layer_type=GA, scale=SCALE, sink=x.sink.numpy(),
                          kv_base=x.kv_base.numpy())
    compare(out, lse, ro, rl, what)
    return x, d, out, lse


@pytest.mark.parametrize("split", [0, 32, 96])
def test_many_short_sequences(split):
    """600 sequences with 0..70 cached keys: chunks hold pieces of many
    sequences, and each scan thread sums three sequences."""
    g = np.random.default_rng(3)
    ctx = [int(c) for c in g.integers(0, 71, 600)]
    log(f"[case] GA decode plan: 600 short sequences, split {split}")
    _decode_vs_oracle(ctx, split, 90, f"600 short sequences split {split}")


@pytest.mark.parametrize("split", [0, 32, 512])
def test_tile_edges_mixed_lengths(split):
    """Contexts on 32-key tile edges mixed with long ones."""
    ctx = [0, 1, 31, 32, 33, 63, 64, 65, 5000, 20000, 2, 4095, 4096, 4097]
    log(f"[case] GA decode plan: tile edges, split {split}")
    _decode_vs_oracle(ctx, split, 91, f"tile edges split {split}")


def test_context_past_max_ctx_inside_a_shared_chunk():
    """A sequence past max_ctx between two covered ones whose pieces share its
    chunk: its outputs are NaN, its neighbours' are exact."""
    ctx = [40, 3000, 50, 7]
    x = synth.decode_inputs(ctx, GA, seed=92, headroom=2)
    d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "ctx_lens",
                                            "sink")}
    log("[case] GA decode plan: context past max_ctx")
    out, lse = B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], 100, GA,
                        sink=d["sink"], kv_base=d["kv_base"], split_tokens=64)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all() and torch.isnan(lse[1]).all()
    keep = [0, 2, 3]
    ro, rl = orc().decode(bits(x.q)[keep], bits(x.k_new)[keep], bits(x.v_new)[keep], bits(x.k_cache),
                          bits(x.v_cache), x.ctx_lens.numpy()[keep], layer_type=GA, scale=SCALE, sink=x.sink.numpy(),
                          kv_base=x.kv_base.numpy()[keep])
    compare(out[keep], lse[keep], ro, rl, "neighbours of a context past max_ctx")


@pytest.mark.parametrize("page_size,split", [(16, 4096), (16, 6000), (32, 8192), (64, 16384)])
def test_paged_chunks_longer_than_the_page_preload(page_size, split):
    """Chunks of 4096-16384 keys over pages of 16-64 rows span up to 256 pages,
    so a workgroup walks them in spans of at most 128 pages: bit-identical to
    the contiguous pool and within the bars of the oracle."""
    ctx = [10000, 4100, 1, 33000]
    log(f"[case] paged decode spans: page {page_size}, split {split}")
    x = synth.decode_inputs(ctx, GA, seed=93, headroom=2)
    table, npages = synth.paged_block_table(ctx, page_size, seed=page_size + 1)
    rows = npages * page_size
    kp = torch.zeros((rows, 4, 192), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros((rows, 4, 128), dtype=torch.bfloat16, device=DEV)
    kc, vc = to_dev(x.k_cache), to_dev(x.v_cache)
    for b, c in enumerate(ctx):
        j = torch.arange(c, device=DEV)
        dst = table.to(DEV)[b, j // page_size].long() * page_size + j % page_size
        src = int(x.kv_base[b]) + j
        kp[dst] = kc[src]
        vp[dst] = vc[src]
    q, kn, vn, sink, ctx_d = (to_dev(t) for t in (x.q, x.k_new, x.v_new, x.sink, x.ctx_lens))
    op, lp = B.decode_paged(q, kn, vn, kp, vp, table.to(DEV), page_size, ctx_d, max(ctx), sink=sink,
                            split_tokens=split)
    of, lf = B.decode(q, kn, vn, kc, vc, ctx_d, max(ctx), GA, sink=sink, kv_base=to_dev(x.kv_base),
                      split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(op, of) and torch.equal(lp, lf), "paged decode is not bit-identical to the contiguous pool"
    ro, rl = orc().decode(bits(x.q), bits(x.k_new), bits(x.v_new), bits(x.k_cache), bits(x.v_cache),
                          x.ctx_lens.numpy(), layer_type=GA, scale=SCALE, sink=sink_array(x.sink),
                          kv_base=x.kv_base.numpy())
    compare(op, lp, ro, rl, f"paged spans page {page_size} split {split}")


def test_workspace_is_scratch_between_calls():
    """Two decodes of different batches through one workspace, the second one
    smaller: the plan header and partials of the first call leave no trace."""
    ws = torch.full((B.mimo_attn_decode_workspace_size(B.make_dims(), GA, 300, 9000, 0) // 4 + 4,), float("nan"),
                    dtype=torch.float32, device=DEV)
    log("[case] GA decode plan: one workspace, two calls")
    for ctx, seed in (([9000] * 7 + [3] * 293, 94), ([700, 0, 8000], 95)):
        x = synth.decode_inputs(ctx, GA, seed=seed, headroom=2)
        d = {f: to_dev(getattr(x, f)) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "kv_base", "ctx_lens",
                                                "sink")}
        out, lse = B.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ctx_lens"], 9000, GA,
                            sink=d["sink"], kv_base=d["kv_base"], workspace=ws)
        torch.cuda.synchronize()
        ro, rl = orc().decode(bits(x.q), bits(x.k_new), bits(x.v_new), bits(x.k_cache), bits(x.v_cache),
                              x.ctx_lens.numpy(), layer_type=GA, scale=SCALE, sink=x.sink.numpy(),
                              kv_base=x.kv_base.numpy())
        compare(out, lse, ro, rl, f"shared workspace batch {len(ctx)}")
