"""pkv_decode_attn_noalloc, the decode entry point that allocates nothing
(its workspace is the library's static device array), against
pkv_decode_attn with a caller's workspace: two calls in a row, the second
on a smaller batch, each bit-identical to the ordinary entry point and
within the oracle bar, through the item launches and through the tree
launch; a call that needs more than the array holds is refused with
PKV_E_WORKSPACE."""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import configs, generate, scaled  # noqa: E402
from workloads.configs import replace_shape  # noqa: E402

from gpu_helpers import build_library, build_oracle, errors, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

B16 = configs.BEAM
# a plan of 7 KB (written into the array by the copy kernels), then a
# smaller tree whose plan travels in the launch arguments
FIRST = scaled("mcts", "mcts_d6", shape=replace_shape(B16, L=2, Hq=8, Hkv=2), root_len=300, depth=6,
               edge_len=20)
SECOND = scaled("beam", "beam_s", shape=replace_shape(B16, L=3, Hq=8, Hkv=2), root_len=200,
                n_branches=5, branch_len=37)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("tree", [0, 2])
def test_noalloc_matches_the_workspace_entry_point(pkv, tree):
    from paged_kv_cache_amd import binding
    for w in (FIRST, SECOND):
        inp = generate(w)
        c, h = build_library(pkv, w, inp)
        c.set_option("tree", tree)
        seqs = [h[s] for s in w.query_sids]
        info = c.plan_info(seqs)
        note(f"noalloc {w.name} (tree {tree}): plan {info['plan_bytes']} B, "
             f"workspace {info['workspace_bytes']} B, items {info['n_items']}")
        assert (info["n_items"] == 0) == (tree == 2)
        q = to_device(inp.q)
        ref = c.decode(seqs, q, scale=w.softmax_scale)
        got = torch.full_like(ref, float("nan"))
        binding.pkv_decode_attn_noalloc(c.handle, seqs, 0, w.shape.L, q, got, w.softmax_scale)
        torch.cuda.synchronize()
        ref, got = ref.cpu().numpy(), got.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
        want = oracle.decode(build_oracle(w, inp), w.query_sids, inp.q.f32(), w.softmax_scale)
        ma, rl = errors(got, want)
        note(f"noalloc {w.name}: max_abs={ma:.3e} rel_l2={rl:.3e}")
        assert ma <= 2e-3 and rl <= 1e-2
        c.close()


def test_noalloc_refuses_a_workspace_above_its_limit(pkv):
    """16 branches over a 4096-token root cut into 32-token chunks, 8 layers
    x 8 KV heads: 8192 partial rows per plane, about 272 MB of partial
    states, more than the 128 MiB array."""
    from paged_kv_cache_amd import binding
    L, Hkv, Hq, D, BS = 8, 8, 32, 128, 16
    c = pkv.PagedKVCache(256 + 16 + 16, BS, L, Hkv, Hq, D, dtype="bf16", device="cuda")
    root = c.create()
    z = torch.zeros((L, 4096, Hkv, D), dtype=torch.bfloat16, device="cuda")
    c.append([root], [4096], z, z)
    kids = [c.fork(root) for _ in range(16)]
    z1 = torch.zeros((L, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    c.append(kids, [1] * 16, z1, z1)
    c.set_option("chunk_tokens", 32)
    need = c.plan_info(kids)["workspace_bytes"]
    assert need > (128 << 20)       # PKV_NOALLOC_WORKSPACE_BYTES
    q = torch.zeros((L, 16, Hq, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((L, 16, Hq, D), dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        binding.pkv_decode_attn_noalloc(c.handle, kids, 0, L, q, out, 0.1)
    assert e.value.code == pkv.PKV_E_WORKSPACE
    torch.cuda.synchronize()
    c.close()
