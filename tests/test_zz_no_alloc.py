"""moe_permute_noalloc (no workspace argument, nothing allocated) against moe_permute with a
caller workspace, through the C ABI: counts, offsets, row_of, src_of and x_perm bit-identical,
and equal to the oracle's permutation, on calls in a row that reuse the library's scratch
array with shrinking inputs (the first at the array's full size: E = 1024, 256 chunks)."""
import numpy as np
import pytest

from moe_cases import O, log, synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _outputs(T, E, k, H, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    R = T * k
    return dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                row_of=torch.full((max(R, 1),), -7, **i32), src_of=torch.full((max(R, 1),), -7, **i32),
                x_perm=torch.full((max(R, 1), H), 3.0, dtype=torch.bfloat16, device=dev))


def _permute_both(T, E, k, H, seed, stream):
    from grouped_gemm_weights_amd import binding as B
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed)
    logits_np = rng.standard_normal((T, E)).astype(np.float32)
    x_bits = synth.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = torch.from_numpy(logits_np).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    B.moe_route(logits, T, E, k, idx, w, status, stream)
    a, b = _outputs(T, E, k, H, dev), _outputs(T, E, k, H, dev)
    ws_bytes = B.moe_permute_workspace_size(T, E, k)
    ws = torch.empty((max(1, ws_bytes),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    B.moe_permute(idx, T, E, k, x, H, B.MOE_BF16, a["counts"], a["offsets"], a["row_of"],
                  a["src_of"], a["x_perm"], ws, ws_bytes, status, stream)
    B.moe_permute_noalloc(idx, T, E, k, x, H, B.MOE_BF16, b["counts"], b["offsets"], b["row_of"],
                          b["src_of"], b["x_perm"], status, stream)
    stream.synchronize()
    assert int(status.item()) == 0
    for key in a:
        assert torch.equal(a[key].view(torch.int16) if key == "x_perm" else a[key],
                           b[key].view(torch.int16) if key == "x_perm" else b[key]), key
    # and both are the oracle's stable counting sort
    oidx, _ = O.route(logits_np, k)
    row_of, src_of = O.permutation(oidx, E)
    R = T * k
    np.testing.assert_array_equal(b["src_of"].cpu().numpy()[:R], src_of)
    np.testing.assert_array_equal(b["row_of"].cpu().numpy()[:R], row_of)
    np.testing.assert_array_equal(b["counts"].cpu().numpy(), O.expert_counts(oidx, E))
    assert b["x_perm"].cpu().view(torch.int16).numpy()[:R].view(np.uint16).tobytes() == \
        x_bits[src_of // k].tobytes()
    return ws_bytes


def test_noalloc_permute_matches_workspace_permute_on_shrinking_calls():
    from grouped_gemm_weights_amd import binding as B
    stream = torch.cuda.Stream()
    sizes = [(2048, 1024, 8, 64), (6000, 256, 8, 136), (300, 64, 6, 72), (1, 8, 2, 8)]
    used = []
    for i, (T, E, k, H) in enumerate(sizes):
        log(f"case moe_permute_noalloc call {i}: T={T} E={E} k={k} H={H}")
        used.append(_permute_both(T, E, k, H, 900 + i, stream))
    log(f"workspace bytes per call: {used}")
    assert used[0] == 2 * 256 * 1024 * 4             # the first call fills the whole array
    assert used == sorted(used, reverse=True)


def test_noalloc_permute_argument_errors():
    from grouped_gemm_weights_amd import binding as B
    dev = torch.device("cuda")
    z = torch.zeros((16,), dtype=torch.int32, device=dev)
    with pytest.raises(B.MoEError) as e:
        B.moe_permute_noalloc(z, 2, 2048, 2, None, 8, B.MOE_BF16, z, z, z, z, None)
    assert e.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoEError) as e:
        B.moe_permute_noalloc(z, -1, 8, 2, None, 8, B.MOE_BF16, z, z, z, z, None)
    assert e.value.code == B.MOE_ERR_ARG
