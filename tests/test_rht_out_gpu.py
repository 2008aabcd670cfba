"""The output-side (inverse) transform and the shard-batched transform
(rht_apply_shards) against the oracle, and the whole fused-linear sequence
of a gate-up layer: input transform and decode in one kernel, then both
shards' output transforms in one launch, compared with the oracle's exact
transform, product and inverse transform."""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import device_weight, ensure_built, oracle_indices, oracle_w64, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def block_bound(v64, shard_lens, max_block, per_elem=None):
    """Elementwise bound of the fp32 transform of v64 [B, n] per shard and
    block: (log2(nb) + 2) 2^-24 ||v_block||_2 * 1.01, plus, when the input
    itself carries an error of at most per_elem [B, n], that error carried
    through the orthonormal block: sum_{j in block} per_elem_j / sqrt(nb)."""
    out = np.empty_like(v64)
    off = 0
    for n in shard_lens:
        for nb in oracle.rht_blocks(n, max_block):
            sl = slice(off, off + nb)
            nrm = np.linalg.norm(v64[:, sl], axis=1, keepdims=True)
            out[:, sl] = (np.log2(nb) + 2) * 2.0 ** -24 * nrm * 1.01
            if per_elem is not None:
                out[:, sl] += per_elem[:, sl].sum(axis=1, keepdims=True) / np.sqrt(nb)
            off += nb
    return out


def run_shards(vq, x64, xs, dtype, lens, mb, inverse, seed):
    import torch
    n = sum(lens)
    signs = vqsynth.make_signs(n, np.random.SeedSequence(seed))
    got = vq.rht_apply_shards(x_to_device(xs, dtype), torch.from_numpy(signs).cuda(), mb, lens, inverse=inverse)
    torch.cuda.synchronize()
    want = oracle.rht_shards_ref(x64, lens, signs, mb, inverse=inverse)
    err = np.abs(got.cpu().numpy().astype(np.float64) - want)
    lim = block_bound(x64, lens, mb)
    assert np.all(err <= lim), f"{lens}/{mb} inverse={inverse}: worst {np.max(err / lim):.3g} of the bound"
    return got, signs


# (shard lengths, max_block): the 70B gate-up pair, a QKV split, one
# shard of a non-power-of-two size, SmolLM's 576-wide QKV, small ragged
# shards on the scalar path, sixteen shards
CASES = [
    ([28672, 28672], 8192), ([4096, 1024, 1024], 4096), ([14336], 8192), ([576, 192, 192], 64),
    ([12, 8], 8), ([40, 24, 8], 16), ([256] * 16, 128), ([2688], 8192),
]


@pytest.mark.parametrize("lens,mb", CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("inverse", [False, True], ids=["fwd", "inv"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shards(vq, lens, mb, inverse, dtype):
    n = sum(lens)
    print(f"rht shards {lens} mb={mb} inverse={inverse} {dtype}", flush=True)
    xs, x64 = vqsynth.make_x(3, n, dtype, np.random.SeedSequence(n + mb))
    run_shards(vq, x64, xs, dtype, lens, mb, inverse, seed=len(lens) + mb)


@pytest.mark.parametrize("n,mb,dtype", [(28672, 8192, "f32"), (2688, 8192, "bf16"), (4096, 1, "f32")])
def test_single_shard_forward_is_rht_apply(vq, n, mb, dtype):
    """One forward shard is rht_apply: the same kernels, bit for bit."""
    import torch
    xs, _ = vqsynth.make_x(2, n, dtype, np.random.SeedSequence(n))
    signs = torch.from_numpy(vqsynth.make_signs(n, np.random.SeedSequence(n + 1))).cuda()
    x = x_to_device(xs, dtype)
    a = vq.rht_apply(x, signs, mb)
    b = vq.rht_apply_shards(x, signs, mb, [n])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_inverse_undoes_forward(vq):
    """inverse(forward(x)) returns x to within two transforms' rounding."""
    import torch
    n, mb = 57344, 8192
    xs, x64 = vqsynth.make_x(2, n, "f32", np.random.SeedSequence(5))
    signs = torch.from_numpy(vqsynth.make_signs(n, np.random.SeedSequence(6))).cuda()
    fwd = vq.rht_apply_shards(x_to_device(xs, "f32"), signs, mb, [28672, 28672])
    back = vq.rht_apply_shards(fwd, signs, mb, [28672, 28672], inverse=True)
    torch.cuda.synchronize()
    err = np.abs(back.cpu().numpy().astype(np.float64) - x64)
    assert np.all(err <= 2 * block_bound(x64, [28672, 28672], mb))


def test_fused_gate_up_linear(vq):
    """A gate-up weight of two 4096-row shards, rotated on both sides:
    y' = W' RHT_in(x) in the decode kernel, then y = D H y' per shard in one
    launch.  Every output is compared with the oracle's exact sequence; the
    bound carries the product's tolerance through the orthonormal output
    blocks and adds the transform's own rounding."""
    import torch
    n_sh, k, mb = 4096, 4096, 4096
    sw = vqsynth.random_weight(2 * n_sh, k, 1, 16, k, seed=21)
    xs, x64 = vqsynth.make_x(4, k, "bf16", np.random.SeedSequence(22))
    s_in = vqsynth.make_signs(k, np.random.SeedSequence(23))
    s_out = vqsynth.make_signs(2 * n_sh, np.random.SeedSequence(24))
    w = device_weight(sw)
    y_rot = vq.vq_gemv_rht(w, x_to_device(xs, "bf16"), torch.from_numpy(s_in).cuda(), mb)
    y = vq.rht_apply_shards(y_rot, torch.from_numpy(s_out).cuda(), mb, [n_sh, n_sh], inverse=True)
    torch.cuda.synchronize()
    xr = oracle.rht_ref(x64, s_in, mb)
    y_rot_ref, mag = oracle.matmul_ref(oracle_w64(sw, None, oracle_indices(sw)), xr)
    want = oracle.rht_shards_ref(y_rot_ref, [n_sh, n_sh], s_out, mb, inverse=True)
    tol = oracle.MATMUL_RTOL * mag + oracle.MATMUL_ATOL
    lim = block_bound(y_rot_ref, [n_sh, n_sh], mb, per_elem=tol)
    err = np.abs(y.cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= lim), f"worst {np.max(err / lim):.3g} of the bound"
