"""sparse_attn_decode_step_noalloc (scratch in the library's fixed per-GPU
array) against sparse_attn_decode_step (caller workspace), through the C ABI:
two calls in a row, the second on a smaller input, must give identical block
sets, outputs and compressed keys."""
import pytest
import torch

import block_sparse_attention_12_amd as sa

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
BITS = {"f32": torch.int32, "bf16": torch.int16}


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TD[dt]).to(DEV)


def lens_t(lens):
    return torch.tensor(lens, dtype=torch.int32, device=DEV)


def _pair(dt, mode, G, B, Hkv, T, lens, k, seed):
    Hq = 4 * Hkv
    K = rand((B, Hkv, T, 128), dt, seed)
    V = rand((B, Hkv, T, 128), dt, seed + 1)
    Q = rand((B, Hq, 128), dt, seed + 2, scale=128 ** -0.5)
    sel = Q if G == 4 else rand((B, Hkv * G, 128), dt, seed + 3, scale=128 ** -0.5)
    nc_cap = sa.n_compressed(T)
    lp = [max(0, L - 1) for L in lens]
    Kc_a = torch.zeros((B, Hkv, nc_cap, 128), dtype=TD[dt], device=DEV)
    sa.compress(K, Kc_a, lens_t([0] * B), lens_t(lp))
    Kc_b = Kc_a.clone()
    Lp, Ln = lens_t(lp), lens_t(lens)
    O1, l1, i1, c1 = sa.decode_step_noalloc(Q, sel, K, V, Kc_a, Lp, Ln, k, 1, 2, mode)
    O2, l2, i2, c2 = sa.decode_step(Q, sel, K, V, Kc_b, Lp, Ln, k, 1, 2, mode)
    torch.cuda.synchronize()
    print("case", dt, mode, G, B, Hkv, T, lens, k, flush=True)
    assert torch.equal(i1, i2) and torch.equal(c1, c2)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    assert torch.equal(Kc_a.view(BITS[dt]), Kc_b.view(BITS[dt]))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mode,G", [("raw_sum", 1), ("softmax_sum", 4)])
def test_noalloc_step_equals_workspace_step_twice(dt, mode, G):
    _pair(dt, mode, G, B=4, Hkv=4, T=20000, lens=[20000, 19000, 7000, 3], k=40, seed=11)
    _pair(dt, mode, G, B=2, Hkv=2, T=3000, lens=[2999, 1500], k=12, seed=21)     # smaller


def test_noalloc_step_refuses_a_step_beyond_its_scratch():
    B, Hkv, T = 64, 8, 131072
    Q = torch.zeros((B, 4 * Hkv, 128), dtype=torch.bfloat16, device=DEV)
    K = torch.zeros((B, Hkv, 64, 128), dtype=torch.bfloat16, device=DEV)   # shapes only checked on host
    p = sa.make_params(64, 1, 2, "softmax_sum")
    need = sa.decode_step_workspace_size(B, 4 * Hkv, Hkv, 4 * Hkv, T, p, 67)
    assert need > sa.NOALLOC_SCRATCH_BYTES
    st = sa.lib().sparse_attn_decode_step_noalloc(
        Q.data_ptr(), Q.data_ptr(), 4 * Hkv, K.data_ptr(), K.data_ptr(), K.data_ptr(), sa.SA_BF16,
        B, 4 * Hkv, Hkv, 128, T, sa.n_compressed(T), Q.data_ptr(), Q.data_ptr(), 1,
        __import__("ctypes").byref(p), 1.0, Q.data_ptr(), 67, Q.data_ptr(), Q.data_ptr(), sa.SA_F32,
        None, 0, None)
    assert st == sa.SA_ERR_WORKSPACE
