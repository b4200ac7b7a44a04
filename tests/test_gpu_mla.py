"""GPU parity of the section 09 MLA decode attention with weight absorption
against the CPU oracle (float64), at small shapes, the limits (1024-wide
latent, 16384 cache rows) and the GLM shape (64 heads, latent 512, nope 192,
rope 64, value 256)."""
import numpy as np
import pytest
import torch

import int4_expert_gemv_moe_amd as moe
import oracle
from gpu_util import assert_close_rows, say, to_np

pytestmark = pytest.mark.gpu


def _inputs(H, kvl, nope, rope, vdim, S, T, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, H, nope + rope)).astype(np.float32)
    kv_b = (rng.standard_normal((H * (nope + vdim), kvl)) / np.sqrt(kvl)).astype(np.float32)
    L = rng.standard_normal((T, kvl)).astype(np.float32)
    R = rng.standard_normal((T, max(rope, 1))).astype(np.float32)[:, :rope]
    return q, kv_b, np.ascontiguousarray(L), np.ascontiguousarray(R)


@pytest.mark.parametrize("dims,S,T", [
    ((4, 64, 24, 8, 32), 1, 1),
    ((4, 64, 24, 8, 32), 4, 4),             # T = S: query s sees s + 1 rows
    ((4, 64, 24, 8, 32), 3, 50),
    ((4, 128, 24, 8, 40), 2, 300),          # three chunks, the last one partial
    ((3, 64, 16, 0, 24), 2, 129),           # no rotary part, heads not a multiple of 8
    ((2, 192, 16, 8, 8), 2, 260),           # latent width not a power of two
    ((2, 1024, 16, 64, 8), 2, 16384),       # widest latent, most cache rows
    ((12, 256, 32, 16, 24), 2, 5000),       # 128-row chunks, heads not a multiple of 4
    ((8, 448, 32, 36, 64), 2, 777),         # rotary width not a multiple of 16, 7 column tiles
    ((64, 512, 192, 64, 256), 1, 9000),     # GLM shape, long cache
    ((64, 512, 192, 64, 256), 1, 1000),     # GLM shape, decode
    ((64, 512, 192, 64, 256), 4, 2048),     # GLM shape, 4 queries
])
def test_mla_decode_parity(dims, S, T):
    H, kvl, nope, rope, vdim = dims
    say(f"mla H={H} kvl={kvl} nope={nope} rope={rope} vdim={vdim} S={S} T={T}")
    scale = float(1.0 / np.sqrt(nope + rope))
    q, kv_b, L, R = _inputs(H, kvl, nope, rope, vdim, S, T, seed=T + S)
    ref = oracle.mla_decode(oracle.MlaConfig(H, kvl, nope, rope, vdim, scale), q, kv_b, L, R)
    cfg = moe.MlaConfig(H, kvl, nope, rope, vdim, scale)
    ws = moe.MlaWorkspace(cfg, S, T)
    Rd = torch.from_numpy(R).cuda() if rope else torch.zeros(1, dtype=torch.float32, device="cuda")
    ctx = moe.moe_mla_decode(cfg, torch.from_numpy(q).cuda(), torch.from_numpy(kv_b).cuda(),
                             torch.from_numpy(L).cuda(), Rd, ws)
    torch.cuda.synchronize()
    assert_close_rows(to_np(ctx).reshape(S * H, vdim), ref.reshape(S * H, vdim), what="mla ctx")


def test_mla_decode_repeated_calls_on_one_workspace():
    """A second call with fewer queries and cache rows on the same workspace
    gives the fresh result (no state carries over)."""
    H, kvl, nope, rope, vdim = 8, 128, 32, 16, 48
    scale = float(1.0 / np.sqrt(nope + rope))
    cfg = moe.MlaConfig(H, kvl, nope, rope, vdim, scale)
    ws = moe.MlaWorkspace(cfg, 4, 700)
    for S, T in ((4, 700), (1, 90)):
        q, kv_b, L, R = _inputs(H, kvl, nope, rope, vdim, S, T, seed=S * T)
        ctx = moe.moe_mla_decode(cfg, torch.from_numpy(q).cuda(), torch.from_numpy(kv_b).cuda(),
                                 torch.from_numpy(L).cuda(), torch.from_numpy(R).cuda(), ws)
        torch.cuda.synchronize()
        ref = oracle.mla_decode(oracle.MlaConfig(H, kvl, nope, rope, vdim, scale), q, kv_b, L, R)
        assert_close_rows(to_np(ctx).reshape(S * H, vdim), ref.reshape(S * H, vdim), what=f"S={S}")
