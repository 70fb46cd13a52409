"""GPU projection against the oracle bit for bit, where the arithmetic is exact.

With hidden states and weights drawn from the small integers {-2, ..., 2}
(bf16 holds them exactly) every product and every partial sum of X . W^T is
an integer below 2^24 in magnitude, so fp32 accumulation in any order gives
the exact value the fp64 oracle gives.  With every rotary position 0 the
rotation is the identity.  Q and the written K/V must then carry exactly the
oracle's bf16 bits (both round the same exact value to nearest even), and the
slot mapping and every untouched cache byte must match too.  This pins the
projection's operand layout, swizzles and accumulation across every kernel
form the library picks: the split-K kernel at <= 64 rows with and without a
split reduction, and the three tiled forms (512, 1024 and 2048 rows at hidden
4096).  [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
Memory-Efficient Diffusion LLMs", paragraph 1 (the projection feeding the cache).
"""

import numpy as np
import pytest

import oracle as O
import synth

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"

# (rows, hidden, heads, head_dim): split-K at 64 rows; split-K with a split
# reduction (narrow layer); the one-per-CU six-wave tiles (512 rows), their
# 256-row form (1024 rows) and the eight-wave tiles (2048 rows).
CASES = [(64, 4096, 32, 128), (40, 1024, 2, 128), (24, 512, 4, 64), (512, 4096, 32, 128),
         (1024, 4096, 32, 128), (2048, 4096, 32, 128), (300, 384, 6, 64)]


def _small_int_bf16(seed, shape):
    g = np.random.default_rng([77, seed])
    a = g.integers(-2, 3, size=shape).astype(np.float32)
    return synth.to_bf16_bits(a)


@pytest.mark.gpu
@pytest.mark.parametrize("rows,hid,heads,d", CASES)
def test_projection_bit_exact_on_integer_inputs(rows, hid, heads, d):
    import kv_cache_attention_flash_amd as fd
    fd.load()
    print(f"[exact] rows={rows} hidden={hid} heads={heads}x{d}", flush=True)
    bs = 32
    per_seq = 64
    batch = -(-rows // per_seq)
    cu = np.minimum(np.arange(batch + 1) * per_seq, rows).astype(np.int32)
    slots = np.concatenate([np.arange(cu[b + 1] - cu[b]) for b in range(batch)]).astype(np.int32)
    # a slot order that is not the row order: reverse each sequence's slots
    for b in range(batch):
        slots[cu[b]:cu[b + 1]] = slots[cu[b]:cu[b + 1]][::-1]
    positions = np.zeros(rows, np.int32)
    nblk = per_seq // bs
    num_blocks = batch * nblk
    perm = np.random.default_rng([77, 3]).permutation(num_blocks).astype(np.int32)
    bt = perm.reshape(batch, nblk)
    x = _small_int_bf16(1, (rows, hid))
    w = _small_int_bf16(2, (3 * heads * d, hid))
    k0 = _small_int_bf16(3, (num_blocks, heads, bs, d))
    v0 = _small_int_bf16(4, (num_blocks, heads, bs, d))

    cache = fd.PagedKVCache(G.bf16_tensor(k0, DEV), G.bf16_tensor(v0, DEV), G.i32(bt, DEV))
    q, sm = fd.flash_cache_step(cache, G.bf16_tensor(x, DEV), G.bf16_tensor(w, DEV),
                                G.i32(cu, DEV), G.i32(positions, DEV), G.i32(slots, DEV), 5.0e5)
    torch.cuda.synchronize()

    q_ref, k_ref, v_ref, ps = O.flash_cache_step(x, w, heads, d, positions, 5.0e5, cu, slots, bt,
                                                 bs, k0, v0)
    assert np.array_equal(sm.cpu().numpy(), ps), "slot mapping"
    q_gpu = G.bits_of(q)
    assert np.array_equal(q_gpu, q_ref), \
        f"Q differs in {int(np.count_nonzero(q_gpu != q_ref))} of {q_ref.size} elements"
    k_gpu, v_gpu = G.bits_of(cache.k_cache), G.bits_of(cache.v_cache)
    assert np.array_equal(k_gpu, k_ref), \
        f"K cache differs in {int(np.count_nonzero(k_gpu != k_ref))} elements"
    assert np.array_equal(v_gpu, v_ref), \
        f"V cache differs in {int(np.count_nonzero(v_gpu != v_ref))} elements"


def test_integer_inputs_are_exact_in_fp32():
    """The premise of the test above, on the host: the largest partial sum
    magnitude (4 * hidden) stays below 2^24, and the oracle's fp64 projection
    of such inputs is integral."""
    hid = max(c[1] for c in CASES)
    assert 4 * hid < 2 ** 24
    x = _small_int_bf16(1, (8, hid))
    w = _small_int_bf16(2, (16, hid))
    y = O.qkv_projection(x, w)
    assert np.array_equal(y, np.rint(y))
