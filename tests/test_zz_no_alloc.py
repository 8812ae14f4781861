"""bs_verify_noalloc, the verify call whose partials live in the library's
static device array (no handle, no allocation), against bs_verify through
the C ABI: two calls in a row, the second on a smaller input (the row-segment
kernel, then the tile kernel), element by element; bf16 logits; and the host
checks that refuse shapes beyond the array before anything is launched."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    import beam_search_step_amd as bs
    bs.library()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda", 0)


def _both(dev, B, k, V, seed, dtype="f32"):
    import beam_search_step_amd as bs
    lg, prop = synth.verify_inputs(B, k, V, seed=seed)
    x = torch.from_numpy(lg).to(dev)
    if dtype == "bf16":
        x = torch.from_numpy(synth.f32_to_bf16_bits(lg).view(np.int16)).to(dev)
    p = torch.from_numpy(prop).to(dev)
    ver = bs.Verifier(B, k, V, dtype=dtype)
    acc0, am0 = ver(x, p)
    acc0, am0 = acc0.clone(), am0.clone()
    ver.close()
    acc1 = torch.full((B,), -7, dtype=torch.int32, device=dev)
    am1 = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    bs.bs_verify_noalloc(x, bs.DTYPES[dtype], B, k, V, p, acc1, am1)
    torch.cuda.synchronize()
    assert torch.equal(am1, am0), f"B={B} k={k} V={V}: argmax differs"
    assert torch.equal(acc1, acc0), f"B={B} k={k} V={V}: accepted lengths differ"
    return acc1


def test_noalloc_matches_bs_verify_on_two_calls(dev):
    # 512 rows (row segments), then 15 rows (tiles) that reuse the same array
    acc = _both(dev, 64, 8, 32000, seed=5)
    assert (acc >= 1).all()
    _both(dev, 3, 5, 1001, seed=6)


def test_noalloc_bf16_and_alone(dev):
    _both(dev, 40, 8, 20001, seed=7, dtype="bf16")   # 320 rows, unaligned bf16 rows
    _both(dev, 2, 3, 70000, seed=8, dtype="bf16")


def test_noalloc_refuses_shapes_beyond_the_array(dev):
    import beam_search_step_amd as bs
    L = bs.library()
    x = torch.zeros(16, dtype=torch.float32, device=dev)
    y = torch.zeros(16, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    # 255 rows of 8.4M+ logits: 255 * 2057 tiles of partials exceed 4 MiB
    # (refused on the host: nothing is read through the small tensor)
    V = 2057 * 4096
    assert L.bs_verify_noalloc(s, x.data_ptr(), 0, 51, 5, V, V, y.data_ptr(), y.data_ptr(),
                               y.data_ptr()) == bs.BS_EINVAL
    assert L.bs_verify_noalloc(s, x.data_ptr(), 0, 1, 65, 4, 4, y.data_ptr(), y.data_ptr(),
                               y.data_ptr()) == bs.BS_EINVAL
    assert L.bs_verify_noalloc(s, x.data_ptr(), 2, 1, 1, 4, 4, y.data_ptr(), y.data_ptr(),
                               y.data_ptr()) == bs.BS_EINVAL
    assert L.bs_verify_noalloc(s, x.data_ptr(), 0, 1, 1, 4, 3, y.data_ptr(), y.data_ptr(),
                               y.data_ptr()) == bs.BS_EINVAL
    torch.cuda.synchronize()
