"""Fine-grained FP8 cast ('Chapter 41 Training at Scale', section 41.5) against the oracle (GPU)."""
import sys

import numpy as np
import pytest

import inputs
import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mp():
    import torch
    assert torch.cuda.is_available()
    import optimizer_step_tensor_amd as m
    m.lib()
    return m


def _cast(mp, x, block):
    import torch
    n = x.numel()
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n // block, dtype=torch.float32, device="cuda")
    mp.mp_cast_fp8_blocks(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), n, block)
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_e4m3_every_fp32_value_up_to_448(mp):
    """Every fp32 pattern with |x| <= 448, both signs, in blocks of 16 whose last value is 448
    (so the block scale is exactly 1): the device codes equal the oracle's E4M3 rounding."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    top = 0x43E00000                         # bits of 448
    per = 15 * (1 << 24)                     # patterns per chunk
    L = oracle.lib()
    bad = 0
    for sign in (0, 0x80000000):
        for c0 in range(0, top + 1, per):
            c1 = min(top + 1, c0 + per)
            cnt = c1 - c0
            nb = -(-cnt // 15)
            pat = torch.arange(c0, c0 + nb * 15, dtype=torch.int64, device="cuda")
            pat = torch.where(pat < c1, pat, torch.zeros_like(pat)) | sign
            x = torch.empty(nb, 16, dtype=torch.int32, device="cuda")
            x[:, :15] = pat.view(nb, 15).to(torch.int32)
            x[:, 15] = top
            xf = x.view(torch.float32).reshape(-1)
            codes, scales = _cast(mp, xf, 16)
            assert (scales == 1.0).all()
            xs = xf.cpu().numpy()
            parts = np.array_split(np.arange(xs.size), 16)

            def ref(idx):
                return oracle.e4m3(xs[idx[0]:idx[-1] + 1], L)

            with ThreadPoolExecutor(16) as ex:
                want = np.concatenate(list(ex.map(ref, parts)))
            bad += int((codes != want).sum())
        say("e4m3 sign %x: mismatches so far %d" % (sign, bad))
    assert bad == 0


@pytest.mark.parametrize("block", [16, 32, 128, 1024])
def test_fp8_blocks_match_the_oracle(mp, block):
    """Seeded values whose magnitude varies by block (2^-40 .. 2^40), zero blocks, and blocks
    holding inf or NaN: codes and scales are bit-exact."""
    import torch
    nblocks = 4099
    n = nblocks * block
    base = inputs.gen_host_f32(n, inputs.recipe(inputs.key(77, block), inputs.NORMAL, sigma=1.0))
    exps = inputs.gen_host_f32(nblocks, inputs.recipe(inputs.key(78, block), inputs.NORMAL,
                                                      sigma=12.0))
    x = (base.reshape(nblocks, block) * np.exp2(np.round(exps))[:, None]).astype(np.float32)
    x[5] = 0.0
    x[7, 3] = np.inf
    x[11, 1] = np.nan
    x[13, :] = np.nan
    x[17, 2] = -np.inf
    x = x.ravel()
    codes, scales = _cast(mp, torch.from_numpy(x).cuda(), block)
    want_c, want_s = oracle.fp8_block_cast(x, block)
    assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(codes, want_c)


def test_fp8_argument_errors(mp):
    import torch
    x = torch.zeros(48, dtype=torch.float32, device="cuda")
    c = torch.zeros(48, dtype=torch.uint8, device="cuda")
    s = torch.zeros(3, dtype=torch.float32, device="cuda")
    for n, block in ((48, 8), (40, 16), (48, 2048), (-16, 16)):
        with pytest.raises(mp.MpError) as e:
            mp.mp_cast_fp8_blocks(x.data_ptr(), c.data_ptr(), s.data_ptr(), n, block)
        assert e.value.status == mp.MP_ERR_INVALID
