"""GPU parity over seeded random configurations: each case draws a layout,
dtype, head dims, GQA ratio, lengths (including 0, 1 and ragged tails), mask
mode and cache kind within the documented limits, and the HIP path through
the C ABI is compared with the fp64 oracle on the same inputs.  The draws are
fixed by the seed, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import bsa_plan, compare, fia_plan, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _lengths(rng, B, S):
    L = rng.integers(0, S + 1, size=B)
    L[rng.integers(B)] = S                       # one full-length sequence
    if B > 1 and rng.random() < 0.5:
        L[rng.integers(B)] = int(rng.choice([0, 1]))
    return L


def _check_fia(case):
    say(f"[rand] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} Skv={case.Skv} D={case.Dqk}/{case.Dv} mode={case.sparse_mode} "
        f"lq={None if case.lq is None else list(case.lq)} lkv={None if case.lkv is None else list(case.lkv)} "
        f"paged={case.block_table is not None} dtype={case.dtype}")
    ref = oracle.attention(case)
    to_dev(case)
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    rng = np.random.default_rng(700 + seed)
    layout = str(rng.choice(["BNSD", "BSND", "BSH", "TND"]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    Dqk, Dv = [(64, 64), (128, 128), (192, 128)][rng.integers(3)]
    if layout != "TND" and Dqk == 192:
        Dqk, Dv = 128, 128
    KVN = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    Sq = int(rng.integers(1, 400))
    if layout == "TND":
        lq = rng.integers(1, 300, size=B)
        lkv = lq.copy()
        mode = int(rng.choice([0, 2, 3]))
        case = W.make_fia(f"rand_prefill_{seed}", layout=layout, dtype=dtype, B=B, QN=KVN * G, KVN=KVN,
                          Dqk=Dqk, Dv=Dv, sparse_mode=mode, lq=lq, lkv=lkv, seed=710 + seed,
                          mask_kind="template" if mode >= 2 else None)
    else:
        Skv = int(rng.integers(1, 500))
        mode = int(rng.choice([0, 1, 2, 3, 4]))
        mask_kind = "random" if mode in (0, 1) and rng.random() < 0.5 else None
        if mode == 1:
            mask_kind = "random"
        if mode >= 2:
            mask_kind = "template"
        case = W.make_fia(f"rand_prefill_{seed}", layout=layout, dtype=dtype, B=B, QN=KVN * G, KVN=KVN,
                          Sq=max(Sq, 2), Skv=Skv, Dqk=Dqk, Dv=Dv, sparse_mode=mode,
                          pre_tokens=int(rng.integers(0, 300)), next_tokens=int(rng.integers(0, 300)),
                          lq=_lengths(rng, B, max(Sq, 2)), lkv=_lengths(rng, B, Skv),
                          mask_kind=mask_kind, seed=710 + seed, nan_padding=True)
    if case.atten_mask is not None and case.sparse_mode in (0, 1):
        # the pages do not support fully masked rows with an explicit mask: keep
        # the diagonal band of each row unmasked where it exists
        m = case.atten_mask.clone()
        for i in range(m.shape[-2]):
            m[..., i, min(i, m.shape[-1] - 1)] = 0
        case.atten_mask = m
    _check_fia(case)


@pytest.mark.parametrize("seed", range(16))
def test_random_paged(seed):
    rng = np.random.default_rng(800 + seed)
    KVN = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 5, 8]))
    B = int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    S = int(rng.choice([1, 1, 2, 3, 4, 9, 64, 200]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    lkv = rng.integers(S, 3000, size=B)
    if S == 1:
        bs = int(rng.choice([16, 64, 128, 256]))
        case = W.make_paged_decode(f"rand_paged_{seed}", dtype=dtype, B=B, QN=KVN * G, KVN=KVN, D=D,
                                   lkv=lkv, block_size=bs, pool_layout=int(rng.integers(2)),
                                   seed=810 + seed, extra_blocks=2,
                                   mask_p=0.3 if rng.random() < 0.4 else None)
    else:
        bs = int(rng.choice([128, 256, 512]))
        case = W.make_paged_prefill(f"rand_paged_{seed}", layout=str(rng.choice(["BNSD", "BSND"])),
                                    dtype=dtype, B=B, QN=KVN * G, KVN=KVN, D=D, Sq=S,
                                    lq=rng.integers(1, S + 1, size=B), lkv=lkv, block_size=bs,
                                    pool_layout=int(rng.integers(2)), sparse_mode=3,
                                    mask_kind="template", seed=810 + seed, extra_blocks=2, nan_pool=True)
    _check_fia(case)


@pytest.mark.parametrize("seed", range(16))
def test_random_int8_decode(seed):
    rng = np.random.default_rng(900 + seed)
    KVN = int(rng.choice([1, 2]))
    S = int(rng.choice([1, 1, 2, 4]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * S <= 16]))
    B = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    layout = str(rng.choice(["BNSD", "BSND", "BSH"]))
    lkv = rng.integers(S, 2500, size=B)
    # legal mode pairs: equal, or key 0 with value 1 at query S 1; a paged
    # int8 cache (block size a multiple of 32) at query S 1 only
    if S == 1:
        km, vm = [(0, 0), (1, 1), (0, 1)][int(rng.integers(3))]
        paged = bool(rng.random() < 0.5)
    else:
        km = vm = int(rng.integers(2))
        paged = False
    bs = int(rng.choice([32, 64, 128])) if paged else 0
    case = W.make_quant_decode(f"rand_int8_{seed}", layout=layout, B=B, QN=KVN * G, KVN=KVN, D=D,
                               Sq=S, lkv=lkv, kmode=km, vmode=vm,
                               offsets=bool(rng.random() < 0.7), sparse_mode=3 if S > 1 else 0,
                               seed=910 + seed, block_size=bs, pool_layout=int(rng.integers(2)),
                               extra_blocks=2 if paged else 0)
    _check_fia(case)


@pytest.mark.parametrize("seed", range(12))
def test_random_block_sparse(seed):
    rng = np.random.default_rng(1000 + seed)
    layout = str(rng.choice(["BNSD", "BSND"]))
    B = int(rng.integers(1, 3))
    KVN = int(rng.choice([1, 2]))
    QN = KVN * int(rng.choice([1, 2, 4]))
    Sq, Skv = int(rng.integers(1, 700)), int(rng.integers(1, 900))
    lq, lkv = rng.integers(1, Sq + 1, size=B), rng.integers(1, Skv + 1, size=B)
    if seed % 2 == 0:
        Y = int(rng.choice([256, 512]))
        case = W.make_bsa_fp8(f"rand_fp8_{seed}", layout=layout, B=B, QN=QN, KVN=KVN, Sq=Sq, Skv=Skv,
                              D=128, Y=Y, p=float(rng.uniform(0.2, 0.9)), lq=lq, lkv=lkv, seed=1010 + seed)
        ref = oracle.block_sparse(case)
    else:
        X, Y = int(rng.choice([64, 128, 200])), int(rng.choice([128, 256]))
        case = W.make_bsa(f"rand_bsa_{seed}", layout=layout,
                          dtype=torch.bfloat16 if rng.random() < 0.5 else torch.float16, B=B, QN=QN,
                          KVN=KVN, Sq=Sq, Skv=Skv, D=int(rng.choice([64, 128])), X=X, Y=Y,
                          p=float(rng.uniform(0.2, 0.9)), lq=lq, lkv=lkv, seed=1010 + seed)
        ref = oracle.block_sparse(case)
    say(f"[rand] {case.name} layout={layout} B={B} QN={QN} KVN={KVN} Sq={Sq} Skv={Skv} "
        f"X={case.X} Y={case.Y} lq={list(lq)} lkv={list(lkv)} dtype={case.dtype}")
    to_dev(case)
    p = bsa_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()


@pytest.mark.parametrize("seed", range(8))
def test_random_mla_decode(seed):
    rng = np.random.default_rng(1100 + seed)
    S = int(rng.choice([1, 1, 2, 3, 8, 16]))
    QN = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    B = int(rng.integers(1, 4))
    bs = int(rng.choice([16, 128]))
    lkv = rng.integers(0, 2500, size=B)
    lkv[rng.integers(B)] = int(rng.integers(1, 40))
    lq = rng.integers(1, S + 1, size=B) if S > 1 and rng.random() < 0.5 else None
    case = W.make_mla_decode(f"rand_mla_{seed}", layout=str(rng.choice(["BSND", "BNSD", "BSH"])),
                             dtype=torch.bfloat16 if rng.random() < 0.6 else torch.float16, B=B, QN=QN,
                             Sq=S, lq=lq, lkv=lkv, block_size=bs, pool_layout=int(rng.integers(2)),
                             seed=1110 + seed, extra_blocks=1, nan_pool=True)
    _check_fia(case)


@pytest.mark.parametrize("seed", range(12))
def test_random_tnd_band_and_paged(seed):
    # TND queries: the bottom-right band (sparse_mode 4) on a contiguous cache,
    # or a paged cache with block size 128, 512 or 1024 (TND constraints)
    rng = np.random.default_rng(1200 + seed)
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    KVN = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 5))
    pre, nxt = int(rng.integers(0, 400)), int(rng.integers(0, 200))
    if seed % 2 == 0:
        Dqk, Dv = [(64, 64), (128, 128), (192, 128)][rng.integers(3)]
        lq = rng.integers(1, 400, size=B)
        lkv = lq + rng.integers(0, 300, size=B)
        case = W.make_fia(f"rand_tnd_band_{seed}", layout="TND", dtype=dtype, B=B, QN=KVN * G, KVN=KVN,
                          Dqk=Dqk, Dv=Dv, sparse_mode=4, pre_tokens=pre, next_tokens=nxt, lq=lq,
                          lkv=lkv, seed=1210 + seed, mask_kind="template")
    else:
        mode = int(rng.choice([0, 3, 4]))
        lq = rng.integers(1, 300, size=B)
        lkv = lq + rng.integers(0, 3000, size=B)
        case = W.make_paged_prefill(f"rand_tnd_paged_{seed}", layout="TND", dtype=dtype, B=B,
                                    QN=KVN * G, KVN=KVN, D=int(rng.choice([64, 128])), lq=lq, lkv=lkv,
                                    block_size=(128, 512, 1024)[(seed // 2) % 3],
                                    pool_layout=int(rng.integers(2)), sparse_mode=mode,
                                    pre_tokens=pre if mode == 4 else W.INT_MAX,
                                    next_tokens=nxt if mode == 4 else W.INT_MAX,
                                    mask_kind="template" if mode else None, seed=1210 + seed,
                                    extra_blocks=2, nan_pool=True)
    _check_fia(case)


@pytest.mark.parametrize("seed", range(12))
def test_random_mla_variants(seed):
    # MLA decode beyond the plain form: the bottom-right band (sparse_mode 4,
    # block size 64 or 128), TND queries, and value passed as the key tensor
    rng = np.random.default_rng(1300 + seed)
    kind = seed % 3
    QN = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    B = int(rng.integers(1, 4))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float16
    vk = kind == 2 or bool(rng.random() < 0.3)
    if kind == 0:
        S = (1, 2, 4)[(seed // 3) % 3]
        lkv = rng.integers(S, 2500, size=B)
        band = (int(rng.integers(0, 1500)), int(rng.choice([0, 1, 5])))
        case = W.make_mla_decode(f"rand_mla_band_{seed}", dtype=dtype, B=B, QN=QN, Sq=S, lkv=lkv,
                                 block_size=int(rng.choice([64, 128])), band=band,
                                 pool_layout=int(rng.integers(2)), seed=1310 + seed,
                                 extra_blocks=2, nan_pool=True)
    elif kind == 1:
        lq = rng.integers(1, 17, size=B)
        lkv = rng.integers(0, 2500, size=B)
        case = W.make_mla_decode(f"rand_mla_tnd_{seed}", layout="TND", dtype=dtype, B=B, QN=QN, lq=lq,
                                 lkv=lkv, block_size=int(rng.choice([16, 128])), pool_layout=1,
                                 seed=1310 + seed, extra_blocks=2, nan_pool=True)
    else:
        S = int(rng.choice([1, 1, 2, 3, 8, 16]))
        lkv = rng.integers(0, 2500, size=B)
        case = W.make_mla_decode(f"rand_mla_vk_{seed}", layout=str(rng.choice(["BSND", "BNSD", "BSH"])),
                                 dtype=dtype, B=B, QN=QN, Sq=S, lkv=lkv,
                                 block_size=int(rng.choice([16, 128])), pool_layout=int(rng.integers(2)),
                                 seed=1310 + seed, extra_blocks=2, nan_pool=True)
    if vk:
        case.v = case.k
    say(f"[rand] {case.name} layout={case.layout} QN={QN} B={B} Sq={case.Sq} mode={case.sparse_mode} "
        f"band=({case.pre_tokens},{case.next_tokens}) lq={None if case.lq is None else list(case.lq)} "
        f"lkv={list(case.lkv)} bs={case.block_size} value=key={vk} dtype={dtype}")
    ref = oracle.attention(case)
    to_dev(case)
    if vk:
        case.v = case.k                  # one device tensor for both
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()
