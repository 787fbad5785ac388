"""GPU parity of the cache insert (msa_cache_insert through the C ABI) with the
oracle's insert: every byte of the K / V planes, the scale arrays and the
index cache, on caches filled with random bytes beforehand; then a decode step
run on caches written by the insert against the oracle on its own insert."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _case(seed, T, num_pages, kv_fp8, scale_mode, with_index, layout="random"):
    rng = syn.SplitMix64(seed)
    # magnitudes spread over ~2^-20 .. 2^6 so that scaled values reach the
    # e4m3 subnormal range, plus whole rows of zeros
    mag = np.exp2(rng.uniform(T).reshape(T, 1, 1) * 26.0 - 20.0)
    k = rng.normal(T * 128).reshape(T, 1, 128) * mag
    v = rng.normal(T * 128).reshape(T, 1, 128) * mag[::-1]
    k[3], v[5] = 0.0, 0.0
    ik = rng.normal(T * 128).reshape(T, 128)
    if layout == "random":                  # decode-like: scattered slots
        slots = rng.permutation(num_pages * 128)[:T].astype(np.int32)
        drop = rng.uniform(T) < 0.1
        slots[drop] = -1
        slots[7] = num_pages * 128 + 5      # outside the caches: skipped
    else:                                   # a prefill chunk: tokens fill permuted pages in order
        start = 0 if layout == "chunk" else 8
        perm = rng.permutation(num_pages)
        pos = start + np.arange(T)
        slots = (perm[pos // 128] * 128 + pos % 128).astype(np.int32)
        if layout == "chunk":
            slots[40] = -1                  # one sub-page not whole: its tokens go one by one
            slots[70], slots[71] = slots[71], slots[70]   # and one out of order
    nbytes = 1 if kv_fp8 else 2
    sub_elems = num_pages * 8 * 16 * 128
    garbage = rng.integers(0, (1 << (8 * nbytes)) - 1, 2 * sub_elems + num_pages * 128 * 128)
    dt = np.uint8 if kv_fp8 else np.uint16
    kc = garbage[:sub_elems].astype(dt).reshape(num_pages * 8, 1, 4, 4, 16, 8)
    vc = garbage[sub_elems:2 * sub_elems].astype(dt).reshape(num_pages * 8, 1, 128, 16)
    ikc = (garbage[2 * sub_elems:] & 0xFFFF).astype(np.uint16).reshape(num_pages, 8, 4, 4, 16, 8)
    if scale_mode == 2:
        ks = rng.uniform(num_pages * 128).astype(np.float32).reshape(num_pages * 8, 16, 1) + 7.0
        vs = rng.uniform(num_pages * 128).astype(np.float32).reshape(num_pages * 8, 16, 1) + 9.0
    elif scale_mode == 1:
        ks, vs = np.array([0.375], np.float32), np.array([1.5], np.float32)
    else:
        ks = vs = None
    return dict(T=T, P=num_pages, kv_dtype=1 if kv_fp8 else 0, scale_mode=scale_mode,
                k_new=syn.to_bf16_bits(k), v_new=syn.to_bf16_bits(v),
                ik_new=syn.to_bf16_bits(ik) if with_index else None, slots=slots,
                kc=kc, vc=vc, ikc=ikc, ks=ks, vs=vs)


def _run_device(c):
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, vc, ikc, ks, vs = dev(c["kc"]), dev(c["vc"]), dev(c["ikc"]), dev(c["ks"]), dev(c["vs"])
    kv = msa.make_kv(kc, vc, c["kv_dtype"], c["scale_mode"], c["P"], ks, vs)
    msa.msa_cache_insert(c["T"], dev(c["slots"]), dev(c["k_new"]), dev(c["v_new"]), kv,
                         dev(c["ik_new"]), ikc)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy()
    return host(kc), host(vc), host(ks), host(vs), host(ikc)


CASES = [
    # (kv fp8, scale mode, index rows)
    (False, syn.SCALE_NONE, True),
    (False, syn.SCALE_SCALAR, True),
    (False, syn.SCALE_PER_TOKEN_HEAD, False),
    (True, syn.SCALE_SCALAR, True),
    (True, syn.SCALE_PER_TOKEN_HEAD, True),
    (True, syn.SCALE_PER_TOKEN_HEAD, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("T,layout", [(37, "random"), (2048, "random"), (2088, "chunk"), (300, "chunk_offset")])
def test_insert_bitexact(gpu_lib, case, T, layout):
    fp8, sm, with_index = CASES[case]
    c = _case(200 + 10 * case + T % 7, T, max(24, T // 64), fp8, sm, with_index, layout)
    print(f"[insert] fp8={fp8} scale_mode={sm} index={with_index} T={T} slots={layout}", flush=True)
    want = O.cache_insert(c["kc"], c["vc"], c["ks"], c["vs"], c["ikc"], c["slots"], c["k_new"], c["v_new"],
                          c["ik_new"], c["kv_dtype"], c["scale_mode"])
    got = _run_device(c)
    for name, g, w in zip(("k_cache", "v_cache", "k_scale", "v_scale", "index_k"), got, want):
        if w is None:
            continue
        g = np.asarray(g).view(np.uint32) if g.dtype == np.float32 else g
        w = np.asarray(w).view(np.uint32) if w.dtype == np.float32 else w
        bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
        assert bad.size == 0, f"{name}: {bad.size} elements differ, first at flat index {bad[:5].tolist()}"


def test_insert_then_fused_decode_matches_oracle(gpu_lib):
    """Each request's newest token goes in through the insert (fp8 caches,
    per-token-head scales); the fused step on those caches matches the oracle
    step on the oracle's own insert."""
    b = syn.make_batch("insdec", 260, [9000, 3000, 700], [1, 1, 2], topk=16, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    rng = syn.SplitMix64(261)
    new_tok = [(r, int(L) - 1 - i) for r, (L, ql) in enumerate(zip(b.seq_lens, b.query_lens)) for i in range(int(ql))]
    T = len(new_tok)
    slots = np.array([int(b.block_table[r, t // 128]) * 128 + t % 128 for r, t in new_tok], np.int32)
    k_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 1, 128) * 1.7)
    v_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 1, 128) * 0.6)
    ik_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 128))
    kc, vc, ks, vs, ik = O.cache_insert(b.k_cache, b.v_cache, b.k_scale, b.v_scale, b.index_k, slots,
                                        k_new, v_new, ik_new, b.kv_dtype, b.scale_mode)
    b_ref = dataclasses.replace(b, k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs, index_k=ik)
    d = H.upload(b)            # the original caches: the insert overwrites the new tokens
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    msa.msa_cache_insert(T, dev(slots), dev(k_new), dev(v_new), d.ckv, dev(ik_new), d.index_k)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    torch.cuda.synchronize()
    assert np.array_equal(d.k_cache.cpu().numpy(), kc)
    assert np.array_equal(d.index_k.cpu().numpy().view(np.uint16), ik)
    ref = O.decode_step(b_ref, scores_fp32=o.scores.cpu().numpy())
    rows = list(range(b.num_rows))
    table, ctx = o.table.cpu().numpy(), o.ctx.cpu().numpy()
    assert table.tolist() == ref["table"].tolist() and ctx.tolist() == ref["ctx"].tolist()
    out = H.bf16_to_np(o.out)
    err = np.abs(out[rows] - ref["out"]).max()
    assert err <= 6e-2, f"attention after insert: max abs err {err}"
