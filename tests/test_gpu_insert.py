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


# Values exactly halfway between two storage codes, as in the oracle's tie
# pins: e4m3fn midpoints (stored with scale 1), and 1.5 / 3.0 under the two
# scalar scales that put fl32(x / s) on a bf16 midpoint.
E4M3_MIDPOINTS = np.array([1.0625, 1.1875, 1.9375, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10,
                           15 * 2.0 ** -10, 400.0, 432.0])
BF16_TIE_K_SCALE = np.array([0x3FBF40BF], np.uint32).view(np.float32)   # 1.5 / s = 1 + 2^-8: rounds down
BF16_TIE_V_SCALE = np.array([0x3FBDC6AC], np.uint32).view(np.float32)   # 1.5 / s = 1 + 3*2^-8: rounds up


def _tie_rows(rng, T, values, anchor):
    """T rows of 128: tie values with random signs at random places, the
    rest zero, and +-anchor in one slot (448 makes a per-token scale of 1)."""
    x = np.zeros((T, 128))
    pick = (rng.uniform(T * 128).reshape(T, 128) * len(values)).astype(np.int64)
    sign = np.where(rng.uniform(T * 128).reshape(T, 128) < 0.5, -1.0, 1.0)
    x[:] = values[pick] * sign
    if anchor is not None:
        x[np.arange(T), (np.arange(T) * 37) % 128] = anchor * sign[:, 0]
    return x


@pytest.mark.parametrize("mode", ["fp8_scalar", "fp8_per_token_head", "bf16_scalar", "fp8_index"])
def test_insert_rounding_ties_bitexact(gpu_lib, mode):
    """Rows made of exact midpoints between storage codes: the device stores
    the same (even) neighbour as the oracle, byte for byte, on both insert
    paths (whole in-order sub-pages and scattered single tokens)."""
    T, P = 160, 8
    rng = syn.SplitMix64(290 + len(mode))
    perm = rng.permutation(P)
    pos = np.arange(T)
    slots = (perm[pos // 128] * 128 + pos % 128).astype(np.int32)     # tokens 0..127: whole sub-pages
    # the scattered tail must not hit the in-order tokens' slots
    used = set(slots[:128].tolist())
    free = [s for s in rng.permutation(P * 128).tolist() if s not in used]
    slots[128:] = np.array(free[:32], np.int32)
    print(f"[insert ties] {mode}", flush=True)
    if mode == "bf16_scalar":
        vals = np.array([1.5, 3.0])
        k, v = _tie_rows(rng, T, vals, None), _tie_rows(rng, T, vals, None)
        kv_dtype, sm, ks, vs = 0, syn.SCALE_SCALAR, BF16_TIE_K_SCALE.copy(), BF16_TIE_V_SCALE.copy()
    else:
        anchor = 448.0 if mode != "fp8_scalar" else None
        k, v = _tie_rows(rng, T, E4M3_MIDPOINTS, anchor), _tie_rows(rng, T, E4M3_MIDPOINTS, anchor)
        kv_dtype = 1
        if mode == "fp8_scalar":
            sm, ks, vs = syn.SCALE_SCALAR, np.array([1.0], np.float32), np.array([1.0], np.float32)
        else:
            sm = syn.SCALE_PER_TOKEN_HEAD
            ks = np.full((P * 8, 16, 1), 5.0, np.float32)
            vs = np.full((P * 8, 16, 1), 5.0, np.float32)
    elt = np.uint8 if kv_dtype == 1 else np.uint16
    kc = rng.integers(0, 255, P * 8 * 2048).astype(elt).reshape(P * 8, 1, 4, 4, 16, 8)
    vc = rng.integers(0, 255, P * 8 * 2048).astype(elt).reshape(P * 8, 1, 128, 16)
    k_bits, v_bits = syn.to_bf16_bits(k[:, None, :]), syn.to_bf16_bits(v[:, None, :])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dkc, dvc, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    kv = msa.make_kv(dkc, dvc, kv_dtype, sm, P, dks, dvs)
    want = O.cache_insert(kc, vc, ks, vs, None, slots, k_bits, v_bits, None, kv_dtype, sm)
    if mode == "fp8_index":
        ik = syn.to_bf16_bits(_tie_rows(rng, T, E4M3_MIDPOINTS, 448.0))
        ikc = rng.integers(0, 255, P * 128 * 128).astype(np.uint8).reshape(P, 8, 4, 4, 16, 8)
        isc = np.full((P, 128), 3.0, np.float32)
        dikc, disc = dev(ikc), dev(isc)
        msa.msa_cache_insert_ex(T, dev(slots), dev(k_bits), dev(v_bits), kv, dev(ik), dikc, disc)
        want_ik, want_isc = O.index_insert_fp8(ikc, isc, slots, ik)
    else:
        msa.msa_cache_insert(T, dev(slots), dev(k_bits), dev(v_bits), kv, None, None)
    torch.cuda.synchronize()
    got = {"k_cache": dkc.cpu().numpy(), "v_cache": dvc.cpu().numpy()}
    exp = {"k_cache": want[0], "v_cache": want[1]}
    if sm == syn.SCALE_PER_TOKEN_HEAD:
        got["k_scale"], exp["k_scale"] = dks.cpu().numpy().view(np.uint32), want[2].view(np.uint32)
        got["v_scale"], exp["v_scale"] = dvs.cpu().numpy().view(np.uint32), want[3].view(np.uint32)
        assert np.all(want[2].reshape(-1)[slots] == 1.0), "every written token-head has scale 1"
    if mode == "fp8_index":
        got["index_k"], exp["index_k"] = dikc.cpu().numpy(), want_ik
        got["index_scale"], exp["index_scale"] = disc.cpu().numpy().view(np.uint32), want_isc.view(np.uint32)
    for name in got:
        bad = np.flatnonzero(got[name].reshape(-1) != exp[name].reshape(-1))
        assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[:5].tolist()}"
