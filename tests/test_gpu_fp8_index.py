"""GPU parity on an FP8 index cache (e4m3fn codes, one fp32 scale per token):
the scores (msa_index_score_ex), the fused step (msa_sparse_decode_ex) and the
insert of new index keys (msa_cache_insert_ex) through the C ABI, against the
oracle on the same seeded inputs. Bars as for the bf16 index: scores within
1e-3 * max(|oracle|, 1) with exact -inf tails; selection, tables and context
lengths bit-exact on the device's own scores; attention within 2e-2 / 6e-2;
the insert bit-exact on every byte and scale."""
import numpy as np
import pytest
import torch

import block_sparse_paged_msa_amd as msa
import msa_synth as syn
from oracle import msa_oracle as O
from tests import helpers as H
from tests.test_gpu_parity import check_attention, check_metadata, check_scores, check_selection

pytestmark = pytest.mark.gpu

SHAPES = [
    # (name, lengths, query rows, top-k): decode rows, speculative rows, a
    # prefill request past 64 rows (extra row groups), ragged tails, an empty request
    ("decode", [9000, 700, 129, 1, 20000], [1, 1, 1, 1, 1], 16),
    ("spec", [65536, 3000, 0, 4100], [4, 4, 0, 3], 32),
    ("prefill", [5000, 3000, 8000], [1, 200, 70], 8),
]


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_fp8_index_scores(gpu_lib, case):
    name, L, ql, topk = SHAPES[case]
    b = syn.make_batch(name, 600 + case, L, ql, topk=topk, num_q_heads=16, index_dtype=syn.INDEX_FP8)
    print(f"[fp8 index] scores {name} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    H.run_metadata(d)
    scores = H.run_scores(d)
    check_scores(b, scores, list(range(b.num_rows)))


@pytest.mark.parametrize("kv,sm", [(syn.KV_BF16, syn.SCALE_NONE), (syn.KV_FP8, syn.SCALE_PER_TOKEN_HEAD)])
@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_fused_decode_on_fp8_index(gpu_lib, case, kv, sm):
    name, L, ql, topk = SHAPES[case]
    b = syn.make_batch(name, 610 + case, L, ql, topk=topk, num_q_heads=16, kv_dtype=kv, scale_mode=sm,
                       index_dtype=syn.INDEX_FP8)
    print(f"[fp8 index] fused {name} kv={kv} rows={b.num_rows}", flush=True)
    d = H.upload(b)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    check_metadata(b, H.read_metadata(d))
    scores = o.scores.cpu().numpy()
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    rows = list(range(b.num_rows))
    check_scores(b, scores, rows)
    check_selection(b, scores, table, ctx, sel, rows)
    check_attention(b, H.bf16_to_np(o.out), table, ctx, rows)
    # the standalone scores give the same bits
    H.run_metadata(d)
    assert np.array_equal(H.run_scores(d), scores)


def _insert_case(seed, T, P, layout):
    rng = syn.SplitMix64(seed)
    mag = np.exp2(rng.uniform(T).reshape(T, 1) * 26.0 - 20.0)
    ik = rng.normal(T * 128).reshape(T, 128) * mag
    ik[4] = 0.0                                     # an all-zero key: scale 1
    k = rng.normal(T * 128).reshape(T, 1, 128)
    v = rng.normal(T * 128).reshape(T, 1, 128)
    if layout == "random":
        slots = rng.permutation(P * 128)[:T].astype(np.int32)
        slots[rng.uniform(T) < 0.1] = -1
        slots[2] = P * 128 + 9
    else:
        perm = rng.permutation(P)
        pos = np.arange(T)
        slots = (perm[pos // 128] * 128 + pos % 128).astype(np.int32)
        slots[33] = -1                              # that sub-page goes token by token
    ikc = rng.integers(0, 255, P * 128 * 128).astype(np.uint8).reshape(P, 8, 4, 4, 16, 8)
    isc = (rng.uniform(P * 128) + 3.0).astype(np.float32).reshape(P, 128)
    kc = rng.integers(0, 255, P * 8 * 2048).astype(np.uint8).reshape(P * 8, 1, 4, 4, 16, 8)
    vc = rng.integers(0, 255, P * 8 * 2048).astype(np.uint8).reshape(P * 8, 1, 128, 16)
    ks = (rng.uniform(P * 128) + 1.0).astype(np.float32).reshape(P * 8, 16, 1)
    vs = (rng.uniform(P * 128) + 1.0).astype(np.float32).reshape(P * 8, 16, 1)
    return dict(T=T, P=P, slots=slots, k=syn.to_bf16_bits(k), v=syn.to_bf16_bits(v), ik=syn.to_bf16_bits(ik),
                ikc=ikc, isc=isc, kc=kc, vc=vc, ks=ks, vs=vs)


@pytest.mark.parametrize("T,layout", [(45, "random"), (2048, "random"), (1024, "chunk")])
def test_insert_fp8_index_bitexact(gpu_lib, T, layout):
    c = _insert_case(620 + T % 11, T, max(16, T // 64), layout)
    print(f"[fp8 index] insert T={T} slots={layout}", flush=True)
    want_ik, want_isc = O.index_insert_fp8(c["ikc"], c["isc"], c["slots"], c["ik"])
    want = O.cache_insert(c["kc"], c["vc"], c["ks"], c["vs"], None, c["slots"], c["k"], c["v"], None, 1, 2)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, vc, ks, vs, ikc, isc = (dev(c[x]) for x in ("kc", "vc", "ks", "vs", "ikc", "isc"))
    kv = msa.make_kv(kc, vc, 1, 2, c["P"], ks, vs)
    msa.msa_cache_insert_ex(c["T"], dev(c["slots"]), dev(c["k"]), dev(c["v"]), kv, dev(c["ik"]), ikc, isc)
    torch.cuda.synchronize()
    got = dict(k_cache=kc.cpu().numpy(), v_cache=vc.cpu().numpy(), k_scale=ks.cpu().numpy().view(np.uint32),
               v_scale=vs.cpu().numpy().view(np.uint32), index_k=ikc.cpu().numpy(),
               index_scale=isc.cpu().numpy().view(np.uint32))
    exp = dict(k_cache=want[0], v_cache=want[1], k_scale=want[2].view(np.uint32), v_scale=want[3].view(np.uint32),
               index_k=want_ik, index_scale=want_isc.view(np.uint32))
    for name in got:
        bad = np.flatnonzero(got[name].reshape(-1) != exp[name].reshape(-1))
        assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[:5].tolist()}"


def test_insert_then_decode_on_fp8_index(gpu_lib):
    """New tokens' index keys go in through the insert (fp8 index cache); the
    fused step on the written caches selects exactly as the oracle selector on
    the device's scores, and its scores match the oracle's on the oracle's own
    insert."""
    b = syn.make_batch("f8ins", 630, [9000, 3000, 700], [1, 2, 1], topk=16, num_q_heads=16,
                       index_dtype=syn.INDEX_FP8)
    rng = syn.SplitMix64(631)
    new_tok = [(r, int(L) - 1 - i) for r, (L, ql) in enumerate(zip(b.seq_lens, b.query_lens)) for i in range(int(ql))]
    T = len(new_tok)
    slots = np.array([int(b.block_table[r, t // 128]) * 128 + t % 128 for r, t in new_tok], np.int32)
    k_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 1, 128))
    v_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 1, 128))
    ik_new = syn.to_bf16_bits(rng.normal(T * 128).reshape(T, 128) * 3.0)
    kc, vc, _, _, _ = O.cache_insert(b.k_cache, b.v_cache, None, None, None, slots, k_new, v_new, None, 0, 0)
    ik, isc = O.index_insert_fp8(b.index_k, b.index_scale, slots, ik_new)
    import dataclasses
    b_ref = dataclasses.replace(b, k_cache=kc, v_cache=vc, index_k=ik, index_scale=isc)
    d = H.upload(b)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    msa.msa_cache_insert_ex(T, dev(slots), dev(k_new), dev(v_new), d.ckv, dev(ik_new), d.index_k, d.index_scale)
    o = H.alloc_decode(d)
    H.run_decode(d, o)
    torch.cuda.synchronize()
    assert np.array_equal(d.index_k.cpu().numpy(), ik)
    assert np.array_equal(d.index_scale.cpu().numpy().view(np.uint32), isc.view(np.uint32))
    rows = list(range(b.num_rows))
    scores = o.scores.cpu().numpy()
    check_scores(b_ref, scores, rows)
    table, ctx, sel = o.table.cpu().numpy(), o.ctx.cpu().numpy(), o.sel.cpu().numpy()
    check_selection(b_ref, scores, table, ctx, sel, rows)
    check_attention(b_ref, H.bf16_to_np(o.out), table, ctx, rows)
