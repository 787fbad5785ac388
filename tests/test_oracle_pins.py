"""Pins of the CPU oracle against things other than itself.

Every check here ties an oracle function to a closed form, a brute-force
enumeration, an independent library routine, a hand-derived fixture or an
invariant of the mathematics, so that a dropped term, a wrong index or sign, or
a transposed operand in the oracle fails at least one test. No GPU is used.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import msa_synth as syn

if os.environ.get("MSA_ORACLE_UNDER_TEST"):
    # a copy of the oracle with one planted mistake (tests/test_oracle_mutations.py):
    # the pins below must fail on it
    import importlib.util
    _spec = importlib.util.spec_from_file_location("msa_oracle_under_test", os.environ["MSA_ORACLE_UNDER_TEST"])
    O = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(O)
else:
    from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers written independently of the oracle: a writer that scatters logical
# per-token arrays into the paged layouts, and bf16 / fp8 encoders from torch
# ---------------------------------------------------------------------------
def bf16_bits(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def fp8_codes(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def shuffle_into(tile, tok, row):
    # token `tok` of a [4][4][16][8] tile: dim d -> [d // 32][(d % 32) // 8][tok][d % 8]
    for d in range(128):
        tile[d // 32, (d % 32) // 8, tok, d % 8] = row[d]


def write_paged(logical_k, logical_v, page_of_block, num_pages, dtype=np.uint16):
    """Scatter logical K [T][Hkv][D] and V [T][Hkv][D] (already encoded) into
    K sub-pages [8P][Hkv][4][4][16][8] (shuffled tiles) and V sub-pages
    [8P][Hkv][D][16] (dim-major)."""
    T, hkv, D = logical_k.shape
    kc = np.zeros((num_pages * 8, hkv, 4, 4, 16, 8), dtype=dtype)
    vc = np.zeros((num_pages * 8, hkv, D, 16), dtype=dtype)
    for t in range(T):
        page = page_of_block[t // 128]
        sub = page * 8 + (t % 128) // 16
        for h in range(hkv):
            shuffle_into(kc[sub, h], t % 16, logical_k[t, h])
            vc[sub, h, :, t % 16] = logical_v[t, h]
    return kc, vc


def write_scales(logical_s, page_of_block, num_pages):
    T, hkv = logical_s.shape
    s = np.ones((num_pages * 8, 16, hkv), dtype=np.float32)
    for t in range(T):
        page = page_of_block[t // 128]
        s[page * 8 + (t % 128) // 16, t % 16] = logical_s[t]
    return s


def write_index_pages(logical_ik, page_of_block, num_pages):
    T, D = logical_ik.shape
    out = np.zeros((num_pages, 8, 4, 4, 16, 8), dtype=np.uint16)
    for t in range(T):
        s = t % 128
        shuffle_into(out[page_of_block[t // 128], s // 16], s % 16, logical_ik[t])
    return out


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # the signalling-NaN patterns raise the invalid flag when widened
        ours = O.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0xB8, -1.0), (0x77, 240.0),
])
def test_e4m3fn_spec_values(code, value):
    # values fixed by the OCP 8-bit floating point specification (E4M3, bias 7)
    assert O.e4m3fn_to_f64(np.array([code], np.uint8))[0] == value


def test_e4m3fn_nan_and_negative_zero():
    v = O.e4m3fn_to_f64(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1])
    assert v[2] == 0.0 and math.copysign(1.0, v[2]) == -1.0


# ---------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------
def test_metadata_hand_derived_example():
    g = json.load(open(os.path.join(GOLDEN, "metadata_example.json")))
    m = O.build_metadata(np.array(g["seq_lens"]), np.array(g["query_lens"]))
    for key in ("cu_seqlens_q", "cu_seqlens_k", "cu_blocks", "row_req", "row_pos"):
        assert m[key].tolist() == g[key], key


@pytest.mark.parametrize("seed", range(5))
def test_metadata_invariants(seed):
    rng = syn.SplitMix64(100 + seed)
    R = int(rng.integers(1, 40, 1)[0])
    L = rng.integers(0, 5000, R)
    ql = np.minimum(rng.integers(0, 9, R), L)
    m = O.build_metadata(L, ql)
    # library prefix sums
    assert m["cu_seqlens_k"].tolist() == [0] + np.cumsum(L).tolist()
    assert m["cu_seqlens_q"].tolist() == [0] + np.cumsum(ql).tolist()
    assert m["cu_blocks"].tolist() == [0] + np.cumsum(-(-L // 128)).tolist()
    # every request's last row sits at position L-1, rows are contiguous per request
    for r in range(R):
        rows = np.nonzero(m["row_req"] == r)[0]
        assert len(rows) == ql[r]
        if ql[r]:
            assert rows.tolist() == list(range(m["cu_seqlens_q"][r], m["cu_seqlens_q"][r + 1]))
            assert m["row_pos"][rows[-1]] == L[r] - 1
            assert np.all(np.diff(m["row_pos"][rows]) == 1)


def test_metadata_prefill_slice_matches_page_formula():
    # the prefill metadata of the PR #56170 page is the prefill part of the
    # batch: cu_seqlens_q = query_start_loc[num_decodes:] - num_decode_tokens and
    # cu_seqlens_k = [0, cumsum(seq_lens[num_decodes:])]
    L = np.array([16384] * 6 + [32768, 5000])
    ql = np.array([1] * 6 + [4096, 17])
    nd = 6
    m = O.build_metadata(L, ql)
    qsl = np.concatenate([[0], np.cumsum(ql)])
    assert (m["cu_seqlens_q"][nd:] - m["cu_seqlens_q"][nd]).tolist() == (qsl[nd:] - qsl[nd]).tolist()
    pf = np.empty(len(L) - nd + 1, dtype=np.int64)
    pf[:1] = 0
    np.cumsum(L[nd:], out=pf[1:])
    assert (m["cu_seqlens_k"][nd:] - m["cu_seqlens_k"][nd]).tolist() == pf.tolist()
    ctx = L - ql
    first_prefill_row = int(qsl[nd])
    assert m["row_pos"][first_prefill_row] == ctx[nd]


# ---------------------------------------------------------------------------
# scores and pooling
# ---------------------------------------------------------------------------
def _one_request(seed, L, nreq_pages_extra=3):
    rng = syn.SplitMix64(seed)
    nb = -(-L // 128)
    P = nb + nreq_pages_extra
    pages = rng.permutation(P)[:nb]
    logical = syn.bf16_normal(rng, (L, 128))
    ik = write_index_pages(logical, pages, P)
    return pages, logical, ik


def test_scores_one_hot_query_reads_one_coordinate():
    L = 300
    pages, logical, ik = _one_request(1, L)
    for d in (0, 37, 127):
        q = np.zeros(128, np.float32)
        q[d] = 1.0
        keys = O.index_keys_of_request(ik, pages, L)
        s = O.token_scores(bf16_bits(q), keys, L)
        np.testing.assert_array_equal(s, O.bf16_to_f64(logical[:, d]))


def test_scores_all_ones_equal_dim():
    L = 200
    ik = np.full((2, 8, 4, 4, 16, 8), bf16_bits([1.0])[0], np.uint16)
    keys = O.index_keys_of_request(ik, np.array([1, 0]), L)
    s = O.token_scores(bf16_bits(np.ones(128)), keys, L)
    assert np.all(s == 128.0)


def test_scores_brute_force_tiny():
    L = 150
    pages, logical, ik = _one_request(2, L)
    rng = syn.SplitMix64(3)
    q = syn.bf16_normal(rng, (128,))
    keys = O.index_keys_of_request(ik, pages, L)
    s = O.token_scores(q, keys, L)
    qf = [float(x) for x in torch.from_numpy(q.view(np.int16).copy()).view(torch.bfloat16).float()]
    for t in range(L):
        page, slot = int(pages[t // 128]), t % 128
        raw = np.array([ik[page, slot // 16, d // 32, (d % 32) // 8, slot % 16, d % 8] for d in range(128)], np.uint16)
        row = torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).float()
        ref = math.fsum(qf[d] * float(row[d]) for d in range(128))
        assert abs(s[t] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_scores_invariant_under_page_permutation():
    L = 700
    rng = syn.SplitMix64(4)
    logical = syn.bf16_normal(rng, (L, 128))
    q = syn.bf16_normal(rng, (128,))
    nb = -(-L // 128)
    outs = []
    for seed in (5, 6):
        pages = syn.SplitMix64(seed).permutation(nb + 2)[:nb]
        ik = write_index_pages(logical, pages, nb + 2)
        outs.append(O.token_scores(q, O.index_keys_of_request(ik, pages, L), L))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_pool_planted_maxima_and_partial_block():
    L = 3 * 128 + 10           # 4 blocks, the last one partial
    rng = syn.SplitMix64(7)
    logical = bf16_bits(0.01 * O.bf16_to_f64(syn.bf16_normal(rng, (L + 118, 128))))
    logical = logical.reshape(L + 118, 128)
    q = np.zeros(128, np.float32)
    q[5] = 1.0
    # values at block edges catch a pooled range that is off by one at either end
    planted = {0: (17, 3.0), 1: (128, 5.0), 2: (383, 4.0), 3: (384 + 9, 2.5)}
    for b, (t, val) in planted.items():
        logical[t, 5] = bf16_bits([val])[0]
    # a huge value in the invisible tail of block 3 must not be pooled
    logical[384 + 50, 5] = bf16_bits([100.0])[0]
    pages = np.array([3, 0, 2, 1])
    ik = write_index_pages(logical, pages, 4)
    keys = O.index_keys_of_request(ik, pages, L + 118)
    s = O.token_scores(bf16_bits(q), keys, L)
    pooled = O.pool_blocks(s, 4)
    assert pooled.tolist() == [3.0, 5.0, 4.0, 2.5]


def test_block_scores_tail_is_minus_inf_and_rows_follow_positions():
    b = syn.make_batch("t", 9, seq_lens=[300, 129], query_lens=[3, 2], topk=2, num_q_heads=16,
                       max_seq_len=1024)
    s = O.block_scores(b.index_q, b.index_k, b.block_table, b.seq_lens, b.query_lens, b.ld_s)
    # request 0 rows at pos 297, 298, 299 -> 3 blocks; request 1 rows at 127, 128 -> 1, 2 blocks
    nbs = [3, 3, 3, 1, 2]
    for n, nb in enumerate(nbs):
        assert np.all(np.isfinite(s[n, :nb]))
        assert np.all(s[n, nb:] == -np.inf)


# ---------------------------------------------------------------------------
# selection, table, context length
# ---------------------------------------------------------------------------
def test_table_and_ctx_hand_derived_cases():
    g = json.load(open(os.path.join(GOLDEN, "table_example.json")))
    for c in g["cases"]:
        nb = O.num_blocks(c["v"])
        sel = O.select_blocks(np.array(c["scores"]), nb, c["topk"])
        assert O.selection_row_outputs(sel, c["topk"]).tolist()[:len(c["sel"])] == c["sel"]
        tab = O.sparse_table_row(sel, np.array(c["bt_row"]), c["topk"])
        assert len(tab) == 8 * c["topk"]
        assert tab.tolist()[:len(c["table"])] == c["table"]
        assert np.all(tab[len(c["table"]):] == 0)
        assert O.context_length(sel, c["v"]) == c["ctx"]


def _greedy_select(scores, nb, topk):
    # brute force: repeatedly extract the best remaining block (max score, then
    # lowest id), then list the extracted ids in ascending order
    left = list(range(nb))
    got = []
    for _ in range(min(topk, nb)):
        best = left[0]
        for b in left[1:]:
            if scores[b] > scores[best]:
                best = b
        got.append(best)
        left.remove(best)
    return sorted(got)


@pytest.mark.parametrize("seed", range(12))
def test_selection_formulations_agree(seed):
    rng = syn.SplitMix64(200 + seed)
    nb = int(rng.integers(1, 70, 1)[0])
    topk = int(rng.integers(1, 80, 1)[0])
    mode = seed % 3
    if mode == 0:
        s = rng.normal(nb)
    elif mode == 1:                       # heavy ties
        s = np.round(rng.normal(nb) * 2) / 2
    else:                                 # signed zeros and a few values
        s = np.where(rng.uniform(nb) < 0.5, 0.0, -0.0)
        s[rng.integers(0, nb - 1, 3)] = 1.0
    a = O.select_blocks(s, nb, topk)
    b = O.select_blocks_by_rank(s, nb, topk)
    c = _greedy_select(s, nb, topk)
    assert a.tolist() == b.tolist() == c
    assert len(a) == min(topk, nb)


def test_selection_all_signed_zeros_picks_lowest_ids():
    s = np.array([-0.0, 0.0, -0.0, 0.0, 0.0, -0.0])
    assert O.select_blocks(s, 6, 4).tolist() == [0, 1, 2, 3]


def test_selection_ignores_scores_past_nb():
    s = np.array([1.0, 2.0, 3.0, 99.0, 98.0])
    assert O.select_blocks(s, 3, 2).tolist() == [1, 2]


def test_table_never_exceeds_width_and_encodes_subpages():
    rng = syn.SplitMix64(11)
    for _ in range(20):
        nb = int(rng.integers(1, 30, 1)[0])
        topk = int(rng.integers(1, 40, 1)[0])
        bt = rng.permutation(nb + 5)[:nb]
        sel = O.select_blocks(rng.normal(nb), nb, topk)
        tab = O.sparse_table_row(sel, bt, topk)
        assert tab.shape == (8 * topk,)
        for j, blk in enumerate(sel):
            assert (tab[8 * j:8 * j + 8] // 8 == bt[blk]).all()
            assert (tab[8 * j:8 * j + 8] % 8 == np.arange(8)).all()
        assert (tab[8 * len(sel):] == 0).all()


def test_ctx_all_blocks_equals_visible_keys():
    for v in (1, 127, 128, 129, 1000, 4096):
        nb = O.num_blocks(v)
        assert O.context_length(np.arange(nb), v) == v


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _paged_kv_case(seed, L, hq=8, kv_fp8=False, per_token_scales=False):
    rng = syn.SplitMix64(seed)
    nb = -(-L // 128)
    P = nb + 2
    pages = rng.permutation(P)[:nb]
    if kv_fp8:
        kl = syn.fp8_normal(rng, (L, 1, 128))
        vl = syn.fp8_normal(rng, (L, 1, 128))
        kc, vc = write_paged(kl, vl, pages, P, dtype=np.uint8)
        kf = torch.from_numpy(kl.copy()).view(torch.float8_e4m3fn).double().numpy()
        vf = torch.from_numpy(vl.copy()).view(torch.float8_e4m3fn).double().numpy()
    else:
        kl = syn.bf16_normal(rng, (L, 1, 128))
        vl = syn.bf16_normal(rng, (L, 1, 128))
        kc, vc = write_paged(kl, vl, pages, P)
        kf = torch.from_numpy(kl.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
        vf = torch.from_numpy(vl.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ks = vs = None
    mode = 0
    if per_token_scales:
        mode = 2
        ksl = (0.5 + 1.5 * rng.uniform(L)).astype(np.float32).reshape(L, 1)
        vsl = (0.5 + 1.5 * rng.uniform(L)).astype(np.float32).reshape(L, 1)
        ks = write_scales(ksl, pages, P)
        vs = write_scales(vsl, pages, P)
        kf = kf * ksl.astype(np.float64)[:, :, None]
        vf = vf * vsl.astype(np.float64)[:, :, None]
    q = syn.bf16_normal(rng, (hq, 128))
    qf = torch.from_numpy(q.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return dict(pages=pages, kc=kc, vc=vc, ks=ks, vs=vs, mode=mode, q=q, qf=qf, kf=kf, vf=vf,
                dtype=1 if kv_fp8 else 0)


def _sdpa(qf, kf, vf, v, scale):
    # library routine: torch's scaled-dot-product attention on the logical arrays
    q = torch.from_numpy(qf)[None, :, None, :]                          # [1,H,1,D]
    k = torch.from_numpy(kf[:v, 0, :]).expand(qf.shape[0], v, 128)[None]
    vv = torch.from_numpy(vf[:v, 0, :]).expand(qf.shape[0], v, 128)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("fp8,pth", [(False, False), (True, False), (True, True)])
def test_dense_attention_matches_torch_sdpa_through_paged_layout(fp8, pth):
    L = 333
    c = _paged_kv_case(20, L, kv_fp8=fp8, per_token_scales=pth)
    sc = 1 / math.sqrt(128)
    got = O.dense_causal_attention_row(c["q"], c["kc"], c["vc"], c["dtype"], c["mode"], c["ks"],
                                       c["vs"], c["pages"], L, sc)
    np.testing.assert_allclose(got, _sdpa(c["qf"], c["kf"], c["vf"], L, sc), rtol=0, atol=1e-12)


@pytest.mark.parametrize("fp8,pth", [(False, False), (True, True)])
def test_sparse_with_all_blocks_equals_dense(fp8, pth):
    L = 600
    c = _paged_kv_case(21, L, kv_fp8=fp8, per_token_scales=pth)
    nb = O.num_blocks(L)
    sc = 1 / math.sqrt(128)
    for v in (L, 513, 130, 1):
        sel = O.select_blocks(np.zeros(nb), O.num_blocks(v), nb + 3)
        a = O.sparse_attention_row(c["q"], c["kc"], c["vc"], c["dtype"], c["mode"], c["ks"], c["vs"],
                                   c["pages"], sel, v, sc)
        d = O.dense_causal_attention_row(c["q"], c["kc"], c["vc"], c["dtype"], c["mode"], c["ks"],
                                         c["vs"], c["pages"], v, sc)
        np.testing.assert_allclose(a, d, rtol=0, atol=1e-12)


def test_sparse_attention_matches_sdpa_on_selected_tokens():
    L = 900
    c = _paged_kv_case(22, L)
    sel = np.array([1, 4, 7])                 # block 7 is partial: tokens 896..899
    sc = 0.07
    got = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 0, 0, None, None, c["pages"], sel, L, sc)
    toks = [t for b in sel for t in range(128 * b, min(128 * b + 128, L))]
    ref = _sdpa(c["qf"], c["kf"][toks], c["vf"][toks], len(toks), sc)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_zero_query_is_mean_of_values():
    L = 300
    c = _paged_kv_case(23, L)
    q0 = bf16_bits(np.zeros((8, 128)))
    sel = np.array([0, 2])
    got = O.sparse_attention_row(q0, c["kc"], c["vc"], 0, 0, None, None, c["pages"], sel, L, 0.1)
    toks = list(range(0, 128)) + list(range(256, 300))
    mean = c["vf"][toks, 0, :].mean(axis=0)
    np.testing.assert_allclose(got, np.broadcast_to(mean, got.shape), rtol=0, atol=1e-12)


def test_attention_constant_values_and_single_key():
    L = 200
    c = _paged_kv_case(24, L)
    vc = np.full_like(c["vc"], bf16_bits([1.75])[0])
    got = O.sparse_attention_row(c["q"], c["kc"], vc, 0, 0, None, None, c["pages"], np.array([0, 1]), L, 0.1)
    assert np.all(np.abs(got - 1.75) < 1e-12)
    one = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 0, 0, None, None, c["pages"], np.array([0]), 1, 0.1)
    np.testing.assert_array_equal(one, np.broadcast_to(c["vf"][0, 0], one.shape))


def test_online_softmax_agrees_with_two_pass():
    L = 500
    c = _paged_kv_case(25, L)
    sc = 1 / math.sqrt(128)
    ref = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 0, 0, None, None, c["pages"],
                                 np.arange(4), L, sc)
    # streaming (online) softmax over 16-token chunks, float64
    m = np.full(8, -np.inf)
    l = np.zeros(8)
    acc = np.zeros((8, 128))
    for s in range(0, L, 16):
        kk = c["kf"][s:min(s + 16, L), 0]
        vv = c["vf"][s:min(s + 16, L), 0]
        z = sc * c["qf"] @ kk.T
        mn = np.maximum(m, z.max(axis=1))
        a = np.exp(m - mn)
        p = np.exp(z - mn[:, None])
        l = l * a + p.sum(axis=1)
        acc = acc * a[:, None] + p @ vv
        m = mn
    np.testing.assert_allclose(acc / l[:, None], ref, rtol=0, atol=1e-12)


def test_fp8_scalar_equals_constant_per_token_head():
    L = 260
    c = _paged_kv_case(26, L, kv_fp8=True)
    P8 = c["kc"].shape[0]
    sel = np.array([0, 2])
    a = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 1, 1, np.array([1.5], np.float32),
                               np.array([0.75], np.float32), c["pages"], sel, L, 0.09)
    b = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 1, 2, np.full((P8, 16, 1), 1.5, np.float32),
                               np.full((P8, 16, 1), 0.75, np.float32), c["pages"], sel, L, 0.09)
    np.testing.assert_array_equal(a, b)


def test_fp8_power_of_two_scale_equals_bf16_of_scaled_values():
    # e4m3 values times a power of two are exact in bf16, so the fp8 path with
    # scale 2^k must equal the bf16 path on the bf16 encoding of 2^k * value
    L = 300
    c = _paged_kv_case(27, L, kv_fp8=True)
    kf = torch.from_numpy(c["kc"].copy()).view(torch.float8_e4m3fn).float() * 4.0
    vf = torch.from_numpy(c["vc"].copy()).view(torch.float8_e4m3fn).float() * 0.5
    kb = kf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vb = vf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    sel = np.array([0, 1, 2])
    a = O.sparse_attention_row(c["q"], c["kc"], c["vc"], 1, 1, np.array([4.0], np.float32),
                               np.array([0.5], np.float32), c["pages"], sel, L, 0.05)
    b = O.sparse_attention_row(c["q"], kb, vb, 0, 0, None, None, c["pages"], sel, L, 0.05)
    np.testing.assert_array_equal(a, b)


def test_table_walk_equals_logical_walk():
    b = syn.make_batch("t", 30, seq_lens=[1000, 260], query_lens=[2, 1], topk=3, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    res = O.decode_step(b)
    via_table = O.attention_from_table(b, res["table"], res["ctx"], res["rows"])
    np.testing.assert_allclose(via_table, res["out"], rtol=0, atol=1e-13)


def test_decode_step_chain_on_tiny_workload():
    b = syn.config("tiny")
    res = O.decode_step(b)
    assert res["ctx"][0] == 4 * 128
    sel = res["sel"][0]
    assert len(sel) == 4 and (np.diff(sel) > 0).all()
    # the kept blocks beat every other block
    s = res["scores_fp32"][0]
    others = [x for x in range(16) if x not in sel]
    assert s[sel].min() >= s[others].max()
    assert res["table"][0].tolist() == [8 * int(blk) + i for blk in sel for i in range(8)]


# ---------------------------------------------------------------------------
# natural-log LSE and per-head sinks
# ---------------------------------------------------------------------------
def _lse_case(seed, T, H=8, scale=0.09):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, 128))
    k = rng.standard_normal((T, 128)) * 1.5
    v = rng.standard_normal((T, 128))
    return q, k, v, scale


def test_lse_matches_torch_logsumexp_and_output_matches_sdpa():
    q, k, v, sc = _lse_case(40, 77)
    out, lse = O.softmax_attention_lse(q, k, v, sc)
    z = sc * torch.from_numpy(q) @ torch.from_numpy(k).T
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k).expand(q.shape[0], -1, -1)[None],
        torch.from_numpy(v).expand(q.shape[0], -1, -1)[None], scale=sc)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_lse_closed_forms():
    # all-zero keys: every logit 0, lse = ln T, output = mean of the values
    q, _, v, sc = _lse_case(41, 37)
    out, lse = O.softmax_attention_lse(q, np.zeros((37, 128)), v, sc)
    np.testing.assert_allclose(lse, np.full(8, math.log(37)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), rtol=0, atol=1e-13)
    # one key: lse is its logit; two keys: ln(e^a + e^b) = max + log1p(e^-|a-b|)
    q, k, v, sc = _lse_case(42, 2)
    _, l1 = O.softmax_attention_lse(q, k[:1], v[:1], sc)
    a = np.array([sc * math.fsum(q[h] * k[0]) for h in range(8)])
    np.testing.assert_allclose(l1, a, rtol=0, atol=1e-12)
    _, l2 = O.softmax_attention_lse(q, k, v, sc)
    b = np.array([sc * math.fsum(q[h] * k[1]) for h in range(8)])
    np.testing.assert_allclose(l2, np.maximum(a, b) + np.log1p(np.exp(-np.abs(a - b))), rtol=0, atol=1e-12)


def test_lse_merges_splits():
    """Attention over a union of key sets from its parts: lse = logaddexp of
    the parts' lse, output = sum of part outputs weighted by exp(lse_i - lse)."""
    q, k, v, sc = _lse_case(43, 300)
    cuts = [0, 16, 128, 129, 300]
    parts = [O.softmax_attention_lse(q, k[a:b], v[a:b], sc) for a, b in zip(cuts, cuts[1:])]
    out, lse = O.softmax_attention_lse(q, k, v, sc)
    lse_m = parts[0][1]
    for _, l in parts[1:]:
        lse_m = np.logaddexp(lse_m, l)
    np.testing.assert_allclose(lse, lse_m, rtol=0, atol=1e-12)
    out_m = sum(o * np.exp(l - lse)[:, None] for o, l in parts)
    np.testing.assert_allclose(out, out_m, rtol=0, atol=1e-12)


def test_sink_is_an_extra_logit_with_a_zero_value():
    """torch softmax over the logits with the sink appended as one more column,
    applied to the values with a zero row appended."""
    q, k, v, sc = _lse_case(44, 50)
    sinks = np.random.default_rng(45).uniform(-3.0, 6.0, 8).astype(np.float32)
    out, lse = O.softmax_attention_lse(q, k, v, sc, sinks)
    z = sc * torch.from_numpy(q) @ torch.from_numpy(k).T
    z = torch.cat([z, torch.from_numpy(sinks.astype(np.float64))[:, None]], dim=1)
    vv = torch.cat([torch.from_numpy(v), torch.zeros(1, 128, dtype=torch.float64)], dim=0)
    np.testing.assert_allclose(out, (torch.softmax(z, dim=1) @ vv).numpy(), rtol=0, atol=1e-12)
    # the lse is that of the keys alone
    np.testing.assert_array_equal(lse, O.softmax_attention_lse(q, k, v, sc)[1])


def test_sink_special_values():
    q, k, v, sc = _lse_case(46, 90)
    out0, lse0 = O.softmax_attention_lse(q, k, v, sc)
    # -inf: no sink at all
    out, _ = O.softmax_attention_lse(q, k, v, sc, np.full(8, -np.inf))
    np.testing.assert_array_equal(out, out0)
    # a sink equal to the lse takes half of the mass
    out, _ = O.softmax_attention_lse(q, k, v, sc, lse0)
    np.testing.assert_allclose(out, out0 / 2, rtol=0, atol=1e-13)
    # no keys: zeros and -inf, with or without sinks, never NaN
    for sinks in (None, np.zeros(8), np.full(8, -np.inf)):
        out, lse = O.softmax_attention_lse(q, k[:0], v[:0], sc, sinks)
        assert np.all(out == 0) and np.all(lse == -np.inf)


def test_table_lse_equals_logical_walk():
    b = syn.make_batch("t", 31, seq_lens=[1000, 260, 40], query_lens=[2, 1, 1], topk=3, num_q_heads=16,
                       kv_dtype=syn.KV_FP8, scale_mode=syn.SCALE_PER_TOKEN_HEAD)
    res = O.decode_step(b)
    ctx = res["ctx"].copy()
    ctx[1] = 0                                   # a row with nothing to attend
    sinks = np.linspace(-2.0, 3.0, 16).astype(np.float32)
    out, lse = O.attention_lse_from_table(b, res["table"], ctx, res["rows"], sinks)
    plain = O.attention_from_table(b, res["table"], ctx, res["rows"])
    for i, n in enumerate(res["rows"]):
        c = int(ctx[n])
        if c == 0:
            assert np.all(out[i] == 0) and np.all(lse[i] == -np.inf)
            continue
        # logits of the logical tokens the selection covers (walked through the page-128 table)
        r = int(res["meta"]["row_req"][n])
        v_n = O.visible_keys(res["meta"]["row_pos"][n])
        toks = [t for blk in res["sel"][n] if blk >= 0 for t in range(128 * blk, min(128 * blk + 128, v_n))]
        assert len(toks) == c
        kh = O.dequant_tokens(b.k_cache, b.k_scale, b.scale_mode, b.kv_dtype, b.block_table[r], toks, 0, "k")
        qf = O.bf16_to_f64(b.q[n])
        z = b.sm_scale * torch.from_numpy(qf) @ torch.from_numpy(kh).T
        np.testing.assert_allclose(lse[i], torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)
        factor = 1.0 / (1.0 + np.exp(sinks.astype(np.float64) - lse[i]))
        np.testing.assert_allclose(out[i], plain[i] * factor[:, None], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# cache insert (new tokens into the paged caches, FP8 quantisation)
# ---------------------------------------------------------------------------
def _insert_case(seed, T, num_pages, kv_fp8, scale_mode, with_index=True):
    rng = np.random.default_rng(seed)
    k_new = bf16_bits(rng.standard_normal((T, 1, 128)) * rng.uniform(0.1, 4.0, (T, 1, 1)))
    v_new = bf16_bits(rng.standard_normal((T, 1, 128)) * rng.uniform(0.1, 4.0, (T, 1, 1)))
    ik_new = bf16_bits(rng.standard_normal((T, 128)))
    slots = rng.choice(num_pages * 128, size=T, replace=False).astype(np.int32)
    slots[rng.uniform(size=T) < 0.15] = -1
    dt = np.uint8 if kv_fp8 else np.uint16
    kc = rng.integers(0, 256 if kv_fp8 else 65536, (num_pages * 8, 1, 4, 4, 16, 8)).astype(dt)
    vc = rng.integers(0, 256 if kv_fp8 else 65536, (num_pages * 8, 1, 128, 16)).astype(dt)
    ik = rng.integers(0, 65536, (num_pages, 8, 4, 4, 16, 8)).astype(np.uint16)
    if scale_mode == 2:
        ks = rng.uniform(0.5, 2.0, (num_pages * 8, 16, 1)).astype(np.float32)
        vs = rng.uniform(0.5, 2.0, (num_pages * 8, 16, 1)).astype(np.float32)
    elif scale_mode == 1:
        ks, vs = np.array([0.75], np.float32), np.array([1.25], np.float32)
    else:
        ks = vs = None
    return dict(k_new=k_new, v_new=v_new, ik_new=ik_new if with_index else None, slots=slots,
                kc=kc, vc=vc, ik=ik, ks=ks, vs=vs, kv_dtype=1 if kv_fp8 else 0, scale_mode=scale_mode)


def _run_insert(c):
    return O.cache_insert(c["kc"], c["vc"], c["ks"], c["vs"], c["ik"], c["slots"], c["k_new"], c["v_new"],
                          c["ik_new"], c["kv_dtype"], c["scale_mode"])


def test_insert_bf16_is_an_exact_scatter_into_the_documented_layouts():
    """bf16 caches with no scale: the insert is a copy; checked against this
    file's own scatter (shuffle_into / dim-major V / index tiles)."""
    c = _insert_case(31, 40, 6, kv_fp8=False, scale_mode=0)
    kc, vc, _, _, ik = _run_insert(c)
    ek, ev, eik = c["kc"].copy(), c["vc"].copy(), c["ik"].copy()
    for t, slot in enumerate(c["slots"]):
        if slot < 0:
            continue
        page, off = divmod(int(slot), 128)
        sub, j = page * 8 + off // 16, off % 16
        shuffle_into(ek[sub, 0], j, c["k_new"][t, 0])
        ev[sub, 0, :, j] = c["v_new"][t, 0]
        shuffle_into(eik[page, off // 16], j, c["ik_new"][t])
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev) and np.array_equal(ik, eik)


def test_insert_leaves_skipped_slots_and_the_index_cache_alone():
    c = _insert_case(32, 30, 4, kv_fp8=True, scale_mode=2, with_index=False)
    c["slots"][:] = -1
    kc, vc, ks, vs, ik = _run_insert(c)
    assert np.array_equal(kc, c["kc"]) and np.array_equal(vc, c["vc"])
    assert np.array_equal(ks, c["ks"]) and np.array_equal(ik, c["ik"])
    c = _insert_case(33, 30, 4, kv_fp8=True, scale_mode=2, with_index=False)
    _, _, _, _, ik = _run_insert(c)
    assert np.array_equal(ik, c["ik"]), "no index rows given: the index cache is untouched"


def test_insert_fp8_per_token_head_scale_is_amax_over_448_and_roundtrips():
    """The largest |x| of each token-head lands exactly on code +-448 (0x7E /
    0xFE); every value comes back within half an e4m3 step (relative 2^-4,
    absolute s*2^-10 in the subnormal range)."""
    c = _insert_case(34, 48, 6, kv_fp8=True, scale_mode=2)
    kc, vc, ks, vs, _ = _run_insert(c)
    bt = np.arange(6)
    for t, slot in enumerate(c["slots"]):
        if slot < 0:
            continue
        for plane, cache, sc, new in (("k", kc, ks, c["k_new"]), ("v", vc, vs, c["v_new"])):
            x = O.bf16_to_f64(new[t, 0])
            s = O.token_scale(sc, 2, bt, int(slot), 0)
            assert s == float(np.float32(np.float32(np.abs(x).max()) / np.float32(448.0)))
            stored = O.kv_token(cache, bt, int(slot), 0, 1, plane)
            assert np.abs(stored).max() == 448.0
            assert stored[np.argmax(np.abs(x))] == np.sign(x[np.argmax(np.abs(x))]) * 448.0
            err = np.abs(s * stored - x)
            assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6))


def test_insert_fp8_exact_on_representable_values_and_zero_rows():
    """x = s * (e4m3 value) with the row's max at 448: codes are exact, the
    dequantised row equals x; an all-zero row stores zeros with scale 1."""
    rng = np.random.default_rng(35)
    codes = rng.integers(0, 0x7F, 128).astype(np.uint8)          # finite, positive
    codes[5] = 0x7E                                                 # 448
    codes[rng.uniform(size=128) < 0.5] |= 0x80                      # signs
    vals = O.e4m3fn_to_f64(codes)
    s = 0.25                                                        # power of two: x exact in bf16
    x_bits = bf16_bits(vals * s)
    stored, scale = O.quantize_row(x_bits, 1, 2, None)
    assert scale == s and np.array_equal(O.e4m3fn_to_f64(stored), vals)
    stored, scale = O.quantize_row(np.zeros(128, np.uint16), 1, 2, None)
    assert scale == 1.0 and not stored.any()


def test_insert_scalar_scale_divides_and_clamps():
    x = np.array([1.0, -3.0, 0.5, 1000.0, -1000.0] + [0.0] * 123)
    stored, s = O.quantize_row(bf16_bits(x), 1, 1, 0.5)
    back = O.e4m3fn_to_f64(stored)
    assert s == 0.5 and back[:5].tolist() == [2.0, -6.0, 1.0, 448.0, -448.0]
    stored, s = O.quantize_row(bf16_bits(x), 0, 1, 0.5)            # bf16 storage: x / s
    assert O.bf16_to_f64(stored)[:5].tolist() == [2.0, -6.0, 1.0, 2000.0, -2000.0]


# Values exactly halfway between two e4m3fn codes, with the code that round to
# nearest, ties to even gives, written out by hand from the OCP layout
# S.EEEE.MMM (bias 7; E = 0: M/8 * 2^-6). A quantiser that rounds ties away
# from zero, up, or by truncation fails at least one of them.
E4M3_TIES = [
    (1.0625, 0x38),        # 1.0 (M=0) | 1.125 (M=1): even M=0
    (1.1875, 0x3A),        # 1.125 (M=1) | 1.25 (M=2): even M=2 (rounds up)
    (-1.0625, 0xB8),
    (-1.1875, 0xBA),
    (1.9375, 0x40),        # 1.875 (0x3F) | 2.0 (E=8, M=0): up into the next binade
    (2.0 ** -10, 0x00),    # 0 | 2^-9, the smallest subnormal: even is zero
    (3 * 2.0 ** -10, 0x02),   # 2^-9 (M=1) | 2^-8 (M=2)
    (5 * 2.0 ** -10, 0x02),   # 2^-8 (M=2) | 3*2^-9 (M=3)
    (15 * 2.0 ** -10, 0x08),  # 7*2^-9, the largest subnormal | 2^-6 (E=1, M=0)
    (400.0, 0x7C),         # 384 (M=4) | 416 (M=5)
    (432.0, 0x7E),         # 416 (M=5) | 448 (M=6), the largest finite value
]


def test_quantize_e4m3_ties_round_to_even():
    """Insert quantisation to e4m3fn rounds to nearest, ties to even: with a
    scalar scale of 1 the stored code of each halfway value is the one
    written out by hand; per-token-head scaling of a row whose largest
    magnitude is exactly 448 has s = 1 and gives the same codes."""
    x = np.array([v for v, _ in E4M3_TIES])
    want = np.array([c for _, c in E4M3_TIES], np.uint8)
    assert np.array_equal(O.bf16_to_f64(bf16_bits(x)), x), "tie values are exact bf16 inputs"
    row = np.zeros(128)
    row[:len(x)] = x
    codes, s = O.quantize_row(bf16_bits(row), 1, 1, 1.0)
    assert s == 1.0 and codes[:len(x)].tolist() == want.tolist()
    row[100] = -448.0
    codes, s = O.quantize_row(bf16_bits(row), 1, 2, None)
    assert s == 1.0 and codes[:len(x)].tolist() == want.tolist() and codes[100] == 0xFE
    # just off each tie the nearest code wins, whichever side it is on
    for v, c in E4M3_TIES[:2]:
        up = O.quantize_row(bf16_bits(np.full(128, v * (1 + 2.0 ** -7))), 1, 1, 1.0)[0][0]
        dn = O.quantize_row(bf16_bits(np.full(128, v * (1 - 2.0 ** -7))), 1, 1, 1.0)[0][0]
        assert O.e4m3fn_to_f64(np.array([dn]))[0] <= O.e4m3fn_to_f64(np.array([c]))[0] <= \
            O.e4m3fn_to_f64(np.array([up]))[0]


# Scalar scales under which fl32(1.5 / s) lands exactly halfway between two
# bf16 values (found by solving s = fl32(1.5 / y) for the midpoint y and
# checking fl32(1.5 / s) == y), with the bf16 bits that ties to even give.
BF16_TIE_SCALES = [
    # (fp32 bits of s, x, fl32(x / s), bf16 bits of the even neighbour)
    (0x3FBF40BF, 1.5, 1.0 + 2.0 ** -8, 0x3F80),        # 1.0 | 1.0078125: rounds down
    (0x3FBF40BF, -1.5, -(1.0 + 2.0 ** -8), 0xBF80),
    (0x3FBF40BF, 3.0, 2.0 + 2.0 ** -7, 0x4000),        # 2.0 | 2.015625
    (0x3FBDC6AC, 1.5, 1.0 + 3 * 2.0 ** -8, 0x3F82),    # 1.0078125 | 1.015625: rounds up
    (0x3FBDC6AC, -1.5, -(1.0 + 3 * 2.0 ** -8), 0xBF82),
    (0x3FBDC6AC, 3.0, 2.0 + 3 * 2.0 ** -7, 0x4002),    # 2.015625 | 2.03125
]


def test_quantize_bf16_ties_round_to_even():
    """bf16 storage with a scalar scale keeps bf16 RNE(fl32(x) / s): at the
    exact midpoints below the even neighbour is stored, one case rounding
    down and one up, so ties away from zero and truncation both fail."""
    for sbits in sorted({c[0] for c in BF16_TIE_SCALES}):
        s = float(np.array([sbits], np.uint32).view(np.float32)[0])
        cases = [c for c in BF16_TIE_SCALES if c[0] == sbits]
        row = np.zeros(128)
        row[:len(cases)] = [c[1] for c in cases]
        for x, y in ((c[1], c[2]) for c in cases):   # each quotient really is the midpoint
            assert float(np.float32(np.float32(x) / np.float32(s))) == y
        stored, s_out = O.quantize_row(bf16_bits(row), 0, 1, s)
        assert s_out == float(np.float32(s))
        assert stored[:len(cases)].tolist() == [c[3] for c in cases]


def test_tie_pins_catch_a_round_half_away_quantiser(monkeypatch):
    """Plants rounding half away from zero into the oracle's two casts (on the
    CPU) and checks that both tie pins above then fail."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = O.e4m3fn_to_f64(finite)

    def e4m3_half_away(x32):
        x = np.asarray(x32, np.float64).reshape(-1)
        out = np.empty(x.size, np.uint8)
        for i, v in enumerate(x):
            d = np.abs(vals - v)
            best = np.flatnonzero(d == d.min())
            out[i] = finite[best[np.argmax(np.abs(vals[best]))]] if v != 0 else 0
        return out.reshape(np.shape(x32))

    def bf16_half_away(x32):
        u = np.ascontiguousarray(x32, np.float32).view(np.uint32)
        return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)

    monkeypatch.setattr(O, "_f32_to_e4m3fn_codes", e4m3_half_away)
    with pytest.raises(AssertionError):
        test_quantize_e4m3_ties_round_to_even()
    monkeypatch.setattr(O, "_f32_to_bf16_bits", bf16_half_away)
    with pytest.raises(AssertionError):
        test_quantize_bf16_ties_round_to_even()


def test_insert_then_decode_equals_decode_on_the_written_cache():
    """Writing a request's last token through the insert and then running the
    decode step gives the same output as a cache built with that token in
    place by this file's own scatter (bf16, no scale)."""
    b = syn.make_batch("ins", 36, [700, 300], [1, 1], topk=4, num_q_heads=8)
    last = [int(L) - 1 for L in b.seq_lens]
    slots = np.array([int(b.block_table[r, t // 128]) * 128 + t % 128 for r, t in enumerate(last)], np.int32)
    k_new = np.stack([O.tile_row(b.k_cache[int(s) // 128 * 8 + (int(s) % 128) // 16, 0], int(s) % 16)
                      for s in slots])[:, None, :]
    v_new = np.stack([b.v_cache[int(s) // 128 * 8 + (int(s) % 128) // 16, 0, :, int(s) % 16]
                      for s in slots])[:, None, :]
    ref = O.decode_step(b)["out"]
    # wipe the two tokens, then insert them back
    kc, vc = b.k_cache.copy(), b.v_cache.copy()
    for s in slots:
        sub, j = int(s) // 128 * 8 + (int(s) % 128) // 16, int(s) % 16
        kc[sub, 0, :, :, j, :] = 0
        vc[sub, 0, :, j] = 0
    kc, vc, _, _, _ = O.cache_insert(kc, vc, None, None, None, slots, k_new, v_new, None, 0, 0)
    b2 = syn.Batch(**{**b.__dict__, "k_cache": kc, "v_cache": vc})
    assert np.array_equal(O.decode_step(b2)["out"], ref)


# ---------------------------------------------------------------------------
# FP8 index cache (e4m3fn codes, one fp32 scale per token)
# ---------------------------------------------------------------------------
def test_fp8_index_with_power_of_two_scales_equals_the_bf16_path():
    """e4m3 values times 2^k are exact in bf16: an fp8 index cache whose
    per-token scales are random powers of two must score exactly like a bf16
    index cache holding bf16(scale * e4m3(code)), written by this file's own
    writer at the same logical positions."""
    rng = np.random.default_rng(50)
    L = [700, 300, 1]
    nb = [-(-x // 128) for x in L]
    P = sum(nb) + 2
    perm = rng.permutation(P)
    bt = np.zeros((3, max(nb)), np.int32)
    pos = 0
    for r in range(3):
        bt[r, :nb[r]] = perm[pos:pos + nb[r]]
        pos += nb[r]
    codes = fp8_codes(rng.standard_normal((P, 8, 4, 4, 16, 8)))
    scale = np.exp2(rng.integers(-3, 4, (P, 128))).astype(np.float32)
    # logical keys of every physical slot, then the bf16 cache through the test's writer
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    bf = np.zeros((P, 8, 4, 4, 16, 8), np.uint16)
    for p in range(P):
        for s_ in range(128):
            row = np.array([vals[p, s_ // 16, d // 32, (d % 32) // 8, s_ % 16, d % 8] for d in range(128)])
            shuffle_into(bf[p, s_ // 16], s_ % 16, bf16_bits(row * float(scale[p, s_])))
    iq = bf16_bits(rng.standard_normal((5, 128)))
    ql = np.array([2, 2, 1])
    a = O.block_scores(iq, codes, bt, np.array(L), ql, 8, index_scale=scale)
    b = O.block_scores(iq, bf, bt, np.array(L), ql, 8)
    np.testing.assert_array_equal(a, b)


def test_fp8_index_scale_of_one_token_moves_only_its_score():
    """One-hot query on dim d: each token's score is scale x e4m3(code[d]);
    doubling one token's scale doubles that token's score and leaves the
    block max of every other block alone."""
    rng = np.random.default_rng(51)
    P = 3
    codes = fp8_codes(rng.standard_normal((P, 8, 4, 4, 16, 8)))
    scale = rng.uniform(0.5, 2.0, (P, 128)).astype(np.float32)
    bt = np.array([[2, 0, 1]], np.int32)
    d = 77
    keys = O.index_keys_of_request(codes, bt[0], 300, scale)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    for t in (0, 130, 299):
        p, s_ = int(bt[0, t // 128]), t % 128
        want = float(scale[p, s_]) * vals[p, s_ // 16, d // 32, (d % 32) // 8, s_ % 16, d % 8]
        assert keys[t, d] == want
    scale2 = scale.copy()
    scale2[0, 5] *= 2                              # token 128 + 5 lives in page 0
    keys2 = O.index_keys_of_request(codes, bt[0], 300, scale2)
    changed = np.flatnonzero(np.any(keys2 != keys, axis=1))
    assert changed.tolist() == [133]
    np.testing.assert_array_equal(keys2[133], 2 * keys[133])


def test_index_insert_fp8_scale_rule_placement_and_skips():
    rng = np.random.default_rng(52)
    P, T = 4, 40
    x = rng.standard_normal((T, 128)) * rng.uniform(0.01, 30.0, (T, 1))
    x[7] = 0.0                                     # all-zero row: scale 1, zero codes
    new = bf16_bits(x)
    slots = rng.choice(P * 128, size=T, replace=False).astype(np.int32)
    slots[3], slots[9] = -1, P * 128 + 2           # skipped
    ik0 = rng.integers(0, 256, (P, 8, 4, 4, 16, 8)).astype(np.uint8)
    sc0 = rng.uniform(1, 2, (P, 128)).astype(np.float32)
    ik, sc = O.index_insert_fp8(ik0, sc0, slots, new)
    touched = np.zeros((P, 128), bool)
    for t, slot in enumerate(slots.tolist()):
        if slot < 0 or slot >= P * 128:
            continue
        p, off = slot // 128, slot % 128
        touched[p, off] = True
        xf = O.bf16_to_f64(new[t])
        amax = np.float32(np.abs(xf).max())
        s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        assert sc[p, off] == s
        # the stored row, read back through this file's own tile addressing
        stored = np.array([ik[p, off // 16, d // 32, (d % 32) // 8, off % 16, d % 8] for d in range(128)],
                          np.uint8)
        vals = torch.from_numpy(stored.copy()).view(torch.float8_e4m3fn).double().numpy()
        if amax == 0:
            assert np.all(vals == 0)
            continue
        assert np.abs(vals).max() == 448.0
        err = np.abs(float(s) * vals - xf)
        assert np.all(err <= np.maximum(np.abs(xf) * 2.0 ** -4, float(s) * 2.0 ** -10) * (1 + 1e-6))
    # untouched slots keep their codes and scales
    np.testing.assert_array_equal(sc[~touched], sc0[~touched])
    for p in range(P):
        for off in range(128):
            if not touched[p, off]:
                assert np.array_equal(ik[p, off // 16, :, :, off % 16, :], ik0[p, off // 16, :, :, off % 16, :])


def test_decode_step_on_an_fp8_index_cache_scores_with_the_scales():
    """The whole oracle step on an fp8 index batch: its scores equal the
    scores of the same batch with the index cache dequantised into fp64 keys
    by hand (scale x code value) and scored by matrix product."""
    b = syn.make_batch("f8i", 53, [1000, 260], [2, 1], topk=3, num_q_heads=16, index_dtype=syn.INDEX_FP8)
    res = O.decode_step(b)
    vals = torch.from_numpy(b.index_k.copy()).view(torch.float8_e4m3fn).double().numpy()
    for n, (r, pos) in enumerate([(0, 998), (0, 999), (1, 259)]):
        keys = []
        for t in range(pos + 1):
            p, s_ = int(b.block_table[r, t // 128]), t % 128
            keys.append(vals[p, s_ // 16].transpose(2, 0, 1, 3)[s_ % 16].reshape(-1) * float(b.index_scale[p, s_]))
        z = np.array(keys) @ O.bf16_to_f64(b.index_q[n])
        want = [z[128 * j:128 * (j + 1)].max() for j in range(-(-(pos + 1) // 128))]
        np.testing.assert_allclose(res["scores"][n, :len(want)], want, rtol=1e-13, atol=0)
