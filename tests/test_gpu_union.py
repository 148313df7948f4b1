"""GPU checks of csa_union_rows and the multi-layer selector (integer work:
bit-exact against the CPU oracle)."""
import numpy as np
import pytest

import csa_inputs
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import lightning_indexer_top_02_amd as L  # noqa: E402


def _say(msg):
    print(f"[csa-test] {msg}", flush=True)


@pytest.mark.parametrize("T,widths,cap", [(1000, (64, 200, 17), 300),      # union larger than some lists
                                          (1000, (64, 200, 17), 40),       # cap below the union size
                                          (1 << 20, (2048, 2048), 4096),   # the largest T the bitmap covers
                                          (33, (5,), 8)])                  # one list, tiny T
def test_union_matches_oracle(T, widths, cap):
    rng = np.random.default_rng(T + cap)
    rows = (3, 5)
    lists = [rng.integers(-2, T + 3, size=rows + (w,)).astype(np.int32) for w in widths]
    lists[0][0, 0, :3] = lists[-1][0, 0, :3]                               # shared entries
    _say(f"union T={T} widths={widths} cap={cap}")
    out, cnt = L.union_rows([torch.from_numpy(x).cuda() for x in lists], T, cap)
    torch.cuda.synchronize()
    ref, rcnt = oracle.oracle_union(lists, T, cap)
    assert (out.cpu().numpy() == ref).all()
    assert (cnt.cpu().numpy() == rcnt).all()


def _layer(seed, S_q=3, T=500):
    p = csa_inputs.make_integer(B=2, S_q=S_q, T=T, H=64, D=128, m=4, topk=64, q_pos0=4 * T - S_q, seed=seed,
                                qk_range=2, w_range=2)
    p["q"] = csa_inputs.f32_to_bf16_bits(p["q"])
    p["k"] = csa_inputs.f32_to_bf16_bits(p["k"])
    p["dtype"] = "bf16"
    return p


def _dev(p):
    q = torch.from_numpy(p["q"].view(np.int16)).view(torch.bfloat16).cuda()
    k = torch.from_numpy(p["k"].view(np.int16)).view(torch.bfloat16).cuda()
    return q, k, torch.from_numpy(p["w"]).cuda()


@pytest.mark.parametrize("mode", ["batched", "sequential", "overlap"])
def test_multilayer_union_and_refresh(mode):
    probs = [_layer(s) for s in (21, 22, 23)]
    layers = [_dev(p) for p in probs]
    cap, ucap = 96, 320
    sel = L.MultiLayerSelector(tau=4, prob_threshold=0.5, cap=cap, union_cap=ucap, overlap=mode == "overlap",
                               batched=mode == "batched")
    _say(f"multi-layer union, mode={mode}")
    u, c = sel.select(0, layers, m=4, q_pos0=probs[0]["q_pos0"])
    torch.cuda.synchronize()
    ref, rcnt = oracle.oracle_multilayer(probs, 0.5, cap, ucap)
    assert (u.cpu().numpy() == ref).all()
    assert (c.cpu().numpy() == rcnt).all()
    for step in (1, 2, 3):                                               # reused between refreshes
        assert sel.select(step, layers, m=4, q_pos0=probs[0]["q_pos0"])[0] is u
    assert sel.refreshes == 1
    u2, _ = sel.select(4, layers, m=4, q_pos0=probs[0]["q_pos0"])
    torch.cuda.synchronize()
    assert sel.refreshes == 2 and (u2.cpu().numpy() == ref).all()


@pytest.mark.parametrize("case", ["integer", "decode_workload"])
def test_batched_threshold_matches_per_layer(case):
    """One batched launch over the layers gives, layer by layer, exactly the
    indices and counts of separate csa_index_threshold_select calls."""
    if case == "integer":                       # ragged kv_len, non-causal, cap below some counts
        probs = [_layer(s, S_q=5, T=900) for s in (31, 32, 33, 34)]
        layers = [_dev(p) for p in probs]
        kv = torch.tensor([900, 517], dtype=torch.int32).cuda()
        kw = dict(m=4, q_pos0=0, kv_len=kv, causal=False)
        cap, tau = 40, 0.5
    else:                                       # three layers at B=32, T=32768, cap 2048
        pd = [csa_inputs.make_decode(seed=s) for s in (1007, 1008, 1009)]
        layers = [(torch.from_numpy(p["q"].view(np.int16)).view(torch.bfloat16).cuda(),
                   torch.from_numpy(p["k"].view(np.int16)).view(torch.bfloat16).cuda(),
                   torch.from_numpy(p["w"]).cuda()) for p in pd]
        kw = dict(m=pd[0]["m"], q_pos0=pd[0]["q_pos0"])
        cap, tau = 2048, 0.5
    _say(f"batched threshold selection, case {case}, {len(layers)} layers")
    got = L.index_threshold_select_layers(layers, cap, prob_threshold=tau, **kw)
    for (q, k, w), (gi, gc) in zip(layers, got):
        ri, rc = L.index_threshold_select(q, k, w, cap, prob_threshold=tau, **kw)
        torch.cuda.synchronize()
        assert torch.equal(gc, rc)
        a, b = gi.cpu().numpy(), ri.cpu().numpy()
        assert (np.sort(a, axis=-1) == np.sort(b, axis=-1)).all()


def test_batched_threshold_sorted_with_scores_eight_layers():
    """The C entry point with all 8 layers, CSA_SORTED and score outputs: each
    layer's indices, scores and order equal a separate sorted call's."""
    import ctypes
    from lightning_indexer_top_02_amd import _binding as Bd
    probs = [_layer(s, S_q=4, T=700) for s in range(51, 59)]
    layers = [_dev(p) for p in probs]
    cap, n = 48, len(layers)
    B, S_q = 2, 4
    cps = [L.make_problem(q, k, w, m=4, q_pos0=probs[0]["q_pos0"]) for q, k, w in layers]
    idx = [torch.empty((B, S_q, cap), dtype=torch.int32, device="cuda") for _ in range(n)]
    cnt = [torch.empty((B, S_q), dtype=torch.int32, device="cuda") for _ in range(n)]
    sco = [torch.empty((B, S_q, cap), dtype=torch.float32, device="cuda") for _ in range(n)]
    nws = n * L.workspace_size(L.OP_THRESHOLD, cps[0], cap, 1, L.CSA_SORTED)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    PP = (ctypes.POINTER(Bd.CsaProblem) * n)(*[ctypes.pointer(p) for p in cps])
    V = ctypes.c_void_p * n
    _say("batched threshold selection: 8 layers, sorted, with scores")
    st = L.load_library().csa_index_threshold_select_layers(
        PP, n, 0.5, 0.0, cap, L.CSA_SORTED, V(*[t.data_ptr() for t in idx]), V(*[t.data_ptr() for t in cnt]),
        V(*[t.data_ptr() for t in sco]), ctypes.c_void_p(ws.data_ptr()), nws,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.load_library().csa_last_error()
    for li, (q, k, w) in enumerate(layers):
        ri, rc, rs = L.index_threshold_select(q, k, w, cap, prob_threshold=0.5, m=4, q_pos0=probs[0]["q_pos0"],
                                              sorted=True, return_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(cnt[li], rc) and torch.equal(idx[li], ri) and torch.equal(sco[li], rs), f"layer {li}"


def test_batched_threshold_decode_workload_vs_oracle():
    """Three layers at the decode workload (B=32, T=32768, tau = 0.5, cap
    2048) in one batched launch, checked against the fp64 oracle on sampled
    rows of every layer: the survivor count within the bf16 tolerance band
    around the threshold, and the kept keys the survivors' best 2048 up to
    the band around the 2048-th (or every survivor when fewer survive)."""
    from gpu_common import REL, FLOOR_DIV
    pd = [csa_inputs.make_decode(seed=s) for s in (1007, 1008, 1009)]
    layers = [(torch.from_numpy(p["q"].view(np.int16)).view(torch.bfloat16).cuda(),
               torch.from_numpy(p["k"].view(np.int16)).view(torch.bfloat16).cuda(),
               torch.from_numpy(p["w"]).cuda()) for p in pd]
    cap, tau = 2048, 0.5
    _say("batched threshold selection at the decode workload: 3 layers vs the oracle on sampled rows")
    got = L.index_threshold_select_layers(layers, cap, prob_threshold=tau, m=pd[0]["m"], q_pos0=pd[0]["q_pos0"])
    torch.cuda.synchronize()
    theta = oracle.logit_threshold(tau, 0.0)
    for li, (p, (gi, gc)) in enumerate(zip(pd, got)):
        idx, cnt = gi.cpu().numpy(), gc.cpu().numpy()
        scorer = oracle.RowScorer(p)
        for b in (0, 17, 31):
            I = scorer(b, 0)
            floor = float(np.sqrt(np.mean(I * I))) / FLOOR_DIV
            band = REL * max(abs(theta), floor)
            true_cnt = int((I > theta).sum())
            near = int((np.abs(I - theta) <= band).sum())
            assert abs(int(cnt[b, 0]) - true_cnt) <= near, f"layer {li} row {b}: count {cnt[b, 0]} vs {true_cnt}"
            n = min(cap, int(cnt[b, 0]))
            sel = idx[b, 0, :n]
            assert (idx[b, 0, n:] == -1).all() and len(set(sel.tolist())) == n
            surv = oracle.order_desc(I, np.nonzero(I > theta)[0])
            if true_cnt > cap:
                ref = surv[:cap]
                vc = I[ref].min()
                bc = REL * max(abs(vc), floor)
                for s_ in set(sel.tolist()) ^ set(ref.tolist()):
                    assert abs(I[s_] - vc) <= bc, f"layer {li} row {b}: index {s_} outside the band"
            else:
                for s_ in set(sel.tolist()) ^ set(surv.tolist()):
                    assert abs(I[s_] - theta) <= band, f"layer {li} row {b}: survivor {s_} missing or extra"
            assert set(p["planted"][b].tolist()) <= set(sel.tolist()), f"layer {li} row {b}: a planted key is missing"
