"""GPU parity of the varlen chunked prefill against the fp64 oracle.

All calls go through the C ABI (ctypes binding) on seeded inputs from
linear_attention_rule_amd.workloads.  Small cases are compared element by
element in full.  At the full workload sizes the GPU runs the real launch (all
heads, all sequences) and the oracle recomputes every (sequence, head) pair over
its whole length (about 30 s of one host core for the three workloads); a sampled
variant recomputes a few pairs only, as a fast first check.
"""

import numpy as np
import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import chunk_prefill, recurrent_verify
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _call(d, **kw):
    return chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
                         d["lower_bound"], d["cu_seqlens"], initial_state=d["initial_state"],
                         initial_state_idx=d["initial_state_idx"], scale=d["scale"], **kw)


def _oracle(data, heads=None, seqs=None):
    """Oracle on a subset of heads / sequences.  Returns (out [T_sel, h_sel, V], final [n_sel, h_sel, K, V])."""
    f = W.to_f64
    cu = data["cu_seqlens"].numpy().astype(np.int64)
    N = len(cu) - 1
    H = data["q"].shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    seqs = list(range(N)) if seqs is None else list(seqs)
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]) if seqs else np.zeros(0, int)
    sub_cu = np.concatenate([[0], np.cumsum([cu[n + 1] - cu[n] for n in seqs])]).astype(np.int64)
    pick = lambda t: f(t)[rows][:, heads]
    init = data["initial_state"]
    idx = data["initial_state_idx"]
    sub_init = None
    sub_idx = None
    if init is not None:
        if idx is None:
            sub_init = init.numpy()[seqs][:, heads]
        else:
            sub_init = init.numpy()[:, heads]
            sub_idx = idx.numpy()[seqs]       # out-of-pool indices start from zero in the oracle
    o, fs = O.chunk_prefill(pick(data["q"]), pick(data["k"]), pick(data["v"]), pick(data["g"]),
                            f(data["beta_logits"])[rows][:, heads], f(data["A_log"])[heads],
                            f(data["dt_bias"])[heads], data["lower_bound"], sub_cu, sub_init,
                            sub_idx, scale=data["scale"])
    return o, fs, rows


def _compare(data, out, final, heads=None, seqs=None):
    o_ref, f_ref, rows = _oracle(data, heads, seqs)
    H = data["q"].shape[1]
    N = data["cu_seqlens"].numel() - 1
    heads = list(range(H)) if heads is None else list(heads)
    seqs = list(range(N)) if seqs is None else list(seqs)
    og = out[torch.as_tensor(rows, device=out.device)][:, heads] if len(rows) else out[:0]
    e = TOL.assert_output_ok(og, o_ref) if len(rows) else {}
    r = None
    if final is not None:
        fg = final[seqs][:, heads]
        r = TOL.assert_state_ok(fg, f_ref)
    print("output errors", e, "state rel", r, flush=True)
    return e, r


def test_prefill_tiny_1x256_h2():
    case = W.TINY
    print(f"case {case.name} seed {case.seed}", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


@pytest.mark.parametrize("lens,H,init", [
    ([1, 63, 64, 65, 200, 0, 130], 3, "per_seq"),
    ([64], 1, None),
    ([5], 2, "per_seq"),
    ([127, 1, 129], 2, None),
])
def test_prefill_ragged_varlen(lens, H, init):
    case = W.PrefillCase(f"ragged_{len(lens)}_h{H}", lens, H, init=init, seed=3000 + sum(lens) + H)
    print(f"case {case.name} lens {lens}", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


def test_prefill_many_short_sequences():
    """120 sequences of 0..129 tokens: a deep chunk-map search, many chunk slots that
    belong to no chunk, and the scan configuration for more pairs than CUs."""
    lens = np.random.default_rng(3200).integers(0, 130, size=120).tolist()
    case = W.PrefillCase("many_short_120_h2", lens, 2, init="per_seq", seed=3200)
    print(f"case {case.name} tokens {sum(lens)}", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


def test_prefill_pool_gather_and_bad_index():
    case = W.PrefillCase("pool_gather", [70, 100, 33], 2, init="pool", pool_slots=6, seed=3101)
    data = W.make_prefill(case)
    data["initial_state_idx"] = torch.tensor([4, -1, 6], dtype=torch.int32)   # -1 and 6 start from zero
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


@pytest.mark.parametrize("lb", [0.0, -1.0, -5.0])
def test_prefill_lower_bound_values(lb):
    case = W.PrefillCase(f"lb_{lb}", [150, 90], 2, init="per_seq", seed=3102, lower_bound=lb)
    data = W.make_prefill(case)
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


def _saturate(data):
    """Degenerate values in place: all-zero q or k rows (the l2 norm's epsilon case), gate
    logits far past both ends of the sigmoid (decay pinned at the lower bound, or none at
    all) over runs longer than a chunk, and beta logits that give beta = 1 or beta ~ 0."""
    T = data["q"].shape[0]
    t = torch.arange(T)
    data["q"][t % 11 == 3] = 0
    data["k"][t % 13 == 5] = 0
    data["g"][(t >= 20) & (t < 150), 0] = 64.0      # head 0: decay at the bound for 130 tokens
    data["g"][(t >= 160) & (t < 230), 1] = -64.0    # head 1: no decay for 70 tokens
    data["g"][(t >= 600) & (t < 1400), 0] = 64.0    # long runs span whole scan segments
    data["g"][(t >= 1500) & (t < 2500), 1] = -64.0
    data["beta_logits"][t % 7 == 0] = 32.0
    data["beta_logits"][t % 7 == 1] = -32.0


@pytest.mark.parametrize("lens", [[230, 1, 97], [64 * 40 + 17]])   # the second: segmented scan
def test_prefill_saturated_and_degenerate_inputs(lens):
    case = W.PrefillCase("saturated", lens, 2, init="per_seq", seed=3106)
    print(f"case {case.name} lens {case.seq_lens}", flush=True)
    data = W.make_prefill(case)
    _saturate(data)
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(final).all()
    _compare(data, out, final)


def _random_prefill_case(seed):
    """A seeded random call shape: sequence lengths mixing the chunk boundaries (0, 1, 63,
    64, 65, 127-129) with arbitrary lengths and, at times, one long enough for the
    segment-parallel scan; 1-4 heads; zero, per-sequence or pooled start states; one of
    the supported lower bounds."""
    rng = np.random.default_rng(seed)
    pick = [0, 1, 63, 64, 65, 127, 128, 129]
    lens = []
    for _ in range(int(rng.integers(1, 7))):
        r = rng.random()
        lens.append(int(rng.choice(pick)) if r < 0.4 else
                    int(rng.integers(2, 300)) if r < 0.9 else int(rng.integers(1000, 2600)))
    H = int(rng.integers(1, 5))
    init = [None, "per_seq", "pool"][int(rng.integers(0, 3))]
    lb = float(rng.choice([-5.0, -2.5, -1.0, 0.0]))
    return W.PrefillCase(f"rand_{seed}", lens, H, init=init, pool_slots=len(lens) + 2,
                         seed=seed, lower_bound=lb)


@pytest.mark.parametrize("seed", range(3300, 3316))
def test_prefill_random_shapes(seed):
    case = _random_prefill_case(seed)
    print(f"case {case.name} lens {case.seq_lens} H {case.heads} init {case.init} "
          f"lb {case.lower_bound}", flush=True)
    data = W.make_prefill(case)
    if case.init == "pool":
        # some sequences start from zero: a negative index or one past the pool
        idx = data["initial_state_idx"]
        idx[::3] = -1
        idx[1::4] = case.pool_slots
    d = _dev(data)
    out, final = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, final)


def test_prefill_writes_only_its_rows_and_handles_empty():
    case = W.PrefillCase("canary", [0, 77, 0], 2, init="per_seq", seed=3103)
    data = W.make_prefill(case)
    d = _dev(data)
    T = 77
    big = torch.full((T + 8, 2, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    out_view = big[4:4 + T]
    fin = torch.full((3, 2, 128, 128), 9.0, dtype=torch.float32, device="cuda")
    _call(d, out=out_view, final_state=fin)
    torch.cuda.synchronize()
    assert torch.all(big[:4] == 5.0) and torch.all(big[4 + T:] == 5.0)
    _compare(data, out_view, fin)
    # empty sequences copy their start state
    assert torch.equal(fin[0], d["initial_state"][0]) and torch.equal(fin[2], d["initial_state"][2])


def test_prefill_no_tokens_only_state_copy():
    case = W.PrefillCase("empty_all", [0, 0], 2, init="per_seq", seed=3104)
    data = W.make_prefill(case)
    d = _dev(data)
    out, fin = _call(d)
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert torch.equal(fin, d["initial_state"])


def test_prefill_strided_inputs_bitwise_equal_dense():
    case = W.PrefillCase("strided", [100, 160], 4, init="per_seq", seed=3105)
    data = W.make_prefill(case)
    d = _dev(data)
    T, H = 260, 4
    fused = torch.empty((T, 4 * H * 128 + 64), dtype=torch.bfloat16, device="cuda")
    views = {}
    for i, name in enumerate(("q", "k", "v", "g")):
        fused[:, i * H * 128:(i + 1) * H * 128] = d[name].reshape(T, H * 128)
        views[name] = fused[:, i * H * 128:(i + 1) * H * 128].view(T, H, 128)
    o1, f1 = _call(d)
    o2, f2 = _call(dict(d, **views))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_prefill_deterministic():
    data = W.make_prefill(W.PrefillCase("det", [300, 200, 500], 8, init="per_seq", seed=3106))
    d = _dev(data)
    o1, f1 = _call(d)
    o2, f2 = _call(d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_prefill_resume_matches_single_call():
    """prefill(x[:a]) then prefill(x[a:], start = final) matches prefill(x) (chunk edges differ)."""
    data = W.make_prefill(W.PrefillCase("resume", [333], 2, init="per_seq", seed=3107))
    d = _dev(data)
    o_full, f_full = _call(d)
    a = 150
    cuA = torch.tensor([0, a], dtype=torch.int32, device="cuda")
    cuB = torch.tensor([0, 333 - a], dtype=torch.int32, device="cuda")
    sl = lambda x, s: x[s]
    dA = dict(d, q=d["q"][:a], k=d["k"][:a], v=d["v"][:a], g=d["g"][:a],
              beta_logits=d["beta_logits"][:a], cu_seqlens=cuA)
    oA, fA = _call(dA)
    dB = dict(d, q=d["q"][a:], k=d["k"][a:], v=d["v"][a:], g=d["g"][a:],
              beta_logits=d["beta_logits"][a:], cu_seqlens=cuB, initial_state=fA)
    oB, fB = _call(dB)
    torch.cuda.synchronize()
    o_ref, f_ref, _ = _oracle(data)
    TOL.assert_output_ok(torch.cat([oA, oB]), o_ref)
    TOL.assert_state_ok(fB, f_ref)
    TOL.assert_output_ok(o_full, o_ref)


def test_prefill_final_state_in_place_over_initial():
    data = W.make_prefill(W.PrefillCase("inplace", [90, 190], 2, init="per_seq", seed=3108))
    d = _dev(data)
    o_ref_gpu, f_ref_gpu = _call(d)
    pool = d["initial_state"].clone()
    o2, f2 = _call(dict(d, initial_state=pool), final_state=pool)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref_gpu) and torch.equal(pool, f_ref_gpu)


def test_prefill_matches_verify_on_block_sequences():
    """Verify rows of T tokens and prefill of sequences of T tokens from the same pool states
    both match the oracle (each output is rounded to bf16 once, so they are compared
    to the fp64 reference rather than to each other)."""
    vcase = W.VerifyCase("pv", 6, 8, 4, pool_slots=10, seed=3109)
    vdata = W.make_verify(vcase)
    vd = _dev(vdata)
    ov, iv = recurrent_verify(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                              vd["dt_bias"], vd["lower_bound"], vd["state_pool"], vd["state_idx"], 8)
    cu = torch.arange(0, 49, 8, dtype=torch.int32, device="cuda")
    op, fp = chunk_prefill(vd["q"], vd["k"], vd["v"], vd["g"], vd["beta_logits"], vd["A_log"],
                           vd["dt_bias"], vd["lower_bound"], cu, initial_state=vd["state_pool"],
                           initial_state_idx=vd["state_idx"])
    torch.cuda.synchronize()
    f = W.to_f64
    o_ref, i_ref = O.recurrent_verify(f(vdata["q"]), f(vdata["k"]), f(vdata["v"]), f(vdata["g"]),
                                      f(vdata["beta_logits"]), f(vdata["A_log"]),
                                      f(vdata["dt_bias"]), vdata["lower_bound"],
                                      vdata["state_pool"].numpy(), vdata["state_idx"].numpy(), 8)
    TOL.assert_output_ok(op, o_ref)
    TOL.assert_output_ok(ov, o_ref)
    TOL.assert_state_ok(fp, i_ref[:, -1])
    TOL.assert_state_ok(iv[:, -1], i_ref[:, -1])


# ---------------------------------------------------------------- fp16 operand range

def test_prefill_large_values_near_2_13():
    """v and the start states scaled by a power of two to |v| in [2^12, 2^13): the fp16
    scan operands (S, X = V - K_Gamma S, U = T'X) grow with them and must stay in range;
    the relative bar is unchanged.  check=True accepts the call."""
    case = W.PrefillCase("large_v", [2048, 700, 64], 4, init="per_seq", seed=3301)
    data = W.make_prefill(case)
    c = 2.0 ** np.floor(np.log2(2.0 ** 13 / float(data["v"].float().abs().max())))
    data["v"] = (data["v"].float() * c).to(torch.bfloat16)             # exact: power of two
    data["initial_state"] = data["initial_state"] * c
    vmax = float(data["v"].float().abs().max())
    print(f"case {case.name} max|v| {vmax:.0f}", flush=True)
    assert 2.0 ** 12 <= vmax < 2.0 ** 13
    d = _dev(data)
    out, final = _call(d, check=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(final).all())
    _compare(data, out, final)


def test_prefill_check_rejects_values_past_the_fp16_range():
    case = W.PrefillCase("too_large_v", [100], 2, init="per_seq", seed=3302)
    data = W.make_prefill(case)
    d = _dev(data)
    big = d["v"].clone()
    big[3, 1, 7] = 2.0 ** 14
    with pytest.raises(ValueError, match="v"):
        chunk_prefill(d["q"], d["k"], big, d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
                      d["lower_bound"], d["cu_seqlens"], initial_state=d["initial_state"],
                      check=True)
    init = d["initial_state"].clone()
    init[0, 0, 5, 5] = -2.0 ** 14
    with pytest.raises(ValueError, match="initial_state"):
        chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"],
                      d["dt_bias"], d["lower_bound"], d["cu_seqlens"], initial_state=init,
                      check=True)


# ---------------------------------------------------------------- full workload sizes (sampled heads)

FULL = [
    (W.VARLEN, [0, 9], [0, 7]),
    (W.LONG, [3, 12], [0, 3]),
    (W.SINGLE_LONG, [5], [0]),
]


@pytest.mark.parametrize("case,heads,seqs", FULL, ids=[c[0].name for c in FULL])
def test_prefill_full_size_sampled(case, heads, seqs):
    print(f"case {case.name} seed {case.seed} heads {heads} seqs {seqs}", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    out = None
    if case.init == "pool":
        # the layer buffer is preallocated and written in place
        out = torch.empty((d["q"].shape[0], d["q"].shape[1], 128), dtype=torch.bfloat16, device="cuda")
    o, fin = _call(d, out=out) if out is not None else _call(d)
    torch.cuda.synchronize()
    if out is not None:
        assert o.data_ptr() == out.data_ptr()
    _compare(data, o, fin, heads=heads, seqs=seqs)


@pytest.mark.parametrize("case", [c[0] for c in FULL], ids=[c[0].name for c in FULL])
def test_prefill_full_size_every_pair(case):
    """The launch the benchmark times, compared with the oracle on every (sequence, head)
    pair: each pair's outputs against that pair's RMS and each pair's final state on its
    own.  This covers every work unit of the scan's workgroup maps (value slices, XCD
    interleave, segments)."""
    print(f"case {case.name} seed {case.seed}: GPU call", flush=True)
    data = W.make_prefill(case)
    d = _dev(data)
    out = None
    if case.init == "pool":
        out = torch.empty((d["q"].shape[0], d["q"].shape[1], 128), dtype=torch.bfloat16, device="cuda")
    o, fin = _call(d, out=out) if out is not None else _call(d)
    torch.cuda.synchronize()
    o_gpu = o.cpu()
    f_gpu = fin.cpu()
    del d, o, fin
    print("  oracle over every pair", flush=True)
    o_ref, f_ref, _ = _oracle(data)
    cu = data["cu_seqlens"].numpy().astype(np.int64)
    N, H = len(cu) - 1, data["q"].shape[1]
    worst_e, worst_r = 0.0, 0.0
    for n in range(N):
        for h in range(H):
            e = TOL.assert_output_ok(o_gpu[cu[n]:cu[n + 1], h], o_ref[cu[n]:cu[n + 1], h])
            r = TOL.assert_state_ok(f_gpu[n, h], f_ref[n, h])
            worst_e, worst_r = max(worst_e, e["excess_over_rms"]), max(worst_r, r)
    print(f"  {N * H} pairs: worst output excess/RMS {worst_e:.2e}, worst state rel L2 "
          f"{worst_r:.2e}", flush=True)


# ---------------------------------------------------------------- segment-parallel scan
# Few (sequence, head) pairs with long sequences take the segment-parallel scan: each
# segment's state map and offset from a zero start, a combine, then the later segments
# from their start states.  These shapes force it (2 heads leave most CUs idle) with
# ragged tails, empty segments of a short sequence, gathered and out-of-pool starts.

@pytest.mark.parametrize("lens,H,init", [
    ([64 * 40 + 17], 2, "per_seq"),
    ([3000, 100, 1500], 2, "pool"),
    ([64 * 33, 64 * 12], 1, None),
    ([64 * 24 + 5], 14, "per_seq"),   # 14 pairs: G = 5, phases A and C on 224 workgroups
])
def test_prefill_segmented_scan(lens, H, init):
    case = W.PrefillCase(f"seg_{len(lens)}x{H}", lens, H, init=init, pool_slots=5,
                         seed=3200 + sum(lens) % 97)
    print(f"case {case.name} lens {lens} seed {case.seed}", flush=True)
    data = W.make_prefill(case)
    if init == "pool":
        data["initial_state_idx"][1] = -1          # a sequence starting from zero
    d = _dev(data)
    out, fin = _call(d)
    torch.cuda.synchronize()
    _compare(data, out, fin)


def test_prefill_segmented_scan_scatter_and_in_place_final():
    case = W.PrefillCase("seg_scatter", [64 * 40 + 17], 2, init="per_seq", seed=3210)
    data = W.make_prefill(case)
    d = _dev(data)
    T, H = d["q"].shape[:2]
    plain, fin_plain = _call(d)
    R = T + 9
    idx = torch.from_numpy(np.random.default_rng(3211).permutation(R)[:T].astype(np.int32)).cuda()
    out = torch.zeros((R, H, 128), dtype=torch.bfloat16, device="cuda")
    state = d["initial_state"].clone()
    chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"], d["dt_bias"],
                  d["lower_bound"], d["cu_seqlens"], initial_state=state, out=out,
                  final_state=state, scale=d["scale"], out_token_index=idx)
    torch.cuda.synchronize()
    assert torch.equal(out[idx.long()].view(torch.int16).cpu(), plain.view(torch.int16).cpu())
    assert torch.equal(state.cpu(), fin_plain.cpu())
