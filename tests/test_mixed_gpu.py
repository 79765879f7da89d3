"""GPU parity of the mixed speculative step pieces: outputs scattered by token index
straight into the layer buffer (prefill and verify), and the rollback commit.

All calls go through the C ABI (ctypes binding) on seeded inputs from
linear_attention_rule_amd.workloads.  The scatter changes only where rows land, so
a scattered call must equal the plain call row for row, bit for bit, and leave
every row no token names untouched; the merged step is also compared with the
oracle (its outputs placed by oracle.scatter_rows).  The commit is a copy, so it is
compared bit for bit with oracle.commit_accepted on the same (seeded) inputs, and
end to end (verify, then commit) with the oracle's prefill over each accepted prefix.
"""

import numpy as np
import pytest
import torch

import tolerances as TOL
from linear_attention_rule_amd import chunk_prefill, commit_accepted, recurrent_verify
from linear_attention_rule_amd import workloads as W
from oracle import kda_oracle as O

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1   # a bf16 NaN pattern no kernel writes


def _dev(data):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in data.items()}


def _prefill(d, **kw):
    return chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"],
                         d["dt_bias"], d["lower_bound"], d["cu_seqlens"],
                         initial_state=d["initial_state"], initial_state_idx=d["initial_state_idx"],
                         scale=d["scale"], **kw)


def _verify(d, **kw):
    return recurrent_verify(d["q"], d["k"], d["v"], d["g"], d["beta_logits"], d["A_log"],
                            d["dt_bias"], d["lower_bound"], d["state_pool"], d["state_idx"],
                            d["num_steps"], scale=d["scale"], **kw)


def _sentinel_out(rows, H):
    return torch.full((rows, H, 128), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu()


def test_prefill_scatter_equals_plain_rows():
    case = W.PrefillCase("scatter_pre", [100, 64, 0, 37, 130], 3, init="per_seq", seed=3100)
    print(f"case {case.name} seed {case.seed}", flush=True)
    d = _dev(W.make_prefill(case))
    T, H = d["q"].shape[:2]
    plain, fin_plain = _prefill(d)
    R = T + 23
    rng = np.random.default_rng(3101)
    idx = torch.from_numpy(rng.permutation(R)[:T].astype(np.int32)).cuda()
    out = _sentinel_out(R, H)
    _, fin = _prefill(d, out=out, out_token_index=idx)
    torch.cuda.synchronize()
    ob, pb = _bits(out), _bits(plain)
    il = idx.long().cpu()
    assert torch.equal(ob[il], pb)
    rest = torch.ones(R, dtype=torch.bool)
    rest[il] = False
    assert bool((ob[rest] == SENTINEL).all())
    assert torch.equal(fin.cpu(), fin_plain.cpu())


def test_prefill_scatter_drops_out_of_range_rows():
    case = W.PrefillCase("scatter_drop", [70, 61], 2, seed=3102)
    d = _dev(W.make_prefill(case))
    T, H = d["q"].shape[:2]
    plain, _ = _prefill(d)
    R = T
    idx_np = np.arange(T, dtype=np.int32)[::-1].copy()
    drop = [0, 5, 64, 130]
    idx_np[drop[0]], idx_np[drop[1]], idx_np[drop[2]], idx_np[drop[3]] = -1, R, R + 7, -100
    idx = torch.from_numpy(idx_np).cuda()
    out = _sentinel_out(R, H)
    _prefill(d, out=out, out_token_index=idx)
    torch.cuda.synchronize()
    ob, pb = _bits(out), _bits(plain)
    keep = [t for t in range(T) if t not in drop]
    assert torch.equal(ob[torch.from_numpy(idx_np[keep]).long()], pb[keep])
    unnamed = sorted(set(range(R)) - set(int(idx_np[t]) for t in keep))
    assert bool((ob[unnamed] == SENTINEL).all())


def test_verify_scatter_equals_plain_rows_with_padding():
    case = W.VerifyCase("scatter_ver", 6, 3, 2, pool_slots=9, seed=3103, padding_rows=[2])
    d = _dev(W.make_verify(case))
    BT, H = d["q"].shape[:2]
    plain, inter_plain = _verify(d)
    R = BT + 11
    rng = np.random.default_rng(3104)
    idx = torch.from_numpy(rng.permutation(R)[:BT].astype(np.int32)).cuda()
    out = _sentinel_out(R, H)
    _, inter = _verify(d, out=out, out_token_index=idx)
    torch.cuda.synchronize()
    ob, pb = _bits(out), _bits(plain)
    il = idx.long().cpu()
    assert torch.equal(ob[il], pb)          # padding row 2's tokens: zeros at their rows
    assert bool((pb[6:9] == 0).all())
    rest = torch.ones(R, dtype=torch.bool)
    rest[il] = False
    assert bool((ob[rest] == SENTINEL).all())
    live = [b for b in range(6) if b != 2]
    assert torch.equal(inter.cpu()[live], inter_plain.cpu()[live])


def _mixed_small():
    return W.MixedCase("mixed_small",
                       W.PrefillCase("mixed_small_pre", [90, 0, 200, 64], 3, init=None, seed=3105),
                       W.VerifyCase("mixed_small_spec", 7, 4, 3, pool_slots=12, seed=3106),
                       extra_rows=9, seed=3107)


def _run_mixed(m):
    pre, spec = _dev(m["prefill"]), _dev(m["spec"])
    H = pre["q"].shape[1]
    core = _sentinel_out(m["out_rows"], H)
    _, fin = _prefill(pre, out=core, out_token_index=m["non_spec_idx"].cuda())
    _, inter = _verify(spec, out=core, out_token_index=m["spec_idx"].cuda())
    return core, fin, inter, spec


def test_mixed_step_matches_oracle():
    case = _mixed_small()
    print(f"case {case.name} seed {case.seed}", flush=True)
    m = W.make_mixed(case)
    core, fin, inter, _ = _run_mixed(m)
    torch.cuda.synchronize()
    f = W.to_f64
    p, s = m["prefill"], m["spec"]
    op, fp = O.chunk_prefill(f(p["q"]), f(p["k"]), f(p["v"]), f(p["g"]), f(p["beta_logits"]),
                             f(p["A_log"]), f(p["dt_bias"]), p["lower_bound"],
                             p["cu_seqlens"].numpy(), scale=p["scale"])
    ov, iv = O.recurrent_verify(f(s["q"]), f(s["k"]), f(s["v"]), f(s["g"]), f(s["beta_logits"]),
                                f(s["A_log"]), f(s["dt_bias"]), s["lower_bound"],
                                s["state_pool"].numpy(), s["state_idx"].numpy(), s["num_steps"],
                                scale=s["scale"])
    R = m["out_rows"]
    merged = O.scatter_rows(ov, m["spec_idx"].numpy(), R,
                            O.scatter_rows(op, m["non_spec_idx"].numpy(), R))
    named = np.concatenate([m["non_spec_idx"].numpy(), m["spec_idx"].numpy()])
    TOL.assert_output_ok(core[torch.from_numpy(named).long().cuda()], merged[named])
    unnamed = sorted(set(range(R)) - set(int(x) for x in named))
    assert bool((_bits(core)[unnamed] == SENTINEL).all())
    for n in range(fp.shape[0]):
        assert TOL.state_rel_l2(fin[n].cpu().numpy(), fp[n]) <= TOL.STATE_TOL
    for b in range(iv.shape[0]):
        assert TOL.state_rel_l2(inter[b].cpu().numpy(), iv[b]) <= TOL.STATE_TOL


def test_commit_bitwise_on_seeded_inputs():
    rng = np.random.default_rng(3108)
    B, T, H, slots = 9, 5, 2, 12
    inter = torch.from_numpy(rng.standard_normal((B, T, H, 128, 128), dtype=np.float32))
    pool = torch.from_numpy(rng.standard_normal((slots, H, 128, 128), dtype=np.float32))
    idx = rng.permutation(slots)[:B].astype(np.int32)
    idx[3], idx[7] = -1, slots            # padding rows
    nacc = np.array([1, 5, 3, 2, 0, 6, 4, 1, 2], dtype=np.int32)   # 0 and 6 > T commit nothing
    want = O.commit_accepted(pool.numpy(), inter.numpy(), idx, nacc)
    got = commit_accepted(inter.cuda(), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(nacc).cuda(), pool.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_verify_then_commit_equals_prefill_of_accepted_prefix():
    case = W.VerifyCase("commit_e2e", 5, 6, 2, pool_slots=8, seed=3109, padding_rows=[4])
    data = W.make_verify(case)
    d = _dev(data)
    _, inter = _verify(d)
    nacc = torch.tensor([2, 6, 1, 4, 3], dtype=torch.int32)
    pool = d["state_pool"].clone()
    commit_accepted(inter, d["state_idx"], nacc.cuda(), pool)
    torch.cuda.synchronize()
    f = W.to_f64
    got = pool.cpu().numpy()
    idx = data["state_idx"].numpy()
    T = data["num_steps"]
    for b in range(case.batch):
        s, n = int(idx[b]), int(nacc[b])
        if not (0 <= s < case.pool_slots):
            continue
        rows = slice(b * T, b * T + n)
        _, fin = O.chunk_prefill(f(data["q"])[rows], f(data["k"])[rows], f(data["v"])[rows],
                                 f(data["g"])[rows], f(data["beta_logits"])[rows],
                                 f(data["A_log"]), f(data["dt_bias"]), data["lower_bound"],
                                 [0, n], data["state_pool"].numpy(), [s], scale=data["scale"])
        assert TOL.state_rel_l2(got[s], fin[0]) <= 2e-5
    named = {int(idx[b]) for b in range(case.batch) if 0 <= int(idx[b]) < case.pool_slots}
    for s in set(range(case.pool_slots)) - named:
        assert np.array_equal(got[s], data["state_pool"].numpy()[s])


def test_commit_looping_workgroups_with_skipped_rows():
    """48 rows x 16 heads is more than two (row, head) items per CU on 256 CUs: each
    workgroup loops, loading its next item before storing the current one.  Rows that
    commit nothing (padding slots, no accepted token, more than T) sit among them and
    leave their pool slots as they were."""
    rng = np.random.default_rng(3112)
    B, T, H, slots = 48, 4, 16, 64
    inter = torch.from_numpy(rng.standard_normal((B, T, H, 128, 128), dtype=np.float32))
    pool = torch.from_numpy(rng.standard_normal((slots, H, 128, 128), dtype=np.float32))
    idx = rng.permutation(slots)[:B].astype(np.int32)
    idx[0], idx[17], idx[B - 1] = -1, slots, -3
    nacc = rng.integers(1, T + 1, size=B).astype(np.int32)
    nacc[5], nacc[30] = 0, T + 1
    want = O.commit_accepted(pool.numpy(), inter.numpy(), idx, nacc)
    got = commit_accepted(inter.cuda(), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(nacc).cuda(), pool.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_commit_full_size_64x8_h16():
    """Full verify size: 64 rows, 8 steps, 16 heads, 256-slot pool, seeded intermediate."""
    rng = np.random.default_rng(3110)
    B, T, H, slots = 64, 8, 16, 256
    inter = torch.from_numpy(rng.standard_normal((B, T, H, 128, 128), dtype=np.float32))
    pool = torch.from_numpy(rng.standard_normal((slots, H, 128, 128), dtype=np.float32))
    idx = rng.permutation(slots)[:B].astype(np.int32)
    nacc = rng.integers(1, T + 1, size=B).astype(np.int32)
    got = commit_accepted(inter.cuda(), torch.from_numpy(idx).cuda(),
                          torch.from_numpy(nacc).cuda(), pool.cuda())
    torch.cuda.synchronize()
    want = O.commit_accepted(pool.numpy(), inter.numpy(), idx, nacc)
    assert np.array_equal(got.cpu().numpy(), want)


def test_mixed_full_size_sampled():
    """The MIXED workload at full size; the oracle checks sampled heads of two prefill
    sequences and of every spec row, placed through the merge indices."""
    m = W.make_mixed(W.MIXED)
    print(f"case {W.MIXED.name} seed {W.MIXED.seed}", flush=True)
    core, fin, inter, _ = _run_mixed(m)
    torch.cuda.synchronize()
    f = W.to_f64
    p, s = m["prefill"], m["spec"]
    heads = [0, 11]
    cu = p["cu_seqlens"].numpy()
    for n in (0, 5):
        rows = np.arange(cu[n], cu[n + 1])
        op, _ = O.chunk_prefill(f(p["q"])[rows][:, heads], f(p["k"])[rows][:, heads],
                                f(p["v"])[rows][:, heads], f(p["g"])[rows][:, heads],
                                f(p["beta_logits"])[rows][:, heads], f(p["A_log"])[heads],
                                f(p["dt_bias"])[heads], p["lower_bound"], [0, len(rows)],
                                scale=p["scale"])
        dst = torch.from_numpy(m["non_spec_idx"].numpy()[rows]).long().cuda()
        TOL.assert_output_ok(core[dst][:, heads], op)
    ov, _ = O.recurrent_verify(f(s["q"])[:, heads], f(s["k"])[:, heads], f(s["v"])[:, heads],
                               f(s["g"])[:, heads], f(s["beta_logits"])[:, heads],
                               f(s["A_log"])[heads], f(s["dt_bias"])[heads], s["lower_bound"],
                               s["state_pool"].numpy()[:, heads], s["state_idx"].numpy(),
                               s["num_steps"], scale=s["scale"])
    TOL.assert_output_ok(core[m["spec_idx"].long().cuda()][:, heads], ov)
