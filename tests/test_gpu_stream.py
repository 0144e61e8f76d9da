"""ffnq_moe_routed_streamed: routed experts kept in pinned host memory, each
sub-batch's union copied into a device slot cache before its phases run.
The result is checked against the oracle (the routed half over the whole
expert set), including caps that split the batch into several sub-batches and
caches just big enough for one union; the slot table is checked for reuse
(experts already held are not copied again) and a plan that does not fit the
cache, or that is not a plan for its ids, is refused before any copy."""
import numpy as np
import pytest
import torch

import gen
import moe_expert_dequant_amd as fq
import oracle
from test_gpu_parity import check, dev, dev16, host16, mats_dev, say

pytestmark = pytest.mark.gpu


def routed_inputs(hidden, E, inter, m, k, cap, seed):
    inp = gen.moe_inputs(hidden, E, inter, m, seed=seed)
    rc, ids_o, w_o, plan_o = oracle.moe_route(inp["logits"], k, cap)
    assert rc == 0
    ids = torch.zeros((m, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    plan = torch.zeros((fq.plan_ints(m, k),), dtype=torch.int32, device="cuda")
    fq.moe_route(dev(inp["logits"].astype(np.float32)), m, E, k, cap, ids, w, plan)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_o) and np.array_equal(plan.cpu().numpy(), plan_o)
    return inp, ids, w, plan, ids_o, w_o, plan_o


@pytest.mark.parametrize("m,E,k,cap,n_slots", [
    (1, 16, 4, 8, 8),
    (5, 16, 4, 6, 6),      # several sub-batches, every slot refilled
    (5, 16, 4, 6, 12),     # several sub-batches, room to keep experts between them
    (8, 16, 8, 16, 16),    # 64 pairs
    (4, 128, 8, 32, 32),   # Qwen-like routing: one union of up to 32 experts
    (20, 16, 2, 16, 16),   # more rows per expert
])
def test_streamed_matches_oracle(m, E, k, cap, n_slots):
    hidden, inter = 512, 256
    say("streamed", m, E, k, cap, n_slots)
    inp, ids, w, plan, ids_o, w_o, plan_o = routed_inputs(hidden, E, inter, m, k, cap, 6100 + m + E + k)
    d = mats_dev(inp["experts"], True, E)
    hx_d, hx = fq.host_experts(d)
    del d
    seed_bits = gen.act_rows(gen.tensor_key(6101, m), m, hidden)
    cache = fq.SlotCache(n_slots, hidden, inter)
    resid = dev16(inp["resid"])
    fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, dev16(inp["x"]), ids, w, plan,
                           dev16(seed_bits), resid, cache)
    torch.cuda.synchronize()
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids_o, w_o, seed_bits,
                             inp["resid"])
    check(host16(resid), want, f"streamed m {m} E {E} k {k} cap {cap} slots {n_slots}")
    # every union expert of every sub-batch went through a slot; the table names what the slots hold
    f = oracle.plan_fields(plan_o, m, k)
    S = f["n_sub"]
    unions = [set(f["union_expert"][f["sub_union_begin"][b]:f["sub_union_begin"][b + 1]]) for b in range(S)]
    assert cache.copied >= len(unions[-1]) and cache.copied <= sum(len(u) for u in unions)
    held = set(int(e) for e in cache.expert if e >= 0)
    assert unions[-1] <= held


def test_streamed_cache_reuse():
    hidden, inter, E, m, k, cap = 512, 256, 16, 3, 4, 12
    say("streamed cache reuse")
    inp, ids, w, plan, ids_o, w_o, plan_o = routed_inputs(hidden, E, inter, m, k, cap, 6200)
    d = mats_dev(inp["experts"], True, E)
    hx_d, hx = fq.host_experts(d)
    cache = fq.SlotCache(16, hidden, inter)
    x = dev16(inp["x"])
    outs = []
    for call in range(2):
        resid = dev16(inp["resid"])
        before = cache.copied
        fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, x, ids, w, plan, None, resid, cache)
        torch.cuda.synchronize()
        outs.append(host16(resid))
        union = len(set(ids_o.ravel().tolist()))
        assert cache.copied - before == (union if call == 0 else 0), call   # the second call copies nothing
    assert np.array_equal(outs[0], outs[1])
    want = oracle.moe_routed(inp["experts"], E, hidden, inter, gen.ACT_SILU, inp["x"], ids_o, w_o, None,
                             inp["resid"])
    check(outs[1], want, "streamed from a warm cache")
    # a slot the table no longer claims: the next call copies that expert again, and only that one
    s = int(np.flatnonzero(cache.expert >= 0)[0])
    cache.expert[s] = -1
    resid = dev16(inp["resid"])
    before = cache.copied
    fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, x, ids, w, plan, None, resid, cache)
    torch.cuda.synchronize()
    assert cache.copied - before == 1
    assert np.array_equal(host16(resid), outs[0])


def test_streamed_refuses_union_past_cache_and_bad_plan():
    hidden, inter, E, m, k, cap = 512, 256, 16, 4, 4, 8
    say("streamed refusals")
    inp, ids, w, plan, ids_o, w_o, plan_o = routed_inputs(hidden, E, inter, m, k, cap, 6300)
    d = mats_dev(inp["experts"], True, E)
    hx_d, hx = fq.host_experts(d)
    x = dev16(inp["x"])
    f = oracle.plan_fields(plan_o, m, k)
    largest = max(f["sub_union_begin"][b + 1] - f["sub_union_begin"][b] for b in range(f["n_sub"]))
    small = fq.SlotCache(int(largest) - 1, hidden, inter)
    resid = dev16(inp["resid"])
    with pytest.raises(fq.FfnqError) as e:
        fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, x, ids, w, plan, None, resid, small)
    assert e.value.status == -3 and small.copied == 0
    # a pair slot outside its union: refused before any copy, resid untouched
    bad = plan.clone()
    bad[2 * m + 3 + m * k] = 31
    cache = fq.SlotCache(16, hidden, inter)
    with pytest.raises(fq.FfnqError) as e:
        fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, x, ids, w, bad, None, resid, cache)
    assert e.value.status == -1 and cache.copied == 0
    # ids that disagree with the plan's union
    bad_ids = ids.clone()
    bad_ids[0, 0] = (int(ids_o[0, 0]) + 1) % E
    with pytest.raises(fq.FfnqError) as e:
        fq.moe_routed_streamed(hx, E, hidden, inter, m, k, gen.ACT_SILU, x, bad_ids, w, plan, None, resid, cache)
    assert e.value.status == -1 and cache.copied == 0
    torch.cuda.synchronize()
    assert np.array_equal(host16(resid), inp["resid"])
