"""The GPU parity sweep's random shapes (fuzz_cases.py), on the CPU: each is a
valid chunk step for the library, and together they cover every head dim,
page size and dtype and each of the method's edge cases."""
import paged_sparse_attention_amd as P

import fuzz_cases


def test_cases_are_valid_and_cover_the_edges():
    cs = fuzz_cases.cases()
    assert len(cs) == fuzz_cases.N_CASES
    assert cs == fuzz_cases.cases()                      # deterministic
    for seed, p in cs:
        desc = P.make_desc(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.k, p.slots, dtype=p.dtype, softmax_scale=p.scale)
        assert P.oomb_bwd_workspace_bytes(desc) > 0, p      # 0 means the descriptor is rejected
        assert P.oomb_select_workspace_bytes(desc) > 0, p
    ps = [p for _, p in cs]
    assert {p.d for p in ps} == {64, 128}
    assert {p.ps for p in ps} == {16, 32, 64, 128}
    assert {p.dtype for p in ps} == {"bf16", "f32"}
    assert any(p.n == 0 for p in ps)                      # no prior pages
    assert any(p.n > 0 and p.k == 0 for p in ps)          # local chunk only
    assert any(p.n > 0 and p.k >= p.n for p in ps)        # every prior page (dense)
    assert any(0 < p.k < p.n for p in ps)                 # a true top-K
    assert any(p.c == p.ps for p in ps)                   # a one-page chunk
    assert any(p.n_slots > p.n + p.c // p.ps for p in ps) # spare pool slots
    assert any(p.scale > 0 for p in ps)                   # softmax-scale override
    assert any(p.hq == p.hkv for p in ps) and any(p.hq // p.hkv >= 7 for p in ps)
