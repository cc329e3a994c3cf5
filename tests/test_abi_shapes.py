"""moe_ctx_create against the shape contract that include/moe_ep.h states, over random shapes (CPU only: no
device memory, no launch).  The expected status is computed here from the header's wording; a shape the
library accepts must report the sizes the header defines."""

import ctypes

from hypothesis import given, settings, strategies as st

def _expected(P, Tp, E, k, H, dt):
    if P < 1 or Tp < 0 or E < 1 or E % P != 0 or k < 1 or k > E or H < 8 or H % 8 != 0 or dt not in (0, 1):
        return -1
    T = P * Tp
    Na = T * k
    if (E > 1024 or E // P > 32767 or k > 32 or H > 65536 or (dt == 1 and H % 128 != 0) or Na >= 1 << 31
            or Na * (H // 1024 + 1) >= 1 << 31 or (Na + P) * (H // 8 + 512) >= 1 << 32):
        return -2
    return 0


_sizes = st.one_of(st.integers(-2, 70), st.integers(70, 70_000), st.sampled_from([1 << 16, 1 << 20, 1 << 28]))


@settings(max_examples=600, deadline=None)
@given(P=st.integers(-1, 40), Tp=_sizes, E=st.one_of(st.integers(-1, 300), st.sampled_from([512, 1024, 1025, 2048])),
       k=st.integers(-1, 40), H=st.one_of(st.integers(-8, 300), st.sampled_from([7168, 8192, 65536, 65544, 131072])),
       dt=st.integers(-1, 2))
def test_ctx_create_follows_the_header_contract(P, Tp, E, k, H, dt):
    from combine_router_softmax_expert_amd import binding as b
    s = b.MoeShape(P, Tp, E, k, H, dt)
    h = ctypes.c_void_p()
    status = b.lib.moe_ctx_create(ctypes.byref(s), ctypes.byref(h))
    want = _expected(P, Tp, E, k, H, dt)
    assert status == want, (P, Tp, E, k, H, dt, status, want)
    if status != 0:
        assert not h.value
        return
    try:
        assert b.lib.moe_num_assignments(h) == P * Tp * k
        assert b.lib.moe_dispatch_row_bytes(h) == (H if dt == 1 else 2 * H)
        assert b.lib.moe_scales_per_row(h) == (H // 128 if dt == 1 else 0)
        ws = b.lib.moe_workspace_bytes(h)
        assert ws > 0 and ws % 256 == 0
        # at least the two 16-byte handle records and four int32 arrays per assignment
        assert ws >= P * Tp * k * (2 * 16 + 4 * 4)
    finally:
        b.lib.moe_ctx_destroy(h)
