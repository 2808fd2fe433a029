"""CPU tier: host-side address arithmetic of the kernels' range-checked loads.

The decoder brings each 64-token group of K into LDS with buffer loads whose
descriptor covers exactly the group's valid rows.  The hardware compares only
the per-lane (VGPR) offset with that range, so every byte offset must sit in
the lane operand: a lane whose token is past the end then reads zeros rather
than memory past the tensor.  These tests replay the load offsets of
``decode_bf16_kernel`` (K slot loads: lane l of load t reads token
(64 / ROWC) t + l / ROWC, chunk (l mod ROWC) XOR-swizzled by token bits 2..3)
for every ragged group size and both head widths, and check that each 16-byte
read is either wholly inside the valid rows of its own head or wholly outside
the descriptor's range.
"""
import pytest


def decoder_k_loads(D, sl):
    """(token, byte offset) of every 16-byte load lane of one K group."""
    rowc = D // 8
    kops = 64 * rowc // 64
    out = []
    for t in range(kops):
        for lane in range(64):
            tok0, sw = lane // rowc, lane % rowc
            dc = sw ^ ((tok0 >> 2) & (3 if D == 32 else 1))
            tok = tok0 + (64 // rowc) * t
            out.append((tok, (tok * sl + dc * 8) * 2, dc))
    return out


@pytest.mark.parametrize("D", [16, 32])
@pytest.mark.parametrize("layout", ["head", "token"])
def test_decoder_k_loads_stay_in_range(D, layout):
    H = 8
    sl = D if layout == "head" else H * D  # token stride in elements
    loads = decoder_k_loads(D, sl)
    # every token of the group is loaded once per 16-byte chunk
    seen = {}
    for tok, off, dc in loads:
        seen.setdefault(tok, set()).add(dc)
    assert sorted(seen) == list(range(64))
    assert all(s == set(range(D // 8)) for s in seen.values())
    for rows in range(1, 65):
        limit = rows * sl * 2  # bytes the descriptor covers
        for tok, off, dc in loads:
            if tok < rows:
                # inside the range, and inside this head's D features of a valid row
                assert off + 16 <= limit
                assert tok * sl * 2 <= off and off + 16 <= tok * sl * 2 + D * 2
            else:
                # wholly outside the range: the hardware returns zeros
                assert off >= limit
