"""Host-side checks of bi_gemm's configuration rule (bi_gemm_tile; no GPU work).

The rule only chooses how the product is computed, never its bits, so these
tests check the properties the library relies on: the exclusions that keep
zero padding uniform, when non-temporal weight loads are used, the vocabulary
rule, and that the choice is a function of the arguments alone."""
import itertools

import pytest

from _helpers import bi

SHAPES = list(itertools.product((1, 7, 16, 33, 64, 65, 128, 129, 256, 300, 1024, 2300, 4096),
                                (100, 1024, 4096, 6144, 12288, 24576),
                                (64, 96, 160, 192, 512, 4096, 12288)))


def test_rule_excludes_128_wide_stages_when_k_pads_them():
    """K a multiple of 64 but not of 128: no configuration with 128-wide K
    stages (every candidate then ends K without zero-padded MFMA steps); K not
    a multiple of 64: both kinds may run (every candidate pads)."""
    for m, n, k in SHAPES:
        c = bi.gemm_config(m, n, k)
        if k % 128 == 64:
            assert c[5] == 64, (m, n, k, c)


def test_stream_w_only_when_one_small_m_tile_holds_every_row():
    for m, n, k in SHAPES:
        c = bi.gemm_config(m, n, k)
        tn, tm, stream = c[0], c[1], c[7]
        if stream:
            assert tm <= 64 and m <= tm, (m, n, k, c)
        elif tm <= 64:
            assert m > tm, (m, n, k, c)


def test_vocabulary_rule():
    """N >= 32768: 128 x 256 below 512 rows (non-temporal weight loads up to 256
    rows), 256 x 256 from 512 rows."""
    for m in (1, 64, 256, 257, 511, 512, 2048):
        c = bi.gemm_config(m, 151936, 4096)
        if m < 512:
            assert c[:2] == (128, 256) and c[7] == (1 if m <= 256 else 0), (m, c)
        else:
            assert c[:2] == (256, 256) and c[7] == 0, (m, c)


def test_fused_gate_up_decode_rule():
    """N >= 16384 (below the vocabulary rule) at M <= 32: the 32 x 64 tile with
    two workgroups per CU and non-temporal weight loads."""
    for m in (1, 8, 32):
        assert bi.gemm_config(m, 24576, 4096) == (32, 64, 2, 2, 6, 64, 2, 1)


def test_rule_is_a_function_of_its_arguments():
    first = [bi.gemm_config(m, n, k) for m, n, k in SHAPES]
    again = [bi.gemm_config(m, n, k) for m, n, k in reversed(SHAPES)][::-1]
    assert first == again


def test_rule_respects_buffer_offset_limits():
    """A stride that makes every tile's slice of W span 2^31 bytes or more has
    no configuration that fits: bi_gemm_tile still answers (the launch then
    reports BI_ERR_UNSUPPORTED), and a stride that only the narrow tiles fit
    picks one of them."""
    c = bi.gemm_config(4, 4, 64, ldw=1 << 26)
    assert c[:2] == (32, 16)
    # (TN - 1) * ldw * 2 + 2 k < 2^31 at ldw = 2^25 holds for tiles of at most 32 weight rows
    c = bi.gemm_config(200, 4096, 4096, ldw=1 << 25)
    assert c[0] <= 32, c
