"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a textual edit of oracle.c compiled into a throw-away library in a
temporary directory (the committed oracle is never touched).  The edits are the
plausible slips of this computation: a wrong head mapping, a dropped or doubled
scale, a dropped normalisation, an off-by-one in the causal range or the context,
a leak across sequences, a wrong page slot, values swapped for keys, an ignored
start position, a wrong query row, a float accumulator, a flipped exponent sign,
a missing max subtraction.  Every edit keeps memory accesses inside the buffers,
so a mutant can only produce wrong numbers, not crash the test process.
"""

import shutil
from pathlib import Path

import pytest

import oracle_pins as P
from oracle import Oracle
from oracle.build import build

SRC = Path(__file__).resolve().parent.parent / "oracle"

# (id, text in oracle.c, replacement)
MUTANTS = [
    ("interleaved_kv_head", "const int32_t h = qh / group;", "const int32_t h = qh % num_kv_heads;"),
    ("scale_dropped", "return scale * acc;", "return acc;"),
    ("scale_squared", "return scale * acc;", "return scale * scale * acc;"),
    ("no_normalisation", "for (int64_t j = 0; j < n; ++j) p[j] = p[j] / z;", ""),
    ("no_max_subtraction", "p[j] = exp(s[j] - m);", "p[j] = exp(s[j]);"),
    ("exp_sign_flipped", "p[j] = exp(s[j] - m);", "p[j] = exp(m - s[j]);"),
    ("decode_drops_last_token", "const int64_t n = context_lens[b];", "const int64_t n = context_lens[b] - 1;"),
    ("causal_excludes_diagonal", "const int64_t last = causal ? i :", "const int64_t last = causal ? i - 1 :"),
    ("cross_sequence_leak", "int64_t first = cu_seqlens[seq];", "int64_t first = 0;"),
    ("decode_slot_shifted", "const int64_t slot = j % block_size;", "const int64_t slot = (j + 1) % block_size;"),
    ("values_are_keys", "softmax_weighted_sum(s, n - lo, v_cache, voff, head_dim, dtype, p, o);\n            if (probs)", "softmax_weighted_sum(s, n - lo, k_cache, voff, head_dim, dtype, p, o);\n            if (probs)"),
    ("write_ignores_start_pos", "const int64_t pos = (int64_t)start_pos[b] + (t - cu_seqlens[b]);",
     "const int64_t pos = (t - cu_seqlens[b]);"),
    ("gather_ignores_head", "const int64_t src = page_offset(blk, h, slot,", "const int64_t src = page_offset(blk, 0, slot,"),
    ("query_of_head_zero", "const int64_t qo = u * head_dim;", "const int64_t qo = (u - qh) * head_dim;"),
    ("prefill_kv_head_zero", "const int64_t ko = ((first + j) * num_kv_heads + h)",
     "const int64_t ko = ((first + j) * num_kv_heads + 0)"),
    ("float_accumulator", "double acc = 0.0;\n    for (int32_t x = 0; x < head_dim; ++x) acc += elem(q,",
     "float acc = 0.0f;\n    for (int32_t x = 0; x < head_dim; ++x) acc += elem(q,"),
    ("table_ignored", "int64_t blk = block_table[(int64_t)b * max_blocks_per_seq + page];",
     "int64_t blk = ((int64_t)b * max_blocks_per_seq + page) % num_blocks;"),
    ("extend_top_left_alignment", "const int64_t pos = (int64_t)context_lens[b] - q_len + i;",
     "const int64_t pos = i;"),
    ("extend_drops_own_key", "const int64_t n = pos + 1;   /* keys 0 .. pos */", "const int64_t n = pos;"),
    ("decode_window_one_extra_key", "const int64_t lo = (window > 0 && n > window) ? n - window : 0;\n            const int64_t qo = u * head_dim;",
     "const int64_t lo = (window > 0 && n > window) ? n - window - 1 : 0;\n            const int64_t qo = u * head_dim;"),
    ("prefill_window_one_extra_key", "if (window > 0 && i - window + 1 > first) first = i - window + 1;",
     "if (window > 0 && i - window > first) first = i - window;"),
    ("extend_window_ignored", "const int64_t lo = (window > 0 && n > window) ? n - window : 0;   /* newest",
     "const int64_t lo = 0;   /* newest"),
    ("fp8_ties_to_odd", "if (du < dl || (du == dl && ((lo + 1) & 1) == 0)) best = lo + 1;",
     "if (du < dl || (du == dl && ((lo + 1) & 1) == 1)) best = lo + 1;"),
    ("fp8_scale_over_127", "const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;",
     "const float sc = amax > 0.0f ? amax / 127.0f : 1.0f;"),
    ("fp8_subnormal_exponent", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    ("fp8_dequant_ignores_scale", "out[r * head_dim + i] = e4m3_value(codes[r * head_dim + i]) * (double)scales[r];",
     "out[r * head_dim + i] = e4m3_value(codes[r * head_dim + i]);"),
    ("copy_skips_v", "memmove((char*)v_cache + to * es, (const char*)v_cache + from * es, row_bytes);", ""),
    ("copy_head_zero", "const int64_t from = page_offset(src[i], h, slot,", "const int64_t from = page_offset(src[i], 0, slot,"),
]


def _build_variant(tmp: Path, old: str, new: str) -> Oracle:
    shutil.copy(SRC / "oracle.h", tmp / "oracle.h")
    text = (SRC / "oracle.c").read_text()
    if old is not None:
        assert old in text, f"mutation target not found: {old!r}"
        text = text.replace(old, new)
    (tmp / "oracle.c").write_text(text)
    return Oracle(build(tmp / "oracle.c", tmp / "liboracle_variant.so", extra_flags=("-w",)))


def _failures(orc):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # a pin fails by assertion or by the oracle's own error
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_copy_passes(tmp_path):
    assert _failures(_build_variant(tmp_path, None, None)) == []


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, old, new):
    failed = _failures(_build_variant(tmp_path, old, new))
    assert failed, f"planted mistake {mid} passed every pin"


# Planted mistakes in the block-refcount model (oracle/block_model.py), applied by
# patching one method of the class for the duration of the test.
def _append_without_copy(self, seq, n):
    table, length = self.tables[seq], self.lengths[seq]
    for _ in range(self._pages(length + n) - len(table)):
        b = self.free_blocks()[0]
        self.ref[b] = 1
        table.append(b)
    self.lengths[seq] = length + n
    return None


def _free_without_release(self, seq):
    self.tables.pop(seq)
    del self.lengths[seq]


def _fork_without_reference(self, parent):
    child = self.new_sequence()
    self.tables[child] = list(self.tables[parent])
    self.lengths[child] = self.lengths[parent]
    return child


MODEL_MUTANTS = [("append_without_copy", "append", _append_without_copy),
                 ("free_without_release", "free", _free_without_release),
                 ("fork_without_reference", "fork", _fork_without_reference)]


@pytest.mark.parametrize("mid,name,fn", MODEL_MUTANTS, ids=[m[0] for m in MODEL_MUTANTS])
def test_model_mutant_is_caught(monkeypatch, mid, name, fn):
    from oracle.block_model import BlockModel
    monkeypatch.setattr(BlockModel, name, fn)
    failed = []
    for pin in (P.pin_block_model_invariants, P.pin_block_model_shared_prompt):
        try:
            pin(None)
        except Exception as e:
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"planted mistake {mid} passed every model pin"
