"""The C ABI from a plain C program: include/chunkattn.h compiles as C99 and
C++17, and a C99 program linked against libchunkattn.so drives a host-only
context (no device pool, so no GPU is needed) through inserts that share and
split chunks, the table export, the status codes and the error text."""

import os
import shutil
import subprocess

import pytest

from decode_attention_prefix_tree_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = r"""
#include "chunkattn.h"
#include <stdio.h>
#include <string.h>

int main(void) {
  ca_ctx* c = NULL;
  if (ca_create(8, 128, 64, &c) != CA_OK || c == NULL) return 10;
  if (ca_attach_pool(c, NULL, 100) != CA_OK) return 11;
  int32_t t[100];
  for (int i = 0; i < 100; ++i) t[i] = i;
  int32_t matched = -1;
  if (ca_insert(c, 7, t, 100, NULL, NULL, NULL, &matched) != CA_OK || matched != 0) return 12;
  /* 70 tokens: the first chunk shared, the second split after 6 tokens */
  if (ca_insert(c, 9, t, 70, NULL, NULL, NULL, &matched) != CA_OK || matched != 70) return 13;
  if (ca_insert(c, 9, t, 3, NULL, NULL, NULL, NULL) != CA_E_DUP_SEQ) return 14;
  if (strlen(ca_last_error(c)) == 0) return 15;
  if (ca_remove(c, 5) != CA_E_UNKNOWN_SEQ) return 16;
  int n_rows = 0, n_seqs = 0;
  if (ca_export_table(c, NULL, 0, NULL, 0, &n_rows, &n_seqs) != CA_OK) return 17;
  int32_t rows[7 * 8];
  int64_t order[8];
  if (n_rows > 8 || ca_export_table(c, rows, 8, order, 8, &n_rows, &n_seqs) != CA_OK) return 18;
  int64_t ids[4];
  if (ca_list_sequences(c, ids, 4) != 2 || ids[0] != 7 || ids[1] != 9) return 19;
  printf("rows %d seqs %d\n", n_rows, n_seqs);
  for (int r = 0; r < n_rows; ++r)
    printf("row %d %d %d %d %d %d %d\n", rows[7 * r], rows[7 * r + 1], rows[7 * r + 2], rows[7 * r + 3],
           rows[7 * r + 4], rows[7 * r + 5], rows[7 * r + 6]);
  printf("slot_bytes %zu\n", ca_slot_bytes(32, 128, 64));
  ca_stats_t st;
  if (ca_stats(c, &st) != CA_OK) return 20;
  printf("stats %lld %lld %lld %lld %lld\n", (long long)st.live_sequences, (long long)st.chunks,
         (long long)st.shared_chunks, (long long)st.unique_tokens, (long long)st.attended_tokens);
  if (ca_set_option(c, CA_OPT_CF_CHUNKS_PER_TASK, 65) != CA_E_INVALID_ARG) return 21;
  if (ca_set_option(c, 12345, 0) != CA_E_UNSUPPORTED) return 22;
  if (ca_set_option(c, CA_OPT_SF_CHUNKS_PER_TASK, 1) != CA_OK) return 23;
  if (ca_stats(c, &st) != CA_OK || st.sf_chunks_per_task != 1) return 24;
  if (ca_remove(c, 7) != CA_OK || ca_stats(c, &st) != CA_OK || st.live_sequences != 1) return 25;
  ca_destroy(c);
  ca_destroy(NULL);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_cxx(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "chunkattn.h"\nint main(void) { return ca_slot_bytes(1, 128, 64) == 0; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", INCLUDE, "-c", str(src),
                    "-o", str(tmp_path / "h.o")], check=True)
    if shutil.which("g++"):
        subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-x", "c++", "-I", INCLUDE, "-c",
                        str(src), "-o", str(tmp_path / "h2.o")], check=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_drives_a_host_only_context(tmp_path):
    lib = _capi.LIB_PATH
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(lib)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src), "-o", str(exe),
                    "-L", libdir, "-l:" + os.path.basename(lib), "-Wl,-rpath," + libdir], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    lines = res.stdout.splitlines()
    assert lines[0] == "rows 3 seqs 2", res.stdout
    # DFS pre-order: the shared first chunk (64 tokens, both sequences), the
    # shared 6-token head of the split chunk, then its 30-token tail (sequence 7)
    fills = [int(line.split()[4]) for line in lines[1:4]]
    assert fills == [64, 6, 30], res.stdout
    assert lines[4] == f"slot_bytes {4 * 33 * 64 * 128}", res.stdout
    # two sequences, three chunks (two shared), 100 unique tokens, 170 attended
    assert lines[5] == "stats 2 3 2 100 170", res.stdout
