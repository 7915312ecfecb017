/*
 * fa_check_harness.c - drives the host validation unit (fa_check.c) from a
 * table on stdin, one call per line, and prints each returned status.  Built
 * by tests/test_sanitizers.py with gcc and -fsanitize=address,undefined so
 * that every argument table of the boundary tests also runs under the host
 * sanitizers (signed overflow, out-of-bounds access, misaligned loads...).
 *
 * Line formats (pointers are plain integers, never dereferenced; the scale is
 * a C99 hexadecimal float so that it crosses the text exactly):
 *   F q k v o lse B H M N D scale causal dtype
 *   B q k v o lse dout dq dk dv delta B H M N D scale causal dtype
 *   S q k v o lse B H M N D scale causal dtype splits ws ws_bytes
 */
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

static void* P(const char* s) { return (void*)(uintptr_t)strtoull(s, NULL, 0); }
static int64_t I(const char* s) { return (int64_t)strtoll(s, NULL, 0); }

int main(void) {
  char line[1024];
  while (fgets(line, sizeof line, stdin)) {
    char* tok[32];
    int n = 0;
    for (char* t = strtok(line, " \t\r\n"); t && n < 32; t = strtok(NULL, " \t\r\n")) tok[n++] = t;
    if (n == 0) continue;
    int st = -1;
    if (tok[0][0] == 'F' && n == 14) {
      st = fa_check_args(P(tok[1]), P(tok[2]), P(tok[3]), P(tok[4]), P(tok[5]), I(tok[6]),
                         I(tok[7]), I(tok[8]), I(tok[9]), I(tok[10]), strtof(tok[11], NULL),
                         (int)I(tok[12]), (int)I(tok[13]));
    } else if (tok[0][0] == 'B' && n == 19) {
      st = fa_bwd_check_args(P(tok[1]), P(tok[2]), P(tok[3]), P(tok[4]), P(tok[5]), P(tok[6]),
                             P(tok[7]), P(tok[8]), P(tok[9]), P(tok[10]), I(tok[11]), I(tok[12]),
                             I(tok[13]), I(tok[14]), I(tok[15]), strtof(tok[16], NULL),
                             (int)I(tok[17]), (int)I(tok[18]));
    } else if (tok[0][0] == 'S' && n == 17) {
      st = fa_splitkv_check_args(P(tok[1]), P(tok[2]), P(tok[3]), P(tok[4]), P(tok[5]), I(tok[6]),
                                 I(tok[7]), I(tok[8]), I(tok[9]), I(tok[10]),
                                 strtof(tok[11], NULL), (int)I(tok[12]), (int)I(tok[13]),
                                 (int)I(tok[14]), P(tok[15]), I(tok[16]));
    } else {
      fprintf(stderr, "bad line with %d fields\n", n);
      return 2;
    }
    printf("%d %s\n", st, fa_status_string(st));
  }
  return 0;
}
