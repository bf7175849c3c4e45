/* Calls libvsa.so from plain C99 through include/vsa.h alone: the ABI
 * version, the host helpers (token order and cube table, both cube orders)
 * and argument checks that return before any device work.  Prints one line
 * per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vsa.h"

#define CHECK(cond, what)                         \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "FAIL: %s\n", what);        \
      return 1;                                   \
    }                                             \
    printf("ok: %s\n", what);                     \
  } while (0)

int main(void) {
  CHECK((vsa_abi_version() >> 16) == 3, "ABI major version 3");
  CHECK(strcmp(vsa_status_str(VSA_OK), "ok") == 0, "status string of VSA_OK");

  vsa_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1; p.heads = 2; p.T = 5; p.H = 6; p.W = 7;
  p.ct = 2; p.ch = 2; p.cw = 2; p.head_dim = 64;
  /* cube grid 3 x 3 x 4 = 36 cubes of 8 positions, padded from 210 tokens */
  int32_t perm[36 * 8];
  CHECK(vsa_perm_index(&p, perm) == VSA_OK, "raster token order");
  int seen[210];
  memset(seen, 0, sizeof seen);
  int pad = 0;
  for (int i = 0; i < 36 * 8; ++i) {
    if (perm[i] < 0) { ++pad; continue; }
    if (perm[i] >= 210 || seen[perm[i]]++) { fprintf(stderr, "FAIL: not a bijection at %d\n", i); return 1; }
  }
  CHECK(pad == 36 * 8 - 210, "every token once, the rest padding");

  p.cube_order = VSA_CUBES_HILBERT;
  int32_t table[36];
  CHECK(vsa_cube_table(&p, table) == VSA_OK, "Hilbert cube table");
  int cells[36];
  memset(cells, 0, sizeof cells);
  for (int c = 0; c < 36; ++c) {
    const int t = (table[c] >> 20) & 1023, h = (table[c] >> 10) & 1023, w = table[c] & 1023;
    if (t >= 3 || h >= 3 || w >= 4 || cells[(t * 3 + h) * 4 + w]++) {
      fprintf(stderr, "FAIL: cube table entry %d\n", c);
      return 1;
    }
  }
  CHECK(table[0] == 0, "curve starts at the origin cube");
  CHECK(vsa_perm_index(&p, perm) == VSA_OK, "Hilbert token order");
  /* a compute entry point with the Hilbert order needs the device table */
  CHECK(vsa_permute(&p, VSA_BF16, (const void*)16, (void*)16, NULL) == VSA_ERR_NULL,
        "Hilbert order without cube_coords is refused");
  p.cube_order = 7;
  CHECK(vsa_perm_index(&p, perm) == VSA_ERR_UNSUPPORTED, "unknown cube order");
  p.cube_order = VSA_CUBES_RASTER;
  p.head_dim_v = 96;
  CHECK(vsa_perm_index(&p, perm) == VSA_ERR_UNSUPPORTED, "value head size 96");
  p.head_dim_v = 0;
  p.T = 0;
  CHECK(vsa_perm_index(&p, perm) == VSA_ERR_SHAPE, "empty grid");
  CHECK(vsa_perm_index(NULL, perm) == VSA_ERR_NULL, "no problem");
  return 0;
}
