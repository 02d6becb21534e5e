// Host-only driver for the sanitizer build of libhinm's host code
// (hinm_plan.cpp): region counts, per-tile plans, workspace sizes, launch
// options and status strings over many random and malformed arguments.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitize.py; any sanitizer report aborts the run, and every
// invariant below that fails makes the exit status non-zero.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "hinm.h"

static int g_failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                     \
    }                                                                   \
  } while (0)

// Region-count invariants of a plan (FlexHiNM-GP notes, key design 1):
// every row keeps cin - z entries, n_pruned + n_24 / 2 = z.
static void check_counts(const hinm_plan_t& p) {
  CHECK(p.n_dense >= 0 && p.n_24 >= 0 && p.n_pruned >= 0);
  CHECK(p.n_dense + p.n_24 + p.n_pruned == p.cin);
  CHECK(2 * p.z == 2 * p.n_pruned + p.n_24);
  CHECK(p.n_24 % 4 == 0 && p.groups * 4 == p.n_24);
  CHECK(p.n_dense_pad % HINM_KB_DENSE == 0 && p.n_dense_pad >= p.n_dense && p.n_dense_pad - p.n_dense < HINM_KB_DENSE);
  CHECK(p.n_24_pad % HINM_KB_24 == 0 && p.n_24_pad >= p.n_24 && p.n_24_pad - p.n_24 < HINM_KB_24);
  CHECK(p.n_tiles * p.tile_rows == p.cout);
  CHECK(p.bytes_val_dense == (int64_t)p.n_tiles * p.n_dense_pad * p.tile_rows * 2);
  CHECK(p.bytes_val_24 == (int64_t)p.n_tiles * (p.n_24_pad / 2) * p.tile_rows * 2);
  CHECK(p.bytes_meta_24 == (int64_t)p.n_tiles * (p.n_24_pad / 64) * p.tile_rows * 8);
}

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](double a, double b) { return std::uniform_real_distribution<double>(a, b)(rng); };
  auto pick = [&](int64_t a, int64_t b) { return std::uniform_int_distribution<int64_t>(a, b)(rng); };

  // hinm_plan on valid and malformed arguments.
  int ok_plans = 0;
  for (int i = 0; i < 20000; ++i) {
    const int32_t R = (int32_t)(16 * pick(-1, 8));
    const int64_t cout = (int64_t)R * pick(-1, 40) + (pick(0, 9) == 0 ? pick(-3, 3) : 0);
    const int64_t cin = 4 * pick(-2, 3000) + (pick(0, 9) == 0 ? pick(-3, 3) : 0);
    double t = uni(-0.1, 1.05), v = uni(-0.1, 1.05);
    if (pick(0, 19) == 0) t = NAN;
    if (pick(0, 19) == 0) v = INFINITY;
    if (pick(0, 3) == 0) v = uni(fmax(0.0, 2 * t - 1), t);
    hinm_plan_t p;
    memset(&p, 0xab, sizeof(p));
    const int st = hinm_plan(cout, cin, R, t, v, &p);
    CHECK(hinm_status_str(st) != nullptr && hinm_last_error() != nullptr);
    if (st == HINM_OK) {
      ++ok_plans;
      check_counts(p);
      size_t ws = 0;
      CHECK(hinm_pack_workspace_bytes(&p, &ws) == HINM_OK && ws > 0);
      for (int b = 0; b < 8; ++b) {
        const int64_t batch = pick(0, 5000);
        size_t sw = 1;
        CHECK(hinm_spmm_workspace_bytes(&p, batch, &sw) == HINM_OK);
        CHECK(batch != 0 || sw == 0);
      }
      CHECK(hinm_spmm_workspace_bytes(&p, -1, nullptr) != HINM_OK);
      // a plan whose fields do not match its arguments is refused
      hinm_plan_t q = p;
      q.n_dense += 1;
      size_t sq = 0;
      CHECK(hinm_spmm_workspace_bytes(&q, 16, &sq) == HINM_EINVAL);
      q = p;
      q.abi_version = HINM_ABI_VERSION + 1;
      CHECK(hinm_pack_workspace_bytes(&q, &sq) == HINM_EINVAL);
    } else {
      CHECK(strlen(hinm_last_error()) > 0);
    }
  }
  CHECK(ok_plans > 1000);
  CHECK(hinm_plan(64, 64, 16, 0.5, 0.25, nullptr) == HINM_EINVAL);
  CHECK(hinm_spmm_workspace_bytes(nullptr, 16, nullptr) == HINM_EINVAL);

  // Per-tile plans: the tile table lays the tiles' K-blocks end to end.
  for (int i = 0; i < 2000; ++i) {
    const int32_t R = (int32_t)(16 * pick(1, 8));
    const int64_t T = pick(1, 24), cout = R * T, cin = 4 * pick(1, 1500);
    const double t = uni(0.0, 0.95);
    std::vector<double> v(T);
    for (auto& x : v) x = uni(fmax(0.0, 2 * t - 1), t);
    if (pick(0, 9) == 0) v[pick(0, T - 1)] = t + 0.5;   // out of range in one tile
    hinm_tplan_t tp;
    std::vector<int32_t> tiles(4 * T, -7);
    const int st = hinm_plan_tiles(cout, cin, R, t, v.data(), &tp, tiles.data());
    if (st != HINM_OK) continue;
    int64_t kd = 0, ks = 0;
    for (int64_t k = 0; k < T; ++k) {
      hinm_plan_t pk;
      CHECK(hinm_plan(cout, cin, R, t, v[k], &pk) == HINM_OK);
      CHECK(tiles[4 * k] == kd && tiles[4 * k + 1] == pk.n_dense);
      CHECK(tiles[4 * k + 2] == ks && tiles[4 * k + 3] == pk.n_24);
      kd += pk.n_dense_pad / HINM_KB_DENSE;
      ks += pk.n_24_pad / HINM_KB_24;
    }
    CHECK(tp.dense_blocks == kd && tp.blocks_24 == ks);
    size_t a = 0, b = 0;
    CHECK(hinm_pack_tiles_workspace_bytes(&tp, &a) == HINM_OK && a > 0);
    CHECK(hinm_spmm_tiles_workspace_bytes(&tp, pick(1, 4096), &b) == HINM_OK);
  }

  // Launch options: set, read back, refuse unknown keys and values out of range.
  for (int k = HINM_OPT_DECODE_PATH; k < HINM_OPT_COUNT; ++k) {
    int64_t before = -1, after = -1;
    CHECK(hinm_get_option(k, &before) == HINM_OK);
    CHECK(hinm_set_option(k, -5) == HINM_EINVAL);
    CHECK(hinm_get_option(k, &after) == HINM_OK && after == before);
    CHECK(hinm_set_option(k, before) == HINM_OK);
  }
  CHECK(hinm_set_option(0, 1) == HINM_EINVAL && hinm_set_option(HINM_OPT_COUNT, 1) == HINM_EINVAL);
  CHECK(hinm_get_option(HINM_OPT_DECODE_WGS, nullptr) == HINM_EINVAL);
  CHECK(hinm_set_option(HINM_OPT_PREFILL_SPLITS, 3) == HINM_EINVAL);
  CHECK(hinm_set_option(HINM_OPT_PREFILL_SPLITS, 4) == HINM_OK);
  CHECK(hinm_set_option(HINM_OPT_PREFILL_SPLITS, 0) == HINM_OK);

  for (int s = -2; s < 12; ++s) CHECK(hinm_status_str(s) != nullptr && strlen(hinm_status_str(s)) > 0);
  CHECK(hinm_abi_version() == HINM_ABI_VERSION);

  if (g_failures) {
    fprintf(stderr, "%d checks failed\n", g_failures);
    return 1;
  }
  printf("host sanitizer driver: %d valid plans, all checks passed\n", ok_plans);
  return 0;
}
