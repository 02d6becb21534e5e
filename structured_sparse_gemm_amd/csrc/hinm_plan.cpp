// Host-only part of libhinm: region counts, status strings, error text.
// Makes no HIP call, so it runs (and is tested) on a host without a GPU.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "hinm_internal.h"

static_assert(sizeof(hinm_plan_t) == 120, "hinm_plan_t must have no padding");

namespace hinm {

static thread_local char g_last_error[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

int check_plan(const hinm_plan_t* p) {
  if (!p) return fail(HINM_EINVAL, "plan is NULL");
  if (p->abi_version != HINM_ABI_VERSION)
    return fail(HINM_EINVAL, "plan has abi_version %d, library is %d", p->abi_version, HINM_ABI_VERSION);
  hinm_plan_t q;
  int st = hinm_plan(p->cout, p->cin, p->tile_rows, p->t_s, p->v_s, &q);
  if (st != HINM_OK) return st;
  if (memcmp(&q, p, sizeof(q)) != 0) return fail(HINM_EINVAL, "plan fields do not match hinm_plan of its arguments");
  return HINM_OK;
}

int check_tplan(const hinm_tplan_t* p) {
  if (!p) return fail(HINM_EINVAL, "plan is NULL");
  if (p->abi_version != HINM_ABI_VERSION)
    return fail(HINM_EINVAL, "plan has abi_version %d, library is %d", p->abi_version, HINM_ABI_VERSION);
  hinm_plan_t q;
  int st = hinm_plan(p->cout, p->cin, p->tile_rows, p->t_s, p->t_s, &q);
  if (st != HINM_OK) return st;
  const int64_t R = p->tile_rows, cin_pad_d = (int64_t)(p->cin + 31) / 32 * 32, cin_pad_s = (int64_t)(p->cin + 63) / 64 * 64;
  bool ok = p->n_tiles == q.n_tiles && p->z == q.z && p->max_n_dense_pad >= 0 && p->max_n_dense_pad <= cin_pad_d &&
            p->max_n_dense_pad % HINM_KB_DENSE == 0 && p->max_n_24_pad >= 0 && p->max_n_24_pad <= cin_pad_s &&
            p->max_n_24_pad % HINM_KB_24 == 0 && p->dense_blocks >= 0 && p->blocks_24 >= 0 &&
            (int64_t)p->dense_blocks <= (int64_t)p->n_tiles * (p->max_n_dense_pad / HINM_KB_DENSE) &&
            (int64_t)p->blocks_24 <= (int64_t)p->n_tiles * (p->max_n_24_pad / HINM_KB_24);
  ok = ok && p->bytes_val_dense == (int64_t)p->dense_blocks * R * 64 && p->bytes_idx_dense == (int64_t)p->dense_blocks * 128 &&
       p->bytes_val_24 == (int64_t)p->blocks_24 * R * 64 && p->bytes_meta_24 == (int64_t)p->blocks_24 * R * 8 &&
       p->bytes_idx_24 == (int64_t)p->blocks_24 * 256 && p->bytes_tiles == (int64_t)p->n_tiles * 16;
  if (!ok) return fail(HINM_EINVAL, "per-tile plan fields are not consistent (use hinm_plan_tiles)");
  return HINM_OK;
}

hinm_plan_t shape_plan(const hinm_tplan_t& p) {
  hinm_plan_t q;
  memset(&q, 0, sizeof(q));
  q.abi_version = p.abi_version;
  q.cout = p.cout;
  q.cin = p.cin;
  q.tile_rows = p.tile_rows;
  q.n_tiles = p.n_tiles;
  q.z = p.z;
  q.n_dense_pad = p.max_n_dense_pad;
  q.n_24_pad = p.max_n_24_pad;
  q.kb_dense = HINM_KB_DENSE;
  q.kb_24 = HINM_KB_24;
  q.t_s = p.t_s;
  q.bytes_val_dense = p.bytes_val_dense;
  q.bytes_idx_dense = p.bytes_idx_dense;
  q.bytes_val_24 = p.bytes_val_24;
  q.bytes_meta_24 = p.bytes_meta_24;
  q.bytes_idx_24 = p.bytes_idx_24;
  return q;
}

// Launch-shape options: process-wide, each read from its environment variable
// once (at the first use of any option), then changed only through
// hinm_set_option.  Atomic, so a setting made in one thread is seen whole by
// a product launched from another.
namespace {
struct OptionDef {
  const char* env;
  int64_t def;
};
constexpr OptionDef kOptionDefs[HINM_OPT_COUNT] = {
    {nullptr, 0},                      // 0: unused
    {"HINM_DECODE_PATH", 0},           // HINM_OPT_DECODE_PATH
    {"HINM_DECODE_WGS", 256},          // HINM_OPT_DECODE_WGS
    {"HINM_PREFILL_NT", 0},            // HINM_OPT_PREFILL_NT
    {"HINM_PREFILL_SPLITS", 0},        // HINM_OPT_PREFILL_SPLITS
    {"HINM_PREFILL_PATH", 0},          // HINM_OPT_PREFILL_PATH
    {"HINM_PREFILL_PER_XCD", 0},       // HINM_OPT_PREFILL_PER_XCD
    {"HINM_PREFILL_TB_GROUP", 0},      // HINM_OPT_PREFILL_TB_GROUP
    {"HINM_PREFILL_STAGGER", 0},       // HINM_OPT_PREFILL_STAGGER
};

bool option_valid(int key, int64_t v) {
  switch (key) {
    case HINM_OPT_DECODE_PATH: return v == 0 || v == 1;
    case HINM_OPT_DECODE_WGS: return v >= 1 && v <= (1 << 20);
    case HINM_OPT_PREFILL_NT: return v == 0 || v == 128 || v == 256;
    case HINM_OPT_PREFILL_SPLITS: return v == 0 || v == 1 || v == 2 || v == 4;
    case HINM_OPT_PREFILL_PATH: return v == 0 || v == 1;
    case HINM_OPT_PREFILL_PER_XCD: return v >= 0 && v <= 1024;
    case HINM_OPT_PREFILL_TB_GROUP: return v >= 0 && v <= 64;
    case HINM_OPT_PREFILL_STAGGER: return v == 0 || v == 1;
    default: return false;
  }
}

// Environment value of an option: the names HINM_DECODE_PATH=rows16 and
// HINM_PREFILL_PATH=staged select 1, other variables hold a number.  An
// unset, unparsable or out-of-range value leaves the default.
int64_t option_from_env(int key) {
  const OptionDef& d = kOptionDefs[key];
  const char* e = getenv(d.env);
  if (!e || !*e) return d.def;
  if (key == HINM_OPT_DECODE_PATH) return strcmp(e, "rows16") == 0 ? 1 : 0;
  if (key == HINM_OPT_PREFILL_PATH) return strcmp(e, "staged") == 0 ? 1 : 0;
  char* end = nullptr;
  const long long v = strtoll(e, &end, 10);
  if (end == e || *end != '\0' || !option_valid(key, v)) return d.def;
  return v;
}

struct Options {
  std::atomic<int64_t> v[HINM_OPT_COUNT];
  Options() {
    for (int k = 0; k < HINM_OPT_COUNT; ++k) v[k].store(k == 0 ? 0 : option_from_env(k), std::memory_order_relaxed);
  }
};

Options& options() {
  static Options o;   // initialised once, thread-safe
  return o;
}
}  // namespace

int64_t option(int key) { return options().v[key].load(std::memory_order_relaxed); }

}  // namespace hinm

using hinm::fail;

extern "C" int hinm_abi_version(void) { return HINM_ABI_VERSION; }

extern "C" int hinm_set_option(int option, int64_t value) {
  hinm::clear_error();
  if (option <= 0 || option >= HINM_OPT_COUNT) return fail(HINM_EINVAL, "unknown option %d", option);
  if (!hinm::option_valid(option, value))
    return fail(HINM_EINVAL, "value %lld is out of range for option %d", (long long)value, option);
  hinm::options().v[option].store(value, std::memory_order_relaxed);
  return HINM_OK;
}

extern "C" int hinm_get_option(int option, int64_t* value) {
  hinm::clear_error();
  if (option <= 0 || option >= HINM_OPT_COUNT) return fail(HINM_EINVAL, "unknown option %d", option);
  if (!value) return fail(HINM_EINVAL, "value is NULL");
  *value = hinm::option(option);
  return HINM_OK;
}

// FlexHiNM-GP notes, key design 1: t_s = v_s + (1 - v_s) p_s / 2.  The counts
// are rounded half-up so that every row keeps exactly cin - z entries:
// n_pruned + n_24 / 2 = z.
extern "C" int hinm_plan(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double v_s,
                         hinm_plan_t* out) {
  hinm::clear_error();
  if (!out) return fail(HINM_EINVAL, "out is NULL");
  if (cout <= 0 || cin <= 0 || tile_rows <= 0)
    return fail(HINM_ESHAPE, "sizes must be positive (cout=%lld cin=%lld tile_rows=%d)",
                (long long)cout, (long long)cin, tile_rows);
  if (cout > INT32_MAX || cin > INT32_MAX) return fail(HINM_ESHAPE, "cout and cin must fit in int32");
  if (tile_rows % 16 != 0) return fail(HINM_ESHAPE, "tile_rows=%d is not a multiple of 16", tile_rows);
  if (cout % tile_rows != 0)
    return fail(HINM_ESHAPE, "cout=%lld is not a multiple of tile_rows=%d", (long long)cout, tile_rows);
  if (cin % 4 != 0) return fail(HINM_ESHAPE, "cin=%lld is not a multiple of 4", (long long)cin);
  if (!isfinite(t_s) || !isfinite(v_s)) return fail(HINM_EINVAL, "t_s and v_s must be finite");
  if (!(t_s >= 0.0 && t_s < 1.0)) return fail(HINM_EINVAL, "t_s=%g is outside [0, 1)", t_s);
  double lo = 2.0 * t_s - 1.0;
  if (lo < 0.0) lo = 0.0;
  if (!(v_s >= lo && v_s <= t_s))
    return fail(HINM_EINVAL, "v_s=%g is outside [max(0, 2 t_s - 1), t_s] = [%g, %g]", v_s, lo, t_s);
  const int64_t z = (int64_t)floor(t_s * (double)cin + 0.5);
  int64_t g = (int64_t)floor((t_s - v_s) * (double)cin / 2.0 + 0.5);
  const int64_t gmax = (z < cin - z ? z : cin - z) / 2;
  if (g < 0) g = 0;
  if (g > gmax) g = gmax;
  hinm_plan_t p;
  memset(&p, 0, sizeof(p));
  p.abi_version = HINM_ABI_VERSION;
  p.cout = (int32_t)cout;
  p.cin = (int32_t)cin;
  p.tile_rows = tile_rows;
  p.n_tiles = (int32_t)(cout / tile_rows);
  p.z = (int32_t)z;
  p.groups = (int32_t)g;
  p.n_24 = (int32_t)(4 * g);
  p.n_pruned = (int32_t)(z - 2 * g);
  p.n_dense = (int32_t)(cin - z - 2 * g);
  p.n_dense_pad = (p.n_dense + HINM_KB_DENSE - 1) / HINM_KB_DENSE * HINM_KB_DENSE;
  p.n_24_pad = (p.n_24 + HINM_KB_24 - 1) / HINM_KB_24 * HINM_KB_24;
  p.kb_dense = HINM_KB_DENSE;
  p.kb_24 = HINM_KB_24;
  p.t_s = t_s;
  p.v_s = v_s;
  p.p_s = 2.0 * (t_s - v_s) / (1.0 - v_s);
  const int64_t T = p.n_tiles, R = tile_rows;
  p.bytes_val_dense = T * p.n_dense_pad * R * 2;
  p.bytes_idx_dense = T * p.n_dense_pad * 4;
  p.bytes_val_24 = T * (p.n_24_pad / 2) * R * 2;
  p.bytes_meta_24 = T * (p.n_24_pad / HINM_KB_24) * R * 8;
  p.bytes_idx_24 = T * p.n_24_pad * 4;
  *out = p;
  return HINM_OK;
}

extern "C" const char* hinm_status_str(int status) {
  switch (status) {
    case HINM_OK: return "HINM_OK";
    case HINM_EINVAL: return "HINM_EINVAL: invalid argument";
    case HINM_ESHAPE: return "HINM_ESHAPE: unsupported or inconsistent sizes";
    case HINM_EPERM: return "HINM_EPERM: perm row is not a permutation";
    case HINM_EIMPORTANCE: return "HINM_EIMPORTANCE: importance is negative or not finite";
    case HINM_EALIGN: return "HINM_EALIGN: pointer misaligned";
    case HINM_EWORKSPACE: return "HINM_EWORKSPACE: workspace missing or too small";
    case HINM_EHIP: return "HINM_EHIP: HIP runtime error";
    case HINM_EDEVICE: return "HINM_EDEVICE: no usable device";
    default: return "HINM_E?: unknown status";
  }
}

extern "C" const char* hinm_last_error(void) { return hinm::g_last_error; }

// Work decomposition of the product.
//  - batch <= 64 and tile_rows % 64 == 0: the split decode kernel (64-row
//    workgroups, K split over a power-of-two number of workgroups, partial
//    sums through the workspace);
//  - other batch <= 64: the 16-row decode kernel (K split over the waves of
//    a workgroup, no workspace);
//  - larger batches with tile_rows % 64 == 0: the prefill kernel (64-row x
//    128/256-token items on a persistent grid; with fewer items than the grid
//    holds, each item's K range is split over 2 or 4 workgroups and the
//    partial sums go through the workspace);
//  - otherwise the generic kernel, which splits K over workgroups when there
//    are too few of them and reduces the partials through the workspace.
namespace hinm {
SpmmShape spmm_shape(const hinm_plan_t* p, int64_t batch) {
  SpmmShape s;
  s.n_rblocks = (p->tile_rows + 63) / 64;
  s.n_kunits = p->n_dense_pad / HINM_KB_DENSE + 2 * (p->n_24_pad / HINM_KB_24);
  s.splits = 1;
  s.split_rows = 0;
  s.split_mix = false;
  s.two_per_cu = false;
  s.ws_bytes = 0;
  s.ws_counter_bytes = 0;
  if (batch <= 64) {
    s.nt = batch <= 16 ? 16 : (batch <= 32 ? 32 : 64);
    s.n_tblocks = (int)((batch + s.nt - 1) / s.nt);
    if (p->tile_rows % 64 == 0 && option(HINM_OPT_DECODE_PATH) == 0) {
      // 64-row workgroups, K split over a power-of-two number of workgroups
      // so that about `target` workgroups run, each with >= 4 K-blocks.
      s.path = kPathDecodeSplit;
      const int64_t base = (int64_t)p->n_tiles * (p->tile_rows / 64) * s.n_tblocks;
      const int nblk = p->n_dense_pad / HINM_KB_DENSE + p->n_24_pad / HINM_KB_24;
      const int64_t target = option(HINM_OPT_DECODE_WGS);
      int splits = 1;
      if (base <= kWsCounters)
        while (splits < 64 && base * splits * 2 <= target && nblk / (splits * 2) >= 4) splits *= 2;
      s.splits = splits;
      s.split_rows = (int64_t)p->n_tiles * (p->tile_rows / 64);
      // At 16 tokens two workgroups share a compute unit, so 512 run at
      // once; at 32 tokens too when the launch has more than 256 (the
      // kernel then takes smaller rounds).  When base x splits workgroups
      // leave some units with two whole ranges and others with one (gate
      // and up together: 344 row blocks), the last row blocks take twice
      // the splits, so that exactly 512 run: the first slots hold the whole
      // ranges, the second slots the halves, and no unit holds more than
      // one and a half ranges.  At 64 tokens (one workgroup per unit) the
      // same split turns the second round of whole ranges into halves that
      // start as the first round's halves finish.
      s.two_per_cu = s.nt == 16 || (s.nt == 32 && base * splits > 256);
      const int64_t slots = 512;
      int splits_hi = splits;
      if (s.n_tblocks == 1 && option(HINM_OPT_DECODE_WGS) == 256 && base * splits < slots &&
          base * splits * 2 > slots && slots % splits == 0 && nblk / (splits * 2) >= 4 && base <= kWsCounters) {
        s.split_rows = 2 * base - slots / splits;
        splits_hi = 2 * splits;
      }
      if (splits_hi > 1) {
        s.ws_counter_bytes = kWsCounterBytes;
        s.ws_bytes = kWsCounterBytes + (int64_t)splits_hi * s.n_tblocks * p->cout * s.nt * 4;
      }
      return s;
    }
    s.path = kPathDecode;
    return s;
  }
  if (p->tile_rows % 64 == 0) {
    s.path = kPathPrefill;
    const int64_t rblocks = (int64_t)p->n_tiles * (p->tile_rows / 64);
    const int nblk = p->n_dense_pad / HINM_KB_DENSE + p->n_24_pad / HINM_KB_24;
    const int kunits = p->n_dense_pad / HINM_KB_DENSE + 2 * (p->n_24_pad / HINM_KB_24);
    const int64_t per_xcd_max = option(HINM_OPT_PREFILL_PER_XCD) > 0 ? option(HINM_OPT_PREFILL_PER_XCD) : 64;
    // At most half as many work items as compute units: split each item's K
    // range over 2 or 4 workgroups (at most 512 in all, two per compute unit;
    // each keeps >= 8 K-blocks); partial sums through the workspace.  With
    // more items a split cannot take work off the busiest compute units (172
    // items split 2 ways still put two half items on some of them), and its
    // partials only add traffic: up_proj (172 row blocks) at batch 65-128
    // ran 2-9% faster unsplit; with the weight streamed from HBM, 2 splits at
    // 256 items were slower too.
    auto split_of = [&](int64_t items) {
      int sp = 1;
      if (option(HINM_OPT_PREFILL_SPLITS) != 0) {
        sp = (int)option(HINM_OPT_PREFILL_SPLITS);
      } else if (items <= 128) {
        while (sp < 4 && items * sp * 2 <= 512 && nblk / (sp * 2) >= 8) sp *= 2;
      } else if (items * 2 > 448 && items * 2 <= 512 && kunits >= 120 && nblk / 2 >= 8) {
        // Nearly one item per compute unit on a long K range (down_proj at
        // batch 1024: 256 items of 256 tokens): one workgroup alone on a unit
        // hides its latencies poorly, and two halves per unit pay for their
        // partial sums (65.8 -> 60.8 us); with shorter K ranges (q_proj,
        // up_proj) or fewer items (192: some units would hold two halves and
        // others one) the split is slower.
        sp = 2;
      }
      return sp;
    };
    // Rounds of the persistent grid (8 XCDs x up to per_xcd workgroups) and
    // its size for a token block of nt.
    auto grid_of = [&](int nt, int64_t* rounds, int64_t* nwg) {
      const int64_t wi = rblocks * ((batch + nt - 1) / nt) * split_of(rblocks * ((batch + nt - 1) / nt));
      const int64_t per_xcd = std::min(per_xcd_max, (wi + 7) / 8);
      *rounds = ((wi + 7) / 8 + per_xcd - 1) / per_xcd;
      *nwg = 8 * per_xcd;
    };
    // Token block: 256 from batch 1024; from 256 to 1023 tokens, 256 when it
    // takes fewer rounds of the grid, or as many rounds and at least as many
    // workgroups with a long K range (>= 120 units, a 2:4 block counting two);
    // else 128 (measured over batches 256-896 on 4096x11008, 4096x4096 and
    // 11008x4096 weights).
    s.nt = batch >= 1024 ? 256 : 128;
    if (batch >= 256 && batch < 1024) {
      int64_t r128, w128, r256, w256;
      grid_of(128, &r128, &w128);
      grid_of(256, &r256, &w256);
      if (r256 < r128 || (r256 == r128 && kunits >= 120 && w256 >= w128)) s.nt = 256;
    }
    if (option(HINM_OPT_PREFILL_NT) != 0) s.nt = (int)option(HINM_OPT_PREFILL_NT);
    s.n_tblocks = (int)((batch + s.nt - 1) / s.nt);
    const int64_t items = rblocks * s.n_tblocks;
    const int splits = split_of(items);
    if (splits > 1 && items <= kWsCounters) {
      s.splits = splits;
      s.ws_counter_bytes = kWsCounterBytes;
      s.ws_bytes = kWsCounterBytes + (int64_t)splits * items * 256 * s.nt;   // 256 threads x NT/4 floats
    } else if (splits == 1 && s.nt == 128 && s.n_tblocks >= 2 && items > 256 && items < 512 &&
               per_xcd_max == 64 && option(HINM_OPT_PREFILL_SPLITS) == 0 && items <= kWsCounters) {
      // Between 256 and 512 items the grid's 512 workgroups would leave some
      // compute units with two items and others with one (q, k and v
      // together at batch 129-256: 384; up_proj: 344).  On each XCD the
      // first items run whole and the rest in two K halves, one piece a
      // workgroup, so that a unit holds at most an item and a half; partial
      // sums only for the halved items, and only while they fit the
      // allocation-free product's scratch, so that both entry points always
      // run the same schedule.  Only with 128-token items in two or more
      // token blocks: with 256-token items the partial sums cost more than
      // the balance gains (2% slower for gate/up at batch 256 and up_proj at
      // 512), and with one token block the 7B-shaped stack at batch 128 ran
      // 1% slower although gate/up alone ran 1% faster.
      int64_t n_half = 0;
      for (int x = 0; x < 8; ++x) {
        const int64_t nx = (x + 1) * items / 8 - x * items / 8;
        n_half += nx - std::min(nx, std::max<int64_t>(0, 2 * nx - 64));
      }
      const int64_t ws = kWsCounterBytes + 2 * n_half * 256 * s.nt;
      if (ws <= (int64_t)HINM_NOALLOC_SCRATCH_BYTES) {
        s.splits = 2;
        s.split_mix = true;
        s.ws_counter_bytes = kWsCounterBytes;
        s.ws_bytes = ws;
      }
    }
    return s;
  }
  s.path = kPathGeneric;
  s.nt = 64;
  s.n_tblocks = (int)((batch + s.nt - 1) / s.nt);
  const int64_t wgs = (int64_t)p->n_tiles * s.n_rblocks * s.n_tblocks;
  const int64_t target = 1024;  // about four workgroups per compute unit
  if (wgs < target && s.n_kunits > 1) {
    int splits = (int)((target + wgs - 1) / wgs);
    int max_splits = s.n_kunits / 4;  // keep at least ~4 K units per split
    if (max_splits < 1) max_splits = 1;
    if (splits > max_splits) splits = max_splits;
    if (splits > 32) splits = 32;
    s.splits = splits;
  }
  if (s.splits > 1) {
    s.ws_counter_bytes = kWsCounterBytes;
    s.ws_bytes = kWsCounterBytes + (int64_t)s.splits * p->cout * ((batch + 15) / 16 * 16) * 4;
  }
  return s;
}
}  // namespace hinm

extern "C" int hinm_pack_workspace_bytes(const hinm_plan_t* plan, size_t* bytes) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  const size_t tc = (size_t)plan->n_tiles * plan->cin;
  // [flag 256 B][scores fp64 T*cin][regions u8 T*cin, rounded to 256]
  *bytes = 256 + tc * 8 + (tc + 255) / 256 * 256;
  return HINM_OK;
}

extern "C" int hinm_spmm_workspace_bytes(const hinm_plan_t* plan, int64_t batch, size_t* bytes) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  if (batch < 0) return fail(HINM_ESHAPE, "batch=%lld is negative", (long long)batch);
  *bytes = batch == 0 ? 0 : (size_t)hinm::spmm_shape(plan, batch).ws_bytes;
  return HINM_OK;
}

// Per-tile counts (FlexHiNM-GP notes, "整体框架": region ratios decided in
// each tile): tile t gets the counts of hinm_plan at (t_s, v_s[t]); the
// tiles' K-blocks are laid end to end.
extern "C" int hinm_plan_tiles(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, const double* v_s,
                               hinm_tplan_t* out, int32_t* tiles) {
  hinm::clear_error();
  if (!v_s || !out || !tiles) return fail(HINM_EINVAL, "v_s, out and tiles_out must be non-NULL");
  hinm_plan_t p0;
  int st = hinm_plan(cout, cin, tile_rows, t_s, t_s, &p0);
  if (st) return st;
  int64_t kd = 0, ks = 0;
  int32_t maxd = 0, maxs = 0;
  for (int t = 0; t < p0.n_tiles; ++t) {
    hinm_plan_t pt;
    st = hinm_plan(cout, cin, tile_rows, t_s, v_s[t], &pt);
    if (st) {
      char msg[256];
      snprintf(msg, sizeof(msg), "%s", hinm_last_error());
      return fail(st, "tile %d: %s", t, msg);
    }
    tiles[4 * t + 0] = (int32_t)kd;
    tiles[4 * t + 1] = pt.n_dense;
    tiles[4 * t + 2] = (int32_t)ks;
    tiles[4 * t + 3] = pt.n_24;
    kd += pt.n_dense_pad / HINM_KB_DENSE;
    ks += pt.n_24_pad / HINM_KB_24;
    maxd = pt.n_dense_pad > maxd ? pt.n_dense_pad : maxd;
    maxs = pt.n_24_pad > maxs ? pt.n_24_pad : maxs;
    if (kd > INT32_MAX || ks > INT32_MAX) return fail(HINM_ESHAPE, "too many K-blocks");
  }
  hinm_tplan_t& o = *out;
  memset(&o, 0, sizeof(o));
  o.abi_version = HINM_ABI_VERSION;
  o.cout = p0.cout;
  o.cin = p0.cin;
  o.tile_rows = p0.tile_rows;
  o.n_tiles = p0.n_tiles;
  o.z = p0.z;
  o.max_n_dense_pad = maxd;
  o.max_n_24_pad = maxs;
  o.dense_blocks = (int32_t)kd;
  o.blocks_24 = (int32_t)ks;
  o.t_s = t_s;
  const int64_t R = p0.tile_rows;
  o.bytes_val_dense = kd * R * 64;
  o.bytes_idx_dense = kd * 128;
  o.bytes_val_24 = ks * R * 64;
  o.bytes_meta_24 = ks * R * 8;
  o.bytes_idx_24 = ks * 256;
  o.bytes_tiles = (int64_t)p0.n_tiles * 16;
  return HINM_OK;
}

extern "C" int hinm_pack_tiles_workspace_bytes(const hinm_tplan_t* plan, size_t* bytes) {
  hinm::clear_error();
  int st = hinm::check_tplan(plan);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  const size_t tc = (size_t)plan->n_tiles * plan->cin;
  *bytes = 256 + tc * 8 + (tc + 255) / 256 * 256;
  return HINM_OK;
}

extern "C" int hinm_spmm_tiles_workspace_bytes(const hinm_tplan_t* plan, int64_t batch, size_t* bytes) {
  hinm::clear_error();
  int st = hinm::check_tplan(plan);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  if (batch < 0) return fail(HINM_ESHAPE, "batch=%lld is negative", (long long)batch);
  const hinm_plan_t q = hinm::shape_plan(*plan);
  *bytes = batch == 0 ? 0 : (size_t)hinm::spmm_shape(&q, batch).ws_bytes;
  return HINM_OK;
}
