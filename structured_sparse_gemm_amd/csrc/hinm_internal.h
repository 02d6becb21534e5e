// Internal helpers shared by the translation units of libhinm (not installed).
#ifndef HINM_INTERNAL_H_
#define HINM_INTERNAL_H_

#include <stdarg.h>
#include <stdint.h>

#include "hinm.h"

namespace hinm {

// Records a printf-style message for hinm_last_error() in this thread and
// returns `status`, so call sites read `return fail(HINM_ESHAPE, "...")`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Host-side validation of a plan handed back by a caller.
int check_plan(const hinm_plan_t* p);
// The same for a per-tile plan (its shared fields and buffer sizes; the
// tile table itself lives on the device).
int check_tplan(const hinm_tplan_t* p);
// A hinm_plan_t carrying a per-tile plan's shape (largest per-tile pads), for
// the launch-shape logic shared with the uniform layout.
hinm_plan_t shape_plan(const hinm_tplan_t& p);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Split of the reduction dimension chosen for a batch (1 = no split) and the
// token-block width; shared by hinm_spmm and hinm_spmm_workspace_bytes so the
// workspace size always matches what the launch uses.
// Every workspace starts with a fixed region of arrival counters, kept at
// zero between calls; partial sums start after it, so products of different
// shapes can share one workspace.
constexpr int64_t kWsCounters = 16384;
constexpr int64_t kWsCounterBytes = kWsCounters * 4;

enum { kPathGeneric = 0, kPathDecode = 1, kPathPrefill = 2, kPathDecodeSplit = 3 };
struct SpmmShape {
  int path;        // which kernel runs the product
  int nt;          // tokens per workgroup
  int n_tblocks;   // token blocks
  int n_rblocks;   // 64-row blocks per tile
  int n_kunits;    // K work units per tile (dense block = 1, 2:4 block = 2)
  int splits;      // K splits (>= 1)
  int64_t split_rows;  // split decode: row blocks with `splits` workgroups; the rest have 2 x splits
  bool split_mix;      // prefill: two split counts (items whole or in two K halves, one piece a workgroup)
  bool two_per_cu;     // split decode: two workgroups share a compute unit (16 tokens always; 32 tokens
                       // with the smaller rounds, used when the launch has more than 256 workgroups)
  int64_t ws_counter_bytes;  // arrival counters at the start of the workspace (split decode)
  int64_t ws_bytes;
};
SpmmShape spmm_shape(const hinm_plan_t* p, int64_t batch);

// Current value of a launch-shape option (HINM_OPT_*).
int64_t option(int key);

// Current device is a gfx950 part (checked once per device); HINM_OK or
// HINM_EDEVICE / HINM_EHIP with the message recorded.
int ensure_device();

}  // namespace hinm

#ifdef __HIP__
#include <hip/hip_runtime.h>
namespace hinm {
// The perm and importance checks, scores, regions and index lists of a pack
// (its first stages) into caller buffers; ws is laid out as the pack
// workspace (hinm_pack_workspace_bytes).  Synchronous.
int region_lists(const hinm_plan_t& p, const float* importance, int64_t ldi, const int32_t* perm, int32_t* idx_dense,
                 int32_t* idx_24, void* ws, hipStream_t stream);
}  // namespace hinm
#endif

#endif  // HINM_INTERNAL_H_
