// Host-side checks of the reorder kernels' index arithmetic, run on the CPU:
//  * the span-row division by multiplication (make_reorder's magic): exact for
//    every spans-per-row value and every span index a tensor can have;
//  * the staged unit rule (stage_rows_for): whole tiles, within the largest
//    unit, the fewest rows holding at least 8192 elements, and the LDS a
//    staged launch asks for stays within the CU's 160 KiB.
// Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>

#include "taco_internal.h"

using namespace taco;

static int failures = 0;
static void fail(const char* what, long long a, long long b) {
  if (failures < 20) fprintf(stderr, "%s (%lld, %lld)\n", what, a, b);
  ++failures;
}

int main() {
  // Span index s < 2^26: a call takes at most 2^35 elements, 2^26 spans of 512.
  const uint64_t kSpans = uint64_t(1) << 26;
  long long checked = 0;
  for (int64_t cols = 512; cols <= kReorderMaxCols; cols += 512) {
    int32_t dummy = 0;
    const ReorderArgs ro = make_reorder(&dummy, cols);
    const uint64_t d = ro.spans_per_row;
    if (d != (uint64_t)(cols / 512) || ro.ngroups != cols / 8 || ro.cols != cols) fail("make_reorder fields", cols, d);
    auto check = [&](uint64_t s) {
      const uint64_t row = (s * ro.magic) >> 38;
      if (row != s / d) fail("span row", (long long)s, (long long)d);
      ++checked;
    };
    // every span index below 2^16 and in the top 2^16 (largest error), and
    // the two sides of every multiple of d in between, sampled
    for (uint64_t s = 0; s < 65536; ++s) check(s);
    for (uint64_t s = kSpans - 65536; s < kSpans; ++s) check(s);
    const uint64_t step = d * 977;
    for (uint64_t k = d; k < kSpans; k += step) {
      check(k - 1);
      check(k);
    }
  }

  // staged units
  const int aligns[] = {512, 1024};
  for (int align : aligns) {
    for (int64_t cols = 512; cols <= kReorderMaxCols; cols += 512) {
      const int r = stage_rows_for(cols, align);
      // the fewest rows of whole tiles within the largest unit, preferring
      // units of at least 8192 elements
      int want = 0, first = 0;
      for (int64_t q = 1; q * cols <= kStageMaxElems; ++q) {
        if ((q * cols) % align != 0) continue;
        if (first == 0) first = (int)q;
        if (q * cols >= 8192) {
          want = (int)q;
          break;
        }
      }
      if (want == 0) want = first;
      if (r != want) fail("stage_rows_for", cols, r);
      if (r > 0) {
        if (r * cols > kStageMaxElems || (r * cols) % align != 0) fail("unit size", cols, r);
        ReorderArgs ro{};
        ro.ngroups = (int)(cols / 8);
        const int64_t lds = (int64_t)reorder_stage_offset(ro) * 2 + (int64_t)r * cols * 4;   // float32 decode
        if (lds > 160 * 1024) fail("staged LDS", cols, lds);
        if ((reorder_stage_offset(ro) * 2) % 16 != 0) fail("staged rows alignment", cols, reorder_stage_offset(ro));
      } else if (cols <= kStageMaxElems && cols % align == 0) {
        fail("a row of whole tiles not staged", cols, align);
      }
    }
  }
  // widths the kernels' tests rely on
  if (stage_rows_for(5120, 1024) != 2 || stage_rows_for(8192, 1024) != 1 || stage_rows_for(9728, 1024) != 0 ||
      stage_rows_for(9728, 512) != 1 || stage_rows_for(512, 512) != 16 || stage_rows_for(1536, 1024) != 6 ||
      stage_rows_for(16384, 1024) != 1 || stage_rows_for(16896, 512) != 0)
    fail("named widths", 0, 0);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host_helpers: %lld span rows and every staged width checked\n", checked);
  return 0;
}
