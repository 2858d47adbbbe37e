// attn_window.h -- host-side normalisation of sliding-window edges (plain
// C++, no device code, so that it can be checked on its own).
//
// A window keeps key j for a query at position p when p - left <= j <=
// p + right, -1 leaving a side unbounded (page "Attention Kernel", section
// "可编程 mask": a window is an element rule).  The kernels take the edges in
// int32 and add them to positions, so an edge that excludes no key is turned
// into -1 before any launch.
#pragma once
#include <climits>

namespace attn {

// Edges as the kernels take them.  has_window = false means no window
// (both sides unbounded).  key_extent: every position is below it; row_extent:
// every position is at least key_extent - row_extent (bottom-right alignment).
// Dense calls pass (S_k, S_q); packed calls the longest sequence for both.
//   left  >= key_extent : p - left < 0 for every p, so the left edge keeps all;
//   right >= row_extent : p + right >= key_extent - 1 for every p.
// causal makes the right edge min(right, 0), which is 0 for every valid
// right (>= -1).
inline void window_edges(bool has_window, int in_left, int in_right, int causal, long long key_extent,
                         long long row_extent, int& left, int& right) {
  left = has_window ? in_left : -1;
  right = has_window ? in_right : -1;
  if (left >= key_extent) left = -1;
  if (right >= row_extent) right = -1;
  if (causal) right = 0;
}

// Whether the kernels' int32 position arithmetic (row + offset +- edge, with
// the edges normalised as above) has room for these extents.
inline bool window_arith_fits(bool has_window, long long rows, long long keys) {
  return !has_window || rows + keys + 1024 <= INT_MAX;
}

}  // namespace attn
