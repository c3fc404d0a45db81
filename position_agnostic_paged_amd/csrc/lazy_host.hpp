// Host-side helpers shared by the C entry points: thread-local error text and
// argument validation.  No device code.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include "lazy_attn.h"

namespace lazy {

// Records a formatted message for lazy_last_error() and returns `st`.
lazy_status fail(lazy_status st, const char* fmt, ...);
void clear_error();

// Geometry checks shared by every device call.
lazy_status check_geom(const lazy_geom* g);
// Positional-descriptor checks (needs_rotation: the call reads cos/sin).
lazy_status check_pos(const lazy_geom* g, const lazy_pos_desc* p);

// 16-row blocks per wave of the document-major decode pass (rows = reads of
// one shared document x the query group); the planner and the launch agree
// through this one function.
#ifndef LAZY_DOCPASS_RB128
#define LAZY_DOCPASS_RB128 2
#endif
inline int docpass_row_blocks(const lazy_geom* g) { return g->head_dim == 128 ? LAZY_DOCPASS_RB128 : 4; }
// Waves per workgroup of the document pass.  Above 1, the row-block waves of
// one (document, chunk) are grouped in workgroups of this many (the planner
// pads each group with empty items), so they run on one CU and read the same
// tiles at about the same time; measured slower on MI355X (mixed 70B step
// decode 0.36 ms at 1, 0.50 / 0.57 / 0.51 ms at 2 / 4 / 8: padding and
// whole-workgroup residency cost more than the shared reads gain).
#ifndef LAZY_DOCPASS_WG_WAVES
#define LAZY_DOCPASS_WG_WAVES 1
#endif
constexpr int kDocPassWgWaves = LAZY_DOCPASS_WG_WAVES;

}  // namespace lazy
