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
inline int docpass_row_blocks(const lazy_geom* g) { return g->head_dim == 128 ? 2 : 4; }

}  // namespace lazy
